// wkv_step.hip -- batched single-token RNN step (gfx950).
//
// One token per lane against the carried state, then folded into it (RWKV
// architecture deep dive, youngju.dev, "Numerical stability via log-space
// computation"; output read as in "WKV mechanism: core computation"), for
// L layers x B sequences x C channels in one launch.  Each lane is independent,
// so the kernel is a pure stream: 36 bytes per lane (k, v, y, 3 state planes in
// and out) in float32; k, v, r and y may also be 16-bit (fp16 or bf16), the
// state staying float32.  A thread handles four consecutive channels with 16-byte
// non-temporal loads and stores; a workgroup covers 1024 channels of one
// (layer, sequence) row, so every access of a wave is 1 KiB contiguous.
// With a receptance tensor r ([L][B][C], read beside k and v) the output is
// the time-mixing block's gated sigmoid(r) * wkv (block figure of "RWKV
// architecture overview"): 4 more bytes per lane.
#include "wkv_device.hpp"
#include "wkv_internal.hpp"

namespace wkv {

typedef float f4 __attribute__((ext_vector_type(4)));

// (a, b, o) is the ABI state of one lane (o in natural-log units).
__device__ __forceinline__ float step_one(float &a, float &b, float &o, float k, float v,
                                          float w, float u) {
    Chan ch;
    ch.W = w * kLog2e;
    ch.U = u * kLog2e;
    ch.c1 = 0.0f;  // unused by the two-exponential step
    Lane L = lane_at(a, b, o_in(o));
    const float y = step_safe(L, k * kLog2e, v, ch);
    a = L.a;
    b = L.b;
    o = o_out(lane_o(L, ch.W));
    return y;
}

// Four consecutive elements as floats: one 16-byte access for float32, one
// 8-byte access for the 16-bit formats.
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

template <class IO>
__device__ __forceinline__ f4 ld4(const typename IO::T *p) {
    if constexpr (IO::kBytes == 4) {
        return __builtin_nontemporal_load((const f4 *)p);
    } else {
        const u2 q = __builtin_nontemporal_load((const u2 *)p);
        f4 x;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const unsigned short h = (unsigned short)(q[j >> 1] >> (16 * (j & 1)));
            x[j] = IO::to_f(__builtin_bit_cast(typename IO::T, h));
        }
        return x;
    }
}

template <class IO>
__device__ __forceinline__ void st4(typename IO::T *p, const f4 &x) {
    if constexpr (IO::kBytes == 4) {
        __builtin_nontemporal_store(x, (f4 *)p);
    } else {
        u2 q;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint32_t lo = __builtin_bit_cast(unsigned short, IO::from_f(x[2 * j]));
            const uint32_t hi = __builtin_bit_cast(unsigned short, IO::from_f(x[2 * j + 1]));
            q[j] = lo | (hi << 16);
        }
        __builtin_nontemporal_store(q, (u2 *)p);
    }
}

// VEC = 4: C % 4 == 0 and every pointer aligned to its 4-element access;
// VEC = 1 otherwise.  IO: element format of k, v, r, y (state, w, u: float32).
template <int VEC, bool GATE, class IO>
__global__ __launch_bounds__(256) void step_kernel(int64_t L, int64_t B, int64_t C,
                                                   uint32_t blocks_per_row,
                                                   const float *__restrict__ w,
                                                   const float *__restrict__ u,
                                                   const typename IO::T *__restrict__ k,
                                                   const typename IO::T *__restrict__ v,
                                                   const typename IO::T *__restrict__ r,
                                                   typename IO::T *__restrict__ y,
                                                   const float *s_in, float *s_out) {
    // rows are (layer, sequence) pairs; s_in may equal s_out (in place), so
    // neither is declared restrict
    // L*B rows < 2^31 (checked at launch), so the row split stays in 32 bits
    const uint32_t row32 = blockIdx.x / blocks_per_row;
    const uint32_t cb = blockIdx.x - row32 * blocks_per_row;
    const uint32_t l32 = row32 / (uint32_t)B;
    const int64_t row = row32;
    const int64_t l = l32;
    const int64_t bb = (int64_t)(row32 - l32 * (uint32_t)B);
    const int64_t c = ((int64_t)cb * 256 + threadIdx.x) * VEC;
    if (c >= C) return;
    const int64_t kv = row * C + c;
    const int64_t sa = ((l * 3 + 0) * B + bb) * C + c;
    const int64_t sb = sa + B * C;
    const int64_t so = sb + B * C;
    const int64_t wc = l * C + c;
    if constexpr (VEC == 4) {
        const f4 kk = ld4<IO>(k + kv);
        const f4 vv = ld4<IO>(v + kv);
        f4 aa = __builtin_nontemporal_load((const f4 *)(s_in + sa));
        f4 bq = __builtin_nontemporal_load((const f4 *)(s_in + sb));
        f4 oo = __builtin_nontemporal_load((const f4 *)(s_in + so));
        const f4 ww = *(const f4 *)(w + wc);
        const f4 uu = *(const f4 *)(u + wc);
        f4 rr = {0.0f, 0.0f, 0.0f, 0.0f};
        if constexpr (GATE) rr = ld4<IO>(r + kv);
        f4 yy;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float a = aa[j], b = bq[j], o = oo[j];
            yy[j] = step_one(a, b, o, kk[j], vv[j], ww[j], uu[j]);
            if constexpr (GATE) yy[j] *= gate_of(rr[j]);
            aa[j] = a;
            bq[j] = b;
            oo[j] = o;
        }
        st4<IO>(y + kv, yy);
        __builtin_nontemporal_store(aa, (f4 *)(s_out + sa));
        __builtin_nontemporal_store(bq, (f4 *)(s_out + sb));
        __builtin_nontemporal_store(oo, (f4 *)(s_out + so));
    } else {
        float a = s_in[sa], b = s_in[sb], o = s_in[so];
        float yy = step_one(a, b, o, IO::to_f(k[kv]), IO::to_f(v[kv]), w[wc], u[wc]);
        if constexpr (GATE) yy *= gate_of(IO::to_f(r[kv]));
        y[kv] = IO::from_f(yy);
        s_out[sa] = a;
        s_out[sb] = b;
        s_out[so] = o;
    }
}

template <int VEC, bool GATE, class IO>
static void launch_step_k(const StepArgs &a, int64_t grid, int64_t bpr, hipStream_t st) {
    using T = typename IO::T;
    hipLaunchKernelGGL((step_kernel<VEC, GATE, IO>), dim3((unsigned)grid), dim3(256), 0, st, a.L,
                       a.B, a.C, (uint32_t)bpr, a.w, a.u, (const T *)a.k, (const T *)a.v,
                       (const T *)a.r, (T *)a.y, a.s_in, a.s_out);
}

template <class IO>
static hipError_t launch_step_io(const StepArgs &a, hipStream_t st) {
    // float32 tensors need 16-byte alignment for the 4-wide path, the 16-bit
    // element tensors 8-byte
    const uintptr_t mis32 = (uintptr_t)a.w | (uintptr_t)a.u | (uintptr_t)a.s_in |
                            (uintptr_t)a.s_out;
    const uintptr_t misio = (uintptr_t)a.k | (uintptr_t)a.v | (uintptr_t)a.y | (uintptr_t)a.r;
    const bool vec4 = (a.C % 4 == 0) && (mis32 % 16 == 0) && (misio % (4 * IO::kBytes) == 0);
    const int64_t per_block = 256 * (int64_t)(vec4 ? 4 : 1);
    const int64_t bpr = (a.C + per_block - 1) / per_block;
    const int64_t grid = a.L * a.B * bpr;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (vec4 && a.r)
        launch_step_k<4, true, IO>(a, grid, bpr, st);
    else if (vec4)
        launch_step_k<4, false, IO>(a, grid, bpr, st);
    else if (a.r)
        launch_step_k<1, true, IO>(a, grid, bpr, st);
    else
        launch_step_k<1, false, IO>(a, grid, bpr, st);
    return hipGetLastError();
}

hipError_t launch_step(const StepArgs &a, hipStream_t st) {
    switch (a.io) {
        case kIoF32: return launch_step_io<IoF32>(a, st);
        case kIoF16: return launch_step_io<IoF16>(a, st);
        case kIoBF16: return launch_step_io<IoBF16>(a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace wkv

// wkv_step.hip -- batched single-token RNN step (gfx950).
//
// One token per lane against the carried state, then folded into it (RWKV
// architecture deep dive, youngju.dev, "Numerical stability via log-space
// computation"; output read as in "WKV mechanism: core computation"), for
// L layers x B sequences x C channels in one launch.  Each lane is independent,
// so the kernel is a pure stream: 36 bytes per lane (k, v, y, 3 state planes in
// and out) in float32; k, v, r and y may also be 16-bit (fp16 or bf16), the
// state staying float32.  A thread handles four consecutive channels with 16-byte
// non-temporal loads and stores, in IT chunks 1024 channels apart; a workgroup
// covers IT * 1024 channels of one (layer, sequence) row, so every access of a
// wave is 1 KiB contiguous.  Each thread issues the loads of all its chunks
// before it computes or stores anything: with nine streams per lane (five
// read, four written), more loads in flight per thread is what lifts the
// kernel toward the bandwidth a plain copy reaches.
// With a receptance tensor r ([L][B][C], read beside k and v) the output is
// the time-mixing block's gated sigmoid(r) * wkv (block figure of "RWKV
// architecture overview"): 4 more bytes per lane.
#include "wkv_device.hpp"
#include "wkv_internal.hpp"

namespace wkv {

typedef float f4 __attribute__((ext_vector_type(4)));

// Chunks of 1024 channels per thread (4-wide path), plain and gated.  On
// MI355X at L=24 B=1024 C=4096: 1, 2 and 4 chunks take 686, 634 and 626 us
// per plain step; 1 and 2 chunks 763 and 692 us per gated step (four would
// hold some 170 registers there).
constexpr int kStepChunks = 4;
constexpr int kStepChunksGated = 2;

// (a, b, o) is the ABI state of one lane (o in natural-log units).
//
// The step runs once per token, so the state it hands on must not drift.
// Writing o' = o - w at every token would round o each time, in the same
// direction for similar values: after a few hundred tokens with |o| ~ 60 and
// a slow decay the log-weight is off by more than 1e-4.  So o is written
// back unchanged unless this token became the frame (then o' = k, exactly
// the input), and the decay e^{-w} goes into a and b, whose roundings are
// relative and do not add up that way.  When b has decayed below 2^-20, o
// moves down by a whole number m of natural-log units (exact: o is never
// rounded) and a, b take the factor e^{-m}, which brings b back to [1, e).
__device__ __forceinline__ float step_one(float &a, float &b, float &o, float k, float v,
                                          float w, float u) {
    Chan ch;
    ch.W = w * kLog2e;
    ch.U = u * kLog2e;
    ch.c1 = 0.0f;  // unused by the two-exponential step
    const float o2 = o_in(o);
    Lane L = lane_in(a, b, o2);
    const bool rescaled = L.e0 != o2;  // a far-off b was brought to 1 on the way in
    const float K = k * kLog2e;
    const float y = step_safe(L, K, v, ch);
    if (L.n == 0.0f) {
        // this token is the new frame: the sums are relative to 2^K
        a = L.a;
        b = L.b;
        o = k;
    } else {
        // one decay step past the frame e0: fold it into the sums
        const float d = ex2(-ch.W);
        float an = L.a * d, bn = L.b * d;
        float on = rescaled ? o_out(L.e0) : o;
        if (bn < 0x1p-20f) {
            const float m = floorf(lg2(bn) * kLn2);  // whole natural-log units, <= -14
            const float sc = ex2(-m * kLog2e);
            an *= sc;
            bn *= sc;
            on += m;
        }
        a = an;
        b = bn;
        o = on;
    }
    return y;
}

constexpr uint32_t kStepWindow = 64;

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
// VEC = 1 otherwise (then IT = 1).  IT: chunks of 1024 channels per thread.
// IO: element format of k, v, r, y (state, w, u: float32).
template <int VEC, int IT, bool GATE, class IO>
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
    // The hardware hands consecutive workgroups to the 8 dies in turn; within
    // each window of 64 workgroups every die takes 8 adjacent ones instead
    // (contiguous rows of each tensor per die: measured 1-2% faster at the
    // L=24 B=1024 C=4096 decode shape).
    uint32_t wid = blockIdx.x;
    if (gridDim.x % kStepWindow == 0) {
        const uint32_t in = wid % kStepWindow;
        wid += (in % 8u) * (kStepWindow / 8u) + in / 8u - in;
    }
    const uint32_t row32 = wid / blocks_per_row;
    const uint32_t cb = wid - row32 * blocks_per_row;
    const uint32_t l32 = row32 / (uint32_t)B;
    const int64_t row = row32;
    const int64_t l = l32;
    const int64_t bb = (int64_t)(row32 - l32 * (uint32_t)B);
    const int64_t c0 = ((int64_t)cb * 256 * IT + threadIdx.x) * VEC;
    if (c0 >= C) return;
    // chunk i of this thread: channels c0 + i * 1024 .. + 3
    const int64_t kv = row * C + c0;
    const int64_t sa = ((l * 3 + 0) * B + bb) * C + c0;
    const int64_t sb = sa + B * C;
    const int64_t so = sb + B * C;
    const int64_t wc = l * C + c0;
    if constexpr (VEC == 4) {
        constexpr int64_t kStride = 256 * 4;
        f4 kk[IT], vv[IT], aa[IT], bq[IT], oo[IT], ww[IT], uu[IT], rr[IT];
#pragma unroll
        for (int i = 0; i < IT; ++i) {
            const int64_t d = i * kStride;
            if (i == 0 || c0 + d < C) {
                kk[i] = ld4<IO>(k + kv + d);
                vv[i] = ld4<IO>(v + kv + d);
                aa[i] = __builtin_nontemporal_load((const f4 *)(s_in + sa + d));
                bq[i] = __builtin_nontemporal_load((const f4 *)(s_in + sb + d));
                oo[i] = __builtin_nontemporal_load((const f4 *)(s_in + so + d));
                ww[i] = *(const f4 *)(w + wc + d);
                uu[i] = *(const f4 *)(u + wc + d);
                if constexpr (GATE) rr[i] = ld4<IO>(r + kv + d);
            }
        }
#pragma unroll
        for (int i = 0; i < IT; ++i) {
            const int64_t d = i * kStride;
            if (i == 0 || c0 + d < C) {
                f4 yy;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float a = aa[i][j], b = bq[i][j], o = oo[i][j];
                    yy[j] = step_one(a, b, o, kk[i][j], vv[i][j], ww[i][j], uu[i][j]);
                    if constexpr (GATE) yy[j] *= gate_of(rr[i][j]);
                    aa[i][j] = a;
                    bq[i][j] = b;
                    oo[i][j] = o;
                }
                st4<IO>(y + kv + d, yy);
                __builtin_nontemporal_store(aa[i], (f4 *)(s_out + sa + d));
                __builtin_nontemporal_store(bq[i], (f4 *)(s_out + sb + d));
                __builtin_nontemporal_store(oo[i], (f4 *)(s_out + so + d));
            }
        }
    } else {
        const int64_t c = c0;
        float a = s_in[sa], b = s_in[sb], o = s_in[so];
        float yy = step_one(a, b, o, IO::to_f(k[kv]), IO::to_f(v[kv]), w[wc], u[wc]);
        if constexpr (GATE) yy *= gate_of(IO::to_f(r[kv]));
        y[kv] = IO::from_f(yy);
        s_out[sa] = a;
        s_out[sb] = b;
        s_out[so] = o;
    }
}

template <int VEC, int IT, bool GATE, class IO>
static void launch_step_k(const StepArgs &a, int64_t grid, int64_t bpr, hipStream_t st) {
    using T = typename IO::T;
    hipLaunchKernelGGL((step_kernel<VEC, IT, GATE, IO>), dim3((unsigned)grid), dim3(256), 0, st, a.L,
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
    const int64_t it = vec4 ? (a.r ? kStepChunksGated : kStepChunks) : 1;
    const int64_t per_block = 256 * (int64_t)(vec4 ? 4 : 1) * it;
    const int64_t bpr = (a.C + per_block - 1) / per_block;
    const int64_t grid = a.L * a.B * bpr;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (vec4 && a.r)
        launch_step_k<4, kStepChunksGated, true, IO>(a, grid, bpr, st);
    else if (vec4)
        launch_step_k<4, kStepChunks, false, IO>(a, grid, bpr, st);
    else if (a.r)
        launch_step_k<1, 1, true, IO>(a, grid, bpr, st);
    else
        launch_step_k<1, 1, false, IO>(a, grid, bpr, st);
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

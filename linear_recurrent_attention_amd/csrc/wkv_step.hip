// wkv_step.hip -- batched single-token RNN step (gfx950).
//
// One token per lane against the carried state, then folded into it (RWKV
// architecture deep dive, youngju.dev, "Numerical stability via log-space
// computation"; output read as in "WKV mechanism: core computation"), for
// L layers x B sequences x C channels in one launch.  Each lane is independent,
// so the kernel is a pure stream: 36 bytes per lane (k, v, y, 3 state planes in
// and out).  A thread handles four consecutive channels with 16-byte
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

// VEC = 4: C % 4 == 0 and every pointer 16-byte aligned; VEC = 1 otherwise.
template <int VEC, bool GATE>
__global__ __launch_bounds__(256) void step_kernel(int64_t L, int64_t B, int64_t C,
                                                   uint32_t blocks_per_row,
                                                   const float *__restrict__ w,
                                                   const float *__restrict__ u,
                                                   const float *__restrict__ k,
                                                   const float *__restrict__ v,
                                                   const float *__restrict__ r,
                                                   float *__restrict__ y,
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
        const f4 kk = __builtin_nontemporal_load((const f4 *)(k + kv));
        const f4 vv = __builtin_nontemporal_load((const f4 *)(v + kv));
        f4 aa = __builtin_nontemporal_load((const f4 *)(s_in + sa));
        f4 bq = __builtin_nontemporal_load((const f4 *)(s_in + sb));
        f4 oo = __builtin_nontemporal_load((const f4 *)(s_in + so));
        const f4 ww = *(const f4 *)(w + wc);
        const f4 uu = *(const f4 *)(u + wc);
        f4 rr = {0.0f, 0.0f, 0.0f, 0.0f};
        if constexpr (GATE) rr = __builtin_nontemporal_load((const f4 *)(r + kv));
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
        __builtin_nontemporal_store(yy, (f4 *)(y + kv));
        __builtin_nontemporal_store(aa, (f4 *)(s_out + sa));
        __builtin_nontemporal_store(bq, (f4 *)(s_out + sb));
        __builtin_nontemporal_store(oo, (f4 *)(s_out + so));
    } else {
        float a = s_in[sa], b = s_in[sb], o = s_in[so];
        float yy = step_one(a, b, o, k[kv], v[kv], w[wc], u[wc]);
        if constexpr (GATE) yy *= gate_of(r[kv]);
        y[kv] = yy;
        s_out[sa] = a;
        s_out[sb] = b;
        s_out[so] = o;
    }
}

hipError_t launch_step(const StepArgs &a, hipStream_t st) {
    const uintptr_t mis = (uintptr_t)a.w | (uintptr_t)a.u | (uintptr_t)a.k | (uintptr_t)a.v |
                          (uintptr_t)a.y | (uintptr_t)a.s_in | (uintptr_t)a.s_out |
                          (uintptr_t)a.r;
    const bool vec4 = (a.C % 4 == 0) && (mis % 16 == 0);
    const int vec = vec4 ? 4 : 1;
    const int64_t per_block = 256 * (int64_t)vec;
    const int64_t bpr = (a.C + per_block - 1) / per_block;
    const int64_t rows = a.L * a.B;
    const int64_t grid = rows * bpr;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
#define WKV_STEP_LAUNCH(VEC, GATE)                                                          \
    hipLaunchKernelGGL((step_kernel<VEC, GATE>), dim3((unsigned)grid), dim3(256), 0, st, a.L, \
                       a.B, a.C, (uint32_t)bpr, a.w, a.u, a.k, a.v, a.r, a.y, a.s_in, a.s_out)
    if (vec4 && a.r)
        WKV_STEP_LAUNCH(4, true);
    else if (vec4)
        WKV_STEP_LAUNCH(4, false);
    else if (a.r)
        WKV_STEP_LAUNCH(1, true);
    else
        WKV_STEP_LAUNCH(1, false);
#undef WKV_STEP_LAUNCH
    return hipGetLastError();
}

}  // namespace wkv

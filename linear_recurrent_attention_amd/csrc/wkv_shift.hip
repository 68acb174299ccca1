// wkv_shift.hip -- token shift of the time-mixing block (gfx950).
//
// RWKV architecture deep dive, youngju.dev, "Token shift": before the R, K and
// V projections each input mixes the current token with the previous one,
//     out_m[b][t][c] = mu_m[c] x[b][t][c] + (1 - mu_m[c]) x[b][t-1][c],
// one per-channel weight vector mu_m per projection input (M of them).  For
// the first token of a call, x[b][-1] is the last token of the previous call:
// the att_x_prev state that the rwkv-architecture skill page ("Advanced
// topics") lists beside the WKV state.  A fresh sequence starts from zero.
// The call also returns the new att_x_prev, x[b][T-1].
//
// A pure stream: 4 bytes read and 4 M bytes written per element.  A thread owns
// VEC consecutive channels of one sequence over a tile of TT tokens.  It reads
// the row before the tile once, then every row of the tile once, keeping the
// previous row in registers.  A wave's access to one row is 64 x 16 B
// contiguous (VEC = 4).
#include "wkv_device.hpp"
#include "wkv_internal.hpp"

namespace wkv {

namespace {

// Tokens per tile.  Tiles of 4 to 32 tokens time alike on MI355X; short ones
// give small shapes more workgroups.
constexpr int kTT = 8;

template <int VEC>
struct Vec {
    float x[VEC];
};

template <int VEC>
__device__ __forceinline__ Vec<VEC> vload(const float *p) {
    Vec<VEC> r;
    if constexpr (VEC == 4) {
        typedef float f4 __attribute__((ext_vector_type(4)));
        const f4 q = __builtin_nontemporal_load((const f4 *)p);
#pragma unroll
        for (int i = 0; i < 4; ++i) r.x[i] = q[i];
    } else {
        r.x[0] = __builtin_nontemporal_load(p);
    }
    return r;
}

template <int VEC>
__device__ __forceinline__ void vstore(float *p, const Vec<VEC> &r) {
    if constexpr (VEC == 4) {
        typedef float f4 __attribute__((ext_vector_type(4)));
        f4 q;
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = r.x[i];
        __builtin_nontemporal_store(q, (f4 *)p);
    } else {
        __builtin_nontemporal_store(r.x[0], p);
    }
}

template <int VEC, int M>
__device__ __forceinline__ void emit(float *out, int64_t plane, int64_t off, const Vec<VEC> (&mu)[M],
                                     const Vec<VEC> (&nu)[M], const Vec<VEC> &cur,
                                     const Vec<VEC> &prev) {
#pragma unroll
    for (int m = 0; m < M; ++m) {
        Vec<VEC> o;
#pragma unroll
        for (int i = 0; i < VEC; ++i) o.x[i] = fmaf(mu[m].x[i], cur.x[i], nu[m].x[i] * prev.x[i]);
        vstore<VEC>(out + m * plane + off, o);
    }
}

// 1-D grid: column block fastest, then tile, then sequence.  write_last: this
// kernel also stores x[b][T-1] into x_prev_out (the host clears it when
// x_prev_out is x_prev itself and another workgroup may still read x_prev).
template <int VEC, int M>
__global__ __launch_bounds__(256) void shift_kernel(int64_t B, int64_t T, int64_t C,
                                                    uint32_t cblocks, uint32_t ntiles,
                                                    const float *__restrict__ mu,
                                                    const float *__restrict__ x,
                                                    const float *x_prev,
                                                    float *__restrict__ out, float *x_prev_out,
                                                    int write_last) {
    const uint32_t cb = blockIdx.x % cblocks;
    const uint32_t rest = blockIdx.x / cblocks;
    const uint32_t tile = rest % ntiles;
    const int64_t bb = rest / ntiles;
    const int64_t c = ((int64_t)cb * 256 + threadIdx.x) * VEC;
    if (c >= C) return;
    Vec<VEC> m_[M], n_[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
            m_[m].x[i] = mu[m * C + c + i];
            n_[m].x[i] = 1.0f - m_[m].x[i];
        }
    }
    const int64_t t0 = (int64_t)tile * kTT;
    const int64_t row0 = bb * T;  // first row of this sequence
    const int64_t plane = B * T * C;
    Vec<VEC> prev;
    if (t0 > 0) {
        prev = vload<VEC>(x + (row0 + t0 - 1) * C + c);
    } else if (x_prev) {
        prev = vload<VEC>(x_prev + bb * C + c);
    } else {
#pragma unroll
        for (int i = 0; i < VEC; ++i) prev.x[i] = 0.0f;
    }
    if (t0 + kTT <= T) {
        // whole tile: every row load issued before the first use
        Vec<VEC> cur[kTT];
#pragma unroll
        for (int t = 0; t < kTT; ++t) cur[t] = vload<VEC>(x + (row0 + t0 + t) * C + c);
#pragma unroll
        for (int t = 0; t < kTT; ++t) {
            emit<VEC, M>(out, plane, (row0 + t0 + t) * C + c, m_, n_, cur[t], prev);
            prev = cur[t];
        }
    } else {
        for (int64_t t = t0; t < T; ++t) {
            const Vec<VEC> cur = vload<VEC>(x + (row0 + t) * C + c);
            emit<VEC, M>(out, plane, (row0 + t) * C + c, m_, n_, cur, prev);
            prev = cur;
        }
    }
    if (write_last && x_prev_out && t0 + kTT >= T) vstore<VEC>(x_prev_out + bb * C + c, prev);
}

// x_prev_out[b][c] <- x[b][T-1][c] (T > 0), or x_prev (zero when NULL) for T == 0.
__global__ __launch_bounds__(256) void shift_last_kernel(int64_t B, int64_t T, int64_t C,
                                                         const float *x, const float *x_prev,
                                                         float *x_prev_out) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= B * C) return;
    const int64_t bb = i / C, c = i - bb * C;
    float val;
    if (T > 0)
        val = x[(bb * T + T - 1) * C + c];
    else
        val = x_prev ? x_prev[i] : 0.0f;
    x_prev_out[i] = val;
}

template <int VEC, int M>
hipError_t launch_shift_m(const ShiftArgs &a, uint32_t cblocks, uint32_t ntiles, int write_last,
                          hipStream_t st) {
    const int64_t grid = (int64_t)cblocks * ntiles * a.B;
    hipLaunchKernelGGL((shift_kernel<VEC, M>), dim3((unsigned)grid), dim3(256), 0, st, a.B, a.T,
                       a.C, cblocks, ntiles, a.mu, a.x, a.x_prev, a.out, a.x_prev_out,
                       write_last);
    return hipGetLastError();
}

template <int VEC>
hipError_t launch_shift_vec(const ShiftArgs &a, uint32_t cblocks, uint32_t ntiles,
                            int write_last, hipStream_t st) {
    switch (a.M) {
        case 1: return launch_shift_m<VEC, 1>(a, cblocks, ntiles, write_last, st);
        case 2: return launch_shift_m<VEC, 2>(a, cblocks, ntiles, write_last, st);
        case 3: return launch_shift_m<VEC, 3>(a, cblocks, ntiles, write_last, st);
        case 4: return launch_shift_m<VEC, 4>(a, cblocks, ntiles, write_last, st);
        case 5: return launch_shift_m<VEC, 5>(a, cblocks, ntiles, write_last, st);
        case 6: return launch_shift_m<VEC, 6>(a, cblocks, ntiles, write_last, st);
        case 7: return launch_shift_m<VEC, 7>(a, cblocks, ntiles, write_last, st);
        case 8: return launch_shift_m<VEC, 8>(a, cblocks, ntiles, write_last, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

// B*C > 0 here.  M == 0 or T == 0 only update x_prev_out.
hipError_t launch_token_shift(const ShiftArgs &a, bool in_place_state, hipStream_t st) {
    const int64_t lanes = a.B * a.C;
    const int64_t last_grid = (lanes + 255) / 256;
    if (last_grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    auto launch_last = [&]() {
        hipLaunchKernelGGL(shift_last_kernel, dim3((unsigned)last_grid), dim3(256), 0, st, a.B,
                           a.T, a.C, a.x, a.x_prev, a.x_prev_out);
        return hipGetLastError();
    };
    if (a.T == 0 || a.M == 0) {
        if (!a.x_prev_out || (a.T == 0 && in_place_state)) return hipSuccess;
        return launch_last();
    }
    const uintptr_t mis = (uintptr_t)a.mu | (uintptr_t)a.x | (uintptr_t)a.x_prev |
                          (uintptr_t)a.out | (uintptr_t)a.x_prev_out;
    const bool vec4 = (a.C % 4 == 0) && (mis % 16 == 0);
    const int64_t per_block = 256 * (vec4 ? 4 : 1);
    const int64_t cblocks = (a.C + per_block - 1) / per_block;
    const int64_t ntiles = (a.T + kTT - 1) / kTT;
    if (cblocks > 0x7fffffffLL / ntiles || cblocks * ntiles > 0x7fffffffLL / a.B)
        return hipErrorInvalidConfiguration;
    // In place with several tiles, the workgroup holding the last token could
    // overwrite x_prev before the first tile's workgroup reads it: write the
    // new state in a second launch instead.
    const bool late = a.x_prev_out && in_place_state && ntiles > 1;
    const int write_last = a.x_prev_out && !late ? 1 : 0;
    hipError_t e = vec4 ? launch_shift_vec<4>(a, (uint32_t)cblocks, (uint32_t)ntiles, write_last, st)
                        : launch_shift_vec<1>(a, (uint32_t)cblocks, (uint32_t)ntiles, write_last, st);
    if (e != hipSuccess || !late) return e;
    return launch_last();
}

}  // namespace wkv

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

// VEC consecutive elements of format IO (float32 or a 16-bit format), widened
// to float; 16-byte (float32) or 8-byte (16-bit) accesses when VEC = 4.
template <class IO, int VEC>
__device__ __forceinline__ Vec<VEC> vload(const typename IO::T *p) {
    Vec<VEC> r;
    if constexpr (IO::kBytes == 4) {
        if constexpr (VEC == 4) {
            typedef float f4 __attribute__((ext_vector_type(4)));
            const f4 q = __builtin_nontemporal_load((const f4 *)p);
#pragma unroll
            for (int i = 0; i < 4; ++i) r.x[i] = q[i];
        } else {
            r.x[0] = __builtin_nontemporal_load((const float *)p);
        }
    } else {
        using T = typename IO::T;
        if constexpr (VEC == 4) {
            // one 8-byte access, as two 32-bit words (a vector of four 16-bit
            // elements is split by the compiler into narrower accesses)
            typedef unsigned int u2 __attribute__((ext_vector_type(2)));
            const u2 q = __builtin_nontemporal_load((const u2 *)p);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const unsigned short h = (unsigned short)(q[i >> 1] >> (16 * (i & 1)));
                r.x[i] = IO::to_f(__builtin_bit_cast(T, h));
            }
        } else {
            const unsigned short q = __builtin_nontemporal_load((const unsigned short *)p);
            r.x[0] = IO::to_f(__builtin_bit_cast(T, q));
        }
    }
    return r;
}

// Rounds once to IO (nearest, ties to even) and stores.
template <class IO, int VEC>
__device__ __forceinline__ void vstore(typename IO::T *p, const Vec<VEC> &r) {
    if constexpr (IO::kBytes == 4) {
        if constexpr (VEC == 4) {
            typedef float f4 __attribute__((ext_vector_type(4)));
            f4 q;
#pragma unroll
            for (int i = 0; i < 4; ++i) q[i] = r.x[i];
            __builtin_nontemporal_store(q, (f4 *)p);
        } else {
            __builtin_nontemporal_store(r.x[0], (float *)p);
        }
    } else {
        if constexpr (VEC == 4) {
            typedef unsigned int u2 __attribute__((ext_vector_type(2)));
            u2 q;
#pragma unroll
            for (int j = 0; j < 2; ++j)
                q[j] = (unsigned int)__builtin_bit_cast(unsigned short, IO::from_f(r.x[2 * j])) |
                       ((unsigned int)__builtin_bit_cast(unsigned short, IO::from_f(r.x[2 * j + 1]))
                        << 16);
            __builtin_nontemporal_store(q, (u2 *)p);
        } else {
            __builtin_nontemporal_store(__builtin_bit_cast(unsigned short, IO::from_f(r.x[0])),
                                        (unsigned short *)p);
        }
    }
}

template <class IO, int VEC, int M>
__device__ __forceinline__ void emit(typename IO::T *out, int64_t plane, int64_t off,
                                     const Vec<VEC> (&mu)[M], const Vec<VEC> (&nu)[M],
                                     const Vec<VEC> &cur, const Vec<VEC> &prev) {
#pragma unroll
    for (int m = 0; m < M; ++m) {
        Vec<VEC> o;
#pragma unroll
        for (int i = 0; i < VEC; ++i) o.x[i] = fmaf(mu[m].x[i], cur.x[i], nu[m].x[i] * prev.x[i]);
        vstore<IO, VEC>(out + m * plane + off, o);
    }
}

// 1-D grid: column block fastest, then tile, then sequence.  write_last: this
// kernel also stores x[b][T-1] into x_prev_out (the host clears it when
// x_prev_out is x_prev itself and another workgroup may still read x_prev).
// IO: element format of x, x_prev, out and x_prev_out (mu is float32).
template <class IO, int VEC, int M>
__global__ __launch_bounds__(256) void shift_kernel(int64_t B, int64_t T, int64_t C,
                                                    uint32_t cblocks, uint32_t ntiles,
                                                    const float *__restrict__ mu,
                                                    const typename IO::T *__restrict__ x,
                                                    const typename IO::T *x_prev,
                                                    typename IO::T *__restrict__ out,
                                                    typename IO::T *x_prev_out, int write_last) {
    // The hardware hands consecutive workgroups to the 8 dies in turn; within
    // each window of 64 workgroups every die takes 8 adjacent ones instead
    // (measured 1.5% faster at B=8 T=1024 C=2048; the same remap made the
    // backward below 6% slower, so it keeps the plain order)
    uint32_t wid = blockIdx.x;
    if (gridDim.x % 64u == 0) {
        const uint32_t in = wid % 64u;
        wid += (in % 8u) * 8u + in / 8u - in;
    }
    const uint32_t cb = wid % cblocks;
    const uint32_t rest = wid / cblocks;
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
        prev = vload<IO, VEC>(x + (row0 + t0 - 1) * C + c);
    } else if (x_prev) {
        prev = vload<IO, VEC>(x_prev + bb * C + c);
    } else {
#pragma unroll
        for (int i = 0; i < VEC; ++i) prev.x[i] = 0.0f;
    }
    if (t0 + kTT <= T) {
        // whole tile: every row load issued before the first use
        Vec<VEC> cur[kTT];
#pragma unroll
        for (int t = 0; t < kTT; ++t) cur[t] = vload<IO, VEC>(x + (row0 + t0 + t) * C + c);
#pragma unroll
        for (int t = 0; t < kTT; ++t) {
            emit<IO, VEC, M>(out, plane, (row0 + t0 + t) * C + c, m_, n_, cur[t], prev);
            prev = cur[t];
        }
    } else {
        for (int64_t t = t0; t < T; ++t) {
            const Vec<VEC> cur = vload<IO, VEC>(x + (row0 + t) * C + c);
            emit<IO, VEC, M>(out, plane, (row0 + t) * C + c, m_, n_, cur, prev);
            prev = cur;
        }
    }
    // (the carried token is an x row, so it is stored exactly)
    if (write_last && x_prev_out && t0 + kTT >= T) vstore<IO, VEC>(x_prev_out + bb * C + c, prev);
}

// x_prev_out[b][c] <- x[b][T-1][c] (T > 0), or x_prev (zero when NULL) for T == 0.
template <class IO>
__global__ __launch_bounds__(256) void shift_last_kernel(int64_t B, int64_t T, int64_t C,
                                                         const typename IO::T *x,
                                                         const typename IO::T *x_prev,
                                                         typename IO::T *x_prev_out) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= B * C) return;
    const int64_t bb = i / C, c = i - bb * C;
    typename IO::T val;
    if (T > 0)
        val = x[(bb * T + T - 1) * C + c];
    else
        val = x_prev ? x_prev[i] : IO::from_f(0.0f);
    x_prev_out[i] = val;
}

template <class IO, int VEC, int M>
hipError_t launch_shift_m(const ShiftArgs &a, uint32_t cblocks, uint32_t ntiles, int write_last,
                          hipStream_t st) {
    using T = typename IO::T;
    const int64_t grid = (int64_t)cblocks * ntiles * a.B;
    hipLaunchKernelGGL((shift_kernel<IO, VEC, M>), dim3((unsigned)grid), dim3(256), 0, st, a.B,
                       a.T, a.C, cblocks, ntiles, a.mu, (const T *)a.x, (const T *)a.x_prev,
                       (T *)a.out, (T *)a.x_prev_out, write_last);
    return hipGetLastError();
}

template <class IO, int VEC>
hipError_t launch_shift_vec(const ShiftArgs &a, uint32_t cblocks, uint32_t ntiles,
                            int write_last, hipStream_t st) {
    switch (a.M) {
        case 1: return launch_shift_m<IO, VEC, 1>(a, cblocks, ntiles, write_last, st);
        case 2: return launch_shift_m<IO, VEC, 2>(a, cblocks, ntiles, write_last, st);
        case 3: return launch_shift_m<IO, VEC, 3>(a, cblocks, ntiles, write_last, st);
        case 4: return launch_shift_m<IO, VEC, 4>(a, cblocks, ntiles, write_last, st);
        case 5: return launch_shift_m<IO, VEC, 5>(a, cblocks, ntiles, write_last, st);
        case 6: return launch_shift_m<IO, VEC, 6>(a, cblocks, ntiles, write_last, st);
        case 7: return launch_shift_m<IO, VEC, 7>(a, cblocks, ntiles, write_last, st);
        case 8: return launch_shift_m<IO, VEC, 8>(a, cblocks, ntiles, write_last, st);
        default: return hipErrorInvalidValue;
    }
}

// ---------------------------------------------------------------------------
// Backward.  With d the gradients of the mixes and d_xpo that of the carried
// token handed on, token t feeds mix t with weight mu and mix t + 1 with
// 1 - mu, so
//   dx[t]   = sum_m (d_m[t+1] + mu_m (d_m[t] - d_m[t+1]))   (+ d_xpo at T - 1)
//   dx_prev = sum_m (1 - mu_m) d_m[0]
//   dmu_m   = sum_{b,t} d_m[t] (x[t] - x[t-1]),  x[-1] = x_prev (or 0).
// A pure stream again: x and the M gradients read, dx written.  A lane owns
// VEC channels and walks a segment of kBT tokens, carrying the previous x row
// and the next gradient row in registers; the 4 waves of a workgroup take 4
// consecutive segments, and their dmu sums are combined in LDS in a fixed
// order into one partial per (sequence, 256-token tile), summed over those by
// shift_bwd_reduce_kernel in double precision (deterministic, no atomics).
// Long segments with the loop unrolled by 4 keep several rows in flight per
// wave: on MI355X 64 tokens per wave ran 21% faster than 16 at B=8 T=1024
// C=2048, and 128 left too few workgroups.
constexpr int kBT = 64;  // tokens per wave
constexpr int kBW = 4;   // waves per workgroup, stacked along the sequence

// IO: element format of x, x_prev, d_out, d_xpo, dx and dxp (mu, dmu and the
// partials are float32).
template <class IO, int VEC, int M>
__global__ __launch_bounds__(256) void shift_bwd_kernel(
    int64_t B, int64_t T, int64_t C, uint32_t cblocks, uint32_t nwt, const float *__restrict__ mu,
    const typename IO::T *__restrict__ x, const typename IO::T *__restrict__ x_prev,
    const typename IO::T *__restrict__ dout, const typename IO::T *__restrict__ dxpo,
    typename IO::T *__restrict__ dx, typename IO::T *__restrict__ dxp,
    float *__restrict__ part) {
    __shared__ float red[kBW][M][64 * VEC];
    const uint32_t cb = blockIdx.x % cblocks;
    const uint32_t rest = blockIdx.x / cblocks;
    const uint32_t wt = rest % nwt;
    const int64_t bb = rest / nwt;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t c = ((int64_t)cb * 64 + lane) * VEC;
    const bool active = c < C;  // (VEC = 4 only when C is a multiple of 4)
    const int64_t t0 = ((int64_t)wt * kBW + wave) * kBT;
    const int64_t t1 = t0 + kBT < T ? t0 + kBT : T;
    const int64_t plane = B * T * C;
    Vec<VEC> acc[M];
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int i = 0; i < VEC; ++i) acc[m].x[i] = 0.0f;
    if (active && t0 < T) {
        Vec<VEC> mu_[M], dcur[M], xprev;
#pragma unroll
        for (int m = 0; m < M; ++m) {
#pragma unroll
            for (int i = 0; i < VEC; ++i) mu_[m].x[i] = mu[m * C + c + i];
            dcur[m] = vload<IO, VEC>(dout + m * plane + (bb * T + t0) * C + c);
        }
        if (t0 > 0) {
            xprev = vload<IO, VEC>(x + (bb * T + t0 - 1) * C + c);
        } else if (x_prev) {
            xprev = vload<IO, VEC>(x_prev + bb * C + c);
        } else {
#pragma unroll
            for (int i = 0; i < VEC; ++i) xprev.x[i] = 0.0f;
        }
        if (t0 == 0 && dxp) {
            Vec<VEC> g;
#pragma unroll
            for (int i = 0; i < VEC; ++i) g.x[i] = 0.0f;
#pragma unroll
            for (int m = 0; m < M; ++m)
#pragma unroll
                for (int i = 0; i < VEC; ++i) g.x[i] = fmaf(1.0f - mu_[m].x[i], dcur[m].x[i], g.x[i]);
            vstore<IO, VEC>(dxp + bb * C + c, g);
        }
#pragma unroll 4
        for (int64_t t = t0; t < t1; ++t) {
            const int64_t row = (bb * T + t) * C + c;
            const Vec<VEC> xcur = vload<IO, VEC>(x + row);
            const bool more = t + 1 < T;
            Vec<VEC> dnext[M], g;
#pragma unroll
            for (int m = 0; m < M; ++m) {
                if (more) {
                    dnext[m] = vload<IO, VEC>(dout + m * plane + row + C);
                } else {
#pragma unroll
                    for (int i = 0; i < VEC; ++i) dnext[m].x[i] = 0.0f;
                }
            }
            if (!more && dxpo) {
                g = vload<IO, VEC>(dxpo + bb * C + c);
            } else {
#pragma unroll
                for (int i = 0; i < VEC; ++i) g.x[i] = 0.0f;
            }
#pragma unroll
            for (int m = 0; m < M; ++m)
#pragma unroll
                for (int i = 0; i < VEC; ++i) {
                    const float dc = dcur[m].x[i], dn = dnext[m].x[i];
                    g.x[i] += fmaf(mu_[m].x[i], dc - dn, dn);
                    acc[m].x[i] = fmaf(dc, xcur.x[i] - xprev.x[i], acc[m].x[i]);
                    dcur[m].x[i] = dn;
                }
            vstore<IO, VEC>(dx + row, g);
            xprev = xcur;
        }
    }
    // dmu of this workgroup: the waves' sums added in wave order
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int i = 0; i < VEC; ++i) red[wave][m][lane * VEC + i] = acc[m].x[i];
    __syncthreads();
    if (wave == 0 && active) {
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int i = 0; i < VEC; ++i) {
                float sum = red[0][m][lane * VEC + i];
#pragma unroll
                for (int w = 1; w < kBW; ++w) sum += red[w][m][lane * VEC + i];
                part[((bb * nwt + wt) * M + m) * C + c + i] = sum;
            }
    }
}

// dmu[m][c] = sum over the (sequence, tile) partials in order, in double.
__global__ __launch_bounds__(256) void shift_bwd_reduce_kernel(int64_t n_part, int64_t MC,
                                                               const float *__restrict__ part,
                                                               float *__restrict__ dmu) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= MC) return;
    double s = 0.0;
    for (int64_t p = 0; p < n_part; ++p) s += (double)part[p * MC + i];
    dmu[i] = (float)s;
}

// No mixes: dx is the carried token's gradient at T - 1 and zero elsewhere;
// x_prev feeds nothing, so dx_prev is zero.
template <class IO>
__global__ __launch_bounds__(256) void shift_bwd_nomix_kernel(int64_t B, int64_t T, int64_t C,
                                                              const typename IO::T *dxpo,
                                                              typename IO::T *dx,
                                                              typename IO::T *dxp) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < B * T * C) {
        const int64_t c = i % C, t = (i / C) % T, bb = i / (C * T);
        dx[i] = (t == T - 1 && dxpo) ? dxpo[bb * C + c] : IO::from_f(0.0f);
    }
    if (dxp && i < B * C) dxp[i] = IO::from_f(0.0f);
}

// No tokens: dx_prev = d_xpo (or 0) and dmu = 0.
template <class IO>
__global__ __launch_bounds__(256) void shift_bwd_empty_kernel(int64_t BC, int64_t MC,
                                                              const typename IO::T *dxpo,
                                                              typename IO::T *dxp, float *dmu) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (dxp && i < BC) dxp[i] = dxpo ? dxpo[i] : IO::from_f(0.0f);
    if (dmu && i < MC) dmu[i] = 0.0f;
}

template <class IO, int VEC, int M>
hipError_t launch_shift_bwd_m(const ShiftBwdArgs &a, uint32_t cblocks, uint32_t nwt,
                              hipStream_t st) {
    using T = typename IO::T;
    const int64_t grid = (int64_t)cblocks * nwt * a.B;
    hipLaunchKernelGGL((shift_bwd_kernel<IO, VEC, M>), dim3((unsigned)grid), dim3(256), 0, st,
                       a.B, a.T, a.C, cblocks, nwt, a.mu, (const T *)a.x, (const T *)a.x_prev,
                       (const T *)a.d_out, (const T *)a.d_xpo, (T *)a.dx, (T *)a.dxp, a.part);
    return hipGetLastError();
}

template <class IO, int VEC>
hipError_t launch_shift_bwd_vec(const ShiftBwdArgs &a, uint32_t cblocks, uint32_t nwt,
                                hipStream_t st) {
    switch (a.M) {
        case 1: return launch_shift_bwd_m<IO, VEC, 1>(a, cblocks, nwt, st);
        case 2: return launch_shift_bwd_m<IO, VEC, 2>(a, cblocks, nwt, st);
        case 3: return launch_shift_bwd_m<IO, VEC, 3>(a, cblocks, nwt, st);
        case 4: return launch_shift_bwd_m<IO, VEC, 4>(a, cblocks, nwt, st);
        default: break;
    }
    if constexpr (VEC == 1) {
        switch (a.M) {
            case 5: return launch_shift_bwd_m<IO, 1, 5>(a, cblocks, nwt, st);
            case 6: return launch_shift_bwd_m<IO, 1, 6>(a, cblocks, nwt, st);
            case 7: return launch_shift_bwd_m<IO, 1, 7>(a, cblocks, nwt, st);
            case 8: return launch_shift_bwd_m<IO, 1, 8>(a, cblocks, nwt, st);
            default: break;
        }
    }
    return hipErrorInvalidValue;
}

// The host side of both directions, for one element format.
template <class IO>
hipError_t token_shift_backward_io(const ShiftBwdArgs &a, hipStream_t st) {
    using T = typename IO::T;
    const int64_t BC = a.B * a.C, MC = a.M * a.C;
    if (a.T == 0 || BC == 0) {
        // no tokens (or no lanes): dx_prev = d_xpo, dmu = 0
        const int64_t n = BC > MC ? BC : MC;
        if (n == 0) return hipSuccess;
        if ((n + 255) / 256 > 0x7fffffffLL) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL(shift_bwd_empty_kernel<IO>, dim3((unsigned)((n + 255) / 256)),
                           dim3(256), 0, st, BC, MC, (const T *)a.d_xpo, (T *)a.dxp, a.dmu);
        return hipGetLastError();
    }
    if (a.M == 0) {
        const int64_t n = a.B * a.T * a.C;
        if ((n + 255) / 256 > 0x7fffffffLL) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL(shift_bwd_nomix_kernel<IO>, dim3((unsigned)((n + 255) / 256)),
                           dim3(256), 0, st, a.B, a.T, a.C, (const T *)a.d_xpo, (T *)a.dx,
                           (T *)a.dxp);
        return hipGetLastError();
    }
    // four channels per lane when C and every pointer allow 4-element accesses
    // and M <= 4 (the registers of more mixes would limit occupancy)
    const uintptr_t mis = (uintptr_t)a.x | (uintptr_t)a.x_prev | (uintptr_t)a.d_out |
                          (uintptr_t)a.d_xpo | (uintptr_t)a.dx | (uintptr_t)a.dxp;
    const bool vec4 = (a.C % 4 == 0) && (mis % (4 * IO::kBytes) == 0) &&
                      ((uintptr_t)a.mu % 16 == 0) && a.M <= 4;
    const int64_t per_block = 64 * (vec4 ? 4 : 1);
    const int64_t cblocks = (a.C + per_block - 1) / per_block;
    const int64_t nwt = shift_bwd_tiles(a.T);
    if (cblocks > 0x7fffffffLL / nwt || cblocks * nwt > 0x7fffffffLL / a.B)
        return hipErrorInvalidConfiguration;
    hipError_t e = vec4 ? launch_shift_bwd_vec<IO, 4>(a, (uint32_t)cblocks, (uint32_t)nwt, st)
                        : launch_shift_bwd_vec<IO, 1>(a, (uint32_t)cblocks, (uint32_t)nwt, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(shift_bwd_reduce_kernel, dim3((unsigned)((MC + 255) / 256)), dim3(256), 0,
                       st, a.B * nwt, MC, a.part, a.dmu);
    return hipGetLastError();
}

template <class IO>
hipError_t token_shift_io(const ShiftArgs &a, bool in_place_state, hipStream_t st) {
    using T = typename IO::T;
    const int64_t lanes = a.B * a.C;
    const int64_t last_grid = (lanes + 255) / 256;
    if (last_grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    auto launch_last = [&]() {
        hipLaunchKernelGGL(shift_last_kernel<IO>, dim3((unsigned)last_grid), dim3(256), 0, st,
                           a.B, a.T, a.C, (const T *)a.x, (const T *)a.x_prev,
                           (T *)a.x_prev_out);
        return hipGetLastError();
    };
    if (a.T == 0 || a.M == 0) {
        if (!a.x_prev_out || (a.T == 0 && in_place_state)) return hipSuccess;
        return launch_last();
    }
    const uintptr_t mis =
        (uintptr_t)a.x | (uintptr_t)a.x_prev | (uintptr_t)a.out | (uintptr_t)a.x_prev_out;
    const bool vec4 =
        (a.C % 4 == 0) && (mis % (4 * IO::kBytes) == 0) && ((uintptr_t)a.mu % 16 == 0);
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
    hipError_t e =
        vec4 ? launch_shift_vec<IO, 4>(a, (uint32_t)cblocks, (uint32_t)ntiles, write_last, st)
             : launch_shift_vec<IO, 1>(a, (uint32_t)cblocks, (uint32_t)ntiles, write_last, st);
    if (e != hipSuccess || !late) return e;
    return launch_last();
}

}  // namespace

int64_t shift_bwd_tiles(int64_t T) { return (T + kBW * kBT - 1) / (kBW * kBT); }

// B*C > 0 here (the backward also handles T == 0 and B*C == 0).
hipError_t launch_token_shift_backward(const ShiftBwdArgs &a, hipStream_t st) {
    switch (a.io) {
        case kIoF32: return token_shift_backward_io<IoF32>(a, st);
        case kIoF16: return token_shift_backward_io<IoF16>(a, st);
        case kIoBF16: return token_shift_backward_io<IoBF16>(a, st);
        default: return hipErrorInvalidValue;
    }
}

// B*C > 0 here.  M == 0 or T == 0 only update x_prev_out.
hipError_t launch_token_shift(const ShiftArgs &a, bool in_place_state, hipStream_t st) {
    switch (a.io) {
        case kIoF32: return token_shift_io<IoF32>(a, in_place_state, st);
        case kIoF16: return token_shift_io<IoF16>(a, in_place_state, st);
        case kIoBF16: return token_shift_io<IoBF16>(a, in_place_state, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace wkv

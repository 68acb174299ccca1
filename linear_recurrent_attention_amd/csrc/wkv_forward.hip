// wkv_forward.hip -- GPT / RNN-chunk forward kernels of the WKV operator (gfx950).
//
// What is computed (RWKV architecture deep dive, youngju.dev, "WKV mechanism:
// core computation", with the state of "Numerical stability via log-space
// computation" carried in and out as in the rwkv-architecture skill page,
// "Quick start"): for each lane (b, c), y[b][t][c] for t = 0..T-1 and the state
// after the last token.
//
// Two kernels:
//   fwd_lane_kernel  one thread per lane, sequential over T.  Each wave reads
//                    64 consecutive channels of one token row per load (256 B,
//                    coalesced).  Enough parallelism only when B*C is large.
//   fwd_seg_kernel   one workgroup per (sequence b, 64 channels); NW waves, wave
//                    s owns segment s of every tile of NW*LS tokens.  Per tile:
//                    (1) each wave folds its LS tokens into a summary from the
//                    empty state; (2) the NW summaries are scanned across waves
//                    through LDS, composing with the decay 2^{-W len}; (3) each
//                    wave re-sweeps its LS tokens from its prefix state, emitting
//                    y.  k and v stay in registers between (1) and (3), and the
//                    next tile's k and v are loaded while the current one is
//                    processed.  The section "Parallel training formulation"
//                    says the sequence is computed with a scan; this is one.
#include "wkv_device.hpp"
#include "wkv_internal.hpp"

namespace wkv {

// ---------------------------------------------------------------------------
// One thread per lane.
// ---------------------------------------------------------------------------
template <bool SAFE>
__device__ __forceinline__ void lane_sweep(int64_t T, int64_t C, const float *__restrict__ kp,
                                           const float *__restrict__ vp, float *__restrict__ yp,
                                           Lane &L, const Chan &ch) {
    int64_t t = 0;
    constexpr int U8 = 8;
    for (; t + U8 <= T; t += U8) {
        float K[U8], V[U8];
#pragma unroll
        for (int j = 0; j < U8; ++j) {
            K[j] = kp[(t + j) * C];
            V[j] = vp[(t + j) * C];
        }
#pragma unroll
        for (int j = 0; j < U8; ++j) yp[(t + j) * C] = step<SAFE>(L, K[j] * kLog2e, V[j], ch);
    }
    for (; t < T; ++t) yp[t * C] = step<SAFE>(L, kp[t * C] * kLog2e, vp[t * C], ch);
}

__global__ __launch_bounds__(256) void fwd_lane_kernel(int64_t B, int64_t T, int64_t C,
                                                       const float *__restrict__ w,
                                                       const float *__restrict__ u,
                                                       const float *__restrict__ k,
                                                       const float *__restrict__ v,
                                                       float *__restrict__ y,
                                                       const float *__restrict__ s_in,
                                                       float *__restrict__ s_out) {
    const int64_t lane = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const bool active = lane < B * C;
    const int64_t bb = active ? lane / C : 0;
    const int64_t c = active ? lane - bb * C : 0;
    const Chan ch = make_chan(active ? w[c] : 0.0f, active ? u[c] : 0.0f);
    const bool wave_fast = __all(chan_fast_ok(ch));
    if (!active) return;

    Lane L = lane_empty();
    if (s_in)
        L = lane_at(s_in[(0 * B + bb) * C + c], s_in[(1 * B + bb) * C + c],
                    o_in(s_in[(2 * B + bb) * C + c]));
    const int64_t base = bb * T * C + c;
    if (wave_fast)
        lane_sweep<false>(T, C, k + base, v + base, y + base, L, ch);
    else
        lane_sweep<true>(T, C, k + base, v + base, y + base, L, ch);
    if (s_out) {
        s_out[(0 * B + bb) * C + c] = L.a;
        s_out[(1 * B + bb) * C + c] = L.b;
        s_out[(2 * B + bb) * C + c] = o_out(lane_o(L, ch.W));
    }
}

// ---------------------------------------------------------------------------
// Segmented two-pass scan, one workgroup per (b, 64 channels).
// ---------------------------------------------------------------------------
template <int NW, int LS>
struct SegShared {
    float v[2][4][NW][64];  // ping-pong buffers of segment summaries (a, b, e0, n)

    __device__ __forceinline__ void put(int buf, int s, int lane, const Lane &L) {
        v[buf][0][s][lane] = L.a;
        v[buf][1][s][lane] = L.b;
        v[buf][2][s][lane] = L.e0;
        v[buf][3][s][lane] = L.n;
    }
    __device__ __forceinline__ Lane get(int buf, int s, int lane) const {
        return Lane{v[buf][0][s][lane], v[buf][1][s][lane], v[buf][2][s][lane], v[buf][3][s][lane]};
    }
};

// This wave's LS tokens of one tile: rows t0..t0+LS-1 of a [T][C] sequence,
// seen through a wave-uniform buffer descriptor based at row t0.  Row j is at
// the scalar offset j*C*4 and the lane's channel at the vector offset, so a
// load is one buffer_load_dword with no per-lane 64-bit address.
template <int LS, bool FULL>
__device__ __forceinline__ void seg_load(float (&K)[LS], float (&V)[LS], const TileRows &kr,
                                         const TileRows &vr, int64_t t0, int64_t T) {
    if (FULL || t0 + LS <= T) {
#pragma unroll
        for (int j = 0; j < LS; ++j) {
            K[j] = kr.ld(j);
            V[j] = vr.ld(j);
        }
    } else {
#pragma unroll
        for (int j = 0; j < LS; ++j) {
            // wave-uniform condition: rows past the end are never read
            K[j] = (t0 + j < T) ? kr.ld(j) : 0.0f;
            V[j] = (t0 + j < T) ? vr.ld(j) : 0.0f;
        }
    }
}

// FULL: T is a whole number of tiles, so no token test is needed anywhere (the
// loop body is straight-line code and the next tile's loads stay ahead of the
// current tile's arithmetic); otherwise the last tile is ragged.
template <int NW, int LS, bool SAFE, bool FULL>
__device__ __forceinline__ void seg_body(int64_t B, int64_t T, int64_t C, int64_t bb, int64_t c,
                                         bool active, const Chan &ch, const float *kseq,
                                         const float *vseq, float *yseq, uint32_t voff,
                                         const float *__restrict__ s_in, float *__restrict__ s_out,
                                         SegShared<NW, LS> &sh) {
    constexpr int TT = NW * LS;
    const int lane = threadIdx.x & 63;
    const int s = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // segment = wave
    const int64_t ntiles = (T + TT - 1) / TT;
    const uint32_t rowb = (uint32_t)(C * 4);

    // carry: the state before the current tile
    Lane carry = lane_empty();
    if (s_in && active)
        carry = lane_at(s_in[(0 * B + bb) * C + c], s_in[(1 * B + bb) * C + c],
                        o_in(s_in[(2 * B + bb) * C + c]));

    float Kc[LS], Vc[LS];
    {
        const int64_t t0 = (int64_t)s * LS;
        seg_load<LS, FULL>(Kc, Vc, TileRows(kseq + t0 * C, voff, rowb),
                           TileRows(vseq + t0 * C, voff, rowb), t0, T);
    }

    for (int64_t tile = 0; tile < ntiles; ++tile) {
        const int64_t t0 = tile * TT + (int64_t)s * LS;
        float Kn[LS], Vn[LS];
        if (tile + 1 < ntiles)
            seg_load<LS, FULL>(Kn, Vn, TileRows(kseq + (t0 + TT) * C, voff, rowb),
                               TileRows(vseq + (t0 + TT) * C, voff, rowb), t0 + TT, T);

        // (1) summary of this segment from the empty state
        Lane S = lane_empty();
        if (FULL || t0 + LS <= T) {
#pragma unroll
            for (int j = 0; j < LS; ++j) absorb(S, Kc[j] * kLog2e, Vc[j], ch);
        } else {
#pragma unroll
            for (int j = 0; j < LS; ++j)
                if (t0 + j < T) absorb(S, Kc[j] * kLog2e, Vc[j], ch);
        }

        // (2) inclusive scan over the NW segments of the tile (Hillis-Steele,
        // ping-pong LDS buffers: one barrier per round)
        int buf = 0;
#pragma unroll
        for (int d = 1; d < NW; d <<= 1) {
            sh.put(buf, s, lane, S);
            __syncthreads();
            if (s >= d) {
                Lane X = sh.get(buf, s - d, lane);
                compose(X, S, ch.W, (float)(d * LS));
                S = X;
            }
            buf ^= 1;
        }
        sh.put(buf, s, lane, S);
        __syncthreads();
        // state at the start of this segment: carry, then segments 0..s-1
        Lane R = carry;
        if (s > 0) compose(R, sh.get(buf, s - 1, lane), ch.W, (float)(s * LS));
        // carry for the next tile: carry, then the whole tile
        compose(carry, sh.get(buf, NW - 1, lane), ch.W, (float)TT);

        // (3) re-sweep from the prefix state, emitting y
        const TileRows yr(yseq + t0 * C, voff, rowb);
        if (FULL || t0 + LS <= T) {
#pragma unroll
            for (int j = 0; j < LS; ++j) {
                const float yv = step<SAFE>(R, Kc[j] * kLog2e, Vc[j], ch);
                if (active) yr.st(j, yv);
            }
        } else {
#pragma unroll
            for (int j = 0; j < LS; ++j)
                if (t0 + j < T) {
                    const float yv = step<SAFE>(R, Kc[j] * kLog2e, Vc[j], ch);
                    if (active) yr.st(j, yv);
                }
        }
        // the wave holding token T-1 writes the final state
        if (s_out && active && t0 <= T - 1 && T - 1 < t0 + LS) {
            s_out[(0 * B + bb) * C + c] = R.a;
            s_out[(1 * B + bb) * C + c] = R.b;
            s_out[(2 * B + bb) * C + c] = o_out(lane_o(R, ch.W));
        }
#pragma unroll
        for (int j = 0; j < LS; ++j) {
            Kc[j] = Kn[j];
            Vc[j] = Vn[j];
        }
    }
}

template <int NW, int LS>
__global__ __launch_bounds__(NW * 64) void fwd_seg_kernel(int64_t B, int64_t T, int64_t C,
                                                          const float *__restrict__ w,
                                                          const float *__restrict__ u,
                                                          const float *__restrict__ k,
                                                          const float *__restrict__ v,
                                                          float *__restrict__ y,
                                                          const float *__restrict__ s_in,
                                                          float *__restrict__ s_out) {
    __shared__ SegShared<NW, LS> sh;
    const int64_t ngroups = (C + 63) / 64;
    const int64_t g = blockIdx.x % ngroups;
    const int64_t bb = blockIdx.x / ngroups;
    const int lane = threadIdx.x & 63;
    const int64_t c = g * 64 + lane;
    const bool active = c < C;
    const Chan ch = make_chan(active ? w[c] : 0.0f, active ? u[c] : 0.0f);
    // the choice is uniform over the workgroup (all waves share the channels)
    const bool fast = __syncthreads_and(chan_fast_ok(ch));
    // wave-uniform base of this (sequence, channel group); inactive lanes read
    // the group's first channel and never store
    const int64_t base = bb * T * C + g * 64;
    const uint32_t voff = active ? (uint32_t)lane * 4u : 0u;
    const bool full = T % (NW * LS) == 0;
    if (fast && full)
        seg_body<NW, LS, false, true>(B, T, C, bb, c, active, ch, k + base, v + base, y + base,
                                      voff, s_in, s_out, sh);
    else if (fast)
        seg_body<NW, LS, false, false>(B, T, C, bb, c, active, ch, k + base, v + base, y + base,
                                       voff, s_in, s_out, sh);
    else if (full)
        seg_body<NW, LS, true, true>(B, T, C, bb, c, active, ch, k + base, v + base, y + base,
                                     voff, s_in, s_out, sh);
    else
        seg_body<NW, LS, true, false>(B, T, C, bb, c, active, ch, k + base, v + base, y + base,
                                      voff, s_in, s_out, sh);
}

// ---------------------------------------------------------------------------
// T == 0: state_out <- state_in, or the empty state.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void state_copy_kernel(int64_t n, const float *__restrict__ s_in,
                                                         float *__restrict__ s_out) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= 3 * n) return;
    float x;
    if (s_in)
        x = s_in[i];
    else
        x = (i < 2 * n) ? 0.0f : -1.0e38f;
    s_out[i] = x;
}

// ---------------------------------------------------------------------------
// Launchers.
// ---------------------------------------------------------------------------
hipError_t launch_forward_lane(const FwdArgs &a, hipStream_t st) {
    const int64_t lanes = a.B * a.C;
    const int64_t grid = (lanes + 255) / 256;
    hipLaunchKernelGGL(fwd_lane_kernel, dim3((unsigned)grid), dim3(256), 0, st, a.B, a.T, a.C,
                       a.w, a.u, a.k, a.v, a.y, a.s_in, a.s_out);
    return hipGetLastError();
}

template <int NW, int LS>
static hipError_t launch_seg(const FwdArgs &a, hipStream_t st) {
    const int64_t grid = a.B * ((a.C + 63) / 64);
    hipLaunchKernelGGL((fwd_seg_kernel<NW, LS>), dim3((unsigned)grid), dim3(NW * 64), 0, st, a.B,
                       a.T, a.C, a.w, a.u, a.k, a.v, a.y, a.s_in, a.s_out);
    return hipGetLastError();
}

// Compiled (segments, seg_len) variants of the segmented kernel.
bool forward_seg_supported(int nw, int ls) {
    switch (nw * 1000 + ls) {
        case 16008: case 16016: case 8016: case 8032: case 4032:
            return true;
        default:
            return false;
    }
}

hipError_t launch_forward_seg(const FwdArgs &a, int nw, int ls, hipStream_t st) {
    switch (nw * 1000 + ls) {
        case 16008: return launch_seg<16, 8>(a, st);
        case 16016: return launch_seg<16, 16>(a, st);
        case 8016: return launch_seg<8, 16>(a, st);
        case 8032: return launch_seg<8, 32>(a, st);
        case 4032: return launch_seg<4, 32>(a, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_state_copy(int64_t lanes, const float *s_in, float *s_out, hipStream_t st) {
    const int64_t grid = (3 * lanes + 255) / 256;
    hipLaunchKernelGGL(state_copy_kernel, dim3((unsigned)grid), dim3(256), 0, st, lanes, s_in,
                       s_out);
    return hipGetLastError();
}

}  // namespace wkv

// wkv_forward.hip -- GPT / RNN-chunk forward kernels of the WKV operator (gfx950).
//
// What is computed (RWKV architecture deep dive, youngju.dev, "WKV mechanism:
// core computation", with the state of "Numerical stability via log-space
// computation" carried in and out as in the rwkv-architecture skill page,
// "Quick start"): for each lane (b, c), y[b][t][c] for t = 0..T-1 and the state
// after the last token.  Given a receptance tensor r (layout of k), every
// kernel stores the time-mixing block's gated output sigmoid(r) * wkv instead
// (block figure of "RWKV architecture overview"); r is read with k and v.
//
// Two kernels:
//   fwd_lane_kernel  one thread per lane, sequential over T.  Each wave reads
//                    64 consecutive channels of one token row per load (256 B,
//                    coalesced).  Enough parallelism only when B*C is large.
//   fwd_seg_kernel   one workgroup per (sequence b, CW channels: 64, 32 or 16);
//                    NW waves, each wave holding 64/CW segments side by side,
//                    so that a tile of NSEG = NW*64/CW segments of LS tokens
//                    is covered.  Per tile: (1) each segment's tokens fold into
//                    a summary from the empty state; (2) the NSEG summaries are
//                    scanned through LDS, composing with the decay 2^{-W len};
//                    (3) each segment is re-swept from its prefix state,
//                    emitting y.  k and v stay in registers between (1) and
//                    (3), and the next tile's k and v are loaded while the
//                    current one is processed.  The section "Parallel training
//                    formulation" says the sequence is computed with a scan;
//                    this is one.
// Every forward kernel can also store the state before every 128th token
// (checkpoints, for a backward that starts from them): in the lane kernel
// every 128 tokens of the sweep, in the segmented and look-back kernels where
// a segment's re-sweep starts on such a token.
#include "wkv_device.hpp"
#include "wkv_internal.hpp"

namespace wkv {

// ---------------------------------------------------------------------------
// One thread per lane.
// ---------------------------------------------------------------------------
// GATE: y = sigmoid(r) * wkv with r read beside k and v.  IO: element format.
// ck: NULL, or where the state before every token t = i * kCkptTokens (i >= 1)
// goes, as checkpoint i - 1 of lane `li` among n lanes.
template <bool SAFE, bool GATE, class IO>
__device__ __forceinline__ void lane_sweep(int64_t T, int64_t C,
                                           const typename IO::T *__restrict__ kp,
                                           const typename IO::T *__restrict__ vp,
                                           const typename IO::T *__restrict__ rp,
                                           typename IO::T *__restrict__ yp, Lane &L,
                                           const Chan &ch, float *ck, int64_t n, int64_t li) {
    int64_t t = 0;
    constexpr int U8 = 8;
    static_assert(kCkptTokens % U8 == 0, "checkpoints fall on whole groups of tokens");
    auto checkpoint = [&]() {
        if (ck && t > 0 && t % kCkptTokens == 0)
            store_state(ck + (t / kCkptTokens - 1) * 3 * n, n, li, L, ch.W, 0.0f);
    };
    for (; t + U8 <= T; t += U8) {
        checkpoint();
        float K[U8], V[U8], R[U8];
#pragma unroll
        for (int j = 0; j < U8; ++j) {
            K[j] = IO::to_f(kp[(t + j) * C]);
            V[j] = IO::to_f(vp[(t + j) * C]);
            if constexpr (GATE) R[j] = IO::to_f(rp[(t + j) * C]);
        }
#pragma unroll
        for (int j = 0; j < U8; ++j) {
            float yv = step<SAFE>(L, K[j] * kLog2e, V[j], ch);
            if constexpr (GATE) yv *= gate_of(R[j]);
            yp[(t + j) * C] = IO::from_f(yv);
        }
    }
    for (; t < T; ++t) {
        checkpoint();
        float yv = step<SAFE>(L, IO::to_f(kp[t * C]) * kLog2e, IO::to_f(vp[t * C]), ch);
        if constexpr (GATE) yv *= gate_of(IO::to_f(rp[t * C]));
        yp[t * C] = IO::from_f(yv);
    }
}

template <bool GATE, class IO>
__global__ __launch_bounds__(256) void fwd_lane_kernel(int64_t B, int64_t T, int64_t C,
                                                       const float *__restrict__ w,
                                                       const float *__restrict__ u,
                                                       const typename IO::T *__restrict__ k,
                                                       const typename IO::T *__restrict__ v,
                                                       const typename IO::T *__restrict__ r,
                                                       typename IO::T *__restrict__ y,
                                                       const float *__restrict__ s_in,
                                                       float *__restrict__ s_out,
                                                       float *__restrict__ ck) {
    const int64_t lane = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const bool active = lane < B * C;
    const int64_t bb = active ? lane / C : 0;
    const int64_t c = active ? lane - bb * C : 0;
    const Chan ch = make_chan(active ? w[c] : 0.0f, active ? u[c] : 0.0f);
    const bool wave_fast = __all(chan_fast_ok(ch));
    if (!active) return;

    Lane L = lane_empty();
    if (s_in)
        L = lane_in(s_in[(0 * B + bb) * C + c], s_in[(1 * B + bb) * C + c],
                    o_in(s_in[(2 * B + bb) * C + c]));
    const int64_t base = bb * T * C + c;
    const typename IO::T *rp = GATE ? r + base : nullptr;
    if (wave_fast)
        lane_sweep<false, GATE, IO>(T, C, k + base, v + base, rp, y + base, L, ch, ck, B * C,
                                    lane);
    else
        lane_sweep<true, GATE, IO>(T, C, k + base, v + base, rp, y + base, L, ch, ck, B * C,
                                   lane);
    if (s_out) {
        s_out[(0 * B + bb) * C + c] = L.a;
        s_out[(1 * B + bb) * C + c] = L.b;
        s_out[(2 * B + bb) * C + c] = o_out(lane_o(L, ch.W));
    }
}

// ---------------------------------------------------------------------------
// Segmented two-pass scan, one workgroup per (b, CW channels).
//
// A wave's 64 lanes are SPW = 64/CW segments of CW channels (lane = subsegment
// * CW + channel), and the NW waves hold NSEG = NW*SPW consecutive segments of
// LS tokens: a tile of NSEG*LS tokens.  With lane index l in wave w, the LDS
// slot of (segment, channel) is simply w*64 + l, and segment s - d sits d*CW
// slots below.  CW = 64 reads one 256-byte row per wave instruction; CW = 32
// reads two 128-byte row pieces and gives twice as many workgroups, which lets
// several workgroups share a CU and overlap each other's phases when B*C is
// small.
// ---------------------------------------------------------------------------
template <int NW>
struct SegShared {
    float v[2][4][NW * 64];  // ping-pong buffers of segment summaries (a, b, e0, n)

    __device__ __forceinline__ void put(int buf, int slot, const Lane &L) {
        v[buf][0][slot] = L.a;
        v[buf][1][slot] = L.b;
        v[buf][2][slot] = L.e0;
        v[buf][3][slot] = L.n;
    }
    __device__ __forceinline__ Lane get(int buf, int slot) const {
        return Lane{v[buf][0][slot], v[buf][1][slot], v[buf][2][slot], v[buf][3][slot]};
    }
};

// This lane's LS tokens of one tile, rows t0.. of its segment (rows past the end
// of the sequence are not read and hold 0).
template <int LS, bool FULL, class TR>
__device__ __forceinline__ void seg_load(float (&K)[LS], float (&V)[LS], const TR &kr,
                                         const TR &vr, int64_t t0, int64_t T) {
    if (FULL || t0 + LS <= T) {
#pragma unroll
        for (int j = 0; j < LS; ++j) {
            K[j] = kr.ld(j);
            V[j] = vr.ld(j);
        }
    } else {
#pragma unroll
        for (int j = 0; j < LS; ++j) {
            K[j] = (t0 + j < T) ? kr.ld(j) : 0.0f;
            V[j] = (t0 + j < T) ? vr.ld(j) : 0.0f;
        }
    }
}

// The same rows of the gate's receptance.
template <int LS, bool FULL, class TR>
__device__ __forceinline__ void seg_load_r(float (&R)[LS], const TR &rr, int64_t t0,
                                           int64_t T) {
#pragma unroll
    for (int j = 0; j < LS; ++j) R[j] = (FULL || t0 + j < T) ? rr.ld(j) : 0.0f;
}

// Per-lane geometry of the segmented kernel.
template <int NW, int LS, int CW>
struct SegGeom {
    static constexpr int SPW = 64 / CW;      // segments per wave
    static constexpr int NSEG = NW * SPW;    // segments per tile
    static constexpr int TT = NSEG * LS;     // tokens per tile
    int lane;     // 0..63
    int wave;     // wave-uniform
    int seg;      // this lane's segment within the tile
    int slot;     // LDS slot: wave * 64 + lane
};

// One tile: this lane's LS tokens of k, v are in registers (K, V); `carry` is
// the state before the tile and leaves as the state after it.  FULL: T is a
// whole number of tiles, so no token test is needed (straight-line code).
template <int NW, int LS, int CW, bool SAFE, bool FULL, bool GATE, class IO>
__device__ __forceinline__ void seg_tile(int64_t tile, const float (&K)[LS], const float (&V)[LS],
                                         const float (&Rg)[GATE ? LS : 1], Lane &carry, const SegGeom<NW, LS, CW> &G, int64_t B,
                                         int64_t T, int64_t C, int64_t bb, int64_t c, bool active,
                                         const Chan &ch, typename IO::T *yseq, uint32_t voff,
                                         float *__restrict__ s_out, float *__restrict__ ck,
                                         SegShared<NW> &sh) {
    using Geo = SegGeom<NW, LS, CW>;
    const int64_t t0 = tile * Geo::TT + (int64_t)G.seg * LS;

    // (1) summary of this segment from the empty state
    Lane S = lane_empty();
    if (FULL || t0 + LS <= T) {
#pragma unroll
        for (int j = 0; j < LS; ++j) absorb(S, K[j] * kLog2e, V[j], ch);
    } else {
#pragma unroll
        for (int j = 0; j < LS; ++j)
            if (t0 + j < T) absorb(S, K[j] * kLog2e, V[j], ch);
    }

    // (2) inclusive scan over the NSEG segments of the tile (Hillis-Steele,
    // ping-pong LDS buffers: one barrier per round)
    int buf = 0;
#pragma unroll
    for (int d = 1; d < Geo::NSEG; d <<= 1) {
        sh.put(buf, G.slot, S);
        __syncthreads();
        if (G.seg >= d) {
            Lane X = sh.get(buf, G.slot - d * CW);
            compose(X, S, ch.W, (float)(d * LS));
            S = X;
        }
        buf ^= 1;
    }
    sh.put(buf, G.slot, S);
    __syncthreads();
    // state at the start of this segment: carry, then segments 0..seg-1
    Lane R = carry;
    if (G.seg > 0) compose(R, sh.get(buf, G.slot - CW), ch.W, (float)(G.seg * LS));
    // carry for the next tile: carry, then the whole tile
    compose(carry, sh.get(buf, (Geo::NSEG - 1) * CW + (G.lane % CW)), ch.W, (float)Geo::TT);
    // a segment that starts on a checkpoint token stores its starting state
    static_assert(kCkptTokens % LS == 0, "checkpoints fall on segment starts");
    if (ck && active && t0 > 0 && t0 < T && t0 % kCkptTokens == 0)
        store_state(ck + (t0 / kCkptTokens - 1) * 3 * B * C, B * C, bb * C + c, R, ch.W, 0.0f);

    // (3) re-sweep from the prefix state, emitting y
    const int64_t tw = tile * Geo::TT + (int64_t)G.wave * Geo::SPW * LS;  // wave's first row
    const TileRowsT<IO> yr(yseq + tw * C, voff, (uint32_t)(C * IO::kBytes));
    if (FULL || t0 + LS <= T) {
#pragma unroll
        for (int j = 0; j < LS; ++j) {
            float yv = step<SAFE>(R, K[j] * kLog2e, V[j], ch);
            if constexpr (GATE) yv *= gate_of(Rg[j]);
            if (active) yr.st(j, yv);
        }
    } else {
#pragma unroll
        for (int j = 0; j < LS; ++j)
            if (t0 + j < T) {
                float yv = step<SAFE>(R, K[j] * kLog2e, V[j], ch);
                if constexpr (GATE) yv *= gate_of(Rg[j]);
                if (active) yr.st(j, yv);
            }
    }
    // the lane holding token T-1 writes the final state
    if (s_out && active && t0 <= T - 1 && T - 1 < t0 + LS) {
        s_out[(0 * B + bb) * C + c] = R.a;
        s_out[(1 * B + bb) * C + c] = R.b;
        s_out[(2 * B + bb) * C + c] = o_out(lane_o(R, ch.W));
    }
}

// The whole sequence of one (b, CW-channel group): tiles in order, with the
// next tile's k, v loaded while the current one is processed.  Two register
// sets take turns (A holds even tiles, B odd ones) so that no register copy
// ties a prefetch to the current tile's arithmetic.
template <int NW, int LS, int CW, bool SAFE, bool FULL, bool GATE, class IO>
__device__ __forceinline__ void seg_body(int64_t B, int64_t T, int64_t C, int64_t bb, int64_t c,
                                         bool active, const Chan &ch,
                                         const SegGeom<NW, LS, CW> &G, const typename IO::T *kseq,
                                         const typename IO::T *vseq, const typename IO::T *rseq,
                                         typename IO::T *yseq, uint32_t voff,
                                         const float *__restrict__ s_in, float *__restrict__ s_out,
                                         float *__restrict__ ck, SegShared<NW> &sh) {
    using Geo = SegGeom<NW, LS, CW>;
    const int64_t ntiles = (T + Geo::TT - 1) / Geo::TT;
    const uint32_t rowb = (uint32_t)(C * IO::kBytes);
    using TR = TileRowsT<IO>;
    constexpr int NR = GATE ? LS : 1;
    auto load = [&](float (&K)[LS], float (&V)[LS], int64_t tile) {
        const int64_t tw = tile * Geo::TT + (int64_t)G.wave * Geo::SPW * LS;
        seg_load<LS, FULL>(K, V, TR(kseq + tw * C, voff, rowb), TR(vseq + tw * C, voff, rowb),
                           tile * Geo::TT + (int64_t)G.seg * LS, T);
    };
    // The receptance of a tile is loaded just before the next tile's k and v:
    // loads complete in order, so waiting for it in the re-sweep leaves that
    // prefetch in flight, and one register set suffices.
    auto load_r = [&](float (&R)[NR], int64_t tile) {
        if constexpr (GATE) {
            const int64_t tw = tile * Geo::TT + (int64_t)G.wave * Geo::SPW * LS;
            seg_load_r<LS, FULL>(R, TR(rseq + tw * C, voff, rowb),
                                 tile * Geo::TT + (int64_t)G.seg * LS, T);
        } else {
            R[0] = 0.0f;
        }
    };

    // carry: the state before the current tile
    Lane carry = lane_empty();
    if (s_in && active)
        carry = lane_in(s_in[(0 * B + bb) * C + c], s_in[(1 * B + bb) * C + c],
                        o_in(s_in[(2 * B + bb) * C + c]));

    float KA[LS], VA[LS], KB[LS], VB[LS], Rc[NR];
    load(KA, VA, 0);
    int64_t tile = 0;
    for (; tile + 1 < ntiles; tile += 2) {
        load_r(Rc, tile);
        load(KB, VB, tile + 1);
        seg_tile<NW, LS, CW, SAFE, FULL, GATE, IO>(tile, KA, VA, Rc, carry, G, B, T, C, bb, c, active,
                                               ch, yseq, voff, s_out, ck, sh);
        load_r(Rc, tile + 1);
        if (tile + 2 < ntiles) load(KA, VA, tile + 2);
        seg_tile<NW, LS, CW, SAFE, FULL, GATE, IO>(tile + 1, KB, VB, Rc, carry, G, B, T, C, bb, c,
                                               active, ch, yseq, voff, s_out, ck, sh);
    }
    if (tile < ntiles) {
        load_r(Rc, tile);
        seg_tile<NW, LS, CW, SAFE, FULL, GATE, IO>(tile, KA, VA, Rc, carry, G, B, T, C, bb, c, active,
                                               ch, yseq, voff, s_out, ck, sh);
    }
}

template <int NW, int LS, int CW, bool GATE, class IO>
__global__ __launch_bounds__(NW * 64) void fwd_seg_kernel(int64_t B, int64_t T, int64_t C,
                                                          const float *__restrict__ w,
                                                          const float *__restrict__ u,
                                                          const typename IO::T *__restrict__ k,
                                                          const typename IO::T *__restrict__ v,
                                                          const typename IO::T *__restrict__ r,
                                                          typename IO::T *__restrict__ y,
                                                          const float *__restrict__ s_in,
                                                          float *__restrict__ s_out,
                                                          float *__restrict__ ck) {
    using Geo = SegGeom<NW, LS, CW>;
    __shared__ SegShared<NW> sh;
    const int64_t ngroups = (C + CW - 1) / CW;
    const int64_t g = blockIdx.x % ngroups;
    const int64_t bb = blockIdx.x / ngroups;
    Geo G;
    G.lane = threadIdx.x & 63;
    G.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    G.seg = G.wave * Geo::SPW + G.lane / CW;
    G.slot = G.wave * 64 + G.lane;
    const int ch_local = G.lane % CW;
    const int64_t c = g * CW + ch_local;
    const bool active = c < C;
    const Chan ch = make_chan(active ? w[c] : 0.0f, active ? u[c] : 0.0f);
    // the choice is uniform over the workgroup (all waves share the channels)
    const bool fast = __syncthreads_and(chan_fast_ok(ch));
    // wave-uniform base of this (sequence, channel group); each lane adds its
    // channel and, when a wave holds several segments, its segment's rows.
    // Inactive lanes read the group's first channel and never store.
    const int64_t base = bb * T * C + g * CW;
    const uint32_t voff = (active ? (uint32_t)(ch_local * IO::kBytes) : 0u) +
                          (uint32_t)(G.lane / CW) * (uint32_t)LS * (uint32_t)(C * IO::kBytes);
    const bool full = T % Geo::TT == 0;
    const typename IO::T *rs = GATE ? r + base : nullptr;
    if (fast && full)
        seg_body<NW, LS, CW, false, true, GATE, IO>(B, T, C, bb, c, active, ch, G, k + base, v + base,
                                                rs, y + base, voff, s_in, s_out, ck, sh);
    else if (fast)
        seg_body<NW, LS, CW, false, false, GATE, IO>(B, T, C, bb, c, active, ch, G, k + base,
                                                 v + base, rs, y + base, voff, s_in, s_out, ck, sh);
    else if (full)
        seg_body<NW, LS, CW, true, true, GATE, IO>(B, T, C, bb, c, active, ch, G, k + base, v + base,
                                               rs, y + base, voff, s_in, s_out, ck, sh);
    else
        seg_body<NW, LS, CW, true, false, GATE, IO>(B, T, C, bb, c, active, ch, G, k + base, v + base,
                                                rs, y + base, voff, s_in, s_out, ck, sh);
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
template <bool GATE, class IO>
static hipError_t launch_lane(const FwdArgs &a, hipStream_t st) {
    using T = typename IO::T;
    const int64_t grid = (a.B * a.C + 255) / 256;
    hipLaunchKernelGGL((fwd_lane_kernel<GATE, IO>), dim3((unsigned)grid), dim3(256), 0, st, a.B,
                       a.T, a.C, a.w, a.u, (const T *)a.k, (const T *)a.v, (const T *)a.r,
                       (T *)a.y, a.s_in, a.s_out, a.ck);
    return hipGetLastError();
}

template <bool GATE>
static hipError_t launch_lane_io(const FwdArgs &a, hipStream_t st) {
    switch (a.io) {
        case kIoF32: return launch_lane<GATE, IoF32>(a, st);
        case kIoF16: return launch_lane<GATE, IoF16>(a, st);
        case kIoBF16: return launch_lane<GATE, IoBF16>(a, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_forward_lane(const FwdArgs &a, hipStream_t st) {
    return a.r ? launch_lane_io<true>(a, st) : launch_lane_io<false>(a, st);
}

template <int NW, int LS, int CW, bool GATE, class IO>
static hipError_t launch_seg(const FwdArgs &a, hipStream_t st) {
    using T = typename IO::T;
    const int64_t grid = a.B * ((a.C + CW - 1) / CW);
    hipLaunchKernelGGL((fwd_seg_kernel<NW, LS, CW, GATE, IO>), dim3((unsigned)grid),
                       dim3(NW * 64), 0, st, a.B, a.T, a.C, a.w, a.u, (const T *)a.k,
                       (const T *)a.v, (const T *)a.r, (T *)a.y, a.s_in, a.s_out, a.ck);
    return hipGetLastError();
}

template <int NW, int LS, int CW, class IO>
static hipError_t launch_seg_gate(const FwdArgs &a, hipStream_t st) {
    return a.r ? launch_seg<NW, LS, CW, true, IO>(a, st) : launch_seg<NW, LS, CW, false, IO>(a, st);
}

// Compiled variants of the segmented kernel, keyed by (segments per tile,
// tokens per segment, channels per workgroup); the 16-bit formats have the
// default variant only.
#define WKV_SEG_VARIANTS(X)                                                            \
    X(16, 16, 64) X(16, 8, 64) X(8, 16, 64) X(8, 32, 64) X(4, 32, 64) X(16, 16, 32)   \
    X(32, 8, 32) X(16, 8, 32) X(16, 16, 16) X(32, 8, 16)

bool forward_seg_supported(int nseg, int ls, int cw, int io) {
    if (io == kIoF16 || io == kIoBF16) return nseg == 16 && ls == 16 && cw == 64;
    if (io != kIoF32) return false;
#define X(NSEG, LS, CW) if (nseg == NSEG && ls == LS && cw == CW) return true;
    WKV_SEG_VARIANTS(X)
#undef X
    return false;
}

hipError_t launch_forward_seg(const FwdArgs &a, int nseg, int ls, int cw, hipStream_t st) {
    if (!forward_seg_supported(nseg, ls, cw, a.io)) return hipErrorInvalidValue;
    if (a.io == kIoF16) return launch_seg_gate<16, 16, 64, IoF16>(a, st);
    if (a.io == kIoBF16) return launch_seg_gate<16, 16, 64, IoBF16>(a, st);
#define X(NSEG, LS, CW) \
    if (nseg == NSEG && ls == LS && cw == CW) return launch_seg_gate<NSEG * CW / 64, LS, CW, IoF32>(a, st);
    WKV_SEG_VARIANTS(X)
#undef X
    return hipErrorInvalidValue;
}

__global__ __launch_bounds__(256) void zero_fill_kernel(uint32_t *p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
        p[i] = 0u;
}

hipError_t launch_zero_fill(void *p, size_t bytes, hipStream_t st) {
    const size_t n = bytes / 4;
    if (n == 0) return hipSuccess;
    const size_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(zero_fill_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256),
                       0, st, (uint32_t *)p, n);
    return hipGetLastError();
}

hipError_t launch_state_copy(int64_t lanes, const float *s_in, float *s_out, hipStream_t st) {
    const int64_t grid = (3 * lanes + 255) / 256;
    hipLaunchKernelGGL(state_copy_kernel, dim3((unsigned)grid), dim3(256), 0, st, lanes, s_in,
                       s_out);
    return hipGetLastError();
}

}  // namespace wkv

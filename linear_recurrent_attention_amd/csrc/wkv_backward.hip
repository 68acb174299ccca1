// wkv_backward.hip -- gradients dk, dv, dw, du of the GPT-mode WKV forward (gfx950).
//
// The pages give no backward; this differentiates the closed form (RWKV
// architecture deep dive, youngju.dev, "WKV mechanism: core computation"),
// starting from a carried state or the empty one (RNN mode over chunks,
// rwkv-architecture skill page, "Quick start").  With g_t = dy_t, D_t the
// denominator of output t,
// lambda_t = log2 D_t, and for token i the sums over later outputs
//   R_i  = sum_{t>i} g_t 2^{-(t-1-i)W - lambda_t}          S_i  = same with g_t y_t
//   R'_i = sum_{t>i} (t-1-i) g_t 2^{-(t-1-i)W - lambda_t}  S'_i = same with g_t y_t
// the gradients are
//   dv_i = p_ii g_i + e^{k_i} R_i
//   dk_i = p_ii g_i (v_i - y_i) + e^{k_i} (v_i R_i - S_i)
//   dw  -= e^{k_i} (v_i R'_i - S'_i),      du += p_ii g_i (v_i - y_i)
// where p_ii is the weight of token i in its own output.  Stepping from i to
// i-1:  R_{i-1} = g_i 2^{-lambda_i} + 2^{-W} R_i,  R'_{i-1} = 2^{-W} (R'_i + R_i).
// The four sums are kept scaled by 2^rho, where rho tracks max(-lambda_i,
// rho_i - W) within a fixed margin, so that e^{k_i} 2^{rho_i} stays within a
// bounded factor of the largest weight of token i in any later output (at most
// 1) and nothing overflows.
//
// One workgroup owns (sequence b, 64 channels) and the whole sequence, NW waves
// each owning a segment of LS tokens in every tile of NW*LS tokens:
//   phase 1 (tiles forward)  fold k, v into segment summaries, scan them across
//            waves, and store each segment's starting state (a, b, anchor, steps)
//            in the workspace;
//   phase 2 (tiles backward) reload k, v, dy; recompute y, lambda and p_ii from
//            the stored starting state; fold each segment's tokens backward into
//            a local (R, S, R', S', rho) summary; scan the summaries backward
//            across waves (composing over a stretch of len tokens:
//            R = R_early + 2^{-W len} R_late, R' = R'_early + 2^{-W len}(R'_late +
//            len R_late)); re-sweep backward from each segment's suffix state,
//            emitting dk, dv and accumulating dw, du.
// With the forward's checkpoints (the state before every 128th token: one per
// tile) there is no phase 1: phase 2 folds each segment's tokens from the
// empty state, scans the summaries across the waves and starts from the
// tile's checkpoint, which saves reading k and v a second time.
// dw and du: per-thread float sums, combined across waves and then across the
// batch in double precision in a fixed order (deterministic; no atomics).
//
// Carried states.  The state a chunk starts from enters every output like a
// token before t = 0 whose weights are its true sums A0, B0 (numerator,
// denominator) at decay distance t; so, with R_{-1}, S_{-1}, R'_{-1}, S'_{-1}
// the sums after the reverse sweep has passed token 0,
//   dL/dA0 = R_{-1},  dL/dB0 = -S_{-1},  dw -= A0 R'_{-1} - B0 S'_{-1},
// returned in the state's own coordinates (a0, b0, o0): d_a0 = dL/dA0 e^{o0},
// d_b0 = dL/dB0 e^{o0}, d_o0 = d_a0 a0 + d_b0 b0.  An upstream gradient of the
// state handed on, (g_a, g_b) in the coordinates (a_T, b_T, o_T) of that
// state, is an output after the last token with R_{T-1} = g_a e^{-o_T},
// S_{T-1} = -g_b e^{-o_T}: the wave that holds token T-1 starts both its
// segment summary and its re-sweep from it (every later segment of that tile
// is empty, so nothing else sees a position past the end).
#include "wkv_device.hpp"
#include "wkv_internal.hpp"

namespace wkv {

namespace {

constexpr int kBwdNW = 16;
constexpr int kBwdLS = 8;

// Reverse-scan state: the four sums in the frame 2^rho, rho = r0 - m W kept as
// an anchor and a step count (as for the forward Lane: one rounding per use,
// no drift along the sequence).
struct Rev {
    float R, S, R1, S1;
    float r0;  // anchor exponent (log2 units)
    float m;   // decay steps since the anchor
};

__device__ __forceinline__ Rev rev_empty() { return Rev{0.0f, 0.0f, 0.0f, 0.0f, kEmpty2, 0.0f}; }

// Hysteresis of the reverse frame (log2 units): the frame moves only when a new
// term exceeds it by more than 2^kRevHyst.  After a dominant token (k = +60,
// say) every later denominator decays by exactly W per token, in step with the
// frame itself, so "is the new term above the frame" is a tie decided by
// rounding at every token; re-anchoring on each of those ties chains thousands
// of rounded scale factors into the sums (percent-level errors).  With the
// margin the frame holds, the stored sums grow by at most 2^kRevHyst per part
// (2^(2 kRevHyst) after compositions), far inside float range.
constexpr float kRevHyst = 8.0f;

// Fold output token i (gradient g, output y, lambda = log2 D_i) into the sums.
__device__ __forceinline__ void rev_absorb(Rev &z, float g, float y, float lam, float W) {
    const float m1 = z.m + 1.0f;
    // old frame (r0 - m1 W, the sums decayed one step) minus the new term's
    // exponent -lam, anchors first
    const float d = fmaf(-m1, W, z.r0 + lam);
    const bool keep_old = d > -kRevHyst;
    const float E = ex2(keep_old ? -d : d);
    const float fo = keep_old ? 1.0f : E;
    const float fn = keep_old ? E : 1.0f;
    const float gn = fn * g;
    z.R1 = fo * (z.R1 + z.R);
    z.S1 = fo * (z.S1 + z.S);
    z.R = fmaf(fo, z.R, gn);
    z.S = fmaf(fo, z.S, gn * y);
    z.r0 = keep_old ? z.r0 : -lam;
    z.m = keep_old ? m1 : 0.0f;
}

// e <- e (+) l: the sums of a stretch of `len` tokens (e, earlier in time)
// followed by the sums of everything after it (l), seen from before the
// stretch.  l's frame moves by len decay steps, which only extends its anchor's
// step count.
__device__ __forceinline__ void rev_compose(Rev &e, const Rev &l, float W, float len) {
    const float lm = l.m + len;
    // frame of l moved across the stretch minus the frame of e, anchors first
    const float d = fmaf(-(lm - e.m), W, l.r0 - e.r0);
    // keep the later part's frame unless it is smaller by more than the margin:
    // the later part is the long carried sum, which is then never rescaled
    const bool late_big = d > -kRevHyst;
    const float E = ex2(late_big ? -d : d);
    const float fe = late_big ? E : 1.0f;
    const float fl = late_big ? 1.0f : E;
    e.R1 = fmaf(fe, e.R1, fl * fmaf(len, l.R, l.R1));
    e.S1 = fmaf(fe, e.S1, fl * fmaf(len, l.S, l.S1));
    e.R = fmaf(fe, e.R, fl * l.R);
    e.S = fmaf(fe, e.S, fl * l.S);
    e.r0 = late_big ? l.r0 : e.r0;
    e.m = late_big ? lm : e.m;
}

// Summary of LS whole tokens from the empty state in one frame: the largest
// decayed exponent x_t = K_t - (LS-1-t) W of the segment at its last token,
// one exponential per token and no rescaling.
template <int LS>
__device__ __forceinline__ Lane seg_summary_fixed(const float (&K)[LS], const float (&V)[LS],
                                                  float W) {
    float M = -INFINITY;
#pragma unroll
    for (int t = 0; t < LS; ++t) M = fmaxf(M, fmaf((float)(t - (LS - 1)), W, K[t]));
    float sa = 0.0f, sb = 0.0f;
#pragma unroll
    for (int t = 0; t < LS; ++t) {
        const float e = ex2(fmaf((float)(t - (LS - 1)), W, K[t]) - M);
        sa = fmaf(e, V[t], sa);
        sb += e;
    }
    return Lane{sa, sb, M, 0.0f};
}

// Reverse summary of LS whole tokens (outputs t0..t0+LS-1) seen from before
// the first, from the empty state, in one frame: output j enters R with the
// weight 2^{x_j}, x_j = -lambda_j - j W, and R', S' with j times it; the frame
// is the largest x_j, so each token costs one exponential and no rescaling.
template <int LS>
__device__ __forceinline__ Rev rev_summary_fixed(const float (&G)[LS], const float (&Y)[LS],
                                                 const float (&LAM)[LS], float W) {
    float F = -INFINITY;
#pragma unroll
    for (int j = 0; j < LS; ++j) F = fmaxf(F, fmaf(-(float)j, W, -LAM[j]));
    float R = 0.0f, S = 0.0f, R1 = 0.0f, S1 = 0.0f;
#pragma unroll
    for (int j = 0; j < LS; ++j) {
        const float ge = G[j] * ex2(fmaf(-(float)j, W, -LAM[j]) - F);
        const float gy = ge * Y[j];
        R += ge;
        S += gy;
        R1 = fmaf((float)j, ge, R1);
        S1 = fmaf((float)j, gy, S1);
    }
    return Rev{R, S, R1, S1, F, 0.0f};
}

template <int NW>
struct BwdShared {
    float f[2][4][NW][64];
    float r[2][6][NW][64];
    double red[2][NW][64];
    float seed[3][64];  // upstream state gradient: R, S and frame of R_{T-1}
};

template <int NW>
__device__ __forceinline__ void fwd_put(BwdShared<NW> &sh, int buf, int s, int lane, const Lane &L) {
    sh.f[buf][0][s][lane] = L.a;
    sh.f[buf][1][s][lane] = L.b;
    sh.f[buf][2][s][lane] = L.e0;
    sh.f[buf][3][s][lane] = L.n;
}

template <int NW>
__device__ __forceinline__ Lane fwd_get(const BwdShared<NW> &sh, int buf, int s, int lane) {
    return Lane{sh.f[buf][0][s][lane], sh.f[buf][1][s][lane], sh.f[buf][2][s][lane],
                sh.f[buf][3][s][lane]};
}

template <int NW>
__device__ __forceinline__ void rev_put(BwdShared<NW> &sh, int buf, int s, int lane, const Rev &z) {
    sh.r[buf][0][s][lane] = z.R;
    sh.r[buf][1][s][lane] = z.S;
    sh.r[buf][2][s][lane] = z.R1;
    sh.r[buf][3][s][lane] = z.S1;
    sh.r[buf][4][s][lane] = z.r0;
    sh.r[buf][5][s][lane] = z.m;
}

template <int NW>
__device__ __forceinline__ Rev rev_get(const BwdShared<NW> &sh, int buf, int s, int lane) {
    return Rev{sh.r[buf][0][s][lane], sh.r[buf][1][s][lane], sh.r[buf][2][s][lane],
               sh.r[buf][3][s][lane], sh.r[buf][4][s][lane], sh.r[buf][5][s][lane]};
}

// LS rows t0.. of one tensor through a wave-uniform descriptor (rows past the
// end of the sequence are not read and hold 0).
template <int LS, class TR>
__device__ __forceinline__ void load_seg(float (&X)[LS], const TR &r, int64_t t0, int64_t T) {
    if (t0 + LS <= T) {
#pragma unroll
        for (int j = 0; j < LS; ++j) X[j] = r.ld(j);
    } else {
#pragma unroll
        for (int j = 0; j < LS; ++j) X[j] = (t0 + j < T) ? r.ld(j) : 0.0f;
    }
}

// Forward token for the recompute: y, lambda = log2 D and the own weight p_ii.
template <bool SAFE>
__device__ __forceinline__ void fwd_token(Lane &L, float K, float v, const Chan &ch, float &y,
                                          float &lam, float &pii) {
    const float o = lane_o(L, ch.W);  // frame of the past sums before this token
    const float n1 = L.n + 1.0f;
    const float s = fmaf(n1, ch.W, K - L.e0);
    const float E = ex2(-fabsf(s));
    const bool pos = s > 0.0f;
    const float P = pos ? E : 1.0f;
    const float Q = pos ? 1.0f : E;
    if constexpr (!SAFE) {
        const float aP = L.a * P, bP = L.b * P, Qc = Q * ch.c1;
        const float den = bP + Qc;
        const float r = rcp(den);
        y = fmaf(Qc, v, aP) * r;
        pii = Qc * r;
        // D = 2^{o} (b + c1 2^s) = 2^{max(h, K) + W} den
        lam = (pos ? K + ch.W : o) + lg2(den);
    } else {
        const float x = fmaf(L.n, ch.W, (ch.U + K) - L.e0);
        const float F = ex2(-fabsf(x));
        const bool px = x > 0.0f;
        const float Pp = px ? F : 1.0f, Qq = px ? 1.0f : F;
        const float den = fmaf(L.b, Pp, Qq);
        const float r = rcp(den);
        y = fmaf(Qq, v, L.a * Pp) * r;
        pii = Qq * r;
        // D = 2^{max(o, U + K)} den
        lam = fmaxf(o, ch.U + K) + lg2(den);
    }
    L.a = fmaf(L.a, P, Q * v);
    L.b = fmaf(L.b, P, Q);
    L.e0 = pos ? K : L.e0;
    L.n = pos ? 0.0f : n1;
}

// IO: element format of k, v, dy, dk and dv (the states, w, u, dw, du and all
// arithmetic are float32).  FULL: T is a whole number of tiles, so no token
// needs a bounds test.  CK: the forward's checkpoints `cks` hold the state at
// the start of every tile but the first; there is no phase 1, and each tile's
// segment starting states are rebuilt in phase 2 by the same scan, from the
// tile's checkpoint (or state_in).  GATE: the forward's output was
// sigmoid(r) * wkv and dy its gradient; the recurrence's upstream gradient is
// g = dy sigmoid(r), and dr = g wkv (1 - sigmoid(r)) is stored as well.
template <int NW, int LS, bool SAFE, bool FULL, bool CK, bool GATE, class IO>
__device__ __forceinline__ void bwd_body(int64_t B, int64_t T, int64_t C, int64_t bb, int64_t c,
                                         bool active, const Chan &ch,
                                         const typename IO::T *kseq, const typename IO::T *vseq,
                                         const typename IO::T *gseq, typename IO::T *dkseq,
                                         typename IO::T *dvseq, const typename IO::T *rseq,
                                         typename IO::T *drseq, uint32_t voff,
                                         float *__restrict__ ck,
                                         double *__restrict__ part, const float *s_in,
                                         const float *s_out, const float *ds_out, float *ds_in,
                                         const float *cks, BwdShared<NW> &sh) {
    constexpr int TT = NW * LS;
    static_assert(!CK || TT == kCkptTokens, "one checkpoint per tile");
    const int lane = threadIdx.x & 63;
    const int s = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t rowb = (uint32_t)(C * IO::kBytes);
    auto rows = [&](const typename IO::T *seq, int64_t t0) {
        return TileRowsT<IO>(seq + t0 * C, voff, rowb);
    };
    const int64_t ntiles = (T + TT - 1) / TT;

    // ---------------- phase 1: starting state of every segment ----------------
    if constexpr (!CK) {
        // the carried state: every wave folds it into its segments' starting states
        Lane carry = lane_empty();
        if (s_in && active)
            carry = lane_in(s_in[(0 * B + bb) * C + c], s_in[(1 * B + bb) * C + c],
                            o_in(s_in[(2 * B + bb) * C + c]));
        // keys in log2 units, scaled where each prefetched tile is handed over
        float Kc[LS], Vc[LS];
        load_seg<LS>(Kc, rows(kseq, (int64_t)s * LS), (int64_t)s * LS, T);
        load_seg<LS>(Vc, rows(vseq, (int64_t)s * LS), (int64_t)s * LS, T);
#pragma unroll
        for (int j = 0; j < LS; ++j) Kc[j] *= kLog2e;
        // the scan's LDS buffers alternate from tile to tile, so that a wave's
        // first write of a tile never meets another wave's last read of the
        // previous tile (no barrier lies between them)
        int buf = 0;
        for (int64_t tile = 0; tile < ntiles; ++tile) {
            const int64_t t0 = tile * TT + (int64_t)s * LS;
            float Kn[LS], Vn[LS];
            if (tile + 1 < ntiles) {
                load_seg<LS>(Kn, rows(kseq, t0 + TT), t0 + TT, T);
                load_seg<LS>(Vn, rows(vseq, t0 + TT), t0 + TT, T);
            }
            Lane S = lane_empty();
            if constexpr (FULL) {
                S = seg_summary_fixed<LS>(Kc, Vc, ch.W);
            } else {
#pragma unroll
                for (int j = 0; j < LS; ++j)
                    if (t0 + j < T) absorb(S, Kc[j], Vc[j], ch);
            }
#pragma unroll
            for (int d = 1; d < NW; d <<= 1) {
                fwd_put(sh, buf, s, lane, S);
                __syncthreads();
                if (s >= d) {
                    Lane X = fwd_get(sh, buf, s - d, lane);
                    compose(X, S, ch.W, (float)(d * LS));
                    S = X;
                }
                buf ^= 1;
            }
            fwd_put(sh, buf, s, lane, S);
            __syncthreads();
            Lane R = carry;
            if (s > 0) compose(R, fwd_get(sh, buf, s - 1, lane), ch.W, (float)(s * LS));
            compose(carry, fwd_get(sh, buf, NW - 1, lane), ch.W, (float)TT);
            buf ^= 1;
            float *q = ck + ((tile * NW + s) * 4) * 64 + lane;
            q[0] = R.a;
            q[64] = R.b;
            q[128] = R.e0;
            q[192] = R.n;
#pragma unroll
            for (int j = 0; j < LS; ++j) {
                Kc[j] = Kn[j] * kLog2e;
                Vc[j] = Vn[j];
            }
        }
    }

    // ---------------- phase 2: tiles in reverse ----------------
    // dw's terms are e^{k_i} times sums kept within 2^16 of their frame.  Where
    // the bonus dominates every output (U - W beyond the one-exponential range)
    // all weights of earlier tokens are near 2^{-U}, so that factor can fall
    // below float's normal range, where the hardware exp2 flushes to zero,
    // while the terms it scales make up the whole of dw.  On that path the
    // factor is formed 2^{dwx} larger (dwx from U - W, at most 64) and dw is
    // accumulated at that scale, which stays far inside the float range: each
    // term is a weight of at most 1 times (t-1-i) g (v - y), so a lane's sum is
    // below T^2 max|g| (|v| + |y|) before the factor 2^{dwx}.
    float dwx = 0.0f, dws = 1.0f;
    if constexpr (SAFE) {
        dwx = fminf(fmaxf(rintf(ch.U - ch.W) - 64.0f, 0.0f), 64.0f);
        dws = ex2(-dwx);
    }
    float dw_acc = 0.0f, du_acc = 0.0f;
    Rev carry = rev_empty();
    // the upstream state gradient as R_{T-1}, S_{T-1} (frame -o_T), staged in
    // LDS so that nothing stays live across the tile loop
    if (ds_out) {
        if (s == 0) {
            float ga = 0.0f, gb = 0.0f, r0 = kEmpty2;
            if (active) {
                // (a zero gradient keeps the empty frame: zero sums in a large
                // frame would rescale the real sums toward underflow)
                const float o2T = o_in(s_out[(2 * B + bb) * C + c]);
                const float a_ = ds_out[(0 * B + bb) * C + c], b_ = ds_out[(1 * B + bb) * C + c];
                if (o2T > kEmpty2 && (a_ != 0.0f || b_ != 0.0f)) {
                    ga = a_;
                    gb = b_;
                    r0 = -o2T;
                }
            }
            sh.seed[0][lane] = ga;
            sh.seed[1][lane] = -gb;
            sh.seed[2][lane] = r0;
        }
        __syncthreads();
    }
    auto seed_of = [&]() {
        return Rev{sh.seed[0][lane], sh.seed[1][lane], 0.0f, 0.0f, sh.seed[2][lane], 0.0f};
    };
    // Kc holds the keys in log2 units (k log2 e): the scaling takes the place
    // of the register copy that hands each prefetched tile over.  k and v of
    // the next tile are prefetched; dy is loaded at the top of its own tile,
    // ahead of that prefetch (loads complete in order), and is first needed
    // after the forward recompute, which covers its latency.  Prefetching it
    // as well held 8 more registers across the tile and made the kernel spill.
    float Kc[LS], Vc[LS], Gc[LS];
    {
        const int64_t t0 = (ntiles - 1) * TT + (int64_t)s * LS;
        load_seg<LS>(Kc, rows(kseq, t0), t0, T);
        load_seg<LS>(Vc, rows(vseq, t0), t0, T);
#pragma unroll
        for (int j = 0; j < LS; ++j) Kc[j] *= kLog2e;
    }
    int rb = 0;  // LDS buffer the next reverse scan starts in (alternating as in phase 1)
    for (int64_t tile = ntiles - 1; tile >= 0; --tile) {
        const int64_t t0 = tile * TT + (int64_t)s * LS;
        load_seg<LS>(Gc, rows(gseq, t0), t0, T);
        float Kn[LS], Vn[LS];
        if (tile > 0) {
            load_seg<LS>(Kn, rows(kseq, t0 - TT), t0 - TT, T);
            load_seg<LS>(Vn, rows(vseq, t0 - TT), t0 - TT, T);
        }
        // the receptance of this tile (used once the forward is recomputed)
        float Rc[GATE ? LS : 1];
        if constexpr (GATE) load_seg<LS>(Rc, rows(rseq, t0), t0, T);
        // forward recompute of y, lambda, p_ii from the segment's starting state
        float Y[LS], LAM[LS], PII[LS];
        {
            Lane L;
            if constexpr (CK) {
                // the tile's starting state: state_in for the first tile, else
                // the checkpoint before it
                const float *src = tile == 0 ? s_in : cks + (tile - 1) * 3 * B * C;
                float a0 = 0.0f, b0 = 0.0f, o0 = kEmpty2;
                if (src && active) {
                    a0 = src[(0 * B + bb) * C + c];
                    b0 = src[(1 * B + bb) * C + c];
                    o0 = o_in(src[(2 * B + bb) * C + c]);
                }
                // this segment's summary, scanned over the tile's segments
                Lane S = lane_empty();
                if constexpr (FULL) {
                    S = seg_summary_fixed<LS>(Kc, Vc, ch.W);
                } else {
#pragma unroll
                    for (int j = 0; j < LS; ++j)
                        if (t0 + j < T) absorb(S, Kc[j], Vc[j], ch);
                }
                int fb = 0;
#pragma unroll
                for (int d = 1; d < NW; d <<= 1) {
                    fwd_put(sh, fb, s, lane, S);
                    __syncthreads();
                    if (s >= d) {
                        Lane X = fwd_get(sh, fb, s - d, lane);
                        compose(X, S, ch.W, (float)(d * LS));
                        S = X;
                    }
                    fb ^= 1;
                }
                fwd_put(sh, fb, s, lane, S);
                __syncthreads();
                L = lane_in(a0, b0, o0);
                if (s > 0) compose(L, fwd_get(sh, fb, s - 1, lane), ch.W, (float)(s * LS));
            } else {
                const float *q = ck + ((tile * NW + s) * 4) * 64 + lane;
                L = Lane{q[0], q[64], q[128], q[192]};
            }
#pragma unroll
            for (int j = 0; j < LS; ++j) {
                Y[j] = 0.0f;
                LAM[j] = 0.0f;
                PII[j] = 0.0f;
                if (FULL || t0 + j < T)
                    fwd_token<SAFE>(L, Kc[j], Vc[j], ch, Y[j], LAM[j], PII[j]);
            }
        }
        if constexpr (GATE) {
            // g = dy sigmoid(r) replaces dy, and dr = g wkv (1 - sigmoid(r)) is
            // stored now that wkv is known, so that r is dead before the scans
            const TileRowsT<IO> drr = rows(drseq, t0);
#pragma unroll
            for (int j = 0; j < LS; ++j) {
                if (FULL || t0 + j < T) {
                    const float sg = gate_of(Rc[j]);
                    Gc[j] *= sg;
                    if (active) drr.st(j, Gc[j] * Y[j] * (1.0f - sg));
                }
            }
        }
        // the wave holding token T-1 (last tile) starts from the upstream seed
        const bool seeded = ds_out && tile == ntiles - 1 && t0 <= T - 1 && T - 1 < t0 + LS;
        // local backward summary of this segment
        Rev z = rev_empty();
        if (FULL && !seeded) {
            z = rev_summary_fixed<LS>(Gc, Y, LAM, ch.W);
        } else {
            if (seeded) z = seed_of();
#pragma unroll
            for (int j = LS - 1; j >= 0; --j)
                if (FULL || t0 + j < T) rev_absorb(z, Gc[j], Y[j], LAM[j], ch.W);
        }
        // inclusive scan from the last segment backward (Hillis-Steele)
        int buf = rb;
#pragma unroll
        for (int d = 1; d < NW; d <<= 1) {
            rev_put(sh, buf, s, lane, z);
            __syncthreads();
            if (s + d < NW) rev_compose(z, rev_get(sh, buf, s + d, lane), ch.W, (float)(d * LS));
            buf ^= 1;
        }
        rev_put(sh, buf, s, lane, z);
        __syncthreads();
        Rev suf = rev_empty();
        if (s + 1 < NW) suf = rev_get(sh, buf, s + 1, lane);
        const Rev agg = rev_get(sh, buf, 0, lane);
        rb = buf ^ 1;
        rev_compose(suf, carry, ch.W, (float)((NW - 1 - s) * LS));
        if (seeded) suf = seed_of();  // (later segments and the carry are empty here)
        {
            Rev nc = agg;
            rev_compose(nc, carry, ch.W, (float)TT);
            carry = nc;
        }
        // re-sweep backward from the suffix state, emitting gradients
        const TileRowsT<IO> dkr = rows(dkseq, t0), dvr = rows(dvseq, t0);
#pragma unroll
        for (int j = LS - 1; j >= 0; --j) {
            if (FULL || t0 + j < T) {
                const float K = Kc[j];
                const float v = Vc[j], g = Gc[j], y = Y[j];
                // (dwx = 0 and dws = 1 on the one-exponential path)
                const float ekx = ex2(fmaf(-suf.m, ch.W, K + (SAFE ? suf.r0 + dwx : suf.r0)));
                const float ek = SAFE ? ekx * dws : ekx;
                const float own = PII[j] * g;
                const float vy = v - y;
                if (active) {
                    dvr.st(j, fmaf(ek, suf.R, own));
                    dkr.st(j, fmaf(own, vy, ek * fmaf(v, suf.R, -suf.S)));
                }
                dw_acc = fmaf(-ekx, fmaf(v, suf.R1, -suf.S1), dw_acc);
                du_acc = fmaf(own, vy, du_acc);
                rev_absorb(suf, g, y, LAM[j], ch.W);
            }
        }
        // wave 0 has swept past token 0: suf holds R_{-1}, S_{-1}, R'_{-1}, S'_{-1}.
        // Park them, with their frame, in tile 0's checkpoint slots of segments 0
        // and 1 (every wave read its checkpoint before the scan's barriers) and
        // finish after the loop, where few registers are live.
        if (tile == 0 && s == 0 && active && (s_in || ds_in)) {
            float *q = ck + lane;
            q[0] = suf.R;
            q[64] = suf.S;
            q[128] = suf.R1;
            q[192] = suf.S1;
            q[256] = fmaf(-suf.m, ch.W, suf.r0);
        }
#pragma unroll
        for (int j = 0; j < LS; ++j) {
            Kc[j] = Kn[j] * kLog2e;
            Vc[j] = Vn[j];
        }
    }

    // the carried state as a token before t = 0: its gradient, and its share of dw
    if (s == 0 && active && (s_in || ds_in)) {
        const float *q = ck + lane;
        float a0 = 0.0f, b0 = 0.0f, o20 = kEmpty2;
        if (s_in) {
            a0 = s_in[(0 * B + bb) * C + c];
            b0 = s_in[(1 * B + bb) * C + c];
            o20 = o_in(s_in[(2 * B + bb) * C + c]);
        }
        // 2^{frame + o0}: bounded, since e^{o0 - t w} b0 <= D_t for every output
        const float scx = ex2(SAFE ? (q[256] + o20) + dwx : q[256] + o20);
        const float sc = SAFE ? scx * dws : scx;
        const float da = q[0] * sc, db = -q[64] * sc;
        if (ds_in) {
            ds_in[(0 * B + bb) * C + c] = da;
            ds_in[(1 * B + bb) * C + c] = db;
            ds_in[(2 * B + bb) * C + c] = fmaf(da, a0, db * b0);
        }
        dw_acc = fmaf(-scx, fmaf(a0, q[128], -b0 * q[192]), dw_acc);
    }

    // dw, du of this lane: sum over the waves in a fixed order
    sh.red[0][s][lane] = (double)dw_acc * (double)dws;
    sh.red[1][s][lane] = (double)du_acc;
    __syncthreads();
    if (s == 0 && active) {
        double sw = 0.0, su = 0.0;
        for (int i = 0; i < NW; ++i) {
            sw += sh.red[0][i][lane];
            su += sh.red[1][i][lane];
        }
        part[bb * C + c] = sw;
        part[B * C + bb * C + c] = su;
    }
}

// FULL: T is a whole number of tiles (chosen on the host).  CK: start every
// tile from the forward's checkpoints `cks` instead of a first pass.  GATE:
// the gradient of the gated output, with r read and dr written.
template <int NW, int LS, bool FULL, bool CK, bool GATE, class IO>
__global__ __launch_bounds__(NW * 64) void bwd_seg_kernel(int64_t B, int64_t T, int64_t C,
                                                          const float *__restrict__ w,
                                                          const float *__restrict__ u,
                                                          const typename IO::T *__restrict__ k,
                                                          const typename IO::T *__restrict__ v,
                                                          const typename IO::T *__restrict__ dy,
                                                          typename IO::T *__restrict__ dk,
                                                          typename IO::T *__restrict__ dv,
                                                          float *__restrict__ ckpt,
                                                          double *__restrict__ part,
                                                          const float *s_in, const float *s_out,
                                                          const float *ds_out, float *ds_in,
                                                          const float *cks,
                                                          const typename IO::T *__restrict__ r,
                                                          typename IO::T *__restrict__ dr) {
    __shared__ BwdShared<NW> sh;
    constexpr int TT = NW * LS;
    const int64_t ngroups = (C + 63) / 64;
    const int64_t g = blockIdx.x % ngroups;
    const int64_t bb = blockIdx.x / ngroups;
    const int64_t c = g * 64 + (threadIdx.x & 63);
    const bool active = c < C;
    const Chan ch = make_chan(active ? w[c] : 0.0f, active ? u[c] : 0.0f);
    const bool fast = __syncthreads_and(chan_fast_ok(ch));
    const int64_t ntiles = (T + TT - 1) / TT;
    // wave-uniform base of this (sequence, channel group); inactive lanes read
    // the group's first channel and never store
    const int64_t base = bb * T * C + g * 64;
    const uint32_t voff = active ? (uint32_t)((threadIdx.x & 63) * IO::kBytes) : 0u;
    float *ck = ckpt + (int64_t)blockIdx.x * ntiles * NW * 4 * 64;
    if (fast)
        bwd_body<NW, LS, false, FULL, CK, GATE, IO>(
            B, T, C, bb, c, active, ch, k + base, v + base, dy + base, dk + base, dv + base,
            GATE ? r + base : nullptr, GATE ? dr + base : nullptr, voff, ck, part, s_in, s_out,
            ds_out, ds_in, cks, sh);
    else
        bwd_body<NW, LS, true, FULL, CK, GATE, IO>(
            B, T, C, bb, c, active, ch, k + base, v + base, dy + base, dk + base, dv + base,
            GATE ? r + base : nullptr, GATE ? dr + base : nullptr, voff, ck, part, s_in, s_out,
            ds_out, ds_in, cks, sh);
}

// dw[c], du[c] = sums over the batch of the per-lane parts, in order b = 0..B-1.
__global__ __launch_bounds__(256) void bwd_reduce_kernel(int64_t B, int64_t C,
                                                         const double *__restrict__ part,
                                                         float *__restrict__ dw,
                                                         float *__restrict__ du) {
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c >= C) return;
    double sw = 0.0, su = 0.0;
    for (int64_t b = 0; b < B; ++b) {
        sw += part[b * C + c];
        su += part[B * C + b * C + c];
    }
    dw[c] = (float)sw;
    du[c] = (float)su;
}

// dw = du = 0 when there are no tokens.
__global__ __launch_bounds__(256) void bwd_zero_kernel(int64_t C, float *__restrict__ dw,
                                                       float *__restrict__ du) {
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c >= C) return;
    dw[c] = 0.0f;
    du[c] = 0.0f;
}

// T == 0: the state passes through unchanged, so its gradient is the upstream
// one moved into the coordinates of state_in (e^{o0 - o_T} rescales), or zero.
__global__ __launch_bounds__(256) void bwd_state_pass_kernel(int64_t n, const float *s_in,
                                                             const float *s_out,
                                                             const float *ds_out, float *ds_in) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    float da = 0.0f, db = 0.0f, dov = 0.0f;
    if (s_in && ds_out && s_in[n + i] > 0.0f) {
        const float sc = ex2((s_in[2 * n + i] - s_out[2 * n + i]) * kLog2e);
        da = ds_out[i] * sc;
        db = ds_out[n + i] * sc;
        dov = fmaf(da, s_in[i], db * s_in[n + i]);
    }
    ds_in[i] = da;
    ds_in[n + i] = db;
    ds_in[2 * n + i] = dov;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

template <bool FULL, bool CK, bool GATE, class IO>
void launch_bwd_seg_k(const BwdArgs &a, int64_t grid, float *ck, double *part, hipStream_t st) {
    using T = typename IO::T;
    hipLaunchKernelGGL((bwd_seg_kernel<kBwdNW, kBwdLS, FULL, CK, GATE, IO>),
                       dim3((unsigned)grid), dim3(kBwdNW * 64), 0, st, a.B, a.T, a.C, a.w, a.u,
                       (const T *)a.k, (const T *)a.v, (const T *)a.dy, (T *)a.dk, (T *)a.dv, ck,
                       part, a.s_in, a.s_out, a.ds_out, a.ds_in, a.ck, (const T *)a.r,
                       (T *)a.dr);
}

// The whole-tile variant where T allows it (with the gate as well: its extra
// row array costs some 20 spilled registers there, and it is still faster than
// the general code).
template <bool CK, bool GATE, class IO>
void launch_bwd_seg_full(const BwdArgs &a, int64_t grid, float *ck, double *part,
                         hipStream_t st) {
    if (a.T % (kBwdNW * kBwdLS) == 0)
        launch_bwd_seg_k<true, CK, GATE, IO>(a, grid, ck, part, st);
    else
        launch_bwd_seg_k<false, CK, GATE, IO>(a, grid, ck, part, st);
}

template <bool GATE, class IO>
void launch_bwd_seg_ck(const BwdArgs &a, int64_t grid, float *ck, double *part,
                       hipStream_t st) {
    if (a.from_ck)
        launch_bwd_seg_full<true, GATE, IO>(a, grid, ck, part, st);
    else
        launch_bwd_seg_full<false, GATE, IO>(a, grid, ck, part, st);
}

template <class IO>
void launch_bwd_seg(const BwdArgs &a, int64_t grid, float *ck, double *part, hipStream_t st) {
    if (a.r)
        launch_bwd_seg_ck<true, IO>(a, grid, ck, part, st);
    else
        launch_bwd_seg_ck<false, IO>(a, grid, ck, part, st);
}

}  // namespace

size_t backward_workspace_bytes(int64_t B, int64_t T, int64_t C) {
    if (B <= 0 || T <= 0 || C <= 0) return 0;
    constexpr int64_t TT = kBwdNW * kBwdLS;
    const int64_t ngroups = (C + 63) / 64;
    const int64_t ntiles = (T + TT - 1) / TT;
    const size_t ck = (size_t)B * ngroups * ntiles * kBwdNW * 4 * 64 * sizeof(float);
    const size_t part = (size_t)2 * B * C * sizeof(double);
    return align_up(ck) + align_up(part);
}

hipError_t launch_backward(const BwdArgs &a, hipStream_t st) {
    const int64_t C = a.C;
    if (a.B == 0 || a.T == 0) {
        if (C == 0) return hipSuccess;
        hipLaunchKernelGGL(bwd_zero_kernel, dim3((unsigned)((C + 255) / 256)), dim3(256), 0, st,
                           C, a.dw, a.du);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess || !a.ds_in || a.B == 0) return e;
        const int64_t n = a.B * C;
        hipLaunchKernelGGL(bwd_state_pass_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256),
                           0, st, n, a.s_in, a.s_out, a.ds_out, a.ds_in);
        return hipGetLastError();
    }
    constexpr int64_t TT = kBwdNW * kBwdLS;
    const int64_t ngroups = (C + 63) / 64;
    const int64_t ntiles = (a.T + TT - 1) / TT;
    float *ck = (float *)a.ws;
    double *part = (double *)((char *)a.ws +
                              align_up((size_t)a.B * ngroups * ntiles * kBwdNW * 4 * 64 *
                                       sizeof(float)));
    const int64_t grid = a.B * ngroups;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    switch (a.io) {
        case kIoF32: launch_bwd_seg<IoF32>(a, grid, ck, part, st); break;
        case kIoF16: launch_bwd_seg<IoF16>(a, grid, ck, part, st); break;
        case kIoBF16: launch_bwd_seg<IoBF16>(a, grid, ck, part, st); break;
        default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_reduce_kernel, dim3((unsigned)((C + 255) / 256)), dim3(256), 0, st,
                       a.B, C, part, a.dw, a.du);
    return hipGetLastError();
}

}  // namespace wkv

// wkv_device.hpp -- device-side arithmetic of the WKV operator for gfx950.
//
// The operator (RWKV architecture deep dive, youngju.dev, "WKV mechanism: core
// computation"): per lane, wkv_t = (A_{t-1} + e^{u+k_t} v_t) / (B_{t-1} + e^{u+k_t})
// where A, B are the running sums of e^{k_i} v_i and e^{k_i}, decayed by e^{-w}
// per later token ("Recurrent formulation"), kept as a scaled pair and a running
// maximum exponent ("Numerical stability via log-space computation").
//
// Inside kernels every exponent is held in log2 units (K = k log2 e, W = w log2 e,
// U = u log2 e, o2 = o log2 e) so that each exponential is one v_exp_f32.  The
// register state of a lane is a Lane: the scaled sums and their frame exponent,
// kept as an anchor plus a count of decay steps.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wkv {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Exponent of the empty state inside kernels (log2 units).  Finite, so that
// differences against it stay ordered; exp2 of minus it is exactly 0.
constexpr float kEmpty2 = -1.0e38f;
// |U - W| (log2 units) up to which the one-exponential step is used; beyond it
// e^{u-w} could leave the float range and the two-exponential step runs.
constexpr float kFastLimit2 = 86.0f;

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float rcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float lg2(float x) { return __builtin_amdgcn_logf(x); }

// Per-channel constants of one lane.
struct Chan {
    float W;   // w log2 e
    float U;   // u log2 e
    float c1;  // e^{u-w} = 2^{U-W}: the bonus relative to one step of decay
};

__device__ __forceinline__ Chan make_chan(float w, float u) {
    Chan ch;
    ch.W = w * kLog2e;
    ch.U = u * kLog2e;
    ch.c1 = ex2(ch.U - ch.W);
    return ch;
}

__device__ __forceinline__ bool chan_fast_ok(const Chan &ch) {
    return fabsf(ch.U - ch.W) <= kFastLimit2;
}

// Register state of one lane: the sums (a, b) of all tokens so far, in the
// frame 2^f with f = e0 - n W.  e0 is the exponent at which the frame was last
// re-anchored (the token that became the largest decayed term, or the start of
// a segment) and n the number of decay steps since then.  Deriving f from the
// anchor with one fma keeps its error at one rounding: stepping f <- f - W
// token after token (as a direct transcription of the log-space recurrence
// would) accumulates a systematic rounding bias of up to half an ulp of f per
// token, which at |f| ~ 90 and small W reaches percent-level errors in the
// weights after a few thousand tokens.  Differences of two frames are formed
// as (anchor - anchor) - (steps - steps) W: close anchors subtract exactly, so a
// rescale factor 2^d is as accurate as d itself rather than off by an ulp of
// |f| (~8e-6 at |f| ~ 90).
struct Lane {
    float a, b;  // scaled numerator and denominator
    float e0;    // anchor exponent (log2 units)
    float n;     // decay steps since the anchor (exact in float up to 2^24)
};

__device__ __forceinline__ Lane lane_at(float a, float b, float o) { return Lane{a, b, o, 0.0f}; }

// A carried state as the ABI hands it in (o2 = o log2 e).  A state is defined
// up to a common scale, so one whose denominator b lies far from 1 is first
// rescaled to b = 1 (o2 += log2 b): with b = 1e-30, say, the products the
// step forms with a small bonus would leave float's normal range.  States the
// kernels write have b near 1 or above and pass unchanged.
__device__ __forceinline__ Lane lane_in(float a, float b, float o2) {
    if (b > 0.0f && (b < 0x1p-20f || b > 0x1p20f)) return Lane{a * rcp(b), 1.0f, o2 + lg2(b), 0.0f};
    return Lane{a, b, o2, 0.0f};
}
__device__ __forceinline__ Lane lane_empty() { return Lane{0.0f, 0.0f, kEmpty2, 0.0f}; }
// Frame exponent of the sums after the last token.
__device__ __forceinline__ float lane_o(const Lane &L, float W) { return fmaf(-L.n, W, L.e0); }

// One token against the state, then folded into it.  Returns wkv_t.
//
// The past sums, decayed for this token, sit at h = e0 - (n+1) W.  With
// s = K - h the update keeps the larger of h and K as the new frame:
//   s <= 0:  a' = a + 2^s v,        b' = b + 2^s,        frame h (n+1 steps)
//   s >  0:  a' = a 2^{-s} + v,     b' = b 2^{-s} + 1,   frame K (re-anchored)
// The output needs the bonus term e^{u+k_t} relative to the undecayed past
// frame h + W, i.e. 2^{U + K - h - W} = c1 2^s; scaling numerator and
// denominator by the update's factor (1 or 2^{-s}) gives
//   y = (a P + c1 Q v) / (b P + c1 Q),   (P, Q) = s > 0 ? (2^{-s}, 1) : (1, 2^s)
// so one exponential E = 2^{-|s|} serves both.  Valid while c1 is a normal
// float with margin, i.e. |U - W| <= kFastLimit2.
__device__ __forceinline__ float step_fast(Lane &L, float K, float v, const Chan &ch) {
    const float n1 = L.n + 1.0f;
    const float s = fmaf(n1, ch.W, K - L.e0);  // K - h, anchor difference first
    const float E = ex2(-fabsf(s));
    const bool pos = s > 0.0f;
    const float P = pos ? E : 1.0f;
    const float Q = pos ? 1.0f : E;
    const float aP = L.a * P;
    const float bP = L.b * P;
    const float Qc = Q * ch.c1;
    const float y = fmaf(Qc, v, aP) * rcp(bP + Qc);
    L.a = fmaf(Q, v, aP);
    L.b = bP + Q;
    L.e0 = pos ? K : L.e0;
    L.n = pos ? 0.0f : n1;
    return y;
}

// The same token with the output normalised on its own maximum (two
// exponentials); valid for any finite u, w.
__device__ __forceinline__ float step_safe(Lane &L, float K, float v, const Chan &ch) {
    const float x = fmaf(L.n, ch.W, (ch.U + K) - L.e0);  // (U + K) - frame
    const float F = ex2(-fabsf(x));
    const bool px = x > 0.0f;
    const float Pp = px ? F : 1.0f;
    const float Qq = px ? 1.0f : F;
    const float y = fmaf(Qq, v, L.a * Pp) * rcp(fmaf(L.b, Pp, Qq));
    const float n1 = L.n + 1.0f;
    const float s = fmaf(n1, ch.W, K - L.e0);
    const float E = ex2(-fabsf(s));
    const bool pos = s > 0.0f;
    const float P = pos ? E : 1.0f;
    const float Q = pos ? 1.0f : E;
    L.a = fmaf(L.a, P, Q * v);
    L.b = fmaf(L.b, P, Q);
    L.e0 = pos ? K : L.e0;
    L.n = pos ? 0.0f : n1;
    return y;
}

template <bool SAFE>
__device__ __forceinline__ float step(Lane &L, float K, float v, const Chan &ch) {
    if constexpr (SAFE)
        return step_safe(L, K, v, ch);
    else
        return step_fast(L, K, v, ch);
}

// Fold a token into the state without producing an output (segment summaries).
__device__ __forceinline__ void absorb(Lane &L, float K, float v, const Chan &ch) {
    const float n1 = L.n + 1.0f;
    const float s = fmaf(n1, ch.W, K - L.e0);
    const float E = ex2(-fabsf(s));
    const bool pos = s > 0.0f;
    const float P = pos ? E : 1.0f;
    const float Q = pos ? 1.0f : E;
    L.a = fmaf(L.a, P, Q * v);
    L.b = fmaf(L.b, P, Q);
    L.e0 = pos ? K : L.e0;
    L.n = pos ? 0.0f : n1;
}

// X <- X (+) Y: the state X followed by a stretch of `len` tokens whose
// contribution from an empty start is Y (both anchored Lanes).  X decays by
// 2^{-W len} across the stretch, which only adds len to its step count (exact
// in float), then the two sums add in the larger frame.  No exponent is ever
// rounded and stored, so long chains of compositions (one per tile of a long
// sequence) do not drift.  Empty operands are identities.
__device__ __forceinline__ void compose(Lane &X, const Lane &Y, float W, float len) {
    const float nxl = X.n + len;
    // (X.e0 - nxl W) - (Y.e0 - Y.n W), anchors first: exact when they are close
    const float d = fmaf(-(nxl - Y.n), W, X.e0 - Y.e0);
    const float E = ex2(-fabsf(d));
    const bool xbig = d > 0.0f;
    const float P = xbig ? 1.0f : E;
    const float Q = xbig ? E : 1.0f;
    X.a = fmaf(X.a, P, Y.a * Q);
    X.b = fmaf(X.b, P, Y.b * Q);
    X.e0 = xbig ? X.e0 : Y.e0;
    X.n = xbig ? nxl : Y.n;
}

// Sweep of one whole segment in a single frame.  R is the state before the
// segment and S the segment's own summary (its tokens absorbed from the empty
// state), so S's anchor is the token whose decayed exponent is the largest of
// the segment at its last token.  Measured at the segment's last token, every
// term's weight is fixed: token t's is x_t = K_t - (L-1-t) W, the bonus term of
// token t is c1 2^{x_t}, and R's is its frame G = R.e0 - (R.n + L) W.  (For
// the output at token t, everything present is scaled by the same 2^{-(L-t) W}
// relative to its own time, which cancels in the ratio.)  With F the larger of
// G and max x_t as the frame, y_t = (A + c1 E_t v_t) / (B + c1 E_t), E_t =
// 2^{x_t - F} <= 1, and A, B accumulate E_t v_t, E_t: one exponential and one
// reciprocal per token, no rescaling.  Exponent differences are formed anchor
// first as in step_fast.
//
// Valid when no term that is the largest present at its own time sits more
// than 100 below F (else it could underflow): the present maximum only grows,
// so it suffices that max(G, x_0) >= F - 100.  The first token's denominator
// B + c1 E_0 must also be a normal float (every later one is larger): with an
// empty or nearly empty state and a small bonus c1 it can fall below float's
// normal range, where the reciprocal flushes it to zero.  And with a large
// bonus (c1 > 1) a token far below F still matters through c1 E_t although
// E_t alone would flush, so then every x_t (the smallest, xmin) must lie
// within 100 of F.  seg_frame() returns whether all of this holds for this
// lane.
struct SegFrame {
    float Ae, An;       // anchor of F: F = Ae - An W
    float alpha, beta;  // R's sums in frame F
};

__device__ __forceinline__ bool seg_frame(const Lane &R, const Lane &S, float W, float c1,
                                          float len, float K0, float xmin, SegFrame &f) {
    const float nR = R.n + len;
    const float D = fmaf(-(nR - S.n), W, R.e0 - S.e0);  // G - max x_t
    const bool g = D >= 0.0f;
    f.Ae = g ? R.e0 : S.e0;
    f.An = g ? nR : S.n;
    const float sc = g ? 1.0f : ex2(D);
    f.alpha = R.a * sc;
    f.beta = R.b * sc;
    const float d0 = fmaf(f.An - (len - 1.0f), W, K0 - f.Ae);  // x_0 - F
    const float den0 = fmaf(c1, ex2(d0), f.beta);
    const float dmin = fmaf(f.An, W, xmin - f.Ae);  // xmin - F
    return fmaxf(D, d0) >= -100.0f && den0 >= 0x1p-100f && (c1 <= 1.0f || dmin >= -100.0f);
}

// Token t (0-based within the segment of `len` tokens) in the frame of f.
__device__ __forceinline__ float frame_token(float &A, float &Bs, const SegFrame &f, float K,
                                             float v, float t_from_end, const Chan &ch) {
    const float E = ex2(fmaf(f.An - t_from_end, ch.W, K - f.Ae));
    const float Ec = E * ch.c1;
    const float y = fmaf(Ec, v, A) * rcp(Bs + Ec);
    A = fmaf(E, v, A);
    Bs += E;
    return y;
}

// Element formats of k, v, r and y.  Arithmetic and the state are always
// float32; 16-bit inputs widen exactly, and outputs round to nearest even.
constexpr int kBufferWord3 = 0x00020000;  // buffer descriptor word 3 (gfx9 raw access)
constexpr int kNT = 2;                    // cache-policy operand: non-temporal

struct IoF32 {
    using T = float;
    static constexpr int kBytes = 4;
    __device__ __forceinline__ static float to_f(T x) { return x; }
    __device__ __forceinline__ static T from_f(float x) { return x; }
    // The b32 buffer builtins move raw 32-bit words: bit-cast, never convert.
    __device__ __forceinline__ static float ld(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                               uint32_t soff) {
        return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, kNT));
    }
    __device__ __forceinline__ static void st(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                              uint32_t soff, float x) {
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, x), r, voff, soff, kNT);
    }
};

struct IoF16 {
    using T = _Float16;
    static constexpr int kBytes = 2;
    __device__ __forceinline__ static float to_f(T x) { return (float)x; }
    __device__ __forceinline__ static T from_f(float x) { return (T)x; }  // v_cvt_f16_f32, RNE
    __device__ __forceinline__ static float ld(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                               uint32_t soff) {
        return (float)__builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, kNT));
    }
    __device__ __forceinline__ static void st(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                              uint32_t soff, float x) {
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, from_f(x)), r,
                                              voff, soff, kNT);
    }
};

// bfloat16 is the upper half of a float32: widening is a shift; narrowing is
// gfx950's v_cvt_pk_bf16_f32 (round to nearest even, NaN stays NaN).
struct IoBF16 {
    using T = unsigned short;
    static constexpr int kBytes = 2;
    __device__ __forceinline__ static float to_f(T x) {
        return __builtin_bit_cast(float, (uint32_t)x << 16);
    }
    __device__ __forceinline__ static T from_f(float x) {
        return __builtin_bit_cast(unsigned short, (__bf16)x);
    }
    __device__ __forceinline__ static float ld(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                               uint32_t soff) {
        return to_f(__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, kNT));
    }
    __device__ __forceinline__ static void st(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                              uint32_t soff, float x) {
        __builtin_amdgcn_raw_buffer_store_b16(from_f(x), r, voff, soff, kNT);
    }
};

// Consecutive rows of a row-major [rows][C] tensor of IO::T, seen by one wave.
// `base` must be wave-uniform (it becomes a buffer descriptor in scalar
// registers); `voff` is the lane's byte offset from `base` (its channel, plus a
// whole number of rows when the lanes of a wave cover several row ranges) and
// `rowb` = C * IO::kBytes the row pitch.  Row j is addressed by the scalar
// offset j*rowb, so an access is a single buffer instruction with one 32-bit
// vector offset.  Offsets stay below 2^32 bytes from `base`.  Accesses carry
// the non-temporal hint: every k, v, r and y element is touched once.
template <class IO>
struct TileRowsT {
    __amdgpu_buffer_rsrc_t r;
    uint32_t voff;
    uint32_t rowb;
    __device__ __forceinline__ TileRowsT(const typename IO::T *base, uint32_t voff_,
                                         uint32_t rowb_)
        : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<typename IO::T *>(base), (short)0,
                                              (int)0xffffffffu, kBufferWord3)),
          voff(voff_), rowb(rowb_) {}
    __device__ __forceinline__ float ld(int j) const { return IO::ld(r, voff, (uint32_t)j * rowb); }
    __device__ __forceinline__ void st(int j, float x) const {
        IO::st(r, voff, (uint32_t)j * rowb, x);
    }
};
using TileRows = TileRowsT<IoF32>;

// Receptance gate of the time-mixing block (RWKV architecture deep dive,
// "RWKV architecture overview", block figure): sigmoid(r) = 1 / (1 + 2^{-r log2 e}).
// The tails saturate cleanly: 2^{+large} = inf gives 0, 2^{-large} = 0 gives 1.
__device__ __forceinline__ float gate_of(float r) { return rcp(1.0f + ex2(-r * kLog2e)); }

// ABI state (natural-log exponent) -> kernel exponent (log2), mapping -inf and
// anything below the empty sentinel onto it.
__device__ __forceinline__ float o_in(float o_nat) { return fmaxf(o_nat * kLog2e, kEmpty2); }
__device__ __forceinline__ float o_out(float o2) { return o2 * kLn2; }

// Stores state L of lane i in the public layout [3][n] (a, b, o with o in
// natural-log units), each plane n floats apart.
__device__ __forceinline__ void store_state(float *dst, int64_t n, int64_t i, const Lane &L,
                                            float W, float poison) {
    dst[i] = L.a + poison;
    dst[n + i] = L.b + poison;
    dst[2 * n + i] = o_out(lane_o(L, W)) + poison;
}

}  // namespace wkv

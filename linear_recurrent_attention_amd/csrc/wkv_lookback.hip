// wkv_lookback.hip -- forward by blocks of tokens chained with a decoupled
// look-back (gfx950).
//
// Same result as the other forward kernels (RWKV architecture deep dive,
// youngju.dev, "WKV mechanism: core computation"; state carried as in the
// rwkv-architecture skill page, "Quick start").  Every sequence is cut into
// blocks of NS*LS tokens and its channels into groups of 64 (one wave wide).
// A workgroup takes one block of CG adjacent groups of one sequence: CG waves
// side by side (so each token row is read 256*CG bytes at a time) times NS
// waves stacked along the block.  Wave (g, s) loads its LS tokens of group g,
// folds them into a summary, and the NS summaries of a group compose through
// LDS into the block's aggregate, which is published.  The workgroup then
// looks back over earlier blocks of each of its groups, folding their
// published states until it meets one that holds the whole prefix, publishes
// its own inclusive state, and every wave re-sweeps its tokens from its own
// starting state, writing y (a wave whose segment starts on a multiple of 128
// tokens also stores that state as a checkpoint, when asked to).  Each
// workgroup reads its k and v once and writes its y once, so HBM traffic is
// the algorithmic 12 bytes per lane-token; the workgroups are small and
// short-lived, so many of them per CU keep the memory system busy while
// others wait.
//
// Publishing without fences.  A release fence at device scope writes back the
// issuing die's whole L2 and costs ~0.1 us per workgroup on MI355X, serialised,
// which would dominate.  Instead every published value is its own 64-bit word:
// the high half is a tag (launch epoch and status), the low half the float's
// bits.  A word is written and read with relaxed device-scope atomics, which
// are single-copy atomic and coherent across the dies, so a reader that sees
// the expected tag on a word also sees its value; no ordering between words is
// needed because each word validates itself.  A block's aggregate and its
// inclusive state go to separate slots.  A reader fetches the inclusive slot
// and, only when that is not wholly published (not yet, or caught half-way
// through being written), the aggregate, which its block wrote before it
// began its look-back; a reader that finds neither whole tries again.
//
// Ordering and progress.  Workgroups are numbered block-major (channel set
// fastest, then sequence, then block) and the hardware dispatches them in that
// order, so every workgroup of block j is dispatched after every workgroup of
// blocks < j.  A workgroup waits only on
// blocks before its own, so the earliest unfinished workgroup never waits on
// one that has not started, and the look-back always terminates.  The host
// gives each launch a fresh epoch (per scratch buffer), so nothing on the
// device has to be reset between launches; a launch replayed from a graph
// takes its epoch from a word that a tiny kernel before it advances.  Every spin is bounded as well:
// past the bound the wait gives up, the block's outputs become NaN, the
// inclusive state it publishes carries the NaN to every later block of the
// sequence and to the final state, and a counter in the scratch header records
// the event for the host.
#include "wkv_device.hpp"
#include "wkv_internal.hpp"

namespace wkv {

namespace {

constexpr uint32_t kAgg = 1u;   // block aggregate published
constexpr uint32_t kIncl = 2u;  // inclusive state (after the block) published

// One published state: [4][64] tagged words (a, b, e0, n per lane).
using Word = unsigned long long;
constexpr int kSlotWords = 4 * 64;

__device__ __forceinline__ void publish(Word *slot, int lane, const Lane &L, uint32_t tag) {
    const Word t = (Word)tag << 32;
    const float v[4] = {L.a, L.b, L.e0, L.n};
#pragma unroll
    for (int f = 0; f < 4; ++f)
        __hip_atomic_store(&slot[f * 64 + lane], t | __builtin_bit_cast(uint32_t, v[f]),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Reads one slot; returns whether all four words of this lane carry `tag`.
__device__ __forceinline__ bool fetch(const Word *slot, int lane, uint32_t tag, Lane &L) {
    Word w[4];
#pragma unroll
    for (int f = 0; f < 4; ++f)
        w[f] = __hip_atomic_load(&slot[f * 64 + lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    L = Lane{__builtin_bit_cast(float, (uint32_t)w[0]), __builtin_bit_cast(float, (uint32_t)w[1]),
             __builtin_bit_cast(float, (uint32_t)w[2]), __builtin_bit_cast(float, (uint32_t)w[3])};
    bool ok = true;
#pragma unroll
    for (int f = 0; f < 4; ++f) ok = ok && (uint32_t)(w[f] >> 32) == tag;
    return ok;
}

template <int CG, int NS>
struct LbShared {
    float s[4][NS][CG][64];    // segment summaries
    float pv[4][NS][CG][64];   // predecessor states fetched this round
    uint32_t pst[NS][CG];      // their status: 0 not ready, kAgg, kIncl
    uint32_t gdone[CG];        // group has its whole prefix (or gave up)
};

template <int CG, int NS>
__device__ __forceinline__ Lane lds_lane(const float (&a)[4][NS][CG][64], int s, int g, int lane) {
    return Lane{a[0][s][g][lane], a[1][s][g][lane], a[2][s][g][lane], a[3][s][g][lane]};
}

template <int CG, int NS>
__device__ __forceinline__ void lds_put(float (&a)[4][NS][CG][64], int s, int g, int lane,
                                        const Lane &L) {
    a[0][s][g][lane] = L.a;
    a[1][s][g][lane] = L.b;
    a[2][s][g][lane] = L.e0;
    a[3][s][g][lane] = L.n;
}

// Per-wave view of the block: which group and segment it holds, where its rows
// are.
struct LbWave {
    int lane, g, s;          // lane, group within the workgroup, segment
    int64_t bb, j;           // sequence, block
    int64_t grp;             // group index within the sequence
    bool gok;                // the group exists (C may end inside the last set)
    bool active;             // this lane's channel exists
    int64_t c;               // channel
    int64_t t0;              // first token of the segment
    uint32_t voff, rowb;     // lane byte offset, row pitch
};

// FULL: the whole block lies inside the sequence, so no token needs a bounds
// test (a workgroup-uniform property: only the last block can be partial).
// GATE: Rg holds the wave's receptance rows and y is sigmoid(r) * wkv.
// IO: element format of y (IoF32, IoF16, IoBF16).
template <int CG, int NS, int LS, bool SAFE, bool FULL, bool GATE, class IO>
__device__ __forceinline__ void lb_body(int64_t B, int64_t T, int64_t C, const Chan &ch,
                                        const LbWave &q, const float (&K)[LS], const float (&V)[LS],
                                        const float (&Rg)[GATE ? LS : 1],
                                        typename IO::T *yseq, const float *__restrict__ s_in,
                                        float *__restrict__ s_out, float *__restrict__ ck,
                                        Word *aggs, Word *incls, uint32_t epoch,
                                        uint32_t *giveups, uint32_t spin_limit,
                                        LbShared<CG, NS> &sh) {
    constexpr int TB = NS * LS;
    const int lane = q.lane, g = q.g, s = q.s;
    const int64_t j = q.j;
    const int64_t ngroups = (C + 63) >> 6;
    // slot offset of (block, sequence, group)
    auto slot_of = [&](int64_t blk) { return ((blk * B + q.bb) * ngroups + q.grp) * kSlotWords; };
    const uint32_t tag_agg = (epoch << 2) | kAgg, tag_incl = (epoch << 2) | kIncl;

    // K holds the keys in log2 units (k log2 e)

    // (1) segment summary from the empty state, shared through LDS.  On a
    // whole block it is taken in one frame: the largest decayed exponent
    // x_t = K_t - (LS-1-t) W of the segment at its last token, so that each
    // token costs one exponential and no rescaling (the sums are anchored at
    // that exponent with no decay steps yet).
    Lane S = lane_empty();
    float xmin = INFINITY;  // smallest x_t (the one-frame re-sweep's bonus check)
    if constexpr (FULL) {
        float M = -INFINITY;
#pragma unroll
        for (int t = 0; t < LS; ++t) {
            const float x = fmaf((float)(t - (LS - 1)), ch.W, K[t]);
            M = fmaxf(M, x);
            xmin = fminf(xmin, x);
        }
        float sa = 0.0f, sb = 0.0f;
#pragma unroll
        for (int t = 0; t < LS; ++t) {
            const float e = ex2(fmaf((float)(t - (LS - 1)), ch.W, K[t]) - M);
            sa = fmaf(e, V[t], sa);
            sb += e;
        }
        S = Lane{sa, sb, M, 0.0f};
    } else {
#pragma unroll
        for (int t = 0; t < LS; ++t)
            if (q.t0 + t < T) absorb(S, K[t], V[t], ch);
    }
    lds_put(sh.s, s, g, lane, S);
    __syncthreads();
    // the block's aggregate (the summaries stay in LDS: the segment prefixes
    // are recomputed from them after the look-back, which keeps fewer registers
    // live while it waits)
    Lane agg = lds_lane(sh.s, 0, g, lane);
#pragma unroll
    for (int w = 1; w < NS; ++w) compose(agg, lds_lane(sh.s, w, g, lane), ch.W, (float)LS);

    // (2) state at the start of the block, per group
    Lane P = lane_empty();
    bool failed = false;
    if (j == 0) {
        // only segment 0 reads state_in, before this group's inclusive state is
        // published: the last block may write state_out over it (in-place
        // update) as soon as that state is visible, and it depends on the values
        // read here
        if (s == 0 && s_in && q.active)
            P = lane_in(s_in[(0 * B + q.bb) * C + q.c], s_in[(1 * B + q.bb) * C + q.c],
                        o_in(s_in[(2 * B + q.bb) * C + q.c]));
        if (s == 0) lds_put(sh.pv, 0, g, lane, P);
        __syncthreads();
        P = lds_lane(sh.pv, 0, g, lane);
    } else {
        if (s == 0 && q.gok) publish(aggs + slot_of(j), lane, agg, tag_agg);
        int64_t base = j - 1;  // nearest block of this group not yet folded into P
        float covered = 0.0f;  // tokens covered by P
        uint32_t spins = 0;
        bool done = !q.gok;
        for (;;) {
            // wave (g, s) examines block base - s of its group
            if (!done) {
                const int64_t pj = base - s;
                uint32_t st = 0;
                Lane X = lane_empty();
                if (pj >= 0) {
                    // the inclusive state first; the aggregate only when that
                    // is not (yet wholly) published
                    Lane Xi, Xa;
                    const bool oi = fetch(incls + slot_of(pj), lane, tag_incl, Xi);
                    if (__all(oi)) {
                        st = kIncl;
                        X = Xi;
                    } else {
                        const bool oa = fetch(aggs + slot_of(pj), lane, tag_agg, Xa);
                        if (__all(oa)) {
                            st = kAgg;
                            X = Xa;
                        }
                    }
                }
                lds_put(sh.pv, s, g, lane, X);
                if (lane == 0) sh.pst[s][g] = st;
            }
            __syncthreads();
            if (!done) {
                // fold the leading ready blocks, nearest first, up to the first
                // inclusive one
                int use = 0;
                for (int w = 0; w < NS && base - w >= 0; ++w) {
                    const uint32_t stw = sh.pst[w][g];
                    if (stw == 0) break;
                    Lane Y = lds_lane(sh.pv, w, g, lane);
                    compose(Y, P, ch.W, covered);
                    P = Y;
                    covered += (float)TB;
                    ++use;
                    if (stw == kIncl) {
                        done = true;
                        break;
                    }
                }
                base -= use;
                if (base < 0) done = true;
                if (!done && use == 0) {
                    if (++spins > spin_limit) {
                        failed = true;
                        done = true;
                    } else {
                        __builtin_amdgcn_s_sleep(1);
                    }
                }
            }
            if (s == 0 && lane == 0) sh.gdone[g] = done;
            // also orders this round's LDS reads before the next round's writes
            __syncthreads();
            bool all = true;
#pragma unroll
            for (int h = 0; h < CG; ++h) all = all && sh.gdone[h] != 0;
            if (all) break;
        }
    }
    const float poison = failed ? __builtin_nanf("") : 0.0f;
    if (s == 0 && q.gok) {
        // a block whose wait gave up hands NaN on in its inclusive state, so
        // that every later block of the sequence and the final state show it
        Lane incl = P;
        compose(incl, agg, ch.W, (float)TB);
        incl.a += poison;
        incl.b += poison;
        publish(incls + slot_of(j), lane, incl, tag_incl);
        if (failed && lane == 0)
            __hip_atomic_fetch_add(giveups, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // (3) re-sweep from this segment's starting state, writing y: in one frame
    // when the whole wave's range allows it, else token by token
    Lane R = P;
    for (int w = 0; w < s; ++w) compose(R, lds_lane(sh.s, w, g, lane), ch.W, (float)LS);
    // a segment that starts on a checkpoint token stores its starting state
    static_assert(kCkptTokens % LS == 0, "checkpoints fall on segment starts");
    if (ck && q.active && q.t0 > 0 && q.t0 < T && q.t0 % kCkptTokens == 0)
        store_state(ck + (q.t0 / kCkptTokens - 1) * 3 * B * C, B * C, q.bb * C + q.c, R, ch.W,
                    poison);
    if (q.gok) {
        const TileRowsT<IO> yr(yseq + q.t0 * C, q.voff, q.rowb);
        bool framed = false;
        if constexpr (FULL && !SAFE) {
            SegFrame f;
            const bool ok = seg_frame(R, lds_lane(sh.s, s, g, lane), ch.W, ch.c1, (float)LS,
                                      K[0], xmin, f);
            if (__all(ok || !q.active)) {
                framed = true;
                float A = f.alpha, Bs = f.beta;
#pragma unroll
                for (int t = 0; t < LS; ++t) {
                    float yv = frame_token(A, Bs, f, K[t], V[t], (float)(LS - 1 - t), ch) + poison;
                    if constexpr (GATE) yv *= gate_of(Rg[t]);
                    if (q.active) yr.st(t, yv);
                }
                R = Lane{A, Bs, f.Ae, f.An};
            }
        }
        if (!framed) {
#pragma unroll
            for (int t = 0; t < LS; ++t) {
                if (FULL || q.t0 + t < T) {
                    float yv = step<SAFE>(R, K[t], V[t], ch) + poison;
                    if constexpr (GATE) yv *= gate_of(Rg[t]);
                    if (q.active) yr.st(t, yv);
                }
            }
        }
    }
    if (s_out && q.active && q.t0 <= T - 1 && T - 1 < q.t0 + LS) {
        s_out[(0 * B + q.bb) * C + q.c] = R.a + poison;
        s_out[(1 * B + q.bb) * C + q.c] = R.b + poison;
        s_out[(2 * B + q.bb) * C + q.c] = o_out(lane_o(R, ch.W)) + poison;
    }
}

// 1-D grid over (block, sequence, set of CG groups), set fastest; the host
// guarantees nsets * B < 2^31 so the decode stays in 32 bits
// Waves per SIMD the register allocation must allow: the token registers
// (2 LS per lane) dominate, and the occupancy they leave decides how much of
// the memory latency other workgroups hide.
// The gate's receptance rows add LS registers more.
constexpr int lb_waves_per_simd(int ls, bool gate) {
    return gate ? (ls <= 8 ? 7 : 5) : (ls <= 8 ? 8 : (ls <= 16 ? 6 : 4));
}

template <int CG, int NS, int LS, bool GATE, class IO>
__global__ __launch_bounds__(CG * NS * 64)
__attribute__((amdgpu_waves_per_eu(lb_waves_per_simd(LS, GATE)))) void fwd_lookback_kernel(
    int64_t B, int64_t T, int64_t C, const float *__restrict__ w, const float *__restrict__ u,
    const typename IO::T *__restrict__ k, const typename IO::T *__restrict__ v,
    const typename IO::T *__restrict__ r, typename IO::T *__restrict__ y, const float *s_in,
    float *s_out, float *ck, Word *aggs, Word *incls, uint32_t epoch, uint32_t *giveups,
    uint32_t spin_limit, uint32_t nsets, uint32_t xwin) {
    constexpr int TB = NS * LS;
    __shared__ LbShared<CG, NS> sh;
    // epoch 0: the launch's epoch is header word 1, advanced on the device by
    // the kernel queued before this one (uniform: one read per wave)
    if (epoch == 0) epoch = __builtin_amdgcn_readfirstlane(giveups[1]);
    LbWave q;
    q.lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    q.g = wave % CG;
    q.s = wave / CG;
    const uint32_t per_block = nsets * (uint32_t)B;
    // Within each window of xwin consecutive workgroups (xwin a multiple of 8
    // dividing per_block; 0: the plain order), the 8 dies each take xwin/8 adjacent items (the
    // hardware hands consecutive workgroups to the dies in turn).  A window
    // never straddles two blocks, so every item still waits only on
    // workgroups dispatched before its own, and its predecessors run on its
    // own die as before.
    uint32_t wid = blockIdx.x;
    if (xwin) {
        const uint32_t in = wid % xwin;
        wid += (in % 8u) * (xwin / 8u) + in / 8u - in;
    }
    const uint32_t jb = wid / per_block;
    const uint32_t rem = wid - jb * per_block;
    const uint32_t bb = rem / nsets;
    const uint32_t set = rem - bb * nsets;
    q.bb = bb;
    q.j = jb;
    const int64_t ngroups = (C + 63) >> 6;
    q.grp = (int64_t)set * CG + q.g;
    q.gok = q.grp < ngroups;
    q.c = q.grp * 64 + q.lane;
    q.active = q.gok && q.c < C;
    q.t0 = q.j * TB + (int64_t)q.s * LS;
    q.rowb = (uint32_t)(C * IO::kBytes);
    q.voff = q.active ? (uint32_t)(q.lane * IO::kBytes) : 0u;
    const int64_t base = q.bb * T * C + (q.gok ? q.grp * 64 : 0);

    // channel constants, then this wave's tokens, all issued before any wait:
    // waiting for w and u (issued first) leaves the token loads in flight.
    const int64_t cc = q.active ? q.c : 0;  // a valid channel for every lane
    const float wc = w[cc], uc = u[cc];
    // Every token load is issued unconditionally, back to back, with no branch
    // around them (a branch would make the compiler's wait counts assume the
    // shorter path and wait for all of them at once): rows past the end of the
    // sequence re-read its last row, and a wave whose group lies past the last
    // channel reads group 0 -- valid addresses whose values are never used,
    // since every token loop stops at T and such a wave stores nothing.
    float K[LS], V[LS];
    float Rg[GATE ? LS : 1];  // receptance rows, issued after k and v: used last
    {
        const int64_t t0c = q.t0 < T ? q.t0 : T - 1;  // T >= 1 here
        const int64_t left = T - 1 - t0c;
        const uint32_t tmax =
            __builtin_amdgcn_readfirstlane(left < LS - 1 ? (uint32_t)left : (uint32_t)(LS - 1));
        const TileRowsT<IO> kr(k + base + t0c * C, q.voff, q.rowb);
        const TileRowsT<IO> vr(v + base + t0c * C, q.voff, q.rowb);
#pragma unroll
        for (int t = 0; t < LS; ++t) {
            const uint32_t row = (uint32_t)t < tmax ? (uint32_t)t : tmax;
            K[t] = kr.ld((int)row);
            V[t] = vr.ld((int)row);
        }
        if constexpr (GATE) {
            const TileRowsT<IO> rr(r + base + t0c * C, q.voff, q.rowb);
#pragma unroll
            for (int t = 0; t < LS; ++t)
                Rg[t] = rr.ld((int)((uint32_t)t < tmax ? (uint32_t)t : tmax));
        } else {
            Rg[0] = 0.0f;
        }
    }
    // keep the loads here, in flight while the rest of the prologue runs (the
    // compiler would otherwise sink them into the branches below)
    asm volatile("" ::: "memory");
    const Chan ch = make_chan(q.active ? wc : 0.0f, q.active ? uc : 0.0f);
#pragma unroll
    for (int t = 0; t < LS; ++t) K[t] *= kLog2e;
    const bool fast = __syncthreads_and(chan_fast_ok(ch));
    const bool full = (q.j + 1) * TB <= T;  // the whole block lies inside the sequence
    if (fast) {
        if (full)
            lb_body<CG, NS, LS, false, true, GATE, IO>(B, T, C, ch, q, K, V, Rg, y + base, s_in,
                                                   s_out, ck, aggs, incls, epoch, giveups, spin_limit, sh);
        else
            lb_body<CG, NS, LS, false, false, GATE, IO>(B, T, C, ch, q, K, V, Rg, y + base, s_in,
                                                    s_out, ck, aggs, incls, epoch, giveups, spin_limit, sh);
    } else {
        if (full)
            lb_body<CG, NS, LS, true, true, GATE, IO>(B, T, C, ch, q, K, V, Rg, y + base, s_in,
                                                  s_out, ck, aggs, incls, epoch, giveups, spin_limit, sh);
        else
            lb_body<CG, NS, LS, true, false, GATE, IO>(B, T, C, ch, q, K, V, Rg, y + base, s_in,
                                                   s_out, ck, aggs, incls, epoch, giveups, spin_limit, sh);
    }
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// (CG, NS, LS) variants: CG groups of 64 channels side by side, NS segments of
// LS tokens stacked.  The gated kernel holds a third row array (r), so it is
// compiled only where LS <= 16 leaves the registers for it.  The 16-bit
// formats are compiled for the variants the automatic choice uses.
#define WKV_LB_VARIANTS(X) \
    X(1, 4, 16)            \
    X(1, 8, 32)            \
    X(2, 4, 32)            \
    X(1, 8, 16)            \
    X(1, 4, 32)            \
    X(1, 8, 8)             \
    X(2, 4, 16)            \
    X(2, 2, 16)            \
    X(2, 2, 32)            \
    X(2, 4, 8)             \
    X(4, 2, 16)            \
    X(4, 2, 8)
#define WKV_LB_VARIANTS_16BIT(X) \
    X(1, 4, 16)                  \
    X(1, 4, 32)                  \
    X(1, 8, 16)

constexpr int lb_key(int cg, int ns, int ls) { return (cg * 64 + ns) * 1024 + ls; }

constexpr uint32_t kXcdWindow = 128;
constexpr uint32_t kXcdWindowNarrow = 40;

template <int CG, int NS, int LS, bool GATE, class IO>
hipError_t launch_lb(const FwdArgs &a, const LookbackScratch &sc, hipStream_t st) {
    using T = typename IO::T;
    const int64_t ngroups = (a.C + 63) / 64;
    const int64_t nsets = (ngroups + CG - 1) / CG;
    const int64_t nblocks = (a.T + NS * LS - 1) / (NS * LS);
    const int64_t nslots = nblocks * a.B * ngroups;
    uint32_t *giveups = (uint32_t *)sc.base;
    Word *aggs = (Word *)((char *)sc.base + kLookbackHeaderBytes);
    Word *incls = (Word *)((char *)aggs + align_up((size_t)nslots * kSlotWords * sizeof(Word)));
    // Die-contiguous items (xwin above), chosen from timings on MI355X: windows
    // of 128 where the grid runs in more than one generation of resident
    // workgroups (16-bit activations) or more than two (float32), measured
    // 5-9% and 2-4% faster there and 1-2% slower with fewer generations;
    // windows of 40 where 128 does not divide the workgroups per block but 40
    // does (the B=1 C=5120 stream chunk: 3% faster); never for the gated
    // forward (1.6% slower).
    const int64_t per_block = nsets * a.B;
    const int64_t resident = (int64_t)a.cus * (4 * lb_waves_per_simd(LS, GATE) / (CG * NS));
    const int64_t nwg = per_block * nblocks;
    const bool many = IO::kBytes == 4 ? nwg > 2 * resident : nwg > resident;
    uint32_t xwin = 0;
    if (!GATE) {
        if (per_block % kXcdWindow == 0)
            xwin = many ? kXcdWindow : 0u;
        else if (per_block % kXcdWindowNarrow == 0)
            xwin = kXcdWindowNarrow;
    }
    hipLaunchKernelGGL((fwd_lookback_kernel<CG, NS, LS, GATE, IO>),
                       dim3((unsigned)(nsets * a.B * nblocks)), dim3(CG * NS * 64), 0, st, a.B,
                       a.T, a.C, a.w, a.u, (const T *)a.k, (const T *)a.v, (const T *)a.r,
                       (T *)a.y, a.s_in, a.s_out, a.ck, aggs, incls, sc.epoch, giveups,
                       sc.spin_limit, (uint32_t)nsets, xwin);
    return hipGetLastError();
}

}  // namespace

bool forward_lookback_supported(int cg, int ns, int ls, bool gated, int io) {
    if (gated && ls > 16) return false;
    if (io != kIoF32) {
        switch (lb_key(cg, ns, ls)) {
#define X(CG, NS, LS) case lb_key(CG, NS, LS):
            WKV_LB_VARIANTS_16BIT(X)
#undef X
            return io == kIoF16 || io == kIoBF16;
            default:
                return false;
        }
    }
    switch (lb_key(cg, ns, ls)) {
#define X(CG, NS, LS) case lb_key(CG, NS, LS):
        WKV_LB_VARIANTS(X)
#undef X
        return true;
        default:
            return false;
    }
}

bool lookback_grid_ok(int64_t B, int64_t T, int64_t C, int cg, int ns, int ls) {
    const int64_t nsets = ((C + 63) / 64 + cg - 1) / cg;
    const int64_t nblocks = (T + (int64_t)ns * ls - 1) / ((int64_t)ns * ls);
    // nsets * B * nblocks < 2^31 (grid size; also bounds the 32-bit decode)
    return nsets <= 0x7fffffffLL / B && nsets * B <= 0x7fffffffLL / nblocks;
}

size_t lookback_scratch_bytes(int64_t B, int64_t T, int64_t C, int ns, int ls) {
    const int64_t nblocks = (T + (int64_t)ns * ls - 1) / ((int64_t)ns * ls);
    const int64_t nslots = nblocks * B * ((C + 63) / 64);
    return kLookbackHeaderBytes + 2 * align_up((size_t)nslots * kSlotWords * sizeof(Word));
}

template <int CG, int NS, int LS, class IO>
hipError_t launch_lb_gate(const FwdArgs &a, const LookbackScratch &sc, hipStream_t st) {
    // (a gated call never reaches LS > 16: forward_lookback_supported refuses it)
    if (a.r) return launch_lb<CG, NS, (LS <= 16 ? LS : 16), true, IO>(a, sc, st);
    return launch_lb<CG, NS, LS, false, IO>(a, sc, st);
}

// One workgroup: every thread reads the last device epoch before thread 0
// writes the next; when the range is used up the slots are cleared first
// (vector stores), so that no tag left from the previous pass through the
// range can match.  Word 1 starts at 0 in a fresh buffer, whose slots hold
// no device-range tag, so the first epoch needs no clearing.
__global__ __launch_bounds__(256) void lookback_epoch_kernel(uint32_t *hdr, uint4 *slots,
                                                             size_t n16) {
    const uint32_t e = __hip_atomic_load(hdr + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool wrap = e >= kDeviceEpochLast;
    __syncthreads();
    if (wrap)
        for (size_t i = threadIdx.x; i < n16; i += blockDim.x) slots[i] = make_uint4(0, 0, 0, 0);
    if (threadIdx.x == 0)
        __hip_atomic_store(hdr + 1, (e < kDeviceEpochFirst || wrap) ? kDeviceEpochFirst : e + 1u,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

hipError_t launch_lookback_device_epoch(void *base, size_t bytes, hipStream_t st) {
    if (bytes < kLookbackHeaderBytes || (bytes - kLookbackHeaderBytes) % 16 != 0)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(lookback_epoch_kernel, dim3(1), dim3(256), 0, st, (uint32_t *)base,
                       (uint4 *)((char *)base + kLookbackHeaderBytes),
                       (bytes - kLookbackHeaderBytes) / 16);
    return hipGetLastError();
}

hipError_t launch_forward_lookback(const FwdArgs &a, int cg, int ns, int ls,
                                   const LookbackScratch &sc, hipStream_t st) {
    if (!forward_lookback_supported(cg, ns, ls, a.r != nullptr, a.io)) return hipErrorInvalidValue;
    if (a.io == kIoF32) {
        switch (lb_key(cg, ns, ls)) {
#define X(CG, NS, LS) \
    case lb_key(CG, NS, LS): return launch_lb_gate<CG, NS, LS, IoF32>(a, sc, st);
            WKV_LB_VARIANTS(X)
#undef X
            default:
                return hipErrorInvalidValue;
        }
    }
    switch (lb_key(cg, ns, ls)) {
#define X(CG, NS, LS)                                                      \
    case lb_key(CG, NS, LS):                                              \
        return a.io == kIoF16 ? launch_lb_gate<CG, NS, LS, IoF16>(a, sc, st) \
                              : launch_lb_gate<CG, NS, LS, IoBF16>(a, sc, st);
        WKV_LB_VARIANTS_16BIT(X)
#undef X
        default:
            return hipErrorInvalidValue;
    }
}

}  // namespace wkv

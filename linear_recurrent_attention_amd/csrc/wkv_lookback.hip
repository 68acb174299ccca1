// wkv_lookback.hip -- forward by blocks of tokens chained with a decoupled
// look-back (gfx950).
//
// Same result as the other forward kernels (RWKV architecture deep dive,
// youngju.dev, "WKV mechanism: core computation"; state carried as in the
// rwkv-architecture skill page, "Quick start").  The sequence of every
// (b, 64-channel group) lane group is cut into blocks of NW*LS tokens, and each
// block is one small workgroup: wave s loads its LS tokens of k, v (one 256-byte
// row per load), folds them into a summary, the NW summaries are composed
// through LDS, and the block's aggregate is published.  Wave 0 then walks back
// over earlier blocks of the same lane group, composing their published states
// until it meets one that already holds the whole prefix, publishes the
// block's inclusive state, and every wave re-sweeps its tokens from its own
// starting state, writing y.  Each workgroup touches its k, v and y once, so
// HBM traffic is the algorithmic 12 bytes per lane-token; many independent
// workgroups per CU hide the memory latency.
//
// Ordering and progress.  Workgroups take tickets from an atomic counter and
// process blocks in ticket order, all lane groups' block 0 first, then block 1,
// and so on; a block waits only on blocks with smaller tickets, which started
// earlier and are resident or finished, so the look-back always terminates.
// Flags carry an epoch that the last workgroup of a launch advances (and it
// resets the counters), so consecutive launches on one stream need no clearing
// of the scratch buffer in between.  Every spin is bounded: past the bound the
// block's outputs become NaN instead of hanging.
#include "wkv_device.hpp"
#include "wkv_internal.hpp"

namespace wkv {

namespace {

constexpr uint32_t kAgg = 1u;   // block aggregate published
constexpr uint32_t kIncl = 2u;  // inclusive prefix (state after the block) published
constexpr int kWindow = 8;      // predecessors examined per look-back round
constexpr uint32_t kMaxSpin = 1u << 20;

// Scratch layout (bytes): header | flags[ntiles] | agg[ntiles][4][64] | incl[ntiles][4][64]
struct LbHeader {
    uint32_t ticket;
    uint32_t done;
    uint32_t epoch;
    uint32_t pad[61];
};

__device__ __forceinline__ uint32_t ld_flag(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void put_state(float *slot, int lane, const Lane &L) {
    slot[0 * 64 + lane] = L.a;
    slot[1 * 64 + lane] = L.b;
    slot[2 * 64 + lane] = L.e0;
    slot[3 * 64 + lane] = L.n;
}

__device__ __forceinline__ Lane get_state(const float *slot, int lane) {
    return Lane{slot[0 * 64 + lane], slot[1 * 64 + lane], slot[2 * 64 + lane], slot[3 * 64 + lane]};
}

template <int NW, int LS>
struct LbShared {
    float s[4][NW][64];  // segment summaries
    float p[4][64];      // state at the start of the block
    uint32_t ticket;
    uint32_t epoch;
    uint32_t failed;
};

template <int NW, int LS, bool SAFE>
__device__ __forceinline__ void lb_body(int64_t B, int64_t T, int64_t C, const Chan &ch, int64_t bb,
                                        int64_t c, bool active, int64_t j, int64_t NLG, int64_t lg,
                                        uint32_t ticket, uint32_t epoch, const float *kseq,
                                        const float *vseq, float *yseq, uint32_t voff,
                                        const float *__restrict__ s_in, float *__restrict__ s_out,
                                        uint32_t *flags, float *aggv, float *inclv,
                                        LbShared<NW, LS> &sh) {
    constexpr int TB = NW * LS;
    const int lane = threadIdx.x & 63;
    const int s = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t rowb = (uint32_t)(C * 4);
    const int64_t t0 = j * TB + (int64_t)s * LS;

    // load this wave's tokens (rows past the end of the sequence are not read)
    float K[LS], V[LS];
    {
        const TileRows kr(kseq + t0 * C, voff, rowb), vr(vseq + t0 * C, voff, rowb);
        if (t0 + LS <= T) {
#pragma unroll
            for (int q = 0; q < LS; ++q) {
                K[q] = kr.ld(q);
                V[q] = vr.ld(q);
            }
        } else {
#pragma unroll
            for (int q = 0; q < LS; ++q) {
                K[q] = (t0 + q < T) ? kr.ld(q) : 0.0f;
                V[q] = (t0 + q < T) ? vr.ld(q) : 0.0f;
            }
        }
    }

    // (1) segment summary from the empty state
    Lane S = lane_empty();
#pragma unroll
    for (int q = 0; q < LS; ++q)
        if (t0 + q < T) absorb(S, K[q] * kLog2e, V[q], ch);
    sh.s[0][s][lane] = S.a;
    sh.s[1][s][lane] = S.b;
    sh.s[2][s][lane] = S.e0;
    sh.s[3][s][lane] = S.n;
    __syncthreads();

    if (s == 0) {
        // aggregate of the block: segments 0..NW-1
        Lane agg = S;
#pragma unroll
        for (int w = 1; w < NW; ++w)
            compose(agg, Lane{sh.s[0][w][lane], sh.s[1][w][lane], sh.s[2][w][lane], sh.s[3][w][lane]},
                    ch.W, (float)LS);
        Lane P = lane_empty();  // state at the start of the block
        bool failed = false;
        if (j == 0) {
            if (s_in && active)
                P = lane_at(s_in[(0 * B + bb) * C + c], s_in[(1 * B + bb) * C + c],
                            o_in(s_in[(2 * B + bb) * C + c]));
        } else {
            // publish the aggregate, then walk back
            put_state(aggv + (int64_t)ticket * 256, lane, agg);
            __threadfence();
            if (lane == 0)
                __hip_atomic_store(&flags[ticket], (epoch << 2) | kAgg, __ATOMIC_RELEASE,
                                   __HIP_MEMORY_SCOPE_AGENT);
            int64_t base = j - 1;   // nearest block not yet folded into P
            float covered = 0.0f;   // tokens covered by P
            uint32_t spins = 0;
            for (;;) {
                // lane q < kWindow looks at block base - q
                const int64_t pj = base - lane;
                uint32_t f = 0;
                if (lane < kWindow && pj >= 0) f = ld_flag(&flags[pj * NLG + lg]);
                const bool ready = lane < kWindow && pj >= 0 && (f >> 2) == (epoch & 0x3fffffffu) &&
                                   (f & 3u) != 0;
                const bool incl = ready && (f & 3u) == kIncl;
                const uint64_t not_ready = __ballot(!ready && lane < kWindow && pj >= 0);
                const uint64_t inc = __ballot(incl);
                // consume the leading ready blocks, up to and including the first
                // inclusive one
                const int first_nr = not_ready ? __builtin_ctzll(not_ready) : kWindow;
                const int first_in = inc ? __builtin_ctzll(inc) : kWindow;
                const int avail = (int)((base + 1) < kWindow ? (base + 1) : kWindow);
                int use = first_nr < avail ? first_nr : avail;
                bool done = false;
                if (first_in < use) {
                    use = first_in + 1;
                    done = true;
                }
                if (use == 0) {
                    if (++spins > kMaxSpin) {
                        failed = true;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                    continue;
                }
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                // fold blocks base, base-1, ..., base-use+1 (nearest first)
                Lane X[kWindow];
#pragma unroll
                for (int q = 0; q < kWindow; ++q) {
                    if (q < use) {
                        const int64_t slot = (base - q) * NLG + lg;
                        const bool isin = (inc >> q) & 1ull;
                        X[q] = get_state((isin ? inclv : aggv) + slot * 256, lane);
                    }
                }
#pragma unroll
                for (int q = 0; q < kWindow; ++q) {
                    if (q < use) {
                        compose(X[q], P, ch.W, covered);
                        P = X[q];
                        covered += (float)TB;
                    }
                }
                base -= use;
                if (done || base < 0) break;
            }
        }
        // inclusive state of this block
        Lane incl = P;
        compose(incl, agg, ch.W, (float)TB);
        put_state(inclv + (int64_t)ticket * 256, lane, incl);
        __threadfence();
        if (lane == 0)
            __hip_atomic_store(&flags[ticket], (epoch << 2) | kIncl, __ATOMIC_RELEASE,
                               __HIP_MEMORY_SCOPE_AGENT);
        sh.p[0][lane] = P.a;
        sh.p[1][lane] = P.b;
        sh.p[2][lane] = P.e0;
        sh.p[3][lane] = P.n;
        if (lane == 0) sh.failed = failed ? 1u : 0u;
    }
    __syncthreads();

    // (3) re-sweep from this segment's starting state, writing y
    Lane R{sh.p[0][lane], sh.p[1][lane], sh.p[2][lane], sh.p[3][lane]};
    for (int w = 0; w < s; ++w)
        compose(R, Lane{sh.s[0][w][lane], sh.s[1][w][lane], sh.s[2][w][lane], sh.s[3][w][lane]},
                ch.W, (float)LS);
    const float poison = sh.failed ? __builtin_nanf("") : 0.0f;
    const TileRows yr(yseq + t0 * C, voff, rowb);
#pragma unroll
    for (int q = 0; q < LS; ++q) {
        if (t0 + q < T) {
            const float yv = step<SAFE>(R, K[q] * kLog2e, V[q], ch) + poison;
            if (active) yr.st(q, yv);
        }
    }
    if (s_out && active && t0 <= T - 1 && T - 1 < t0 + LS) {
        s_out[(0 * B + bb) * C + c] = R.a + poison;
        s_out[(1 * B + bb) * C + c] = R.b + poison;
        s_out[(2 * B + bb) * C + c] = o_out(lane_o(R, ch.W)) + poison;
    }
}

template <int NW, int LS>
__global__ __launch_bounds__(NW * 64) void fwd_lookback_kernel(
    int64_t B, int64_t T, int64_t C, const float *__restrict__ w, const float *__restrict__ u,
    const float *__restrict__ k, const float *__restrict__ v, float *__restrict__ y,
    const float *s_in, float *s_out, LbHeader *hdr, uint32_t *flags, float *aggv, float *inclv) {
    __shared__ LbShared<NW, LS> sh;
    constexpr int TB = NW * LS;
    if (threadIdx.x == 0) {
        sh.ticket = atomicAdd(&hdr->ticket, 1u);
        sh.epoch = __hip_atomic_load(&hdr->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    // tickets run 0..gridDim.x-1 within a launch; the modulo only keeps a
    // counter left behind by an aborted launch from indexing past the scratch
    const uint32_t ticket = sh.ticket % gridDim.x;
    const uint32_t epoch = sh.epoch;
    const int64_t ngroups = (C + 63) / 64;
    const int64_t NLG = B * ngroups;
    const int64_t j = ticket / NLG;
    const int64_t lg = ticket - j * NLG;
    const int64_t bb = lg / ngroups;
    const int64_t g = lg - bb * ngroups;
    const int lane = threadIdx.x & 63;
    const int64_t c = g * 64 + lane;
    const bool active = c < C;
    const Chan ch = make_chan(active ? w[c] : 0.0f, active ? u[c] : 0.0f);
    const bool fast = __syncthreads_and(chan_fast_ok(ch));
    const int64_t base = bb * T * C + g * 64;
    const uint32_t voff = active ? (uint32_t)lane * 4u : 0u;
    if (fast)
        lb_body<NW, LS, false>(B, T, C, ch, bb, c, active, j, NLG, lg, ticket, epoch, k + base,
                               v + base, y + base, voff, s_in, s_out, flags, aggv, inclv, sh);
    else
        lb_body<NW, LS, true>(B, T, C, ch, bb, c, active, j, NLG, lg, ticket, epoch, k + base,
                              v + base, y + base, voff, s_in, s_out, flags, aggv, inclv, sh);
    // the last workgroup of the launch readies the scratch for the next one
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t total = gridDim.x;
        if (atomicAdd(&hdr->done, 1u) == total - 1) {
            __hip_atomic_store(&hdr->ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&hdr->done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&hdr->epoch, epoch + 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    (void)TB;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

}  // namespace

bool forward_lookback_supported(int nw, int ls) {
    switch (nw * 1000 + ls) {
        case 4016: case 8016: case 4032: case 8008: case 16008:
            return true;
        default:
            return false;
    }
}

int64_t lookback_tiles(int64_t B, int64_t T, int64_t C, int nw, int ls) {
    const int64_t TB = (int64_t)nw * ls;
    return ((T + TB - 1) / TB) * B * ((C + 63) / 64);
}

size_t lookback_scratch_bytes(int64_t ntiles) {
    return align_up(sizeof(LbHeader)) + align_up((size_t)ntiles * 4) +
           2 * align_up((size_t)ntiles * 256 * sizeof(float));
}

template <int NW, int LS>
static hipError_t launch_lb(const FwdArgs &a, void *scratch, int64_t ntiles, hipStream_t st) {
    char *p = (char *)scratch;
    LbHeader *hdr = (LbHeader *)p;
    p += align_up(sizeof(LbHeader));
    uint32_t *flags = (uint32_t *)p;
    p += align_up((size_t)ntiles * 4);
    float *aggv = (float *)p;
    p += align_up((size_t)ntiles * 256 * sizeof(float));
    float *inclv = (float *)p;
    hipLaunchKernelGGL((fwd_lookback_kernel<NW, LS>), dim3((unsigned)ntiles), dim3(NW * 64), 0, st,
                       a.B, a.T, a.C, a.w, a.u, a.k, a.v, a.y, a.s_in, a.s_out, hdr, flags, aggv,
                       inclv);
    return hipGetLastError();
}

hipError_t launch_forward_lookback(const FwdArgs &a, int nw, int ls, void *scratch,
                                   hipStream_t st) {
    const int64_t ntiles = lookback_tiles(a.B, a.T, a.C, nw, ls);
    switch (nw * 1000 + ls) {
        case 4016: return launch_lb<4, 16>(a, scratch, ntiles, st);
        case 8016: return launch_lb<8, 16>(a, scratch, ntiles, st);
        case 4032: return launch_lb<4, 32>(a, scratch, ntiles, st);
        case 8008: return launch_lb<8, 8>(a, scratch, ntiles, st);
        case 16008: return launch_lb<16, 8>(a, scratch, ntiles, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace wkv

// wkv_api.hip -- C ABI of libwkv: argument checks, kernel choice, launches.
//
// Every check runs on the host before anything touches the HIP runtime, so an
// invalid call returns its status without a launch (and without needing a
// device).  The kernels live in wkv_forward.hip, wkv_step.hip and
// wkv_backward.hip.
#include <atomic>
#include <map>
#include <mutex>
#include <new>
#include <utility>
#include <vector>

#include "../../include/wkv.h"
#include "wkv_internal.hpp"

// Scratch of wkv_forward_noalloc (see launch_with_noalloc_scratch):
// WKV_NOALLOC_SCRATCH_BYTES of device memory per device, zero when the code
// object is loaded and held until the process ends.
constexpr size_t kNoAllocScratchBytes = WKV_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned long long scratch[kNoAllocScratchBytes / 8];

namespace {

using wkv::BwdArgs;
using wkv::FwdArgs;
using wkv::StepArgs;

bool mul_ok(int64_t a, int64_t b, int64_t *out) { return !__builtin_mul_overflow(a, b, out); }

// n elements of 4 bytes (or `elem` bytes), as a byte count, or -1 on overflow.
int64_t bytes_of(int64_t a, int64_t b, int64_t c, int64_t elem = 4) {
    int64_t x, y, z;
    if (!mul_ok(a, b, &x) || !mul_ok(x, c, &y) || !mul_ok(y, elem, &z)) return -1;
    return z;
}

struct Range {
    uintptr_t lo;
    uintptr_t hi;  // exclusive
};

Range rng(const void *p, int64_t bytes) {
    if (!p || bytes <= 0) return Range{0, 0};
    return Range{(uintptr_t)p, (uintptr_t)p + (uintptr_t)bytes};
}

bool overlap(Range a, Range b) {
    if (a.lo == a.hi || b.lo == b.hi) return false;
    return a.lo < b.hi && b.lo < a.hi;
}

// Cached per-device facts (compute-unit count), guarded by a mutex.  Fixed
// arrays indexed by device, so that no call ever allocates host memory for
// them.
constexpr int kMaxDevices = 64;
std::mutex g_mu;
int g_cus[kMaxDevices] = {};

int device_cus() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    std::lock_guard<std::mutex> lk(g_mu);
    if (g_cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        g_cus[dev] = n;
    }
    return g_cus[dev];
}

// Look-back rounds without progress before a wait gives up (a test hook can
// lower it, see wkv_set_lookback_spin_limit).
std::atomic<uint32_t> g_spin_limit{wkv::kDefaultSpinLimit};

// Advances a scratch buffer's host epoch after an accepted launch.  At the end
// of the host's range (below the device-side range) the slots (not the header)
// are cleared by a kernel queued on the stream, so that no stale tag can match
// a reused epoch.
hipError_t advance_epoch(void *p, size_t bytes, uint32_t &epoch, hipStream_t st) {
    if (++epoch < wkv::kDeviceEpochFirst) return hipSuccess;
    epoch = 1;
    return wkv::launch_zero_fill((char *)p + wkv::kLookbackHeaderBytes,
                                 bytes - wkv::kLookbackHeaderBytes, st);
}

// Scratch of the look-back forward owned by the library: one buffer per
// (device, stream), so that calls on different streams never share it.  It is
// allocated on first use and grown, without blocking the host or the device,
// in stream order: the new buffer comes from hipMallocAsync and is zeroed by a
// kernel on the stream, the old one's give-up count is carried over and the
// old buffer released with hipFreeAsync after the launches already queued on
// the stream.  A buffer is kept until wkv_release_stream_scratch or the end of
// the process; its size is bounded by kLookbackScratchMax.  Every launch gets
// a fresh epoch, which tags the states it publishes; the epoch advances only
// when a launch was accepted, under the same lock as the launch itself, so
// launches from several host threads onto one stream stay consistent.
struct Scratch {
    void *p = nullptr;
    size_t bytes = 0;
    uint32_t epoch = 1;
};
std::map<std::pair<int, hipStream_t>, Scratch> g_scratch;

hipError_t launch_with_scratch(const FwdArgs &a, int cg, int ns, int ls, size_t need,
                               hipStream_t st) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lk(g_mu);
    Scratch &s = g_scratch[std::make_pair(dev, st)];
    if (s.bytes < need) {
        const size_t bytes = need < ((size_t)4 << 20) ? ((size_t)4 << 20) : need;
        void *np = nullptr;
        if ((e = hipMallocAsync(&np, bytes, st)) != hipSuccess) return e;
        if ((e = wkv::launch_zero_fill(np, bytes, st)) != hipSuccess) {
            (void)hipFreeAsync(np, st);
            return e;
        }
        if (s.p) {
            if ((e = hipMemcpyAsync(np, s.p, sizeof(uint32_t), hipMemcpyDeviceToDevice, st)) !=
                    hipSuccess ||
                (e = hipFreeAsync(s.p, st)) != hipSuccess) {
                (void)hipFreeAsync(np, st);
                return e;
            }
        }
        s.p = np;
        s.bytes = bytes;
        s.epoch = 1;
    }
    const wkv::LookbackScratch sc{s.p, s.epoch, g_spin_limit.load()};
    e = wkv::launch_forward_lookback(a, cg, ns, ls, sc, st);
    if (e == hipSuccess) e = advance_epoch(s.p, s.bytes, s.epoch, st);
    return e;
}

// Scratch of wkv_forward_noalloc: a fixed array in device memory, one copy per
// device, allocated with the library's code object and zero when loaded.  Its
// address on each device is taken once, with that device current, and kept;
// the host never passes the array's own name to a kernel (in host code that
// name is a stand-in, not a device address).
struct NoAllocScratch {
    void *ptr = nullptr;  // device address of `scratch` on this device
    uint32_t epoch = 1;
};
NoAllocScratch g_noalloc[kMaxDevices];

// Address of this device's copy (under g_mu).
hipError_t noalloc_address(int dev, void **out) {
    NoAllocScratch &n = g_noalloc[dev];
    if (!n.ptr) {
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!ptr) return hipErrorInvalidSymbol;
        n.ptr = ptr;
    }
    *out = n.ptr;
    return hipSuccess;
}

// device_epoch: the call is being recorded into a graph, whose replays cannot
// take a new host epoch each; the launch then takes its epoch on the device
// (a one-workgroup kernel before it advances the header's device epoch).
hipError_t launch_with_noalloc_scratch(const FwdArgs &a, int cg, int ns, int ls,
                                       bool device_epoch, hipStream_t st) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_mu);
    void *p = nullptr;
    if ((e = noalloc_address(dev, &p)) != hipSuccess) return e;
    NoAllocScratch &n = g_noalloc[dev];
    if (device_epoch) {
        if ((e = wkv::launch_lookback_device_epoch(p, kNoAllocScratchBytes, st)) != hipSuccess)
            return e;
        return wkv::launch_forward_lookback(a, cg, ns, ls,
                                            wkv::LookbackScratch{p, 0u, g_spin_limit.load()}, st);
    }
    const wkv::LookbackScratch sc{p, n.epoch, g_spin_limit.load()};
    e = wkv::launch_forward_lookback(a, cg, ns, ls, sc, st);
    if (e == hipSuccess) e = advance_epoch(p, kNoAllocScratchBytes, n.epoch, st);
    return e;
}

// Reads and clears the give-up count in the header at p (synchronous).
hipError_t take_giveups(void *p, uint32_t *count) {
    uint32_t c = 0;
    hipError_t e = hipMemcpy(&c, p, sizeof c, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return e;
    if (c) {
        const uint32_t zero = 0;
        if ((e = hipMemcpy(p, &zero, sizeof zero, hipMemcpyHostToDevice)) != hipSuccess) return e;
    }
    *count += c;
    return hipSuccess;
}

// Largest look-back scratch a call may ask for; longer sequences use the
// segmented kernel, which needs none.
constexpr size_t kLookbackScratchMax = (size_t)256 << 20;

// The plan for a shape.  Pure host arithmetic, given the compute-unit count;
// thresholds from timings on MI355X (256 CUs):
//   - very short sequences, or short ones with many lanes: the lane kernel
//     (one thread per lane, no scan);
//   - very many lanes: the segmented kernel (one workgroup per 64 lanes walks
//     the whole sequence; enough workgroups to fill the chip);
//   - otherwise the look-back kernel, whose workgroups split the sequence as
//     well: blocks of 4 x 32 tokens when that still gives about eight
//     workgroups per CU, else 4 x 16 for more parallelism.
wkv_forward_plan auto_plan(int64_t B, int64_t T, int64_t C, int cus) {
    const int64_t lanes = B * C;
    const int64_t groups = B * ((C + 63) / 64);
    if (T <= 16 || (lanes >= (int64_t)cus * 512 && T <= 128))
        return wkv_forward_plan{WKV_KERNEL_LANE, 0, 0, 0};
    const wkv_forward_plan seg{WKV_KERNEL_SEGMENTED, 16, 16, 64};
    if (lanes >= (int64_t)cus * 1024) return seg;
    const int ls = groups * ((T + 127) / 128) >= (int64_t)cus * 8 ? 32 : 16;
    if (!wkv::lookback_grid_ok(B, T, C, 1, 4, ls) ||
        wkv::lookback_scratch_bytes(B, T, C, 4, ls) > kLookbackScratchMax)
        return seg;
    return wkv_forward_plan{WKV_KERNEL_LOOKBACK, 4, ls, 64};
}

// The automatic plan for the gated forward: the same choice, kept within the
// variants compiled with the gate (look-back blocks of the same length, cut
// into segments of at most 16 tokens).
wkv_forward_plan gated_plan(wkv_forward_plan p) {
    if (p.kernel == WKV_KERNEL_LOOKBACK && p.seg_len > 16) {
        p.segments = p.segments * p.seg_len / 16;
        p.seg_len = 16;
        if (!wkv::forward_lookback_supported(p.channels / 64, p.segments, p.seg_len, true,
                                             wkv::kIoF32))
            p = wkv_forward_plan{WKV_KERNEL_LOOKBACK, 8, 16, 64};
    }
    return p;
}

// Bytes per element of k, v, r, y for a wkv_dtype, 0 for an unknown one.
int64_t elem_bytes(int dtype) {
    switch (dtype) {
        case WKV_DTYPE_F32: return 4;
        case WKV_DTYPE_F16:
        case WKV_DTYPE_BF16: return 2;
        default: return 0;
    }
}

// r: the gate's receptance (same layout as k), NULL for the plain forward.
// esize: bytes per element of k, v, r and y.
wkv_status check_forward(int64_t B, int64_t T, int64_t C, const float *w, const float *u,
                         const void *k, const void *v, const void *y, const float *s_in,
                         const float *s_out, const void *r = nullptr, bool gated = false,
                         int64_t esize = 4) {
    if (B < 0 || T < 0 || C < 0) return WKV_ERR_DIM;
    const int64_t seq = bytes_of(B, T, C, esize);
    const int64_t st = bytes_of(3, B, C);
    const int64_t ch = bytes_of(1, 1, C);
    if (seq < 0 || st < 0 || ch < 0) return WKV_ERR_OVERFLOW;
    if (B * C > 0 && (!w || !u)) return WKV_ERR_NULL;
    if (seq > 0 && (!k || !v || !y)) return WKV_ERR_NULL;
    if (gated && seq > 0 && !r) return WKV_ERR_NULL;
    const Range rw = rng(w, B * C > 0 ? ch : 0), ru = rng(u, B * C > 0 ? ch : 0);
    const Range rk = rng(k, seq), rv = rng(v, seq), ry = rng(y, seq);
    const Range ri = rng(s_in, st), ro = rng(s_out, st), rr = rng(r, seq);
    for (Range x : {rw, ru, rk, rv, ri, ro, rr})
        if (overlap(ry, x)) return WKV_ERR_ALIAS;
    for (Range x : {rw, ru, rk, rv, rr})
        if (overlap(ro, x)) return WKV_ERR_ALIAS;
    if (overlap(ro, ri) && s_out != (float *)s_in) return WKV_ERR_ALIAS;
    return WKV_OK;
}

wkv_status from_hip(hipError_t e) { return e == hipSuccess ? WKV_OK : WKV_ERR_HIP; }

// Checkpoints of a sequence of T tokens: the states before tokens 128, 256, ...
// that lie inside it.
int64_t ckpt_count(int64_t T) { return T > 0 ? (T - 1) / wkv::kCkptTokens : 0; }

// wkv_forward_ex, wkv_forward_gated, wkv_forward_typed and
// wkv_forward_checkpointed: r is NULL for the plain forward; io is the
// wkv_dtype of k, v, r and y; with_ck: the call writes checkpoints to ck.
wkv_status forward_impl(int64_t B, int64_t T, int64_t C, const float *w, const float *u,
                        const void *k, const void *v, const void *r, void *y,
                        const float *state_in, float *state_out, const wkv_forward_plan *plan,
                        bool gated, int io, hipStream_t stream, bool with_ck = false,
                        float *ck = nullptr, bool noalloc = false) {
    const int64_t esize = elem_bytes(io);
    if (esize == 0) return WKV_ERR_UNSUPPORTED;
    wkv_status st = check_forward(B, T, C, w, u, k, v, y, state_in, state_out, r, gated, esize);
    if (st != WKV_OK) return st;
    if (with_ck) {
        const int64_t ckb = bytes_of(3 * ckpt_count(T), B, C);
        if (ckb < 0) return WKV_ERR_OVERFLOW;
        if (ckb > 0 && !ck) return WKV_ERR_NULL;
        const int64_t seq = bytes_of(B, T, C, esize), sts = bytes_of(3, B, C),
                      chs = bytes_of(1, 1, C);
        const Range rc = rng(ck, ckb);
        for (Range x : {rng(w, chs), rng(u, chs), rng(k, seq), rng(v, seq), rng(y, seq),
                        rng(r, gated ? seq : 0), rng(state_in, sts), rng(state_out, sts)})
            if (overlap(rc, x)) return WKV_ERR_ALIAS;
        if (ckb == 0) ck = nullptr;
    } else {
        ck = nullptr;
    }
    wkv_forward_plan p{WKV_KERNEL_AUTO, 0, 0, 0};
    if (plan) p = *plan;
    switch (p.kernel) {
        case WKV_KERNEL_AUTO:
        case WKV_KERNEL_LANE:
            if (p.channels != 0) return WKV_ERR_UNSUPPORTED;
            break;
        case WKV_KERNEL_SEGMENTED:
            if (p.segments == 0) p.segments = 16;
            if (p.seg_len == 0) p.seg_len = 16;
            if (p.channels == 0) p.channels = 64;
            if (!wkv::forward_seg_supported(p.segments, p.seg_len, p.channels, io))
                return WKV_ERR_UNSUPPORTED;
            break;
        case WKV_KERNEL_LOOKBACK:
            if (p.segments == 0) p.segments = 4;
            if (p.seg_len == 0) p.seg_len = 16;
            if (p.channels == 0) p.channels = 64;
            if (p.channels % 64 != 0 ||
                !wkv::forward_lookback_supported(p.channels / 64, p.segments, p.seg_len, gated,
                                                 io))
                return WKV_ERR_UNSUPPORTED;
            break;
        default:
            return WKV_ERR_UNSUPPORTED;
    }
    const int64_t lanes = B * C;
    if (lanes == 0) return WKV_OK;
    if (T == 0) {
        if (!state_out || state_out == state_in) return WKV_OK;
        return from_hip(wkv::launch_state_copy(lanes, state_in, state_out, stream));
    }
    // The look-back kernel tags what it publishes with a per-launch epoch.  A
    // launch recorded into a graph (stream capture) takes its epoch on the
    // device, in the device's fixed scratch, which needs no allocation; a
    // shape whose scratch would not fit there runs the segmented kernel (no
    // state across workgroups) under the automatic plan, and is refused under
    // an explicit look-back plan.
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (stream != nullptr && hipStreamIsCapturing(stream, &cap) != hipSuccess)
        return WKV_ERR_HIP;
    const bool capturing = cap != hipStreamCaptureStatusNone;
    const bool auto_chosen = p.kernel == WKV_KERNEL_AUTO;
    if (auto_chosen) {
        p = auto_plan(B, T, C, device_cus());
        if (gated) p = gated_plan(p);
    }
    FwdArgs a{B, T, C, w, u, k, v, y, state_in, state_out, gated ? r : nullptr, io, ck};
    a.cus = device_cus();
    if (p.kernel == WKV_KERNEL_LANE) {
        if ((lanes + 255) / 256 > 0x7fffffffLL) return WKV_ERR_UNSUPPORTED;
        return from_hip(wkv::launch_forward_lane(a, stream));
    }
    if (p.kernel == WKV_KERNEL_LOOKBACK) {
        const int cg = p.channels / 64;
        if (!wkv::lookback_grid_ok(B, T, C, cg, p.segments, p.seg_len)) return WKV_ERR_UNSUPPORTED;
        const size_t need = wkv::lookback_scratch_bytes(B, T, C, p.segments, p.seg_len);
        if (noalloc || capturing) {
            if (need <= kNoAllocScratchBytes)
                return from_hip(
                    launch_with_noalloc_scratch(a, cg, p.segments, p.seg_len, capturing, stream));
            if (noalloc) return WKV_ERR_WORKSPACE;
            if (!auto_chosen) return WKV_ERR_UNSUPPORTED;
            p = wkv_forward_plan{WKV_KERNEL_SEGMENTED, 16, 16, 64};
        } else {
            if (need > kLookbackScratchMax) return WKV_ERR_UNSUPPORTED;
            return from_hip(launch_with_scratch(a, cg, p.segments, p.seg_len, need, stream));
        }
    }
    if (B * ((C + p.channels - 1) / p.channels) > 0x7fffffffLL) return WKV_ERR_UNSUPPORTED;
    return from_hip(wkv::launch_forward_seg(a, p.segments, p.seg_len, p.channels, stream));
}

// wkv_step, wkv_step_gated and wkv_step_typed: r is NULL for the plain step;
// io is the wkv_dtype of k, v, r and y.
wkv_status step_impl(int64_t L, int64_t B, int64_t C, const float *w, const float *u,
                     const void *k, const void *v, const void *r, void *y,
                     const float *state_in, float *state_out, bool gated, int io,
                     hipStream_t stream) {
    const int64_t esize = elem_bytes(io);
    if (esize == 0) return WKV_ERR_UNSUPPORTED;
    if (L < 0 || B < 0 || C < 0) return WKV_ERR_DIM;
    const int64_t seq = bytes_of(L, B, C, esize);
    const int64_t st = bytes_of(3 * L, B, C);
    const int64_t ch = bytes_of(L, 1, C);
    if (seq < 0 || st < 0 || ch < 0 || L > INT64_MAX / 3) return WKV_ERR_OVERFLOW;
    if (seq == 0) return WKV_OK;
    if (!w || !u || !k || !v || !y || !state_in || !state_out) return WKV_ERR_NULL;
    if (gated && !r) return WKV_ERR_NULL;
    const Range rw = rng(w, ch), ru = rng(u, ch), rk = rng(k, seq), rv = rng(v, seq),
                ry = rng(y, seq), ri = rng(state_in, st), ro = rng(state_out, st),
                rr = rng(r, seq);
    for (Range x : {rw, ru, rk, rv, ri, ro, rr})
        if (overlap(ry, x)) return WKV_ERR_ALIAS;
    for (Range x : {rw, ru, rk, rv, rr})
        if (overlap(ro, x)) return WKV_ERR_ALIAS;
    if (overlap(ro, ri) && state_out != (float *)state_in) return WKV_ERR_ALIAS;
    if (L * B > 0x7fffffffLL) return WKV_ERR_UNSUPPORTED;
    const StepArgs a{L, B, C, w, u, k, v, y, state_in, state_out, gated ? r : nullptr, io};
    return from_hip(wkv::launch_step(a, stream));
}

// wkv_backward, wkv_backward_state, wkv_backward_typed,
// wkv_backward_checkpointed and wkv_backward_gated (the first with no states);
// io is the wkv_dtype of k, v, dy, dk and dv (and r, dr); from_ck: the forward
// states come from the checkpoints cks; gated: dy is the gradient of
// sigmoid(r) * wkv, and dr receives the gradient in r.
wkv_status backward_impl(int64_t B, int64_t T, int64_t C, int io, const float *w, const float *u,
                         const void *k, const void *v, const void *dy, const float *s_in,
                         const float *s_out, const float *ds_out, void *dk, void *dv,
                         float *dw, float *du, float *ds_in, void *workspace,
                         size_t workspace_bytes, hipStream_t stream, bool from_ck = false,
                         const float *cks = nullptr, bool gated = false,
                         const void *r = nullptr, void *dr = nullptr) {
    const int64_t esize = elem_bytes(io);
    if (esize == 0) return WKV_ERR_UNSUPPORTED;
    if (B < 0 || T < 0 || C < 0) return WKV_ERR_DIM;
    const int64_t seq = bytes_of(B, T, C, esize);
    const int64_t ch = bytes_of(1, 1, C);
    const int64_t st = bytes_of(3, B, C);
    if (seq < 0 || ch < 0 || st < 0) return WKV_ERR_OVERFLOW;
    if (C == 0) return WKV_OK;
    if (!dw || !du) return WKV_ERR_NULL;
    if (seq > 0 && (!w || !u || !k || !v || !dy || !dk || !dv)) return WKV_ERR_NULL;
    if (gated && seq > 0 && (!r || !dr)) return WKV_ERR_NULL;
    if (ds_out && !s_out && B > 0) return WKV_ERR_NULL;
    const int64_t ckb = from_ck ? bytes_of(3 * ckpt_count(T), B, C) : 0;
    if (ckb < 0) return WKV_ERR_OVERFLOW;
    if (ckb > 0 && !cks) return WKV_ERR_NULL;
    const size_t need = wkv::backward_workspace_bytes(B, T, C);
    if (need > 0 && (!workspace || workspace_bytes < need)) return WKV_ERR_WORKSPACE;
    const Range rw = rng(w, seq > 0 ? ch : 0), ru = rng(u, seq > 0 ? ch : 0);
    const Range rk = rng(k, seq), rv = rng(v, seq), rg = rng(dy, seq);
    const Range rsi = rng(s_in, st), rso = rng(ds_out ? s_out : nullptr, st),
                rdso = rng(ds_out, st), rck = rng(cks, ckb);
    const Range rdk = rng(dk, seq), rdv = rng(dv, seq), rdw = rng(dw, ch), rdu = rng(du, ch);
    const Range rdsi = rng(ds_in, st);
    const Range rws = rng(workspace, (int64_t)need);
    const Range rr = rng(gated ? r : nullptr, seq), rdr = rng(gated ? dr : nullptr, seq);
    const Range outs[] = {rdk, rdv, rdw, rdu, rws, rdsi, rdr};
    constexpr int kOuts = 7;
    for (int i = 0; i < kOuts; ++i) {
        for (Range q : {rw, ru, rk, rv, rg, rsi, rso, rck, rr})
            if (overlap(outs[i], q)) return WKV_ERR_ALIAS;
        // d_state_in may replace d_state_out exactly (read before it is written)
        if (overlap(outs[i], rdso) && !(i == 5 && (const float *)ds_in == ds_out))
            return WKV_ERR_ALIAS;
        for (int j = i + 1; j < kOuts; ++j)
            if (overlap(outs[i], outs[j])) return WKV_ERR_ALIAS;
    }
    BwdArgs a{B, T, C, w, u, k, v, dy, dk, dv, dw, du, workspace};
    a.io = io;
    a.s_in = s_in;
    a.s_out = s_out;
    a.ds_out = ds_out;
    a.ds_in = ds_in;
    a.from_ck = from_ck;
    a.ck = ckb > 0 ? cks : nullptr;
    a.r = gated ? r : nullptr;
    a.dr = gated ? dr : nullptr;
    return from_hip(wkv::launch_backward(a, stream));
}

// Scratch of the token shift's backward: one dmu partial per (sequence,
// 256-token tile, mix, channel).
int64_t shift_bwd_ws_bytes(int64_t B, int64_t T, int64_t C, int64_t M) {
    if (B <= 0 || T <= 0 || C <= 0 || M <= 0) return 0;
    const int64_t n = bytes_of(wkv::shift_bwd_tiles(T) * B, M, C);
    return n < 0 ? -1 : (n + 255) / 256 * 256;
}

// wkv_token_shift and wkv_token_shift_typed: io is the wkv_dtype of x, x_prev,
// out and x_prev_out (mu is float32).
wkv_status token_shift_impl(int64_t B, int64_t T, int64_t C, int64_t M, int io,
                            const float *mu, const void *x, const void *x_prev, void *out,
                            void *x_prev_out, hipStream_t stream) {
    const int64_t esize = elem_bytes(io);
    if (esize == 0) return WKV_ERR_UNSUPPORTED;
    if (B < 0 || T < 0 || C < 0 || M < 0) return WKV_ERR_DIM;
    const int64_t seq = bytes_of(B, T, C, esize);
    const int64_t lanes = bytes_of(1, B, C, esize);
    const int64_t mus = bytes_of(M, 1, C);
    const int64_t outs = seq < 0 ? -1 : bytes_of(M, 1, seq, 1);
    if (seq < 0 || lanes < 0 || mus < 0 || outs < 0) return WKV_ERR_OVERFLOW;
    if (M > WKV_TOKEN_SHIFT_MAX_MIXES) return WKV_ERR_UNSUPPORTED;
    if (lanes == 0) return WKV_OK;
    if (seq > 0 && !x) return WKV_ERR_NULL;
    if (outs > 0 && (!mu || !out)) return WKV_ERR_NULL;
    const Range rmu = rng(mu, seq > 0 ? mus : 0), rx = rng(x, seq), rp = rng(x_prev, lanes);
    const Range ro = rng(out, outs), rpo = rng(x_prev_out, lanes);
    for (Range q : {rmu, rx, rp, rpo})
        if (overlap(ro, q)) return WKV_ERR_ALIAS;
    for (Range q : {rmu, rx})
        if (overlap(rpo, q)) return WKV_ERR_ALIAS;
    if (overlap(rpo, rp) && x_prev_out != (const void *)x_prev) return WKV_ERR_ALIAS;
    if (!x_prev_out && outs == 0) return WKV_OK;
    wkv::ShiftArgs a{B, T, C, M, mu, x, x_prev, out, x_prev_out};
    a.io = io;
    const bool in_place = x_prev_out != nullptr && x_prev_out == (const void *)x_prev;
    return from_hip(wkv::launch_token_shift(a, in_place, stream));
}

// wkv_token_shift_backward and wkv_token_shift_backward_typed: io is the
// wkv_dtype of x, x_prev, d_out, d_x_prev_out, dx and d_x_prev.
wkv_status token_shift_backward_impl(int64_t B, int64_t T, int64_t C, int64_t M, int io,
                                     const float *mu, const void *x, const void *x_prev,
                                     const void *d_out, const void *d_x_prev_out, void *dx,
                                     void *d_x_prev, float *dmu, void *workspace,
                                     size_t workspace_bytes, hipStream_t stream) {
    const int64_t esize = elem_bytes(io);
    if (esize == 0) return WKV_ERR_UNSUPPORTED;
    if (B < 0 || T < 0 || C < 0 || M < 0) return WKV_ERR_DIM;
    const int64_t seq = bytes_of(B, T, C, esize);
    const int64_t lanes = bytes_of(1, B, C, esize);
    const int64_t mus = bytes_of(M, 1, C);
    const int64_t outs = seq < 0 ? -1 : bytes_of(M, 1, seq, 1);
    const int64_t need = shift_bwd_ws_bytes(B, T, C, M);
    if (seq < 0 || lanes < 0 || mus < 0 || outs < 0 || need < 0) return WKV_ERR_OVERFLOW;
    if (M > WKV_TOKEN_SHIFT_MAX_MIXES) return WKV_ERR_UNSUPPORTED;
    if (seq > 0 && (!x || !dx)) return WKV_ERR_NULL;
    if (outs > 0 && (!mu || !d_out)) return WKV_ERR_NULL;
    if (mus > 0 && !dmu) return WKV_ERR_NULL;
    if (need > 0 && (!workspace || workspace_bytes < (size_t)need)) return WKV_ERR_WORKSPACE;
    const Range rmu = rng(mu, mus), rx = rng(x, seq), rxp = rng(x_prev, lanes),
                rd = rng(d_out, outs), rdp = rng(d_x_prev_out, lanes);
    const Range o[] = {rng(dx, seq), rng(d_x_prev, lanes), rng(dmu, mus), rng(workspace, need)};
    for (int i = 0; i < 4; ++i) {
        for (Range q : {rmu, rx, rxp, rd, rdp})
            if (overlap(o[i], q)) return WKV_ERR_ALIAS;
        for (int j = i + 1; j < 4; ++j)
            if (overlap(o[i], o[j])) return WKV_ERR_ALIAS;
    }
    wkv::ShiftBwdArgs a{B, T, C, M, mu, x, x_prev, d_out, d_x_prev_out, dx, d_x_prev, dmu,
                        (float *)workspace};
    a.io = io;
    return from_hip(wkv::launch_token_shift_backward(a, stream));
}

}  // namespace

extern "C" {

WKV_API const char *wkv_status_string(wkv_status s) {
    switch (s) {
        case WKV_OK: return "ok";
        case WKV_ERR_NULL: return "a required pointer is NULL";
        case WKV_ERR_DIM: return "a dimension is negative";
        case WKV_ERR_OVERFLOW: return "a tensor's byte size overflows int64";
        case WKV_ERR_ALIAS: return "an output overlaps an input or another output";
        case WKV_ERR_WORKSPACE: return "workspace missing or too small";
        case WKV_ERR_UNSUPPORTED: return "no compiled kernel for this plan or shape";
        case WKV_ERR_HIP: return "HIP runtime or launch error";
        case WKV_ERR_LOOKBACK:
            return "a look-back wait gave up: the affected forward outputs and states are NaN";
        default: return "unknown status";
    }
}

WKV_API wkv_status wkv_forward_plan_auto(int64_t B, int64_t T, int64_t C, wkv_forward_plan *plan) {
    if (!plan) return WKV_ERR_NULL;
    if (B < 0 || T < 0 || C < 0) return WKV_ERR_DIM;
    if (bytes_of(B, T, C) < 0) return WKV_ERR_OVERFLOW;
    *plan = auto_plan(B, T, C, device_cus());
    return WKV_OK;
}

WKV_API wkv_status wkv_forward_ex(int64_t B, int64_t T, int64_t C, const float *w, const float *u,
                                  const float *k, const float *v, float *y,
                                  const float *state_in, float *state_out,
                                  const wkv_forward_plan *plan, hipStream_t stream) {
    return forward_impl(B, T, C, w, u, k, v, nullptr, y, state_in, state_out, plan, false,
                        WKV_DTYPE_F32, stream);
}

WKV_API wkv_status wkv_forward_gated(int64_t B, int64_t T, int64_t C, const float *w,
                                     const float *u, const float *k, const float *v,
                                     const float *r, float *y, const float *state_in,
                                     float *state_out, const wkv_forward_plan *plan,
                                     hipStream_t stream) {
    return forward_impl(B, T, C, w, u, k, v, r, y, state_in, state_out, plan, true,
                        WKV_DTYPE_F32, stream);
}

WKV_API wkv_status wkv_forward_typed(int64_t B, int64_t T, int64_t C, wkv_dtype dtype,
                                     const float *w, const float *u, const void *k,
                                     const void *v, const void *r, void *y,
                                     const float *state_in, float *state_out,
                                     const wkv_forward_plan *plan, hipStream_t stream) {
    return forward_impl(B, T, C, w, u, k, v, r, y, state_in, state_out, plan, r != nullptr,
                        (int)dtype, stream);
}

WKV_API wkv_status wkv_forward(int64_t B, int64_t T, int64_t C, const float *w, const float *u,
                               const float *k, const float *v, float *y, const float *state_in,
                               float *state_out, hipStream_t stream) {
    return wkv_forward_ex(B, T, C, w, u, k, v, y, state_in, state_out, nullptr, stream);
}

WKV_API wkv_status wkv_step(int64_t L, int64_t B, int64_t C, const float *w, const float *u,
                            const float *k, const float *v, float *y, const float *state_in,
                            float *state_out, hipStream_t stream) {
    return step_impl(L, B, C, w, u, k, v, nullptr, y, state_in, state_out, false, WKV_DTYPE_F32,
                     stream);
}

WKV_API wkv_status wkv_step_gated(int64_t L, int64_t B, int64_t C, const float *w,
                                  const float *u, const float *k, const float *v,
                                  const float *r, float *y, const float *state_in,
                                  float *state_out, hipStream_t stream) {
    return step_impl(L, B, C, w, u, k, v, r, y, state_in, state_out, true, WKV_DTYPE_F32, stream);
}

WKV_API wkv_status wkv_step_typed(int64_t L, int64_t B, int64_t C, wkv_dtype dtype,
                                  const float *w, const float *u, const void *k, const void *v,
                                  const void *r, void *y, const float *state_in,
                                  float *state_out, hipStream_t stream) {
    return step_impl(L, B, C, w, u, k, v, r, y, state_in, state_out, r != nullptr, (int)dtype,
                     stream);
}

WKV_API wkv_status wkv_token_shift(int64_t B, int64_t T, int64_t C, int64_t M, const float *mu,
                                   const float *x, const float *x_prev, float *out,
                                   float *x_prev_out, hipStream_t stream) {
    return token_shift_impl(B, T, C, M, WKV_DTYPE_F32, mu, x, x_prev, out, x_prev_out, stream);
}

WKV_API wkv_status wkv_token_shift_typed(int64_t B, int64_t T, int64_t C, int64_t M,
                                         wkv_dtype dtype, const float *mu, const void *x,
                                         const void *x_prev, void *out, void *x_prev_out,
                                         hipStream_t stream) {
    return token_shift_impl(B, T, C, M, (int)dtype, mu, x, x_prev, out, x_prev_out, stream);
}

WKV_API size_t wkv_token_shift_backward_workspace_size(int64_t B, int64_t T, int64_t C,
                                                       int64_t M) {
    if (B < 0 || T < 0 || C < 0 || M < 0 || M > WKV_TOKEN_SHIFT_MAX_MIXES) return 0;
    const int64_t n = shift_bwd_ws_bytes(B, T, C, M);
    return n < 0 ? 0 : (size_t)n;
}

WKV_API wkv_status wkv_token_shift_backward(int64_t B, int64_t T, int64_t C, int64_t M,
                                            const float *mu, const float *x,
                                            const float *x_prev, const float *d_out,
                                            const float *d_x_prev_out, float *dx,
                                            float *d_x_prev, float *dmu, void *workspace,
                                            size_t workspace_bytes, hipStream_t stream) {
    return token_shift_backward_impl(B, T, C, M, WKV_DTYPE_F32, mu, x, x_prev, d_out,
                                     d_x_prev_out, dx, d_x_prev, dmu, workspace,
                                     workspace_bytes, stream);
}

WKV_API wkv_status wkv_token_shift_backward_typed(int64_t B, int64_t T, int64_t C, int64_t M,
                                                  wkv_dtype dtype, const float *mu,
                                                  const void *x, const void *x_prev,
                                                  const void *d_out, const void *d_x_prev_out,
                                                  void *dx, void *d_x_prev, float *dmu,
                                                  void *workspace, size_t workspace_bytes,
                                                  hipStream_t stream) {
    return token_shift_backward_impl(B, T, C, M, (int)dtype, mu, x, x_prev, d_out,
                                     d_x_prev_out, dx, d_x_prev, dmu, workspace,
                                     workspace_bytes, stream);
}

WKV_API size_t wkv_backward_workspace_size(int64_t B, int64_t T, int64_t C) {
    if (B < 0 || T < 0 || C < 0 || bytes_of(B, T, C) < 0) return 0;
    return wkv::backward_workspace_bytes(B, T, C);
}

WKV_API wkv_status wkv_backward(int64_t B, int64_t T, int64_t C, const float *w, const float *u,
                                const float *k, const float *v, const float *dy, float *dk,
                                float *dv, float *dw, float *du, void *workspace,
                                size_t workspace_bytes, hipStream_t stream) {
    return backward_impl(B, T, C, WKV_DTYPE_F32, w, u, k, v, dy, nullptr, nullptr, nullptr, dk,
                         dv, dw, du, nullptr, workspace, workspace_bytes, stream);
}

WKV_API wkv_status wkv_backward_state(int64_t B, int64_t T, int64_t C, const float *w,
                                      const float *u, const float *k, const float *v,
                                      const float *dy, const float *state_in,
                                      const float *state_out, const float *d_state_out,
                                      float *dk, float *dv, float *dw, float *du,
                                      float *d_state_in, void *workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
    return backward_impl(B, T, C, WKV_DTYPE_F32, w, u, k, v, dy, state_in, state_out,
                         d_state_out, dk, dv, dw, du, d_state_in, workspace, workspace_bytes,
                         stream);
}

WKV_API wkv_status wkv_backward_typed(int64_t B, int64_t T, int64_t C, wkv_dtype dtype,
                                      const float *w, const float *u, const void *k,
                                      const void *v, const void *dy, const float *state_in,
                                      const float *state_out, const float *d_state_out,
                                      void *dk, void *dv, float *dw, float *du,
                                      float *d_state_in, void *workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
    return backward_impl(B, T, C, (int)dtype, w, u, k, v, dy, state_in, state_out, d_state_out,
                         dk, dv, dw, du, d_state_in, workspace, workspace_bytes, stream);
}

WKV_API wkv_status wkv_forward_checkpointed(int64_t B, int64_t T, int64_t C, wkv_dtype dtype,
                                            const float *w, const float *u, const void *k,
                                            const void *v, const void *r, void *y,
                                            const float *state_in, float *state_out,
                                            float *checkpoints, const wkv_forward_plan *plan,
                                            hipStream_t stream) {
    return forward_impl(B, T, C, w, u, k, v, r, y, state_in, state_out, plan, r != nullptr,
                        (int)dtype, stream, true, checkpoints);
}

WKV_API wkv_status wkv_backward_checkpointed(int64_t B, int64_t T, int64_t C, wkv_dtype dtype,
                                             const float *w, const float *u, const void *k,
                                             const void *v, const void *dy,
                                             const float *state_in, const float *checkpoints,
                                             const float *state_out, const float *d_state_out,
                                             void *dk, void *dv, float *dw, float *du,
                                             float *d_state_in, void *workspace,
                                             size_t workspace_bytes, hipStream_t stream) {
    return backward_impl(B, T, C, (int)dtype, w, u, k, v, dy, state_in, state_out, d_state_out,
                         dk, dv, dw, du, d_state_in, workspace, workspace_bytes, stream, true,
                         checkpoints);
}

WKV_API wkv_status wkv_backward_gated(int64_t B, int64_t T, int64_t C, wkv_dtype dtype,
                                      const float *w, const float *u, const void *k,
                                      const void *v, const void *r, const void *dy,
                                      const float *state_in, const float *checkpoints,
                                      const float *state_out, const float *d_state_out,
                                      void *dk, void *dv, void *dr, float *dw, float *du,
                                      float *d_state_in, void *workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
    return backward_impl(B, T, C, (int)dtype, w, u, k, v, dy, state_in, state_out, d_state_out,
                         dk, dv, dw, du, d_state_in, workspace, workspace_bytes, stream,
                         checkpoints != nullptr, checkpoints, true, r, dr);
}

WKV_API wkv_status wkv_forward_noalloc(int64_t B, int64_t T, int64_t C, const float *w,
                                       const float *u, const float *k, const float *v, float *y,
                                       const float *state_in, float *state_out,
                                       hipStream_t stream) {
    return forward_impl(B, T, C, w, u, k, v, nullptr, y, state_in, state_out, nullptr, false,
                        WKV_DTYPE_F32, stream, false, nullptr, true);
}

WKV_API size_t wkv_forward_scratch_size(int64_t B, int64_t T, int64_t C) {
    if (B < 0 || T < 0 || C < 0 || bytes_of(B, T, C) < 0 || B * C == 0 || T == 0) return 0;
    const wkv_forward_plan p = auto_plan(B, T, C, device_cus());
    if (p.kernel != WKV_KERNEL_LOOKBACK) return 0;
    return wkv::lookback_scratch_bytes(B, T, C, p.segments, p.seg_len);
}

WKV_API wkv_status wkv_release_stream_scratch(hipStream_t stream) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return WKV_ERR_HIP;
    std::lock_guard<std::mutex> lk(g_mu);
    auto it = g_scratch.find(std::make_pair(dev, stream));
    if (it == g_scratch.end()) return WKV_OK;
    const hipError_t e = it->second.p ? hipFreeAsync(it->second.p, stream) : hipSuccess;
    g_scratch.erase(it);
    return from_hip(e);
}

WKV_API wkv_status wkv_lookback_status(hipStream_t stream) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return WKV_ERR_HIP;
    if (hipStreamSynchronize(stream) != hipSuccess) return WKV_ERR_HIP;
    std::lock_guard<std::mutex> lk(g_mu);
    uint32_t count = 0;
    auto it = g_scratch.find(std::make_pair(dev, stream));
    if (it != g_scratch.end() && it->second.p && take_giveups(it->second.p, &count) != hipSuccess)
        return WKV_ERR_HIP;
    if (dev >= 0 && dev < kMaxDevices && g_noalloc[dev].ptr &&
        take_giveups(g_noalloc[dev].ptr, &count) != hipSuccess)
        return WKV_ERR_HIP;
    return count ? WKV_ERR_LOOKBACK : WKV_OK;
}

WKV_API uint32_t wkv_set_lookback_spin_limit(uint32_t rounds) { return g_spin_limit.exchange(rounds); }

}  // extern "C"

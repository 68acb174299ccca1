// wkv_internal.hpp -- launcher interface between the host dispatcher
// (wkv_api.hip) and the kernel translation units.  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace wkv {

// Element format of k, v, r and y (the values of wkv_dtype); w, u and the
// state are always float32.
constexpr int kIoF32 = 0, kIoF16 = 1, kIoBF16 = 2;

// Tokens between two checkpoints of the forward state: the backward's tile.
constexpr int64_t kCkptTokens = 128;

// r: receptance of the time-mixing gate, same layout as k; NULL: y = wkv,
// else y = sigmoid(r) * wkv.  k, v, r, y hold elements of format `io`.
// ck: NULL, or [(T-1)/kCkptTokens][3][B][C]: the state before token
// (i+1)*kCkptTokens goes to ck[i] (every forward kernel writes them).
struct FwdArgs {
    int64_t B, T, C;
    const float *w, *u;
    const void *k, *v;
    void *y;
    const float *s_in;
    float *s_out;
    const void *r;
    int io;
    float *ck = nullptr;
    int cus = 256;  // compute units of the device (sizes launch choices)
};

struct StepArgs {
    int64_t L, B, C;
    const float *w, *u;
    const void *k, *v;
    void *y;
    const float *s_in;
    float *s_out;
    const void *r;
    int io;
};

// x, x_prev, out and x_prev_out hold elements of format `io`; mu is float32.
struct ShiftArgs {
    int64_t B, T, C, M;
    const float *mu;
    const void *x, *x_prev;
    void *out, *x_prev_out;
    int io = kIoF32;
};

// s_in: state before the first token (NULL: empty); s_out, ds_out: the state
// the forward handed on and the upstream gradient in its coordinates (NULL:
// none); ds_in: gradient with respect to s_in (NULL: not wanted).
// k, v, dy, dk, dv hold elements of format `io`.
struct BwdArgs {
    int64_t B, T, C;
    const float *w, *u;
    const void *k, *v, *dy;
    void *dk, *dv;
    float *dw, *du;
    void *ws;
    const float *s_in, *s_out, *ds_out;
    float *ds_in;
    int io;
    // from_ck: the forward states are rebuilt tile by tile from the forward's
    // checkpoints ck (layout of FwdArgs::ck; NULL when T <= kCkptTokens, which
    // has none) instead of by a first pass over k and v
    const float *ck = nullptr;
    bool from_ck = false;
    // r: NULL, or the receptance of a gated forward (layout of k): dy is then
    // the gradient of sigmoid(r) * wkv, and dr receives its gradient in r
    const void *r = nullptr;
    void *dr = nullptr;
};

// forward (wkv_forward.hip)
hipError_t launch_forward_lane(const FwdArgs &a, hipStream_t st);
// (16-bit formats: compiled for the default variant only)
bool forward_seg_supported(int nseg, int ls, int cw, int io);
hipError_t launch_forward_seg(const FwdArgs &a, int nseg, int ls, int cw, hipStream_t st);
hipError_t launch_state_copy(int64_t lanes, const float *s_in, float *s_out, hipStream_t st);

// Fills n bytes (a multiple of 4) with zeros with a kernel on st (wkv_forward.hip).
hipError_t launch_zero_fill(void *p, size_t bytes, hipStream_t st);

// forward with decoupled look-back (wkv_lookback.hip)
// The scratch starts with a header of kLookbackHeaderBytes: word 0 a 32-bit
// count of look-back waits that gave up (the kernel adds to it; the host reads
// and clears it), word 1 the epoch of the last launch that took its epoch on
// the device (see below), then the slot arrays.
constexpr size_t kLookbackHeaderBytes = 256;
// Epochs tag what a launch publishes, so that no launch mistakes a slot left
// by an earlier one for its own.  Epochs the host hands out stay below
// kDeviceEpochFirst; a launch recorded into a graph cannot take a new epoch
// from the host at each replay, so it takes one on the device instead: a
// one-workgroup kernel queued before it advances header word 1 through
// [kDeviceEpochFirst, kDeviceEpochLast] (clearing the slots when the range
// wraps), and the forward kernel, given epoch 0, reads that word.  The two
// ranges never meet, so host-epoch and device-epoch launches can share one
// buffer.
constexpr uint32_t kDeviceEpochFirst = 0x30000000u;
constexpr uint32_t kDeviceEpochLast = 0x3fffffffu;  // tags hold 30 bits of epoch
struct LookbackScratch {
    void *base;           // header then slots; zero-initialised before first use
    uint32_t epoch;       // distinct for every launch on it; 0: read header word 1
    uint32_t spin_limit;  // look-back rounds without progress before a wait gives up
};
// Queues the device-side epoch advance for a buffer of `bytes` (the header
// included) on st.
hipError_t launch_lookback_device_epoch(void *base, size_t bytes, hipStream_t st);
// Default spin limit: 2^16 rounds of a sleep and a device-scope load, tens of
// milliseconds, far above any wait in a healthy launch.
constexpr uint32_t kDefaultSpinLimit = 1u << 16;
// (cg, ns, ls): groups of 64 channels side by side, segments stacked, tokens
// per segment
// (the gated kernel is compiled for the variants with ls <= 16 only, and the
// 16-bit formats for the variants the automatic choice uses)
bool forward_lookback_supported(int cg, int ns, int ls, bool gated, int io);
bool lookback_grid_ok(int64_t B, int64_t T, int64_t C, int cg, int ns, int ls);
// bytes of scratch a look-back launch needs, the header included
size_t lookback_scratch_bytes(int64_t B, int64_t T, int64_t C, int ns, int ls);
hipError_t launch_forward_lookback(const FwdArgs &a, int cg, int ns, int ls,
                                   const LookbackScratch &sc, hipStream_t st);

// step (wkv_step.hip)
hipError_t launch_step(const StepArgs &a, hipStream_t st);

// token shift (wkv_shift.hip); largest number of mixes per call
constexpr int64_t kMaxMixes = 8;
hipError_t launch_token_shift(const ShiftArgs &a, bool in_place_state, hipStream_t st);

// Backward of the token shift: d_out [M][B][T][C] and d_xpo [B][C] (NULL: zero)
// in; dx [B][T][C], dxp [B][C] (NULL: not wanted) and dmu [M][C] out; part is
// scratch of shift_bwd_tiles(T) * B * M * C floats.  x, x_prev, d_out, d_xpo,
// dx and dxp hold elements of format `io`; mu, dmu and part are float32.
struct ShiftBwdArgs {
    int64_t B, T, C, M;
    const float *mu;
    const void *x, *x_prev, *d_out, *d_xpo;
    void *dx, *dxp;
    float *dmu, *part;
    int io = kIoF32;
};
int64_t shift_bwd_tiles(int64_t T);
hipError_t launch_token_shift_backward(const ShiftBwdArgs &a, hipStream_t st);

// backward (wkv_backward.hip)
size_t backward_workspace_bytes(int64_t B, int64_t T, int64_t C);
hipError_t launch_backward(const BwdArgs &a, hipStream_t st);

}  // namespace wkv

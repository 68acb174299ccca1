/*
 * wkv.h -- C ABI of libwkv, the RWKV WKV time-mixing operator on AMD MI355X (gfx950).
 *
 * The operator (RWKV architecture deep dive, youngju.dev, section "WKV
 * mechanism: core computation"): for each lane (b, c) and token t,
 *
 *   wkv_t = ( sum_{i<t} e^{-(t-1-i) w + k_i} v_i + e^{u + k_t} v_t )
 *         / ( sum_{i<t} e^{-(t-1-i) w + k_i}     + e^{u + k_t}     )
 *
 * with a per-channel decay rate w = exp(decay) > 0 and a bonus u that only the
 * current token receives.  The same operator runs in GPT mode over a whole
 * sequence and in RNN mode over chunks or single tokens with a state carried
 * between calls (section "Duality"; rwkv-architecture skill page, "Quick
 * start" and "Workflow 2: Long context processing"); any chunking gives the
 * same outputs as one call over the whole sequence.
 *
 * The state (section "Numerical stability via log-space computation") is three
 * planes per lane: a (scaled numerator), b (scaled denominator) and o (the
 * running maximum exponent, natural-log units).  It stands for the running
 * sums A = a e^o and B = b e^o of every token seen so far, each decayed by
 * e^{-w} per later token; u is not part of it.  The empty state is a = b = 0
 * with o = -1e38 (or -inf, or any o <= -1e30).  A state is defined only up to
 * a common scale: (a e^d, b e^d, o - d) is the same state.
 *
 * Memory and ownership
 *   - Every tensor argument is a device pointer to float32 (IEEE binary32),
 *     except k, v, r and y of the *_typed entry points, which may be 16-bit
 *     (wkv_dtype).  Tensors are allocated and owned by the caller; the library
 *     never frees them and never keeps them after the call returns.
 *   - Layouts are dense row-major with the channel index fastest:
 *       k, v, y, dy, dk, dv : [B][T][C]
 *       w, u, dw, du        : [C]             (wkv_step: w, u are [L][C])
 *       state               : [3][B][C]       planes a, b, o
 *                                             (wkv_step: [L][3][B][C])
 *   - The library owns nothing of the caller's.  The backward and the token
 *     shift's backward take their scratch from the caller (workspace).  The
 *     forward's look-back kernel keeps one scratch buffer per (device, stream)
 *     for the states that workgroups pass along a sequence: the forward's
 *     signature (wkv_forward(B,T,C,w,u,k,v,y,state_in,state_out)) has no
 *     workspace argument.  That buffer holds a 256-byte header and two slot
 *     arrays of 2 KiB per (block, sequence, 64-channel group), for example
 *     8 MiB at B=8 T=1024 C=2048, at most 256 MiB (longer shapes use a kernel
 *     that needs none).  It is allocated in stream order (hipMallocAsync) on
 *     the first call that needs it, grown in stream order (the old buffer is
 *     released with hipFreeAsync after the launches already queued on the
 *     stream, so no call blocks the host or the device), and kept until
 *     wkv_release_stream_scratch(stream) or the end of the process; a caller
 *     that cycles through many streams releases each one it retires.
 *
 * Execution
 *   - Every call is asynchronous on `stream` (0 = the default stream) and
 *     runs on the device that is current on the calling thread.  Calls on one
 *     stream run in order.
 *   - Calls may be captured into a HIP graph (on a non-default stream).  A
 *     look-back forward recorded under capture allocates nothing: it runs in
 *     the device's fixed scratch (the array of wkv_forward_noalloc, see there)
 *     and takes its per-launch tag on the device, from a one-workgroup kernel
 *     recorded before it, so every replay is a fresh launch.  Like
 *     wkv_forward_noalloc calls, replays of such graphs that overlap in time
 *     on one device race on that array: callers serialise them (replays on
 *     one stream are serialised already).  A shape whose look-back scratch
 *     exceeds WKV_NOALLOC_SCRATCH_BYTES is recorded with a kernel that keeps
 *     no state between workgroups under the automatic plan, and a plan that
 *     forces the look-back kernel for it returns WKV_ERR_UNSUPPORTED.
 *   - Indexing is 64-bit: a single call may exceed 2^31 elements.
 *
 * Errors
 *   - Arguments are checked on the host, synchronously, before anything is
 *     launched: a negative dimension (WKV_ERR_DIM), a byte size that overflows
 *     int64 (WKV_ERR_OVERFLOW), a required pointer that is NULL while the
 *     tensor is non-empty (WKV_ERR_NULL), an output that overlaps an input or
 *     another output (WKV_ERR_ALIAS; state_out may equal state_in exactly
 *     but may not overlap it partially), a workspace that is too small
 *     (WKV_ERR_WORKSPACE), or a plan that names no compiled kernel
 *     (WKV_ERR_UNSUPPORTED).  Nothing is launched when a check fails.
 *   - A failed launch or HIP runtime call returns WKV_ERR_HIP; a fault inside a
 *     kernel surfaces at the caller's next synchronisation of the stream.
 *   - Values are not checked on the device.  Preconditions: w > 0 and finite
 *     inputs; NaN and Inf propagate.
 *   - No C++ exception crosses this interface.
 *   - The library keeps no mutable global state other than its per-device
 *     caches, the per-stream scratch above and the look-back spin limit, all
 *     guarded (a mutex, an atomic); calls may come from several threads.
 *   - The look-back kernel relies on the hardware dispatching workgroups in
 *     index order (it does; HIP does not promise it).  Each of its waits is
 *     bounded: past the bound the wait gives up, that block's outputs, every
 *     later block's outputs of the same sequence and the state handed on are
 *     NaN, and wkv_lookback_status reports WKV_ERR_LOOKBACK for the stream.
 */
#ifndef LIBWKV_WKV_H
#define LIBWKV_WKV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define WKV_API __attribute__((visibility("default")))

typedef enum wkv_status {
    WKV_OK = 0,
    WKV_ERR_NULL = 1,
    WKV_ERR_DIM = 2,
    WKV_ERR_OVERFLOW = 3,
    WKV_ERR_ALIAS = 4,
    WKV_ERR_WORKSPACE = 5,
    WKV_ERR_UNSUPPORTED = 6,
    WKV_ERR_HIP = 7,
    WKV_ERR_LOOKBACK = 8, /* reported by wkv_lookback_status only */
    /* not a status: makes every int a value of the type (C++ otherwise limits
       an unfixed enum to the bits its enumerators need), so a caller may pass
       any int to wkv_status_string */
    WKV_STATUS_MAX_ENUM = 0x7FFFFFFF
} wkv_status;

/*
 * GPT / RNN-chunk forward over T tokens of B sequences with C channels.
 * Cites: section "WKV mechanism: core computation" (the output), "Recurrent
 * formulation" and "Numerical stability via log-space computation" (the state
 * it carries), "Parallel training formulation" (zero initial state when no
 * state is passed); skill page "Quick start" (RNN mode carries the state).
 *
 *   w, u       [C]        decay rate (w > 0) and bonus; required when B*C > 0
 *   k, v       [B][T][C]  keys and values; required when B*T*C > 0
 *   y          [B][T][C]  output, fully overwritten; required when B*T*C > 0
 *   state_in   [3][B][C]  state before the first token, or NULL for the empty
 *                         state
 *   state_out  [3][B][C]  state after the last token, or NULL to discard it;
 *                         may equal state_in (updated in place)
 * T == 0 copies state_in (or the empty state) to state_out and writes no y.
 * y must not overlap any input or state buffer.
 */
WKV_API wkv_status wkv_forward(int64_t B, int64_t T, int64_t C, const float *w, const float *u,
                               const float *k, const float *v, float *y, const float *state_in,
                               float *state_out, hipStream_t stream);

/*
 * Batched single-token RNN step for L layers at once: exactly wkv_forward with
 * T = 1 applied to each layer l with its own w[l], u[l] and state[l].
 * Cites: section "Numerical stability via log-space computation" (one token
 * read against, then folded into, the carried state); skill page "Workflow 1:
 * Text generation" (token-by-token use of the state).
 *
 *   w, u       [L][C]
 *   k, v, y    [L][B][C]
 *   state_in   [L][3][B][C]   required when L*B*C > 0 (a step always reads the
 *                             state; pass a buffer holding the empty state to
 *                             start a sequence)
 *   state_out  [L][3][B][C]   required when L*B*C > 0; may equal state_in
 * The state handed on is the same state as wkv_forward's (equal in the
 * canonical a/b and o + ln b) but kept so that it does not drift over many
 * steps: o stays as it was unless the token became the largest term (then
 * o = k exactly), the decay e^{-w} is folded into a and b, and when b has
 * decayed below 2^-20, o moves down by a whole number of units (exactly) and
 * a, b are rescaled to match.
 */
WKV_API wkv_status wkv_step(int64_t L, int64_t B, int64_t C, const float *w, const float *u,
                            const float *k, const float *v, float *y, const float *state_in,
                            float *state_out, hipStream_t stream);

/* Bytes of device workspace wkv_backward needs for this shape (0 when empty).
 * Returns 0 as well for invalid (negative or overflowing) shapes. */
WKV_API size_t wkv_backward_workspace_size(int64_t B, int64_t T, int64_t C);

/*
 * Gradients of L = sum dy * y through the GPT-mode forward with the empty
 * initial state.  The pages state no backward; these are the derivatives of
 * the closed form (section "WKV mechanism: core computation"), with p_{t,i}
 * the weight of token i in output t:
 *   dv_i = sum_{t>=i} dy_t p_{t,i},  dk_i = sum_{t>=i} dy_t p_{t,i} (v_i - y_t)
 *   du   = sum_{b,t} dy_t p_{t,t} (v_t - y_t)
 *   dw   = -sum_{b,t} sum_{i<t} (t-1-i) dy_t p_{t,i} (v_i - y_t)
 * dw is d/dw of the ABI input w (d/d decay = w * dw).
 *
 *   w, u, k, v   as for wkv_forward
 *   dy           [B][T][C] upstream gradient
 *   dk, dv       [B][T][C] outputs, fully overwritten
 *   dw, du       [C] outputs, overwritten with the sums over B and T; the
 *                summation order is fixed, so results are bitwise
 *                reproducible run to run
 *   workspace    device scratch of at least wkv_backward_workspace_size(B,T,C)
 *                bytes, 256-byte aligned, owned by the caller, not read before
 *                it is written; may be NULL when that size is 0
 * Outputs must not overlap inputs, each other, or the workspace.
 */
WKV_API wkv_status wkv_backward(int64_t B, int64_t T, int64_t C, const float *w, const float *u,
                                const float *k, const float *v, const float *dy, float *dk,
                                float *dv, float *dw, float *du, void *workspace,
                                size_t workspace_bytes, hipStream_t stream);

/*
 * wkv_backward for a chunk that starts from a carried state and hands one on:
 * the gradients of L = sum dy * y + (the upstream loss through the state the
 * forward returned).  This is the backward of RNN mode over chunks (skill
 * page, "Quick start"; section "Duality"): chaining it from the last chunk to
 * the first, each chunk's d_state_in as the previous chunk's d_state_out, gives
 * the gradients of one call over the whole sequence.  The pages state no
 * backward; the carried state enters every output as a token before t = 0
 * whose weights are its sums A0 = a0 e^{o0}, B0 = b0 e^{o0}, at decay distance
 * t, and the state handed on is A_T = e^{-T w} A0 + sum_i e^{k_i-(T-1-i)w} v_i,
 * B_T likewise.
 *
 *   w, u, k, v, dy, dk, dv, dw, du, workspace: as for wkv_backward (the
 *                 workspace size is wkv_backward_workspace_size)
 *   state_in      [3][B][C] the state the forward started from, or NULL (empty)
 *   state_out     [3][B][C] the state the forward returned (read only when
 *                 d_state_out is given: the upstream gradient is in its
 *                 coordinates)
 *   d_state_out   [3][B][C] gradient of the upstream loss with respect to
 *                 state_out's planes (a, b, o), or NULL for none.  A consumer
 *                 sees only A_T and B_T, so the gradient flows through
 *                 dL/dA_T = d_a e^{-o_T} and dL/dB_T = d_b e^{-o_T}; the o-plane
 *                 (then d_a a_T + d_b b_T) is not read
 *   d_state_in    [3][B][C] output: the gradient with respect to state_in's
 *                 planes, d_a0 = dL/dA0 e^{o0}, d_b0 = dL/dB0 e^{o0},
 *                 d_o0 = d_a0 a0 + d_b0 b0 (zero for the empty state), or NULL.
 *                 May equal d_state_out exactly (updated in place)
 * dw includes the state's share (d/dw of its decay e^{-t w}).  With state_in,
 * d_state_out and d_state_in all NULL this is wkv_backward.  T == 0 passes the
 * upstream gradient through to d_state_in.  Outputs must not overlap the
 * inputs or each other (except d_state_in == d_state_out).  Errors as for
 * wkv_backward; d_state_out without state_out is WKV_ERR_NULL.
 */
WKV_API wkv_status wkv_backward_state(int64_t B, int64_t T, int64_t C, const float *w,
                                      const float *u, const float *k, const float *v,
                                      const float *dy, const float *state_in,
                                      const float *state_out, const float *d_state_out,
                                      float *dk, float *dv, float *dw, float *du,
                                      float *d_state_in, void *workspace,
                                      size_t workspace_bytes, hipStream_t stream);

/* Static, NUL-terminated description of a status code. */
WKV_API const char *wkv_status_string(wkv_status s);

/*
 * Forward with an explicit kernel choice, for testing every kernel on every
 * shape and for tuning.  Same arguments, semantics and errors as wkv_forward;
 * `plan` NULL or plan->kernel == WKV_KERNEL_AUTO behaves exactly like
 * wkv_forward.  A plan that names no compiled variant returns
 * WKV_ERR_UNSUPPORTED.
 *   WKV_KERNEL_LANE        one thread per lane, sequential over T
 *   WKV_KERNEL_SEGMENTED   one workgroup per (sequence, `channels` channels)
 *                          owns the whole sequence, in tiles of
 *                          segments * seg_len tokens: each segment of seg_len
 *                          tokens is swept by one row of lanes, and segment
 *                          states are composed with the decay e^{-w len}
 *   WKV_KERNEL_LOOKBACK    workgroups own (`channels` channels, block of
 *                          segments * seg_len tokens) and chain block states by a
 *                          decoupled look-back over earlier blocks
 */
typedef enum wkv_kernel {
    WKV_KERNEL_AUTO = 0,
    WKV_KERNEL_LANE = 1,
    WKV_KERNEL_SEGMENTED = 2,
    WKV_KERNEL_LOOKBACK = 3
} wkv_kernel;

typedef struct wkv_forward_plan {
    int32_t kernel;    /* wkv_kernel */
    int32_t segments;  /* segments per tile (SEGMENTED) or block (LOOKBACK); 0 = default */
    int32_t seg_len;   /* tokens per segment (SEGMENTED, LOOKBACK); 0 = default */
    int32_t channels;  /* channels per workgroup: SEGMENTED 64, 32 or 16; LOOKBACK 64,
                          128 or 256; 0 = 64 */
} wkv_forward_plan;

/* Reproducibility: the lane and segmented kernels give the same bits on every
 * call.  The look-back kernel composes a block's starting state from whichever
 * earlier blocks' states are published first, so the rounding of its outputs,
 * always within the documented accuracy, may differ in the last bits from one
 * call to the next.  A caller who needs bitwise reproducible forwards forces
 * WKV_KERNEL_SEGMENTED. */
WKV_API wkv_status wkv_forward_ex(int64_t B, int64_t T, int64_t C, const float *w, const float *u,
                                  const float *k, const float *v, float *y,
                                  const float *state_in, float *state_out,
                                  const wkv_forward_plan *plan, hipStream_t stream);

/* The plan wkv_forward would use for this shape on the current device. */
WKV_API wkv_status wkv_forward_plan_auto(int64_t B, int64_t T, int64_t C, wkv_forward_plan *plan);

/*
 * Time-mixing output gate fused into the forward: y = sigmoid(r) * wkv
 * elementwise, where wkv is what wkv_forward_ex computes and r is the
 * receptance.  Cites: RWKV architecture deep dive, section "RWKV architecture
 * overview" (block figure: the time-mixing output is sigmoid(r_t) * wkv_t).
 *
 *   r          [B][T][C]  receptance (before the sigmoid); required when
 *                         B*T*C > 0; must not overlap y
 *   all other arguments, the state semantics and the errors as for
 *   wkv_forward_ex.  The state carried is that of the ungated operator.
 * The look-back kernel is compiled for the gate only with seg_len <= 16: an
 * explicit look-back plan with a longer seg_len returns WKV_ERR_UNSUPPORTED,
 * and the automatic choice stays within the compiled variants.
 */
WKV_API wkv_status wkv_forward_gated(int64_t B, int64_t T, int64_t C, const float *w,
                                     const float *u, const float *k, const float *v,
                                     const float *r, float *y, const float *state_in,
                                     float *state_out, const wkv_forward_plan *plan,
                                     hipStream_t stream);

/*
 * wkv_step with the same gate: y = sigmoid(r) * wkv for every (layer,
 * sequence, channel).  Cites: as wkv_forward_gated and wkv_step.
 *   r          [L][B][C]  required when L*B*C > 0; must not overlap y
 * Other arguments and errors as for wkv_step.
 */
WKV_API wkv_status wkv_step_gated(int64_t L, int64_t B, int64_t C, const float *w,
                                  const float *u, const float *k, const float *v,
                                  const float *r, float *y, const float *state_in,
                                  float *state_out, hipStream_t stream);

/* Element format of k, v, r and y in the typed entry points.  w, u and the
 * state stay float32 in every format. */
typedef enum wkv_dtype {
    WKV_DTYPE_F32 = 0,   /* IEEE binary32 */
    WKV_DTYPE_F16 = 1,   /* IEEE binary16 */
    WKV_DTYPE_BF16 = 2,  /* bfloat16: the upper 16 bits of a binary32 */
    WKV_DTYPE_MAX_ENUM = 0x7FFFFFFF  /* not a format: every int is a value of the type */
} wkv_dtype;

/*
 * Forward with 16-bit (or 32-bit) activations: k, v, r and y hold `dtype`
 * elements, while w, u and the state are float32 and all arithmetic is
 * float32.  Inputs widen exactly; y is rounded to `dtype` once, to nearest,
 * ties to even.  The pages run the model in half precision (skill page,
 * "Quick start": the 'cuda fp16' strategy) and train it in bfloat16
 * ("Workflow 3: Fine-tuning RWKV").
 *
 *   k, v, y    [B][T][C] of dtype
 *   r          [B][T][C] of dtype, or NULL: with r, y = sigmoid(r) * wkv (as
 *              wkv_forward_gated); without, y = wkv
 *   w, u, state_in, state_out, plan, stream: as for wkv_forward_ex
 * WKV_DTYPE_F32 behaves exactly like wkv_forward_ex or wkv_forward_gated.  For
 * the 16-bit formats the compiled kernels are the lane kernel, the segmented
 * kernel with 16 segments of 16 tokens over 64 channels, and the look-back
 * kernel with 64 channels and 4x16, 4x32 or 8x16 tokens (8x16 and 4x16 when
 * gated); another explicit plan returns WKV_ERR_UNSUPPORTED, and the
 * automatic choice stays within them.  An unknown dtype returns
 * WKV_ERR_UNSUPPORTED.  Other errors as for wkv_forward, with byte sizes
 * taken at the element size of dtype.
 */
WKV_API wkv_status wkv_forward_typed(int64_t B, int64_t T, int64_t C, wkv_dtype dtype,
                                     const float *w, const float *u, const void *k,
                                     const void *v, const void *r, void *y,
                                     const float *state_in, float *state_out,
                                     const wkv_forward_plan *plan, hipStream_t stream);

/*
 * wkv_step with k, v, r and y of `dtype` (r NULL: ungated), w, u and the
 * state float32, as for wkv_forward_typed.  Cites: as wkv_step.
 */
WKV_API wkv_status wkv_step_typed(int64_t L, int64_t B, int64_t C, wkv_dtype dtype,
                                  const float *w, const float *u, const void *k, const void *v,
                                  const void *r, void *y, const float *state_in,
                                  float *state_out, hipStream_t stream);

/*
 * wkv_backward_state with 16-bit (or 32-bit) activation gradients: k, v, dy,
 * dk and dv hold `dtype` elements (wkv_dtype); w, u, dw, du, the states and
 * their gradients are float32, and all arithmetic is float32.  Inputs widen
 * exactly; dk and dv are rounded once to `dtype` (nearest, ties to even).  The
 * pages train the model in bfloat16 (skill page, "Workflow 3: Fine-tuning
 * RWKV").  Arguments, semantics and errors as for wkv_backward_state, with
 * byte sizes at the element size of dtype; an unknown dtype returns
 * WKV_ERR_UNSUPPORTED.  The workspace size is wkv_backward_workspace_size.
 */
WKV_API wkv_status wkv_backward_typed(int64_t B, int64_t T, int64_t C, wkv_dtype dtype,
                                      const float *w, const float *u, const void *k,
                                      const void *v, const void *dy, const float *state_in,
                                      const float *state_out, const float *d_state_out,
                                      void *dk, void *dv, float *dw, float *du,
                                      float *d_state_in, void *workspace,
                                      size_t workspace_bytes, hipStream_t stream);

/* Tokens between two checkpoints of the forward state. */
#define WKV_CHECKPOINT_TOKENS 128
/* Checkpoints of a sequence of T tokens: one before every multiple of
 * WKV_CHECKPOINT_TOKENS that lies strictly inside it. */
#define WKV_CHECKPOINT_COUNT(T) ((T) > 0 ? ((T) - 1) / WKV_CHECKPOINT_TOKENS : 0)

/*
 * wkv_forward_typed that also saves the state every WKV_CHECKPOINT_TOKENS
 * tokens, for a backward that starts from them.  Checkpoint i is the RNN-mode
 * state (a, b, o) after the first (i + 1) * WKV_CHECKPOINT_TOKENS tokens,
 * exactly the state_out of a call over that prefix (rwkv-architecture skill
 * page, "Quick start": the state carried between calls; RWKV architecture
 * deep dive, "Duality": the parallel and recurrent forms agree).  Training
 * keeps them from the forward to the backward (skill page, "Workflow 3:
 * Fine-tuning RWKV").
 *
 *   checkpoints  [WKV_CHECKPOINT_COUNT(T)][3][B][C] float32 output, fully
 *                overwritten; each entry has the layout of state_out, so
 *                checkpoints + i*3*B*C can serve as a later call's state_in.
 *                Required when that count times B*C is positive, else ignored
 *                (may be NULL).  Must not overlap any other argument.
 * Every other argument, the plan, the result and the errors are those of
 * wkv_forward_typed; y and state_out are bitwise those of wkv_forward_typed
 * with the same plan (the look-back kernel excepted, which is not bitwise
 * reproducible from call to call).  Writing the checkpoints adds
 * 12 bytes per lane per WKV_CHECKPOINT_TOKENS tokens to the traffic.
 */
WKV_API wkv_status wkv_forward_checkpointed(int64_t B, int64_t T, int64_t C, wkv_dtype dtype,
                                            const float *w, const float *u, const void *k,
                                            const void *v, const void *r, void *y,
                                            const float *state_in, float *state_out,
                                            float *checkpoints, const wkv_forward_plan *plan,
                                            hipStream_t stream);

/*
 * wkv_backward_typed given the checkpoints that wkv_forward_checkpointed wrote
 * for the same inputs and state_in.  The gradients are the same functions of
 * the inputs; the forward states they need are rebuilt from the checkpoints,
 * tile by tile, instead of by a first pass over k and v, which saves reading
 * k and v twice (8 of the 28 bytes per lane-token that wkv_backward_typed
 * moves in float32).  The pages state no backward; see wkv_backward.
 *
 *   checkpoints  [WKV_CHECKPOINT_COUNT(T)][3][B][C] as written by
 *                wkv_forward_checkpointed for these w, u, k, v and state_in;
 *                read only; required when that count times B*C is positive.
 *                No output may overlap it
 * Every other argument, the workspace size (wkv_backward_workspace_size) and
 * the errors are those of wkv_backward_typed.  Results agree with
 * wkv_backward_typed to rounding (the states pass through the checkpoints'
 * float32 a, b, o once per tile); dw and du stay bitwise reproducible from
 * run to run.
 */
WKV_API wkv_status wkv_backward_checkpointed(int64_t B, int64_t T, int64_t C, wkv_dtype dtype,
                                             const float *w, const float *u, const void *k,
                                             const void *v, const void *dy,
                                             const float *state_in, const float *checkpoints,
                                             const float *state_out, const float *d_state_out,
                                             void *dk, void *dv, float *dw, float *du,
                                             float *d_state_in, void *workspace,
                                             size_t workspace_bytes, hipStream_t stream);

/*
 * Backward of the gated forward (wkv_forward_gated, or a typed or checkpointed
 * forward given r): dy is the gradient of the gated output
 * o = sigmoid(r) * wkv (RWKV architecture deep dive, "RWKV architecture
 * overview", block figure; the pages state no backward).  The recurrence
 * receives g = dy * sigmoid(r), so dk, dv, dw, du and d_state_in are those of
 * wkv_backward_typed for that g, and
 *   dr = dy * wkv * sigmoid(r) * (1 - sigmoid(r))
 * is written beside them (wkv is recomputed, not read).
 *
 *   r            [B][T][C] of `dtype`: the forward's receptance; required when
 *                B*T*C > 0
 *   dr           [B][T][C] of `dtype`: output, fully overwritten, rounded once
 *                to `dtype`; required when B*T*C > 0; overlaps nothing
 *   checkpoints  NULL: the backward makes its own first pass over k and v;
 *                else as for wkv_backward_checkpointed
 * Every other argument, the workspace size and the errors are those of
 * wkv_backward_typed.
 */
WKV_API wkv_status wkv_backward_gated(int64_t B, int64_t T, int64_t C, wkv_dtype dtype,
                                      const float *w, const float *u, const void *k,
                                      const void *v, const void *r, const void *dy,
                                      const float *state_in, const float *checkpoints,
                                      const float *state_out, const float *d_state_out,
                                      void *dk, void *dv, void *dr, float *dw, float *du,
                                      float *d_state_in, void *workspace,
                                      size_t workspace_bytes, hipStream_t stream);

/* Largest number of mixes wkv_token_shift takes in one call. */
#define WKV_TOKEN_SHIFT_MAX_MIXES 8

/*
 * Token shift of the time-mixing block, for M projection inputs at once:
 *   out[m][b][t][c] = mu[m][c] * x[b][t][c] + (1 - mu[m][c]) * x[b][t-1][c]
 * where x[b][-1][c] is x_prev[b][c], the last token of the previous call (the
 * att_x_prev state), or 0 for a fresh sequence (x_prev NULL).  Cites: RWKV
 * architecture deep dive, section "Token shift" (the mix, per-channel mu);
 * rwkv-architecture skill page, "Advanced topics" (att_x_prev is carried
 * between calls like the WKV state).
 *
 *   mu          [M][C]      mix weights; required when M*C > 0
 *   x           [B][T][C]   input tokens; required when B*T*C > 0
 *   x_prev      [B][C]      or NULL (zeros)
 *   out         [M][B][T][C] output, fully overwritten; required when M*B*T*C > 0;
 *                           must not overlap any other argument
 *   x_prev_out  [B][C]      receives x[b][T-1] (x_prev, or zeros, when T == 0),
 *                           or NULL to discard it; may equal x_prev (in place)
 *                           but may not overlap it partially, nor x, mu or out
 * 0 <= M <= WKV_TOKEN_SHIFT_MAX_MIXES, else WKV_ERR_UNSUPPORTED.  Other errors
 * as for wkv_forward.
 */
WKV_API wkv_status wkv_token_shift(int64_t B, int64_t T, int64_t C, int64_t M, const float *mu,
                                   const float *x, const float *x_prev, float *out,
                                   float *x_prev_out, hipStream_t stream);

/*
 * wkv_token_shift with x, x_prev, out and x_prev_out holding `dtype` elements
 * (wkv_dtype; mu stays float32): the mixes are computed in float32 and rounded
 * once to `dtype` (nearest, ties to even); the carried token is copied
 * exactly.  Arguments, semantics and errors as for wkv_token_shift, with byte
 * sizes at the element size of dtype; an unknown dtype returns
 * WKV_ERR_UNSUPPORTED.  Cites: as wkv_token_shift; 16-bit activations as for
 * wkv_forward_typed.
 */
WKV_API wkv_status wkv_token_shift_typed(int64_t B, int64_t T, int64_t C, int64_t M,
                                         wkv_dtype dtype, const float *mu, const void *x,
                                         const void *x_prev, void *out, void *x_prev_out,
                                         hipStream_t stream);

/*
 * Backward of wkv_token_shift, for training the time-mixing block.  With d_out
 * the gradients of the M mixes and d_x_prev_out that of the carried token the
 * forward handed on, token t feeds mix t with weight mu and mix t + 1 with
 * 1 - mu (RWKV architecture deep dive, section "Token shift"; the pages state
 * no backward):
 *   dx[b][t][c]   = sum_m mu[m][c] d_out[m][b][t][c]
 *                 + sum_m (1 - mu[m][c]) d_out[m][b][t+1][c]   (t + 1 < T)
 *                 + d_x_prev_out[b][c]                        (t = T - 1)
 *   d_x_prev[b][c] = sum_m (1 - mu[m][c]) d_out[m][b][0][c]    (T > 0;
 *                    d_x_prev_out when T = 0)
 *   dmu[m][c]     = sum_{b,t} d_out[m][b][t][c] (x[b][t][c] - x[b][t-1][c])
 * with x[b][-1] = x_prev (zeros when NULL).
 *
 *   mu, x, x_prev  as for the forward call
 *   d_out          [M][B][T][C]; required when M*B*T*C > 0
 *   d_x_prev_out   [B][C] or NULL (no gradient reaches the carried token)
 *   dx             [B][T][C] output; required when B*T*C > 0
 *   d_x_prev       [B][C] output, or NULL to discard it
 *   dmu            [M][C] output, the sum over B and T in a fixed order
 *                  (bitwise reproducible); required when M*C > 0
 *   workspace      device scratch of at least
 *                  wkv_token_shift_backward_workspace_size(B,T,C,M) bytes,
 *                  caller-owned; may be NULL when that size is 0
 * Outputs overlap neither the inputs nor each other.  M above
 * WKV_TOKEN_SHIFT_MAX_MIXES is WKV_ERR_UNSUPPORTED; other errors as for
 * wkv_backward.
 */
WKV_API size_t wkv_token_shift_backward_workspace_size(int64_t B, int64_t T, int64_t C,
                                                       int64_t M);
WKV_API wkv_status wkv_token_shift_backward(int64_t B, int64_t T, int64_t C, int64_t M,
                                            const float *mu, const float *x,
                                            const float *x_prev, const float *d_out,
                                            const float *d_x_prev_out, float *dx,
                                            float *d_x_prev, float *dmu, void *workspace,
                                            size_t workspace_bytes, hipStream_t stream);

/*
 * wkv_token_shift_backward with x, x_prev, d_out, d_x_prev_out, dx and
 * d_x_prev holding `dtype` elements (mu and dmu stay float32; all arithmetic
 * is float32, dx and d_x_prev are rounded once to `dtype`).  Arguments,
 * workspace size and errors as for wkv_token_shift_backward, with byte sizes
 * at the element size of dtype.
 */
WKV_API wkv_status wkv_token_shift_backward_typed(int64_t B, int64_t T, int64_t C, int64_t M,
                                                  wkv_dtype dtype, const float *mu,
                                                  const void *x, const void *x_prev,
                                                  const void *d_out, const void *d_x_prev_out,
                                                  void *dx, void *d_x_prev, float *dmu,
                                                  void *workspace, size_t workspace_bytes,
                                                  hipStream_t stream);

/* Size of the fixed scratch array behind wkv_forward_noalloc, per device. */
#define WKV_NOALLOC_SCRATCH_BYTES ((size_t)40 << 20)

/*
 * wkv_forward for callers that cannot allocate device memory: code being
 * captured into a HIP graph, tight serving loops, harnesses that forbid
 * allocation.  It calls no hipMalloc, hipFree or other allocating routine: the
 * look-back kernel's scratch is a fixed array of WKV_NOALLOC_SCRATCH_BYTES in
 * device memory that every device running the library holds until the process
 * ends.  Same arguments, semantics and results (within the documented
 * accuracy) as wkv_forward, with the automatic kernel choice.
 *   - A shape whose look-back scratch (wkv_forward_scratch_size) exceeds
 *     WKV_NOALLOC_SCRATCH_BYTES returns WKV_ERR_WORKSPACE with nothing
 *     launched; such a shape can run through wkv_forward, or through
 *     wkv_forward_ex with a WKV_KERNEL_SEGMENTED plan (no scratch).
 *   - Every call on one device shares that device's array, which keeps the
 *     last call's contents (each launch tags what it writes, so nothing needs
 *     clearing).  Calls that overlap in time on one device, from any stream or
 *     thread, race on it: callers serialise them.
 *   - The first call on a device takes the array's address on it (which may
 *     load the library's device code, and with it the array); a caller that
 *     will capture makes one call on each device beforehand.  Under graph
 *     capture the launch takes its per-launch tag on the device (a
 *     one-workgroup kernel recorded before it), as wkv_forward does there.
 * Waits that give up are reported by wkv_lookback_status on the stream of a
 * later call.
 */
WKV_API wkv_status wkv_forward_noalloc(int64_t B, int64_t T, int64_t C, const float *w,
                                       const float *u, const float *k, const float *v, float *y,
                                       const float *state_in, float *state_out,
                                       hipStream_t stream);

/*
 * Bytes of look-back scratch wkv_forward would use for this shape on the
 * current device (0 when its kernel needs none, or for an invalid shape).
 */
WKV_API size_t wkv_forward_scratch_size(int64_t B, int64_t T, int64_t C);

/*
 * Releases the look-back scratch the library keeps for `stream` on the current
 * device, in stream order (hipFreeAsync on `stream`), so that launches already
 * queued on it finish first.  The next look-back forward on that stream
 * allocates a fresh buffer.  `stream` must still be valid.  Returns WKV_OK
 * (also when there is none) or WKV_ERR_HIP.
 */
WKV_API wkv_status wkv_release_stream_scratch(hipStream_t stream);

/*
 * Synchronises `stream`, then reports whether any look-back wait of a forward
 * on this stream, or of a wkv_forward_noalloc call on the current device, gave
 * up since the last call:
 * WKV_ERR_LOOKBACK if one did (those launches' outputs from the stalled block
 * on, and their state_out, are NaN), WKV_OK if none did, WKV_ERR_HIP on a
 * runtime error.  Clears the record.  Forwards are asynchronous, so this is
 * the only place the condition can be returned as a status.
 */
WKV_API wkv_status wkv_lookback_status(hipStream_t stream);

/*
 * Test hook: the number of look-back rounds without progress after which a
 * wait gives up (default 65536, tens of milliseconds).  Returns the previous
 * value.  Applies to launches issued after the call, from every thread.  A
 * limit of 0 makes every wait that finds no predecessor ready give up at once,
 * which exercises the give-up path while every workgroup still exits normally.
 */
WKV_API uint32_t wkv_set_lookback_spin_limit(uint32_t rounds);

#ifdef __cplusplus
}
#endif

#endif /* LIBWKV_WKV_H */

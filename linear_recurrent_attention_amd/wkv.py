"""Thin Python binding of libwkv (include/wkv.h): argument marshalling only.

Every function here forwards to the C entry point of the same name, passing
device pointers taken from torch tensors and the stream handle of the given
(or current) torch stream.  No arithmetic of the operator happens in Python,
and there is no fallback: if ``libwkv.so`` is not built, or a tensor is not a
float32 tensor on a HIP device, the call raises.

Layouts (C-contiguous, channel fastest):
    w, u            [C]          (wkv_step: [L][C])
    k, v, r, y, dy  [B][T][C]    (wkv_step: [L][B][C]); float32, or float16 /
                                 bfloat16 in the *_typed calls
    state           [3][B][C]    planes a, b, o   (wkv_step: [L][3][B][C])
    token shift     mu [M][C], x [B][T][C], x_prev [B][C], out [M][B][T][C]
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libwkv.so")

# wkv_status values
WKV_OK = 0
WKV_ERR_NULL = 1
WKV_ERR_DIM = 2
WKV_ERR_OVERFLOW = 3
WKV_ERR_ALIAS = 4
WKV_ERR_WORKSPACE = 5
WKV_ERR_UNSUPPORTED = 6
WKV_ERR_HIP = 7
WKV_ERR_LOOKBACK = 8

# wkv_kernel values
WKV_KERNEL_AUTO = 0
WKV_KERNEL_LANE = 1
WKV_KERNEL_SEGMENTED = 2
WKV_KERNEL_LOOKBACK = 3

EXPORTED = ("wkv_forward", "wkv_step", "wkv_backward_workspace_size", "wkv_backward",
            "wkv_status_string", "wkv_forward_ex", "wkv_forward_plan_auto",
            "wkv_forward_gated", "wkv_step_gated", "wkv_token_shift", "wkv_forward_typed",
            "wkv_step_typed", "wkv_backward_state", "wkv_backward_typed",
            "wkv_forward_checkpointed", "wkv_backward_checkpointed", "wkv_backward_gated",
            "wkv_token_shift_backward_workspace_size", "wkv_token_shift_backward",
            "wkv_token_shift_typed", "wkv_token_shift_backward_typed",
            "wkv_forward_scratch_size", "wkv_release_stream_scratch", "wkv_lookback_status",
            "wkv_set_lookback_spin_limit", "wkv_forward_noalloc")

# wkv_dtype values
WKV_DTYPE_F32 = 0
WKV_DTYPE_F16 = 1
WKV_DTYPE_BF16 = 2
_DTYPES = {torch.float32: WKV_DTYPE_F32, torch.float16: WKV_DTYPE_F16,
           torch.bfloat16: WKV_DTYPE_BF16}

WKV_TOKEN_SHIFT_MAX_MIXES = 8
WKV_CHECKPOINT_TOKENS = 128


def checkpoint_count(T: int) -> int:
    """Checkpoints of a sequence of T tokens (WKV_CHECKPOINT_COUNT)."""
    return (T - 1) // WKV_CHECKPOINT_TOKENS if T > 0 else 0


class WkvError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: status {status} ({wkv_status_string(status)})")


class ForwardPlan(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int32), ("segments", ctypes.c_int32),
                ("seg_len", ctypes.c_int32), ("channels", ctypes.c_int32)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libwkv.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m linear_recurrent_attention_amd.build`")
    lib = ctypes.CDLL(path)
    i64, vp, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
    lib.wkv_forward.argtypes = [i64, i64, i64] + [vp] * 7 + [vp]
    lib.wkv_forward.restype = ctypes.c_int
    lib.wkv_forward_ex.argtypes = [i64, i64, i64] + [vp] * 7 + [ctypes.POINTER(ForwardPlan), vp]
    lib.wkv_forward_ex.restype = ctypes.c_int
    lib.wkv_forward_plan_auto.argtypes = [i64, i64, i64, ctypes.POINTER(ForwardPlan)]
    lib.wkv_forward_plan_auto.restype = ctypes.c_int
    lib.wkv_step.argtypes = [i64, i64, i64] + [vp] * 7 + [vp]
    lib.wkv_step.restype = ctypes.c_int
    lib.wkv_backward_workspace_size.argtypes = [i64, i64, i64]
    lib.wkv_backward_workspace_size.restype = sz
    lib.wkv_backward.argtypes = [i64, i64, i64] + [vp] * 9 + [vp, sz, vp]
    lib.wkv_backward.restype = ctypes.c_int
    lib.wkv_forward_gated.argtypes = ([i64, i64, i64] + [vp] * 8 +
                                      [ctypes.POINTER(ForwardPlan), vp])
    lib.wkv_forward_gated.restype = ctypes.c_int
    lib.wkv_step_gated.argtypes = [i64, i64, i64] + [vp] * 8 + [vp]
    lib.wkv_step_gated.restype = ctypes.c_int
    lib.wkv_token_shift.argtypes = [i64, i64, i64, i64] + [vp] * 5 + [vp]
    lib.wkv_token_shift.restype = ctypes.c_int
    lib.wkv_forward_typed.argtypes = ([i64, i64, i64, ctypes.c_int] + [vp] * 8 +
                                      [ctypes.POINTER(ForwardPlan), vp])
    lib.wkv_forward_typed.restype = ctypes.c_int
    lib.wkv_step_typed.argtypes = [i64, i64, i64, ctypes.c_int] + [vp] * 8 + [vp]
    lib.wkv_step_typed.restype = ctypes.c_int
    lib.wkv_backward_state.argtypes = [i64, i64, i64] + [vp] * 13 + [vp, sz, vp]
    lib.wkv_backward_state.restype = ctypes.c_int
    lib.wkv_backward_typed.argtypes = ([i64, i64, i64, ctypes.c_int] + [vp] * 13 +
                                       [vp, sz, vp])
    lib.wkv_backward_typed.restype = ctypes.c_int
    lib.wkv_forward_checkpointed.argtypes = ([i64, i64, i64, ctypes.c_int] + [vp] * 9 +
                                             [ctypes.POINTER(ForwardPlan), vp])
    lib.wkv_forward_checkpointed.restype = ctypes.c_int
    lib.wkv_backward_checkpointed.argtypes = ([i64, i64, i64, ctypes.c_int] + [vp] * 14 +
                                              [vp, sz, vp])
    lib.wkv_backward_checkpointed.restype = ctypes.c_int
    lib.wkv_backward_gated.argtypes = [i64, i64, i64, ctypes.c_int] + [vp] * 16 + [vp, sz, vp]
    lib.wkv_backward_gated.restype = ctypes.c_int
    lib.wkv_token_shift_backward_workspace_size.argtypes = [i64, i64, i64, i64]
    lib.wkv_token_shift_backward_workspace_size.restype = sz
    lib.wkv_token_shift_backward.argtypes = [i64, i64, i64, i64] + [vp] * 8 + [vp, sz, vp]
    lib.wkv_token_shift_backward.restype = ctypes.c_int
    lib.wkv_token_shift_typed.argtypes = [i64, i64, i64, i64, ctypes.c_int] + [vp] * 5 + [vp]
    lib.wkv_token_shift_typed.restype = ctypes.c_int
    lib.wkv_token_shift_backward_typed.argtypes = ([i64, i64, i64, i64, ctypes.c_int] +
                                                   [vp] * 8 + [vp, sz, vp])
    lib.wkv_token_shift_backward_typed.restype = ctypes.c_int
    lib.wkv_status_string.argtypes = [ctypes.c_int]
    lib.wkv_status_string.restype = ctypes.c_char_p
    lib.wkv_forward_scratch_size.argtypes = [i64, i64, i64]
    lib.wkv_forward_scratch_size.restype = sz
    lib.wkv_release_stream_scratch.argtypes = [vp]
    lib.wkv_release_stream_scratch.restype = ctypes.c_int
    lib.wkv_lookback_status.argtypes = [vp]
    lib.wkv_lookback_status.restype = ctypes.c_int
    lib.wkv_forward_noalloc.argtypes = [i64, i64, i64] + [vp] * 7 + [vp]
    lib.wkv_forward_noalloc.restype = ctypes.c_int
    lib.wkv_set_lookback_spin_limit.argtypes = [ctypes.c_uint32]
    lib.wkv_set_lookback_spin_limit.restype = ctypes.c_uint32
    _lib = lib
    return lib


def wkv_status_string(status: int) -> str:
    return load_library().wkv_status_string(int(status)).decode()


def _ptr(t, dtype=torch.float32):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {t.dtype}")
    if t.numel() > 0 and not t.is_cuda:
        raise TypeError("expected a tensor on a HIP device")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return ctypes.c_void_p(t.data_ptr()) if t.numel() > 0 else None


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(fn, status):
    if status != WKV_OK:
        raise WkvError(fn, status)


def _bundle_shape(k):
    if not isinstance(k, torch.Tensor):
        raise TypeError("k: expected a torch.Tensor")
    if k.dim() != 3:
        raise ValueError("k must be 3-D")
    return tuple(int(x) for x in k.shape)


def _expect(device, *spec):
    """Checks (name, tensor, shape) triples before a call: every tensor given
    (None is skipped) must have exactly that shape and, when non-empty, live on
    ``device``.  The C ABI takes bare pointers and cannot check sizes, so a
    wrong-sized buffer would be read or written out of bounds."""
    for name, t, shape in spec:
        if t is None:
            continue
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name}: expected a torch.Tensor")
        if tuple(t.shape) != tuple(int(x) for x in shape):
            raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
        if t.numel() > 0 and t.device != device:
            raise ValueError(f"{name}: on {t.device}, expected {device}")


def _expect_workspace(device, ws, need):
    if not isinstance(ws, torch.Tensor):
        raise TypeError("workspace: expected a torch.Tensor")
    if ws.dtype != torch.uint8 or not ws.is_contiguous():
        raise TypeError("workspace must be a contiguous uint8 tensor")
    if ws.numel() > 0 and ws.device != device:
        raise ValueError(f"workspace: on {ws.device}, expected {device}")
    if ws.numel() < need:
        raise ValueError(f"workspace: {ws.numel()} bytes, need {need}")


def _fwd_expect(k, w, u, v, r, y, state_in, state_out, checkpoints=None):
    B, T, C = (int(x) for x in k.shape)
    _expect(k.device, ("w", w, (C,)), ("u", u, (C,)), ("v", v, (B, T, C)), ("r", r, (B, T, C)),
            ("y", y, (B, T, C)), ("state_in", state_in, (3, B, C)),
            ("state_out", state_out, (3, B, C)),
            ("checkpoints", checkpoints, (checkpoint_count(T), 3, B, C)))


def _bwd_expect(k, w, u, v, dy, dk, dv, dw, du, state_in=None, state_out=None,
                d_state_out=None, d_state_in=None, checkpoints=None, r=None, dr=None):
    B, T, C = (int(x) for x in k.shape)
    seq, st = (B, T, C), (3, B, C)
    _expect(k.device, ("w", w, (C,)), ("u", u, (C,)), ("v", v, seq), ("dy", dy, seq),
            ("dk", dk, seq), ("dv", dv, seq), ("dw", dw, (C,)), ("du", du, (C,)),
            ("state_in", state_in, st), ("state_out", state_out, st),
            ("d_state_out", d_state_out, st), ("d_state_in", d_state_in, st),
            ("checkpoints", checkpoints, (checkpoint_count(T), 3, B, C)), ("r", r, seq),
            ("dr", dr, seq))


def _step_expect(k, w, u, v, r, y, state_in, state_out):
    L, B, C = (int(x) for x in k.shape)
    _expect(k.device, ("w", w, (L, C)), ("u", u, (L, C)), ("v", v, (L, B, C)),
            ("r", r, (L, B, C)), ("y", y, (L, B, C)), ("state_in", state_in, (L, 3, B, C)),
            ("state_out", state_out, (L, 3, B, C)))


def wkv_forward(w, u, k, v, y=None, state_in=None, state_out=None, stream=None, plan=None):
    """GPT / RNN-chunk forward.  Returns (y, state_out).

    ``state_out`` is written when given (it may be ``state_in`` itself for an
    in-place update); pass ``state_out=True`` to have one allocated.  ``plan``
    is an optional (kernel, segments, seg_len[, channels]) tuple for
    ``wkv_forward_ex``.
    """
    B, T, C = _bundle_shape(k)
    if y is None:
        y = torch.empty_like(k)
    if state_out is True:
        state_out = torch.empty((3, B, C), device=k.device, dtype=torch.float32)
    _fwd_expect(k, w, u, v, None, y, state_in, state_out)
    lib = load_library()
    args = [B, T, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(y), _ptr(state_in),
            _ptr(state_out)]
    if plan is None:
        _check("wkv_forward", lib.wkv_forward(*args, _stream(stream)))
    else:
        p = ForwardPlan(*plan) if len(plan) == 4 else ForwardPlan(*plan, 0)
        _check("wkv_forward_ex", lib.wkv_forward_ex(*args, ctypes.byref(p), _stream(stream)))
    return y, state_out


def _plan(plan):
    if plan is None:
        return None
    p = ForwardPlan(*plan) if len(plan) == 4 else ForwardPlan(*plan, 0)
    return ctypes.byref(p)


def wkv_forward_gated(w, u, k, v, r, y=None, state_in=None, state_out=None, stream=None,
                      plan=None):
    """Forward with the time-mixing output gate: y = sigmoid(r) * wkv.
    Arguments as for ``wkv_forward``; r has the layout of k.  Returns
    (y, state_out)."""
    B, T, C = _bundle_shape(k)
    if y is None:
        y = torch.empty_like(k)
    if state_out is True:
        state_out = torch.empty((3, B, C), device=k.device, dtype=torch.float32)
    _fwd_expect(k, w, u, v, r, y, state_in, state_out)
    st = load_library().wkv_forward_gated(B, T, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(r),
                                          _ptr(y), _ptr(state_in), _ptr(state_out), _plan(plan),
                                          _stream(stream))
    _check("wkv_forward_gated", st)
    return y, state_out


def wkv_forward_typed(w, u, k, v, r=None, y=None, state_in=None, state_out=None, stream=None,
                      plan=None):
    """Forward with k, v (r) and y in k's dtype (float32, float16 or bfloat16);
    w, u and the state float32.  With r, y = sigmoid(r) * wkv.  Returns
    (y, state_out)."""
    if k.dtype not in _DTYPES:
        raise TypeError(f"unsupported element type {k.dtype}")
    dt = k.dtype
    B, T, C = _bundle_shape(k)
    if y is None:
        y = torch.empty_like(k)
    if state_out is True:
        state_out = torch.empty((3, B, C), device=k.device, dtype=torch.float32)
    _fwd_expect(k, w, u, v, r, y, state_in, state_out)
    st = load_library().wkv_forward_typed(B, T, C, _DTYPES[dt], _ptr(w), _ptr(u), _ptr(k, dt),
                                          _ptr(v, dt), _ptr(r, dt), _ptr(y, dt),
                                          _ptr(state_in), _ptr(state_out), _plan(plan),
                                          _stream(stream))
    _check("wkv_forward_typed", st)
    return y, state_out


def wkv_forward_checkpointed(w, u, k, v, r=None, y=None, state_in=None, state_out=None,
                             checkpoints=None, stream=None, plan=None):
    """``wkv_forward_typed`` that also writes the state before every multiple of
    WKV_CHECKPOINT_TOKENS tokens inside the sequence into ``checkpoints``
    ([checkpoint_count(T)][3][B][C] float32, allocated when None).  Returns
    (y, state_out, checkpoints)."""
    if k.dtype not in _DTYPES:
        raise TypeError(f"unsupported element type {k.dtype}")
    dt = k.dtype
    B, T, C = _bundle_shape(k)
    if y is None:
        y = torch.empty_like(k)
    if state_out is True:
        state_out = torch.empty((3, B, C), device=k.device, dtype=torch.float32)
    if checkpoints is None:
        checkpoints = torch.empty((checkpoint_count(T), 3, B, C), device=k.device,
                                  dtype=torch.float32)
    _fwd_expect(k, w, u, v, r, y, state_in, state_out, checkpoints)
    st = load_library().wkv_forward_checkpointed(
        B, T, C, _DTYPES[dt], _ptr(w), _ptr(u), _ptr(k, dt), _ptr(v, dt), _ptr(r, dt),
        _ptr(y, dt), _ptr(state_in), _ptr(state_out), _ptr(checkpoints), _plan(plan),
        _stream(stream))
    _check("wkv_forward_checkpointed", st)
    return y, state_out, checkpoints


def bind_forward(w, u, k, v, y, state_in=None, state_out=None, stream=None, plan=None):
    """Marshal the arguments of one ``wkv_forward_ex`` call once and return a
    callable that re-issues exactly that call (same tensors, whose contents
    may change between calls).  For loops bound by the launch rate, such as
    RNN mode over many short chunks, where re-checking every tensor in Python
    on each call would cost as much as the kernel."""
    B, T, C = _bundle_shape(k)
    _fwd_expect(k, w, u, v, None, y, state_in, state_out)
    lib = load_library()
    p = None if plan is None else (ForwardPlan(*plan) if len(plan) == 4 else ForwardPlan(*plan, 0))
    args = (B, T, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(y), _ptr(state_in),
            _ptr(state_out), None if p is None else ctypes.byref(p), _stream(stream))
    fn = lib.wkv_forward_ex
    keep = (w, u, k, v, y, state_in, state_out, p)  # the call's tensors stay alive with it

    def call():
        st = fn(*args)
        if st != WKV_OK:
            raise WkvError("wkv_forward_ex", st)
    call.keep = keep
    return call


WKV_NOALLOC_SCRATCH_BYTES = 40 << 20


def wkv_forward_noalloc(w, u, k, v, y, state_in=None, state_out=None, stream=None):
    """``wkv_forward`` through the entry point that allocates nothing (its
    look-back scratch is a fixed array per device).  y and state_out (if
    wanted) must be given: the call allocates no output either."""
    B, T, C = _bundle_shape(k)
    _fwd_expect(k, w, u, v, None, y, state_in, state_out)
    st = load_library().wkv_forward_noalloc(B, T, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(y),
                                            _ptr(state_in), _ptr(state_out), _stream(stream))
    _check("wkv_forward_noalloc", st)
    return y, state_out


def wkv_forward_scratch_size(B: int, T: int, C: int) -> int:
    """Bytes of look-back scratch wkv_forward uses for this shape (0: none)."""
    return int(load_library().wkv_forward_scratch_size(B, T, C))


def wkv_release_stream_scratch(stream=None):
    """Release (in stream order) the look-back scratch kept for ``stream``."""
    _check("wkv_release_stream_scratch", load_library().wkv_release_stream_scratch(_stream(stream)))


def wkv_lookback_status(stream=None) -> int:
    """Synchronise ``stream`` and return WKV_OK, or WKV_ERR_LOOKBACK if a
    look-back wait of a forward on it gave up since the last call (clears the
    record).  Other failures raise."""
    st = load_library().wkv_lookback_status(_stream(stream))
    if st not in (WKV_OK, WKV_ERR_LOOKBACK):
        raise WkvError("wkv_lookback_status", st)
    return st


def wkv_set_lookback_spin_limit(rounds: int) -> int:
    """Test hook: look-back rounds without progress before a wait gives up.
    Returns the previous limit."""
    return int(load_library().wkv_set_lookback_spin_limit(int(rounds)))


def wkv_forward_plan_auto(B: int, T: int, C: int):
    p = ForwardPlan()
    _check("wkv_forward_plan_auto", load_library().wkv_forward_plan_auto(B, T, C, ctypes.byref(p)))
    return (p.kernel, p.segments, p.seg_len, p.channels)


def wkv_step(w, u, k, v, state_in, state_out=None, y=None, stream=None):
    """Batched T=1 step over L layers.  k, v: [L][B][C]; state: [L][3][B][C].
    ``state_out`` defaults to ``state_in`` (in-place).  Returns (y, state_out)."""
    if k.dim() != 3:
        raise ValueError("k must be [L][B][C]")
    L, B, C = (int(x) for x in k.shape)
    if y is None:
        y = torch.empty_like(k)
    if state_out is None:
        state_out = state_in
    _step_expect(k, w, u, v, None, y, state_in, state_out)
    st = load_library().wkv_step(L, B, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(y),
                                 _ptr(state_in), _ptr(state_out), _stream(stream))
    _check("wkv_step", st)
    return y, state_out


def wkv_step_gated(w, u, k, v, r, state_in, state_out=None, y=None, stream=None):
    """``wkv_step`` with the output gate y = sigmoid(r) * wkv; r: [L][B][C]."""
    if k.dim() != 3:
        raise ValueError("k must be [L][B][C]")
    L, B, C = (int(x) for x in k.shape)
    if y is None:
        y = torch.empty_like(k)
    if state_out is None:
        state_out = state_in
    _step_expect(k, w, u, v, r, y, state_in, state_out)
    st = load_library().wkv_step_gated(L, B, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(r),
                                       _ptr(y), _ptr(state_in), _ptr(state_out), _stream(stream))
    _check("wkv_step_gated", st)
    return y, state_out


def wkv_step_typed(w, u, k, v, state_in, r=None, state_out=None, y=None, stream=None):
    """``wkv_step`` with k, v (r) and y in k's dtype; w, u, state float32."""
    if k.dim() != 3:
        raise ValueError("k must be [L][B][C]")
    if k.dtype not in _DTYPES:
        raise TypeError(f"unsupported element type {k.dtype}")
    dt = k.dtype
    L, B, C = (int(x) for x in k.shape)
    if y is None:
        y = torch.empty_like(k)
    if state_out is None:
        state_out = state_in
    _step_expect(k, w, u, v, r, y, state_in, state_out)
    st = load_library().wkv_step_typed(L, B, C, _DTYPES[dt], _ptr(w), _ptr(u), _ptr(k, dt),
                                       _ptr(v, dt), _ptr(r, dt), _ptr(y, dt), _ptr(state_in),
                                       _ptr(state_out), _stream(stream))
    _check("wkv_step_typed", st)
    return y, state_out


def wkv_token_shift(mu, x, x_prev=None, out=None, x_prev_out=None, stream=None):
    """Token shift of x [B][T][C] by the M weight vectors mu [M][C]:
    out[m] = mu[m] * x_t + (1 - mu[m]) * x_{t-1}, with x_{-1} = x_prev [B][C]
    (zeros when None).  ``x_prev_out`` receives x[:, T-1]; pass True to have it
    allocated, or x_prev itself to update it in place.  Returns
    (out, x_prev_out)."""
    if x.dim() != 3 or mu.dim() != 2:
        raise ValueError("x must be [B][T][C] and mu [M][C]")
    B, T, C = (int(a) for a in x.shape)
    M = int(mu.shape[0])
    dt = x.dtype
    if dt not in _DTYPES:
        raise TypeError(f"unsupported element type {dt}")
    if out is None:
        out = torch.empty((M, B, T, C), device=x.device, dtype=dt)
    if x_prev_out is True:
        x_prev_out = torch.empty((B, C), device=x.device, dtype=dt)
    _expect(x.device, ("mu", mu, (M, C)), ("x_prev", x_prev, (B, C)), ("out", out, (M, B, T, C)),
            ("x_prev_out", x_prev_out, (B, C)))
    lib = load_library()
    if dt == torch.float32:
        st = lib.wkv_token_shift(B, T, C, M, _ptr(mu), _ptr(x), _ptr(x_prev), _ptr(out),
                                 _ptr(x_prev_out), _stream(stream))
        _check("wkv_token_shift", st)
    else:
        # x, x_prev, out and x_prev_out in x's 16-bit format; mu float32
        st = lib.wkv_token_shift_typed(B, T, C, M, _DTYPES[dt], _ptr(mu), _ptr(x, dt),
                                       _ptr(x_prev, dt), _ptr(out, dt), _ptr(x_prev_out, dt),
                                       _stream(stream))
        _check("wkv_token_shift_typed", st)
    return out, x_prev_out


def wkv_token_shift_backward(mu, x, d_out, x_prev=None, d_x_prev_out=None, dx=None,
                             d_x_prev=None, dmu=None, workspace=None, stream=None):
    """Backward of ``wkv_token_shift``: the gradients d_out [M][B][T][C] of the
    mixes and d_x_prev_out [B][C] of the carried token (None: zero) give
    (dx [B][T][C], d_x_prev [B][C] or None, dmu [M][C]).  Pass d_x_prev=True
    to have it allocated."""
    if x.dim() != 3 or mu.dim() != 2:
        raise ValueError("x must be [B][T][C] and mu [M][C]")
    B, T, C = (int(a) for a in x.shape)
    M = int(mu.shape[0])
    dev = x.device
    dt = x.dtype
    if dt not in _DTYPES:
        raise TypeError(f"unsupported element type {dt}")
    dx = torch.empty_like(x) if dx is None else dx
    if d_x_prev is True:
        d_x_prev = torch.empty((B, C), device=dev, dtype=dt)
    dmu = torch.empty((M, C), device=dev, dtype=torch.float32) if dmu is None else dmu
    _expect(dev, ("mu", mu, (M, C)), ("x_prev", x_prev, (B, C)), ("d_out", d_out, (M, B, T, C)),
            ("d_x_prev_out", d_x_prev_out, (B, C)), ("dx", dx, (B, T, C)),
            ("d_x_prev", d_x_prev, (B, C)), ("dmu", dmu, (M, C)))
    lib = load_library()
    need = int(lib.wkv_token_shift_backward_workspace_size(B, T, C, M))
    if workspace is None:
        workspace = torch.empty(max(need, 1), device=dev, dtype=torch.uint8)
    _expect_workspace(dev, workspace, need)
    ws_ptr = ctypes.c_void_p(workspace.data_ptr()) if workspace.numel() > 0 else None
    if dt == torch.float32:
        st = lib.wkv_token_shift_backward(B, T, C, M, _ptr(mu), _ptr(x), _ptr(x_prev),
                                          _ptr(d_out), _ptr(d_x_prev_out), _ptr(dx),
                                          _ptr(d_x_prev), _ptr(dmu), ws_ptr, workspace.numel(),
                                          _stream(stream))
        _check("wkv_token_shift_backward", st)
    else:
        # x, x_prev, the gradients in and dx, d_x_prev out in x's format
        st = lib.wkv_token_shift_backward_typed(
            B, T, C, M, _DTYPES[dt], _ptr(mu), _ptr(x, dt), _ptr(x_prev, dt), _ptr(d_out, dt),
            _ptr(d_x_prev_out, dt), _ptr(dx, dt), _ptr(d_x_prev, dt), _ptr(dmu), ws_ptr,
            workspace.numel(), _stream(stream))
        _check("wkv_token_shift_backward_typed", st)
    return dx, d_x_prev, dmu


def wkv_backward_workspace_size(B: int, T: int, C: int) -> int:
    return int(load_library().wkv_backward_workspace_size(B, T, C))


def wkv_backward(w, u, k, v, dy, dk=None, dv=None, dw=None, du=None, workspace=None,
                 stream=None):
    """Gradients (dk, dv, dw, du) of sum(dy * y) for the GPT-mode forward with the
    empty initial state.  ``workspace`` is a uint8 device tensor of at least
    ``wkv_backward_workspace_size(B, T, C)`` bytes (allocated when omitted)."""
    B, T, C = _bundle_shape(k)
    dev = k.device
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(k) if dv is None else dv
    dw = torch.empty(C, device=dev, dtype=torch.float32) if dw is None else dw
    du = torch.empty(C, device=dev, dtype=torch.float32) if du is None else du
    _bwd_expect(k, w, u, v, dy, dk, dv, dw, du)
    need = wkv_backward_workspace_size(B, T, C)
    if workspace is None:
        workspace = torch.empty(max(need, 1), device=dev, dtype=torch.uint8)
    _expect_workspace(dev, workspace, need)
    ws_ptr = ctypes.c_void_p(workspace.data_ptr()) if workspace.numel() > 0 else None
    st = load_library().wkv_backward(B, T, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(dy),
                                     _ptr(dk), _ptr(dv), _ptr(dw), _ptr(du), ws_ptr,
                                     workspace.numel(), _stream(stream))
    _check("wkv_backward", st)
    return dk, dv, dw, du


def wkv_backward_state(w, u, k, v, dy, state_in=None, state_out=None, d_state_out=None,
                       dk=None, dv=None, dw=None, du=None, d_state_in=None, workspace=None,
                       stream=None):
    """Backward of a chunk with carried states.  ``d_state_out`` is the upstream
    gradient in the coordinates of ``state_out`` (the state the forward
    returned); ``d_state_in=True`` allocates the gradient of ``state_in``.
    Returns (dk, dv, dw, du, d_state_in)."""
    B, T, C = _bundle_shape(k)
    dev = k.device
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(k) if dv is None else dv
    dw = torch.empty(C, device=dev, dtype=torch.float32) if dw is None else dw
    du = torch.empty(C, device=dev, dtype=torch.float32) if du is None else du
    if d_state_in is True:
        d_state_in = torch.empty((3, B, C), device=dev, dtype=torch.float32)
    _bwd_expect(k, w, u, v, dy, dk, dv, dw, du, state_in, state_out, d_state_out, d_state_in)
    need = wkv_backward_workspace_size(B, T, C)
    if workspace is None:
        workspace = torch.empty(max(need, 1), device=dev, dtype=torch.uint8)
    _expect_workspace(dev, workspace, need)
    ws_ptr = ctypes.c_void_p(workspace.data_ptr()) if workspace.numel() > 0 else None
    st = load_library().wkv_backward_state(
        B, T, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(dy), _ptr(state_in), _ptr(state_out),
        _ptr(d_state_out), _ptr(dk), _ptr(dv), _ptr(dw), _ptr(du), _ptr(d_state_in), ws_ptr,
        workspace.numel(), _stream(stream))
    _check("wkv_backward_state", st)
    return dk, dv, dw, du, d_state_in


def wkv_backward_typed(w, u, k, v, dy, state_in=None, state_out=None, d_state_out=None,
                       dk=None, dv=None, dw=None, du=None, d_state_in=None, workspace=None,
                       stream=None):
    """``wkv_backward_state`` with k, v, dy, dk and dv in k's dtype (float32,
    float16 or bfloat16); w, u, dw, du and the states float32."""
    if k.dtype not in _DTYPES:
        raise TypeError(f"unsupported element type {k.dtype}")
    dt = k.dtype
    B, T, C = _bundle_shape(k)
    dev = k.device
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(k) if dv is None else dv
    dw = torch.empty(C, device=dev, dtype=torch.float32) if dw is None else dw
    du = torch.empty(C, device=dev, dtype=torch.float32) if du is None else du
    if d_state_in is True:
        d_state_in = torch.empty((3, B, C), device=dev, dtype=torch.float32)
    _bwd_expect(k, w, u, v, dy, dk, dv, dw, du, state_in, state_out, d_state_out, d_state_in)
    need = wkv_backward_workspace_size(B, T, C)
    if workspace is None:
        workspace = torch.empty(max(need, 1), device=dev, dtype=torch.uint8)
    _expect_workspace(dev, workspace, need)
    ws_ptr = ctypes.c_void_p(workspace.data_ptr()) if workspace.numel() > 0 else None
    st = load_library().wkv_backward_typed(
        B, T, C, _DTYPES[dt], _ptr(w), _ptr(u), _ptr(k, dt), _ptr(v, dt), _ptr(dy, dt),
        _ptr(state_in), _ptr(state_out), _ptr(d_state_out), _ptr(dk, dt), _ptr(dv, dt), _ptr(dw),
        _ptr(du), _ptr(d_state_in), ws_ptr, workspace.numel(), _stream(stream))
    _check("wkv_backward_typed", st)
    return dk, dv, dw, du, d_state_in


def wkv_backward_checkpointed(w, u, k, v, dy, checkpoints, state_in=None, state_out=None,
                              d_state_out=None, dk=None, dv=None, dw=None, du=None,
                              d_state_in=None, workspace=None, stream=None):
    """``wkv_backward_typed`` that rebuilds the forward states from the
    checkpoints ``wkv_forward_checkpointed`` wrote for the same inputs and
    state_in, instead of re-reading k and v in a first pass."""
    if k.dtype not in _DTYPES:
        raise TypeError(f"unsupported element type {k.dtype}")
    dt = k.dtype
    B, T, C = _bundle_shape(k)
    dev = k.device
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(k) if dv is None else dv
    dw = torch.empty(C, device=dev, dtype=torch.float32) if dw is None else dw
    du = torch.empty(C, device=dev, dtype=torch.float32) if du is None else du
    if d_state_in is True:
        d_state_in = torch.empty((3, B, C), device=dev, dtype=torch.float32)
    _bwd_expect(k, w, u, v, dy, dk, dv, dw, du, state_in, state_out, d_state_out, d_state_in,
                checkpoints)
    need = wkv_backward_workspace_size(B, T, C)
    if workspace is None:
        workspace = torch.empty(max(need, 1), device=dev, dtype=torch.uint8)
    _expect_workspace(dev, workspace, need)
    ws_ptr = ctypes.c_void_p(workspace.data_ptr()) if workspace.numel() > 0 else None
    st = load_library().wkv_backward_checkpointed(
        B, T, C, _DTYPES[dt], _ptr(w), _ptr(u), _ptr(k, dt), _ptr(v, dt), _ptr(dy, dt),
        _ptr(state_in), _ptr(checkpoints), _ptr(state_out), _ptr(d_state_out), _ptr(dk, dt),
        _ptr(dv, dt), _ptr(dw), _ptr(du), _ptr(d_state_in), ws_ptr, workspace.numel(),
        _stream(stream))
    _check("wkv_backward_checkpointed", st)
    return dk, dv, dw, du, d_state_in


def wkv_backward_gated(w, u, k, v, r, dy, checkpoints=None, state_in=None, state_out=None,
                       d_state_out=None, dk=None, dv=None, dr=None, dw=None, du=None,
                       d_state_in=None, workspace=None, stream=None):
    """Backward of the gated forward: dy is the gradient of sigmoid(r) * wkv.
    Returns (dk, dv, dr, dw, du, d_state_in); checkpoints None makes the
    backward run its own first pass."""
    if k.dtype not in _DTYPES:
        raise TypeError(f"unsupported element type {k.dtype}")
    dt = k.dtype
    B, T, C = _bundle_shape(k)
    dev = k.device
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(k) if dv is None else dv
    dr = torch.empty_like(k) if dr is None else dr
    dw = torch.empty(C, device=dev, dtype=torch.float32) if dw is None else dw
    du = torch.empty(C, device=dev, dtype=torch.float32) if du is None else du
    if d_state_in is True:
        d_state_in = torch.empty((3, B, C), device=dev, dtype=torch.float32)
    _bwd_expect(k, w, u, v, dy, dk, dv, dw, du, state_in, state_out, d_state_out, d_state_in,
                checkpoints, r, dr)
    need = wkv_backward_workspace_size(B, T, C)
    if workspace is None:
        workspace = torch.empty(max(need, 1), device=dev, dtype=torch.uint8)
    _expect_workspace(dev, workspace, need)
    ws_ptr = ctypes.c_void_p(workspace.data_ptr()) if workspace.numel() > 0 else None
    st = load_library().wkv_backward_gated(
        B, T, C, _DTYPES[dt], _ptr(w), _ptr(u), _ptr(k, dt), _ptr(v, dt), _ptr(r, dt),
        _ptr(dy, dt), _ptr(state_in), _ptr(checkpoints), _ptr(state_out), _ptr(d_state_out),
        _ptr(dk, dt), _ptr(dv, dt), _ptr(dr, dt), _ptr(dw), _ptr(du), _ptr(d_state_in), ws_ptr,
        workspace.numel(), _stream(stream))
    _check("wkv_backward_gated", st)
    return dk, dv, dr, dw, du, d_state_in

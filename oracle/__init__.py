"""Float64 CPU oracle for the RWKV WKV operator -- test infrastructure only.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or executes anything here, and this
package never imports the product.

The arithmetic lives in ``wkv_oracle.c`` (plain C, float64); this module only
compiles it with gcc and marshals numpy arrays.  See the header of that file
for the passages of the pages each function restates and for the parity pin
of each function.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "wkv_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile ``liboracle.so`` with gcc (plain -O2, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fno-fast-math", "-pthread",
             "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build(force=False)
        lib = ctypes.CDLL(_LIB)
        D = ctypes.POINTER(ctypes.c_double)
        i64 = ctypes.c_int64
        lib.wkvo_forward_brute.argtypes = [i64, i64, i64, D, D, D, D, D, D, D]
        lib.wkvo_forward_scan.argtypes = [i64, i64, i64, D, D, D, D, D, D, D, ctypes.c_int]
        lib.wkvo_backward_brute.argtypes = [i64, i64, i64, D, D, D, D, D, D, D, D, D]
        lib.wkvo_backward_scan.argtypes = [i64, i64, i64, D, D, D, D, D, D, D, D, D,
                                           ctypes.c_int]
        lib.wkvo_gate.argtypes = [i64, D, D, D]
        lib.wkvo_gate_backward.argtypes = [i64, D, D, D, D, D]
        lib.wkvo_backward_state.argtypes = [i64, i64, i64] + [D] * 13
        lib.wkvo_backward_magnitude.argtypes = [i64, i64, i64] + [D] * 10 + [ctypes.c_int]
        lib.wkvo_token_shift.argtypes = [i64, i64, i64, i64, D, D, D, D, D]
        lib.wkvo_token_shift_backward.argtypes = [i64, i64, i64, i64] + [D] * 8
        for f in (lib.wkvo_forward_brute, lib.wkvo_forward_scan, lib.wkvo_backward_brute,
                  lib.wkvo_backward_scan, lib.wkvo_gate, lib.wkvo_token_shift,
                  lib.wkvo_backward_state, lib.wkvo_gate_backward,
                  lib.wkvo_token_shift_backward):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _shapes(k, w):
    k = np.asarray(k)
    if k.ndim != 3:
        raise ValueError("k must be [B][T][C]")
    B, T, C = k.shape
    if np.asarray(w).shape != (C,):
        raise ValueError("w and u must be [C]")
    return B, T, C


def forward_brute(w, u, k, v, state_in=None):
    """O(T^2) closed form.  Returns (y [B,T,C], state_out [3,B,C]) in float64."""
    B, T, C = _shapes(k, w)
    w, u, k, v = _f64(w), _f64(u), _f64(k), _f64(v)
    s_in = None if state_in is None else _f64(state_in)
    if s_in is not None and s_in.shape != (3, B, C):
        raise ValueError("state_in must be [3][B][C]")
    y = np.empty((B, T, C))
    s_out = np.empty((3, B, C))
    rc = _load().wkvo_forward_brute(B, T, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(s_in),
                                    _ptr(y), _ptr(s_out))
    if rc:
        raise RuntimeError(f"wkvo_forward_brute failed ({rc})")
    return y, s_out


def forward_scan(w, u, k, v, state_in=None, nthreads: int = 1):
    """O(T) log-space recurrence.  Returns (y [B,T,C], state_out [3,B,C])."""
    B, T, C = _shapes(k, w)
    w, u, k, v = _f64(w), _f64(u), _f64(k), _f64(v)
    s_in = None if state_in is None else _f64(state_in)
    if s_in is not None and s_in.shape != (3, B, C):
        raise ValueError("state_in must be [3][B][C]")
    y = np.empty((B, T, C))
    s_out = np.empty((3, B, C))
    rc = _load().wkvo_forward_scan(B, T, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(s_in),
                                   _ptr(y), _ptr(s_out), int(nthreads))
    if rc:
        raise RuntimeError(f"wkvo_forward_scan failed ({rc})")
    return y, s_out


def backward_brute(w, u, k, v, dy):
    """O(T^2) analytic backward (empty initial state).  Returns (dk, dv, dw, du)."""
    B, T, C = _shapes(k, w)
    w, u, k, v, dy = _f64(w), _f64(u), _f64(k), _f64(v), _f64(dy)
    dk, dv = np.empty((B, T, C)), np.empty((B, T, C))
    dw, du = np.empty(C), np.empty(C)
    rc = _load().wkvo_backward_brute(B, T, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(dy),
                                     _ptr(dk), _ptr(dv), _ptr(dw), _ptr(du))
    if rc:
        raise RuntimeError(f"wkvo_backward_brute failed ({rc})")
    return dk, dv, dw, du


def backward_scan(w, u, k, v, dy, nthreads: int = 1):
    """O(T) reverse-scan backward (empty initial state).  Returns (dk, dv, dw, du)."""
    B, T, C = _shapes(k, w)
    w, u, k, v, dy = _f64(w), _f64(u), _f64(k), _f64(v), _f64(dy)
    dk, dv = np.empty((B, T, C)), np.empty((B, T, C))
    dw, du = np.empty(C), np.empty(C)
    rc = _load().wkvo_backward_scan(B, T, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(dy),
                                    _ptr(dk), _ptr(dv), _ptr(dw), _ptr(du), int(nthreads))
    if rc:
        raise RuntimeError(f"wkvo_backward_scan failed ({rc})")
    return dk, dv, dw, du


def backward_state(w, u, k, v, dy, state_in=None, state_out=None, d_state_out=None):
    """O(T^2) backward with a carried state.  state_in [3][B][C] (None: empty);
    d_state_out [3][B][C] the upstream gradient in the coordinates of state_out
    [3][B][C] (the state the forward returned), or None.  Returns
    (dk, dv, dw, du, d_state_in [3][B][C])."""
    B, T, C = _shapes(k, w)
    w, u, k, v, dy = _f64(w), _f64(u), _f64(k), _f64(v), _f64(dy)
    si = None if state_in is None else _f64(state_in)
    so = None if state_out is None else _f64(state_out)
    ds = None if d_state_out is None else _f64(d_state_out)
    for a in (si, so, ds):
        if a is not None and a.shape != (3, B, C):
            raise ValueError("states must be [3][B][C]")
    if ds is not None and so is None:
        raise ValueError("d_state_out needs state_out")
    dk, dv = np.empty((B, T, C)), np.empty((B, T, C))
    dw, du = np.empty(C), np.empty(C)
    dsi = np.empty((3, B, C))
    rc = _load().wkvo_backward_state(B, T, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(dy),
                                     _ptr(si), _ptr(so), _ptr(ds), _ptr(dk), _ptr(dv), _ptr(dw),
                                     _ptr(du), _ptr(dsi))
    if rc:
        raise RuntimeError(f"wkvo_backward_state failed ({rc})")
    return dk, dv, dw, du, dsi


def backward_magnitude(w, u, k, v, dy, state_in=None, state_out=None, d_state_out=None,
                       nthreads: int = 0):
    """Per channel, sums of the absolute values of the terms of dw (a bound:
    |v_i - y_t| taken as |v_i| + |y_t|) and of du (exact), with the arguments of
    ``backward_state``.  A scale for round-off bounds of dw and du in tests; not
    an operator function.  Returns (mdw [C], mdu [C])."""
    B, T, C = _shapes(k, w)
    w, u, k, v, dy = _f64(w), _f64(u), _f64(k), _f64(v), _f64(dy)
    si = None if state_in is None else _f64(state_in)
    so = None if state_out is None else _f64(state_out)
    ds = None if d_state_out is None else _f64(d_state_out)
    if ds is not None and so is None:
        raise ValueError("d_state_out needs state_out")
    mdw, mdu = np.empty(C), np.empty(C)
    if nthreads <= 0:
        nthreads = max(1, min(16, os.cpu_count() or 1))
    rc = _load().wkvo_backward_magnitude(B, T, C, _ptr(w), _ptr(u), _ptr(k), _ptr(v), _ptr(dy),
                                         _ptr(si), _ptr(so), _ptr(ds), _ptr(mdw), _ptr(mdu),
                                         int(nthreads))
    if rc:
        raise RuntimeError(f"wkvo_backward_magnitude failed ({rc})")
    return mdw, mdu


def gate(y, r):
    """Receptance gate: sigmoid(r) * y, elementwise, float64."""
    y, r = _f64(y), _f64(r)
    if y.shape != r.shape:
        raise ValueError("y and r must have the same shape")
    out = np.empty(y.shape)
    rc = _load().wkvo_gate(int(y.size), _ptr(y), _ptr(r), _ptr(out))
    if rc:
        raise RuntimeError(f"wkvo_gate failed ({rc})")
    return out


def gate_backward(y, r, d):
    """Backward of the gate out = sigmoid(r) * y for the upstream gradient d of
    out: returns (g, dr), g = d * sigmoid(r) the gradient reaching y and
    dr = d * y * sigmoid(r) * (1 - sigmoid(r)).  Elementwise, float64."""
    y, r, d = _f64(y), _f64(r), _f64(d)
    if y.shape != r.shape or y.shape != d.shape:
        raise ValueError("y, r and d must have the same shape")
    g = np.empty(y.shape)
    dr = np.empty(y.shape)
    rc = _load().wkvo_gate_backward(int(y.size), _ptr(y), _ptr(r), _ptr(d), _ptr(g), _ptr(dr))
    if rc:
        raise RuntimeError(f"wkvo_gate_backward failed ({rc})")
    return g, dr


def token_shift(mu, x, x_prev=None):
    """Token shift of x [B][T][C] by M weight vectors mu [M][C], with the last
    token of the previous call x_prev [B][C] (None: zeros).  Returns
    (out [M][B][T][C], x_prev_out [B][C])."""
    x = _f64(x)
    if x.ndim != 3:
        raise ValueError("x must be [B][T][C]")
    B, T, C = x.shape
    mu = _f64(mu)
    if mu.ndim != 2 or mu.shape[1] != C:
        raise ValueError("mu must be [M][C]")
    M = mu.shape[0]
    xp = None if x_prev is None else _f64(x_prev)
    if xp is not None and xp.shape != (B, C):
        raise ValueError("x_prev must be [B][C]")
    out = np.empty((M, B, T, C))
    xpo = np.empty((B, C))
    rc = _load().wkvo_token_shift(B, T, C, M, _ptr(mu), _ptr(x), _ptr(xp), _ptr(out), _ptr(xpo))
    if rc:
        raise RuntimeError(f"wkvo_token_shift failed ({rc})")
    return out, xpo


def token_shift_backward(mu, x, x_prev, d_out, d_x_prev_out=None):
    """Backward of ``token_shift``: upstream gradients d_out [M][B][T][C] of the
    mixes and d_x_prev_out [B][C] of the carried token (None: zero).  Returns
    (dx [B][T][C], d_x_prev [B][C], dmu [M][C])."""
    x = _f64(x)
    if x.ndim != 3:
        raise ValueError("x must be [B][T][C]")
    B, T, C = x.shape
    mu = _f64(mu)
    if mu.ndim != 2 or mu.shape[1] != C:
        raise ValueError("mu must be [M][C]")
    M = mu.shape[0]
    xp = None if x_prev is None else _f64(x_prev)
    d_out = _f64(d_out)
    if d_out.shape != (M, B, T, C):
        raise ValueError("d_out must be [M][B][T][C]")
    dxpo = None if d_x_prev_out is None else _f64(d_x_prev_out)
    dx = np.empty((B, T, C))
    dxp = np.empty((B, C))
    dmu = np.empty((M, C))
    rc = _load().wkvo_token_shift_backward(B, T, C, M, _ptr(mu), _ptr(x), _ptr(xp), _ptr(d_out),
                                           _ptr(dxpo), _ptr(dx), _ptr(dxp), _ptr(dmu))
    if rc:
        raise RuntimeError(f"wkvo_token_shift_backward failed ({rc})")
    return dx, dxp, dmu


def canonical_state(state):
    """(a, b, o) -> (m, lam): m = a/b, the weighted mean of past values, and
    lam = o + ln b, the log of the total decayed weight.  Two (a, b, o) triples
    that describe the same sums give the same (m, lam).  Empty lanes (b == 0)
    give m = 0, lam = -inf."""
    s = np.asarray(state, dtype=np.float64)
    a, b, o = s[0], s[1], s[2]
    with np.errstate(divide="ignore", invalid="ignore"):
        m = np.where(b > 0, a / np.where(b > 0, b, 1.0), 0.0)
        lam = np.where(b > 0, o + np.log(np.where(b > 0, b, 1.0)), -np.inf)
    return m, lam

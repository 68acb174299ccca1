"""torch.autograd functions over libwkv: argument marshalling only.

``wkv_time_mix`` (``WkvFunction``) is the WKV operator of a time-mixing block
as one differentiable op.  Its forward is ``wkv_forward_checkpointed``; its
backward is ``wkv_backward_checkpointed``, or ``wkv_backward_gated`` when the
receptance gate is fused.  Gradients reach w, u, k, v, r and the carried state.
The operator is the closed form of the RWKV architecture deep dive
(youngju.dev, "WKV mechanism: core computation"), run in RNN mode over chunks
(rwkv-architecture skill page, "Quick start"), with the output gate
sigmoid(r) * wkv of the deep dive's "RWKV architecture overview" block figure.

``token_shift`` (``TokenShiftFunction``) is the token shift in front of it
(deep dive, section "Token shift"), as ``wkv_token_shift`` and
``wkv_token_shift_backward``.

Everything runs in libwkv's kernels.  The only work here is choosing the
entry point, making tensors contiguous and allocating outputs; there is no
fallback.  The backward is a kernel call, so it is differentiable once: a
second derivative raises.

The state's gradient: whatever consumes state_out sees only its true sums
A = a e^o and B = b e^o.  So the gradient of state_out flows through its a and
b planes, and its o plane's gradient is not read.  The d_state_in returned for
state_in is complete, o plane included.  Chaining calls over the chunks of a
sequence, each chunk's state_out the next one's state_in, therefore gives the
gradients of one call over the whole sequence.  A loss that reads state_out's
o plane other than through A and B is outside this contract.
"""
from __future__ import annotations

import torch
from torch.autograd.function import once_differentiable

from . import wkv as _w


def _c(t):
    return None if t is None else t.contiguous()


class WkvFunction(torch.autograd.Function):
    """(w, u, k, v, r, state_in) -> (y, state_out).

    w, u [C] float32; k, v, r [B][T][C] float32, float16 or bfloat16 (r may be
    None: no gate); state_in [3][B][C] float32 or None (the empty state).
    y has k's dtype; state_out is float32.  The forward keeps its checkpoints
    (the state before every 128th token) for the backward, which then reads k
    and v once.
    """

    @staticmethod
    def forward(ctx, w, u, k, v, r, state_in):
        w, u, k, v, r, s_in = (_c(t) for t in (w, u, k, v, r, state_in))
        y, s_out, ck = _w.wkv_forward_checkpointed(w, u, k, v, r=r, state_in=s_in,
                                                   state_out=True)
        ctx.gated = r is not None
        ctx.has_state = s_in is not None
        ctx.save_for_backward(w, u, k, v, r, s_in, s_out, ck)
        return y, s_out

    @staticmethod
    @once_differentiable
    def backward(ctx, dy, d_state_out):
        w, u, k, v, r, s_in, s_out, ck = ctx.saved_tensors
        dy = torch.zeros_like(k) if dy is None else dy.to(k.dtype).contiguous()
        d_so = _c(d_state_out)
        s_so = s_out if d_so is not None else None
        want_dsi = True if ctx.has_state and ctx.needs_input_grad[5] else None
        if ctx.gated:
            dk, dv, dr, dw, du, dsi = _w.wkv_backward_gated(
                w, u, k, v, r, dy, checkpoints=ck, state_in=s_in, state_out=s_so,
                d_state_out=d_so, d_state_in=want_dsi)
        else:
            dk, dv, dw, du, dsi = _w.wkv_backward_checkpointed(
                w, u, k, v, dy, ck, state_in=s_in, state_out=s_so, d_state_out=d_so,
                d_state_in=want_dsi)
            dr = None
        return dw, du, dk, dv, dr, dsi


def wkv_time_mix(w, u, k, v, r=None, state_in=None):
    """Differentiable WKV: returns (y, state_out); see ``WkvFunction``."""
    return WkvFunction.apply(w, u, k, v, r, state_in)


class TokenShiftFunction(torch.autograd.Function):
    """(mu, x, x_prev) -> (out, x_prev_out): out[m] = mu[m] x_t + (1 - mu[m])
    x_{t-1} with x_{-1} = x_prev (zeros when None), and x_prev_out = x[:, T-1]
    (the token carried to the next chunk).  mu [M][C] float32; x [B][T][C] and
    x_prev [B][C] float32, float16 or bfloat16."""

    @staticmethod
    def forward(ctx, mu, x, x_prev):
        mu, x, xp = _c(mu), _c(x), _c(x_prev)
        out, xpo = _w.wkv_token_shift(mu, x, xp, x_prev_out=True)
        ctx.has_prev = xp is not None
        ctx.save_for_backward(mu, x, xp)
        return out, xpo

    @staticmethod
    @once_differentiable
    def backward(ctx, d_out, d_x_prev_out):
        mu, x, xp = ctx.saved_tensors
        M, (B, T, C) = mu.shape[0], x.shape
        if d_out is None:
            d_out = torch.zeros((M, B, T, C), device=x.device, dtype=x.dtype)
        d_out = d_out.to(x.dtype).contiguous()
        d_xpo = None if d_x_prev_out is None else d_x_prev_out.to(x.dtype).contiguous()
        want = True if ctx.has_prev and ctx.needs_input_grad[2] else None
        dx, dxp, dmu = _w.wkv_token_shift_backward(mu, x, d_out, x_prev=xp,
                                                   d_x_prev_out=d_xpo, d_x_prev=want)
        return dmu, dx, dxp


def token_shift(mu, x, x_prev=None):
    """Differentiable token shift: returns (out, x_prev_out); see
    ``TokenShiftFunction``."""
    return TokenShiftFunction.apply(mu, x, x_prev)

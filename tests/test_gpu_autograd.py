"""GPU tests of the autograd functions (linear_recurrent_attention_amd.autograd)
against the oracle's gradients.

Expected values come from the oracle on the same seeded inputs, chained by
hand: its forward scan, its gate backward, its carried-state backward and its
token-shift backward.  Tolerances are tests/parity.py's: y within 1e-5 +
1e-4 |r|; gradients within 1e-3 relative + 1e-3 of the tensor's rms + the
float32 round-off floor; 16-bit outputs add the format's relative half-unit.
"""
import sys

import numpy as np
import pytest
import torch

from linear_recurrent_attention_amd import synth, wkv
from linear_recurrent_attention_amd.autograd import token_shift, wkv_time_mix
from parity import (G_FLOOR, G_RTOL, assert_chained_sums_close, assert_grad_close,
                    assert_sums_close, assert_y_close, f64, roundoff_floor)

pytestmark = pytest.mark.gpu

HALF_ULP = {torch.float32: 0.0, torch.float16: 2.0 ** -11, torch.bfloat16: 2.0 ** -8}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no HIP device visible")
    wkv.load_library()


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def leaf(t, dtype=None):
    t = t.cuda() if dtype is None else t.to(dtype).cuda()
    return t.contiguous().requires_grad_()


def reachable_state(oracle, B, C, index):
    p = synth.make(synth.TINY, index=index, B=B, T=11, C=C)
    _, s = oracle.forward_scan(*(f64(p[n]) for n in ("w", "u", "k", "v")))
    return s.astype(np.float32).astype(np.float64)


def close(got, ref, what, h=0.0, floor=0.0):
    got = f64(got)
    assert np.all(np.isfinite(got)), f"{what}: non-finite"
    if ref.size == 0:
        return
    rms = float(np.sqrt(np.mean(ref * ref)))
    e = float(np.max(np.abs(got - ref) / ((G_RTOL + h) * np.abs(ref) + G_FLOOR * rms + floor
                                          + 1e-300)))
    assert e <= 1.0, f"{what}: {e:.3g}x the tolerance"


@pytest.mark.parametrize("chunks", [(300, 213), (128, 1, 256), (77,)],
                         ids=["2chunks", "3chunks", "1chunk"])
def test_chunked_training_matches_one_call(oracle, chunks):
    """Chunks chained through the carried state, the loss on every chunk's
    output: the gradients of k and v (per chunk), w, u and the first state
    are those of one call over the whole sequence from that state."""
    B, C = 2, 96
    T = sum(chunks)
    d = synth.make(synth.STABILITY, index=140, B=B, T=T, C=C, with_dy=True)
    s0 = reachable_state(oracle, B, C, 141)
    note(f"autograd chunks {chunks}")
    w, u = leaf(d["w"]), leaf(d["u"])
    state = leaf(torch.from_numpy(s0.astype(np.float32)))
    s_first = state
    ks, vs, ys, t = [], [], [], 0
    loss = 0.0
    for n in chunks:
        k, v = leaf(d["k"][:, t:t + n]), leaf(d["v"][:, t:t + n])
        y, state = wkv_time_mix(w, u, k, v, state_in=state)
        loss = loss + (y * d["dy"][:, t:t + n].cuda()).sum()
        ks.append(k)
        vs.append(v)
        ys.append(y)
        t += n
    loss.backward()
    torch.cuda.synchronize()
    a = {n: f64(d[n]) for n in ("w", "u", "k", "v", "dy")}
    y_ref, _ = oracle.forward_scan(a["w"], a["u"], a["k"], a["v"], s0)
    assert_y_close(f64(torch.cat(ys, 1)), y_ref)
    dk, dv, dw, du, dsi = oracle.backward_state(a["w"], a["u"], a["k"], a["v"], a["dy"], s0)
    f = roundoff_floor(a["dy"], a["v"])
    fs = roundoff_floor(a["dy"], a["v"], summed=True)
    assert_grad_close(f64(torch.cat([k.grad for k in ks], 1)), dk, "dk", f)
    assert_grad_close(f64(torch.cat([v.grad for v in vs], 1)), dv, "dv", f)
    assert_chained_sums_close(oracle, f64(w.grad), f64(u.grad), dw, du, a["w"], a["u"], a["k"],
                              a["v"], a["dy"], chunks, s0)
    for pl in range(3):
        assert_grad_close(f64(s_first.grad)[pl], dsi[pl], f"d_state_in[{pl}]", fs)


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16, torch.float16],
                         ids=["f32", "bf16", "f16"])
@pytest.mark.parametrize("shape", [(2, 300, 100), (1, 1024, 64)],
                         ids=lambda s: "x".join(map(str, s)))
def test_gated_time_mix_gradients(oracle, dt, shape):
    """y = sigmoid(r) * wkv from the empty state, loss sum(y * G): gradients of
    w, u, k, v and r against the oracle on the values the GPU consumed."""
    B, T, C = shape
    d = synth.make(synth.STABILITY, index=142, B=B, T=T, C=C, with_dy=True)
    r = synth.receptance(synth.STABILITY, 142, (B, T, C))
    note(f"autograd gated {dt} B={B} T={T} C={C}")
    w, u = leaf(d["w"]), leaf(d["u"])
    k, v, rr = leaf(d["k"], dt), leaf(d["v"], dt), leaf(r, dt)
    G = d["dy"].to(dt)
    y, s_out = wkv_time_mix(w, u, k, v, r=rr)
    assert y.dtype == dt and s_out.dtype == torch.float32
    (y.float() * G.cuda().float()).sum().backward()
    torch.cuda.synchronize()
    a = {n: f64(x) for n, x in (("w", w), ("u", u), ("k", k), ("v", v), ("r", rr))}
    g_in = f64(G)
    wkv_ref, _ = oracle.forward_scan(a["w"], a["u"], a["k"], a["v"])
    g, dr = oracle.gate_backward(wkv_ref, a["r"], g_in)
    dk, dv, dw, du, _ = oracle.backward_state(a["w"], a["u"], a["k"], a["v"], g)
    h = HALF_ULP[dt]
    f = roundoff_floor(g, a["v"])
    close(k.grad, dk, "dk", h, f)
    close(v.grad, dv, "dv", h, f)
    close(rr.grad, dr, "dr", h, f)
    assert_sums_close(oracle, f64(w.grad), f64(u.grad), dw, du, a["w"], a["u"], a["k"], a["v"], g)


def test_state_gradient_through_a_loss_on_the_state(oracle):
    """A loss on y and on the state handed on (through its true sums, as the
    next chunk sees it): the state's gradient enters as d_state_out."""
    B, T, C = 2, 257, 64
    d = synth.make(synth.STABILITY, index=143, B=B, T=T, C=C, with_dy=True)
    s0 = reachable_state(oracle, B, C, 144)
    H = synth.normal((2, B, C), 1.0, synth.seed_of(synth.GPT, 9720, 0))
    note("autograd state loss")
    w, u, k, v = leaf(d["w"]), leaf(d["u"]), leaf(d["k"]), leaf(d["v"])
    s_in = leaf(torch.from_numpy(s0.astype(np.float32)))
    y, s_out = wkv_time_mix(w, u, k, v, state_in=s_in)
    # a consumer of the state: its true sums A = a e^o, B = b e^o, scaled by a
    # fixed e^-o so that they stay finite; the gradient of (A, B) times H
    o_fix = s_out[2].detach()
    A = s_out[0] * torch.exp(s_out[2] - o_fix)
    Bs = s_out[1] * torch.exp(s_out[2] - o_fix)
    loss = (y * d["dy"].cuda()).sum() + (A * H[0].cuda()).sum() + (Bs * H[1].cuda()).sum()
    loss.backward()
    torch.cuda.synchronize()
    so = f64(s_out)
    # the upstream gradient of state_out's planes, as autograd formed it
    g_out = np.stack([f64(H[0]), f64(H[1]), f64(H[0]) * so[0] + f64(H[1]) * so[1]])
    a = {n: f64(d[n]) for n in ("w", "u", "k", "v", "dy")}
    dk, dv, dw, du, dsi = oracle.backward_state(a["w"], a["u"], a["k"], a["v"], a["dy"], s0,
                                                so, g_out)
    f = roundoff_floor(a["dy"], a["v"])
    fs = roundoff_floor(a["dy"], a["v"], summed=True)
    assert_grad_close(f64(k.grad), dk, "dk", f)
    assert_grad_close(f64(v.grad), dv, "dv", f)
    assert_sums_close(oracle, f64(w.grad), f64(u.grad), dw, du, a["w"], a["u"], a["k"], a["v"],
                      a["dy"], s0, so, g_out)
    for pl in range(3):
        assert_grad_close(f64(s_in.grad)[pl], dsi[pl], f"d_state_in[{pl}]", fs)


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_time_mix_block_training_path(oracle, dt):
    """Token shift, then the gated WKV on the three mixes (k, v, r taken as the
    mixes themselves), loss sum(y * G): gradients of x, x_prev, mu, w and u
    against the oracle's pieces chained by hand."""
    B, T, C, M = 2, 200, 64, 3
    mu, x, xp = synth.shift_inputs(synth.GPT, 145, B, T, C, M)
    d = synth.make(synth.STABILITY, index=145, B=B, T=T, C=C, with_dy=True)
    note(f"autograd block {dt}")
    mu_d, x_d, xp_d = leaf(mu), leaf(x, dt), leaf(xp, dt)
    w, u = leaf(d["w"]), leaf(d["u"])
    G = d["dy"].to(dt)
    mixes, x_last = token_shift(mu_d, x_d, xp_d)
    y, _ = wkv_time_mix(w, u, mixes[0], mixes[1], r=mixes[2])
    (y.float() * G.cuda().float()).sum().backward()
    torch.cuda.synchronize()
    assert torch.equal(x_last, x_d[:, -1])
    # the oracle on the mixes the GPU produced (the values the WKV consumed)
    mx = f64(mixes)
    ref_mix, _ = oracle.token_shift(f64(mu_d), f64(x_d), f64(xp_d))
    mag, _ = oracle.token_shift(f64(mu_d), np.abs(f64(x_d)), np.abs(f64(xp_d)))
    assert np.all(np.abs(mx - ref_mix) <= (1e-6 + HALF_ULP[dt]) * mag)
    a = {n: f64(d[n]) for n in ("w", "u")}
    g_in = f64(G)
    wkv_ref, _ = oracle.forward_scan(a["w"], a["u"], mx[0], mx[1])
    g, dr = oracle.gate_backward(wkv_ref, mx[2], g_in)
    dk, dv, dw, du, _ = oracle.backward_state(a["w"], a["u"], mx[0], mx[1], g)
    # the mixes' gradients, rounded to the activation format as the GPU stores
    # them, into the token shift's backward
    d_mix = np.stack([dk, dv, dr])
    d_mix_r = torch.from_numpy(d_mix).to(dt).double().numpy()
    mu_, x_, xp_ = f64(mu_d), f64(x_d), f64(xp_d)
    dx, dxp, dmu = oracle.token_shift_backward(mu_, x_, xp_, d_mix_r)
    h = HALF_ULP[dt]
    assert_sums_close(oracle, f64(w.grad), f64(u.grad), dw, du, a["w"], a["u"], mx[0], mx[1], g)
    # Each mix gradient is within (G_RTOL + 2h)|d| + G_FLOOR rms(d) + f of its
    # rounded reference (one rounding to the format on either side), dx and
    # d_x_prev add their own rounding (h), and the shift's weights mu and
    # 1 - mu are non-negative.  So the shift's backward of |d| and of rms(d)
    # bounds the error of dx, d_x_prev and dmu.
    f = roundoff_floor(g, mx[1])
    rms = np.sqrt(np.mean(d_mix_r ** 2, axis=(1, 2, 3), keepdims=True)) + np.zeros_like(d_mix_r)
    ax, axp = np.abs(x_), np.abs(xp_)
    m1x, m1p, _ = oracle.token_shift_backward(mu_, ax, axp, np.abs(d_mix_r))
    m2x, m2p, _ = oracle.token_shift_backward(mu_, ax, axp, rms)
    prev = np.concatenate([xp_[:, None], x_[:, :-1]], axis=1)
    span = ax + np.abs(prev)
    m1mu = np.einsum("mbtc,btc->mc", np.abs(d_mix_r), span)
    m2mu = np.einsum("mbtc,btc->mc", rms, span)
    tol = lambda m1, m2, n: (G_RTOL + 3 * h) * m1 + G_FLOOR * m2 + n * f + 1e-300
    for name, got, ref, m1, m2, n in (("dx", x_d.grad, dx, m1x, m2x, 2 * M),
                                      ("d_x_prev", xp_d.grad, dxp, m1p, m2p, M),
                                      ("dmu", mu_d.grad, dmu, m1mu, m2mu, B * T)):
        got = f64(got)
        assert np.all(np.isfinite(got)), name
        e = float(np.max(np.abs(got - ref) / tol(m1, m2, n)))
        assert e <= 1.0, f"{name}: {e:.3g}x the tolerance"

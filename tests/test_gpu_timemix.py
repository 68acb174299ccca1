"""GPU parity of the time-mixing prologue and epilogue against the oracle:
the output gate fused into the forward and the step (y = sigmoid(r) * wkv), and
the token shift (RWKV architecture deep dive: block figure of "RWKV
architecture overview"; "Token shift").

Tolerances: the gated output uses the forward's bound (tests/parity.py), which
still holds after multiplying by sigmoid(r) <= 1 (the gate's own float32 error
is ~1e-7 relative).  The token shift is two products and a sum per element, so
its bound is 1e-6 (|mu x_t| + |(1 - mu) x_{t-1}|) per element; the carried
token it returns is a copy and must be bit-exact.
"""
import os
import sys

import numpy as np
import pytest
import torch

from linear_recurrent_attention_amd import synth, wkv
from parity import assert_state_close, assert_y_close, f64

pytestmark = pytest.mark.gpu

NTHREADS = max(1, min(16, os.cpu_count() or 1))

GATED_PLANS = {
    "auto": None,
    "lane": (wkv.WKV_KERNEL_LANE, 0, 0),
    "seg16x16": (wkv.WKV_KERNEL_SEGMENTED, 16, 16),
    "seg16x8": (wkv.WKV_KERNEL_SEGMENTED, 16, 8),
    "seg8x32": (wkv.WKV_KERNEL_SEGMENTED, 8, 32),
    "seg16x16c32": (wkv.WKV_KERNEL_SEGMENTED, 16, 16, 32),
    "seg32x8c16": (wkv.WKV_KERNEL_SEGMENTED, 32, 8, 16),
    "lb4x16": (wkv.WKV_KERNEL_LOOKBACK, 4, 16),
    "lb8x16": (wkv.WKV_KERNEL_LOOKBACK, 8, 16),
    "lb8x8": (wkv.WKV_KERNEL_LOOKBACK, 8, 8),
    "lb4x16c128": (wkv.WKV_KERNEL_LOOKBACK, 4, 16, 128),
    "lb2x8c256": (wkv.WKV_KERNEL_LOOKBACK, 2, 8, 256),
}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no HIP device visible")
    wkv.load_library()


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def reachable_state(oracle, B, C, seed):
    d = synth.make(synth.TINY, index=700 + seed, B=B, T=9, C=C)
    _, s = oracle.forward_scan(*(d[n].double().numpy() for n in ("w", "u", "k", "v")))
    return torch.from_numpy(s.astype(np.float32))


def gated_reference(oracle, d, r, s_in=None):
    y, s = oracle.forward_scan(*(f64(d[n]) for n in ("w", "u", "k", "v")),
                               None if s_in is None else s_in.double().numpy(),
                               nthreads=NTHREADS)
    return oracle.gate(y, f64(r)), s


def run_gated(d, r, plan, s_in=None):
    dev = torch.device("cuda")
    w, u, k, v = (d[n].to(dev) for n in ("w", "u", "k", "v"))
    si = None if s_in is None else s_in.to(dev)
    y, so = wkv.wkv_forward_gated(w, u, k, v, r.to(dev), state_in=si, state_out=True, plan=plan)
    torch.cuda.synchronize()
    return y, so


# ------------------------------------------------------------ output gate ---

SHAPES = [(1, 1, 5), (2, 300, 100), (3, 17, 64), (1, 513, 130), (2, 1024, 64), (1, 2049, 33)]


@pytest.mark.parametrize("plan", list(GATED_PLANS))
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("with_state", [False, True])
def test_gated_forward_matches_oracle(oracle, plan, shape, with_state):
    B, T, C = shape
    d = synth.make(synth.GPT, index=31, B=B, T=T, C=C)
    r = synth.receptance(synth.GPT, 31, (B, T, C))
    si = reachable_state(oracle, B, C, 1) if with_state else None
    note(f"gated B={B} T={T} C={C} state={with_state} plan={plan}")
    y, so = run_gated(d, r, GATED_PLANS[plan], si)
    yr, sr = gated_reference(oracle, d, r, si)
    assert_y_close(f64(y), yr, "gated y")
    assert_state_close(f64(so), sr)


@pytest.mark.parametrize("plan", ["auto", "lane", "seg16x16", "lb4x16", "lb8x8"])
def test_gated_forward_wide_exponents(oracle, plan):
    d = synth.make(synth.STABILITY, index=32, B=2, T=1500, C=96)
    r = synth.receptance(synth.STABILITY, 32, (2, 1500, 96))
    note(f"gated stability B=2 T=1500 C=96 plan={plan}")
    y, so = run_gated(d, r, GATED_PLANS[plan])
    yr, sr = gated_reference(oracle, d, r)
    assert_y_close(f64(y), yr, "gated y")
    assert_state_close(f64(so), sr)


def test_gated_forward_saturated_gate(oracle):
    """r far in either tail: the gate is exactly 0 or passes wkv unchanged."""
    d = synth.make(synth.TINY, index=33, B=2, T=40, C=64)
    r = torch.full((2, 40, 64), 200.0)
    r[:, ::2] = -200.0
    y, _ = run_gated(d, r, None)
    yr, _ = gated_reference(oracle, d, r)
    assert torch.all(y.cpu()[:, ::2] == 0)
    assert_y_close(f64(y), yr, "gated y")


def test_gated_gpt_workload_full_size(oracle):
    """B=8 T=1024 C=2048 (one layer of the GPT workload), every element."""
    d = synth.make(synth.GPT, index=3)
    r = synth.receptance(synth.GPT, 3, (8, 1024, 2048))
    note("gated gpt B=8 T=1024 C=2048 auto")
    y, so = run_gated(d, r, None)
    yr, sr = gated_reference(oracle, d, r)
    assert_y_close(f64(y), yr, "gated y")
    assert_state_close(f64(so), sr)


def test_gated_forward_captured_in_a_graph(oracle):
    """Under stream capture the gated forward runs a kernel without cross-launch
    state; every replay matches the oracle."""
    dev = torch.device("cuda")
    d = synth.make(synth.GPT, index=34, B=2, T=700, C=128)
    r = synth.receptance(synth.GPT, 34, (2, 700, 128))
    w, u, k, v, rr = (t.to(dev) for t in (d["w"], d["u"], d["k"], d["v"], r))
    y = torch.empty_like(k)
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            wkv.wkv_forward_gated(w, u, k, v, rr, y=y, stream=s)
    yr, _ = gated_reference(oracle, d, r)
    for i in range(3):
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        note(f"gated graph replay {i}")
        assert_y_close(f64(y), yr, f"gated y, replay {i}")


@pytest.mark.parametrize("shape", [(3, 4, 40), (2, 3, 37), (1, 1, 1), (4, 2, 1030),
                                   (2, 3, 1032), (1, 2, 5128), (2, 2, 2056)],
                         ids=lambda s: "x".join(map(str, s)))
def test_gated_steps_match_oracle(oracle, shape):
    """Several gated steps from a reachable state, in place: y and the state
    against the oracle, one token at a time."""
    L, B, C = shape
    dev = torch.device("cuda")
    w = torch.stack([synth.channel_params(synth.DECODE, 40 + l, C)[0] for l in range(L)])
    u = torch.stack([synth.channel_params(synth.DECODE, 40 + l, C)[1] for l in range(L)])
    st = torch.stack([reachable_state(oracle, B, C, 10 + l) for l in range(L)])
    ref = [st[l].double().numpy() for l in range(L)]
    st_d = st.to(dev)
    note(f"gated step L={L} B={B} C={C}")
    for step in range(3):
        k, v = synth.sequence(synth.DECODE, 900 + step, (L, B, C))
        r = synth.receptance(synth.DECODE, 900 + step, (L, B, C))
        y, _ = wkv.wkv_step_gated(w.to(dev), u.to(dev), k.to(dev), v.to(dev), r.to(dev), st_d)
        torch.cuda.synchronize()
        for l in range(L):
            yl, ref[l] = oracle.forward_scan(f64(w[l]), f64(u[l]), f64(k[l])[:, None, :],
                                             f64(v[l])[:, None, :], ref[l])
            assert_y_close(f64(y[l]), oracle.gate(yl[:, 0, :], f64(r[l])), f"step {step} y")
            assert_state_close(f64(st_d[l]), ref[l], f"step {step} state")


# ------------------------------------------------------------ token shift ---

def shift_bound(mu, x, xp):
    """Per-element bound 1e-6 (|mu x_t| + |(1 - mu) x_{t-1}|) on [M][B][T][C]."""
    mu = np.asarray(mu, dtype=np.float64)[:, None, None, :]
    x = np.asarray(x, dtype=np.float64)
    prev = np.concatenate([np.zeros_like(x[:, :1]) if xp is None else
                           np.asarray(xp, dtype=np.float64)[:, None], x[:, :-1]], axis=1)
    return 1e-6 * (np.abs(mu * x[None]) + np.abs((1 - mu) * prev[None])) + 1e-30


def check_shift(oracle, mu, x, xp, out, xpo):
    ro, rp = oracle.token_shift(f64(mu), f64(x), None if xp is None else f64(xp))
    got = f64(out)
    assert np.all(np.isfinite(got))
    err = np.abs(got - ro) / shift_bound(f64(mu), f64(x), None if xp is None else f64(xp))
    assert float(err.max(initial=0.0)) <= 1.0, f"token shift off by {err.max():.3g}x"
    if xpo is not None:
        assert np.array_equal(f64(xpo), rp), "carried token is not a bit-exact copy"


SHIFT_SHAPES = [(1, 1, 4), (2, 16, 64), (2, 17, 64), (3, 100, 260), (1, 33, 33), (2, 5, 1027),
                (8, 512, 2048)]  # (the last: a grid the forward hands to the dies in windows)


@pytest.mark.parametrize("M", [1, 3, 5, 8])
@pytest.mark.parametrize("shape", SHIFT_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("with_prev", [False, True])
def test_token_shift_matches_oracle(oracle, M, shape, with_prev):
    B, T, C = shape
    mu, x, xp = synth.shift_inputs(synth.GPT, 50, B, T, C, M)
    dev = torch.device("cuda")
    note(f"shift B={B} T={T} C={C} M={M} prev={with_prev}")
    out, xpo = wkv.wkv_token_shift(mu.to(dev), x.to(dev), xp.to(dev) if with_prev else None,
                                   x_prev_out=True)
    torch.cuda.synchronize()
    check_shift(oracle, mu, x, xp if with_prev else None, out, xpo)


@pytest.mark.parametrize("T", [1, 16, 17, 100])
def test_token_shift_state_in_place(oracle, T):
    """x_prev_out == x_prev: the carried token is read before it is replaced,
    whether the sequence spans one tile or several."""
    B, C, M = 3, 200, 3
    mu, x, xp = synth.shift_inputs(synth.GPT, 51, B, T, C, M)
    dev = torch.device("cuda")
    state = xp.to(dev).clone()
    note(f"shift in place T={T}")
    out, _ = wkv.wkv_token_shift(mu.to(dev), x.to(dev), state, x_prev_out=state)
    torch.cuda.synchronize()
    check_shift(oracle, mu, x, xp, out, state)


def test_token_shift_unaligned_rows(oracle):
    """Buffers that are not 16-byte aligned take the one-channel path."""
    B, T, C, M = 2, 40, 64, 3
    mu, x, xp = synth.shift_inputs(synth.GPT, 52, B, T, C, M)
    dev = torch.device("cuda")
    big = torch.empty(B * T * C + 1, device=dev)
    xd = big[1:].view(B, T, C)
    xd.copy_(x.to(dev))
    note("shift unaligned x")
    out, xpo = wkv.wkv_token_shift(mu.to(dev), xd, xp.to(dev), x_prev_out=True)
    torch.cuda.synchronize()
    check_shift(oracle, mu, x, xp, out, xpo)


def test_token_shift_chunking_is_exact(oracle):
    """Calls over chunks with the carried token updated in place give the same
    bits as one call (every element sees the same two operands)."""
    B, T, C, M = 2, 97, 128, 3
    mu, x, _ = synth.shift_inputs(synth.GPT, 53, B, T, C, M)
    dev = torch.device("cuda")
    mu_d, x_d = mu.to(dev), x.to(dev)
    whole, last = wkv.wkv_token_shift(mu_d, x_d, None, x_prev_out=True)
    state = torch.zeros(B, C, device=dev)
    parts, t = [], 0
    for n in (1, 16, 17, 40, 23):
        o, _ = wkv.wkv_token_shift(mu_d, x_d[:, t:t + n].contiguous(), state, x_prev_out=state)
        parts.append(o)
        t += n
    torch.cuda.synchronize()
    note("shift chunked")
    assert torch.equal(torch.cat(parts, dim=2), whole)
    assert torch.equal(state, last)
    check_shift(oracle, mu, x, None, whole, last)


def test_token_shift_empty_calls(oracle):
    dev = torch.device("cuda")
    mu, x, xp = synth.shift_inputs(synth.GPT, 54, 2, 5, 8, 2)
    xpd = xp.to(dev)
    # T == 0: the carried token passes through (zeros for a fresh sequence)
    out, xpo = wkv.wkv_token_shift(mu.to(dev), x[:, :0].to(dev), xpd, x_prev_out=True)
    _, xz = wkv.wkv_token_shift(mu.to(dev), x[:, :0].to(dev), None, x_prev_out=True)
    # M == 0: only the carried token is updated
    out0, xpm = wkv.wkv_token_shift(mu[:0].to(dev), x.to(dev), xpd, x_prev_out=True)
    torch.cuda.synchronize()
    assert out.shape == (2, 2, 0, 8) and out0.shape == (0, 2, 5, 8)
    assert torch.equal(xpo.cpu(), xp)
    assert torch.equal(xz.cpu(), torch.zeros(2, 8))
    assert torch.equal(xpm.cpu(), x[:, -1])


def test_token_shift_gpt_shape_full(oracle):
    """B=8 T=1024 C=2048 with the three mixes of the R, K, V inputs, every element."""
    B, T, C, M = 8, 1024, 2048, 3
    mu, x, xp = synth.shift_inputs(synth.GPT, 55, B, T, C, M)
    dev = torch.device("cuda")
    note("shift B=8 T=1024 C=2048 M=3")
    out, xpo = wkv.wkv_token_shift(mu.to(dev), x.to(dev), xp.to(dev), x_prev_out=True)
    torch.cuda.synchronize()
    check_shift(oracle, mu, x, xp, out, xpo)

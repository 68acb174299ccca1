"""Seeded edge-case inputs through every forward plan, the step, and the
backward (own first pass, from checkpoints, gated), against the oracle.

Each case stresses one place where a kernel's frame or fast path could leave
float's range while the inputs are valid (w > 0, finite):
- spikes:  isolated keys of +60 among zeros, slow decay (w = 1e-3);
- falling: keys falling linearly from +40 to -40 over each 64 tokens, so a
  segment's first token holds its largest exponent;
- rising:  keys rising from -40 to +40, so the first token is far below it;
- edge:    bonuses at both ends of the one-exponential range and just past
  them (|u - w| around 86 in log2 units), with fast and slow decays;
- tiny:    a carried state with denominator 1e-30 and a large exponent;
- huge:    keys of +-200 (far past e^k's float range; only differences of
  exponents are ever formed), decays from 1e-3 to 5.
Bonuses span -59 to +59 across the channels of every case but "edge".
The gated forward with bf16 activations runs the same cases on the look-back
and segmented plans.
"""
import sys

import numpy as np
import pytest
import torch

from linear_recurrent_attention_amd import synth, wkv
from parity import assert_grad_close, assert_state_close, assert_sums_close, assert_y_close, f64
from parity import roundoff_floor

pytestmark = pytest.mark.gpu

B, T, C = 2, 256, 64
RAGGED = (3, 129, 70)  # partial last block and tile, C not a multiple of 64
LOG2E = 1.4426950408889634

PLANS = {
    "auto": None,
    "lane": (wkv.WKV_KERNEL_LANE, 0, 0),
    "seg16x16": (wkv.WKV_KERNEL_SEGMENTED, 16, 16),
    "seg8x32": (wkv.WKV_KERNEL_SEGMENTED, 8, 32),
    "seg32x8c16": (wkv.WKV_KERNEL_SEGMENTED, 32, 8, 16),
    "lb4x16": (wkv.WKV_KERNEL_LOOKBACK, 4, 16),
    "lb4x32": (wkv.WKV_KERNEL_LOOKBACK, 4, 32),
    "lb8x8": (wkv.WKV_KERNEL_LOOKBACK, 8, 8),
    "lb2x16c128": (wkv.WKV_KERNEL_LOOKBACK, 2, 16, 128),
}
CASES = ["spikes", "falling", "rising", "edge", "tiny", "huge"]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no HIP device visible")
    wkv.load_library()


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def make(case, shape=None):
    """(w, u, k, v, dy, state_in or None) on the host, float32."""
    B, T, C = shape or (globals()["B"], globals()["T"], globals()["C"])
    seed = synth.seed_of(synth.TINY, 800 + CASES.index(case), 0)
    v = synth.normal((B, T, C), 1.0, seed)
    dy = synth.normal((B, T, C), 1.0, seed + 1)
    u = torch.linspace(-59.0, 59.0, C)
    w = torch.full((C,), 1e-3)
    k = torch.zeros(B, T, C)
    s_in = None
    t = torch.arange(T, dtype=torch.float32)
    if case == "spikes":
        k[:, 3::37, :] = 60.0
    elif case == "falling":
        k[:] = (40.0 - 80.0 * (t % 64) / 63.0)[None, :, None]
        w = torch.linspace(1e-3, 2.0, C)
    elif case == "rising":
        k[:] = (-40.0 + 80.0 * (t % 64) / 63.0)[None, :, None]
        w = torch.linspace(1e-3, 2.0, C)
    elif case == "edge":
        # U - W at -88..-84 and 84..88 (log2), decays slow and fast
        w = torch.tensor([1e-3, 1.0] * (C // 2))
        du = torch.linspace(-2.0, 2.0, C // 2).repeat_interleave(2) / LOG2E
        if C % 2:
            w, du = torch.cat([w, w[:1]]), torch.cat([du, du[:1]])
        u = torch.where(torch.arange(C) % 4 < 2, -86.0 / LOG2E + w + du, 86.0 / LOG2E + w + du)
        k[:, 7::50, :] = 30.0
    elif case == "tiny":
        s_in = torch.zeros(3, B, C)
        s_in[0] = 1e-30
        s_in[1] = 1e-30
        s_in[2] = 40.0
        k[:, 10::64, :] = -30.0
    elif case == "huge":
        w = torch.linspace(1e-3, 5.0, C)
        k[:, 4::41, :] = 200.0
        k[:, 25::41, :] = -200.0
    return w.float(), u.float(), k, v, dy, s_in


def oracle_fwd(oracle, w, u, k, v, s_in):
    return oracle.forward_scan(f64(w), f64(u), f64(k), f64(v), None if s_in is None else f64(s_in))


@pytest.mark.parametrize("shape", [None, RAGGED], ids=["2x256x64", "3x129x70"])
@pytest.mark.parametrize("plan", list(PLANS))
@pytest.mark.parametrize("case", CASES)
def test_forward_edges(oracle, case, plan, shape):
    w, u, k, v, _, s_in = make(case, shape)
    note(f"edges forward {case} {plan} {shape}")
    dev = torch.device("cuda")
    y, so = wkv.wkv_forward(w.to(dev), u.to(dev), k.to(dev), v.to(dev),
                            state_in=None if s_in is None else s_in.to(dev), state_out=True,
                            plan=PLANS[plan])
    torch.cuda.synchronize()
    yr, sr = oracle_fwd(oracle, w, u, k, v, s_in)
    assert_y_close(f64(y), yr, f"{case} {plan} y")
    assert_state_close(f64(so), sr, f"{case} {plan} state")


@pytest.mark.parametrize("plan", ["auto", "lb4x16", "lb8x16", "seg16x16"])
@pytest.mark.parametrize("case", CASES)
def test_gated_bf16_forward_edges(oracle, case, plan):
    """sigmoid(r) * wkv with k, v, r and y in bf16; the oracle reads the
    rounded inputs, and y may differ by one bf16 rounding more."""
    w, u, k, v, _, s_in = make(case)
    r = synth.normal((B, T, C), 2.0, synth.seed_of(synth.TINY, 898, 0))
    k16, v16, r16 = (x.to(torch.bfloat16) for x in (k, v, r))
    note(f"edges gated bf16 forward {case} {plan}")
    dev = torch.device("cuda")
    p = dict(PLANS, lb8x16=(wkv.WKV_KERNEL_LOOKBACK, 8, 16))[plan]
    y, so = wkv.wkv_forward_typed(w.to(dev), u.to(dev), k16.to(dev), v16.to(dev), r16.to(dev),
                                  state_in=None if s_in is None else s_in.to(dev),
                                  state_out=True, plan=p)
    torch.cuda.synchronize()
    yr, sr = oracle_fwd(oracle, w, u, k16.float(), v16.float(), s_in)
    g = oracle.gate(yr, f64(r16))
    yg = f64(y)
    assert np.all(np.isfinite(yg))
    h = 2.0 ** -8
    e = float(np.max(np.abs(yg - g) / (1e-5 + (1e-4 + h) * np.abs(g))))
    assert e <= 1.0, f"{case} {plan} gated bf16 y: {e:.3g}x the tolerance"
    assert_state_close(f64(so), sr, f"{case} {plan} state")


@pytest.mark.parametrize("case", CASES)
def test_step_edges(oracle, case):
    """The whole sequence as T single steps of one layer, state in place."""
    w, u, k, v, _, s_in = make(case)
    note(f"edges step {case}")
    dev = torch.device("cuda")
    st = torch.zeros(1, 3, B, C, device=dev)
    st[0, 2] = -1e38
    if s_in is not None:
        st[0] = s_in.to(dev)
    ys = []
    for t in range(T):
        y, _ = wkv.wkv_step(w[None].to(dev), u[None].to(dev), k[None, :, t].contiguous().to(dev),
                            v[None, :, t].contiguous().to(dev), st)
        ys.append(y[0])
    torch.cuda.synchronize()
    yr, sr = oracle_fwd(oracle, w, u, k, v, s_in)
    assert_y_close(f64(torch.stack(ys, 1)), yr, f"{case} step y")
    assert_state_close(f64(st[0]), sr, f"{case} step state")


@pytest.mark.parametrize("shape", [None, RAGGED], ids=["2x256x64", "3x129x70"])
@pytest.mark.parametrize("path", ["first_pass", "checkpoints", "gated"])
@pytest.mark.parametrize("case", CASES)
def test_backward_edges(oracle, case, path, shape):
    w, u, k, v, dy, s_in = make(case, shape)
    B, T, C = k.shape
    note(f"edges backward {case} {path} {shape}")
    dev = torch.device("cuda")
    wd, ud, kd, vd, dyd = (x.to(dev) for x in (w, u, k, v, dy))
    sid = None if s_in is None else s_in.to(dev)
    a = {n: f64(x) for n, x in (("w", w), ("u", u), ("k", k), ("v", v))}
    si = None if s_in is None else f64(s_in)
    _, s_end = oracle_fwd(oracle, w, u, k, v, s_in)
    s_out = s_end.astype(np.float32).astype(np.float64) if s_in is not None else None
    sod = None if s_out is None else torch.from_numpy(s_out.astype(np.float32)).to(dev)
    g = f64(dy)
    if path == "gated":
        r = synth.normal((B, T, C), 2.0, synth.seed_of(synth.TINY, 899, 0))
        got = wkv.wkv_backward_gated(wd, ud, kd, vd, r.to(dev), dyd, state_in=sid,
                                     state_out=sod)
        got = (got[0], got[1], got[3], got[4])
        yr, _ = oracle_fwd(oracle, w, u, k, v, s_in)
        g, _ = oracle.gate_backward(yr, f64(r), f64(dy))
    elif path == "checkpoints":
        _, _, ck = wkv.wkv_forward_checkpointed(wd, ud, kd, vd, state_in=sid)
        got = wkv.wkv_backward_checkpointed(wd, ud, kd, vd, dyd, ck, state_in=sid, state_out=sod)
    else:
        got = wkv.wkv_backward_typed(wd, ud, kd, vd, dyd, state_in=sid, state_out=sod)
    torch.cuda.synchronize()
    ref = oracle.backward_state(a["w"], a["u"], a["k"], a["v"], g, si, s_out, None)
    f = roundoff_floor(g, a["v"])
    assert_grad_close(f64(got[0]), ref[0], f"{case} {path} dk", f)
    assert_grad_close(f64(got[1]), ref[1], f"{case} {path} dv", f)
    assert_sums_close(oracle, f64(got[2]), f64(got[3]), ref[2], ref[3], a["w"], a["u"], a["k"],
                      a["v"], g, si, s_out, None, what=f"{case} {path}")


def test_step_long_run_does_not_drift(oracle):
    """4096 single steps with slow decay and rare +60 keys: the state handed
    from step to step keeps its log-weight (rounding o at every token moved
    it past the 1e-4 tolerance within 256 tokens of the "spikes" case)."""
    Bl, Tl, Cl = 1, 4096, 64
    w = torch.full((Cl,), 1e-3)
    u = torch.linspace(-20.0, 20.0, Cl)
    k = torch.zeros(Bl, Tl, Cl)
    k[:, 5::997, :] = 60.0
    v = synth.normal((Bl, Tl, Cl), 1.0, synth.seed_of(synth.TINY, 890, 0))
    note("edges step long run")
    dev = torch.device("cuda")
    st = torch.zeros(1, 3, Bl, Cl, device=dev)
    st[0, 2] = -1e38
    kd, vd = k.to(dev), v.to(dev)
    wl, ul = w[None].to(dev), u[None].to(dev)
    ys = torch.empty(Tl, Bl, Cl, device=dev)
    for t in range(Tl):
        wkv.wkv_step(wl, ul, kd[None, :, t].contiguous(), vd[None, :, t].contiguous(), st,
                     y=ys[t][None])
    torch.cuda.synchronize()
    yr, sr = oracle.forward_scan(f64(w), f64(u), f64(k), f64(v))
    assert_y_close(f64(ys).transpose(1, 0, 2), yr, "long-run step y")
    assert_state_close(f64(st[0]), sr, "long-run step state")

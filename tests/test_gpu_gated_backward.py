"""GPU parity of the gated backward (wkv_backward_gated) against the oracle.

The forward stored o = sigmoid(r) * wkv; dy is the gradient of o.  The oracle
side chains its own pieces: wkv from its forward scan, (g, dr) from its gate
backward (g = dy sigmoid(r) reaches wkv), and dk, dv, dw, du, d_state_in from
its carried-state backward driven by g.  Tolerances: tests/parity.py's
gradient bound for every output, dr included (dr = g wkv (1 - sigmoid(r)) with
wkv recomputed in float32, far inside 1e-3); 16-bit dk, dv, dr add the
format's relative half-unit.
"""
import os
import sys

import numpy as np
import pytest
import torch

from linear_recurrent_attention_amd import synth, wkv
from parity import G_FLOOR, G_RTOL, assert_grad_close, assert_sums_close, f64, roundoff_floor

pytestmark = pytest.mark.gpu

NTHREADS = max(1, min(16, os.cpu_count() or 1))
CK = wkv.WKV_CHECKPOINT_TOKENS
HALF_ULP = {torch.float16: 2.0 ** -11, torch.bfloat16: 2.0 ** -8}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no HIP device visible")
    wkv.load_library()


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(x):
    return None if x is None else torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()


def oracle_checkpoints(oracle, w, u, k, v, s_in=None):
    n = wkv.checkpoint_count(k.shape[1])
    out, s = [], s_in
    for i in range(n):
        _, s = oracle.forward_scan(w, u, k[:, i * CK:(i + 1) * CK], v[:, i * CK:(i + 1) * CK], s)
        out.append(s)
    return np.stack(out) if out else np.zeros((0,) + (3,) + k.shape[::2])


def reference(oracle, a, r, dy, s_in, s_out, g_out):
    y, _ = oracle.forward_scan(a["w"], a["u"], a["k"], a["v"], s_in, nthreads=NTHREADS)
    g, dr = oracle.gate_backward(y, r, dy)
    dk, dv, dw, du, dsi = oracle.backward_state(a["w"], a["u"], a["k"], a["v"], g, s_in, s_out,
                                                g_out)
    return dk, dv, dr, dw, du, dsi, g


def check(oracle, got, ref, a, what, dt=torch.float32, states=(None, None, None)):
    dk, dv, dr, dw, du, dsi, g = ref
    f = roundoff_floor(g, a["v"])
    fs = roundoff_floor(g, a["v"], summed=True)
    h = HALF_ULP.get(dt, 0.0)
    for name, x, r in (("dk", got[0], dk), ("dv", got[1], dv), ("dr", got[2], dr)):
        x = f64(x)
        assert np.all(np.isfinite(x)), f"{what} {name}: non-finite"
        if r.size == 0:
            continue
        rms = float(np.sqrt(np.mean(r * r)))
        e = float(np.max(np.abs(x - r) / ((G_RTOL + h) * np.abs(r) + G_FLOOR * rms + f + 1e-300)))
        assert e <= 1.0, f"{what} {name}: {e:.3g}x the tolerance"
    assert_sums_close(oracle, f64(got[3]), f64(got[4]), dw, du, a["w"], a["u"], a["k"], a["v"], g,
                      *states, what=what)
    if got[5] is not None:
        for pl in range(3):
            assert_grad_close(f64(got[5])[pl], dsi[pl], f"{what} d_state_in[{pl}]", fs)


def reachable_state(oracle, B, C, index):
    p = synth.make(synth.TINY, index=index, B=B, T=11, C=C)
    _, s = oracle.forward_scan(*(f64(p[n]) for n in ("w", "u", "k", "v")))
    return s.astype(np.float32).astype(np.float64)


SHAPES = [(1, 1, 5), (2, 128, 64), (2, 129, 64), (2, 300, 100), (1, 513, 130), (2, 1024, 96)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("recipe", [synth.GPT, synth.STABILITY])
@pytest.mark.parametrize("mode", ["first_pass", "checkpoints", "states"])
def test_gated_backward_matches_oracle(oracle, shape, recipe, mode):
    B, T, C = shape
    d = synth.make(recipe, index=110, B=B, T=T, C=C, with_dy=True)
    r = synth.receptance(recipe, 110, (B, T, C))
    a = {n: f64(d[n]) for n in ("w", "u", "k", "v")}
    s_in = s_out = g_out = ck = None
    if mode == "states":
        s_in = reachable_state(oracle, B, C, 111)
        _, s_out = oracle.forward_scan(a["w"], a["u"], a["k"], a["v"], s_in)
        s_out = s_out.astype(np.float32).astype(np.float64)
        g_out = synth.normal((3, B, C), 1.0, synth.seed_of(synth.GPT, 9700, 0)).double().numpy()
    if mode != "first_pass":
        ck = oracle_checkpoints(oracle, a["w"], a["u"], a["k"], a["v"], s_in)
        ck = ck.astype(np.float32).astype(np.float64)
    note(f"gated bwd B={B} T={T} C={C} recipe={recipe} mode={mode}")
    dev = torch.device("cuda")
    got = wkv.wkv_backward_gated(*(d[n].to(dev) for n in ("w", "u", "k", "v")), r.to(dev),
                                 d["dy"].to(dev), checkpoints=to_dev(ck), state_in=to_dev(s_in),
                                 state_out=to_dev(s_out), d_state_out=to_dev(g_out),
                                 d_state_in=True if mode == "states" else None)
    torch.cuda.synchronize()
    ref = reference(oracle, a, f64(r), f64(d["dy"]), s_in, s_out, g_out)
    check(oracle, got, ref, a, f"gated {mode}", states=(s_in, s_out, g_out))


@pytest.mark.parametrize("dt", [torch.float16, torch.bfloat16], ids=["f16", "bf16"])
@pytest.mark.parametrize("shape", [(2, 300, 100), (1, 1024, 64)],
                         ids=lambda s: "x".join(map(str, s)))
def test_gated_training_path_16bit(oracle, dt, shape):
    """Gated forward with checkpoints, then the gated backward from them, in a
    16-bit format: gradients against the oracle on the rounded inputs."""
    B, T, C = shape
    d = synth.make(synth.STABILITY, index=112, B=B, T=T, C=C, with_dy=True)
    d = {n: (t.to(dt) if n in ("k", "v", "dy") else t) for n, t in d.items()}
    r = synth.receptance(synth.STABILITY, 112, (B, T, C)).to(dt)
    dev = torch.device("cuda")
    w, u, k, v, dy, rd = (x.to(dev) for x in (d["w"], d["u"], d["k"], d["v"], d["dy"], r))
    note(f"gated train {dt} B={B} T={T} C={C}")
    _, _, ck = wkv.wkv_forward_checkpointed(w, u, k, v, r=rd)
    got = wkv.wkv_backward_gated(w, u, k, v, rd, dy, checkpoints=ck)
    torch.cuda.synchronize()
    assert got[2].dtype == dt
    a = {n: f64(d[n]) for n in ("w", "u", "k", "v")}
    ref = reference(oracle, a, f64(r), f64(d["dy"]), None, None, None)
    check(oracle, got, ref, a, f"gated {dt}", dt)


@pytest.mark.parametrize("rv", [800.0, -800.0], ids=["open", "closed"])
def test_gated_backward_saturated_gate(oracle, rv):
    """r = +800 opens the gate exactly (the ungated backward; dr = 0) and
    r = -800 closes it (every gradient exactly zero)."""
    B, T, C = 2, 300, 96
    d = synth.make(synth.STABILITY, index=113, B=B, T=T, C=C, with_dy=True)
    dev = torch.device("cuda")
    w, u, k, v, dy = (d[n].to(dev) for n in ("w", "u", "k", "v", "dy"))
    r = torch.full_like(k, rv)
    got = wkv.wkv_backward_gated(w, u, k, v, r, dy)
    torch.cuda.synchronize()
    assert torch.all(got[2] == 0)
    if rv < 0:
        for x in got[:5]:
            assert torch.all(x == 0)
    a = {n: f64(d[n]) for n in ("w", "u", "k", "v")}
    check(oracle, got, reference(oracle, a, f64(r), f64(d["dy"]), None, None, None), a,
          f"gate {rv}")


def test_gated_stability_training_path_full_size_sampled(oracle):
    """B=8 T=4096 C=2048, gated: the GPU forward's checkpoints feed the GPU
    gated backward; every gradient of 8 sampled channels (all sequences)
    against the oracle."""
    B, T, C = 8, 4096, 2048
    d = synth.make(synth.STABILITY, index=114, with_dy=True)
    r = synth.receptance(synth.STABILITY, 114, (B, T, C))
    cs = np.array([0, 1, 63, 64, 777, 1500, 2046, 2047])
    dev = torch.device("cuda")
    w, u, k, v, dy, rd = (x.to(dev) for x in (d["w"], d["u"], d["k"], d["v"], d["dy"], r))
    note("gated train stability full size")
    _, _, ck = wkv.wkv_forward_checkpointed(w, u, k, v, r=rd)
    got = wkv.wkv_backward_gated(w, u, k, v, rd, dy, checkpoints=ck)
    torch.cuda.synchronize()
    a = {n: (f64(d[n])[:, :, cs] if n in ("k", "v") else f64(d[n])[cs])
         for n in ("w", "u", "k", "v")}
    ref = reference(oracle, a, f64(r)[:, :, cs], f64(d["dy"])[:, :, cs], None, None, None)
    sub = (got[0][:, :, cs], got[1][:, :, cs], got[2][:, :, cs], got[3][cs], got[4][cs], None)
    check(oracle, sub, ref, a, "gated stability")

"""GPU parity of wkv_backward_state (backward of a chunk with carried states)
against the oracle's O(T^2) derivative.

The state a chunk starts from and the state it hands on are the oracle's own
(float32-rounded), and the upstream state gradient is seeded noise, so no
input of the oracle comes from the HIP path.  Tolerances: tests/parity.py
(gradients, per tensor), applied to d_state_in plane by plane as well.
"""
import os
import sys

import numpy as np
import pytest
import torch

from linear_recurrent_attention_amd import synth, wkv
from parity import (assert_chained_sums_close, assert_grad_close, assert_sums_close, f64,
                    roundoff_floor)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no HIP device visible")
    wkv.load_library()


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def oracle_state(oracle, w, u, k, v, s_in=None):
    """The oracle's state after (k, v), rounded to float32."""
    _, s = oracle.forward_scan(w, u, k, v, s_in)
    return s.astype(np.float32).astype(np.float64)


def upstream(B, C, seed):
    return synth.normal((3, B, C), 1.0, synth.seed_of(synth.GPT, 9000 + seed, 0)).double().numpy()


def run_gpu(d, s_in, s_out, g_out, want_ds=True):
    dev = torch.device("cuda")
    t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)
    out = wkv.wkv_backward_state(*(d[n].to(dev) for n in ("w", "u", "k", "v", "dy")),
                                 state_in=t(s_in), state_out=t(s_out), d_state_out=t(g_out),
                                 d_state_in=True if want_ds else None)
    torch.cuda.synchronize()
    return out


def check(oracle, d, s_in, s_out, g_out, got, what):
    a = {n: f64(d[n]) for n in ("w", "u", "k", "v", "dy")}
    ref = oracle.backward_state(a["w"], a["u"], a["k"], a["v"], a["dy"], s_in, s_out, g_out)
    f = roundoff_floor(a["dy"], a["v"])
    fs = roundoff_floor(a["dy"], a["v"], summed=True)
    for name, x, r in zip(("dk", "dv"), got[:2], ref[:2]):
        assert_grad_close(f64(x), r, f"{what} {name}", f)
    assert_sums_close(oracle, f64(got[2]), f64(got[3]), ref[2], ref[3], a["w"], a["u"], a["k"],
                      a["v"], a["dy"], s_in, s_out, g_out, what=what)
    if got[4] is not None:
        for p, name in enumerate(("d_a0", "d_b0", "d_o0")):
            assert_grad_close(f64(got[4])[p], ref[4][p], f"{what} {name}", fs)


SHAPES = [(1, 1, 5), (2, 300, 100), (3, 17, 64), (1, 513, 130), (2, 129, 64), (1, 640, 33),
          (2, 512, 96)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("recipe", [synth.GPT, synth.STABILITY])
@pytest.mark.parametrize("with_in,with_out", [(True, True), (True, False), (False, True)])
def test_backward_state_matches_oracle(oracle, shape, recipe, with_in, with_out):
    B, T, C = shape
    d = synth.make(recipe, index=70, B=B, T=T, C=C, with_dy=True)
    a = {n: f64(d[n]) for n in ("w", "u", "k", "v")}
    s_in = None
    if with_in:
        p = synth.make(synth.TINY, index=71, B=B, T=11, C=C)
        s_in = oracle_state(oracle, a["w"], a["u"], f64(p["k"]), f64(p["v"]))
    s_out = oracle_state(oracle, a["w"], a["u"], a["k"], a["v"], s_in) if with_out else None
    g_out = upstream(B, C, 1) if with_out else None
    note(f"bwd state B={B} T={T} C={C} recipe={recipe} in={with_in} out={with_out}")
    got = run_gpu(d, s_in, s_out, g_out)
    check(oracle, d, s_in, s_out, g_out, got, "bwd_state")


def test_backward_state_without_states_is_the_backward(oracle):
    d = synth.make(synth.STABILITY, index=72, B=2, T=300, C=96, with_dy=True)
    dev = torch.device("cuda")
    args = [d[n].to(dev) for n in ("w", "u", "k", "v", "dy")]
    a = wkv.wkv_backward(*args)
    b = wkv.wkv_backward_state(*args)
    torch.cuda.synchronize()
    for x, y in zip(a, b[:4]):
        assert torch.equal(x, y)


@pytest.mark.parametrize("cuts", [[300], [1, 127, 172], [128, 128, 44], [50, 250]])
def test_backward_chains_over_chunks(oracle, cuts):
    """GPU backward over chunks, last to first, each chunk's d_state_in fed to
    the previous chunk as d_state_out (updated in place), against the oracle's
    backward of one call over the whole sequence."""
    B, T, C = 2, sum(cuts), 96
    d = synth.make(synth.GPT, index=73, B=B, T=T, C=C, with_dy=True)
    a = {n: f64(d[n]) for n in ("w", "u", "k", "v", "dy")}
    p = synth.make(synth.TINY, index=74, B=B, T=9, C=C)
    s0 = oracle_state(oracle, a["w"], a["u"], f64(p["k"]), f64(p["v"]))
    # the states the chunks start from and hand on (the oracle's, float32)
    bounds = np.cumsum([0] + cuts)
    states = [s0]
    for i in range(len(cuts)):
        lo, hi = bounds[i], bounds[i + 1]
        states.append(oracle_state(oracle, a["w"], a["u"], a["k"][:, lo:hi], a["v"][:, lo:hi],
                                   states[-1]))
    g_end = upstream(B, C, 2)
    dev = torch.device("cuda")
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dev)
    g = t(g_end)
    dks, dvs, dw, du = [], [], 0.0, 0.0
    for i in reversed(range(len(cuts))):
        lo, hi = bounds[i], bounds[i + 1]
        chunk = [d[n][:, lo:hi].contiguous().to(dev) if n in ("k", "v", "dy") else d[n].to(dev)
                 for n in ("w", "u", "k", "v", "dy")]
        dk, dv, dwi, dui, _ = wkv.wkv_backward_state(*chunk, state_in=t(states[i]),
                                                     state_out=t(states[i + 1]),
                                                     d_state_out=g, d_state_in=g)
        dks.insert(0, dk)
        dvs.insert(0, dv)
        dw = dw + f64(dwi)
        du = du + f64(dui)
    torch.cuda.synchronize()
    note(f"bwd chain cuts={cuts}")
    ref = oracle.backward_state(a["w"], a["u"], a["k"], a["v"], a["dy"], s0, states[-1], g_end)
    f = roundoff_floor(a["dy"], a["v"])
    fs = roundoff_floor(a["dy"], a["v"], summed=True)
    assert_grad_close(f64(torch.cat(dks, dim=1)), ref[0], "chain dk", f)
    assert_grad_close(f64(torch.cat(dvs, dim=1)), ref[1], "chain dv", f)
    # dw, du summed over the chunks in float64
    assert_chained_sums_close(oracle, dw, du, ref[2], ref[3], a["w"], a["u"], a["k"], a["v"],
                              a["dy"], cuts, s0, g_end)
    for pl in range(3):
        assert_grad_close(f64(g)[pl], ref[4][pl], f"chain d_state_in[{pl}]", fs)


def test_zero_length_chunk_passes_the_gradient_through(oracle):
    B, C = 2, 40
    dev = torch.device("cuda")
    d = synth.make(synth.GPT, index=75, B=B, T=0, C=C, with_dy=True)
    p = synth.make(synth.TINY, index=76, B=B, T=5, C=C)
    s = oracle_state(oracle, f64(d["w"]), f64(d["u"]), f64(p["k"]), f64(p["v"]))
    g = upstream(B, C, 3)
    got = run_gpu(d, s, s, g)
    ref = oracle.backward_state(*(f64(d[n]) for n in ("w", "u", "k", "v", "dy")), s, s, g)
    assert torch.all(got[2] == 0) and torch.all(got[3] == 0)
    np.testing.assert_allclose(f64(got[4]), ref[4], rtol=1e-6, atol=1e-30)
    # fresh sequence: nothing flows into an empty state
    got = run_gpu(d, None, s, g)
    assert torch.all(got[4] == 0)


def test_stability_workload_full_size_sampled(oracle):
    """B=8 T=4096 C=2048 with a carried state and an upstream gradient:
    every output of 8 sampled channels (all sequences) against the oracle."""
    B, T, C = 8, 4096, 2048
    d = synth.make(synth.STABILITY, index=77, with_dy=True)
    p = synth.make(synth.TINY, index=78, B=B, T=16, C=C)
    a = {n: f64(d[n]) for n in ("w", "u")}
    s_in = oracle_state(oracle, a["w"], a["u"], f64(p["k"]), f64(p["v"]))
    cs = np.array([0, 1, 63, 64, 777, 1500, 2046, 2047])
    sub = {n: (f64(d[n])[:, :, cs] if n in ("k", "v", "dy") else f64(d[n])[cs])
           for n in ("w", "u", "k", "v", "dy")}
    # the handed-on state of the sampled channels, from the oracle
    s_out_sub = oracle_state(oracle, sub["w"], sub["u"], sub["k"], sub["v"], s_in[:, :, cs])
    s_out = np.zeros((3, B, C))
    s_out[:, :, cs] = s_out_sub
    s_out[1][:, np.setdiff1d(np.arange(C), cs)] = 1.0    # unsampled lanes: no upstream gradient
    g_out = np.zeros((3, B, C))
    g_out[:, :, cs] = upstream(B, len(cs), 4)
    note("bwd state stability full size, sampled channels")
    got = run_gpu(d, s_in, s_out, g_out)
    ref = oracle.backward_state(sub["w"], sub["u"], sub["k"], sub["v"], sub["dy"],
                                s_in[:, :, cs], s_out_sub, g_out[:, :, cs])
    f = roundoff_floor(sub["dy"], sub["v"])
    fs = roundoff_floor(sub["dy"], sub["v"], summed=True)
    assert_grad_close(f64(got[0])[:, :, cs], ref[0], "dk", f)
    assert_grad_close(f64(got[1])[:, :, cs], ref[1], "dv", f)
    assert_sums_close(oracle, f64(got[2])[cs], f64(got[3])[cs], ref[2], ref[3], sub["w"],
                      sub["u"], sub["k"], sub["v"], sub["dy"], s_in[:, :, cs], s_out_sub,
                      g_out[:, :, cs])
    for pl in range(3):
        assert_grad_close(f64(got[4])[pl][:, cs], ref[4][pl], f"d_state_in[{pl}]", fs)



# ---------------------------------------------------- 16-bit activations ---
# k, v, dy in fp16 / bf16 (widened exactly), dk and dv rounded once to the
# format: their bound gains the relative half-unit h of the format's last
# place (2^-11 fp16, 2^-8 bf16); dw, du and the state gradient are float32.

HALF_ULP = {torch.float16: 2.0 ** -11, torch.bfloat16: 2.0 ** -8}


@pytest.mark.parametrize("dt", [torch.float16, torch.bfloat16], ids=["f16", "bf16"])
@pytest.mark.parametrize("shape", [(1, 1, 5), (2, 300, 100), (1, 513, 130), (2, 129, 64),
                                   (2, 512, 96)],
                         ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("states", [False, True])
def test_typed_backward_matches_oracle(oracle, dt, shape, states):
    from parity import G_FLOOR, G_RTOL
    B, T, C = shape
    d = synth.make(synth.STABILITY, index=80, B=B, T=T, C=C, with_dy=True)
    d = {n: (t.to(dt) if n in ("k", "v", "dy") else t) for n, t in d.items()}
    a = {n: f64(d[n]) for n in ("w", "u", "k", "v", "dy")}
    s_in = s_out = g_out = None
    if states:
        p = synth.make(synth.TINY, index=81, B=B, T=11, C=C)
        s_in = oracle_state(oracle, a["w"], a["u"], f64(p["k"]), f64(p["v"]))
        s_out = oracle_state(oracle, a["w"], a["u"], a["k"], a["v"], s_in)
        g_out = upstream(B, C, 5)
    dev = torch.device("cuda")
    t = lambda x: None if x is None else torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dev)
    note(f"typed bwd {dt} B={B} T={T} C={C} states={states}")
    got = wkv.wkv_backward_typed(*(d[n].to(dev) for n in ("w", "u", "k", "v", "dy")),
                                 state_in=t(s_in), state_out=t(s_out), d_state_out=t(g_out),
                                 d_state_in=True)
    torch.cuda.synchronize()
    assert got[0].dtype == dt and got[1].dtype == dt
    ref = oracle.backward_state(a["w"], a["u"], a["k"], a["v"], a["dy"], s_in, s_out, g_out)
    f = roundoff_floor(a["dy"], a["v"])
    fs = roundoff_floor(a["dy"], a["v"], summed=True)
    for name, x, r in (("dk", got[0], ref[0]), ("dv", got[1], ref[1])):
        x = f64(x)
        assert np.all(np.isfinite(x)), name
        rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
        bound = (G_RTOL + HALF_ULP[dt]) * np.abs(r) + G_FLOOR * rms + f + 1e-300
        e = float(np.max(np.abs(x - r) / bound)) if r.size else 0.0
        assert e <= 1.0, f"{name}: {e:.3g}x the tolerance"
    assert_sums_close(oracle, f64(got[2]), f64(got[3]), ref[2], ref[3], a["w"], a["u"], a["k"],
                      a["v"], a["dy"], s_in, s_out, g_out)
    for pl in range(3):
        assert_grad_close(f64(got[4])[pl], ref[4][pl], f"d_state_in[{pl}]", fs)

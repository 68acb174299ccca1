"""GPU parity of wkv_backward (dk, dv, dw, du) against the oracle's analytic
backward (O(T) reverse scan; brute force on the smallest case)."""
import os
import sys

import numpy as np
import pytest
import torch

from linear_recurrent_attention_amd import synth, wkv
from parity import assert_grad_close, assert_sums_close, f64, roundoff_floor

pytestmark = pytest.mark.gpu

NTHREADS = max(1, min(16, os.cpu_count() or 1))


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no HIP device visible")
    wkv.load_library()


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def gpu_grads(d):
    dev = torch.device("cuda")
    w, u, k, v, dy = (d[n].to(dev) for n in ("w", "u", "k", "v", "dy"))
    out = wkv.wkv_backward(w, u, k, v, dy)
    torch.cuda.synchronize()
    return [f64(t) for t in out]


def check(g, r, d, oracle, what=""):
    """dk, dv per tensor; dw, du per channel against the round-off scale of
    their terms."""
    dy, v = f64(d["dy"]), f64(d["v"])
    for name, x, ref in zip(("dk", "dv"), g[:2], r[:2]):
        assert_grad_close(x, ref, f"{what} {name}", roundoff_floor(dy, v))
    assert_sums_close(oracle, g[2], g[3], r[2], r[3],
                      *(f64(d[n]) for n in ("w", "u", "k", "v", "dy")), what=what)


def test_tiny_backward_matches_brute_force(oracle):
    d = synth.make(synth.STABILITY, index=1, B=1, T=64, C=32, with_dy=True)
    note("backward tiny B=1 T=64 C=32")
    g = gpu_grads(d)
    r = oracle.backward_brute(*(f64(d[n]) for n in ("w", "u", "k", "v", "dy")))
    check(g, r, d, oracle)


SHAPES = [(1, 1, 3), (2, 127, 70), (1, 128, 64), (3, 129, 65), (2, 1000, 130), (1, 2100, 64)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("recipe", [synth.GPT, synth.STABILITY])
def test_ragged_backward_matches_oracle(oracle, shape, recipe):
    B, T, C = shape
    d = synth.make(recipe, index=2, B=B, T=T, C=C, with_dy=True)
    note(f"backward ragged B={B} T={T} C={C} recipe={recipe}")
    g = gpu_grads(d)
    r = oracle.backward_scan(*(f64(d[n]) for n in ("w", "u", "k", "v", "dy")), nthreads=NTHREADS)
    check(g, r, d, oracle)


WHOLE_TILES = [(2, 512, 96), (1, 1024, 130), (3, 256, 64)]


@pytest.mark.parametrize("shape", WHOLE_TILES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("recipe", [synth.GPT, synth.STABILITY])
def test_whole_tile_backward_matches_oracle(oracle, shape, recipe):
    """Sequences of whole 128-token tiles, where each tile's segments are
    recomputed and swept in one frame: the plain backward, the backward from
    the GPU forward's checkpoints and the gated backward."""
    B, T, C = shape
    d = synth.make(recipe, index=12, B=B, T=T, C=C, with_dy=True)
    note(f"backward whole tiles B={B} T={T} C={C} recipe={recipe}")
    a = [f64(d[n]) for n in ("w", "u", "k", "v")]
    ref = oracle.backward_scan(*a, f64(d["dy"]), nthreads=NTHREADS)
    check(gpu_grads(d), ref, d, oracle, "plain")
    dev = torch.device("cuda")
    w, u, k, v, dy = (d[n].to(dev) for n in ("w", "u", "k", "v", "dy"))
    _, _, ck = wkv.wkv_forward_checkpointed(w, u, k, v)
    g = [f64(t) for t in wkv.wkv_backward_checkpointed(w, u, k, v, dy, ck)[:4]]
    torch.cuda.synchronize()
    check(g, ref, d, oracle, "from checkpoints")
    r = synth.receptance(recipe, 12, (B, T, C))
    dk, dv, dr, dw, du, _ = wkv.wkv_backward_gated(w, u, k, v, r.to(dev), dy, checkpoints=ck)
    torch.cuda.synchronize()
    y, _ = oracle.forward_scan(*a)
    gg, dr_ref = oracle.gate_backward(y, f64(r), f64(d["dy"]))
    gref = oracle.backward_scan(*a, gg, nthreads=NTHREADS)
    v64 = f64(d["v"])
    for name, x, rr in (("dk", dk, gref[0]), ("dv", dv, gref[1]), ("dr", dr, dr_ref)):
        assert_grad_close(f64(x), rr, f"gated {name}", roundoff_floor(gg, v64))
    assert_sums_close(oracle, f64(dw), f64(du), gref[2], gref[3], *a, gg, what="gated")


@pytest.mark.parametrize("T", [300, 640])
@pytest.mark.parametrize("hi,lo", [(75.0, -70.0), (88.0, -85.0)], ids=["75", "88"])
def test_extreme_bonus_backward(oracle, hi, lo, T):
    """Channels where the bonus dominates every output (each earlier token's
    weight near e^{-u}, down to float's smallest normal numbers at u = 88) or
    vanishes (own weight near e^{u}): dw and du of those channels are tiny and
    are held, per channel, to the round-off of their own terms."""
    d = synth.make(synth.TINY, index=3, B=2, T=T, C=64, with_dy=True)
    d["u"][::3] = hi
    d["u"][1::5] = lo
    note(f"backward extreme bonus {hi} {lo} T={T}")
    g = gpu_grads(d)
    r = oracle.backward_scan(*(f64(d[n]) for n in ("w", "u", "k", "v", "dy")))
    check(g, r, d, oracle)


@pytest.mark.parametrize("T", [600, 640])
@pytest.mark.parametrize("recipe", [synth.GPT, synth.STABILITY])
def test_extreme_decay_backward(oracle, recipe, T):
    """Per-channel decay rates spread geometrically from 1e-6 (nothing decays
    over the sequence) to 60 (the past vanishes within two tokens): the plain
    backward, the backward from the GPU forward's checkpoints and the gated
    backward, against the oracle (T = 640: whole tiles, where the groups of
    moderate rates run in one frame per segment and the others token by
    token)."""
    B, C = 2, 96
    d = synth.make(recipe, index=8, B=B, T=T, C=C, with_dy=True)
    d["w"] = torch.from_numpy(np.geomspace(1e-6, 60.0, C).astype(np.float32))
    note(f"backward extreme decay recipe={recipe} T={T}")
    check(gpu_grads(d), oracle.backward_scan(*(f64(d[n]) for n in ("w", "u", "k", "v", "dy"))), d,
          oracle, "plain")
    dev = torch.device("cuda")
    w, u, k, v, dy = (d[n].to(dev) for n in ("w", "u", "k", "v", "dy"))
    _, _, ck = wkv.wkv_forward_checkpointed(w, u, k, v)
    g = [f64(t) for t in wkv.wkv_backward_checkpointed(w, u, k, v, dy, ck)[:4]]
    torch.cuda.synchronize()
    check(g, oracle.backward_scan(*(f64(d[n]) for n in ("w", "u", "k", "v", "dy"))), d, oracle,
          "from checkpoints")
    # gated: the recurrence receives g = dy sigmoid(r)
    r = synth.receptance(recipe, 8, (B, T, C))
    dk, dv, dr, dw, du, _ = wkv.wkv_backward_gated(w, u, k, v, r.to(dev), dy, checkpoints=ck)
    torch.cuda.synchronize()
    a = [f64(d[n]) for n in ("w", "u", "k", "v")]
    y, _ = oracle.forward_scan(*a)
    gg, dr_ref = oracle.gate_backward(y, f64(r), f64(d["dy"]))
    ref = oracle.backward_scan(*a, gg)
    v64 = f64(d["v"])
    for name, x, rr in (("dk", dk, ref[0]), ("dv", dv, ref[1]), ("dr", dr, dr_ref)):
        assert_grad_close(f64(x), rr, f"gated {name}", roundoff_floor(gg, v64))
    assert_sums_close(oracle, f64(dw), f64(du), ref[2], ref[3], *a, gg, what="gated")


def test_empty_backward():
    dev = torch.device("cuda")
    C = 33
    w = torch.ones(C, device=dev)
    z = torch.empty((2, 0, C), device=dev)
    note("backward T=0")
    dk, dv, dw, du = wkv.wkv_backward(w, w, z, z, z)
    torch.cuda.synchronize()
    assert torch.all(dw == 0) and torch.all(du == 0)


def test_backward_is_deterministic():
    dev = torch.device("cuda")
    d = synth.make(synth.STABILITY, index=4, B=4, T=700, C=192, with_dy=True, device=dev)
    note("backward determinism")
    a = wkv.wkv_backward(d["w"], d["u"], d["k"], d["v"], d["dy"])
    b = wkv.wkv_backward(d["w"], d["u"], d["k"], d["v"], d["dy"])
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_stability_workload_backward_full_size(oracle):
    """B=8 T=4096 C=2048, k ~ N(0,8) with 0.1% of entries at +-60, decay in
    U(-8,3), u ~ N(0,2), v, dy ~ N(0,1): every gradient element."""
    dev = torch.device("cuda")
    d = synth.make(synth.STABILITY, index=0, device=dev, with_dy=True)
    note("backward full B=8 T=4096 C=2048")
    out = wkv.wkv_backward(d["w"], d["u"], d["k"], d["v"], d["dy"])
    torch.cuda.synchronize()
    g = [f64(t) for t in out]
    r = oracle.backward_scan(*(f64(d[n]) for n in ("w", "u", "k", "v", "dy")), nthreads=NTHREADS)
    check(g, r, d, oracle)

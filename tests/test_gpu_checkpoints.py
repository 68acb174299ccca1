"""GPU parity of the checkpointed forward and the backward that starts from its
checkpoints, against the oracle.

Checkpoint i is the state after the first 128 (i + 1) tokens: the oracle's
state_out over that prefix, which the oracle reaches here by running its scan
over 128-token chunks, carrying the state (RNN mode over chunks equals one
pass; pinned in test_oracle.py).  Checkpoints are compared in canonical form
with the forward's state tolerance; y keeps its own tolerance, and with the
lane and segmented kernels y and state_out must be bitwise those of
wkv_forward_typed.  Gradients: tests/parity.py.  The backward is fed either
the oracle's float32-rounded checkpoints or the ones the GPU forward wrote
(the training path); the expected gradients always come from the oracle on
the seeded inputs.
"""
import os
import sys

import numpy as np
import pytest
import torch

from linear_recurrent_attention_amd import synth, wkv
from parity import (G_FLOOR, G_RTOL, assert_grad_close, assert_state_close, assert_sums_close,
                    assert_y_close, f64, roundoff_floor)

pytestmark = pytest.mark.gpu

NTHREADS = max(1, min(16, os.cpu_count() or 1))
CK = wkv.WKV_CHECKPOINT_TOKENS
HALF_ULP = {torch.float16: 2.0 ** -11, torch.bfloat16: 2.0 ** -8}

PLANS = {
    "auto": None,
    "lane": (wkv.WKV_KERNEL_LANE, 0, 0),
    "seg16x16": (wkv.WKV_KERNEL_SEGMENTED, 16, 16),
    "seg32x8c16": (wkv.WKV_KERNEL_SEGMENTED, 32, 8, 16),
    "lb4x16": (wkv.WKV_KERNEL_LOOKBACK, 4, 16),
    "lb4x32": (wkv.WKV_KERNEL_LOOKBACK, 4, 32),
    "lb8x32": (wkv.WKV_KERNEL_LOOKBACK, 8, 32),
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


def oracle_checkpoints(oracle, w, u, k, v, s_in=None):
    """[count][3][B][C]: the oracle's state after every 128-token prefix that
    ends inside the sequence, and its state after the whole sequence."""
    B, T, C = k.shape
    n = wkv.checkpoint_count(T)
    out, s = [], s_in
    for i in range(n):
        _, s = oracle.forward_scan(w, u, k[:, i * CK:(i + 1) * CK], v[:, i * CK:(i + 1) * CK], s,
                                   nthreads=NTHREADS)
        out.append(s)
    _, s_end = oracle.forward_scan(w, u, k[:, n * CK:], v[:, n * CK:], s, nthreads=NTHREADS)
    return (np.stack(out) if out else np.zeros((0, 3, B, C))), s_end


def reachable_state(oracle, B, C, index):
    p = synth.make(synth.TINY, index=index, B=B, T=11, C=C)
    _, s = oracle.forward_scan(*(f64(p[n]) for n in ("w", "u", "k", "v")))
    # (w and u of this tiny draw differ from the sequence's: any state is a
    # valid start, and this one has finite, mixed exponents)
    return s.astype(np.float32).astype(np.float64)


def to_dev(x, dtype=torch.float32):
    if x is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(x, np.float64)).to(dtype).to("cuda")


def assert_ckpts_close(got, ref, what):
    assert tuple(got.shape) == ref.shape, (what, tuple(got.shape), ref.shape)
    for i in range(ref.shape[0]):
        assert_state_close(f64(got[i]), ref[i], f"{what} checkpoint {i}")


SHAPES = [(1, 1, 5), (2, 128, 64), (2, 129, 64), (2, 300, 100), (1, 513, 130), (3, 1024, 64),
          (1, 2049, 33)]


@pytest.mark.parametrize("plan", list(PLANS))
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("with_in", [False, True])
def test_forward_checkpoints_match_oracle(oracle, plan, shape, with_in):
    B, T, C = shape
    d = synth.make(synth.GPT, index=90, B=B, T=T, C=C)
    a = {n: f64(d[n]) for n in ("w", "u", "k", "v")}
    s_in = reachable_state(oracle, B, C, 91) if with_in else None
    note(f"fwd ckpt plan={plan} B={B} T={T} C={C} state_in={with_in}")
    dev = torch.device("cuda")
    w, u, k, v = (d[n].to(dev) for n in ("w", "u", "k", "v"))
    y, so, ck = wkv.wkv_forward_checkpointed(w, u, k, v, state_in=to_dev(s_in), state_out=True,
                                             plan=PLANS[plan])
    torch.cuda.synchronize()
    ref_ck, ref_end = oracle_checkpoints(oracle, a["w"], a["u"], a["k"], a["v"], s_in)
    assert_ckpts_close(ck, ref_ck, plan)
    assert_state_close(f64(so), ref_end)
    yr, _ = oracle.forward_scan(a["w"], a["u"], a["k"], a["v"], s_in, nthreads=NTHREADS)
    assert_y_close(f64(y), yr)
    if plan in ("lane", "seg16x16", "seg32x8c16"):
        # the same kernel without checkpoints: identical bits
        y2, so2 = wkv.wkv_forward_typed(w, u, k, v, state_in=to_dev(s_in), state_out=True,
                                        plan=PLANS[plan])
        torch.cuda.synchronize()
        assert torch.equal(y, y2) and torch.equal(so, so2)


@pytest.mark.parametrize("dt", [torch.float16, torch.bfloat16], ids=["f16", "bf16"])
@pytest.mark.parametrize("plan", ["auto", "lane", "seg16x16", "lb4x16", "lb4x32"])
def test_forward_checkpoints_16bit(oracle, dt, plan):
    B, T, C = 2, 700, 96
    d = synth.make(synth.STABILITY, index=92, B=B, T=T, C=C)
    d = {n: (t.to(dt) if n in ("k", "v") else t) for n, t in d.items()}
    a = {n: f64(d[n]) for n in ("w", "u", "k", "v")}
    # gated, except on the 4x32 look-back variant, which has no gated build
    gated = plan != "lb4x32"
    r = synth.receptance(synth.STABILITY, 92, (B, T, C)).to(dt) if gated else None
    note(f"fwd ckpt {dt} plan={plan} gated={gated}")
    dev = torch.device("cuda")
    y, so, ck = wkv.wkv_forward_checkpointed(*(d[n].to(dev) for n in ("w", "u", "k", "v")),
                                             r=r.to(dev) if gated else None, state_out=True,
                                             plan=PLANS[plan])
    torch.cuda.synchronize()
    ref_ck, ref_end = oracle_checkpoints(oracle, a["w"], a["u"], a["k"], a["v"])
    assert_ckpts_close(ck, ref_ck, plan)
    assert_state_close(f64(so), ref_end)
    yr, _ = oracle.forward_scan(a["w"], a["u"], a["k"], a["v"], nthreads=NTHREADS)
    if gated:
        yr = oracle.gate(yr, f64(r))
    e = float(np.max(np.abs(f64(y) - yr) / (1e-5 + (1e-4 + HALF_ULP[dt]) * np.abs(yr))))
    assert e <= 1.0, f"y: {e:.3g}x the tolerance"


def test_forward_checkpoints_gpt_workload_full_size(oracle):
    """B=8 T=1024 C=2048 (one layer of the GPT workload): all 7 checkpoints,
    every lane, with the automatic plan the forward uses."""
    d = synth.make(synth.GPT, index=5)
    a = {n: f64(d[n]) for n in ("w", "u", "k", "v")}
    dev = torch.device("cuda")
    note("fwd ckpt gpt full size")
    y, so, ck = wkv.wkv_forward_checkpointed(*(d[n].to(dev) for n in ("w", "u", "k", "v")),
                                             state_out=True)
    torch.cuda.synchronize()
    ref_ck, ref_end = oracle_checkpoints(oracle, a["w"], a["u"], a["k"], a["v"])
    assert ck.shape[0] == 7
    assert_ckpts_close(ck, ref_ck, "gpt")
    assert_state_close(f64(so), ref_end)


# ------------------------------------------------------------- backward ---

def backward_ref(oracle, d, s_in, s_out, g_out):
    a = {n: f64(d[n]) for n in ("w", "u", "k", "v", "dy")}
    return oracle.backward_state(a["w"], a["u"], a["k"], a["v"], a["dy"], s_in, s_out, g_out)


def check_grads(oracle, got, ref, d, what, dt=torch.float32, states=(None, None, None)):
    dy, v = f64(d["dy"]), f64(d["v"])
    f = roundoff_floor(dy, v)
    fs = roundoff_floor(dy, v, summed=True)
    h = HALF_ULP.get(dt, 0.0)
    for name, x, r in (("dk", got[0], ref[0]), ("dv", got[1], ref[1])):
        x = f64(x)
        assert np.all(np.isfinite(x)), f"{what} {name}"
        if r.size == 0:
            continue
        rms = float(np.sqrt(np.mean(r * r)))
        e = float(np.max(np.abs(x - r) / ((G_RTOL + h) * np.abs(r) + G_FLOOR * rms + f + 1e-300)))
        assert e <= 1.0, f"{what} {name}: {e:.3g}x the tolerance"
    assert_sums_close(oracle, f64(got[2]), f64(got[3]), ref[2], ref[3],
                      *(f64(d[n]) for n in ("w", "u", "k", "v", "dy")), *states, what=what)
    if got[4] is not None:
        for pl in range(3):
            assert_grad_close(f64(got[4])[pl], ref[4][pl], f"{what} d_state_in[{pl}]", fs)


BSHAPES = [(1, 1, 5), (2, 128, 64), (2, 129, 64), (2, 300, 100), (1, 513, 130), (2, 1024, 96),
           (1, 1100, 33)]


@pytest.mark.parametrize("shape", BSHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("recipe", [synth.GPT, synth.STABILITY])
@pytest.mark.parametrize("states", [False, True])
def test_backward_from_oracle_checkpoints(oracle, shape, recipe, states):
    B, T, C = shape
    d = synth.make(recipe, index=93, B=B, T=T, C=C, with_dy=True)
    a = {n: f64(d[n]) for n in ("w", "u", "k", "v")}
    s_in = reachable_state(oracle, B, C, 94) if states else None
    ck, s_end = oracle_checkpoints(oracle, a["w"], a["u"], a["k"], a["v"], s_in)
    ck = ck.astype(np.float32).astype(np.float64)
    s_out = s_end.astype(np.float32).astype(np.float64) if states else None
    g_out = (synth.normal((3, B, C), 1.0, synth.seed_of(synth.GPT, 9500, 0)).double().numpy()
             if states else None)
    note(f"bwd ckpt B={B} T={T} C={C} recipe={recipe} states={states}")
    dev = torch.device("cuda")
    got = wkv.wkv_backward_checkpointed(*(d[n].to(dev) for n in ("w", "u", "k", "v", "dy")),
                                        to_dev(ck), state_in=to_dev(s_in), state_out=to_dev(s_out),
                                        d_state_out=to_dev(g_out),
                                        d_state_in=True if states else None)
    torch.cuda.synchronize()
    check_grads(oracle, got, backward_ref(oracle, d, s_in, s_out, g_out), d, "bwd ckpt",
                states=(s_in, s_out, g_out))


@pytest.mark.parametrize("dt", [torch.float32, torch.float16, torch.bfloat16],
                         ids=["f32", "f16", "bf16"])
@pytest.mark.parametrize("shape", [(2, 300, 100), (1, 1024, 64), (3, 129, 40)],
                         ids=lambda s: "x".join(map(str, s)))
def test_training_path_forward_then_backward(oracle, dt, shape):
    """The GPU forward writes the checkpoints, the GPU backward reads them; the
    gradients are held to the oracle's on the seeded inputs."""
    B, T, C = shape
    d = synth.make(synth.STABILITY, index=95, B=B, T=T, C=C, with_dy=True)
    d = {n: (t.to(dt) if n in ("k", "v", "dy") else t) for n, t in d.items()}
    dev = torch.device("cuda")
    w, u, k, v, dy = (d[n].to(dev) for n in ("w", "u", "k", "v", "dy"))
    note(f"train path {dt} B={B} T={T} C={C}")
    _, _, ck = wkv.wkv_forward_checkpointed(w, u, k, v)
    got = wkv.wkv_backward_checkpointed(w, u, k, v, dy, ck)
    torch.cuda.synchronize()
    assert got[0].dtype == dt
    check_grads(oracle, got, backward_ref(oracle, d, None, None, None), d, "train", dt)


def test_backward_checkpointed_is_reproducible(oracle):
    d = synth.make(synth.STABILITY, index=96, B=2, T=700, C=96, with_dy=True)
    dev = torch.device("cuda")
    w, u, k, v, dy = (d[n].to(dev) for n in ("w", "u", "k", "v", "dy"))
    _, _, ck = wkv.wkv_forward_checkpointed(w, u, k, v, plan=PLANS["seg16x16"])
    a = wkv.wkv_backward_checkpointed(w, u, k, v, dy, ck)
    b = wkv.wkv_backward_checkpointed(w, u, k, v, dy, ck)
    torch.cuda.synchronize()
    for x, y in zip(a[:4], b[:4]):
        assert torch.equal(x, y)


def test_stability_training_path_full_size_sampled(oracle):
    """B=8 T=4096 C=2048 with a carried state and an upstream state gradient:
    the GPU forward's 31 checkpoints feed the GPU backward; the checkpoints and
    every gradient of 8 sampled channels (all sequences) against the oracle."""
    B, T, C = 8, 4096, 2048
    d = synth.make(synth.STABILITY, index=97, with_dy=True)
    cs = np.array([0, 1, 63, 64, 777, 1500, 2046, 2047])
    sub = {n: (f64(d[n])[:, :, cs] if n in ("k", "v", "dy") else f64(d[n])[cs])
           for n in ("w", "u", "k", "v", "dy")}
    p = synth.make(synth.TINY, index=98, B=B, T=16, C=C)
    _, s_in = oracle.forward_scan(f64(d["w"]), f64(d["u"]), f64(p["k"]), f64(p["v"]))
    s_in = s_in.astype(np.float32).astype(np.float64)
    ref_ck, ref_end = oracle_checkpoints(oracle, sub["w"], sub["u"], sub["k"], sub["v"],
                                         s_in[:, :, cs])
    # the upstream gradient is given in the coordinates of the oracle's final
    # state (sampled channels; the others get none)
    s_out_sub = ref_end.astype(np.float32).astype(np.float64)
    s_out = np.zeros((3, B, C))
    s_out[:, :, cs] = s_out_sub
    s_out[1][:, np.setdiff1d(np.arange(C), cs)] = 1.0
    g_out = np.zeros((3, B, C))
    g_out[:, :, cs] = synth.normal((3, B, len(cs)), 1.0,
                                   synth.seed_of(synth.GPT, 9600, 0)).double().numpy()
    dev = torch.device("cuda")
    w, u, k, v, dy = (d[n].to(dev) for n in ("w", "u", "k", "v", "dy"))
    note("train path stability full size")
    _, so, ck = wkv.wkv_forward_checkpointed(w, u, k, v, state_in=to_dev(s_in), state_out=True)
    got = wkv.wkv_backward_checkpointed(w, u, k, v, dy, ck, state_in=to_dev(s_in),
                                        state_out=to_dev(s_out), d_state_out=to_dev(g_out),
                                        d_state_in=True)
    torch.cuda.synchronize()
    assert ck.shape[0] == 31
    assert_ckpts_close(ck[:, :, :, cs], ref_ck, "stability")
    assert_state_close(f64(so)[:, :, cs], ref_end)
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

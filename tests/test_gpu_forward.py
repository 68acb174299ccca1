"""GPU parity of wkv_forward (every compiled kernel variant) against the oracle.

Inputs are seeded (linear_recurrent_attention_amd.synth) and the oracle reads
back the exact float32 values the GPU consumed.  Tolerances: tests/parity.py.
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

PLANS = {
    "auto": None,
    "lane": (wkv.WKV_KERNEL_LANE, 0, 0),
    "seg16x8": (wkv.WKV_KERNEL_SEGMENTED, 16, 8),
    "seg16x16": (wkv.WKV_KERNEL_SEGMENTED, 16, 16),
    "seg8x16": (wkv.WKV_KERNEL_SEGMENTED, 8, 16),
    "seg8x32": (wkv.WKV_KERNEL_SEGMENTED, 8, 32),
    "seg4x32": (wkv.WKV_KERNEL_SEGMENTED, 4, 32),
    "seg16x16c32": (wkv.WKV_KERNEL_SEGMENTED, 16, 16, 32),
    "seg32x8c32": (wkv.WKV_KERNEL_SEGMENTED, 32, 8, 32),
    "seg16x8c32": (wkv.WKV_KERNEL_SEGMENTED, 16, 8, 32),
    "seg16x16c16": (wkv.WKV_KERNEL_SEGMENTED, 16, 16, 16),
    "seg32x8c16": (wkv.WKV_KERNEL_SEGMENTED, 32, 8, 16),
    "lb4x16": (wkv.WKV_KERNEL_LOOKBACK, 4, 16),
    "lb8x16": (wkv.WKV_KERNEL_LOOKBACK, 8, 16),
    "lb4x32": (wkv.WKV_KERNEL_LOOKBACK, 4, 32),
    "lb8x8": (wkv.WKV_KERNEL_LOOKBACK, 8, 8),
    "lb2x16c128": (wkv.WKV_KERNEL_LOOKBACK, 2, 16, 128),
    "lb4x16c128": (wkv.WKV_KERNEL_LOOKBACK, 4, 16, 128),
    "lb2x32c128": (wkv.WKV_KERNEL_LOOKBACK, 2, 32, 128),
    "lb4x8c128": (wkv.WKV_KERNEL_LOOKBACK, 4, 8, 128),
    "lb2x16c256": (wkv.WKV_KERNEL_LOOKBACK, 2, 16, 256),
    "lb2x8c256": (wkv.WKV_KERNEL_LOOKBACK, 2, 8, 256),
    "lb8x32": (wkv.WKV_KERNEL_LOOKBACK, 8, 32),
    "lb4x32c128": (wkv.WKV_KERNEL_LOOKBACK, 4, 32, 128),
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
    """A non-empty state from the oracle (float32-rounded), so no input of a
    parity test comes from the HIP path."""
    d = synth.make(synth.TINY, index=500 + seed, B=B, T=9, C=C)
    _, s = oracle.forward_scan(*(d[n].double().numpy() for n in ("w", "u", "k", "v")))
    return torch.from_numpy(s.astype(np.float32))


def run(d, plan, state_in=None):
    dev = torch.device("cuda")
    w, u, k, v = (d[n].to(dev) for n in ("w", "u", "k", "v"))
    si = None if state_in is None else state_in.to(dev)
    y, so = wkv.wkv_forward(w, u, k, v, state_in=si, state_out=True, plan=plan)
    torch.cuda.synchronize()
    return y, so


@pytest.mark.parametrize("plan", list(PLANS))
def test_tiny_config_matches_brute_force(oracle, plan):
    d = synth.make(synth.TINY, index=0)
    note(f"tiny B=1 T=64 C=32 plan={plan}")
    y, so = run(d, PLANS[plan])
    yr, sr = oracle.forward_brute(*(f64(d[n]) for n in ("w", "u", "k", "v")))
    assert_y_close(f64(y), yr)
    assert_state_close(f64(so), sr)


SHAPES = [(1, 1, 5), (2, 300, 100), (3, 17, 64), (1, 513, 130), (2, 1024, 64), (1, 2049, 33)]


@pytest.mark.parametrize("plan", list(PLANS))
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("with_state", [False, True])
def test_ragged_shapes_match_oracle(oracle, plan, shape, with_state):
    B, T, C = shape
    d = synth.make(synth.GPT, index=1, B=B, T=T, C=C)
    si = reachable_state(oracle, B, C, 1) if with_state else None
    note(f"ragged B={B} T={T} C={C} state={with_state} plan={plan}")
    y, so = run(d, PLANS[plan], si)
    yr, sr = oracle.forward_scan(*(f64(d[n]) for n in ("w", "u", "k", "v")),
                                 None if si is None else si.double().numpy(), nthreads=NTHREADS)
    assert_y_close(f64(y), yr)
    assert_state_close(f64(so), sr)


@pytest.mark.parametrize("plan", list(PLANS))
def test_wide_exponents_match_oracle(oracle, plan):
    """Stability recipe: k ~ N(0,8) with +-60 outliers, decay in U(-8,3), u ~ N(0,2)."""
    d = synth.make(synth.STABILITY, index=2, B=2, T=1500, C=96)
    note(f"stability B=2 T=1500 C=96 plan={plan}")
    y, so = run(d, PLANS[plan])
    yr, sr = oracle.forward_scan(*(f64(d[n]) for n in ("w", "u", "k", "v")), nthreads=NTHREADS)
    assert_y_close(f64(y), yr)
    assert_state_close(f64(so), sr)


@pytest.mark.parametrize("plan", list(PLANS))
@pytest.mark.parametrize("with_state", [False, True])
def test_extreme_decays_match_oracle(oracle, plan, with_state):
    """Decay rates spread geometrically from 1e-6 (nothing decays over the
    sequence) to 60 (the past vanishes within two tokens), stability keys."""
    B, T, C = 2, 700, 96
    d = synth.make(synth.STABILITY, index=9, B=B, T=T, C=C)
    d["w"] = torch.from_numpy(np.geomspace(1e-6, 60.0, C).astype(np.float32))
    si = reachable_state(oracle, B, C, 9) if with_state else None
    note(f"extreme decays plan={plan} state={with_state}")
    y, so = run(d, PLANS[plan], si)
    yr, sr = oracle.forward_scan(*(f64(d[n]) for n in ("w", "u", "k", "v")),
                                 None if si is None else si.double().numpy(), nthreads=NTHREADS)
    assert_y_close(f64(y), yr)
    assert_state_close(f64(so), sr)


@pytest.mark.parametrize("plan", ["lane", "seg16x16", "seg8x32", "seg32x8c16", "lb4x16",
                                  "lb4x16c128"])
def test_extreme_bonus_takes_the_two_exponential_path(oracle, plan):
    """|u - w| beyond the one-exponential step's range on some channels."""
    d = synth.make(synth.TINY, index=3, B=2, T=200, C=128)
    d["u"][::3] = 75.0
    d["u"][1::7] = -70.0
    note(f"extreme bonus plan={plan}")
    y, so = run(d, PLANS[plan])
    yr, sr = oracle.forward_scan(*(f64(d[n]) for n in ("w", "u", "k", "v")), nthreads=NTHREADS)
    assert_y_close(f64(y), yr)
    assert_state_close(f64(so), sr)


@pytest.mark.parametrize("plan", list(PLANS))
@pytest.mark.parametrize("with_state", [False, True], ids=["empty", "tiny_state"])
def test_small_bonus_first_token_below_the_segment_maximum(oracle, plan, with_state):
    """A bonus near the one-exponential step's lower limit (u down to -59 with
    w = 0.01) and a key 45 above the first token's a few tokens later, from
    the empty state or from a state whose denominator is tiny: a frame taken
    at the segment's largest exponent puts the first token's denominator
    below float's normal range, so such a segment must take the token-by-token
    path (the output of a first token from the empty state is its own v)."""
    B, T, C = 2, 192, 64
    w = torch.full((C,), 0.01)
    u = torch.linspace(-30.0, -59.0, C)
    k = torch.zeros(B, T, C)
    k[:, 5::64, :] = 45.0
    v = synth.normal((B, T, C), 1.0, synth.seed_of(synth.TINY, 700, 0))
    d = dict(w=w, u=u, k=k, v=v)
    si = None
    if with_state:
        si = torch.zeros(3, B, C)
        si[1] = 1e-30
        si[2] = -5.0
    note(f"small bonus, first token low, plan={plan} state={with_state}")
    y, so = run(d, PLANS[plan], si)
    yr, sr = oracle.forward_scan(*(f64(d[n]) for n in ("w", "u", "k", "v")),
                                 None if si is None else f64(si))
    assert_y_close(f64(y), yr)
    assert_state_close(f64(so), sr)


@pytest.mark.parametrize("plan", ["auto", "lane", "seg16x16", "seg16x16c32", "lb4x16", "lb8x8",
                                  "lb2x16c256"])
def test_state_updated_in_place(oracle, plan):
    B, T, C = 2, 333, 80
    d = synth.make(synth.GPT, index=4, B=B, T=T, C=C)
    si = reachable_state(oracle, B, C, 4)
    dev = torch.device("cuda")
    st = si.to(dev).clone()
    w, u, k, v = (d[n].to(dev) for n in ("w", "u", "k", "v"))
    note(f"in-place state plan={plan}")
    y, _ = wkv.wkv_forward(w, u, k, v, state_in=st, state_out=st, plan=PLANS[plan])
    torch.cuda.synchronize()
    yr, sr = oracle.forward_scan(*(f64(d[n]) for n in ("w", "u", "k", "v")), si.double().numpy())
    assert_y_close(f64(y), yr)
    assert_state_close(f64(st), sr)


def test_zero_length_and_empty_calls(oracle):
    dev = torch.device("cuda")
    B, C = 2, 40
    si = reachable_state(oracle, B, C, 5).to(dev)
    w = torch.ones(C, device=dev)
    u = torch.zeros(C, device=dev)
    k = torch.empty((B, 0, C), device=dev)
    note("T=0 calls")
    y, so = wkv.wkv_forward(w, u, k, k, state_in=si, state_out=True)
    torch.cuda.synchronize()
    assert y.shape == (B, 0, C)
    assert torch.equal(so, si)
    _, so = wkv.wkv_forward(w, u, k, k, state_in=None, state_out=True)
    torch.cuda.synchronize()
    s = f64(so)
    assert np.all(s[0] == 0) and np.all(s[1] == 0) and np.all(s[2] <= -1e30)
    # an empty state written by T=0 behaves as no state
    d = synth.make(synth.TINY, index=6, B=B, T=50, C=C)
    y1, s1 = run(d, None, so.cpu())
    y0, s0 = run(d, None, None)
    assert torch.equal(y1, y0)
    # B == 0: nothing to do
    z = torch.empty((0, 7, C), device=dev)
    wkv.wkv_forward(w, u, z, z, state_out=None)
    torch.cuda.synchronize()


def test_gpt_workload_full_size(oracle):
    """B=8 T=1024 C=2048 (the 24-layer, 2048-wide model at ctx 1024), two of the
    24 seeded layers, every element against the oracle."""
    dev = torch.device("cuda")
    sh = synth.SHAPES[synth.GPT]
    for layer in (0, 23):
        d = synth.make(synth.GPT, index=layer, device=dev)
        note(f"gpt full layer={layer} plan={wkv.wkv_forward_plan_auto(sh['B'], sh['T'], sh['C'])}")
        y, so = wkv.wkv_forward(d["w"], d["u"], d["k"], d["v"], state_out=True)
        torch.cuda.synchronize()
        yr, sr = oracle.forward_scan(*(f64(d[n]) for n in ("w", "u", "k", "v")),
                                     nthreads=NTHREADS)
        assert_y_close(f64(y), yr)
        assert_state_close(f64(so), sr)


def test_stability_workload_forward_full_size(oracle):
    """B=8 T=4096 C=2048 with the wide-exponent recipe, every element."""
    dev = torch.device("cuda")
    d = synth.make(synth.STABILITY, index=0, device=dev)
    note("stability full forward B=8 T=4096 C=2048")
    y, so = wkv.wkv_forward(d["w"], d["u"], d["k"], d["v"], state_out=True)
    torch.cuda.synchronize()
    yr, sr = oracle.forward_scan(*(f64(d[n]) for n in ("w", "u", "k", "v")), nthreads=NTHREADS)
    assert_y_close(f64(y), yr)
    assert_state_close(f64(so), sr)


@pytest.mark.parametrize("plan", [p for p in PLANS if p != "auto"])
def test_every_kernel_on_the_gpt_workload_sampled(oracle, plan):
    """Each forced kernel at the full B=8 T=1024 C=2048 shape; 96 sampled lanes
    checked over all tokens."""
    dev = torch.device("cuda")
    d = synth.make(synth.GPT, index=7, device=dev)
    note(f"gpt full forced plan={plan}")
    y, so = wkv.wkv_forward(d["w"], d["u"], d["k"], d["v"], state_out=True, plan=PLANS[plan])
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    bs = torch.from_numpy(rng.integers(0, 8, 96)).to(dev)
    cs = torch.from_numpy(rng.integers(0, 2048, 96)).to(dev)

    def lanes(t):  # [B][T][C] -> [1][T][96]
        return t[bs, :, cs].transpose(0, 1).unsqueeze(0)

    yr, sr = oracle.forward_scan(f64(d["w"][cs]), f64(d["u"][cs]), f64(lanes(d["k"])),
                                 f64(lanes(d["v"])))
    assert_y_close(f64(lanes(y)), yr)
    assert_state_close(f64(so[:, bs, cs].unsqueeze(1)), sr)


# Grids whose workgroups the look-back forward hands to the dies in windows:
# 128 workgroups per block over more than two generations (B=4, C=2048,
# 18 blocks of 128 tokens, the last one ragged), 80 per block (B=1, C=5120)
# and 40 per block (B=1, C=2560), each from a carried state.
@pytest.mark.parametrize("shape", [(4, 2200, 2048), (1, 1000, 5120), (1, 777, 2560)],
                         ids=lambda s: "x".join(map(str, s)))
def test_die_windows_match_oracle(oracle, shape):
    B, T, C = shape
    d = synth.make(synth.GPT, index=63, B=B, T=T, C=C)
    si = reachable_state(oracle, B, C, 4)
    note(f"die windows B={B} T={T} C={C}")
    y, so = run(d, None, si)
    yr, sr = oracle.forward_scan(*(f64(d[n]) for n in ("w", "u", "k", "v")), si.double().numpy(),
                                 nthreads=NTHREADS)
    assert_y_close(f64(y), yr)
    assert_state_close(f64(so), sr)

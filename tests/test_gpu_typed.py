"""GPU parity of the 16-bit activation formats (fp16, bf16) against the oracle.

k, v and r are stored in the format and widened exactly; w, u and the state are
float32; y is rounded once to the format.  The oracle reads the exact 16-bit
values the GPU consumed (widened to float64) and computes in float64.

Tolerance of y: the forward's bound plus one rounding to the format,
|x - r| <= 1e-5 + (1e-4 + h)|r| with h = 2^-8 for bfloat16 (8 significant bits)
and 2^-11 for fp16 (11 bits): the relative half-unit of the last place.  The
state is float32 and keeps the forward's canonical-state bound.
"""
import os
import sys

import numpy as np
import pytest
import torch

from linear_recurrent_attention_amd import synth, wkv
from parity import Y_ATOL, Y_RTOL, assert_state_close, assert_y_close, f64

pytestmark = pytest.mark.gpu

NTHREADS = max(1, min(16, os.cpu_count() or 1))
HALF_ULP = {torch.float16: 2.0 ** -11, torch.bfloat16: 2.0 ** -8}
DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16}

PLANS = {
    "auto": None,
    "lane": (wkv.WKV_KERNEL_LANE, 0, 0),
    "seg16x16": (wkv.WKV_KERNEL_SEGMENTED, 16, 16),
    "lb4x16": (wkv.WKV_KERNEL_LOOKBACK, 4, 16),
    "lb4x32": (wkv.WKV_KERNEL_LOOKBACK, 4, 32),
    "lb8x16": (wkv.WKV_KERNEL_LOOKBACK, 8, 16),
}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no HIP device visible")
    wkv.load_library()


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def assert_y16_close(x, r, dt, what="y"):
    x = f64(x)
    assert np.all(np.isfinite(x)), f"{what}: non-finite values"
    if x.size == 0:
        return
    e = float(np.max(np.abs(x - r) / (Y_ATOL + (Y_RTOL + HALF_ULP[dt]) * np.abs(r))))
    assert e <= 1.0, f"{what}: error {e:.3g}x the tolerance"


def cast(d, dt, names=("k", "v")):
    return {n: (t.to(dt) if n in names else t) for n, t in d.items()}


def reachable_state(oracle, B, C, seed):
    d = synth.make(synth.TINY, index=800 + seed, B=B, T=9, C=C)
    _, s = oracle.forward_scan(*(d[n].double().numpy() for n in ("w", "u", "k", "v")))
    return torch.from_numpy(s.astype(np.float32))


def run(d, plan, r=None, s_in=None):
    dev = torch.device("cuda")
    w, u, k, v = (d[n].to(dev) for n in ("w", "u", "k", "v"))
    y, so = wkv.wkv_forward_typed(w, u, k, v, None if r is None else r.to(dev),
                                  state_in=None if s_in is None else s_in.to(dev),
                                  state_out=True, plan=plan)
    torch.cuda.synchronize()
    return y, so


def reference(oracle, d, r=None, s_in=None):
    y, s = oracle.forward_scan(*(f64(d[n]) for n in ("w", "u", "k", "v")),
                               None if s_in is None else s_in.double().numpy(),
                               nthreads=NTHREADS)
    return (y if r is None else oracle.gate(y, f64(r))), s


SHAPES = [(1, 1, 5), (2, 300, 100), (3, 17, 64), (1, 513, 130), (2, 1024, 64), (1, 2049, 33)]


@pytest.mark.parametrize("dt", list(DTYPES))
@pytest.mark.parametrize("plan", list(PLANS))
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("gated", [False, True])
def test_typed_forward_matches_oracle(oracle, dt, plan, shape, gated):
    if gated and plan == "lb4x32":
        pytest.skip("no gated 4x32 look-back variant (refused; see test_abi)")
    B, T, C = shape
    dtype = DTYPES[dt]
    d = cast(synth.make(synth.GPT, index=61, B=B, T=T, C=C), dtype)
    r = synth.receptance(synth.GPT, 61, (B, T, C)).to(dtype) if gated else None
    si = reachable_state(oracle, B, C, 2) if B * C % 2 == 0 else None
    note(f"typed {dt} B={B} T={T} C={C} gated={gated} state={si is not None} plan={plan}")
    y, so = run(d, PLANS[plan], r, si)
    assert y.dtype == dtype
    yr, sr = reference(oracle, d, r, si)
    assert_y16_close(y, yr, dtype)
    assert_state_close(f64(so), sr)


@pytest.mark.parametrize("dt", list(DTYPES))
@pytest.mark.parametrize("plan", ["auto", "lane", "seg16x16", "lb4x16"])
def test_typed_wide_exponents(oracle, dt, plan):
    """Stability recipe (k ~ N(0,8) with +-60 outliers) in 16-bit activations."""
    dtype = DTYPES[dt]
    d = cast(synth.make(synth.STABILITY, index=62, B=2, T=1500, C=96), dtype)
    note(f"typed {dt} stability plan={plan}")
    y, so = run(d, PLANS[plan])
    yr, sr = reference(oracle, d)
    assert_y16_close(y, yr, dtype)
    assert_state_close(f64(so), sr)


@pytest.mark.parametrize("dt", list(DTYPES))
@pytest.mark.parametrize("gated", [False, True])
def test_typed_gpt_workload_full_size(oracle, dt, gated):
    """B=8 T=1024 C=2048 (one layer of the GPT workload), every element."""
    dtype = DTYPES[dt]
    d = cast(synth.make(synth.GPT, index=4), dtype)
    r = synth.receptance(synth.GPT, 4, (8, 1024, 2048)).to(dtype) if gated else None
    note(f"typed {dt} gpt full gated={gated}")
    y, so = run(d, None, r)
    yr, sr = reference(oracle, d, r)
    assert_y16_close(y, yr, dtype)
    assert_state_close(f64(so), sr)


def test_typed_f32_is_the_float32_forward(oracle):
    """dtype float32 runs the same kernels as wkv_forward_ex: identical bits
    for the lane and segmented kernels.  The look-back kernel composes a
    block's prefix from whichever earlier states are published first, so its
    last bits may differ from call to call; it is held to the oracle."""
    dev = torch.device("cuda")
    d = synth.make(synth.GPT, index=63, B=2, T=700, C=128)
    w, u, k, v = (d[n].to(dev) for n in ("w", "u", "k", "v"))
    for plan in (PLANS["lane"], PLANS["seg16x16"]):
        y1, s1 = wkv.wkv_forward(w, u, k, v, state_out=True, plan=plan)
        y2, s2 = wkv.wkv_forward_typed(w, u, k, v, state_out=True, plan=plan)
        torch.cuda.synchronize()
        assert torch.equal(y1, y2) and torch.equal(s1, s2), plan
    yr, sr = reference(oracle, d)
    for plan in (None, PLANS["lb4x32"]):
        y2, s2 = wkv.wkv_forward_typed(w, u, k, v, state_out=True, plan=plan)
        torch.cuda.synchronize()
        assert y2.dtype == torch.float32
        assert_y_close(f64(y2), yr)
        assert_state_close(f64(s2), sr)


def test_typed_chunked_state_carry(oracle):
    """RNN mode in bf16: chunks with the float32 state carried in place match
    the oracle over the whole sequence."""
    dev = torch.device("cuda")
    dtype = torch.bfloat16
    d = cast(synth.make(synth.STREAM, index=64, B=1, T=700, C=320), dtype)
    w, u = d["w"].to(dev), d["u"].to(dev)
    st = torch.empty((3, 1, 320), device=dev)
    st[:2].zero_()
    st[2].fill_(-1e38)
    ys, t = [], 0
    for n in (1, 100, 255, 16, 328):
        y, _ = wkv.wkv_forward_typed(w, u, d["k"][:, t:t + n].contiguous().to(dev),
                                     d["v"][:, t:t + n].contiguous().to(dev), state_in=st,
                                     state_out=st)
        ys.append(y)
        t += n
    torch.cuda.synchronize()
    yr, sr = reference(oracle, d)
    assert_y16_close(torch.cat(ys, dim=1), yr, dtype)
    assert_state_close(f64(st), sr)


@pytest.mark.parametrize("dt", list(DTYPES))
@pytest.mark.parametrize("gated", [False, True])
# (1032 and 5128: the last 1024-channel chunk of a thread partly filled)
@pytest.mark.parametrize("shape", [(3, 4, 40), (2, 3, 37), (4, 2, 1030), (2, 3, 1032),
                                   (1, 2, 5128)],
                         ids=lambda s: "x".join(map(str, s)))
def test_typed_steps_match_oracle(oracle, dt, gated, shape):
    L, B, C = shape
    dtype = DTYPES[dt]
    dev = torch.device("cuda")
    w = torch.stack([synth.channel_params(synth.DECODE, 60 + l, C)[0] for l in range(L)])
    u = torch.stack([synth.channel_params(synth.DECODE, 60 + l, C)[1] for l in range(L)])
    st = torch.stack([reachable_state(oracle, B, C, 20 + l) for l in range(L)])
    ref = [st[l].double().numpy() for l in range(L)]
    st_d = st.to(dev)
    note(f"typed step {dt} gated={gated} L={L} B={B} C={C}")
    for step in range(3):
        k, v = (t.to(dtype) for t in synth.sequence(synth.DECODE, 950 + step, (L, B, C)))
        r = synth.receptance(synth.DECODE, 950 + step, (L, B, C)).to(dtype) if gated else None
        y, _ = wkv.wkv_step_typed(w.to(dev), u.to(dev), k.to(dev), v.to(dev), st_d,
                                  r=None if r is None else r.to(dev))
        torch.cuda.synchronize()
        for l in range(L):
            yl, ref[l] = oracle.forward_scan(f64(w[l]), f64(u[l]), f64(k[l])[:, None, :],
                                             f64(v[l])[:, None, :], ref[l])
            yl = yl[:, 0, :]
            if gated:
                yl = oracle.gate(yl, f64(r[l]))
            assert_y16_close(y[l], yl, dtype, f"step {step} y")
            assert_state_close(f64(st_d[l]), ref[l], f"step {step} state")


# Grids whose workgroups the look-back forward hands to the dies in windows
# (of 128 or of 40 workgroups): several generations of 128 workgroups per
# block in 16-bit, a block of 80 (B=1, C=5120), and 40 workgroups per block.
@pytest.mark.parametrize("dt", list(DTYPES))
@pytest.mark.parametrize("shape", [(2, 1100, 4096), (1, 700, 5120), (1, 333, 2560)],
                         ids=lambda s: "x".join(map(str, s)))
def test_typed_die_windows_match_oracle(oracle, dt, shape):
    B, T, C = shape
    dtype = DTYPES[dt]
    d = cast(synth.make(synth.GPT, index=62, B=B, T=T, C=C), dtype)
    si = reachable_state(oracle, B, C, 3)
    note(f"typed die windows {dt} B={B} T={T} C={C}")
    y, so = run(d, None, None, si)
    yr, sr = reference(oracle, d, None, si)
    assert_y16_close(y, yr, dtype)
    assert_state_close(f64(so), sr)

"""GPU parity of the token shift in fp16 and bf16 (wkv_token_shift_typed and
wkv_token_shift_backward_typed) against the oracle.

The oracle reads the exact 16-bit values the GPU consumed, widened to float64.
Outputs are computed in float32 and rounded once to the format, so each is held
to the float32 bound of its float32 twin plus the format's relative half-unit h
(2^-11 fp16, 2^-8 bf16) of its own magnitude; the carried token is an exact
copy; dmu stays float32 and keeps the float32 bound.
"""
import sys

import numpy as np
import pytest
import torch

from linear_recurrent_attention_amd import synth, wkv
from parity import f64

pytestmark = pytest.mark.gpu

HALF_ULP = {torch.float16: 2.0 ** -11, torch.bfloat16: 2.0 ** -8}
DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no HIP device visible")
    wkv.load_library()


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def close(got, ref, bound, what):
    got = f64(got)
    assert got.shape == ref.shape, what
    assert np.all(np.isfinite(got)), f"{what}: non-finite"
    if ref.size:
        e = float(np.max(np.abs(got - ref) / (bound + 1e-30)))
        assert e <= 1.0, f"{what}: {e:.3g}x the tolerance"


SHAPES = [(1, 1, 4, 1), (2, 17, 64, 3), (2, 100, 100, 3), (1, 257, 96, 8), (2, 300, 36, 2),
          (2, 64, 2048, 3)]


@pytest.mark.parametrize("dt", list(DTYPES))
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_typed_shift_forward_matches_oracle(oracle, dt, shape):
    B, T, C, M = shape
    dtype = DTYPES[dt]
    mu, x, xp = synth.shift_inputs(synth.GPT, 130, B, T, C, M)
    x, xp = x.to(dtype), xp.to(dtype)
    note(f"typed shift {dt} B={B} T={T} C={C} M={M}")
    dev = torch.device("cuda")
    out, xl = wkv.wkv_token_shift(mu.to(dev), x.to(dev), xp.to(dev), x_prev_out=True)
    torch.cuda.synchronize()
    assert out.dtype == dtype and xl.dtype == dtype
    ref, ref_last = oracle.token_shift(f64(mu), f64(x), f64(xp))
    mag, _ = oracle.token_shift(f64(mu), np.abs(f64(x)), np.abs(f64(xp)))
    close(out, ref, (1e-6 + HALF_ULP[dtype]) * mag, "out")
    assert np.array_equal(f64(xl), ref_last), "carried token"


@pytest.mark.parametrize("dt", list(DTYPES))
def test_typed_shift_in_place_carried_token(oracle, dt):
    """RNN mode over chunks in a 16-bit format: x_prev updated in place."""
    dtype = DTYPES[dt]
    B, C, M = 2, 64, 3
    mu, x, xp = synth.shift_inputs(synth.GPT, 131, B, 90, C, M)
    x, xp = x.to(dtype), xp.to(dtype)
    dev = torch.device("cuda")
    carry = xp.to(dev).clone()
    outs, t = [], 0
    for n in (1, 40, 49):
        o, _ = wkv.wkv_token_shift(mu.to(dev), x[:, t:t + n].contiguous().to(dev), carry,
                                   x_prev_out=carry)
        outs.append(o)
        t += n
    torch.cuda.synchronize()
    ref, ref_last = oracle.token_shift(f64(mu), f64(x), f64(xp))
    mag, _ = oracle.token_shift(f64(mu), np.abs(f64(x)), np.abs(f64(xp)))
    close(torch.cat(outs, dim=2), ref, (1e-6 + HALF_ULP[dtype]) * mag, "chunked out")
    assert np.array_equal(f64(carry), ref_last)


@pytest.mark.parametrize("dt", list(DTYPES))
@pytest.mark.parametrize("shape", SHAPES + [(2, 0, 64, 3)], ids=lambda s: "x".join(map(str, s)))
def test_typed_shift_backward_matches_oracle(oracle, dt, shape):
    B, T, C, M = shape
    dtype = DTYPES[dt]
    mu, x, xp = synth.shift_inputs(synth.GPT, 132, B, T, C, M)
    d_out = synth.normal((M, B, T, C), 1.0, synth.seed_of(synth.GPT, 9810, 0))
    d_xpo = synth.normal((B, C), 1.0, synth.seed_of(synth.GPT, 9910, 0))
    x, xp, d_out, d_xpo = (t.to(dtype) for t in (x, xp, d_out, d_xpo))
    note(f"typed shift bwd {dt} B={B} T={T} C={C} M={M}")
    dev = torch.device("cuda")
    dx, dxp, dmu = wkv.wkv_token_shift_backward(mu.to(dev), x.to(dev), d_out.to(dev),
                                                x_prev=xp.to(dev), d_x_prev_out=d_xpo.to(dev),
                                                d_x_prev=True)
    torch.cuda.synchronize()
    assert dx.dtype == dtype and dxp.dtype == dtype and dmu.dtype == torch.float32
    a = [f64(t) for t in (mu, x, xp, d_out, d_xpo)]
    rx, rxp, rmu = oracle.token_shift_backward(*a)
    # magnitudes: the same sums over absolute values
    mx, mxp, _ = oracle.token_shift_backward(a[0], a[1], a[2], np.abs(a[3]), np.abs(a[4]))
    prev = np.concatenate([a[2][:, None], a[1][:, :-1]], axis=1) if T > 0 else a[1]
    mmu = np.einsum("mbtc,btc->mc", np.abs(a[3]), np.abs(a[1]) + np.abs(prev))
    h = HALF_ULP[dtype]
    close(dx, rx, (2e-6 + h) * np.abs(mx), "dx")
    close(dxp, rxp, (2e-6 + h) * np.abs(mxp), "d_x_prev")
    close(dmu, rmu, 4e-6 * mmu, "dmu")

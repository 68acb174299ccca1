"""GPU parity of the token shift's backward (wkv_token_shift_backward) against
the oracle.

Expected values come from the oracle's token_shift_backward on the same seeded
inputs.  Tolerances follow the float32 arithmetic: dx and d_x_prev are sums of
at most 2M + 1 products, held to 2e-6 of the sum of the terms' magnitudes;
dmu adds d (x_t - x_{t-1}) over B*T tokens in float32 partials of 16 tokens,
then 4, then in double across tiles, held to 4e-6 of the magnitudes' sum.
"""
import sys

import numpy as np
import pytest
import torch

from linear_recurrent_attention_amd import synth, wkv
from parity import f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no HIP device visible")
    wkv.load_library()


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def inputs(B, T, C, M, index):
    mu, x, xp = synth.shift_inputs(synth.GPT, index, B, T, C, M)
    d_out = synth.normal((M, B, T, C), 1.0, synth.seed_of(synth.GPT, 9800 + index, 0))
    d_xpo = synth.normal((B, C), 1.0, synth.seed_of(synth.GPT, 9900 + index, 0))
    return mu, x, xp, d_out, d_xpo


def magnitudes(mu, x, xp, d_out, d_xpo):
    """Sums of the absolute values of the terms of dx, d_x_prev and dmu (for the
    tolerance only)."""
    ad, adp = np.abs(d_out), (np.zeros(x.shape[::2]) if d_xpo is None else np.abs(d_xpo))
    mx = np.einsum("mc,mbtc->btc", mu, ad)
    mx[:, :-1] += np.einsum("mc,mbtc->btc", 1.0 - mu, ad[:, :, 1:])
    if x.shape[1] > 0:
        mx[:, -1] += adp
    mxp = np.einsum("mc,mbc->bc", 1.0 - mu, ad[:, :, 0]) if x.shape[1] > 0 else adp
    prev = np.concatenate([(np.zeros_like(x[:, :1]) if xp is None else xp[:, None]), x[:, :-1]],
                          axis=1)
    mmu = np.einsum("mbtc,btc->mc", ad, np.abs(x) + np.abs(prev))
    return mx, mxp, mmu


def close(got, ref, mag, rel, what):
    got = f64(got)
    assert got.shape == ref.shape, what
    assert np.all(np.isfinite(got)), f"{what}: non-finite"
    if ref.size:
        e = float(np.max(np.abs(got - ref) / (rel * mag + 1e-30)))
        assert e <= 1.0, f"{what}: {e:.3g}x the tolerance"


def run(oracle, B, T, C, M, index, with_prev, with_dxpo, want_dxp=True, offset=0):
    mu, x, xp, d_out, d_xpo = inputs(B, T, C, M, index)
    xp = xp if with_prev else None
    d_xpo = d_xpo if with_dxpo else None
    dev = torch.device("cuda")
    g = lambda t: None if t is None else t.to(dev)
    if offset:
        # views at a 4-byte offset: the kernel must fall back to one channel per lane
        base = torch.empty(x.numel() + 1, device=dev)
        xd = base[1:].view(x.shape)
        xd.copy_(x.to(dev))
    else:
        xd = x.to(dev)
    note(f"shift bwd B={B} T={T} C={C} M={M} prev={with_prev} dxpo={with_dxpo} off={offset}")
    dx, dxp, dmu = wkv.wkv_token_shift_backward(g(mu), xd, g(d_out), x_prev=g(xp),
                                                d_x_prev_out=g(d_xpo),
                                                d_x_prev=True if want_dxp else None)
    torch.cuda.synchronize()
    a = [f64(t) if t is not None else None for t in (mu, x, xp, d_out, d_xpo)]
    rx, rxp, rmu = oracle.token_shift_backward(*a[:4], a[4])
    mx, mxp, mmu = magnitudes(a[0], a[1], a[2], a[3], a[4])
    close(dx, rx, mx, 2e-6, "dx")
    if want_dxp:
        close(dxp, rxp, mxp, 2e-6, "d_x_prev")
    close(dmu, rmu, mmu, 4e-6, "dmu")
    return dx, dxp, dmu


SHAPES = [(1, 1, 4, 1), (2, 17, 64, 3), (2, 100, 100, 3), (3, 130, 256, 2), (1, 257, 96, 8),
          (2, 64, 2048, 3), (1, 65, 36, 4), (2, 300, 20, 5)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("with_prev,with_dxpo", [(True, True), (False, True), (True, False)])
def test_shift_backward_matches_oracle(oracle, shape, with_prev, with_dxpo):
    run(oracle, *shape, 120, with_prev, with_dxpo)


def test_shift_backward_unaligned_buffers(oracle):
    run(oracle, 2, 100, 128, 3, 121, True, True, offset=1)


def test_shift_backward_without_d_x_prev(oracle):
    run(oracle, 2, 70, 64, 2, 122, True, True, want_dxp=False)


@pytest.mark.parametrize("shape", [(2, 0, 64, 3), (0, 10, 64, 3), (2, 40, 64, 0)],
                         ids=["T0", "B0", "M0"])
def test_shift_backward_degenerate(oracle, shape):
    """No tokens: the carried token's gradient passes to d_x_prev and dmu is 0.
    No sequences: dmu is 0.  No mixes: dx is the carried token's gradient at
    T - 1 only, and d_x_prev is 0."""
    run(oracle, *shape, 123, True, True)


def test_shift_backward_gpt_shape_full(oracle):
    """B=8 T=1024 C=2048 with the 3 mixes of R, K, V: every element."""
    run(oracle, 8, 1024, 2048, 3, 124, True, True)


def test_shift_backward_is_reproducible():
    B, T, C, M = 2, 700, 256, 3
    mu, x, xp, d_out, d_xpo = (t.cuda() for t in inputs(B, T, C, M, 125))
    a = wkv.wkv_token_shift_backward(mu, x, d_out, x_prev=xp, d_x_prev_out=d_xpo, d_x_prev=True)
    b = wkv.wkv_token_shift_backward(mu, x, d_out, x_prev=xp, d_x_prev_out=d_xpo, d_x_prev=True)
    torch.cuda.synchronize()
    for p, q in zip(a, b):
        assert torch.equal(p, q)

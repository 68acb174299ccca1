"""GPU parity of wkv_step (batched T=1 RNN step over layers): against the oracle,
against wkv_forward with T=1, in place, and at the decode workload's full shape
(24 layers x 1024 sequences x 4096 channels, 256 warm-up tokens) on sampled
lanes."""
import os
import sys

import numpy as np
import pytest
import torch

from linear_recurrent_attention_amd import synth, wkv
from parity import assert_state_close, assert_y_close, f64

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


def oracle_states(oracle, L, B, C, seed):
    """[L][3][B][C] float32 states produced by the oracle from seeded prefixes."""
    out = []
    for l in range(L):
        d = synth.make(synth.DECODE, index=9000 + 17 * seed + l, B=B, T=11, C=C)
        _, s = oracle.forward_scan(*(d[n].double().numpy() for n in ("w", "u", "k", "v")))
        out.append(s)
    return torch.from_numpy(np.stack(out).astype(np.float32))


# C = 37 and 1030 take the one-channel path; 1032, 2056 and 5128 leave the
# last 1024-channel chunk of the four-wide path partly filled; grids of 64
# workgroups (4x16x40, and 2x16x5128 with two per row) are handed to the dies
# in windows.
@pytest.mark.parametrize("shape", [(3, 4, 40), (2, 3, 37), (1, 1, 1), (4, 2, 1030),
                                   (2, 3, 1032), (1, 2, 5128), (2, 2, 2056), (4, 16, 40),
                                   (2, 16, 5128)],
                         ids=lambda s: "x".join(map(str, s)))
def test_steps_match_oracle(oracle, shape):
    L, B, C = shape
    dev = torch.device("cuda")
    wu = [synth.channel_params(synth.DECODE, l, C) for l in range(L)]
    w = torch.stack([x[0] for x in wu])
    u = torch.stack([x[1] for x in wu])
    s0 = oracle_states(oracle, L, B, C, 0)
    st = s0.to(dev).clone()
    ks, vs, ys = [], [], []
    note(f"step L={L} B={B} C={C}")
    for r in range(5):
        k, v = synth.sequence(synth.DECODE, 100 + r, (L, B, C))
        y, _ = wkv.wkv_step(w.to(dev), u.to(dev), k.to(dev), v.to(dev), st)
        ks.append(k)
        vs.append(v)
        ys.append(y.cpu())
    torch.cuda.synchronize()
    for l in range(L):
        k = torch.stack([x[l] for x in ks], dim=1)   # [B][5][C]
        v = torch.stack([x[l] for x in vs], dim=1)
        yr, sr = oracle.forward_scan(f64(w[l]), f64(u[l]), f64(k), f64(v), f64(s0[l]))
        yg = torch.stack([x[l] for x in ys], dim=1)
        assert_y_close(f64(yg), yr, f"y layer {l}")
        assert_state_close(f64(st[l]), sr, f"state layer {l}")


def test_steps_at_extreme_decays_match_oracle(oracle):
    """Decay rates from 1e-6 to 60 across the channels of every layer, bonus
    from -70 to +75: 40 steps from oracle states, state updated in place."""
    L, B, C = 2, 3, 96
    dev = torch.device("cuda")
    w = torch.from_numpy(np.geomspace(1e-6, 60.0, C).astype(np.float32)).repeat(L, 1)
    u = torch.from_numpy(np.linspace(-70.0, 75.0, C).astype(np.float32))[torch.randperm(
        C, generator=torch.Generator().manual_seed(5))].repeat(L, 1)
    s0 = oracle_states(oracle, L, B, C, 3)
    st = s0.to(dev).clone()
    ks, vs, ys = [], [], []
    note("step extreme decays")
    for r in range(40):
        k, v = synth.sequence(synth.DECODE, 300 + r, (L, B, C))
        y, _ = wkv.wkv_step(w.to(dev), u.to(dev), k.to(dev), v.to(dev), st)
        ks.append(k)
        vs.append(v)
        ys.append(y.cpu())
    torch.cuda.synchronize()
    for l in range(L):
        k = torch.stack([x[l] for x in ks], dim=1)
        v = torch.stack([x[l] for x in vs], dim=1)
        yr, sr = oracle.forward_scan(f64(w[l]), f64(u[l]), f64(k), f64(v), f64(s0[l]))
        assert_y_close(f64(torch.stack([x[l] for x in ys], dim=1)), yr, f"y layer {l}")
        assert_state_close(f64(st[l]), sr, f"state layer {l}")


def test_step_equals_forward_with_one_token(oracle):
    L, B, C = 3, 8, 256
    dev = torch.device("cuda")
    wu = [synth.channel_params(synth.DECODE, l, C, device=dev) for l in range(L)]
    w = torch.stack([x[0] for x in wu])
    u = torch.stack([x[1] for x in wu])
    s0 = oracle_states(oracle, L, B, C, 1).to(dev)
    k, v = synth.sequence(synth.DECODE, 7, (L, B, C), device=dev)
    note("step vs forward(T=1)")
    y_step, s_step = wkv.wkv_step(w, u, k, v, s0, state_out=torch.empty_like(s0))
    for l in range(L):
        y_f, s_f = wkv.wkv_forward(w[l], u[l], k[l].unsqueeze(1).contiguous(),
                                   v[l].unsqueeze(1).contiguous(), state_in=s0[l],
                                   state_out=True)
        torch.cuda.synchronize()
        assert_y_close(f64(y_step[l]), f64(y_f[:, 0]), "step vs forward y")
        assert_state_close(f64(s_step[l]), f64(s_f), "step vs forward state")


def test_decode_workload_full_shape_sampled(oracle):
    """L=24 B=1024 C=4096: per-layer states from 256 warm-up tokens through
    wkv_forward, then 8 batched steps; 2048 sampled (layer, sequence, channel)
    lanes checked over all 264 tokens against the oracle."""
    sh = synth.SHAPES[synth.DECODE]
    L, B, C, WU = sh["L"], sh["B"], sh["C"], sh["warmup"]
    NSTEP = 8
    dev = torch.device("cuda")
    rng = np.random.default_rng(3)
    n = 2048
    ls = rng.integers(0, L, n)
    bs = rng.integers(0, B, n)
    cs = rng.integers(0, C, n)
    state = torch.empty((L, 3, B, C), device=dev)
    w_all = torch.empty((L, C), device=dev)
    u_all = torch.empty((L, C), device=dev)
    seq_k = np.zeros((1, WU + NSTEP, n))
    seq_v = np.zeros((1, WU + NSTEP, n))
    for l in range(L):
        w, u = synth.channel_params(synth.DECODE, l, C, device=dev)
        w_all[l] = w
        u_all[l] = u
        k, v = synth.sequence(synth.DECODE, l, (B, WU, C), device=dev)
        note(f"decode warm-up layer {l}")
        wkv.wkv_forward(w, u, k, v, state_out=state[l])
        sel = ls == l
        bi = torch.from_numpy(bs[sel]).to(dev)
        ci = torch.from_numpy(cs[sel]).to(dev)
        seq_k[0, :WU][:, sel] = f64(k[bi, :, ci]).T   # [WU][n_sel]
        seq_v[0, :WU][:, sel] = f64(v[bi, :, ci]).T
        del k, v
    torch.cuda.synchronize()
    li, bi, ci = (torch.from_numpy(x).to(dev) for x in (ls, bs, cs))
    y_s = np.zeros((1, NSTEP, n))
    for r in range(NSTEP):
        k, v = synth.sequence(synth.DECODE, 1000 + r, (L, B, C), device=dev)
        note(f"decode step {r}")
        y, _ = wkv.wkv_step(w_all, u_all, k, v, state)
        seq_k[0, WU + r] = f64(k[li, bi, ci])
        seq_v[0, WU + r] = f64(v[li, bi, ci])
        y_s[0, r] = f64(y[li, bi, ci])
    torch.cuda.synchronize()
    yr, sr = oracle.forward_scan(f64(w_all[li, ci]), f64(u_all[li, ci]), seq_k, seq_v,
                                 nthreads=NTHREADS)
    assert_y_close(y_s, yr[:, WU:], "decode y")
    assert_state_close(f64(state[li, :, bi, ci]).T[:, None, :], sr, "decode state")

"""GPU parity of RNN chunk mode: a long sequence fed as consecutive chunks with
the state carried (rwkv-architecture skill page, "Workflow 2: Long context
processing") equals one call over the whole sequence and the oracle.

Full size: B=1, C=5120, T = 1,048,576 as 1024 chunks of 1024 tokens.  The oracle
checks 128 sampled channels over every token and the final state; the chunked
GPU run is compared with one unchunked GPU call (T*C > 2^31 elements, 64-bit
indexing) on every element."""
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


def test_small_stream_all_lanes(oracle):
    C, TC, NCH = 200, 96, 12
    dev = torch.device("cuda")
    w, u = synth.channel_params(synth.STREAM, 0, C, device=dev)
    st = None
    ks, vs, ys = [], [], []
    note("small stream")
    for j in range(NCH):
        k, v = synth.sequence(synth.STREAM, j, (1, TC, C), device=dev)
        y, st = wkv.wkv_forward(w, u, k, v, state_in=st, state_out=True)
        ks.append(k)
        vs.append(v)
        ys.append(y)
    torch.cuda.synchronize()
    k, v, y = (torch.cat(x, dim=1) for x in (ks, vs, ys))
    yr, sr = oracle.forward_scan(f64(w), f64(u), f64(k), f64(v))
    assert_y_close(f64(y), yr)
    assert_state_close(f64(st), sr)
    yu, su = wkv.wkv_forward(w, u, k, v, state_out=True)
    torch.cuda.synchronize()
    assert_y_close(f64(yu), yr)
    assert_state_close(f64(su), sr)


@pytest.mark.parametrize("plan", [None, (wkv.WKV_KERNEL_SEGMENTED, 16, 16),
                                  (wkv.WKV_KERNEL_LOOKBACK, 4, 16)])
def test_bound_calls_replay_the_stream(oracle, plan):
    """bind_forward: calls marshalled once and re-issued over the chunks (the
    state updated in place, the chunk inputs rewritten between replays) match
    the oracle over the whole sequence on every replay."""
    C, TC, NCH = 200, 96, 6
    dev = torch.device("cuda")
    w, u = synth.channel_params(synth.STREAM, 1, C, device=dev)
    k = torch.empty((NCH, 1, TC, C), device=dev)
    v = torch.empty_like(k)
    y = torch.empty_like(k)
    st = torch.empty((3, 1, C), device=dev)
    calls = [wkv.bind_forward(w, u, k[j], v[j], y[j], state_in=None if j == 0 else st,
                              state_out=st, plan=plan) for j in range(NCH)]
    for rep in range(2):
        for j in range(NCH):
            k[j], v[j] = synth.sequence(synth.STREAM, 100 * rep + j, (1, TC, C), device=dev)
        for c in calls:
            c()
        torch.cuda.synchronize()
        note(f"bound stream plan={plan} replay {rep}")
        kk, vv = (x.reshape(1, NCH * TC, C) for x in (k, v))
        yr, sr = oracle.forward_scan(f64(w), f64(u), f64(kk), f64(vv))
        assert_y_close(f64(y.reshape(1, NCH * TC, C)), yr)
        assert_state_close(f64(st), sr)


def test_stream_workload_full_size(oracle):
    sh = synth.SHAPES[synth.STREAM]
    C, TC, NCH = sh["C"], sh["T"], sh["chunks"]
    T = TC * NCH
    dev = torch.device("cuda")
    w, u = synth.channel_params(synth.STREAM, 0, C, device=dev)
    rng = np.random.default_rng(5)
    cs_np = np.sort(rng.choice(C, 128, replace=False))
    cs = torch.from_numpy(cs_np).to(dev)
    k_full = torch.empty((1, T, C), device=dev)
    v_full = torch.empty((1, T, C), device=dev)
    y_chunk = torch.empty((1, T, C), device=dev)
    st = None
    note(f"stream full: {NCH} chunks of {TC} x {C}")
    for j in range(NCH):
        k, v = synth.sequence(synth.STREAM, j, (1, TC, C), device=dev)
        sl = slice(j * TC, (j + 1) * TC)
        k_full[:, sl] = k
        v_full[:, sl] = v
        _, st = wkv.wkv_forward(w, u, k, v, y=y_chunk[:, sl], state_in=st, state_out=True)
        del k, v
    torch.cuda.synchronize()
    note("stream full: unchunked call")
    y_one, st_one = wkv.wkv_forward(w, u, k_full, v_full, state_out=True)
    torch.cuda.synchronize()
    note("stream full: oracle on sampled channels")
    yr, sr = oracle.forward_scan(f64(w[cs]), f64(u[cs]), f64(k_full[:, :, cs]),
                                 f64(v_full[:, :, cs]), nthreads=NTHREADS)
    assert_y_close(f64(y_chunk[:, :, cs]), yr, "chunked y")
    assert_state_close(f64(st[:, :, cs]), sr, "chunked state")
    assert_y_close(f64(y_one[:, :, cs]), yr, "unchunked y")
    assert_state_close(f64(st_one[:, :, cs]), sr, "unchunked state")
    # chunked vs unchunked on every element (on the device)
    worst = 0.0
    for j in range(0, T, 1 << 16):
        a = y_chunk[:, j:j + (1 << 16)].double()
        b = y_one[:, j:j + (1 << 16)].double()
        worst = max(worst, float(((a - b).abs() / (1e-5 + 1e-4 * b.abs())).max()))
    assert worst <= 1.0, f"chunked vs unchunked: {worst:.3g}x the tolerance"
    assert_state_close(f64(st), f64(st_one), "chunked vs unchunked state")

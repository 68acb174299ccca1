"""GPU tests of the look-back forward's scratch handling and of the bounded
wait's give-up path.

- Growing a stream's scratch happens in stream order: the call returns while
  earlier work on the stream is still running, and its outputs match the
  oracle.
- With the test hook's spin limit at 0, every wait that finds no predecessor
  ready gives up at once (every workgroup still exits normally): the blocks
  that gave up, and the blocks that folded their poisoned state, are NaN as a
  whole; every finite output matches the oracle; wkv_lookback_status reports
  it; and the next launch on the same scratch, at the default limit, is
  correct.
"""
import sys
import time

import numpy as np
import pytest
import torch

from linear_recurrent_attention_amd import synth, wkv
from parity import assert_state_close, assert_y_close

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no HIP device visible")
    wkv.load_library()


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def oracle_lanes(oracle, d, bs, cs):
    """Oracle y [len][T] and state [3][len] of the lanes (bs[i], cs[i])."""
    w, u, k, v = (d[n].double().cpu().numpy() for n in ("w", "u", "k", "v"))
    ys, ss = [], []
    for b, c in zip(bs, cs):
        y, s = oracle.forward_scan(w[c:c + 1], u[c:c + 1], k[b:b + 1, :, c:c + 1],
                                   v[b:b + 1, :, c:c + 1])
        ys.append(y[0, :, 0])
        ss.append(s[:, 0, 0])
    return np.array(ys), np.array(ss).T


def test_scratch_growth_does_not_block(oracle):
    """A look-back forward that needs a larger scratch than its stream holds
    returns while a long kernel queued before it is still running."""
    dev = torch.device("cuda")
    st = torch.cuda.Stream()
    small = {n: t.to(dev) for n, t in synth.make(synth.GPT, index=3, B=2, T=256, C=256).items()}
    big_host = synth.make(synth.STABILITY, index=5, B=4, T=4096, C=1024)
    big = {n: t.to(dev) for n, t in big_host.items()}
    need_small = wkv.wkv_forward_scratch_size(2, 256, 256)
    need_big = wkv.wkv_forward_scratch_size(4, 4096, 1024)
    note(f"scratch small {need_small} B, big {need_big} B")
    assert need_big > (4 << 20) > need_small > 0  # the first buffer (4 MiB) is outgrown
    with torch.cuda.stream(st):
        wkv.wkv_forward(small["w"], small["u"], small["k"], small["v"], state_out=True, stream=st)
    st.synchronize()
    with torch.cuda.stream(st):
        torch.cuda._sleep(200_000_000)  # ~0.1 s of GPU time queued first
        t0 = time.perf_counter()
        y, so = wkv.wkv_forward(big["w"], big["u"], big["k"], big["v"], state_out=True,
                                stream=st)
        host_ms = (time.perf_counter() - t0) * 1e3
        busy = not st.query()
    note(f"growth call returned after {host_ms:.2f} ms, stream busy: {busy}")
    assert busy, "the call waited for the stream"
    st.synchronize()
    assert wkv.wkv_lookback_status(st) == wkv.WKV_OK
    rng = np.random.default_rng(11)
    bs, cs = rng.integers(0, 4, 24), rng.integers(0, 1024, 24)
    yr, sr = oracle_lanes(oracle, big_host, bs, cs)
    yg = y.cpu().numpy()
    assert_y_close(np.array([yg[b, :, c] for b, c in zip(bs, cs)]), yr)
    sg = so.cpu().numpy()
    assert_state_close(np.stack([sg[:, b, c] for b, c in zip(bs, cs)], axis=1), sr)
    wkv.wkv_release_stream_scratch(st)
    st.synchronize()


def test_give_up_path_poisons_whole_blocks_and_is_reported(oracle):
    """Spin limit 0: waits that find nothing ready give up at once.  NaN comes in
    whole (block, 64-channel group) tiles, every finite output is correct, the
    final state of a sequence is NaN exactly when its last block is, and the
    status call reports it; the default limit then gives a correct launch on
    the same scratch."""
    dev = torch.device("cuda")
    st = torch.cuda.Stream()
    B, T, C = 8, 1024, 2048
    host = synth.make(synth.GPT, index=7)
    d = {n: t.to(dev) for n, t in host.items()}
    plan = wkv.wkv_forward_plan_auto(B, T, C)
    assert plan[0] == wkv.WKV_KERNEL_LOOKBACK
    TB = plan[1] * plan[2]
    old = wkv.wkv_set_lookback_spin_limit(0)
    try:
        with torch.cuda.stream(st):
            y, so = wkv.wkv_forward(d["w"], d["u"], d["k"], d["v"], state_out=True, stream=st)
        status = wkv.wkv_lookback_status(st)
    finally:
        wkv.wkv_set_lookback_spin_limit(old)
    yg = y.cpu().numpy()
    sg = so.cpu().numpy()
    # [sequence][block][group][token * channel]
    per_tile = (np.isnan(yg).reshape(B, T // TB, TB, C // 64, 64).transpose(0, 1, 3, 2, 4)
                .reshape(B, T // TB, C // 64, TB * 64))
    any_nan = per_tile.any(axis=3)
    all_nan = per_tile.all(axis=3)
    note(f"spin limit 0: {int(any_nan.sum())} of {any_nan.size} tiles NaN, status {status}")
    assert np.array_equal(any_nan, all_nan), "NaN must cover whole tiles"
    assert (status == wkv.WKV_ERR_LOOKBACK) == bool(any_nan.any())
    last = any_nan[:, -1, :]  # [B][groups]
    s_nan = np.isnan(sg).any(axis=0).reshape(B, C // 64, 64)
    assert np.array_equal(s_nan.any(axis=2), last) and np.array_equal(s_nan.all(axis=2), last)
    # finite outputs are correct: check 32 lanes, all of their finite tiles
    rng = np.random.default_rng(5)
    bs, cs = rng.integers(0, B, 32), rng.integers(0, C, 32)
    yr, _ = oracle_lanes(oracle, host, bs, cs)
    for i, (b, c) in enumerate(zip(bs, cs)):
        ok = ~np.isnan(yg[b, :, c])
        if ok.any():
            assert_y_close(yg[b, ok, c], yr[i, ok], what=f"finite y of lane ({b}, {c})")
    # the same scratch at the default limit: correct and reported clean
    with torch.cuda.stream(st):
        y2, so2 = wkv.wkv_forward(d["w"], d["u"], d["k"], d["v"], state_out=True, stream=st)
    assert wkv.wkv_lookback_status(st) == wkv.WKV_OK
    y2g = y2.cpu().numpy()
    assert np.all(np.isfinite(y2g))
    assert_y_close(np.array([y2g[b, :, c] for b, c in zip(bs, cs)]), yr)
    wkv.wkv_release_stream_scratch(st)
    st.synchronize()


def test_concurrent_streams_keep_their_own_scratch(oracle):
    """Look-back forwards of two shapes issued alternately on two streams, so
    that they run concurrently, each stream on its own scratch: every output
    matches the same call made alone on the default stream."""
    dev = torch.device("cuda")
    a_host = synth.make(synth.GPT, index=21, B=8, T=1024, C=2048)
    b_host = synth.make(synth.STREAM, index=22, B=1, T=1024, C=5120)
    A = {n: t.to(dev) for n, t in a_host.items()}
    Bd = {n: t.to(dev) for n, t in b_host.items()}
    for d in (A, Bd):
        assert wkv.wkv_forward_plan_auto(*d["k"].shape)[0] == wkv.WKV_KERNEL_LOOKBACK
    ya_ref, sa_ref = wkv.wkv_forward(A["w"], A["u"], A["k"], A["v"], state_out=True)
    yb_ref, sb_ref = wkv.wkv_forward(Bd["w"], Bd["u"], Bd["k"], Bd["v"], state_out=True)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for rep in range(6):
        with torch.cuda.stream(s1):
            ya, sa = wkv.wkv_forward(A["w"], A["u"], A["k"], A["v"], state_out=True, stream=s1)
        with torch.cuda.stream(s2):
            yb, sb = wkv.wkv_forward(Bd["w"], Bd["u"], Bd["k"], Bd["v"], state_out=True,
                                     stream=s2)
        outs.append((ya, sa, yb, sb))
    torch.cuda.synchronize()
    note("concurrent look-back forwards on two streams")
    assert wkv.wkv_lookback_status(s1) == wkv.WKV_OK
    assert wkv.wkv_lookback_status(s2) == wkv.WKV_OK
    for ya, sa, yb, sb in outs:
        # same arithmetic, possibly another composition order: the y tolerance
        assert_y_close(ya.double().cpu().numpy(), ya_ref.double().cpu().numpy(), "stream 1 y")
        assert_y_close(yb.double().cpu().numpy(), yb_ref.double().cpu().numpy(), "stream 2 y")
        assert_state_close(sa.double().cpu().numpy(), sa_ref.double().cpu().numpy())
        assert_state_close(sb.double().cpu().numpy(), sb_ref.double().cpu().numpy())
    for st in (s1, s2):
        wkv.wkv_release_stream_scratch(st)
        st.synchronize()


def test_host_threads_on_their_own_streams(oracle):
    """Four host threads, each issuing look-back forwards on a stream of its
    own (ctypes drops the GIL during the call, so the library's host side
    runs concurrently: scratch creation, growth and epochs under its lock)."""
    import threading
    dev = torch.device("cuda")
    shapes = [(2, 512, 256), (1, 1024, 512), (4, 256, 128), (2, 768, 320)]
    inputs = [{n: t.to(dev) for n, t in synth.make(synth.GPT, index=30 + i, B=b, T=t, C=c).items()}
              for i, (b, t, c) in enumerate(shapes)]
    for b, t, c in shapes:
        assert wkv.wkv_forward_plan_auto(b, t, c)[0] == wkv.WKV_KERNEL_LOOKBACK
    refs = [wkv.wkv_forward(d["w"], d["u"], d["k"], d["v"], state_out=True) for d in inputs]
    torch.cuda.synchronize()
    results, errors = [None] * 4, []

    def work(i):
        try:
            st = torch.cuda.Stream()
            d = inputs[i]
            outs = []
            with torch.cuda.stream(st):
                for _ in range(25):
                    outs.append(wkv.wkv_forward(d["w"], d["u"], d["k"], d["v"], state_out=True,
                                                stream=st))
            st.synchronize()
            status = wkv.wkv_lookback_status(st)
            wkv.wkv_release_stream_scratch(st)
            st.synchronize()
            results[i] = (outs, status)
        except Exception as e:  # reported below, on the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=work, args=(i,)) for i in range(4)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    note(f"host threads: errors {errors}")
    assert not errors and all(r is not None for r in results)
    for i, (outs, status) in enumerate(results):
        assert status == wkv.WKV_OK
        yr, sr = refs[i]
        for y, so in outs:
            assert_y_close(y.double().cpu().numpy(), yr.double().cpu().numpy(), f"thread {i} y")
            assert_state_close(so.double().cpu().numpy(), sr.double().cpu().numpy())

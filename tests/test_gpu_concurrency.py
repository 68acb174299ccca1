"""Concurrent use of the library: look-back forwards on several streams at once
(each stream has its own scratch and launch tags) and calls from several host
threads.  Every result is checked against the same call made alone."""
import threading

import numpy as np
import pytest
import torch

from linear_recurrent_attention_amd import synth, wkv
from parity import assert_y_close, f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no HIP device visible")
    wkv.load_library()


def inputs(n, B, T, C):
    dev = torch.device("cuda")
    return [synth.make(synth.GPT, index=40 + i, B=B, T=T, C=C, device=dev) for i in range(n)]


def alone(d, plan):
    y, s = wkv.wkv_forward(d["w"], d["u"], d["k"], d["v"], state_out=True, plan=plan)
    torch.cuda.synchronize()
    return y, s


@pytest.mark.parametrize("plan", [None, (wkv.WKV_KERNEL_LOOKBACK, 4, 32),
                                  (wkv.WKV_KERNEL_LOOKBACK, 4, 16)])
def test_forwards_on_several_streams_at_once(plan):
    sets = inputs(4, 4, 1024, 1024)
    refs = [alone(d, plan) for d in sets]
    streams = [torch.cuda.Stream() for _ in sets]
    outs = [(torch.empty_like(d["k"]), torch.empty((3, 4, 1024), device="cuda")) for d in sets]
    torch.cuda.synchronize()
    for rep in range(3):
        for d, st, (y, s) in zip(sets, streams, outs):
            with torch.cuda.stream(st):
                for _ in range(2):  # back-to-back launches on one stream as well
                    wkv.wkv_forward(d["w"], d["u"], d["k"], d["v"], y=y, state_out=s, stream=st,
                                    plan=plan)
        torch.cuda.synchronize()
        for (yr, sr), (y, s) in zip(refs, outs):
            assert_y_close(f64(y), f64(yr), what=f"y rep {rep}")
            assert np.allclose(f64(s), f64(sr), rtol=1e-5, atol=1e-6)


def test_calls_from_several_host_threads():
    sets = inputs(4, 2, 777, 320)
    refs = [alone(d, None) for d in sets]
    results = [None] * len(sets)
    errors = []

    def work(i):
        try:
            st = torch.cuda.Stream()
            d = sets[i]
            with torch.cuda.stream(st):
                for _ in range(5):
                    y, s = wkv.wkv_forward(d["w"], d["u"], d["k"], d["v"], state_out=True,
                                           stream=st)
            st.synchronize()
            results[i] = (y, s)
        except Exception as e:  # reported below
            errors.append(e)

    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(sets))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for (yr, sr), (y, s) in zip(refs, results):
        assert_y_close(f64(y), f64(yr))

"""GPU test of wkv_forward_noalloc, the forward entry point that allocates
nothing (its look-back scratch is a fixed device array), called through the C
ABI: two calls in a row, the second on a smaller input, each checked against
wkv_forward's output to the forward tolerance (|x - r| <= 1e-5 + 1e-4 |r|) and
on sampled lanes against the oracle.  Also: no device memory is allocated by a
call, and a shape whose scratch exceeds the array is refused on the host."""
import ctypes
import sys

import numpy as np
import pytest
import torch

from linear_recurrent_attention_amd import synth, wkv
from parity import assert_state_close, assert_y_close

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.fail("no HIP device visible")
    return wkv.load_library()


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def vp(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def call_noalloc(lib, d, y, state_in, state_out, stream):
    B, T, C = (int(x) for x in d["k"].shape)
    return lib.wkv_forward_noalloc(B, T, C, vp(d["w"]), vp(d["u"]), vp(d["k"]), vp(d["v"]), vp(y),
                                   vp(state_in), vp(state_out),
                                   ctypes.c_void_p(stream.cuda_stream))


def check_against_forward(lib, oracle, host, state_in_host, seed):
    dev = torch.device("cuda")
    st = torch.cuda.current_stream()
    d = {n: t.to(dev) for n, t in host.items()}
    B, T, C = (int(x) for x in d["k"].shape)
    si = None if state_in_host is None else state_in_host.to(dev)
    y = torch.empty_like(d["k"])
    so = torch.empty((3, B, C), device=dev)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    status = call_noalloc(lib, d, y, si, so, st)
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    assert status == wkv.WKV_OK, wkv.wkv_status_string(status)
    note(f"noalloc B={B} T={T} C={C} scratch {wkv.wkv_forward_scratch_size(B, T, C)} B, "
         f"free device memory {free0} -> {free1}")
    assert free1 == free0, "the call allocated device memory"
    yr, sr = wkv.wkv_forward(d["w"], d["u"], d["k"], d["v"], state_in=si, state_out=True)
    torch.cuda.synchronize()
    assert_y_close(y.cpu().numpy(), yr.cpu().numpy(), what="noalloc y vs wkv_forward")
    assert_state_close(so.cpu().numpy(), sr.cpu().numpy(), what="noalloc state vs wkv_forward")
    # and on sampled lanes against the oracle
    rng = np.random.default_rng(seed)
    w, u, k, v = (host[n].double().numpy() for n in ("w", "u", "k", "v"))
    s0 = None if state_in_host is None else state_in_host.double().numpy()
    yg = y.cpu().numpy()
    for b, c in zip(rng.integers(0, B, 8), rng.integers(0, C, 8)):
        ss = None if s0 is None else s0[:, b:b + 1, c:c + 1]
        yo, _ = oracle.forward_scan(w[c:c + 1], u[c:c + 1], k[b:b + 1, :, c:c + 1],
                                    v[b:b + 1, :, c:c + 1], state_in=ss)
        assert_y_close(yg[b, :, c], yo[0, :, 0], what=f"noalloc y lane ({b}, {c}) vs oracle")
    return so


def warm_up(lib):
    """One small call first: the first call on a device takes the array's
    address, which may load the library's code object (and with it the
    array); the calls measured below must then allocate nothing."""
    d = {n: t.cuda() for n, t in synth.make(synth.TINY, index=1).items()}
    assert wkv.wkv_forward_plan_auto(1, 64, 32)[0] == wkv.WKV_KERNEL_LOOKBACK
    y = torch.empty_like(d["k"])
    assert call_noalloc(lib, d, y, None, None, torch.cuda.current_stream()) == wkv.WKV_OK
    torch.cuda.synchronize()


def test_noalloc_forward_matches_wkv_forward_twice(lib, oracle):
    """Two calls in a row on the shared array: the look-back shape B=8 T=1024
    C=2048, then a smaller, ragged one (T=300, C=320) carrying a state."""
    warm_up(lib)
    big = synth.make(synth.GPT, index=2)
    B, T, C = 8, 1024, 2048
    assert wkv.wkv_forward_plan_auto(B, T, C)[0] == wkv.WKV_KERNEL_LOOKBACK
    assert 0 < wkv.wkv_forward_scratch_size(B, T, C) <= wkv.WKV_NOALLOC_SCRATCH_BYTES
    check_against_forward(lib, oracle, big, None, 1)
    small = synth.make(synth.GPT, index=3, B=2, T=300, C=320)
    assert wkv.wkv_forward_plan_auto(2, 300, 320)[0] == wkv.WKV_KERNEL_LOOKBACK
    pre = synth.make(synth.GPT, index=4, B=2, T=40, C=320)
    _, s0 = oracle.forward_scan(*(pre[n].double().numpy() for n in ("w", "u", "k", "v")))
    s0 = torch.from_numpy(s0.astype(np.float32))
    small["w"], small["u"] = pre["w"], pre["u"]
    check_against_forward(lib, oracle, small, s0, 2)
    assert wkv.wkv_lookback_status(torch.cuda.current_stream()) == wkv.WKV_OK


def test_noalloc_refuses_shapes_beyond_its_array(lib):
    """A look-back shape needing more scratch than the array returns
    WKV_ERR_WORKSPACE from the host check, before any launch."""
    B, T, C = 8, 16384, 2048
    need = wkv.wkv_forward_scratch_size(B, T, C)
    assert need > wkv.WKV_NOALLOC_SCRATCH_BYTES
    P = 1 << 40  # never dereferenced: nothing is launched
    args = [ctypes.c_void_p(P + i * (1 << 34)) for i in range(5)]
    st = lib.wkv_forward_noalloc(B, T, C, *args, None, None, None)
    assert st == wkv.WKV_ERR_WORKSPACE

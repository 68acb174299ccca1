"""HIP graph capture of the library's calls: every replay of a captured graph
matches the eager result (the look-back kernel, whose launches are tagged by
the host, is replaced by a stateless kernel under capture)."""
import numpy as np
import pytest
import torch

from linear_recurrent_attention_amd import synth, wkv

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no HIP device visible")
    wkv.load_library()


@pytest.mark.parametrize("shape", [(8, 1024, 2048), (1, 1024, 5120), (2, 300, 100)],
                         ids=lambda s: "x".join(map(str, s)))
def test_captured_forward_replays_match_eager(shape):
    B, T, C = shape
    dev = torch.device("cuda")
    d = synth.make(synth.GPT, index=31, B=B, T=T, C=C, device=dev)
    s0 = torch.zeros((3, B, C), device=dev)
    s0[2] = -1e38
    # eager reference (whatever kernel the plan picks outside capture)
    y_ref, s_ref = wkv.wkv_forward(d["w"], d["u"], d["k"], d["v"], state_in=s0, state_out=True)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    y = torch.empty_like(d["k"])
    so = torch.empty_like(s0)
    with torch.cuda.stream(side):
        # warm-up on the capture stream, then capture
        wkv.wkv_forward(d["w"], d["u"], d["k"], d["v"], y=y, state_in=s0, state_out=so,
                        stream=side)
    side.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        wkv.wkv_forward(d["w"], d["u"], d["k"], d["v"], y=y, state_in=s0, state_out=so,
                        stream=side)
    for rep in range(4):
        y.fill_(float("nan"))
        so.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        # eager work between replays, on the default stream
        wkv.wkv_forward(d["w"], d["u"], d["k"], d["v"], state_in=s0, state_out=True)
        torch.cuda.synchronize()
        # same arithmetic up to the kernel's rounding order: a tight bound
        yr, yg = y_ref.double().cpu().numpy(), y.double().cpu().numpy()
        assert np.all(np.isfinite(yg)), f"replay {rep}: non-finite y"
        assert np.max(np.abs(yg - yr) / (1e-5 + 1e-4 * np.abs(yr))) <= 1.0, f"replay {rep}"
        sg = so.double().cpu().numpy()
        assert np.all(np.isfinite(sg[:2])), f"replay {rep}: non-finite state"


def test_forced_lookback_is_refused_under_capture():
    dev = torch.device("cuda")
    d = synth.make(synth.TINY, index=3, B=1, T=64, C=64, device=dev)
    side = torch.cuda.Stream()
    y = torch.empty_like(d["k"])
    with torch.cuda.stream(side):
        wkv.wkv_forward(d["w"], d["u"], d["k"], d["v"], y=y, stream=side,
                        plan=(wkv.WKV_KERNEL_LOOKBACK, 4, 16))
    side.synchronize()
    g = torch.cuda.CUDAGraph()
    with pytest.raises(wkv.WkvError, match="status 6"):
        with torch.cuda.graph(g, stream=side):
            wkv.wkv_forward(d["w"], d["u"], d["k"], d["v"], y=y, stream=side,
                            plan=(wkv.WKV_KERNEL_LOOKBACK, 4, 16))

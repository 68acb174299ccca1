"""HIP graph capture of the library's calls: every replay of a captured graph
matches the eager result.  A look-back forward recorded under capture runs in
the device's fixed scratch and takes its per-launch tag on the device, so each
replay is a fresh launch; eager calls between replays (wkv_forward on its own
scratch, wkv_forward_noalloc on the same fixed array with host tags) must not
disturb it."""
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


def _close(got, ref, what):
    yr, yg = ref.double().cpu().numpy(), got.double().cpu().numpy()
    assert np.all(np.isfinite(yg)), f"{what}: non-finite"
    assert np.max(np.abs(yg - yr) / (1e-5 + 1e-4 * np.abs(yr))) <= 1.0, what


@pytest.mark.parametrize("shape", [(8, 1024, 2048), (1, 1024, 5120), (3, 300, 130)],
                         ids=lambda s: "x".join(map(str, s)))
def test_forced_lookback_under_capture_takes_device_epochs(shape):
    """A forced look-back plan recorded under capture, replayed 6 times with
    eager wkv_forward_noalloc calls (host-tagged launches on the same fixed
    array) and a carried-state chain between the replays."""
    B, T, C = shape
    dev = torch.device("cuda")
    d = synth.make(synth.GPT, index=32, B=B, T=T, C=C, device=dev)
    e = synth.make(synth.GPT, index=33, B=B, T=T, C=C, device=dev)
    plan = (wkv.WKV_KERNEL_LOOKBACK, 4, 16)
    y_ref, s_ref = wkv.wkv_forward(d["w"], d["u"], d["k"], d["v"], state_out=True, plan=plan)
    ye_ref, _ = wkv.wkv_forward(e["w"], e["u"], e["k"], e["v"], state_in=s_ref, state_out=True,
                                plan=plan)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    y, so = torch.empty_like(d["k"]), torch.empty((3, B, C), device=dev)
    ye = torch.empty_like(e["k"])

    def chain():
        wkv.wkv_forward(d["w"], d["u"], d["k"], d["v"], y=y, state_out=so, stream=side, plan=plan)
        wkv.wkv_forward(e["w"], e["u"], e["k"], e["v"], y=ye, state_in=so, stream=side, plan=plan)

    g = _capture(chain, side)
    for rep in range(6):
        y.fill_(float("nan"))
        ye.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        side.synchronize()
        _close(y, y_ref, f"replay {rep} first chunk")
        _close(ye, ye_ref, f"replay {rep} second chunk")
        # host-tagged launches on the same fixed array between replays
        yn = torch.empty_like(e["k"])
        wkv.wkv_forward_noalloc(e["w"], e["u"], e["k"], e["v"], yn)
        torch.cuda.synchronize()
    assert wkv.wkv_lookback_status(side) == wkv.WKV_OK


def test_captured_lookback_gated_bf16_with_checkpoints():
    """The training forward (gated, bf16 activations, 128-token checkpoints)
    on a forced look-back plan, recorded under capture: replays match the
    eager call within the 16-bit tolerance, checkpoints within the float one."""
    B, T, C = 4, 1000, 192
    dev = torch.device("cuda")
    d = synth.make(synth.STABILITY, index=35, B=B, T=T, C=C, device=dev)
    r = synth.receptance(synth.STABILITY, 35, (B, T, C), device=dev).to(torch.bfloat16)
    k, v = d["k"].to(torch.bfloat16), d["v"].to(torch.bfloat16)
    plan = (wkv.WKV_KERNEL_LOOKBACK, 4, 16)
    y_ref, s_ref, ck_ref = wkv.wkv_forward_checkpointed(d["w"], d["u"], k, v, r=r,
                                                        state_out=True, plan=plan)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    y, so = torch.empty_like(k), torch.empty((3, B, C), device=dev)
    ck = torch.empty_like(ck_ref)
    g = _capture(lambda: wkv.wkv_forward_checkpointed(d["w"], d["u"], k, v, r=r, y=y,
                                                       state_out=so, checkpoints=ck,
                                                       stream=side, plan=plan), side)
    # both sides rounded to bf16 once from float32 values within the float
    # tolerance of each other: at most one unit in the last place apart, which
    # is 2^-7 relative at the bottom of a binade
    h = 2.0 ** -7
    for rep in range(4):
        y.fill_(float("nan"))
        ck.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        side.synchronize()
        yr, yg = y_ref.double().cpu().numpy(), y.double().cpu().numpy()
        assert np.all(np.isfinite(yg)), f"replay {rep}: non-finite y"
        assert np.max(np.abs(yg - yr) / (1e-5 + (1e-4 + h) * np.abs(yr))) <= 1.0, f"replay {rep}"
        cr, cg = ck_ref.double().cpu().numpy(), ck.double().cpu().numpy()
        # the a, b planes at one frame (o) agree up to rounding of the frame
        m_r, m_g = cr[:, 0] / cr[:, 1], cg[:, 0] / cg[:, 1]
        assert np.max(np.abs(m_g - m_r) / (1e-5 + 1e-4 * np.abs(m_r))) <= 1.0, f"replay {rep}"


# the refused capture records nothing, and torch warns that the graph is empty
@pytest.mark.filterwarnings("ignore:The CUDA Graph is empty")
def test_oversize_lookback_under_capture():
    """A shape whose look-back scratch exceeds the fixed array: a forced
    look-back plan is refused under capture, and the automatic plan records
    the segmented kernel, whose replays match the eager (look-back) result."""
    B, T, C = 8, 16384, 2048
    need = wkv.wkv_forward_scratch_size(B, T, C)
    assert need > wkv.WKV_NOALLOC_SCRATCH_BYTES
    dev = torch.device("cuda")
    d = synth.make(synth.GPT, index=34, B=B, T=T, C=C, device=dev)
    y_ref, _ = wkv.wkv_forward(d["w"], d["u"], d["k"], d["v"])
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    y = torch.empty_like(d["k"])
    with torch.cuda.stream(side):
        wkv.wkv_forward(d["w"], d["u"], d["k"], d["v"], y=y, stream=side,
                        plan=(wkv.WKV_KERNEL_SEGMENTED, 16, 16))
    side.synchronize()
    g = torch.cuda.CUDAGraph()
    with pytest.raises(wkv.WkvError, match="status 6"):
        with torch.cuda.graph(g, stream=side):
            wkv.wkv_forward(d["w"], d["u"], d["k"], d["v"], y=y, stream=side,
                            plan=(wkv.WKV_KERNEL_LOOKBACK, 4, 32))
    g = _capture(lambda: wkv.wkv_forward(d["w"], d["u"], d["k"], d["v"], y=y, stream=side),
                 side)
    for rep in range(2):
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        side.synchronize()
        _close(y, y_ref, f"replay {rep}")


def _capture(fn, side):
    with torch.cuda.stream(side):
        fn()                       # warm-up on the capture stream
    side.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        fn()
    return g


def test_captured_time_mixing_calls_replay_exactly():
    """Token shift, gated step, typed (bf16) forward and the backward with
    carried states, captured together: each replay reproduces the eager bits
    (none of these uses state shared across launches; the forward is forced
    to the segmented kernel, which is bitwise reproducible)."""
    dev = torch.device("cuda")
    B, T, C, L = 2, 300, 128, 3
    side = torch.cuda.Stream()
    mu, x, xp = (t.to(dev) for t in synth.shift_inputs(synth.GPT, 90, B, T, C, 3))
    d = synth.make(synth.STABILITY, index=91, B=B, T=T, C=C, device=dev, with_dy=True)
    r16 = synth.receptance(synth.GPT, 91, (B, T, C), device=dev).to(torch.bfloat16)
    k16, v16 = d["k"].to(torch.bfloat16), d["v"].to(torch.bfloat16)
    wl = torch.stack([d["w"]] * L)
    ul = torch.stack([d["u"]] * L)
    ks, vs = synth.sequence(synth.DECODE, 92, (L, B, C), device=dev)
    rs = synth.receptance(synth.DECODE, 92, (L, B, C), device=dev)
    st0 = torch.zeros((L, 3, B, C), device=dev)
    st0[:, 2] = -1e38
    s_in = torch.zeros((3, B, C), device=dev)
    s_in[1] = 1.0
    s_in[2] = 0.5
    s_out = torch.zeros((3, B, C), device=dev)
    s_out[1] = 2.0
    s_out[2] = 3.0
    g_out = synth.normal((3, B, C), 1.0, synth.seed_of(synth.GPT, 93, 0), device=dev)
    ws = torch.empty(wkv.wkv_backward_workspace_size(B, T, C), device=dev, dtype=torch.uint8)
    outs = dict(sh=torch.empty((3, B, T, C), device=dev), xl=torch.empty((B, C), device=dev),
                ys=torch.empty((L, B, C), device=dev), st=torch.empty_like(st0),
                y16=torch.empty_like(k16), dk=torch.empty_like(d["k"]),
                dv=torch.empty_like(d["k"]), dw=torch.empty(C, device=dev),
                du=torch.empty(C, device=dev), dsi=torch.empty((3, B, C), device=dev))

    def work(stream):
        wkv.wkv_token_shift(mu, x, xp, out=outs["sh"], x_prev_out=outs["xl"], stream=stream)
        wkv.wkv_step_gated(wl, ul, ks, vs, rs, st0, state_out=outs["st"], y=outs["ys"],
                           stream=stream)
        wkv.wkv_forward_typed(d["w"], d["u"], k16, v16, r16, y=outs["y16"], stream=stream,
                              plan=(wkv.WKV_KERNEL_SEGMENTED, 16, 16))
        wkv.wkv_backward_state(d["w"], d["u"], d["k"], d["v"], d["dy"], state_in=s_in,
                               state_out=s_out, d_state_out=g_out, dk=outs["dk"], dv=outs["dv"],
                               dw=outs["dw"], du=outs["du"], d_state_in=outs["dsi"],
                               workspace=ws, stream=stream)

    work(torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref = {n: t.clone() for n, t in outs.items()}
    g = _capture(lambda: work(side), side)
    for rep in range(4):
        for t in outs.values():
            t.fill_(float("nan")) if t.is_floating_point() else t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        work(torch.cuda.current_stream())       # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n, t in outs.items():
            assert torch.equal(t, ref[n]), f"replay {rep}: {n} differs from the eager result"


def test_captured_training_path_replays_exactly():
    """The forward that writes its 128-token checkpoints, the backward that
    starts from them (plain and gated) and the token shift's backward, captured
    together: every replay reproduces the eager bits (the segmented forward and
    every backward are bitwise reproducible)."""
    dev = torch.device("cuda")
    B, T, C = 2, 700, 96
    side = torch.cuda.Stream()
    d = synth.make(synth.STABILITY, index=94, B=B, T=T, C=C, device=dev, with_dy=True)
    ws = torch.empty(wkv.wkv_backward_workspace_size(B, T, C), device=dev, dtype=torch.uint8)
    r = synth.receptance(synth.STABILITY, 94, (B, T, C), device=dev)
    mu, x, xp = (t.to(dev) for t in synth.shift_inputs(synth.GPT, 95, B, T, C, 3))
    d_mix = synth.normal((3, B, T, C), 1.0, synth.seed_of(synth.GPT, 96, 0), device=dev)
    d_xpo = synth.normal((B, C), 1.0, synth.seed_of(synth.GPT, 97, 0), device=dev)
    ws_shift = torch.empty(max(1, int(wkv.load_library().wkv_token_shift_backward_workspace_size(
        B, T, C, 3))), device=dev, dtype=torch.uint8)
    outs = dict(y=torch.empty_like(d["k"]), so=torch.empty((3, B, C), device=dev),
                ck=torch.empty((wkv.checkpoint_count(T), 3, B, C), device=dev),
                dk=torch.empty_like(d["k"]), dv=torch.empty_like(d["k"]),
                dw=torch.empty(C, device=dev), du=torch.empty(C, device=dev),
                gdk=torch.empty_like(d["k"]), gdv=torch.empty_like(d["k"]),
                gdr=torch.empty_like(d["k"]), gdw=torch.empty(C, device=dev),
                gdu=torch.empty(C, device=dev), sdx=torch.empty_like(x),
                sdxp=torch.empty((B, C), device=dev), sdmu=torch.empty((3, C), device=dev))

    def work(stream):
        wkv.wkv_forward_checkpointed(d["w"], d["u"], d["k"], d["v"], y=outs["y"],
                                     state_out=outs["so"], checkpoints=outs["ck"], stream=stream,
                                     plan=(wkv.WKV_KERNEL_SEGMENTED, 16, 16))
        wkv.wkv_backward_checkpointed(d["w"], d["u"], d["k"], d["v"], d["dy"], outs["ck"],
                                      dk=outs["dk"], dv=outs["dv"], dw=outs["dw"], du=outs["du"],
                                      workspace=ws, stream=stream)
        wkv.wkv_backward_gated(d["w"], d["u"], d["k"], d["v"], r, d["dy"], checkpoints=outs["ck"],
                               dk=outs["gdk"], dv=outs["gdv"], dr=outs["gdr"], dw=outs["gdw"],
                               du=outs["gdu"], workspace=ws, stream=stream)
        wkv.wkv_token_shift_backward(mu, x, d_mix, x_prev=xp, d_x_prev_out=d_xpo, dx=outs["sdx"],
                                     d_x_prev=outs["sdxp"], dmu=outs["sdmu"], workspace=ws_shift,
                                     stream=stream)

    work(torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref = {n: t.clone() for n, t in outs.items()}
    g = _capture(lambda: work(side), side)
    for rep in range(4):
        for t in outs.values():
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        work(torch.cuda.current_stream())       # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n, t in outs.items():
            assert torch.equal(t, ref[n]), f"replay {rep}: {n} differs from the eager result"

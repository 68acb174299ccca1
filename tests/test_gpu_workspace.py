"""Every entry point that takes a caller workspace, run twice on the same
inputs: once with the workspace and every output buffer filled with NaN
bytes (0xFF), once with both zero-filled.  An output that depends on scratch
the call never wrote, or an output element the call never writes, shows as a
difference between the two runs (NaN is not equal to itself, and a NaN or a
zero left in an output differs from the value written in the other run).
The plain backward's and the token shift's first runs are also held to the
oracle, so that both runs being wrong the same way does not pass there; the
other entry points' values are checked against the oracle in their own tests.

Workspaces are sized exactly as the size query says (no slack).
"""
import sys

import numpy as np
import pytest
import torch

from linear_recurrent_attention_amd import synth, wkv
from parity import assert_grad_close, f64, roundoff_floor

pytestmark = pytest.mark.gpu

SHAPES = [(1, 1, 5), (2, 129, 70), (3, 300, 100), (1, 1025, 64)]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no HIP device visible")
    wkv.load_library()


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def filled(shape, dtype, nan: bool):
    """A device tensor of `shape`, every byte 0xFF (NaN in every float format)
    or 0x00."""
    t = torch.empty(shape, device="cuda", dtype=dtype)
    t.view(torch.uint8).fill_(0xFF if nan else 0x00)
    return t


def ws(nbytes, nan):
    return filled((max(int(nbytes), 1),), torch.uint8, nan)


def same(a, b, what):
    """Bitwise equal and free of NaN (every element written, no NaN read)."""
    assert a.shape == b.shape, what
    assert not torch.isnan(a.float()).any().item(), f"{what}: NaN in the output"
    assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), \
        f"{what}: differs between NaN- and zero-filled workspace"


def runs(fn):
    """fn(nan) -> tuple of output tensors; returns both runs' outputs."""
    out = [fn(True), fn(False)]
    torch.cuda.synchronize()
    return out


def inputs(shape, dt=torch.float32, index=200):
    B, T, C = shape
    d = synth.make(synth.STABILITY, index=index, B=B, T=T, C=C, with_dy=True)
    dev = {n: (t.to(dt) if n in ("k", "v", "dy") else t).cuda() for n, t in d.items()}
    return d, dev


def reachable_state(oracle, B, C, index):
    p = synth.make(synth.TINY, index=index, B=B, T=11, C=C)
    _, s = oracle.forward_scan(*(f64(p[n]) for n in ("w", "u", "k", "v")))
    return s.astype(np.float32).astype(np.float64)


def dev32(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_backward(oracle, shape):
    B, T, C = shape
    d, g = inputs(shape)
    need = wkv.wkv_backward_workspace_size(B, T, C)
    note(f"workspace wkv_backward {shape}: {need} B")

    def call(nan):
        outs = dict(dk=filled((B, T, C), torch.float32, nan),
                    dv=filled((B, T, C), torch.float32, nan),
                    dw=filled((C,), torch.float32, nan), du=filled((C,), torch.float32, nan))
        return wkv.wkv_backward(g["w"], g["u"], g["k"], g["v"], g["dy"], workspace=ws(need, nan),
                                **outs)

    a, b = runs(call)
    for name, x, y in zip(("dk", "dv", "dw", "du"), a, b):
        same(x, y, f"{shape} {name}")
    r = oracle.backward_scan(*(f64(d[n]) for n in ("w", "u", "k", "v", "dy")))
    f = roundoff_floor(f64(d["dy"]), f64(d["v"]))
    assert_grad_close(f64(a[1]), r[1], "dv", f)


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_backward_with_states(oracle, shape, dt):
    """wkv_backward_typed with a carried state, an upstream state gradient and
    d_state_in."""
    B, T, C = shape
    d, g = inputs(shape, dt, 201)
    s_in = reachable_state(oracle, B, C, 202)
    _, s_out = oracle.forward_scan(*(f64(d[n]) for n in ("w", "u", "k", "v")), s_in)
    g_out = synth.normal((3, B, C), 1.0, synth.seed_of(synth.GPT, 9900, 0)).cuda()
    si, so = dev32(s_in), dev32(s_out)
    need = wkv.wkv_backward_workspace_size(B, T, C)
    note(f"workspace wkv_backward_typed {dt} {shape}")

    def call(nan):
        outs = dict(dk=filled((B, T, C), dt, nan), dv=filled((B, T, C), dt, nan),
                    dw=filled((C,), torch.float32, nan), du=filled((C,), torch.float32, nan),
                    d_state_in=filled((3, B, C), torch.float32, nan))
        return wkv.wkv_backward_typed(g["w"], g["u"], g["k"], g["v"], g["dy"], state_in=si,
                                      state_out=so, d_state_out=g_out, workspace=ws(need, nan),
                                      **outs)

    a, b = runs(call)
    for name, x, y in zip(("dk", "dv", "dw", "du", "d_state_in"), a, b):
        same(x, y, f"{shape} {name}")


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("checkpoints", [False, True], ids=["first_pass", "checkpoints"])
def test_backward_gated(oracle, shape, checkpoints):
    B, T, C = shape
    d, g = inputs(shape, index=203)
    r = synth.receptance(synth.STABILITY, 203, (B, T, C)).cuda()
    ck = None
    if checkpoints:
        _, _, ck = wkv.wkv_forward_checkpointed(g["w"], g["u"], g["k"], g["v"], r=r)
    need = wkv.wkv_backward_workspace_size(B, T, C)
    note(f"workspace wkv_backward_gated {shape} checkpoints={checkpoints}")

    def call(nan):
        outs = dict(dk=filled((B, T, C), torch.float32, nan),
                    dv=filled((B, T, C), torch.float32, nan),
                    dr=filled((B, T, C), torch.float32, nan),
                    dw=filled((C,), torch.float32, nan), du=filled((C,), torch.float32, nan))
        return wkv.wkv_backward_gated(g["w"], g["u"], g["k"], g["v"], r, g["dy"],
                                      checkpoints=ck, workspace=ws(need, nan), **outs)

    a, b = runs(call)
    for name, x, y in zip(("dk", "dv", "dr", "dw", "du"), a[:5], b[:5]):
        same(x, y, f"{shape} {name}")


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_token_shift_backward(oracle, shape, dt):
    B, T, C = shape
    M = 3
    mu, x, xp = synth.shift_inputs(synth.GPT, 204, B, T, C, M)
    d_out = synth.normal((M, B, T, C), 1.0, synth.seed_of(synth.GPT, 9901, 0))
    d_xp_out = synth.normal((B, C), 1.0, synth.seed_of(synth.GPT, 9902, 0))
    mu, x, xp, d_out, d_xp_out = mu.cuda(), x.to(dt).cuda(), xp.to(dt).cuda(), \
        d_out.to(dt).cuda(), d_xp_out.to(dt).cuda()
    need = int(wkv.load_library().wkv_token_shift_backward_workspace_size(B, T, C, M))
    note(f"workspace wkv_token_shift_backward {dt} {shape}: {need} B")

    def call(nan):
        outs = dict(dx=filled((B, T, C), dt, nan), d_x_prev=filled((B, C), dt, nan),
                    dmu=filled((M, C), torch.float32, nan))
        return wkv.wkv_token_shift_backward(mu, x, d_out, x_prev=xp, d_x_prev_out=d_xp_out,
                                            workspace=ws(need, nan), **outs)

    a, b = runs(call)
    for name, p, q in zip(("dx", "d_x_prev", "dmu"), a, b):
        same(p, q, f"{shape} {name}")
    # dmu against the oracle on the values the GPU consumed, within 1e-4 of
    # the sum of its terms' sizes |d| (|x_t| + |x_{t-1}|)
    x64, xp64, d64 = f64(x), f64(xp), f64(d_out)
    _, _, dmu = oracle.token_shift_backward(f64(mu), x64, xp64, d64, f64(d_xp_out))
    prev = np.concatenate([xp64[:, None, :], x64[:, :-1, :]], axis=1)
    mag = np.sum(np.abs(d64) * (np.abs(x64) + np.abs(prev))[None], axis=(1, 2))
    assert np.all(np.abs(f64(a[2]) - dmu) <= 1e-4 * mag + 1e-30)

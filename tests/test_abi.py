"""CPU-only checks of the C ABI: the library loads, exports every entry point the
header declares, and rejects invalid arguments with the documented status
before touching the HIP runtime.  No call here reaches a kernel launch: every
argument set is invalid, so the host checks return first."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wkv.h")
LIB = os.environ.get("WKV_ABI_TEST_LIB") or os.path.join(ROOT, "linear_recurrent_attention_amd", "libwkv.so")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from linear_recurrent_attention_amd import build
        build.build()
    from linear_recurrent_attention_amd import wkv
    return wkv.load_library(LIB)


def declared_entry_points():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"WKV_API\s+[\w\s\*]*?\b(wkv_\w+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared_entry_points()
    for n in ("wkv_forward", "wkv_step", "wkv_backward", "wkv_backward_workspace_size",
              "wkv_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\sT\s+(\w+)$", out, flags=re.M))
    for n in declared_entry_points():
        assert n in exported, n
        assert getattr(lib, n) is not None
    from linear_recurrent_attention_amd import wkv
    assert set(wkv.EXPORTED) == set(declared_entry_points())


def test_status_strings(lib):
    from linear_recurrent_attention_amd import wkv
    seen = set()
    for s in range(9):
        txt = wkv.wkv_status_string(s)
        assert txt and txt not in seen
        seen.add(txt)
    assert wkv.wkv_status_string(99) == "unknown status"


# Fake, never dereferenced device addresses for the validation paths.
P = 1 << 40


def fwd(lib, B, T, C, w=P, u=P + 0x1000, k=P + 0x100000, v=P + 0x10000000, y=P + 0x20000000,
        si=None, so=None):
    vp = ctypes.c_void_p
    return lib.wkv_forward(B, T, C, vp(w) if w else None, vp(u) if u else None,
                           vp(k) if k else None, vp(v) if v else None, vp(y) if y else None,
                           vp(si) if si else None, vp(so) if so else None, None)


def test_forward_rejects_invalid_arguments(lib):
    from linear_recurrent_attention_amd import wkv as W
    assert fwd(lib, -1, 4, 4) == W.WKV_ERR_DIM
    assert fwd(lib, 4, -1, 4) == W.WKV_ERR_DIM
    assert fwd(lib, 4, 4, -2) == W.WKV_ERR_DIM
    assert fwd(lib, 1 << 30, 1 << 20, 1 << 20) == W.WKV_ERR_OVERFLOW
    assert fwd(lib, 2, 8, 16, k=None) == W.WKV_ERR_NULL
    assert fwd(lib, 2, 8, 16, y=None) == W.WKV_ERR_NULL
    assert fwd(lib, 2, 8, 16, w=None) == W.WKV_ERR_NULL
    # y overlapping k, v, w, a state buffer
    assert fwd(lib, 2, 8, 16, y=P + 0x100000 + 64) == W.WKV_ERR_ALIAS
    assert fwd(lib, 2, 8, 16, y=P + 0x10000000) == W.WKV_ERR_ALIAS
    assert fwd(lib, 2, 8, 16, y=P - 16) == W.WKV_ERR_ALIAS
    assert fwd(lib, 2, 8, 16, si=P + 0x20000000 + 8) == W.WKV_ERR_ALIAS
    # state_out partially overlapping state_in, or overlapping an input
    si = P + 0x30000000
    assert fwd(lib, 2, 8, 16, si=si, so=si + 4) == W.WKV_ERR_ALIAS
    assert fwd(lib, 2, 8, 16, so=P + 0x100000) == W.WKV_ERR_ALIAS


def test_step_rejects_invalid_arguments(lib):
    from linear_recurrent_attention_amd import wkv as W
    vp = ctypes.c_void_p
    base = [vp(P), vp(P + 0x1000), vp(P + 0x100000), vp(P + 0x200000), vp(P + 0x300000)]
    si, so = vp(P + 0x400000), vp(P + 0x400000)
    assert lib.wkv_step(-1, 2, 4, *base, si, so, None) == W.WKV_ERR_DIM
    assert lib.wkv_step(2, 2, 4, *base, None, so, None) == W.WKV_ERR_NULL
    assert lib.wkv_step(2, 2, 4, *base, si, vp(P + 0x400000 + 4), None) == W.WKV_ERR_ALIAS
    assert lib.wkv_step(2, 2, 4, *base[:4], vp(P + 0x100000), si, so, None) == W.WKV_ERR_ALIAS
    assert lib.wkv_step(1 << 40, 1 << 20, 1 << 10, *base, si, so, None) == W.WKV_ERR_OVERFLOW


def test_backward_workspace_and_checks(lib):
    from linear_recurrent_attention_amd import wkv as W
    assert lib.wkv_backward_workspace_size(0, 10, 10) == 0
    assert lib.wkv_backward_workspace_size(-1, 10, 10) == 0
    need = lib.wkv_backward_workspace_size(8, 4096, 2048)
    assert need > 2 * 8 * 2048 * 8
    assert lib.wkv_backward_workspace_size(8, 4097, 2048) > need   # one more tile
    vp = ctypes.c_void_p
    ins = [vp(P + i * 0x10000000) for i in range(5)]           # w u k v dy
    outs = [vp(P + (8 + i) * 0x10000000) for i in range(4)]    # dk dv dw du
    ws = vp(P + 16 * 0x10000000)
    n = lib.wkv_backward_workspace_size(2, 64, 32)
    assert lib.wkv_backward(2, 64, 32, *ins, *outs, ws, n - 1, None) == W.WKV_ERR_WORKSPACE
    assert lib.wkv_backward(2, 64, 32, *ins, *outs, None, n, None) == W.WKV_ERR_WORKSPACE
    bad = list(outs)
    bad[0] = ins[2]                                            # dk == k
    assert lib.wkv_backward(2, 64, 32, *ins, *bad, ws, n, None) == W.WKV_ERR_ALIAS
    bad = list(outs)
    bad[3] = vp(P + 9 * 0x10000000 + 4)                        # du inside dv
    assert lib.wkv_backward(2, 64, 32, *ins, *bad, ws, n, None) == W.WKV_ERR_ALIAS
    assert lib.wkv_backward(2, 64, 32, *ins, *outs, outs[1], n, None) == W.WKV_ERR_ALIAS
    assert lib.wkv_backward(-2, 64, 32, *ins, *outs, ws, n, None) == W.WKV_ERR_DIM
    assert lib.wkv_backward(2, 64, 32, *ins[:4], None, *outs, ws, n, None) == W.WKV_ERR_NULL


def test_backward_state_checks(lib):
    from linear_recurrent_attention_amd import wkv as W
    vp = ctypes.c_void_p
    ins = [vp(P + i * 0x10000000) for i in range(5)]           # w u k v dy
    si, so, dso = (vp(P + (20 + i) * 0x10000000) for i in range(3))
    outs = [vp(P + (8 + i) * 0x10000000) for i in range(4)]    # dk dv dw du
    dsi = vp(P + 24 * 0x10000000)
    ws = vp(P + 16 * 0x10000000)
    n = lib.wkv_backward_workspace_size(2, 64, 32)
    f = lib.wkv_backward_state
    assert f(2, 64, 32, *ins, si, None, dso, *outs, dsi, ws, n, None) == W.WKV_ERR_NULL
    assert f(2, 64, 32, *ins, si, so, dso, *outs, si, ws, n, None) == W.WKV_ERR_ALIAS
    assert f(2, 64, 32, *ins, si, so, dso, *outs, vp(P + 22 * 0x10000000 + 8), ws, n,
             None) == W.WKV_ERR_ALIAS                           # partly over d_state_out
    assert f(2, 64, 32, *ins, si, so, dso, *outs, outs[0], ws, n, None) == W.WKV_ERR_ALIAS
    assert f(2, 64, 32, *ins, si, so, dso, *outs, dsi, ws, n - 1, None) == W.WKV_ERR_WORKSPACE
    assert f(-1, 64, 32, *ins, si, so, dso, *outs, dsi, ws, n, None) == W.WKV_ERR_DIM


def test_backward_typed_checks(lib):
    from linear_recurrent_attention_amd import wkv as W
    vp = ctypes.c_void_p
    ins = [vp(P + i * 0x10000000) for i in range(5)]           # w u k v dy
    outs = [vp(P + (8 + i) * 0x10000000) for i in range(4)]    # dk dv dw du
    ws = vp(P + 16 * 0x10000000)
    n = lib.wkv_backward_workspace_size(2, 64, 32)
    f = lib.wkv_backward_typed
    assert f(2, 64, 32, 9, *ins, None, None, None, *outs, None, ws, n, None) == \
        W.WKV_ERR_UNSUPPORTED
    # 2 x 64 x 32 bf16 elements are 8 KiB: dk 6 KiB into k overlaps it
    bad = list(outs)
    bad[0] = vp(P + 2 * 0x10000000 + 6144)
    assert f(2, 64, 32, W.WKV_DTYPE_BF16, *ins, None, None, None, *bad, None, ws, n,
             None) == W.WKV_ERR_ALIAS
    assert f(2, 64, 32, W.WKV_DTYPE_F16, *ins[:4], None, None, None, None, *outs, None, ws, n,
             None) == W.WKV_ERR_NULL


def test_checkpoint_count_matches_the_header():
    from linear_recurrent_attention_amd import wkv as W
    src = open(HEADER).read()
    m = re.search(r"#define WKV_CHECKPOINT_TOKENS (\d+)", src)
    assert m and int(m.group(1)) == W.WKV_CHECKPOINT_TOKENS == 128
    # one checkpoint before every multiple of 128 strictly inside the sequence
    for T, n in ((0, 0), (1, 0), (127, 0), (128, 0), (129, 1), (256, 1), (257, 2), (4096, 31),
                 (1024, 7)):
        assert W.checkpoint_count(T) == n, T


def test_checkpointed_calls_reject_invalid_arguments(lib):
    from linear_recurrent_attention_amd import wkv as W
    vp = ctypes.c_void_p
    w, u, k, v = vp(P), vp(P + 0x1000), vp(P + 0x100000), vp(P + 0x10000000)
    y, ck = vp(P + 0x20000000), vp(P + 0x40000000)
    f = lib.wkv_forward_checkpointed
    # B=2 T=300 C=16: two checkpoints, 2 x 3 x 2 x 16 floats = 768 bytes
    assert f(2, 300, 16, W.WKV_DTYPE_F32, w, u, k, v, None, y, None, None, None, None,
             None) == W.WKV_ERR_NULL
    assert f(2, 300, 16, 5, w, u, k, v, None, y, None, None, ck, None, None) == \
        W.WKV_ERR_UNSUPPORTED
    assert f(-2, 300, 16, W.WKV_DTYPE_F32, w, u, k, v, None, y, None, None, ck, None,
             None) == W.WKV_ERR_DIM
    assert f(2, 300, 16, W.WKV_DTYPE_F32, w, u, k, v, None, y, None, None,
             vp(P + 0x20000000 + 4), None, None) == W.WKV_ERR_ALIAS      # on y
    assert f(2, 300, 16, W.WKV_DTYPE_F32, w, u, k, v, None, y, None, vp(P + 0x40000000 + 764),
             ck, None, None) == W.WKV_ERR_ALIAS                           # state_out on its end
    assert f(2, 300, 16, W.WKV_DTYPE_BF16, w, u, k, v, vp(P + 0x30000000), y, None, None,
             vp(P + 0x30000000 + 8), None, None) == W.WKV_ERR_ALIAS      # on r
    p = W.ForwardPlan(W.WKV_KERNEL_SEGMENTED, 3, 16, 0)
    assert f(2, 300, 16, W.WKV_DTYPE_F32, w, u, k, v, None, y, None, None, ck, ctypes.byref(p),
             None) == W.WKV_ERR_UNSUPPORTED
    ins = [vp(P + i * 0x10000000) for i in range(5)]           # w u k v dy
    outs = [vp(P + (8 + i) * 0x10000000) for i in range(4)]    # dk dv dw du
    ws = vp(P + 16 * 0x10000000)
    n = lib.wkv_backward_workspace_size(2, 300, 16)
    g = lib.wkv_backward_checkpointed
    assert g(2, 300, 16, W.WKV_DTYPE_F32, *ins, None, None, None, None, *outs, None, ws, n,
             None) == W.WKV_ERR_NULL                              # checkpoints missing
    assert g(2, 300, 16, 9, *ins, None, ck, None, None, *outs, None, ws, n, None) == \
        W.WKV_ERR_UNSUPPORTED
    bad = list(outs)
    bad[1] = vp(P + 0x40000000 + 512)                          # dv over the checkpoints
    assert g(2, 300, 16, W.WKV_DTYPE_F32, *ins, None, ck, None, None, *bad, None, ws, n,
             None) == W.WKV_ERR_ALIAS
    assert g(2, 300, 16, W.WKV_DTYPE_F32, *ins, None, ck, None, None, *outs,
             vp(P + 0x40000000 + 8), ws, n, None) == W.WKV_ERR_ALIAS    # d_state_in on them
    assert g(2, 300, 16, W.WKV_DTYPE_F32, *ins, None, ck, None, None, *outs, None, ck, n,
             None) == W.WKV_ERR_ALIAS                             # workspace on them
    assert g(2, 300, 16, W.WKV_DTYPE_F32, *ins, None, ck, None, None, *outs, None, ws, n - 1,
             None) == W.WKV_ERR_WORKSPACE


def test_gated_backward_rejects_invalid_arguments(lib):
    from linear_recurrent_attention_amd import wkv as W
    vp = ctypes.c_void_p
    w, u, k, v = (vp(P + i * 0x10000000) for i in range(4))
    dy, r = vp(P + 4 * 0x10000000), vp(P + 5 * 0x10000000)
    dk, dv, dw, du = (vp(P + (8 + i) * 0x10000000) for i in range(4))
    dr, ws = vp(P + 12 * 0x10000000), vp(P + 16 * 0x10000000)
    n = lib.wkv_backward_workspace_size(2, 300, 16)
    g = lib.wkv_backward_gated
    ok = [w, u, k, v, r, dy, None, None, None, None, dk, dv, dr, dw, du, None, ws, n, None]

    def call(dtype=W.WKV_DTYPE_F32, **over):
        args = list(ok)
        names = ["w", "u", "k", "v", "r", "dy", "si", "ck", "so", "dso", "dk", "dv", "dr", "dw",
                 "du", "dsi", "ws", "n", "stream"]
        for key, val in over.items():
            args[names.index(key)] = val
        return g(2, 300, 16, dtype, *args)

    assert call(r=None) == W.WKV_ERR_NULL
    assert call(dr=None) == W.WKV_ERR_NULL
    assert call(dtype=7) == W.WKV_ERR_UNSUPPORTED
    assert call(dr=vp(P + 5 * 0x10000000 + 64)) == W.WKV_ERR_ALIAS      # dr over r
    assert call(dr=vp(P + 8 * 0x10000000 + 64)) == W.WKV_ERR_ALIAS      # dr over dk
    assert call(dk=vp(P + 5 * 0x10000000 + 4)) == W.WKV_ERR_ALIAS       # dk over r
    assert call(n=n - 1) == W.WKV_ERR_WORKSPACE
    assert call(ck=vp(P + 12 * 0x10000000 + 256)) == W.WKV_ERR_ALIAS    # checkpoints under dr


def test_token_shift_backward_rejects_invalid_arguments(lib):
    from linear_recurrent_attention_amd import wkv as W
    vp = ctypes.c_void_p
    B, T, C, M = 2, 100, 64, 3
    need = lib.wkv_token_shift_backward_workspace_size(B, T, C, M)
    assert need == 2 * 1 * 3 * 64 * 4                      # one 256-token tile per sequence
    assert lib.wkv_token_shift_backward_workspace_size(B, 0, C, M) == 0
    assert lib.wkv_token_shift_backward_workspace_size(B, T, C, 9) == 0
    mu, x, xp, d, dxpo = (vp(P + i * 0x10000000) for i in range(5))
    dx, dxp, dmu, ws = (vp(P + (8 + i) * 0x10000000) for i in range(4))
    f = lib.wkv_token_shift_backward
    ok = [B, T, C, M, mu, x, xp, d, dxpo, dx, dxp, dmu, ws, need, None]

    def call(**over):
        names = ["B", "T", "C", "M", "mu", "x", "xp", "d", "dxpo", "dx", "dxp", "dmu", "ws", "n",
                 "stream"]
        args = list(ok)
        for key, val in over.items():
            args[names.index(key)] = val
        return f(*args)

    assert call(B=-1) == W.WKV_ERR_DIM
    assert call(M=9) == W.WKV_ERR_UNSUPPORTED
    assert call(x=None) == W.WKV_ERR_NULL
    assert call(d=None) == W.WKV_ERR_NULL
    assert call(dmu=None) == W.WKV_ERR_NULL
    assert call(n=need - 1) == W.WKV_ERR_WORKSPACE
    assert call(ws=None) == W.WKV_ERR_WORKSPACE
    assert call(dx=vp(P + 1 * 0x10000000 + 128)) == W.WKV_ERR_ALIAS      # dx over x
    assert call(dmu=vp(P + 8 * 0x10000000 + 64)) == W.WKV_ERR_ALIAS      # dmu over dx
    assert call(dxp=vp(P + 4 * 0x10000000)) == W.WKV_ERR_ALIAS           # d_x_prev on d_x_prev_out
    assert call(ws=vp(P + 3 * 0x10000000 + 4)) == W.WKV_ERR_ALIAS        # workspace over d_out


def test_typed_token_shift_calls_reject_invalid_arguments(lib):
    from linear_recurrent_attention_amd import wkv as W
    vp = ctypes.c_void_p
    mu, x, xp, out, xpo = (vp(P + i * 0x10000000) for i in range(5))
    f = lib.wkv_token_shift_typed
    assert f(2, 8, 16, 3, 7, mu, x, xp, out, xpo, None) == W.WKV_ERR_UNSUPPORTED
    assert f(2, 8, 16, 9, W.WKV_DTYPE_BF16, mu, x, xp, out, xpo, None) == W.WKV_ERR_UNSUPPORTED
    assert f(2, 8, 16, 3, W.WKV_DTYPE_BF16, mu, None, xp, out, xpo, None) == W.WKV_ERR_NULL
    # 2 x 8 x 16 bf16 elements are 512 bytes: out 500 bytes into x overlaps it
    assert f(2, 8, 16, 3, W.WKV_DTYPE_BF16, mu, x, xp, vp(P + 0x10000000 + 500), xpo,
             None) == W.WKV_ERR_ALIAS
    # the carried token is 2 x 16 bf16 = 64 bytes: x_prev_out 32 bytes into x_prev
    assert f(2, 8, 16, 3, W.WKV_DTYPE_F16, mu, x, xp, out, vp(P + 2 * 0x10000000 + 32),
             None) == W.WKV_ERR_ALIAS
    g = lib.wkv_token_shift_backward_typed
    need = lib.wkv_token_shift_backward_workspace_size(2, 100, 64, 3)
    d, dxpo, dx, dxp, dmu, ws = (vp(P + (5 + i) * 0x10000000) for i in range(6))
    assert g(2, 100, 64, 3, 4, mu, x, xp, d, dxpo, dx, dxp, dmu, ws, need, None) == \
        W.WKV_ERR_UNSUPPORTED
    # dx 2 x 100 x 64 bf16 = 25,600 bytes: x placed just below dx overlaps it
    assert g(2, 100, 64, 3, W.WKV_DTYPE_BF16, mu, vp(P + 7 * 0x10000000 - 25000), xp, d, dxpo,
             dx, dxp, dmu, ws, need, None) == W.WKV_ERR_ALIAS
    assert g(2, 100, 64, 3, W.WKV_DTYPE_BF16, mu, x, xp, d, dxpo, dx, dxp, dmu, ws, need - 1,
             None) == W.WKV_ERR_WORKSPACE


def test_forward_ex_rejects_unknown_plans(lib):
    from linear_recurrent_attention_amd import wkv as W
    vp = ctypes.c_void_p
    args = [2, 8, 16, vp(P), vp(P + 0x1000), vp(P + 0x100000), vp(P + 0x10000000),
            vp(P + 0x20000000), None, None]
    for plan in ((9, 0, 0, 0), (W.WKV_KERNEL_SEGMENTED, 3, 16, 0),
                 (W.WKV_KERNEL_SEGMENTED, 16, 7, 0), (W.WKV_KERNEL_LANE, 0, 0, 32),
                 (W.WKV_KERNEL_SEGMENTED, 16, 16, 48), (W.WKV_KERNEL_LOOKBACK, 4, 16, 32)):
        p = W.ForwardPlan(*plan)
        assert lib.wkv_forward_ex(*args, ctypes.byref(p), None) == W.WKV_ERR_UNSUPPORTED


def test_gated_calls_reject_invalid_arguments(lib):
    from linear_recurrent_attention_amd import wkv as W
    vp = ctypes.c_void_p
    w, u, k, v = vp(P), vp(P + 0x1000), vp(P + 0x100000), vp(P + 0x10000000)
    r, y = vp(P + 0x30000000), vp(P + 0x20000000)
    g = lib.wkv_forward_gated
    assert g(-1, 8, 16, w, u, k, v, r, y, None, None, None, None) == W.WKV_ERR_DIM
    assert g(2, 8, 16, w, u, k, v, None, y, None, None, None, None) == W.WKV_ERR_NULL
    assert g(2, 8, 16, w, u, k, v, vp(P + 0x20000000 + 4), y, None, None, None,
             None) == W.WKV_ERR_ALIAS                                   # r overlaps y
    assert g(2, 8, 16, w, u, k, v, r, y, None, vp(P + 0x30000000), None,
             None) == W.WKV_ERR_ALIAS                                   # state_out on r
    # the gated look-back kernel exists only for segments of <= 16 tokens
    p = W.ForwardPlan(W.WKV_KERNEL_LOOKBACK, 4, 32, 64)
    assert g(2, 8, 16, w, u, k, v, r, y, None, None, ctypes.byref(p), None) == \
        W.WKV_ERR_UNSUPPORTED
    p = W.ForwardPlan(W.WKV_KERNEL_LOOKBACK, 4, 16, 32)
    assert g(2, 8, 16, w, u, k, v, r, y, None, None, ctypes.byref(p), None) == \
        W.WKV_ERR_UNSUPPORTED
    si, so = vp(P + 0x400000), vp(P + 0x400000)
    base = [vp(P), vp(P + 0x1000), vp(P + 0x100000), vp(P + 0x200000)]
    sg = lib.wkv_step_gated
    assert sg(2, 2, 4, *base, None, vp(P + 0x300000), si, so, None) == W.WKV_ERR_NULL
    assert sg(2, 2, 4, *base, vp(P + 0x300000), vp(P + 0x300000 + 8), si, so,
              None) == W.WKV_ERR_ALIAS
    assert sg(-2, 2, 4, *base, vp(P + 0x500000), vp(P + 0x300000), si, so, None) == W.WKV_ERR_DIM


def test_typed_calls_reject_invalid_arguments(lib):
    from linear_recurrent_attention_amd import wkv as W
    vp = ctypes.c_void_p
    w, u, k, v = vp(P), vp(P + 0x1000), vp(P + 0x100000), vp(P + 0x10000000)
    y = vp(P + 0x20000000)
    f = lib.wkv_forward_typed
    assert f(2, 8, 16, 7, w, u, k, v, None, y, None, None, None, None) == W.WKV_ERR_UNSUPPORTED
    assert f(2, 8, 16, W.WKV_DTYPE_BF16, w, u, None, v, None, y, None, None, None,
             None) == W.WKV_ERR_NULL
    # 2 x 8 x 16 bf16 elements are 512 bytes: y 300 bytes into k overlaps it
    assert f(2, 8, 16, W.WKV_DTYPE_BF16, w, u, k, v, None, vp(P + 0x100000 + 300), None, None,
             None, None) == W.WKV_ERR_ALIAS
    # 16-bit formats: only the variants the automatic choice uses are compiled
    for plan in ((W.WKV_KERNEL_SEGMENTED, 16, 8, 64), (W.WKV_KERNEL_SEGMENTED, 16, 16, 32),
                 (W.WKV_KERNEL_LOOKBACK, 8, 8, 64), (W.WKV_KERNEL_LOOKBACK, 4, 16, 128)):
        p = W.ForwardPlan(*plan)
        for dt in (W.WKV_DTYPE_F16, W.WKV_DTYPE_BF16):
            assert f(2, 8, 16, dt, w, u, k, v, None, y, None, None, ctypes.byref(p),
                     None) == W.WKV_ERR_UNSUPPORTED, (plan, dt)
    p = W.ForwardPlan(W.WKV_KERNEL_LOOKBACK, 4, 32, 64)     # no gated 4x32 variant
    assert f(2, 8, 16, W.WKV_DTYPE_F16, w, u, k, v, vp(P + 0x30000000), y, None, None,
             ctypes.byref(p), None) == W.WKV_ERR_UNSUPPORTED
    si, so = vp(P + 0x400000), vp(P + 0x400000)
    base = [vp(P), vp(P + 0x1000), vp(P + 0x100000), vp(P + 0x200000)]
    sf = lib.wkv_step_typed
    assert sf(2, 2, 4, 5, *base, None, vp(P + 0x300000), si, so, None) == W.WKV_ERR_UNSUPPORTED
    assert sf(2, 2, 4, W.WKV_DTYPE_F16, *base, None, vp(P + 0x100000 + 8), si, so,
              None) == W.WKV_ERR_ALIAS


def test_token_shift_rejects_invalid_arguments(lib):
    from linear_recurrent_attention_amd import wkv as W
    vp = ctypes.c_void_p
    mu, x, xp = vp(P), vp(P + 0x100000), vp(P + 0x200000)
    out, xpo = vp(P + 0x10000000), vp(P + 0x300000)
    ts = lib.wkv_token_shift
    assert ts(2, 8, 16, -1, mu, x, xp, out, xpo, None) == W.WKV_ERR_DIM
    assert ts(2, 8, 16, 9, mu, x, xp, out, xpo, None) == W.WKV_ERR_UNSUPPORTED
    assert ts(2, 8, 16, 3, None, x, xp, out, xpo, None) == W.WKV_ERR_NULL
    assert ts(2, 8, 16, 3, mu, None, xp, out, xpo, None) == W.WKV_ERR_NULL
    assert ts(2, 8, 16, 3, mu, x, xp, None, xpo, None) == W.WKV_ERR_NULL
    assert ts(2, 8, 16, 3, mu, x, xp, vp(P + 0x100000 + 64), xpo, None) == W.WKV_ERR_ALIAS
    assert ts(2, 8, 16, 3, mu, x, xp, out, vp(P + 0x200000 + 4), None) == W.WKV_ERR_ALIAS
    assert ts(2, 8, 16, 3, mu, x, xp, out, vp(P + 0x100000), None) == W.WKV_ERR_ALIAS
    assert ts(1 << 30, 1 << 20, 1 << 20, 3, mu, x, xp, out, xpo, None) == W.WKV_ERR_OVERFLOW
    # nothing to write: returns before any launch
    assert ts(2, 8, 16, 0, None, x, xp, None, None, None) == W.WKV_OK
    assert ts(0, 8, 16, 3, mu, None, None, None, None, None) == W.WKV_OK


def test_binding_fails_loudly_without_library(tmp_path):
    from linear_recurrent_attention_amd import wkv
    with pytest.raises(RuntimeError, match="missing"):
        wkv._lib_saved = wkv._lib
        wkv._lib = None
        try:
            wkv.load_library(str(tmp_path / "libwkv.so"))
        finally:
            wkv._lib = wkv._lib_saved


def test_autograd_functions_refuse_host_tensors(lib):
    """The differentiable wrappers marshal arguments only: host tensors are
    refused before any call, with no CPU fallback."""
    import torch
    from linear_recurrent_attention_amd.autograd import token_shift, wkv_time_mix
    w, u = torch.ones(8), torch.zeros(8)
    k = torch.zeros(1, 4, 8, requires_grad=True)
    with pytest.raises(TypeError, match="HIP device"):
        wkv_time_mix(w, u, k, torch.zeros(1, 4, 8))
    with pytest.raises(TypeError, match="HIP device"):
        token_shift(torch.full((3, 8), 0.5), torch.zeros(1, 4, 8))


def test_auto_plan_follows_its_thresholds(lib):
    """The automatic kernel choice is host arithmetic (with 256 CUs when no
    device answers): lane kernel for T <= 16 or for >= 131072 lanes with
    T <= 128; segmented for >= 262144 lanes; otherwise the look-back kernel
    with 32-token segments when there are >= 8 blocks per CU, else 16."""
    from linear_recurrent_attention_amd import wkv as W
    L, S, K = W.WKV_KERNEL_LANE, W.WKV_KERNEL_SEGMENTED, W.WKV_KERNEL_LOOKBACK
    cases = {
        (8, 1024, 2048): (K, 4, 32, 64),      # gpt: 256 groups x 8 blocks = 2048 blocks
        (8, 4096, 2048): (K, 4, 32, 64),
        (1, 1024, 5120): (K, 4, 16, 64),      # stream: 80 groups x 8 blocks < 2048
        (1, 16, 8): (L, 0, 0, 0),
        (1, 17, 8): (K, 4, 16, 64),
        (1024, 1, 4096): (L, 0, 0, 0),        # decode-like
        (32, 128, 4096): (L, 0, 0, 0),        # 131072 lanes, T = 128
        (32, 129, 4096): (K, 4, 32, 64),      # 2048 groups x 2 blocks
        (64, 1024, 4096): (S, 16, 16, 64),    # 262144 lanes
    }
    for shape, want in cases.items():
        assert W.wkv_forward_plan_auto(*shape) == want, shape
    with pytest.raises(W.WkvError):
        W.wkv_forward_plan_auto(-1, 4, 4)


def test_forward_scratch_size_is_host_arithmetic(lib):
    """The look-back scratch a shape needs: a 256-byte header and two slot
    arrays of 2 KiB per (block, sequence, 64-channel group); none for shapes the
    automatic plan gives to a kernel without cross-workgroup state."""
    from linear_recurrent_attention_amd import wkv as W
    B, T, C = 8, 1024, 2048
    plan = W.wkv_forward_plan_auto(B, T, C)
    assert plan[0] == W.WKV_KERNEL_LOOKBACK
    blocks = -(-T // (plan[1] * plan[2]))
    slots = blocks * B * (C // 64)
    assert W.wkv_forward_scratch_size(B, T, C) == 256 + 2 * slots * 2048
    assert W.wkv_forward_scratch_size(1, 8, 64) == 0          # lane kernel
    assert W.wkv_forward_scratch_size(-1, 8, 64) == 0         # invalid
    assert W.wkv_forward_scratch_size(4, 0, 64) == 0          # nothing to do


def test_spin_limit_hook_round_trips(lib):
    from linear_recurrent_attention_amd import wkv as W
    old = W.wkv_set_lookback_spin_limit(7)
    assert old == 1 << 16
    assert W.wkv_set_lookback_spin_limit(old) == 7


def _bad_shape_cases():
    """(name of the binding call, callable) pairs, each with exactly one tensor
    of the wrong shape; the binding must raise before any library call."""
    import torch
    from linear_recurrent_attention_amd import wkv as W
    B, T, C = 2, 5, 8
    f = lambda *s: torch.zeros(*s)
    seq, st = (B, T, C), (3, B, C)
    k = f(*seq)
    good = dict(w=f(C), u=f(C), k=k, v=f(*seq))
    cases = [
        ("v", lambda: W.wkv_forward(good["w"], good["u"], k, f(B, T, C + 1))),
        ("w", lambda: W.wkv_forward(f(C - 1), good["u"], k, good["v"])),
        ("u", lambda: W.wkv_forward(good["w"], f(C, 1), k, good["v"])),
        ("y", lambda: W.wkv_forward(good["w"], good["u"], k, good["v"], y=f(B, T + 1, C))),
        ("state_in", lambda: W.wkv_forward(good["w"], good["u"], k, good["v"], state_in=f(3, B, C + 1))),
        ("state_out", lambda: W.wkv_forward(good["w"], good["u"], k, good["v"], state_out=f(2, B, C))),
        ("r", lambda: W.wkv_forward_gated(good["w"], good["u"], k, good["v"], f(B, T, 1))),
        ("r", lambda: W.wkv_forward_typed(good["w"], good["u"], k, good["v"], r=f(B, 1, C))),
        ("checkpoints", lambda: W.wkv_forward_checkpointed(
            good["w"], good["u"], f(B, 300, C), f(B, 300, C), checkpoints=f(1, 3, B, C))),
        ("v", lambda: W.bind_forward(good["w"], good["u"], k, f(B, T), f(*seq))),
        ("state_in", lambda: W.wkv_step(f(3, C), f(3, C), f(3, B, C), f(3, B, C), f(3, 3, B))),
        ("w", lambda: W.wkv_step(f(C), f(3, C), f(3, B, C), f(3, B, C), f(3, 3, B, C))),
        ("r", lambda: W.wkv_step_gated(f(3, C), f(3, C), f(3, B, C), f(3, B, C), f(3, B),
                                       f(3, 3, B, C))),
        ("dy", lambda: W.wkv_backward(good["w"], good["u"], k, good["v"], f(B, T, C + 2))),
        ("dw", lambda: W.wkv_backward(good["w"], good["u"], k, good["v"], f(*seq), dw=f(C + 1))),
        ("d_state_out", lambda: W.wkv_backward_state(
            good["w"], good["u"], k, good["v"], f(*seq), state_out=f(*st), d_state_out=f(3, C))),
        ("checkpoints", lambda: W.wkv_backward_checkpointed(
            good["w"], good["u"], f(B, 300, C), f(B, 300, C), f(B, 300, C), f(3, 3, B, C))),
        ("dr", lambda: W.wkv_backward_gated(good["w"], good["u"], k, good["v"], f(*seq), f(*seq),
                                            dr=f(B, T, C, 1))),
        ("workspace", lambda: W.wkv_backward(good["w"], good["u"], k, good["v"], f(*seq),
                                             workspace=torch.zeros(1, dtype=torch.float32))),
        ("x_prev", lambda: W.wkv_token_shift(f(3, C), f(*seq), x_prev=f(B, C + 1))),
        ("mu", lambda: W.wkv_token_shift(f(3, C + 1), f(*seq))),
        ("out", lambda: W.wkv_token_shift(f(3, C), f(*seq), out=f(2, B, T, C))),
        ("d_out", lambda: W.wkv_token_shift_backward(f(3, C), f(*seq), f(3, B, T, C - 1))),
        ("dmu", lambda: W.wkv_token_shift_backward(f(3, C), f(*seq), f(3, B, T, C), dmu=f(2, C))),
    ]
    return cases


def test_binding_checks_every_shape_before_calling():
    """Each binding call checks the shape of every tensor it passes against k's
    (or x's) dimensions: the C ABI receives bare pointers and could not."""
    for name, call in _bad_shape_cases():
        with pytest.raises((ValueError, TypeError)) as e:
            call()
        assert name in str(e.value) or "workspace" in str(e.value), (name, str(e.value))


def test_binding_checks_devices():
    """A tensor on another device than k's is refused before any call."""
    import torch
    from linear_recurrent_attention_amd import wkv as W
    k = torch.zeros(2, 3, 4, device="meta")
    w = torch.zeros(4, device="meta")
    with pytest.raises(ValueError, match="expected meta"):
        W.wkv_forward(w, w, k, torch.zeros(2, 3, 4), y=torch.empty(2, 3, 4, device="meta"))

"""Tolerances of the HIP path against the float64 oracle, and small helpers.

Forward outputs y (float32 vs float64):  |x - r| <= 1e-5 + 1e-4 |r|, elementwise
(1e-4 relative with a 1e-5 absolute floor, since y can cross zero).
States are compared in canonical form, because (a, b, o) and
(a e^d, b e^d, o - d) are the same state: m = a/b by the rule for y, and
lam = o + ln b (log of the total decayed weight) within 1e-4.
Gradients, per tensor: |x - r| <= 1e-3 |r| + 1e-3 rms(r) + f (1e-3 relative with
a floor of 1e-3 of the tensor's rms, since dk sums terms that cancel).  f is a
float32 round-off floor, 1e-6 rms(dy) (1 + max|v|) per element and that times
sqrt(B T) for the summed dw, du; it only matters where the reference is
identically zero (a one-token sequence: the token's own weight is 1, so dk, dw
and du vanish exactly while float32 leaves v - y at one rounding of v).
"""
import numpy as np

Y_RTOL, Y_ATOL = 1e-4, 1e-5
LAM_ATOL = 1e-4
G_RTOL, G_FLOOR = 1e-3, 1e-3


def y_excess(x, r):
    """max over elements of |x - r| / (atol + rtol |r|); <= 1 passes."""
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    if x.size == 0:
        return 0.0
    return float(np.max(np.abs(x - r) / (Y_ATOL + Y_RTOL * np.abs(r))))


def assert_y_close(x, r, what="y"):
    assert np.all(np.isfinite(x)), f"{what}: non-finite values"
    e = y_excess(x, r)
    assert e <= 1.0, f"{what}: error {e:.3g}x the tolerance (1e-5 + 1e-4|r|)"
    return e


def canonical(state):
    s = np.asarray(state, dtype=np.float64)
    a, b, o = s[0], s[1], s[2]
    empty = b <= 0
    bb = np.where(empty, 1.0, b)
    m = np.where(empty, 0.0, a / bb)
    lam = np.where(empty, -np.inf, o + np.log(bb))
    return m, lam, empty


def assert_state_close(x, r, what="state"):
    mx, lx, ex = canonical(x)
    mr, lr, er = canonical(r)
    assert np.array_equal(ex, er), f"{what}: empty lanes differ"
    e = y_excess(mx[~ex], mr[~er])
    assert e <= 1.0, f"{what}: mean m off by {e:.3g}x the tolerance"
    if np.any(~ex):
        dl = float(np.max(np.abs(lx[~ex] - lr[~er])))
        assert dl <= LAM_ATOL, f"{what}: log weight off by {dl:.3g} > {LAM_ATOL}"
    return e


def grad_excess(x, r, floor=0.0):
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    if r.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(r * r)))
    return float(np.max(np.abs(x - r) / (G_RTOL * np.abs(r) + G_FLOOR * rms + floor + 1e-300)))


def roundoff_floor(dy, v, summed=False):
    dy = np.asarray(dy, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if dy.size == 0:
        return 0.0
    f = 1e-6 * float(np.sqrt(np.mean(dy * dy))) * (1.0 + float(np.max(np.abs(v))))
    if summed:
        f *= float(np.sqrt(dy.shape[0] * dy.shape[1]))
    return f


def assert_grad_close(x, r, what, floor=0.0):
    assert np.all(np.isfinite(x)), f"{what}: non-finite values"
    e = grad_excess(x, r, floor)
    assert e <= 1.0, f"{what}: error {e:.3g}x the tolerance (1e-3|r| + 1e-3 rms)"
    return e


def f64(t):
    return t.detach().cpu().double().numpy()

"""Tolerances of the HIP path against the float64 oracle, and small helpers.

Forward outputs y (float32 vs float64):  |x - r| <= 1e-5 + 1e-4 |r|, elementwise
(1e-4 relative with a 1e-5 absolute floor, since y can cross zero).
States are compared in canonical form, because (a, b, o) and
(a e^d, b e^d, o - d) are the same state: m = a/b by the rule for y, and
lam = o + ln b (log of the total decayed weight) within 1e-4.
Gradients dk, dv (and the state's), per tensor: |x - r| <= 1e-3 |r| + 1e-3 rms(r)
(1e-3 relative with a floor of 1e-3 of the tensor's rms, since dk sums terms
that cancel).  Only where the reference is identically zero (a one-token
sequence: the token's own weight is 1, so dk vanishes exactly while float32
leaves v - y at one rounding of v) does a float32 round-off floor f replace
the rms floor: 1e-6 rms(dy) (1 + max|v|) per element.

dw and du, per channel (assert_sums_close): each is a sum over the batch and
the sequence of signed terms that can cancel, and a float32 evaluation errs
relative to the terms' sizes, not to the result.  So
    |x_c - r_c| <= 1e-3 |r_c| + 8 sqrt(T) eps32 m_c,
with m_c the oracle's sum of the terms' absolute values
(oracle.backward_magnitude) and eps32 = 2^-24 the float32 unit round-off:
each term carries a few roundings relative to its size, and the reverse scan
that builds it runs over up to T tokens, whose rounding errors add up like a
random walk.  Each term that is a difference (du's v_t - y_t, dw's v_i - y_t)
counts its two parts by size, since float32 forms it from parts that each
carry rounding.  Where little cancels, m_c is a small multiple of |r_c| and
the second term is a few 1e-5 |r_c| at T = 4096, so the check is the 1e-3
relative one.
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


EPS32 = 2.0 ** -24
SUM_ROUNDOFF = 8.0


def grad_excess(x, r, floor=0.0):
    """max over elements of |x - r| / (1e-3 |r| + 1e-3 rms(r)); the round-off
    floor `floor` is used only when r is identically zero."""
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    if r.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(r * r)))
    base = G_FLOOR * rms if rms > 0 else floor
    return float(np.max(np.abs(x - r) / (G_RTOL * np.abs(r) + base + 1e-300)))


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


def sum_excess(x, r, mag, T):
    """max over channels of |x - r| / (1e-3 |r| + 8 sqrt(T) eps32 mag)."""
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    mag = np.asarray(mag, dtype=np.float64)
    if r.size == 0:
        return 0.0
    tol = G_RTOL * np.abs(r) + SUM_ROUNDOFF * np.sqrt(max(int(T), 1)) * EPS32 * mag
    return float(np.max(np.abs(x - r) / (tol + 1e-300)))


def assert_sums_close(oracle, got_dw, got_du, ref_dw, ref_du, w, u, k, v, g, state_in=None,
                      state_out=None, d_state_out=None, what=""):
    """dw and du per channel against the oracle's, with the round-off scale of
    their terms taken from oracle.backward_magnitude on the same inputs (g: the
    gradient that reaches the recurrence)."""
    mdw, mdu = oracle.backward_magnitude(w, u, k, v, g, state_in, state_out, d_state_out)
    T = np.asarray(k).shape[1]
    for name, x, r, m in (("dw", got_dw, ref_dw, mdw), ("du", got_du, ref_du, mdu)):
        assert np.all(np.isfinite(x)), f"{what} {name}: non-finite values"
        e = sum_excess(x, r, m, T)
        assert e <= 1.0, (f"{what} {name}: error {e:.3g}x the tolerance "
                          f"(1e-3|r| + 8 sqrt(T) eps32 sum|terms|, per channel)")


def assert_chained_sums_close(oracle, got_dw, got_du, ref_dw, ref_du, w, u, k, v, g, cuts,
                              state_in=None, d_state_out=None, what="chain"):
    """dw and du of a sequence run as chunks of lengths `cuts`, chained through
    the carried state.  Each chunk's float32 sum errs relative to its own
    terms, so the round-off scale is the sum of the chunks' magnitudes, each
    with the state it starts from and hands on and the upstream state gradient
    it receives (the oracle's), and the walk length is the longest chunk."""
    k, v, g = (np.asarray(x, dtype=np.float64) for x in (k, v, g))
    bounds = np.cumsum([0] + list(cuts))
    states = [state_in]
    for i in range(len(cuts)):
        lo, hi = bounds[i], bounds[i + 1]
        states.append(oracle.forward_scan(w, u, k[:, lo:hi], v[:, lo:hi], states[-1])[1])
    mdw = np.zeros(k.shape[2])
    mdu = np.zeros(k.shape[2])
    g_i = d_state_out
    for i in reversed(range(len(cuts))):
        lo, hi = bounds[i], bounds[i + 1]
        args = (w, u, k[:, lo:hi], v[:, lo:hi], g[:, lo:hi], states[i], states[i + 1], g_i)
        m = oracle.backward_magnitude(*args)
        mdw, mdu = mdw + m[0], mdu + m[1]
        g_i = oracle.backward_state(*args)[4]
    for name, x, r, m in (("dw", got_dw, ref_dw, mdw), ("du", got_du, ref_du, mdu)):
        assert np.all(np.isfinite(x)), f"{what} {name}: non-finite values"
        e = sum_excess(x, r, m, max(cuts))
        assert e <= 1.0, f"{what} {name}: error {e:.3g}x the tolerance"

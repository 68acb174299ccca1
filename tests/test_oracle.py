"""Pins of the float64 oracle against what the pages and the mathematics fix.

Nothing here touches a GPU.  Each test pins the oracle to something other than
itself: a library routine in a limiting case, a closed-form series, the pages'
other two statements of the same operator, invariants, brute force, and
central finite differences for the backward.

Pages cited:
  RWKV architecture deep dive (youngju.dev): sections "WKV mechanism: core
  computation" (closed form), "Recurrent formulation", "Numerical stability via
  log-space computation", "Parallel training formulation", "Duality".
  rwkv-architecture skill page: "Quick start" (GPT mode = RNN mode over chunks),
  "Workflow 2: Long context processing".
"""
import os

import numpy as np
import pytest
from scipy.special import softmax

from linear_recurrent_attention_amd import synth

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_case(seed, B=2, T=23, C=5, recipe=synth.RECIPES[synth.TINY]):
    d = synth.make(synth.TINY, index=seed, B=B, T=T, C=C, recipe=recipe)
    return {n: t.double().numpy() for n, t in d.items()}


def rand_state(oracle, seed, B, C, T0=7):
    """A reachable non-empty state: the oracle's state after T0 random tokens."""
    d = rand_case(1000 + seed, B=B, T=T0, C=C)
    _, s = oracle.forward_brute(d["w"], d["u"], d["k"], d["v"])
    return s


# ---------------------------------------------------------------- forward ---

@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("with_state", [False, True])
def test_brute_equals_scan(oracle, seed, with_state):
    d = rand_case(seed, B=2, T=41, C=6)
    s_in = rand_state(oracle, seed, 2, 6) if with_state else None
    yb, sb = oracle.forward_brute(d["w"], d["u"], d["k"], d["v"], s_in)
    ys, ss = oracle.forward_scan(d["w"], d["u"], d["k"], d["v"], s_in)
    np.testing.assert_allclose(ys, yb, rtol=1e-12, atol=1e-13)
    mb, lb = oracle.canonical_state(sb)
    ms, ls = oracle.canonical_state(ss)
    np.testing.assert_allclose(ms, mb, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(ls, lb, rtol=1e-12, atol=1e-12)


def test_single_token_from_empty_state_is_v(oracle):
    # Core computation: with no past terms the weight of the only token cancels.
    d = rand_case(7, B=3, T=1, C=9)
    for fn in (oracle.forward_brute, oracle.forward_scan):
        y, s = fn(d["w"], d["u"], d["k"], d["v"])
        np.testing.assert_allclose(y, d["v"], rtol=1e-15, atol=0)


def test_constant_v_gives_v(oracle):
    d = rand_case(8, B=2, T=30, C=4)
    v = np.broadcast_to(np.linspace(-2, 3, 4), d["v"].shape).copy()
    for fn in (oracle.forward_brute, oracle.forward_scan):
        y, _ = fn(d["w"], d["u"], d["k"], v)
        np.testing.assert_allclose(y, v, rtol=1e-14, atol=1e-14)


def test_fast_decay_limit_is_two_token_softmax(oracle):
    """w -> inf: only the newest past token (distance 0 in the closed form) and the
    current token survive, so wkv_t is a softmax over (k_{t-1}, u+k_t).  This is
    what tells the closed-form placement of exp(-w) from the recurrence section's
    (which would give v_t in this limit)."""
    d = rand_case(9, B=1, T=12, C=3)
    w = np.full(3, 60.0)
    y, _ = oracle.forward_brute(w, d["u"], d["k"], d["v"])
    k, v, u = d["k"][0], d["v"][0], d["u"]
    for t in range(1, 12):
        scores = np.stack([k[t - 1], u + k[t]])
        ref = (softmax(scores, axis=0) * np.stack([v[t - 1], v[t]])).sum(0)
        np.testing.assert_allclose(y[0, t], ref, rtol=1e-12, atol=1e-14)
    ys, _ = oracle.forward_scan(w, d["u"], d["k"], d["v"])
    np.testing.assert_allclose(ys, y, rtol=1e-12, atol=1e-14)


def test_no_decay_limit_is_causal_softmax_attention(oracle):
    """w -> 0+: wkv_t is softmax attention over tokens 1..t with scores k_i, the
    current token's score raised by the bonus u."""
    d = rand_case(10, B=1, T=20, C=4)
    w = np.full(4, 1e-14)
    y, _ = oracle.forward_brute(w, d["u"], d["k"], d["v"])
    ys, _ = oracle.forward_scan(w, d["u"], d["k"], d["v"])
    k, v, u = d["k"][0], d["v"][0], d["u"]
    for t in range(20):
        scores = k[: t + 1].copy()
        scores[t] += u
        ref = (softmax(scores, axis=0) * v[: t + 1]).sum(0)
        np.testing.assert_allclose(y[0, t], ref, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(ys[0, t], ref, rtol=1e-11, atol=1e-12)


def test_constant_k_geometric_series(oracle):
    """Constant k: the past weights form a geometric series in e^{-w}.  With v the
    indicator of token j, y_t is the share of token j in output t."""
    T, C, kappa, j = 25, 3, 0.7, 6
    w = np.array([0.05, 0.4, 2.0])
    u = np.array([0.3, -1.1, 0.8])
    k = np.full((1, T, C), kappa)
    v = np.zeros((1, T, C))
    v[0, j] = 1.0
    r = np.exp(-w)
    for fn in (oracle.forward_brute, oracle.forward_scan):
        y, s = fn(w, u, k, v)
        for t in range(T):
            geom = (1 - r ** t) / (1 - r)            # sum_{m<t} r^m: t past tokens
            den = geom + np.exp(u)
            if t < j:
                ref = np.zeros(C)
            elif t == j:
                ref = np.exp(u) / den
            else:
                ref = r ** (t - 1 - j) / den
            np.testing.assert_allclose(y[0, t], ref, rtol=1e-12, atol=1e-15)
        # state after T tokens: total weight e^kappa (1 - r^T)/(1 - r)
        m, lam = oracle.canonical_state(s)
        np.testing.assert_allclose(lam[0], kappa + np.log((1 - r ** T) / (1 - r)), rtol=1e-12)
        np.testing.assert_allclose(m[0], r ** (T - 1 - j) / ((1 - r ** T) / (1 - r)), rtol=1e-12)


def test_recurrent_section_form_is_closed_form_with_shifted_bonus(oracle):
    """The recurrence section multiplies the whole past by e^{-w} in the output
    while the closed form does not; the two agree once the bonus is shifted by w
    (the common factor cancels in the ratio).  Here the recurrence section's
    formulas are run directly (plain float64, no stabilisation, small inputs)."""
    d = rand_case(11, B=1, T=16, C=5)
    w, u, k, v = d["w"], d["u"], d["k"][0], d["v"][0]

    def recurrent_section(bonus):
        alpha = np.zeros(5)
        beta = np.zeros(5)
        out = []
        for t in range(16):
            ek = np.exp(k[t])
            euk = np.exp(bonus + k[t])
            out.append((np.exp(-w) * alpha + euk * v[t]) / (np.exp(-w) * beta + euk))
            alpha = np.exp(-w) * alpha + ek * v[t]
            beta = np.exp(-w) * beta + ek
        return np.array(out)

    y, _ = oracle.forward_brute(w, u, d["k"], d["v"])
    np.testing.assert_allclose(recurrent_section(u - w), y[0], rtol=1e-12, atol=1e-14)
    assert np.max(np.abs(recurrent_section(u) - y[0])) > 1e-3


def test_parallel_section_loop_equals_closed_form(oracle):
    """The parallel-training section's loop: zero running sums, the bonus on the
    current token only, sums decayed after each output."""
    d = rand_case(12, B=1, T=19, C=4)
    w, u, k, v = d["w"], d["u"], d["k"][0], d["v"][0]
    alpha = np.zeros(4)
    beta = np.zeros(4)
    ref = []
    for t in range(19):
        euk = np.exp(u + k[t])
        ref.append((alpha + euk * v[t]) / (beta + euk))
        alpha = np.exp(-w) * alpha + np.exp(k[t]) * v[t]
        beta = np.exp(-w) * beta + np.exp(k[t])
    y, _ = oracle.forward_brute(w, u, d["k"], d["v"])
    np.testing.assert_allclose(y[0], np.array(ref), rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("seed", range(3))
def test_outputs_are_convex_combinations(oracle, seed):
    d = rand_case(20 + seed, B=2, T=50, C=7, recipe=synth.RECIPES[synth.STABILITY])
    s_in = rand_state(oracle, seed, 2, 7)
    m0, _ = oracle.canonical_state(s_in)
    y, _ = oracle.forward_scan(d["w"], d["u"], d["k"], d["v"], s_in)
    v = d["v"]
    lo = np.minimum(np.minimum.accumulate(v, axis=1), m0[:, None, :])
    hi = np.maximum(np.maximum.accumulate(v, axis=1), m0[:, None, :])
    tol = 1e-12 * (1 + np.abs(v).max())
    assert np.all(y >= lo - tol) and np.all(y <= hi + tol)


def test_state_invariant(oracle):
    """Max-normalised state: the largest decayed weight is exactly 1, so
    1 <= b <= number of tokens absorbed, and |a| <= b * max|v|."""
    d = rand_case(30, B=3, T=64, C=8, recipe=synth.RECIPES[synth.STABILITY])
    for T in (1, 5, 64):
        _, s = oracle.forward_scan(d["w"], d["u"], d["k"][:, :T], d["v"][:, :T])
        a, b = s[0], s[1]
        assert np.all(b >= 1 - 1e-12) and np.all(b <= T + 1e-9)
        vmax = np.abs(d["v"][:, :T]).max(axis=1)
        assert np.all(np.abs(a) <= b * vmax + 1e-12)


def test_empty_state_forms_agree(oracle):
    d = rand_case(31, B=2, T=9, C=3)
    empty = np.zeros((3, 2, 3))
    empty[2] = -np.inf
    for fn in (oracle.forward_brute, oracle.forward_scan):
        y0, s0 = fn(d["w"], d["u"], d["k"], d["v"])
        y1, s1 = fn(d["w"], d["u"], d["k"], d["v"], empty)
        np.testing.assert_array_equal(y0, y1)
        np.testing.assert_array_equal(s0, s1)


def test_state_is_defined_up_to_common_scale(oracle):
    """(a, b, o) and (a e^d, b e^d, o - d) are the same state."""
    d = rand_case(32, B=2, T=13, C=4)
    s = rand_state(oracle, 5, 2, 4)
    s2 = s.copy()
    s2[0] *= np.exp(3.5)
    s2[1] *= np.exp(3.5)
    s2[2] -= 3.5
    for fn in (oracle.forward_brute, oracle.forward_scan):
        y1, o1 = fn(d["w"], d["u"], d["k"], d["v"], s)
        y2, o2 = fn(d["w"], d["u"], d["k"], d["v"], s2)
        np.testing.assert_allclose(y2, y1, rtol=1e-13, atol=1e-14)
        for x1, x2 in zip(oracle.canonical_state(o1), oracle.canonical_state(o2)):
            np.testing.assert_allclose(x2, x1, rtol=1e-13, atol=1e-13)


def _chunked(oracle, fn, d, cuts, s_in=None):
    ys, s = [], s_in
    t0 = 0
    for n in cuts:
        sl = slice(t0, t0 + n)
        y, s = fn(d["w"], d["u"], d["k"][:, sl], d["v"][:, sl], s)
        ys.append(y)
        t0 += n
    return np.concatenate(ys, axis=1), s


def _golden_cuts():
    total, cuts = None, None
    with open(os.path.join(GOLDEN, "quickstart_chunking.txt")) as f:
        for line in f:
            if line.startswith("total"):
                total = int(line.split()[1])
            elif line.startswith("chunks"):
                cuts = [int(x) for x in line.split()[1:]]
    assert sum(cuts) == total
    return total, cuts


@pytest.mark.parametrize("pattern", ["quickstart", "all_ones", "random"])
def test_gpt_mode_equals_rnn_mode_over_chunks(oracle, pattern):
    """Same weights, same results: one call over the sequence equals calls over
    any chunking of it with the state carried (Quick start; Duality)."""
    if pattern == "quickstart":
        T, cuts = _golden_cuts()
    elif pattern == "all_ones":
        T, cuts = 17, [1] * 17
    else:
        T = 97
        rng = np.random.default_rng(5)
        pts = np.sort(rng.choice(np.arange(1, T), size=9, replace=False))
        cuts = list(np.diff(np.concatenate([[0], pts, [T]])))
    d = rand_case(40, B=2, T=T, C=6)
    s_in = rand_state(oracle, 9, 2, 6)
    yb, sb = oracle.forward_brute(d["w"], d["u"], d["k"], d["v"], s_in)
    for fn in (oracle.forward_brute, oracle.forward_scan):
        yc, sc = _chunked(oracle, fn, d, cuts, s_in)
        np.testing.assert_allclose(yc, yb, rtol=1e-12, atol=1e-13)
        for x1, x2 in zip(oracle.canonical_state(sb), oracle.canonical_state(sc)):
            np.testing.assert_allclose(x2, x1, rtol=1e-12, atol=1e-12)


def test_zero_length_call_keeps_state(oracle):
    d = rand_case(41, B=1, T=0, C=3)
    s = rand_state(oracle, 3, 1, 3)
    for fn in (oracle.forward_brute, oracle.forward_scan):
        y, s2 = fn(d["w"], d["u"], d["k"], d["v"], s)
        assert y.shape == (1, 0, 3)
        np.testing.assert_allclose(s2, s, rtol=1e-15)


def test_wide_exponents_stay_finite(oracle):
    """Stability recipe (k ~ N(0,8) with +-60 outliers, decay up to e^3): no
    overflow, and brute force and scan agree."""
    d = rand_case(42, B=2, T=200, C=8, recipe=synth.RECIPES[synth.STABILITY])
    assert np.abs(d["k"]).max() == 60.0
    yb, sb = oracle.forward_brute(d["w"], d["u"], d["k"], d["v"])
    ys, ss = oracle.forward_scan(d["w"], d["u"], d["k"], d["v"])
    assert np.all(np.isfinite(yb)) and np.all(np.isfinite(sb))
    np.testing.assert_allclose(ys, yb, rtol=1e-11, atol=1e-12)


# --------------------------------------------------------------- backward ---

def _loss(oracle, w, u, k, v, dy):
    y, _ = oracle.forward_brute(w, u, k, v)
    return float((y * dy).sum())


@pytest.mark.parametrize("seed", range(3))
def test_backward_brute_equals_scan(oracle, seed):
    d = synth.make(synth.STABILITY, index=seed, B=2, T=45, C=6, with_dy=True)
    d = {n: t.double().numpy() for n, t in d.items()}
    gb = oracle.backward_brute(d["w"], d["u"], d["k"], d["v"], d["dy"])
    gs = oracle.backward_scan(d["w"], d["u"], d["k"], d["v"], d["dy"])
    for a, b in zip(gs, gb):
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-12 * (1 + np.abs(b).max()))


def test_backward_brute_equals_scan_at_extreme_decays(oracle):
    """Decay rates from 1e-6 (no decay over the sequence) to 60 (the past
    vanishes within two tokens): the O(T) scan still equals the O(T^2) closed
    form, and dw equals central differences of the loss."""
    d = synth.make(synth.STABILITY, index=8, B=2, T=60, C=12, with_dy=True)
    d = {n: t.double().numpy() for n, t in d.items()}
    w = np.geomspace(1e-6, 60.0, 12)
    gb = oracle.backward_brute(w, d["u"], d["k"], d["v"], d["dy"])
    gs = oracle.backward_scan(w, d["u"], d["k"], d["v"], d["dy"])
    for a, b in zip(gs, gb):
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-12 * (1 + np.abs(b).max()))
    for c in (0, 5, 11):
        h = 1e-6 * max(1.0, w[c])
        wp, wm = w.copy(), w.copy()
        wp[c] += h
        wm[c] -= h
        ref = (_loss(oracle, wp, d["u"], d["k"], d["v"], d["dy"]) -
               _loss(oracle, wm, d["u"], d["k"], d["v"], d["dy"])) / (2 * h)
        assert abs(gs[2][c] - ref) <= 1e-6 * max(1e-3, np.abs(gs[2]).max()), (c, gs[2][c], ref)


@pytest.mark.parametrize("outlier", [False, True])
def test_backward_matches_finite_differences(oracle, outlier):
    """Central differences of L = sum dy*y on a B=1, T=32, C=8 slice of the
    stability workload; the second copy forces a +60 entry into k."""
    d = synth.make(synth.STABILITY, index=3, B=1, T=32, C=8, with_dy=True)
    d = {n: t.double().numpy() for n, t in d.items()}
    if outlier:
        d["k"][0, 11, 2] = 60.0
        d["k"][0, 20, 5] = -60.0
    w, u, k, v, dy = d["w"], d["u"], d["k"], d["v"], d["dy"]
    dk, dv, dw, du = oracle.backward_scan(w, u, k, v, dy)
    dkb, dvb, dwb, dub = oracle.backward_brute(w, u, k, v, dy)

    def fd(arr, idx):
        x0 = arr[idx]
        h = 1e-6 * max(1.0, abs(x0))
        arr[idx] = x0 + h
        lp = _loss(oracle, w, u, k, v, dy)
        arr[idx] = x0 - h
        lm = _loss(oracle, w, u, k, v, dy)
        arr[idx] = x0
        return (lp - lm) / (2 * h)

    rng = np.random.default_rng(0)
    picks = [(0, int(t), int(c)) for t, c in zip(rng.integers(0, 32, 24), rng.integers(0, 8, 24))]
    if outlier:
        picks += [(0, 11, 2), (0, 20, 5), (0, 12, 2)]
    for grad, gbrute, arr in ((dk, dkb, k), (dv, dvb, v)):
        for idx in picks:
            ref = fd(arr, idx)
            scale = max(1e-3, np.abs(grad).max())
            assert abs(grad[idx] - ref) <= 1e-6 * scale, (idx, grad[idx], ref)
            assert abs(gbrute[idx] - ref) <= 1e-6 * scale
    for grad, gbrute, arr in ((dw, dwb, w), (du, dub, u)):
        for c in range(8):
            ref = fd(arr, (c,))
            scale = max(1e-3, np.abs(grad).max())
            assert abs(grad[c] - ref) <= 1e-6 * scale, (c, grad[c], ref)
            assert abs(gbrute[c] - ref) <= 1e-6 * scale


def test_backward_invariants(oracle):
    """Shifting every k of a lane leaves y unchanged, so sum_i dk_i = 0 per lane;
    the weights of each output sum to one, so sum_i dv_i = sum_t dy_t per lane;
    adding a constant to every v shifts every y by it, so dk, dw, du are unchanged."""
    d = synth.make(synth.STABILITY, index=5, B=3, T=60, C=5, with_dy=True)
    d = {n: t.double().numpy() for n, t in d.items()}
    dk, dv, dw, du = oracle.backward_scan(d["w"], d["u"], d["k"], d["v"], d["dy"])
    scale = np.abs(dk).max()
    np.testing.assert_allclose(dk.sum(axis=1), 0.0, atol=1e-11 * scale * 60)
    np.testing.assert_allclose(dv.sum(axis=1), d["dy"].sum(axis=1), rtol=1e-11, atol=1e-11)
    dk2, dv2, dw2, du2 = oracle.backward_scan(d["w"], d["u"], d["k"], d["v"] + 2.5, d["dy"])
    np.testing.assert_allclose(dk2, dk, rtol=1e-9, atol=1e-10 * scale)
    np.testing.assert_allclose(dv2, dv, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dw2, dw, rtol=1e-9, atol=1e-9 * np.abs(dw).max())
    np.testing.assert_allclose(du2, du, rtol=1e-9, atol=1e-9 * np.abs(du).max())


def test_threads_do_not_change_results(oracle):
    d = synth.make(synth.GPT, index=0, B=2, T=33, C=16, with_dy=True)
    d = {n: t.double().numpy() for n, t in d.items()}
    y1, s1 = oracle.forward_scan(d["w"], d["u"], d["k"], d["v"], nthreads=1)
    y4, s4 = oracle.forward_scan(d["w"], d["u"], d["k"], d["v"], nthreads=4)
    np.testing.assert_array_equal(y1, y4)
    np.testing.assert_array_equal(s1, s4)
    g1 = oracle.backward_scan(d["w"], d["u"], d["k"], d["v"], d["dy"], nthreads=1)
    g4 = oracle.backward_scan(d["w"], d["u"], d["k"], d["v"], d["dy"], nthreads=4)
    for a, b in zip(g1, g4):
        np.testing.assert_array_equal(a, b)


# ------------------------------------------------- receptance gate, shift ---
# RWKV architecture deep dive: "RWKV architecture overview" (block figure:
# the time-mixing output is sigmoid(r_t) * wkv_t) and "Token shift".

def test_gate_is_the_logistic_function(oracle):
    """sigmoid(r) * y against scipy's logistic function, including the tails
    where exp(-r) overflows a double."""
    from scipy.special import expit
    rng = np.random.default_rng(11)
    r = np.concatenate([rng.normal(0.0, 3.0, 500), [0.0, 30.0, -30.0, 745.0, -745.0, 1e300,
                                                     -1e300]])
    y = rng.normal(0.0, 2.0, r.size)
    got = oracle.gate(y, r)
    np.testing.assert_allclose(got, expit(r) * y, rtol=1e-15, atol=1e-300)


def test_gate_limits_and_symmetry(oracle):
    y = np.array([3.0, -1.5, 7.25])
    np.testing.assert_array_equal(oracle.gate(y, np.zeros(3)), y / 2)      # sigmoid(0) = 1/2
    np.testing.assert_array_equal(oracle.gate(y, np.full(3, 800.0)), y)     # open gate
    np.testing.assert_array_equal(oracle.gate(y, np.full(3, -800.0)), 0 * y)  # closed gate
    r = np.linspace(-20, 20, 81)
    one = np.ones_like(r)
    np.testing.assert_allclose(oracle.gate(one, r) + oracle.gate(one, -r), one, rtol=1e-15)


def test_gate_backward_is_the_derivative_of_the_gate(oracle):
    """Central differences of sum(d * gate(y, r)) in y and in r.  Each output
    depends on its own y and r only, so one perturbation of every element at
    once gives every partial derivative."""
    rng = np.random.default_rng(12)
    n = 2000
    y = rng.normal(0.0, 2.0, n)
    r = rng.normal(0.0, 4.0, n)
    d = rng.normal(0.0, 1.0, n)
    g, dr = oracle.gate_backward(y, r, d)
    h = 1e-5
    num_y = d * (oracle.gate(y + h, r) - oracle.gate(y - h, r)) / (2 * h)
    num_r = d * (oracle.gate(y, r + h) - oracle.gate(y, r - h)) / (2 * h)
    np.testing.assert_allclose(g, num_y, rtol=1e-8, atol=1e-10)
    np.testing.assert_allclose(dr, num_r, rtol=1e-6, atol=1e-10)


def test_gate_backward_tails_and_zero(oracle):
    y = np.array([2.0, -3.0, 0.5, 1.0])
    d = np.array([1.0, 0.5, -2.0, 4.0])
    # r = 0: g = d / 2, dr = d y / 4
    g, dr = oracle.gate_backward(y, np.zeros(4), d)
    np.testing.assert_array_equal(g, d / 2)
    np.testing.assert_array_equal(dr, d * y / 4)
    # saturated gate: open passes d through, closed passes nothing; dr vanishes
    g, dr = oracle.gate_backward(y, np.full(4, 800.0), d)
    np.testing.assert_array_equal(g, d)
    assert np.all(dr == 0)
    g, dr = oracle.gate_backward(y, np.full(4, -800.0), d)
    assert np.all(g == 0) and np.all(dr == 0)
    # dr is even in r (s (1 - s) is), g(r) + g(-r) = d
    r = np.linspace(-20, 20, 4)
    g1, dr1 = oracle.gate_backward(y, r, d)
    g2, dr2 = oracle.gate_backward(y, -r, d)
    np.testing.assert_allclose(dr1, dr2, rtol=1e-14)
    np.testing.assert_allclose(g1 + g2, d, rtol=1e-14)


def _shift_loss(oracle, mu, x, xp, d_out, d_xpo):
    out, xpo = oracle.token_shift(mu, x, xp)
    return float(np.sum(d_out * out) + np.sum(d_xpo * xpo))


def test_token_shift_backward_per_element_differences(oracle):
    """Every partial derivative of sum(d_out * out) + sum(d_xpo * x_prev_out),
    by central differences of the oracle's own token shift (the loss is
    bilinear in mu and x, so the differences are exact up to rounding)."""
    rng = np.random.default_rng(21)
    B, T, C, M = 2, 4, 3, 2
    mu, x, xp = rng.uniform(0, 1, (M, C)), rng.normal(size=(B, T, C)), rng.normal(size=(B, C))
    d_out, d_xpo = rng.normal(size=(M, B, T, C)), rng.normal(size=(B, C))
    dx, dxp, dmu = oracle.token_shift_backward(mu, x, xp, d_out, d_xpo)
    h = 1e-6
    for arr, got in ((x, dx), (xp, dxp), (mu, dmu)):
        num = np.empty_like(arr)
        for i in np.ndindex(arr.shape):
            keep = arr[i]
            arr[i] = keep + h
            lp = _shift_loss(oracle, mu, x, xp, d_out, d_xpo)
            arr[i] = keep - h
            lm = _shift_loss(oracle, mu, x, xp, d_out, d_xpo)
            arr[i] = keep
            num[i] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(got, num, rtol=1e-7, atol=1e-8)


def test_token_shift_backward_directional_differences(oracle):
    """Along random directions on a larger case, with and without a carried
    token (x_prev None is zeros and receives no gradient that matters)."""
    rng = np.random.default_rng(22)
    B, T, C, M = 3, 50, 7, 3
    mu, x = rng.uniform(0, 1, (M, C)), rng.normal(size=(B, T, C))
    d_out, d_xpo = rng.normal(size=(M, B, T, C)), rng.normal(size=(B, C))
    for xp in (rng.normal(size=(B, C)), None):
        dx, dxp, dmu = oracle.token_shift_backward(mu, x, xp, d_out, d_xpo)
        xp0 = np.zeros((B, C)) if xp is None else xp
        h = 1e-5
        for _ in range(3):
            ex, ep, em = rng.normal(size=x.shape), rng.normal(size=(B, C)), rng.normal(size=mu.shape)
            lp = _shift_loss(oracle, mu + h * em, x + h * ex, xp0 + h * ep, d_out, d_xpo)
            lm = _shift_loss(oracle, mu - h * em, x - h * ex, xp0 - h * ep, d_out, d_xpo)
            want = (lp - lm) / (2 * h)
            got = float(np.sum(dx * ex) + np.sum(dxp * ep) + np.sum(dmu * em))
            assert abs(got - want) <= 1e-7 * (1 + abs(want)), (got, want)


def test_token_shift_backward_limits(oracle):
    rng = np.random.default_rng(23)
    B, T, C, M = 2, 6, 4, 3
    x, xp = rng.normal(size=(B, T, C)), rng.normal(size=(B, C))
    d_out, d_xpo = rng.normal(size=(M, B, T, C)), rng.normal(size=(B, C))
    # mu = 1: no shift; every mix passes its gradient straight to its own token
    dx, dxp, _ = oracle.token_shift_backward(np.ones((M, C)), x, xp, d_out, d_xpo)
    want = d_out.sum(axis=0)
    want[:, T - 1] += d_xpo
    np.testing.assert_allclose(dx, want, rtol=1e-15, atol=1e-15)
    assert np.all(dxp == 0)
    # mu = 0: a pure shift by one token
    dx, dxp, _ = oracle.token_shift_backward(np.zeros((M, C)), x, xp, d_out, d_xpo)
    want = np.zeros_like(x)
    want[:, :T - 1] = d_out.sum(axis=0)[:, 1:]
    want[:, T - 1] = d_xpo
    np.testing.assert_allclose(dx, want, rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(dxp, d_out.sum(axis=0)[:, 0], rtol=1e-15)
    # no tokens: the carried token's gradient passes through; dmu is zero
    dx, dxp, dmu = oracle.token_shift_backward(rng.uniform(0, 1, (M, C)), np.zeros((B, 0, C)),
                                               xp, np.zeros((M, B, 0, C)), d_xpo)
    np.testing.assert_array_equal(dxp, d_xpo)
    assert dx.size == 0 and np.all(dmu == 0)


def _shift_fixture():
    rows = {"x": [], "mu": [], "out": {}, "prev": None, "last": None}
    with open(os.path.join(GOLDEN, "token_shift_worked.txt")) as f:
        for line in f:
            p = line.split()
            if not p or p[0].startswith("#"):
                continue
            if p[0] in ("x", "mu"):
                rows[p[0]].append([float(a) for a in p[1:]])
            elif p[0] == "out":
                rows["out"].setdefault(int(p[1]), []).append([float(a) for a in p[2:]])
            else:
                rows[p[0]] = [float(a) for a in p[1:]]
    return rows


def test_token_shift_worked_example(oracle):
    g = _shift_fixture()
    x = np.array(g["x"])[None]                  # [1][3][2]
    out, last = oracle.token_shift(np.array(g["mu"]), x, np.array(g["prev"])[None])
    for m, rows in g["out"].items():
        np.testing.assert_array_equal(out[m, 0], np.array(rows))
    np.testing.assert_array_equal(last[0], np.array(g["last"]))


def test_token_shift_limits(oracle):
    """mu = 1 passes x_t through; mu = 0 gives the previous token (the carried
    one first, zero for a fresh sequence)."""
    rng = np.random.default_rng(12)
    x = rng.normal(size=(2, 9, 5))
    prev = rng.normal(size=(2, 5))
    mu = np.stack([np.ones(5), np.zeros(5)])
    for p, first in ((prev, prev), (None, np.zeros((2, 5)))):
        out, last = oracle.token_shift(mu, x, p)
        np.testing.assert_array_equal(out[0], x)
        np.testing.assert_array_equal(out[1][:, 0], first)
        np.testing.assert_array_equal(out[1][:, 1:], x[:, :-1])
        np.testing.assert_array_equal(last, x[:, -1])


@pytest.mark.parametrize("cuts", [[4, 1, 6], [1] * 11, [11]])
def test_token_shift_chunking(oracle, cuts):
    """Calls over chunks with the last token carried equal one call (the
    state contract of Quick start, applied to the shift's state)."""
    rng = np.random.default_rng(13)
    x = rng.normal(size=(3, 11, 4))
    mu = rng.uniform(0, 1, size=(3, 4))
    whole, last = oracle.token_shift(mu, x, None)
    parts, p, t = [], None, 0
    for n in cuts:
        o, p = oracle.token_shift(mu, x[:, t:t + n], p)
        parts.append(o)
        t += n
    np.testing.assert_array_equal(np.concatenate(parts, axis=2), whole)
    np.testing.assert_array_equal(p, last)
    o, p2 = oracle.token_shift(mu, x[:, :0], p)       # empty call keeps the state
    assert o.shape == (3, 3, 0, 4)
    np.testing.assert_array_equal(p2, p)


# ------------------------------------------------ backward with the state ---
# Quick start (RNN mode carries the state between calls): training over chunks
# needs the gradient with respect to the state a chunk starts from, and takes
# the gradient with respect to the state it hands on.

def _state_loss(oracle, w, u, k, v, dy, s_in, gA, gB):
    """L = sum dy*y + gA*A_T + gB*B_T with A_T, B_T the true sums after the
    last token (smooth in every input, unlike the (a, b, o) planes)."""
    y, s = oracle.forward_brute(w, u, k, v, s_in)
    A = s[0] * np.exp(s[2])
    Bt = s[1] * np.exp(s[2])
    return float((y * dy).sum() + (gA * A).sum() + (gB * Bt).sum())


@pytest.mark.parametrize("recipe", [synth.GPT, synth.STABILITY])
def test_backward_state_matches_finite_differences(oracle, recipe):
    B, T, C = 2, 24, 3
    d = synth.make(recipe, index=7, B=B, T=T, C=C, with_dy=True)
    d = {n: t.double().numpy() for n, t in d.items()}
    w, u, k, v, dy = d["w"], d["u"], d["k"], d["v"], d["dy"]
    s_in = rand_state(oracle, 30, B, C)
    _, s_out = oracle.forward_brute(w, u, k, v, s_in)
    rng = np.random.default_rng(8)
    g_state = rng.normal(size=(3, B, C))               # upstream (a, b, o) gradient
    gA = g_state[0] * np.exp(-s_out[2])                # -> true-sum gradient
    gB = g_state[1] * np.exp(-s_out[2])
    dk, dv, dw, du, dsi = oracle.backward_state(w, u, k, v, dy, s_in, s_out, g_state)

    def fd(arr, idx):
        x0 = arr[idx]
        h = 1e-6 * max(1.0, abs(x0))
        arr[idx] = x0 + h
        lp = _state_loss(oracle, w, u, k, v, dy, s_in, gA, gB)
        arr[idx] = x0 - h
        lm = _state_loss(oracle, w, u, k, v, dy, s_in, gA, gB)
        arr[idx] = x0
        return (lp - lm) / (2 * h)

    def check(grad, arr, idx):
        ref = fd(arr, idx)
        scale = max(1e-3, np.abs(grad).max())
        assert abs(grad[idx] - ref) <= 2e-6 * scale, (idx, grad[idx], ref)

    for idx in [(b, t, c) for b in range(B) for t in (0, 1, 11, T - 2, T - 1) for c in range(C)]:
        check(dk, k, idx)
        check(dv, v, idx)
    for c in range(C):
        check(dw, w, (c,))
        check(du, u, (c,))
    for p in range(3):                                 # a0, b0, o0 of every lane
        for b in range(B):
            for c in range(C):
                check(dsi, s_in, (p, b, c))


def test_backward_state_reduces_to_the_stateless_backward(oracle):
    d = rand_case(31, B=2, T=40, C=4)
    dy = synth.make(synth.TINY, index=31, B=2, T=40, C=4, with_dy=True)["dy"].double().numpy()
    ref = oracle.backward_brute(d["w"], d["u"], d["k"], d["v"], dy)
    got = oracle.backward_state(d["w"], d["u"], d["k"], d["v"], dy)
    for x, r in zip(got[:4], ref):
        np.testing.assert_allclose(x, r, rtol=1e-13, atol=1e-15)
    np.testing.assert_array_equal(got[4], 0.0)        # nothing flows into an empty state


@pytest.mark.parametrize("cut", [1, 17, 39])
def test_backward_state_chains_over_chunks(oracle, cut):
    """Backward over [0, T) equals the backward of the second chunk, whose
    state gradient is handed to the backward of the first (state coordinates
    exactly as the forward handed them on)."""
    B, T, C = 2, 40, 4
    d = rand_case(32, B=B, T=T, C=C)
    w, u, k, v = d["w"], d["u"], d["k"], d["v"]
    dy = synth.make(synth.TINY, index=32, B=B, T=T, C=C, with_dy=True)["dy"].double().numpy()
    s0 = rand_state(oracle, 33, B, C)
    _, s_end = oracle.forward_brute(w, u, k, v, s0)
    g_end = np.random.default_rng(9).normal(size=(3, B, C))
    full = oracle.backward_state(w, u, k, v, dy, s0, s_end, g_end)
    _, s_mid = oracle.forward_brute(w, u, k[:, :cut], v[:, :cut], s0)
    _, s_end2 = oracle.forward_brute(w, u, k[:, cut:], v[:, cut:], s_mid)
    second = oracle.backward_state(w, u, k[:, cut:], v[:, cut:], dy[:, cut:], s_mid, s_end2, g_end)
    first = oracle.backward_state(w, u, k[:, :cut], v[:, :cut], dy[:, :cut], s0, s_mid, second[4])
    np.testing.assert_allclose(np.concatenate([first[0], second[0]], axis=1), full[0],
                               rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(np.concatenate([first[1], second[1]], axis=1), full[1],
                               rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(first[2] + second[2], full[2], rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(first[3] + second[3], full[3], rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(first[4], full[4], rtol=1e-9, atol=1e-12)


# Magnitudes of dw's and du's terms: the scale the GPU tests' round-off bound
# for these cancelling sums is taken from.

def _magnitude_pairwise(w, u, k, v, dy, s_in=None, s_out=None, g_state=None):
    """The sums of wkvo_backward_magnitude written out term by term from the
    closed form ("WKV mechanism: core computation", with the carried state's
    weight e^{-t w}), O(T^2) per lane, no scan."""
    B, T, C = k.shape
    mdw, mdu = np.zeros(C), np.zeros(C)
    for b in range(B):
        for c in range(C):
            wc, uc = w[c], u[c]
            A0 = B0 = 0.0
            if s_in is not None and s_in[1, b, c] > 0:
                A0 = s_in[0, b, c] * np.exp(s_in[2, b, c])
                B0 = s_in[1, b, c] * np.exp(s_in[2, b, c])
            kk, vv, gg = k[b, :, c], v[b, :, c], np.abs(dy[b, :, c])
            for t in range(T):
                past = np.exp(kk[:t] - (t - 1 - np.arange(t)) * wc)
                bonus = np.exp(uc + kk[t])
                st = np.exp(-t * wc)
                D = st * B0 + past.sum() + bonus
                y = (st * A0 + (past * vv[:t]).sum() + bonus * vv[t]) / D
                mdu[c] += gg[t] * bonus / D * (abs(vv[t]) + abs(y))
                mdw[c] += (gg[t] * (t - 1 - np.arange(t)) * past / D * (np.abs(vv[:t]) + abs(y))).sum()
                mdw[c] += t * gg[t] * st * (abs(A0) + abs(y) * B0) / D
            if g_state is not None:
                gA = g_state[0, b, c] * np.exp(-s_out[2, b, c])
                gB = g_state[1, b, c] * np.exp(-s_out[2, b, c])
                dist = T - 1 - np.arange(T)
                e = np.exp(kk - dist * wc)
                mdw[c] += (dist * e * (np.abs(gA * vv) + abs(gB))).sum()
                mdw[c] += T * np.exp(-T * wc) * (abs(gA * A0) + abs(gB) * B0)
    return mdw, mdu


@pytest.mark.parametrize("recipe", [synth.GPT, synth.STABILITY])
@pytest.mark.parametrize("with_state", [False, True])
def test_backward_magnitude_matches_pairwise_sums(oracle, recipe, with_state):
    B, T, C = 2, 23, 3
    d = synth.make(recipe, index=41, B=B, T=T, C=C, with_dy=True)
    d = {n: t.double().numpy() for n, t in d.items()}
    w, u, k, v, dy = d["w"], d["u"], d["k"], d["v"], d["dy"]
    s_in = s_out = g = None
    if with_state:
        s_in = rand_state(oracle, 42, B, C)
        _, s_out = oracle.forward_brute(w, u, k, v, s_in)
        g = np.random.default_rng(43).normal(size=(3, B, C))
    mdw, mdu = oracle.backward_magnitude(w, u, k, v, dy, s_in, s_out, g)
    rw, ru = _magnitude_pairwise(w, u, k, v, dy, s_in, s_out, g)
    np.testing.assert_allclose(mdw, rw, rtol=1e-10)
    np.testing.assert_allclose(mdu, ru, rtol=1e-10)
    # never below the gradients themselves (every term counted by size)
    _, _, dw, du, _ = oracle.backward_state(w, u, k, v, dy, s_in, s_out, g)
    assert np.all(mdw >= np.abs(dw) * (1 - 1e-12))
    assert np.all(mdu >= np.abs(du) * (1 - 1e-12))


def test_backward_magnitude_one_token_closed_form(oracle):
    """One token from the empty state: the output is v itself (its weight is
    the whole denominator), du's term dy (v - y) vanishes while its two parts
    are |dy| |v| each, and there is no pair for dw."""
    B, T, C = 3, 1, 5
    d = synth.make(synth.STABILITY, index=44, B=B, T=T, C=C, with_dy=True)
    w, u, k, v, dy = (d[n].double().numpy() for n in ("w", "u", "k", "v", "dy"))
    mdw, mdu = oracle.backward_magnitude(w, u, k, v, dy)
    np.testing.assert_allclose(mdu, 2.0 * np.sum(np.abs(dy * v), axis=(0, 1)), rtol=1e-12)
    np.testing.assert_array_equal(mdw, np.zeros(C))
    _, _, dw, du, _ = oracle.backward_state(w, u, k, v, dy)
    assert np.all(np.abs(du) <= 1e-12 * mdu)

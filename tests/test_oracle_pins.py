"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Source: "Pretraining Transformers with Quantized Softmax in Attention"
(paperlayer digest).  The pages print no worked numeric example, so the oracle
is pinned by closed forms, brute force, interpolation bounds, the softmax
limit (a library routine), finite differences of its own forward, an
independent autograd re-expression, and the identities the pages state.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle as O
from oracle import Params

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "calibration_constants.json")


def rand_row(rng, n, scale=1.0):
    return rng.standard_normal(n) * scale


# --------------------------------------------------------------------------
# calibration constants (App. A; App. C.3)
# --------------------------------------------------------------------------

def test_golden_calibration_constants():
    g = json.load(open(GOLDEN))
    s = np.array([0.3, -2.0, 1.1, 0.0])
    cal = O.calibrate(s, Params(K=4, tau=g["fwm_tau"]["value"], calibration=O.FWM))
    assert cal.h == g["fwm_K4_h"]["value"]
    cal = O.calibrate(s, Params(K=4, calibration=O.MINMAX))
    assert cal.h == pytest.approx(g["minmax_K4_h_over_span"]["value"] * (1.1 + 2.0), rel=1e-15)
    assert cal.m == 1.1 and cal.a == 2 and cal.n == -2.0 and cal.b == 1
    assert len(O.grid(1.5, 4)) == g["grid_values_for_K"]["K4_levels"]
    assert O.EPS_SPAN == g["eps_span"]["value"]


def test_extremum_ties_take_lowest_index():
    s = np.array([1.0, 3.0, -1.0, 3.0, -1.0])
    cal = O.calibrate(s, Params(K=4))
    assert (cal.a, cal.b) == (1, 2)


# --------------------------------------------------------------------------
# LERP forward: grid exactness, K = 1 closed form, interpolation bound
# --------------------------------------------------------------------------

def test_lerp_exact_on_grid_points():
    K, h0 = 8, 0.37
    s = -h0 * np.array([0, 3, 1, 8, 5, 2, 7, 4, 6], dtype=np.float64)
    fw = O.row_forward(s, Params(K=K))
    assert fw.cal.h == pytest.approx(h0, rel=1e-15)
    u = -s / h0
    np.testing.assert_allclose(fw.w, np.exp(-u * h0), rtol=1e-14, atol=0)


def test_lerp_k1_closed_form():
    rng = np.random.default_rng(1)
    s = rand_row(rng, 40, 2.0)
    fw = O.row_forward(s, Params(K=1))
    span = s.max() - s.min()
    ref = 1.0 - (1.0 - math.exp(-span)) * (s.max() - s) / span
    np.testing.assert_allclose(fw.w, ref, rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("K", [2, 4, 16, 32])
@pytest.mark.parametrize("cal", [O.MINMAX, O.FWM])
def test_lerp_interpolation_error_bound(K, cal):
    """|wL - exp(s - m)| <= h^2/8 * exp(-i h) on segment i (linear interpolation
    of a convex function; its second derivative is at most exp(-i h))."""
    rng = np.random.default_rng(2)
    s = rand_row(rng, 500, 3.0)
    p = Params(K=K, calibration=cal)
    fw = O.row_forward(s, p)
    rec, h = fw.rec, fw.cal.h
    z = s - fw.cal.m
    inwin = rec.mask > 0
    err = np.abs(fw.w - np.exp(z))[inwin]
    bound = (h * h / 8.0) * np.exp(-rec.i * h)[inwin]
    assert np.all(err <= bound * (1 + 1e-12) + 1e-300)
    # LERP never undershoots the exponential (convexity)
    assert np.all(fw.w[inwin] >= np.exp(z[inwin]) * (1 - 1e-14))


# --------------------------------------------------------------------------
# Nearest forward: brute force and relative bound
# --------------------------------------------------------------------------

@pytest.mark.parametrize("K", [1, 4, 16])
def test_nearest_matches_brute_force(K):
    rng = np.random.default_rng(3)
    s = rand_row(rng, 300, 4.0)
    p = Params(K=K, reconstruction=O.NEAREST)
    fw = O.row_forward(s, p)
    h, m = fw.cal.h, fw.cal.m
    u = (m - s) / h
    pts = np.arange(K + 1)
    for j in range(len(s)):
        dist = np.abs(u[j] - pts)
        best = np.flatnonzero(dist == dist.min())
        assert fw.rec.r[j] == best.max()       # R1: a half-way score goes to the higher index
        assert fw.w[j] == pytest.approx(math.exp(-best.max() * h), rel=4e-16)


def test_nearest_half_way_rounds_up_in_u():
    K, h0 = 4, 1.0
    s = np.array([0.0, -0.5, -1.5, -2.5, -3.5, -4.0])
    fw = O.row_forward(s, Params(K=K, reconstruction=O.NEAREST))
    assert fw.cal.h == h0
    assert list(fw.rec.r) == [0, 1, 2, 3, 4, 4]


@pytest.mark.parametrize("K", [2, 4, 32])
def test_nearest_relative_bound(K):
    rng = np.random.default_rng(4)
    s = rand_row(rng, 400, 3.0)
    fw = O.row_forward(s, Params(K=K, reconstruction=O.NEAREST))
    rel = np.abs(fw.w / np.exp(s - fw.cal.m) - 1.0)
    assert np.all(rel <= math.expm1(fw.cal.h / 2) * (1 + 1e-12))


def test_nearest_is_normalised_not_one_hot():
    s = np.array([0.0, -0.1, -0.2, -5.0])
    fw = O.row_forward(s, Params(K=4, reconstruction=O.NEAREST))
    assert fw.P.sum() == pytest.approx(1.0, abs=1e-15)
    assert np.count_nonzero(fw.P) == 4


# --------------------------------------------------------------------------
# FWM window, degenerate rows, single key
# --------------------------------------------------------------------------

def test_fwm_tail_zero_weight_and_inert():
    rng = np.random.default_rng(5)
    s = rand_row(rng, 60, 4.0)
    p = Params(K=4, tau=6.0, calibration=O.FWM)
    fw = O.row_forward(s, p)
    tail = s < fw.cal.m - 6.0
    assert tail.any() and (~tail).sum() > 2
    assert np.all(fw.w[tail] == 0) and np.all(fw.w[~tail] > 0)
    dP = rng.standard_normal(60)
    bw = O.row_backward(fw, dP, p)
    assert np.all(bw.dS[tail] == 0)
    # moving a tail key (the row min among them) further down changes nothing
    s2 = s.copy()
    s2[np.argmin(s)] -= 17.0
    fw2 = O.row_forward(s2, p)
    bw2 = O.row_backward(fw2, dP, p)
    np.testing.assert_array_equal(fw2.P, fw.P)
    np.testing.assert_array_equal(bw2.dS, bw.dS)


def test_fwm_window_edge_inclusive():
    s = np.array([0.0, -6.0, -6.0 - 1e-9])
    fw = O.row_forward(s, Params(K=4, calibration=O.FWM))
    assert fw.w[1] == pytest.approx(math.exp(-6.0), rel=1e-15) and fw.w[2] == 0


@pytest.mark.parametrize("rec", [O.LERP, O.NEAREST])
def test_degenerate_span_uniform(rec):
    s = np.full(7, 0.25)
    p = Params(K=4, reconstruction=rec)
    fw = O.row_forward(s, p)
    assert fw.cal.degenerate
    np.testing.assert_array_equal(fw.P, np.full(7, 1 / 7))
    dP = np.arange(7.0)
    bw = O.row_backward(fw, dP, p)
    np.testing.assert_allclose(bw.dS, (dP - dP.mean()) / 7, atol=1e-15)
    assert bw.Cm == 0 and bw.Cn == 0


def test_single_key_row():
    Q = np.array([[0.3, -1.0]])
    Kt = np.array([[2.0, 0.5]])
    V = np.array([[1.5, -2.5]])
    dO = np.array([[0.7, 0.1]])
    for p in [Params(K=4), Params(K=4, calibration=O.FWM), Params(K=4, reconstruction=O.NEAREST)]:
        r = O.head_backward(Q, Kt, V, dO, p)
        np.testing.assert_array_equal(O.head_forward(Q, Kt, V, p)["O"], V)
        assert np.all(r["dQ"] == 0) and np.all(r["dK"] == 0)
        np.testing.assert_array_equal(r["dV"], dO)


# --------------------------------------------------------------------------
# K -> infinity: exp recovered (softmax attention is a library routine)
# --------------------------------------------------------------------------

def _softmax_attention(Q, Kt, V, dO):
    import torch
    q, k, v = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (Q, Kt, V))
    o = torch.nn.functional.scaled_dot_product_attention(q[None, None], k[None, None], v[None, None],
                                                          is_causal=True)[0, 0]
    (o * torch.tensor(dO, dtype=torch.float64)).sum().backward()
    return o.detach().numpy(), q.grad.numpy(), k.grad.numpy(), v.grad.numpy()


def _small_head(seed, T=24, d=8, qs=1.5):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((T, d)) * qs, rng.standard_normal((T, d)),
            rng.standard_normal((T, d)), rng.standard_normal((T, d)))


def test_forward_converges_to_softmax_quadratically():
    Q, Kt, V, dO = _small_head(6)
    Osm, *_ = _softmax_attention(Q, Kt, V, dO)
    errs = []
    for K in (256, 512, 1024, 2048):
        Ok = O.head_forward(Q, Kt, V, Params(K=K))["O"]
        errs.append(np.abs(Ok - Osm).max())
    # second order: about 4x per halving of h, averaged over three halvings
    # (single steps wobble with where the scores fall relative to the knots)
    rate = (errs[0] / errs[-1]) ** (1.0 / 3.0)
    assert 3.3 < rate < 4.8, errs
    assert all(errs[i + 1] < errs[i] for i in range(len(errs) - 1)), errs
    assert errs[-1] < 1e-6


def test_backward_converges_to_softmax_gradient():
    Q, Kt, V, dO = _small_head(7)
    _, gq, gk, gv = _softmax_attention(Q, Kt, V, dO)
    errs = []
    for K in (128, 256, 512, 1024):
        r = O.head_backward(Q, Kt, V, dO, Params(K=K))
        errs.append(max(np.abs(r["dQ"] - gq).max(), np.abs(r["dK"] - gk).max(), np.abs(r["dV"] - gv).max()))
    assert all(errs[i + 1] < errs[i] * 0.7 for i in range(len(errs) - 1)), errs
    assert errs[-1] < 5e-3 * max(np.abs(gq).max(), np.abs(gk).max())


def test_fwm_converges_to_truncated_softmax():
    """FWM with large K tends to softmax restricted to the tau window."""
    rng = np.random.default_rng(8)
    s = rand_row(rng, 200, 3.0)
    fw = O.row_forward(s, Params(K=4096, tau=6.0, calibration=O.FWM))
    e = np.exp(s - s.max()) * (s >= s.max() - 6.0)
    np.testing.assert_allclose(fw.P, e / e.sum(), atol=2e-8)


# --------------------------------------------------------------------------
# gradient identities (section 3 "Calibration gradients"; App. B)
# --------------------------------------------------------------------------

ALL_SURROGATES = [(O.LERP, O.WEIGHT_STE), (O.NEAREST, O.WEIGHT_STE), (O.NEAREST, O.PROB_STE)]


@pytest.mark.parametrize("cal", [O.MINMAX, O.FWM])
@pytest.mark.parametrize("rec,ste", ALL_SURROGATES)
@pytest.mark.parametrize("K", [1, 4, 32])
def test_full_gradient_zero_sum(cal, rec, ste, K):
    rng = np.random.default_rng(9)
    for _ in range(5):
        s = rand_row(rng, 80, 3.0)
        dP = rng.standard_normal(80)
        p = Params(K=K, calibration=cal, reconstruction=rec, surrogate=ste, grad_rule=O.FULL)
        bw = O.row_backward(O.row_forward(s, p), dP, p)
        assert abs(bw.dS.sum()) <= 1e-12 * np.abs(bw.dS).sum()


@pytest.mark.parametrize("cal", [O.MINMAX, O.FWM])
def test_detach_breaks_zero_sum_and_p1_restores_it(cal):
    rng = np.random.default_rng(10)
    s = rand_row(rng, 80, 3.0)
    dP = rng.standard_normal(80)
    pd = Params(K=8, calibration=cal, grad_rule=O.DETACH)
    bd = O.row_backward(O.row_forward(s, pd), dP, pd)
    assert abs(bd.dS.sum()) > 1e-3 * np.abs(bd.dS).sum()
    pp = Params(K=8, calibration=cal, grad_rule=O.P1)
    bp = O.row_backward(O.row_forward(s, pp), dP, pp)
    assert abs(bp.dS.sum()) <= 1e-13 * np.abs(bp.dS).sum()
    np.testing.assert_allclose(bp.dS - bd.dS, np.full(80, -bd.dS.mean()), atol=1e-15)


def test_fwm_rule_algebra():
    """Under FWM the min plays no role: min-only = detach, max-only = full."""
    rng = np.random.default_rng(11)
    s = rand_row(rng, 50, 3.0)
    dP = rng.standard_normal(50)
    out = {}
    for rule in (O.FULL, O.DETACH, O.MAX_ONLY, O.MIN_ONLY):
        p = Params(K=4, calibration=O.FWM, grad_rule=rule)
        out[rule] = O.row_backward(O.row_forward(s, p), dP, p).dS
    np.testing.assert_array_equal(out[O.MIN_ONLY], out[O.DETACH])
    np.testing.assert_array_equal(out[O.MAX_ONLY], out[O.FULL])


@pytest.mark.parametrize("rec,ste", ALL_SURROGATES)
def test_forward_independent_of_rule_and_placement(rec, ste):
    Q, Kt, V, _ = _small_head(12)
    base = O.head_forward(Q, Kt, V, Params(K=4, reconstruction=rec, surrogate=ste))["O"]
    for rule in (O.DETACH, O.MAX_ONLY, O.MIN_ONLY, O.P1):
        o = O.head_forward(Q, Kt, V, Params(K=4, reconstruction=rec, surrogate=ste, grad_rule=rule))["O"]
        np.testing.assert_array_equal(o, base)
    if rec == O.NEAREST:
        other = O.PROB_STE if ste == O.WEIGHT_STE else O.WEIGHT_STE
        o = O.head_forward(Q, Kt, V, Params(K=4, reconstruction=rec, surrogate=other))["O"]
        np.testing.assert_array_equal(o, base)


def test_ste_backwards_coincide_on_grid_points():
    """Scores on grid points: hard and interpolated weights agree, so both
    placements and LERP give the same backward (section 3, Surrogate placement)."""
    K, h0 = 4, 0.75
    rng = np.random.default_rng(13)
    ks = rng.integers(0, K + 1, size=30)
    ks[0], ks[1] = 0, K
    s = 1.25 - h0 * ks
    dP = rng.standard_normal(30)
    res = []
    for rec, ste in ALL_SURROGATES:
        p = Params(K=K, reconstruction=rec, surrogate=ste)
        res.append(O.row_backward(O.row_forward(s, p), dP, p).dS)
    np.testing.assert_allclose(res[1], res[0], rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(res[2], res[0], rtol=1e-13, atol=1e-16)


@pytest.mark.parametrize("rec,ste", ALL_SURROGATES)
def test_weighted_orthogonality_at_evaluation_point(rec, ste):
    rng = np.random.default_rng(14)
    s = rand_row(rng, 70, 3.0)
    dP = rng.standard_normal(70)
    p = Params(K=4, reconstruction=rec, surrogate=ste)
    fw = O.row_forward(s, p)
    bw = O.row_backward(fw, dP, p)
    we = fw.wL if (rec == O.NEAREST and ste == O.PROB_STE) else fw.w
    assert abs(np.dot(bw.gt, we)) < 1e-13 * np.abs(bw.gt).sum()
    if rec == O.NEAREST:   # the other placement's weights are not orthogonal in general
        wo = fw.w if ste == O.PROB_STE else fw.wL
        assert abs(np.dot(bw.gt, wo)) > 1e-8 * np.abs(bw.gt).sum()


# --------------------------------------------------------------------------
# untruncated fixed step (App. D.4) and the exact-softmax reference (App. D.5)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("rec,ste", ALL_SURROGATES)
@pytest.mark.parametrize("rule", [O.FULL, O.DETACH])
def test_untruncated_equals_fwm_inside_the_window(rec, ste, rule):
    """With every score within tau of the max the tail is empty, so the
    untruncated step and FWM coincide, forward and backward."""
    rng = np.random.default_rng(41)
    s = rng.uniform(-5.5, 0.0, 30)
    s[3] = 0.0
    dP = rng.standard_normal(30)
    kw = dict(K=8, tau=6.0, reconstruction=rec, surrogate=ste, grad_rule=rule)
    fa, fb = O.row_forward(s, Params(calibration=O.FWM, **kw)), O.row_forward(s, Params(calibration=O.FWM_UNTRUNC, **kw))
    np.testing.assert_array_equal(fa.w, fb.w)
    ba = O.row_backward(fa, dP, Params(calibration=O.FWM, **kw))
    bb = O.row_backward(fb, dP, Params(calibration=O.FWM_UNTRUNC, **kw))
    np.testing.assert_allclose(bb.dS, ba.dS, rtol=0, atol=1e-15)


def test_untruncated_tail_key_closed_form():
    """A key 2.5 steps past the window edge lies on segment K+2 at f = 1/2: its
    LERP weight is the mean of exp(-(K+2) h) and exp(-(K+3) h) (nonzero, where
    FWM gives 0); Nearest rounds it up to exp(-(K+3) h)."""
    K, tau = 4, 6.0
    h = tau / K
    s = np.array([0.0, -0.3, -(K + 2.5) * h])
    pl = Params(K=K, tau=tau, calibration=O.FWM_UNTRUNC)
    w = O.row_forward(s, pl).w
    assert w[2] == pytest.approx(0.5 * (np.exp(-(K + 2) * h) + np.exp(-(K + 3) * h)), rel=1e-12)
    assert O.row_forward(s, Params(K=K, tau=tau, calibration=O.FWM)).w[2] == 0.0
    wn = O.row_forward(s, Params(K=K, tau=tau, calibration=O.FWM_UNTRUNC, reconstruction=O.NEAREST)).w
    assert wn[2] == pytest.approx(np.exp(-(K + 3) * h), rel=1e-12)


def test_untruncated_converges_to_softmax():
    """With tau fixed and K growing the step h = tau/K shrinks and no key is
    dropped, so P tends to softmax(s) with the LERP error O(h^2): each doubling
    of K cuts the error by about 4."""
    from scipy.special import softmax
    rng = np.random.default_rng(43)
    s = rng.standard_normal(40) * 4.0
    ref = softmax(s)
    errs = [np.abs(O.row_forward(s, Params(K=K, tau=3.0, calibration=O.FWM_UNTRUNC)).P - ref).max()
            for K in (8, 16, 32, 64)]
    rates = [errs[i] / errs[i + 1] for i in range(3)]
    assert np.mean(rates) == pytest.approx(4.0, rel=0.2), rates
    assert errs[-1] < 1e-3


@pytest.mark.parametrize("rule", [O.FULL, O.DETACH, O.MAX_ONLY, O.MIN_ONLY, O.P1])
def test_exact_reference_is_softmax(rule):
    """The exact reference is softmax attention: P = softmax(s) (a library
    routine) and, under every rule, dS = P (dP - P.dP), the softmax
    Jacobian, which already sums to zero."""
    from scipy.special import softmax
    rng = np.random.default_rng(44)
    s = rng.standard_normal(25) * 3.0
    dP = rng.standard_normal(25)
    p = Params(K=4, reconstruction=O.EXACT, grad_rule=rule)
    fw = O.row_forward(s, p)
    P = softmax(s)
    np.testing.assert_allclose(fw.P, P, rtol=1e-13, atol=0)
    bw = O.row_backward(fw, dP, p)
    np.testing.assert_allclose(bw.dS, P * (dP - P @ dP), rtol=0, atol=1e-14)


# ---------------------------------------------------------------------------
# reduced-precision exponential baselines (App. D.5; reading R14)
# ---------------------------------------------------------------------------

def _format_probe_values():
    """fp32 values over the range the rounded exponentials take: random values
    across the exponent range, their neighbours, and exact ties of both
    formats (so round-half-even is exercised)."""
    rng = np.random.default_rng(61)
    x = np.exp(-rng.uniform(0, 40, 20000))
    ties = []
    for frac_bits, emin in ((7, -126), (3, -6)):
        for E in range(-12, 0):
            q = 2.0 ** (max(E, emin) - frac_bits)
            for k in range(0, 2 ** (frac_bits + 1)):
                v = 2.0 ** E + (k + 0.5) * q
                if v < 2.0 ** (E + 1):
                    ties.append(v)
        for k in range(0, 16):                      # subnormal ties of E4M3
            ties.append((k + 0.5) * 2.0 ** -9)
    return np.concatenate([x, np.array(ties), [0.0, 1.0]]).astype(np.float32)


@pytest.mark.parametrize("rec", [O.EXP_BF16, O.EXP_FP8])
def test_rounding_matches_torch_casts(rec):
    """round_to_format against torch's own round-to-nearest-even casts of
    fp32 values to bfloat16 and float8_e4m3fn (library routines)."""
    import torch
    x = _format_probe_values()
    fmt = torch.bfloat16 if rec == O.EXP_BF16 else torch.float8_e4m3fn
    want = torch.from_numpy(x).to(fmt).to(torch.float64).numpy()
    got = O.round_to_format(x.astype(np.float64), *O.FORMATS[rec])
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, [(float(x[i]), got[i], want[i]) for i in bad[:5]]


@pytest.mark.parametrize("rec", [O.EXP_BF16, O.EXP_FP8])
def test_rounded_exponential_on_representable_row_is_softmax(rec):
    """Scores at m - j ln 2 have exponentials 2^-j, exact in both formats
    (down to 2^-9 for E4M3), so the rounded baseline is softmax there."""
    j = np.array([0, 1, 3, 2, 5, 9, 0, 4])
    s = 1.5 - j * math.log(2.0)
    p = Params(K=4, reconstruction=rec)
    fw = O.row_forward(s, p)
    np.testing.assert_array_equal(fw.w, 2.0 ** -j)
    w = 2.0 ** -j
    np.testing.assert_allclose(fw.P, w / w.sum(), rtol=1e-15, atol=0)


def test_fp8_exponential_underflow_closed_form():
    """E4M3 keeps nothing below half its smallest subnormal 2^-9: a key 8 nats
    below the max (e^-8 < 2^-10) gets P = 0, yet straight-through still gives
    it the direct term (dP - delta) e^-8 / W; a key ln 2 below gets 1/2."""
    s = np.array([0.0, -8.0, -math.log(2.0)])
    dP = np.array([0.3, -1.2, 0.7])
    for rule in (O.FULL, O.DETACH):
        p = Params(K=4, reconstruction=O.EXP_FP8, grad_rule=rule)
        fw = O.row_forward(s, p)
        np.testing.assert_array_equal(fw.w, [1.0, 0.0, 0.5])
        W = 1.5
        P = np.array([1.0, 0.0, 0.5]) / W
        delta = P @ dP
        bw = O.row_backward(fw, dP, p)
        e = np.exp(s)
        direct = (dP - delta) * e / W
        want = direct.copy()
        if rule == O.FULL:
            want[0] = direct[0] - direct.sum()          # the max carries -sum(direct)
        np.testing.assert_allclose(bw.dS, want, rtol=1e-14, atol=1e-16)


@pytest.mark.parametrize("rec", [O.EXP_BF16, O.EXP_FP8])
def test_rounded_exponential_zero_sum_under_full_only(rec):
    rng = np.random.default_rng(62)
    s = rng.standard_normal(30) * 3
    dP = rng.standard_normal(30)
    full = O.row_backward(O.row_forward(s, Params(K=4, reconstruction=rec)), dP, Params(K=4, reconstruction=rec))
    assert abs(full.dS.sum()) <= 1e-14 * np.abs(full.dS).sum()
    pd = Params(K=4, reconstruction=rec, grad_rule=O.DETACH)
    det = O.row_backward(O.row_forward(s, pd), dP, pd)
    # the rounding leaves sum_j P_j dP_j - delta * sum_j e_j / W != 0 under detach
    assert abs(det.dS.sum()) > 1e-6 * np.abs(det.dS).sum()


def test_equal_keys_score_equally():
    """Equal keys get bitwise-equal scores wherever they sit in the row, so
    the lowest-index rule decides their ties (reading R3)."""
    rng = np.random.default_rng(12)
    for d in (5, 64, 128):
        keys = (rng.standard_normal((700, d)) * 0.2).astype(np.float32)
        keys[[3, 64, 65, 333, 699]] = rng.standard_normal(d).astype(np.float32)
        q = rng.standard_normal(d).astype(np.float32)
        s = O.row_scores(q, keys)
        assert len(set(s[[3, 64, 65, 333, 699]].tolist())) == 1
        q_max = keys[3] * 10
        cal = O.calibrate(O.row_scores(q_max, keys), Params(K=4))
        assert cal.a == 3

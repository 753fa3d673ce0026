"""Pins of the oracle's whole-tensor entry points and of its per-key decision
override, against closed forms and the pinned per-row / per-head functions.

The decision override evaluates the operator with a rounding decision taken
the other way at a key whose u (or exponential) lies within rounding of a
boundary; the GPU parity tests use it to accept either admissible decision.
Source: "Pretraining Transformers with Quantized Softmax in Attention"
(paperlayer digest), section 3 "Reconstruction" and App. A (grid points,
segments, window), App. D.5 (rounded exponentials).
"""
import numpy as np
import pytest

import oracle as O
from oracle import Params
from tests.test_oracle_gradients import mutated_oracle


def _distinct_slices(B=3, H=3, T=9, d=5, seed=4):
    """[B, H, T, d] inputs whose slices all differ in scale, so any mix-up of
    the batch and head indices changes the result."""
    rng = np.random.default_rng(seed)
    q, k, v, do = (rng.standard_normal((B, H, T, d)) for _ in range(4))
    for b in range(B):
        for h in range(H):
            q[b, h] *= 0.5 + b + 0.3 * h
            v[b, h] += 10.0 * b - 3.0 * h
    return q, k, v, do


def check_whole_tensor(mod, p):
    """forward / backward over [B, H, T, d] equal the per-head functions on
    every (b, h) slice (slices are independent: no state crosses heads)."""
    q, k, v, do = _distinct_slices()
    B, H = q.shape[:2]
    o, st = mod.forward(q, k, v, p)
    g = mod.backward(q, k, v, do, p)
    for b in range(B):
        for h in range(H):
            hf = mod.head_forward(q[b, h], k[b, h], v[b, h], p)
            hb = mod.head_backward(q[b, h], k[b, h], v[b, h], do[b, h], p)
            assert np.array_equal(o[b, h], hf["O"]), (b, h)
            for key in ("m", "n", "a", "b", "W"):
                assert np.array_equal(st[key][b, h], hf["stats"][key]), (key, b, h)
            for key in ("dQ", "dK", "dV", "Cm", "Cn", "dS_sum"):
                assert np.array_equal(g[key][b, h], hb[key]), (key, b, h)


@pytest.mark.parametrize("rec", [O.LERP, O.NEAREST])
def test_whole_tensor_entry_points_match_heads(rec):
    check_whole_tensor(O, Params(K=4, reconstruction=rec, surrogate=O.PROB_STE))


@pytest.mark.parametrize("old,new", [
    ("r = head_forward(q[bi, hi], k[bi, hi], v[bi, hi], p)", "r = head_forward(q[hi, bi], k[hi, bi], v[hi, bi], p)"),
    ("            O[bi, hi] = r[\"O\"]", "            O[hi, bi] = r[\"O\"]"),
    ("r = head_backward(q[bi, hi], k[bi, hi], v[bi, hi], do[bi, hi], p)",
     "r = head_backward(q[bi, hi], k[bi, hi], v[bi, hi], do[hi, bi], p)"),
    ("                out[key][bi, hi] = r[key]", "                out[key][hi, bi] = r[key]"),
], ids=["forward reads (h, b)", "forward writes (h, b)", "backward reads dO of (h, b)", "backward writes (h, b)"])
def test_whole_tensor_index_swap_is_caught(old, new):
    p = Params(K=4)
    check_whole_tensor(O, p)
    with pytest.raises(AssertionError):
        check_whole_tensor(mutated_oracle(old, new), p)


# ---------------------------------------------------------------------------
# decision override
# ---------------------------------------------------------------------------

def _row(seed=3, n=23, scale=2.0):
    rng = np.random.default_rng(seed)
    return rng.standard_normal(n) * scale, rng.standard_normal(n)


def _own_decisions(fw, p):
    if p.reconstruction in O.FORMATS:
        e = np.exp(fw.s - fw.cal.m)
        return {j: int(fw.w[j] > e[j]) for j in range(len(e))}
    rec = fw.rec
    lev = rec.i if p.reconstruction == O.LERP else rec.r
    return {j: (int(lev[j]) if rec.mask[j] > 0 else -1) for j in range(len(lev))}


@pytest.mark.parametrize("cal,rec,ste", [(O.MINMAX, O.LERP, O.WEIGHT_STE), (O.FWM, O.LERP, O.WEIGHT_STE),
                                         (O.MINMAX, O.NEAREST, O.PROB_STE), (O.FWM, O.NEAREST, O.WEIGHT_STE),
                                         (O.FWM_UNTRUNC, O.NEAREST, O.PROB_STE), (O.MINMAX, O.EXP_BF16, O.WEIGHT_STE),
                                         (O.MINMAX, O.EXP_FP8, O.WEIGHT_STE)])
def test_own_decisions_change_nothing(cal, rec, ste):
    s, dP = _row()
    p = Params(K=4, tau=2.0, calibration=cal, reconstruction=rec, surrogate=ste)
    fw = O.row_forward(s, p)
    fw2 = O.row_forward(s, p, _own_decisions(fw, p))
    bw, bw2 = O.row_backward(fw, dP, p), O.row_backward(fw2, dP, p)
    assert np.array_equal(fw.w, fw2.w) and np.array_equal(fw.P, fw2.P)
    assert np.array_equal(bw.dS, bw2.dS)


def test_nearest_forced_point_closed_form():
    """A key moved to the next grid point takes exactly exp(-(r+1) h); every
    other weight is unchanged."""
    s, _ = _row()
    p = Params(K=4, reconstruction=O.NEAREST)
    fw = O.row_forward(s, p)
    j = int(np.flatnonzero(fw.rec.r < p.K)[0])
    r1 = int(fw.rec.r[j]) + 1
    fw2 = O.row_forward(s, p, {j: r1})
    assert fw2.w[j] == np.exp(-r1 * fw.cal.h)
    others = np.arange(len(s)) != j
    assert np.array_equal(fw2.w[others], fw.w[others])
    assert fw2.W == pytest.approx(fw.W - fw.w[j] + fw2.w[j], rel=1e-15)


def test_lerp_forced_segment_at_a_knot():
    """At an exact knot u = k the two segments give the same weight, and the
    left one's direct term is the secant slope of its own segment:
    dS_j = gt_j (g_{k-1} - g_k) / h."""
    K, h0 = 6, 0.5          # exact binary fractions: u = 2 is an exact knot
    u = np.array([0.0, 2.0, 3.5, 6.0, 1.25])
    s = -h0 * u
    p = Params(K=K)
    rng = np.random.default_rng(8)
    dP = rng.standard_normal(len(s))
    fw = O.row_forward(s, p)
    assert fw.rec.i[1] == 2
    fw2 = O.row_forward(s, p, {1: 1})
    np.testing.assert_allclose(fw2.w, fw.w, rtol=1e-14, atol=0)
    bw2 = O.row_backward(fw2, dP, p)
    h = fw.cal.h
    expect = bw2.gt[1] * (np.exp(-1 * h) - np.exp(-2 * h)) / h
    assert bw2.dS_direct[1] == pytest.approx(expect, rel=1e-13)
    bw = O.row_backward(fw, dP, p)
    expect_right = bw.gt[1] * (np.exp(-2 * h) - np.exp(-3 * h)) / h
    assert bw.dS_direct[1] == pytest.approx(expect_right, rel=1e-13)


@pytest.mark.parametrize("rec", [O.LERP, O.NEAREST])
def test_fwm_forced_window_edge(rec):
    """A key just outside the window forced in takes the last grid value
    exp(-K h); a key inside forced out takes zero weight and zero gradient."""
    K, tau = 4, 2.0
    h = tau / K
    s = np.array([0.0, -0.7, -(tau + 1e-9), -1.9, -0.2])
    p = Params(K=K, tau=tau, calibration=O.FWM, reconstruction=rec)
    fw = O.row_forward(s, p)
    assert fw.w[2] == 0.0 and fw.w[3] > 0.0
    fw2 = O.row_forward(s, p, {2: K if rec == O.NEAREST else K - 1, 3: -1})
    assert fw2.w[2] == pytest.approx(np.exp(-K * h), rel=1e-8)
    assert fw2.w[3] == 0.0
    bw2 = O.row_backward(fw2, np.arange(5.0), p)
    assert bw2.dS_direct[3] == 0.0


@pytest.mark.parametrize("rec", [O.EXP_BF16, O.EXP_FP8])
def test_rounded_exponential_forced_neighbours(rec):
    """Forcing a rounding direction picks the format value below or above
    exp(s - m); the two bracket it and are one quantum apart."""
    s, _ = _row(seed=9, n=40, scale=1.5)
    p = Params(K=1, reconstruction=rec)
    fw = O.row_forward(s, p)
    e = np.exp(s - fw.cal.m)
    lo, hi = O.format_neighbours(e, *O.FORMATS[rec])
    j = int(np.flatnonzero(lo < hi)[0])
    up = O.row_forward(s, p, {j: 1}).w[j]
    dn = O.row_forward(s, p, {j: 0}).w[j]
    assert dn <= e[j] <= up and dn < up
    assert O.round_to_format(np.array([up]), *O.FORMATS[rec])[0] == up
    assert O.round_to_format(np.array([dn]), *O.FORMATS[rec])[0] == dn
    assert fw.w[j] in (dn, up)
    assert fw.w[j] == (up if up - e[j] <= e[j] - dn else dn)

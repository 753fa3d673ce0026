"""Pins of the oracle's geometry probe (reading R13: section 4 "Geometry
probe", section 5.4 and App. D.6 of "Pretraining Transformers with Quantized
Softmax in Attention").

Each check takes the oracle module, so the mutation tests at the bottom can
run it against a copy with a planted mistake.  Expected values come from
closed forms worked out from the operator's definition (App. A), from SciPy's
own entropy and softmax routines, and from limits and orderings that hold for
any row; none comes from the oracle's probe itself.
"""
from __future__ import annotations

import importlib.util
import os
import sys

import numpy as np
import pytest
from scipy.special import softmax as sp_softmax
from scipy.stats import entropy as sp_entropy

import oracle as O

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "kia_oracle.py")


def _rows(seed=3, n=6, L=40):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal(L) * sc for sc in np.linspace(0.5, 6.0, n)]


def check_uniform(m):
    """A constant row: span 0, both distributions uniform, everything in the
    top bucket; MinMax reports width 0 (degenerate), FWM tau/K."""
    s = np.full(7, 1.25)
    for cal in (m.MINMAX, m.FWM, m.FWM_UNTRUNC):
        for rec in (m.LERP, m.NEAREST, m.EXACT):
            g = m.row_geometry(s, m.Params(K=4, tau=3.0, calibration=cal, reconstruction=rec))
            assert g.span == 0.0
            want_h = 0.75 if cal != m.MINMAX and rec != m.EXACT else 0.0
            assert g.h == want_h, (cal, rec, g.h)
            assert abs(g.entropy_p - np.log(7)) < 1e-14
            assert abs(g.entropy_soft - np.log(7)) < 1e-14
            assert g.tv < 1e-15 and abs(g.top_mass - 1.0) < 1e-15


def check_on_grid(m):
    """Scores that sit exactly on MinMax grid points are reconstructed exactly
    by LERP and Nearest, so P equals the softmax; the top bucket holds the
    two keys at the max."""
    h = 0.75
    j = np.array([0, 0, 1, 2, 3, 4, 4, 2])
    s = 2.0 - h * j                       # span 3 = K h with K = 4
    mass = np.exp(-h * j)
    for rec in (m.LERP, m.NEAREST):
        g = m.row_geometry(s, m.Params(K=4, reconstruction=rec))
        assert abs(g.h - h) < 1e-15 and abs(g.span - 3.0) < 1e-15
        assert g.tv < 1e-14
        assert abs(g.entropy_p - g.entropy_soft) < 1e-13
        assert abs(g.top_mass - 2.0 / mass.sum()) < 1e-14


def check_closed_form_k1(m):
    """MinMax K = 1 on scores 0, -0.4x, -0.7x, -x (u = 0, 0.4, 0.7, 1): the
    grid is {1, e^-x}; Nearest rounds u = 0.4 up to point 0 and u = 0.7 down
    to point 1; LERP with c = 1 - e^-x gives 1 - u c.  The top bucket is the
    keys with u < 1/2."""
    x = 2.0
    u = np.array([0.0, 0.4, 0.7, 1.0])
    s = -u * x
    soft = np.exp(s) / np.exp(s).sum()
    c = 1.0 - np.exp(-x)
    cases = {
        m.NEAREST: np.array([1.0, 1.0, np.exp(-x), np.exp(-x)]),
        m.LERP: 1.0 - u * c,
    }
    for rec, w in cases.items():
        P = w / w.sum()
        g = m.row_geometry(s, m.Params(K=1, reconstruction=rec))
        assert abs(g.h - x) < 1e-15
        assert abs(g.tv - 0.5 * np.abs(P - soft).sum()) < 1e-15, rec
        assert abs(g.entropy_p - sp_entropy(P)) < 1e-14, rec
        assert abs(g.entropy_soft - sp_entropy(soft)) < 1e-14, rec
        assert abs(g.top_mass - (soft[0] + soft[1])) < 1e-15, rec


def check_library_and_ranges(m):
    """Random rows under every operator: the softmax entropy is SciPy's on
    SciPy's softmax; the operator entropy is SciPy's on the operator's P;
    TV lies in [0, 1] and is the half L1 distance of the two; the top bucket
    is the keys above m - h/2 and always holds the argmax."""
    for s in _rows():
        for cal in (m.MINMAX, m.FWM, m.FWM_UNTRUNC):
            for rec in (m.LERP, m.NEAREST, m.EXACT):
                p = m.Params(K=4, tau=5.0, calibration=cal, reconstruction=rec)
                g = m.row_geometry(s, p)
                soft = sp_softmax(s)
                P = m.row_forward(s, p).P
                assert abs(g.entropy_soft - sp_entropy(soft)) < 1e-12
                assert abs(g.entropy_p - sp_entropy(P)) < 1e-12
                assert 0.0 <= g.tv <= 1.0
                assert abs(g.tv - 0.5 * np.abs(P - soft).sum()) < 1e-14
                assert 0.0 <= g.entropy_p <= np.log(len(s)) + 1e-12
                above = s > s.max() - g.h / 2
                assert abs(g.top_mass - soft[above].sum()) < 1e-14
                assert g.top_mass >= soft.max() - 1e-15
                assert abs(g.span - np.ptp(s)) < 1e-15
                if rec == m.EXACT:
                    assert g.tv < 1e-14 and abs(g.entropy_p - g.entropy_soft) < 1e-12
                    assert abs(g.h - np.ptp(s) / 4) < 1e-15


def check_widths(m):
    """MinMax's width follows the span, FWM's is tau/K whatever the span;
    MinMax's top bucket can only shrink as K grows."""
    for s in _rows(seed=5):
        for K in (1, 3, 16):
            gm = m.row_geometry(s, m.Params(K=K))
            gf = m.row_geometry(s, m.Params(K=K, tau=7.0, calibration=m.FWM))
            assert abs(gm.h - np.ptp(s) / K) < 1e-15
            assert gf.h == 7.0 / K
        tops = [m.row_geometry(s, m.Params(K=K)).top_mass for K in (1, 2, 4, 8, 64)]
        assert all(a >= b - 1e-15 for a, b in zip(tops, tops[1:]))


def check_softmax_limit(m):
    """As K grows, LERP and Nearest approach the softmax: TV -> 0 and the
    operator entropy -> the softmax entropy."""
    s = _rows(seed=9, n=1, L=60)[0] * 3
    for rec in (m.LERP, m.NEAREST):
        tvs = [m.row_geometry(s, m.Params(K=K, reconstruction=rec)).tv for K in (4, 64, 4096)]
        assert tvs[0] > tvs[1] > tvs[2]
        g = m.row_geometry(s, m.Params(K=65536, reconstruction=rec))
        assert g.tv < (1e-7 if rec == m.LERP else 1e-3)
        assert abs(g.entropy_p - g.entropy_soft) < (1e-7 if rec == m.LERP else 1e-3)


def check_norms(m):
    """Row norms belong to position t itself: Q_t = c_t e_0, K_t = 2 c_t e_1."""
    T, d = 5, 4
    c = np.arange(1.0, T + 1)
    Q = np.zeros((T, d))
    Kt = np.zeros((T, d))
    Q[:, 0] = c
    Kt[:, 1] = 2 * c
    g = m.head_geometry(Q, Kt, m.Params(K=2))
    assert np.allclose(g["q_norm"], c, rtol=0, atol=1e-15)
    assert np.allclose(g["k_norm"], 2 * c, rtol=0, atol=1e-15)
    # Q orthogonal to K: every score is 0, so each row is uniform over t+1 keys
    assert np.allclose(g["entropy_soft"], np.log(np.arange(1, T + 1)), rtol=0, atol=1e-14)


CHECKS = [check_uniform, check_on_grid, check_closed_form_k1, check_library_and_ranges,
          check_widths, check_softmax_limit, check_norms]


@pytest.mark.parametrize("check", CHECKS, ids=[c.__name__ for c in CHECKS])
def test_geometry_pin(check):
    check(O)


def test_geometry_whole_tensor_matches_heads():
    rng = np.random.default_rng(11)
    q, k = (rng.standard_normal((2, 3, 9, 8)).astype(np.float32) for _ in range(2))
    p = O.Params(K=4, reconstruction=O.NEAREST)
    whole = O.geometry(q, k, p)
    one = O.head_geometry(q[1, 2], k[1, 2], p)
    for f in O.GEOMETRY_FIELDS:
        assert np.array_equal(whole[f][1, 2], one[f])


# --------------------------------------------------------------------------
# mutation tests: a planted mistake in a copy of the oracle must trip a pin
# --------------------------------------------------------------------------

def _mutated(old, new):
    src = open(ORACLE_SRC).read()
    assert src.count(old) == 1, old
    name = f"kia_oracle_geo_mutant_{abs(hash(old)) % 10**8}"
    spec = importlib.util.spec_from_loader(name, loader=None)
    mod = importlib.util.module_from_spec(spec)
    sys.modules[name] = mod
    exec(compile(src.replace(old, new), ORACLE_SRC + " (mutant)", "exec"), mod.__dict__)
    return mod


MUTANTS = [
    ("total variation without the half",
     "tv=0.5 * float(np.abs(fw.P - soft).sum())", "tv=float(np.abs(fw.P - soft).sum())",
     check_closed_form_k1),
    ("softmax entropy taken from the operator's P",
     "entropy_soft=_entropy(soft)", "entropy_soft=_entropy(fw.P)",
     check_closed_form_k1),
    ("top bucket taken as the first LERP segment",
     "top = (m - s) / h < 0.5", "top = (m - s) / h < 1.0",
     check_closed_form_k1),
    ("FWM width from the span",
     "        h = p.tau / p.K\n    else:", "        h = span / p.K\n    else:",
     check_uniform),
    ("key norm of the previous position",
     "np.sqrt((K64[t] ** 2).sum())", "np.sqrt((K64[max(t - 1, 0)] ** 2).sum())",
     check_norms),
    ("softmax built from the operator's weights",
     "    e = np.exp(s - m)\n    soft = e / e.sum()", "    e = fw.w\n    soft = e / e.sum()",
     check_library_and_ranges),
]


@pytest.mark.parametrize("desc,old,new,check", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_geometry_mistake_is_caught(desc, old, new, check):
    check(O)
    with pytest.raises(AssertionError):
        check(_mutated(old, new))

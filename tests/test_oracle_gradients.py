"""Derivative pins of the oracle: finite differences, autograd re-expression,
and mutation tests showing the pins catch planted mistakes in the oracle."""
import importlib.util
import os
import sys

import numpy as np
import pytest

import oracle as O
from oracle import Params
from tests.oracle_checks import (check_autograd, check_qkv_fd, check_score_fd,
                                 check_zero_sum)

RULES = [O.FULL, O.DETACH, O.MAX_ONLY, O.MIN_ONLY]
SURR = [(O.LERP, O.WEIGHT_STE), (O.NEAREST, O.WEIGHT_STE), (O.NEAREST, O.PROB_STE)]
EXPS = [(O.EXACT, O.WEIGHT_STE), (O.EXP_BF16, O.WEIGHT_STE), (O.EXP_FP8, O.WEIGHT_STE)]


@pytest.mark.parametrize("cal", [O.MINMAX, O.FWM, O.FWM_UNTRUNC])
@pytest.mark.parametrize("rec,ste", SURR + EXPS)
@pytest.mark.parametrize("rule", RULES)
@pytest.mark.parametrize("K", [1, 4, 16])
def test_score_level_finite_differences(cal, rec, ste, rule, K):
    rng = np.random.default_rng(100 + K)
    s = rng.standard_normal(14) * 2.5
    dP = rng.standard_normal(14)
    check_score_fd(O, Params(K=K, tau=6.0 if K > 1 else 3.0, calibration=cal, reconstruction=rec,
                             surrogate=ste, grad_rule=rule), s, dP)


@pytest.mark.parametrize("cal", [O.MINMAX, O.FWM, O.FWM_UNTRUNC])
def test_qkv_finite_differences_lerp_full(cal):
    rng = np.random.default_rng(21)
    T, d = 6, 4
    Q, Kt, V, dO = (rng.standard_normal((T, d)) * sc for sc in (2.0, 1.0, 1.0, 1.0))
    check_qkv_fd(O, Params(K=4, tau=3.0, calibration=cal), Q, Kt, V, dO)


@pytest.mark.parametrize("cal", [O.MINMAX, O.FWM, O.FWM_UNTRUNC])
@pytest.mark.parametrize("rec,ste", SURR + EXPS)
@pytest.mark.parametrize("rule", RULES + [O.P1])
def test_autograd_reexpression(cal, rec, ste, rule):
    rng = np.random.default_rng(31)
    T, d = 20, 8
    Q, Kt, V, dO = (rng.standard_normal((T, d)) * sc for sc in (2.5, 1.0, 1.0, 1.0))
    p = Params(K=4, tau=6.0, calibration=cal, reconstruction=rec, surrogate=ste, grad_rule=rule)
    if rule == O.P1:
        # P1 is not a stop-gradient placement; check it as detach minus the row mean
        pd = Params(K=4, tau=6.0, calibration=cal, reconstruction=rec, surrogate=ste, grad_rule=O.DETACH)
        r1 = O.head_backward(Q, Kt, V, dO, p, keep_rows=True)["rows"]
        rd = O.head_backward(Q, Kt, V, dO, pd, keep_rows=True)["rows"]
        for t in range(T):
            ds1, dsd = r1[t][1].dS, rd[t][1].dS
            np.testing.assert_allclose(ds1, dsd - dsd.mean(), atol=1e-14)
        return
    check_autograd(O, p, Q, Kt, V, dO)


# --------------------------------------------------------------------------
# mutation tests: a planted mistake in a copy of the oracle must trip a pin
# --------------------------------------------------------------------------

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "kia_oracle.py")


def mutated_oracle(old, new):
    src = open(ORACLE_SRC).read()
    assert src.count(old) == 1, old
    name = f"kia_oracle_mutant_{abs(hash(old)) % 10**8}"
    spec = importlib.util.spec_from_loader(name, loader=None)
    mod = importlib.util.module_from_spec(spec)
    sys.modules[name] = mod          # dataclasses look the module up by name
    exec(compile(src.replace(old, new), ORACLE_SRC + " (mutant)", "exec"), mod.__dict__)
    return mod


def _row_inputs(seed=7, n=14):
    rng = np.random.default_rng(seed)
    return rng.standard_normal(n) * 2.5, rng.standard_normal(n)


def _head_inputs(seed=8, T=6, d=4):
    rng = np.random.default_rng(seed)
    return tuple(rng.standard_normal((T, d)) * sc for sc in (2.0, 1.0, 1.0, 1.0))


MUTANTS = [
    # (description, old, new, check)
    ("drop the i+1 grid-value term of dw/dh",
     "f * (-(i + 1) * gi1)", "f * (-i * gi1)",
     lambda m: check_score_fd(m, m.Params(K=4), *_row_inputs())),
    ("route the min term with the max term's dh",
     "Cn = float(np.sum(gt * dw_dh_total * dh_dn))", "Cn = float(np.sum(gt * dw_dh_total * dh_dm))",
     lambda m: check_zero_sum(m, m.Params(K=4), *_row_inputs())),
    ("wrong sign of du/dh",
     "du_dh = -rec.uc / h", "du_dh = rec.uc / h",
     lambda m: check_score_fd(m, m.Params(K=8), *_row_inputs())),
    ("Prob-STE evaluated at the hard point",
     "Pe, We = rec.wL / fw.WL, fw.WL", "Pe, We = fw.P, fw.W",
     lambda m: check_score_fd(m, m.Params(K=4, reconstruction=m.NEAREST, surrogate=m.PROB_STE),
                              *_row_inputs())),
    ("detach that keeps the max term",
     "        if p.carries_max():\n            dS[cal.a] += Cm\n        if p.carries_min():",
     "        if True:\n            dS[cal.a] += Cm\n        if p.carries_min():",
     lambda m: check_score_fd(m, m.Params(K=4, grad_rule=m.DETACH), *_row_inputs())),
    ("dK built from dO instead of Q (transposed operand)",
     "dK[: t + 1] += np.outer(bw.dS, Q64[t]) * scale", "dK[: t + 1] += np.outer(bw.dS, dO64[t]) * scale",
     lambda m: check_qkv_fd(m, m.Params(K=4), *_head_inputs())),
    ("dV from the LERP probabilities under a hard forward",
     "dV[: t + 1] += np.outer(fw.P, dO64[t])", "dV[: t + 1] += np.outer(fw.wL / fw.WL, dO64[t])",
     lambda m: check_autograd(m, m.Params(K=4, reconstruction=m.NEAREST), *_head_inputs(T=12, d=6))),
    ("score scale dropped",
     "return (keys.astype(np.float64) * q_t.astype(np.float64)).sum(axis=1) / np.sqrt(d)",
     "return (keys.astype(np.float64) * q_t.astype(np.float64)).sum(axis=1)",
     lambda m: check_autograd(m, m.Params(K=4), *_head_inputs(T=12, d=6))),
    ("untruncated step keeps FWM's zero tail",
     "        mask = np.ones_like(u)\n    g = grid(h, K)", "        mask = (u <= K).astype(np.float64)\n    g = grid(h, K)",
     lambda m: check_autograd(m, m.Params(K=2, tau=1.0, calibration=m.FWM_UNTRUNC), *_head_inputs(T=12, d=6))),
    ("untruncated step clamps its segment at K - 1",
     "i = np.maximum(np.floor(uc), 0).astype(np.int64)", "i = np.clip(np.floor(uc), 0, K - 1).astype(np.int64)",
     lambda m: check_autograd(m, m.Params(K=2, tau=1.0, calibration=m.FWM_UNTRUNC), *_head_inputs(T=12, d=6))),
    ("exact softmax gradient taken at the unnormalised weights",
     "gt = (dP - delta) / fw.W\n        e = np.exp", "gt = (dP - delta)\n        e = np.exp",
     lambda m: check_autograd(m, m.Params(K=4, reconstruction=m.EXACT), *_head_inputs(T=12, d=6))),
    ("straight-through derivative taken at the rounded exponentials",
     "dS_direct = gt * e ", "dS_direct = gt * fw.w ",
     lambda m: check_score_fd(m, m.Params(K=4, reconstruction=m.EXP_BF16), *_row_inputs())),
    ("rounded exponential truncated instead of rounded to nearest",
     "return np.rint(x / quantum) * quantum", "return np.floor(x / quantum) * quantum",
     lambda m: check_autograd(m, m.Params(K=4, reconstruction=m.EXP_FP8), *_head_inputs(T=12, d=6))),
    ("FP8 exponential without gradual underflow",
     "FORMATS = {EXP_BF16: (7, -126), EXP_FP8: (3, -6)}", "FORMATS = {EXP_BF16: (7, -126), EXP_FP8: (3, -60)}",
     lambda m: check_autograd(m, m.Params(K=4, reconstruction=m.EXP_FP8), *_head_inputs(T=12, d=6))),
    ("Nearest truncates instead of rounding (forward checked by autograd forward value)",
     "r = np.clip(np.floor(uc + 0.5), 0, K)", "r = np.clip(np.floor(uc), 0, K)",
     lambda m: check_autograd(m, m.Params(K=4, reconstruction=m.NEAREST), *_head_inputs(T=12, d=6))),
]


@pytest.mark.parametrize("desc,old,new,check", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(desc, old, new, check):
    check(O)                                   # the real oracle passes the check
    mod = mutated_oracle(old, new)
    with pytest.raises(AssertionError):
        check(mod)

"""Reusable checks of the oracle's backward, parameterised by the oracle module
so the mutation tests can run them against a deliberately broken copy.

Each check raises AssertionError when the backward disagrees with what it is
checked against.  Source of the rules checked: "Pretraining Transformers with
Quantized Softmax in Attention" (paperlayer digest), section 3 ("Calibration
gradients", "Surrogate placement") and App. B ("Gradient derivations").
"""
import numpy as np


def surrogate_objective(mod, s, s0, dP, p):
    """L(s) = sum_j P_j(s) dP_j for the differentiable surrogate whose exact
    derivative at s0 the rule's backward must be.

    * extrema: live (max(s), min(s)) or held at their value at s0 per rule;
    * LERP: P = wL / sum(wL);
    * Weight-STE: w = wL(s) + [wN - wL](s0), P = w / sum(w)  (replacement before
      normalisation, so the Jacobian sees the hard weights);
    * Prob-STE: P = PL(s) + [PN - PL](s0)  (replacement after normalisation).
    """
    cal0 = mod.calibrate(s0, p)
    live_max = p.grad_rule in (mod.FULL, mod.MAX_ONLY)
    live_min = p.grad_rule in (mod.FULL, mod.MIN_ONLY)
    m = s.max() if live_max else cal0.m
    n = s.min() if live_min else cal0.n
    if p.reconstruction in (mod.EXACT, mod.EXP_BF16, mod.EXP_FP8):
        w = np.exp(s - m)
        if p.reconstruction != mod.EXACT:
            # straight-through rounding: the offset of the rounded exponential,
            # frozen at s0, added before normalisation
            e0 = np.exp(s0 - cal0.m)
            w = w + (mod.round_to_format(e0, *mod.FORMATS[p.reconstruction]) - e0)
        rec = mod.reconstruct(s, m, 1.0, mod.Params(K=1))       # placeholder decisions (none)
        return float((w / w.sum()) @ dP), rec
    h = (m - n) / p.K if p.calibration == mod.MINMAX else p.tau / p.K
    rec = mod.reconstruct(s, m, h, p, clamp=False)
    rec0 = mod.reconstruct(s0, cal0.m, cal0.h, p, clamp=False)
    wL = rec.wL
    if p.reconstruction == mod.LERP:
        P = wL / wL.sum()
    elif p.surrogate == mod.WEIGHT_STE:
        w = wL + (rec0.wN - rec0.wL)
        P = w / w.sum()
    else:
        P = wL / wL.sum() + (rec0.wN / rec0.wN.sum() - rec0.wL / rec0.wL.sum())
    return float(P @ dP), rec


def check_score_fd(mod, p, s, dP, eps=1e-6, rtol=2e-7):
    """Central differences of the surrogate objective against row_backward.dS."""
    fw = mod.row_forward(s, p)
    bw = mod.row_backward(fw, dP, p)
    _, rec0 = surrogate_objective(mod, s, s, dP, p)
    scale = np.abs(bw.dS).max() + 1e-300
    checked = 0
    for j in range(len(s)):
        e = np.zeros_like(s)
        e[j] = eps
        lp, rp = surrogate_objective(mod, s + e, s, dP, p)
        lm, rm = surrogate_objective(mod, s - e, s, dP, p)
        # skip coordinates whose perturbation crosses a decision
        same = all(np.array_equal(r.i, rec0.i) and np.array_equal(r.mask, rec0.mask) for r in (rp, rm))
        same = same and np.argmax(s + e) == np.argmax(s - e) == fw.cal.a
        same = same and np.argmin(s + e) == np.argmin(s - e) == fw.cal.b
        if not same:
            continue
        num = (lp - lm) / (2 * eps)
        assert abs(num - bw.dS[j]) <= rtol * scale + 1e-10, (j, num, bw.dS[j])
        checked += 1
    assert checked >= len(s) - 2
    return bw


def check_zero_sum(mod, p, s, dP):
    bw = mod.row_backward(mod.row_forward(s, p), dP, p)
    assert abs(bw.dS.sum()) <= 1e-12 * np.abs(bw.dS).sum()


def check_qkv_fd(mod, p, Q, Kt, V, dO, eps=1e-6, rtol=1e-6):
    """Central differences of sum(dO * O) w.r.t. every entry of Q, K, V."""
    ref = mod.head_backward(Q, Kt, V, dO, p)

    def loss(Q_, K_, V_):
        return float(np.sum(mod.head_forward(Q_, K_, V_, p)["O"] * dO))

    for name, X, G in (("Q", Q, ref["dQ"]), ("K", Kt, ref["dK"]), ("V", V, ref["dV"])):
        scale = np.abs(G).max() + 1e-300
        for idx in np.ndindex(X.shape):
            Xp, Xm = X.copy(), X.copy()
            Xp[idx] += eps
            Xm[idx] -= eps
            args_p = [Q, Kt, V]
            args_m = [Q, Kt, V]
            k = "QKV".index(name)
            args_p[k], args_m[k] = Xp, Xm
            num = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert abs(num - G[idx]) <= rtol * scale + 1e-9, (name, idx, num, G[idx])


def torch_reexpression(mod, p, Q, Kt, V, dO):
    """The operator written again in torch fp64 with stop-gradients placed per
    rule and surrogate; autograd supplies dQ, dK, dV (App. B reports closed
    form vs autograd agreement below 1e-9)."""
    import torch
    q, k, v = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (Q, Kt, V))
    T, d = Q.shape
    S = (q @ k.T) / np.sqrt(d)
    outs = []
    for t in range(T):
        s = S[t, : t + 1]
        m, n = s.max(), s.min()
        if p.grad_rule in (mod.DETACH, mod.MIN_ONLY, mod.P1):
            m = m.detach()
        if p.grad_rule in (mod.DETACH, mod.MAX_ONLY, mod.P1):
            n = n.detach()
        if p.reconstruction in (mod.EXACT, mod.EXP_BF16, mod.EXP_FP8):
            w = torch.exp(s - m)
            if p.reconstruction != mod.EXACT:
                # torch's own casts round to nearest even (via fp32, whose extra
                # rounding can matter only at an exact fp32 tie)
                fmt = torch.bfloat16 if p.reconstruction == mod.EXP_BF16 else torch.float8_e4m3fn
                wd = w.detach()
                w = w + (wd.float().to(fmt).to(torch.float64) - wd)
            outs.append((w / w.sum()) @ v[: t + 1])
            continue
        if p.calibration == mod.MINMAX:
            if float((m - n).detach()) < mod.EPS_SPAN:
                w = torch.ones_like(s)
                outs.append((w / w.sum()) @ v[: t + 1])
                continue
            h = (m - n) / p.K
        else:
            h = torch.tensor(p.tau / p.K, dtype=torch.float64)
        u = (m - s) / h
        mask = (u <= p.K).double().detach() if p.calibration == mod.FWM else torch.ones_like(u)
        if p.calibration == mod.FWM_UNTRUNC:             # the grid continues below max - tau
            uc = u
            i = torch.floor(uc).clamp(min=0).detach()
            r = torch.floor(uc + 0.5).clamp(min=0).detach()
        else:
            uc = u - (u - p.K).clamp(min=0).detach()    # value min(u, K), derivative 1
            i = torch.floor(uc).clamp(0, p.K - 1).detach()
            r = torch.floor(uc + 0.5).clamp(0, p.K).detach()
        f = uc - i
        wL = mask * ((1 - f) * torch.exp(-i * h) + f * torch.exp(-(i + 1) * h))
        wN = mask * torch.exp(-r * h)
        if p.reconstruction == mod.LERP:
            P = wL / wL.sum()
        elif p.surrogate == mod.WEIGHT_STE:
            w = wL + (wN - wL).detach()
            P = w / w.sum()
        else:
            P = wL / wL.sum() + (wN / wN.sum() - wL / wL.sum()).detach()
        outs.append(P @ v[: t + 1])
    o = torch.stack(outs)
    (o * torch.tensor(dO, dtype=torch.float64)).sum().backward()
    return o.detach().numpy(), q.grad.numpy(), k.grad.numpy(), v.grad.numpy()


def check_autograd(mod, p, Q, Kt, V, dO, rtol=1e-9):
    o, gq, gk, gv = torch_reexpression(mod, p, Q, Kt, V, dO)
    ref = mod.head_backward(Q, Kt, V, dO, p)
    np.testing.assert_allclose(mod.head_forward(Q, Kt, V, p)["O"], o, rtol=0, atol=rtol * np.abs(o).max())
    for g, r in ((gq, ref["dQ"]), (gk, ref["dK"]), (gv, ref["dV"])):
        np.testing.assert_allclose(r, g, rtol=0, atol=rtol * max(np.abs(g).max(), 1e-300))

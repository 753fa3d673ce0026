"""GPU parity of the score-geometry probe (kia_geometry through the C ABI)
against the fp64 oracle's probe (section 4 "Geometry probe"; section 5.4;
App. D.6 of "Pretraining Transformers with Quantized Softmax in Attention").

Bars: span and width within 1e-5 of the slice's max span; norms within 1e-6
relative; entropies within 1e-5 * max(1, log(t + 1)) nats; total variation and
top-bucket mass (both in [0, 1]) within 1e-5 absolute.  The probe reduces the
forward's fp32 scores, whose error against the exact scores is at most a few
1e-6 of the row's |Q||K| scale; fp32 sums within a tile and fp64 across tiles
add a few 1e-7.

Decisions (Nearest point, FWM window edge, the top bucket's u < 1/2) are
taken in fp32 on the GPU and in fp64 by the oracle; a row whose oracle u sits
closer to such a boundary than the two sides' u can differ is excluded from
the fields that decision moves (top mass, or the entropy of P and the total
variation), with the same band as the operator's parity tests.
"""
import numpy as np
import pytest

import oracle as O
from tests.gpu_harness import score_bound, to_oracle_params
from workloads import WORKLOADS, Workload, make_inputs

pytestmark = pytest.mark.gpu

FIELDS = O.GEOMETRY_FIELDS


def P(**kw):
    from quantized_softmax_attention_amd import Params
    return Params(**kw)


def run_probe(q, k, v, params):
    import torch
    import quantized_softmax_attention_amd as kia
    dev = torch.device("cuda:0")
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in (q, k, v))
    B, H, T, d = q.shape
    o, stats = kia.kia_forward(tq, tk, tv, params)
    geo = kia.kia_geometry(tq, tk, stats, params)
    L = kia.kia_stats_layout_query(params, B, H, T, d)
    n = B * H * T
    m = stats[L.row_m: L.row_m + 4 * n].view(torch.float32).reshape(B, H, T)
    torch.cuda.synchronize()
    return {"geo": geo.cpu().numpy(), "m": m.cpu().numpy(), "stats": stats, "L": L,
            "_tensors": (tq, tk, tv)}


def gpu_scores_rows(run, b, h, rows):
    """The forward's fp32 scores of the rows asked for (dense [len(rows), T])."""
    import torch
    import quantized_softmax_attention_amd as kia
    tq = run["_tensors"][0]
    B, H, T, d = tq.shape
    dense = kia.kia_tiles_to_dense(B, H, T, run["stats"][run["L"].scores:], False)
    out = dense[b, h].index_select(0, torch.as_tensor(list(rows), device=dense.device)).cpu().numpy()
    del dense
    return out


def ambiguous(p_or, s_ref, sg, m_gpu, K):
    """(top_amb, p_amb, n_keys): whether the top-bucket decision, or a
    decision that moves the operator's weights, can differ between the fp32
    and fp64 sides, and how many keys of the row carry such a decision."""
    m_ref, n_ref = s_ref.max(), s_ref.min()
    n_gpu = float(sg.min())
    span_ref = m_ref - n_ref
    p_keys = np.zeros(s_ref.shape, dtype=bool)
    if p_or.reconstruction in O.FORMATS:
        # rounded exponentials: a key near a rounding midpoint of the format
        frac_bits, emin = O.FORMATS[p_or.reconstruction]
        x_ref = s_ref - m_ref
        e_ref = np.exp(x_ref)
        d_obs = np.abs((sg.astype(np.float64) - m_gpu) - x_ref)
        band_e = 2 * e_ref * (d_obs + 8 * 2.0 ** -24 * (np.abs(x_ref) + 1))
        _, ex = np.frexp(e_ref)
        q = np.ldexp(1.0, np.maximum(ex - 1, emin) - frac_bits)
        p_keys |= np.abs(e_ref / q - np.floor(e_ref / q) - 0.5) * q <= band_e
    if p_or.calibration == O.MINMAX or p_or.reconstruction in O.EXP_FAMILY:
        if span_ref < 1e-6:
            return False, bool(p_keys.any()), int(p_keys.sum())
        h_ref, h_gpu = span_ref / K, (m_gpu - n_gpu) / K
    else:
        h_ref = h_gpu = p_or.tau / K
    u_ref = (m_ref - s_ref) / h_ref
    u_gpu = (m_gpu - sg.astype(np.float64)) / h_gpu
    band = 2 * (np.abs(u_gpu - u_ref) + 4 * 2.0 ** -24 * (np.abs(u_ref) + 1))
    top_keys = np.abs(u_ref - 0.5) < band
    if p_or.reconstruction == O.NEAREST:
        p_keys |= np.abs(u_ref - 0.5 - np.round(u_ref - 0.5)) < band
    if p_or.calibration == O.FWM and p_or.reconstruction not in O.EXP_FAMILY:
        p_keys |= np.abs(u_ref - K) < band
    return bool(top_keys.any()), bool(p_keys.any()), int((top_keys | p_keys).sum())


def compare_rows(q, k, params, run, b, h, rows):
    """Compare the probe's fields on the rows asked for; returns (worst error
    per field, [rows excluded from top mass, rows excluded from the entropy
    of P and the total variation, ambiguous keys, keys checked])."""
    p_or = to_oracle_params(params)
    Qh, Kh = q[b, h], k[b, h]
    geo = run["geo"][:, b, h]
    sg_rows = gpu_scores_rows(run, b, h, rows)
    ref = O.head_geometry(Qh, Kh, p_or, rows=rows)
    span_scale = max(np.nanmax(ref["span"][rows]), 1e-30)
    worst = {f: 0.0 for f in FIELDS}
    excl = [0, 0, 0, 0]
    for i, t in enumerate(rows):
        s_ref = O.row_scores(Qh[t].astype(np.float64), Kh[: t + 1].astype(np.float64))
        sg = sg_rows[i, : t + 1]
        sb = score_bound(Qh[t: t + 1], Kh[: t + 1])[0]
        assert (np.abs(sg - s_ref) <= sb + 1e-30).all(), ("scores outside the fp32 bound", b, h, t)
        top_amb, p_amb, n_keys = ambiguous(p_or, s_ref, sg, float(run["m"][b, h, t]), params.K)
        excl[0] += top_amb
        excl[1] += p_amb
        excl[2] += n_keys
        excl[3] += t + 1
        for fi, f in enumerate(FIELDS):
            if f == "top_mass" and top_amb:
                continue
            if f in ("entropy_p", "tv") and p_amb:
                continue
            gv, rv = float(geo[fi, t]), float(ref[f][t])
            if f in ("span", "h"):
                err = abs(gv - rv) / span_scale
                tol = 1e-5
            elif f in ("q_norm", "k_norm"):
                err = abs(gv - rv) / max(rv, 1e-30)
                tol = 1e-6
            elif f in ("entropy_p", "entropy_soft"):
                err = abs(gv - rv) / max(1.0, np.log(t + 1))
                tol = 1e-5
            else:
                err = abs(gv - rv)
                tol = 1e-5
            worst[f] = max(worst[f], err)
            assert err <= tol, (f, (b, h, t), gv, rv, err)
    return worst, excl


SMALL = Workload("small_ragged", 2, 2, 80, 64, "scaled", q_scale=2.0)
SMALL128 = Workload("small_ragged_d128", 1, 2, 75, 128, "head_temp", lo=0.5, hi=3.0)
OPERATORS = [("minmax", "lerp"), ("minmax", "nearest"), ("fwm", "lerp"), ("fwm", "nearest"),
             ("fwm_untrunc", "lerp"), ("fwm_untrunc", "nearest"), ("minmax", "exact"),
             ("minmax", "exp_bf16"), ("minmax", "exp_fp8")]


@pytest.mark.parametrize("w", [SMALL, SMALL128], ids=lambda w: w.name)
@pytest.mark.parametrize("cal,rec", OPERATORS)
@pytest.mark.parametrize("K", [1, 4, 32])
def test_geometry_small(w, cal, rec, K):
    params = P(K=K, tau=6.0, calibration=cal, reconstruction=rec)
    q, k, v, _ = make_inputs(w)
    print(f"[case] geometry {w.name} {params}", flush=True)
    run = run_probe(q, k, v, params)
    rows = list(range(w.T))
    for b in range(w.B):
        for h in range(w.H):
            worst, excl = compare_rows(q, k, params, run, b, h, rows)
            # decisions near a boundary stay a small share of the keys
            assert excl[2] <= 0.02 * excl[3], excl
    print(f"  worst {worst}  excluded rows (top, P) and keys {excl}", flush=True)


def test_geometry_edge_cases():
    """T = 1 (one key: zero span, zero entropies, all mass on top); zero
    queries (constant rows: MinMax degenerate, uniform P); a ragged T = 33."""
    rng = np.random.default_rng(5)
    for T, zero_q in ((1, False), (33, True), (33, False)):
        q = rng.standard_normal((1, 2, T, 64)).astype(np.float32)
        if zero_q:
            q[:] = 0
        k = rng.standard_normal((1, 2, T, 64)).astype(np.float32)
        v = rng.standard_normal((1, 2, T, 64)).astype(np.float32)
        for cal, rec in OPERATORS:
            params = P(K=4, tau=6.0, calibration=cal, reconstruction=rec)
            print(f"[case] geometry edge T{T} zero_q={zero_q} {params}", flush=True)
            run = run_probe(q, k, v, params)
            for h in range(2):
                compare_rows(q, k, params, run, 0, h, list(range(T)))
            geo = run["geo"]
            if T == 1 or zero_q:
                assert np.all(geo[0] == 0.0)                          # span
                assert np.all(np.abs(geo[6]) <= 1e-6)                 # tv
                assert np.all(np.abs(geo[7] - 1.0) <= 1e-6)           # top mass


def _sample_rows(T, rng, n=24):
    fixed = [0, 1, 2, 31, 32, 33, 63, 64, T // 2, T - 33, T - 32, T - 2, T - 1]
    extra = rng.choice(T, size=n, replace=False).tolist()
    return sorted({t for t in fixed + extra if 0 <= t < T})


@pytest.mark.parametrize("cal,rec", [("minmax", "lerp"), ("minmax", "nearest"), ("fwm", "nearest"),
                                     ("minmax", "exact")])
def test_geometry_full_size_c2(cal, rec):
    """GPT-2 124M shape (B 8, H 12, T 1024, d 64) in the launch configuration
    the benchmark times: sampled rows against the oracle, and properties that
    hold at any size on every row."""
    w = WORKLOADS["c2"]
    K = 4
    params = P(K=K, tau=6.0, calibration=cal, reconstruction=rec)
    q, k, v, _ = make_inputs(w)
    print(f"[case] geometry c2 {params}", flush=True)
    run = run_probe(q, k, v, params)
    rng = np.random.default_rng(17)
    for (b, h) in [(0, 0), (3, 7), (7, 11)]:
        worst, excl = compare_rows(q, k, params, run, b, h, _sample_rows(w.T, rng))
        print(f"  slice {(b, h)} worst {worst} excluded {excl}", flush=True)
    geo = run["geo"]
    t = np.arange(w.T)
    logn = np.log(t + 1.0)
    assert np.all(geo[0] >= 0) and np.all(np.isfinite(geo))
    assert np.all((geo[6] >= -1e-6) & (geo[6] <= 1 + 1e-6))
    assert np.all((geo[7] > 0) & (geo[7] <= 1 + 1e-6))
    for f in (4, 5):
        assert np.all((geo[f] >= -1e-5) & (geo[f] <= logn + 1e-5))
    if cal == "minmax":
        assert np.allclose(geo[1], geo[0] / K, rtol=1e-6, atol=0)
    if rec == "exact":
        assert np.all(geo[6] <= 1e-5)
        assert np.all(np.abs(geo[4] - geo[5]) <= 1e-5 * np.maximum(1, logn))
    # position t's norms are the inputs' own
    assert np.allclose(geo[2], np.linalg.norm(q.astype(np.float64), axis=-1), rtol=1e-6)
    assert np.allclose(geo[3], np.linalg.norm(k.astype(np.float64), axis=-1), rtol=1e-6)

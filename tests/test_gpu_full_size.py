"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times: sampled (b, h) slices against the fp64 oracle, properties
checked over every row, and bitwise identities.  A second run with the index
dump (asserted bitwise equal to the first) supplies the kernel's decisions:
every decision must match the oracle's exactly, except at keys inside the two
sides' rounding band, where either admissible decision is accepted and the
oracle row is evaluated with the one taken.  Each slice check must compare at
least 95% of its rows (O, dQ) and keys (dK, dV).

Per workload, the runs follow the variants each configuration is quoted on:
  c2  MinMax LERP, K in {4, 16, 32} x {full, detach, max-only, min-only}
  c3  Nearest K=4 x {MinMax, FWM} x {Weight-STE, Prob-STE}, full
  c4  FWM tau=6 K=16 Nearest Prob-STE full, and MinMax LERP K=64 full
  c5  MinMax LERP K in {4, 64} x {full, detach}; zero row sums over all rows
The long-sequence workload (T=8192) is compared on sampled rows (including
rows with a constructed dominant key) and on its last keys, whose dK / dV
only the last rows reach.
"""
import numpy as np
import pytest

from tests.gpu_harness import TOL, SliceCheck, run_gpu, to_oracle_params
from workloads import WORKLOADS, Workload, make_inputs, spike_rows

pytestmark = pytest.mark.gpu

_INPUTS = {}


def inputs(name):
    if name not in _INPUTS:
        _INPUTS[name] = make_inputs(_workload(name))
    return _INPUTS[name]


def _workload(name):
    """A named workload, or one defined in place (a Workload)."""
    return name if isinstance(name, Workload) else WORKLOADS[name]


def P(**kw):
    from quantized_softmax_attention_amd import Params
    return Params(**kw)


def zero_sum_all_rows(g, params, tol=1e-5):
    """Rows of the GPU's dS (calibration terms folded in) whose |sum| exceeds
    tol * L1, over every row of every slice.  Under MinMax, rows whose stored
    span is below the degenerate threshold are skipped (their softmax-limit
    gradient cancels only to the rounding of two dot products; single-key rows
    have dS = 0 and pass anyway)."""
    import torch
    dS = g["dS"].double()
    if params.grad_rule == "p1":
        # the stored detached gradient minus the row mean on the causal keys
        T = dS.shape[-1]
        causal = torch.ones(T, T, dtype=torch.bool, device=dS.device).tril()
        dS = dS - g["cm"].double()[..., None] * causal
    sums = dS.sum(-1)
    l1 = dS.abs().sum(-1)
    bad = sums.abs() > tol * l1
    if params.calibration == "minmax" and params.reconstruction not in ("exact", "exp_bf16", "exp_fp8"):
        bad &= (g["m"] - g["n"]).double() >= 1e-12
    idx = torch.nonzero(bad)[:5].tolist()
    detail = [(tuple(i), float(sums[tuple(i)]), float(l1[tuple(i)]), int(g["a"][tuple(i)]), int(g["b"][tuple(i)]),
               float(g["cm"][tuple(i)]), float(g["cn"][tuple(i)])) for i in idx]
    return int(bad.sum().item()), int(bad.numel()), detail


MIN_COVERAGE = 0.95    # share of the rows (O, dQ) and keys (dK, dV) each slice check must compare


def full_check(name, params, heads, rows=None, tail=None, zero_sum=None, want_idx=True):
    """Run the workload in the launch configuration the benchmark times, then
    again with the index dump (the decisions the harness replays at
    boundary-near keys), assert the two runs bitwise equal, and compare the
    sampled slices with the oracle."""
    import torch
    q, k, v, do = inputs(name)
    w = _workload(name)
    print(f"[case] full-size {w.name} B{w.B} H{w.H} T{w.T} d{w.d} {params} slices {heads}", flush=True)
    g = run_gpu(q, k, v, do, params, want_dense=True, want_idx=False)
    if want_idx:
        gi = run_gpu(q, k, v, do, params, want_dense=False, want_idx=True)
        for key in ("O", "dQ", "dK", "dV", "m", "n", "a", "b", "W", "WL"):
            assert torch.equal(g[key].view(torch.int32), gi[key].view(torch.int32)), \
                f"{key} differs between the runs with and without the index dump"
        g["idx"] = gi["idx"]
        del gi
    p_or = to_oracle_params(params)
    worst = {}
    ties = excluded = replayed = idx_checked = 0
    for (b, h) in heads:
        r = rows(b, h) if callable(rows) else rows
        sc = SliceCheck(q, k, v, do, p_or, g, b, h, rows=r, tail=tail)
        assert sc.score_viol == 0, f"scores outside the fp32 bound in slice {(b, h)}"
        assert sc.idx_mismatch == 0, f"{sc.idx_mismatch} decisions differ from the oracle's in slice {(b, h)}"
        cover = []
        for nm in ("O", "dQ", "dK", "dV"):
            err, kept, region = sc.compare(nm)
            worst[nm] = max(worst.get(nm, 0.0), err)
            assert err <= TOL, f"{nm} rel err {err:.3e} in slice {(b, h)} ({kept} of {region} compared)"
            assert kept >= MIN_COVERAGE * region, f"{nm} compared on only {kept} of {region} in slice {(b, h)}"
            cover.append(f"{nm} {kept}/{region}")
        print(f"  slice {(b, h)}: compared " + ", ".join(cover) +
              f"; replayed decisions {sc.n_replayed} in {sc.rows_replayed} rows", flush=True)
        if params.grad_rule in ("full", "p1"):
            bad = sc.zero_sum_violations(q, k, v, do, b, h)
            assert not bad, f"zero-sum violated in slice {(b, h)}: {bad[:3]}"
        ties += int(sc.amb_bwd.sum())
        excluded += sc.n_amb_pairs
        replayed += sc.n_replayed
        idx_checked += sc.idx_checked
    if zero_sum if zero_sum is not None else params.grad_rule in ("full", "p1"):
        nbad, nrows, detail = zero_sum_all_rows(g, params)
        assert nbad == 0, f"{nbad} of {nrows} rows violate the zero row sum: (b,h,t), sum, L1, a, b, cm, cn = {detail}"
        print(f"  zero row sum holds on all {nrows} rows", flush=True)
    print(f"  worst rel err {worst}; rows with a boundary-near decision {ties}; "
          f"boundary-near pairs {excluded} (replayed {replayed}); decisions checked bit-exact {idx_checked}",
          flush=True)
    return g


def _heads(i, w, n=1):
    return [((i + 3 * j) % w.B, (5 * i + 7 * j) % w.H) for j in range(n)]


@pytest.mark.parametrize("K", [4, 16, 32])
@pytest.mark.parametrize("rule", ["full", "detach", "max_only", "min_only"])
def test_c2_full_size(K, rule):
    i = [4, 16, 32].index(K) * 4 + ["full", "detach", "max_only", "min_only"].index(rule)
    full_check("c2", P(K=K, calibration="minmax", reconstruction="lerp", grad_rule=rule),
               _heads(i, WORKLOADS["c2"]))


@pytest.mark.parametrize("K", [4, 32])
def test_c2_full_size_p1(K):
    """P1 (zero-sum projection of the detached gradient) at full size."""
    full_check("c2", P(K=K, calibration="minmax", reconstruction="lerp", grad_rule="p1"),
               _heads(13 + K, WORKLOADS["c2"]))


@pytest.mark.parametrize("rec,ste", [("lerp", "weight"), ("nearest", "prob")])
def test_c2_full_size_untruncated_step(rec, ste):
    """The untruncated fixed step (FWM's step without the zero tail) at full size."""
    full_check("c2", P(K=4, tau=6.0, calibration="fwm_untrunc", reconstruction=rec, surrogate=ste),
               _heads(21 if rec == "lerp" else 22, WORKLOADS["c2"]))


@pytest.mark.parametrize("rule", ["full", "detach"])
def test_c2_full_size_exact_softmax(rule):
    """The exact-softmax reference on the same kernels at full size.  Only the
    full rule folds the calibration term into the argmax entry, which is what
    makes each row sum exact; under detach the direct terms cancel only to the
    rounding of delta = dO.O, so the row-sum bar applies to the full rule."""
    full_check("c2", P(K=1, reconstruction="exact", grad_rule=rule), _heads(30, WORKLOADS["c2"]),
               zero_sum=(rule == "full"))


@pytest.mark.parametrize("rec", ["exp_bf16", "exp_fp8"])
@pytest.mark.parametrize("rule", ["full", "detach"])
def test_c2_full_size_rounded_exponential(rec, rule):
    """The BF16- and FP8-rounded exponential baselines at full size; the row
    sum vanishes under the full rule only."""
    full_check("c2", P(K=1, reconstruction=rec, grad_rule=rule), _heads(31 if rec == "exp_bf16" else 32,
                                                                       WORKLOADS["c2"]),
               zero_sum=(rule == "full"))


@pytest.mark.parametrize("cal", ["minmax", "fwm"])
@pytest.mark.parametrize("ste", ["weight", "prob"])
def test_c3_full_size(cal, ste):
    i = ["minmax", "fwm"].index(cal) * 2 + ["weight", "prob"].index(ste)
    full_check("c3", P(K=4, tau=6.0, calibration=cal, reconstruction="nearest", surrogate=ste),
               _heads(i, WORKLOADS["c3"], 2))


def test_c4_full_size_fwm_nearest_prob():
    full_check("c4", P(K=16, tau=6.0, calibration="fwm", reconstruction="nearest", surrogate="prob"),
               [(1, 5)])


def test_c4_full_size_minmax_lerp():
    full_check("c4", P(K=64, calibration="minmax", reconstruction="lerp"), [(3, 12)])


def _c5_rows(b, h):
    w = WORKLOADS["c5"]
    sp = sorted(t for (bb, hh, t, _) in spike_rows(w) if (bb, hh) == (b, h))
    picked = sp[:: max(1, len(sp) // 12)][:12]
    spread = list(np.linspace(1, w.T - 200, 12).astype(int))
    return sorted(set(picked) | set(spread) | {0})


@pytest.mark.parametrize("K", [4, 64])
@pytest.mark.parametrize("rule", ["full", "detach"])
def test_c5_full_size(K, rule):
    w = WORKLOADS["c5"]
    full_check("c5", P(K=K, calibration="minmax", reconstruction="lerp", grad_rule=rule),
               [(0, [4, 64].index(K) * 5 + 2)], rows=_c5_rows, tail=w.T - 96)


LONGEST = Workload("len32768", 1, 3, 32768, 64, "scaled", q_scale=2.0)


def test_longest_rows_past_4gb_buffers():
    """T = 32768 with three heads: 524,800 score tiles per head, so each of the
    score, probability and gradient tile buffers holds 6.4 GB and the third
    head's tiles start past 2^32 bytes (64-bit tile offsets throughout).
    Sampled rows across the sequence (tile and block edges included) and the
    last 96 keys' dK / dV of every head against the oracle; the zero row sum
    over all 98,304 rows."""
    T = LONGEST.T
    rows = [0, 1, 31, 32, 127, 128, 4095, 16383, 16384, 24577, 32000, T - 97]
    full_check(LONGEST, P(K=32, calibration="minmax", reconstruction="lerp"), [(0, 0), (0, 2)],
               rows=rows, tail=T - 96)


# ---------------------------------------------------------------------------
# bitwise identities and determinism at full size
# ---------------------------------------------------------------------------

def _fwd(name, params):
    import torch
    import quantized_softmax_attention_amd as kia
    q, k, v, _ = inputs(name)
    dev = torch.device("cuda:0")
    tq, tk, tv = (torch.from_numpy(x).to(dev) for x in (q, k, v))
    o, st = kia.kia_forward(tq, tk, tv, params)
    L = kia.kia_stats_layout_query(params, *q.shape)
    torch.cuda.synchronize()
    # the score tiles and each row array (m, n, a, b, W, WL), without the
    # alignment padding between sections
    B, H, T, _ = q.shape
    n_tiles = L.tiles_per_head * B * H
    secs = [(L.scores, n_tiles * 4096)] + [(off, B * H * T * 4) for off in
                                          (L.row_m, L.row_n, L.row_a, L.row_b, L.row_w, L.row_wl)]
    return o.cpu().numpy(), np.concatenate([st[a: a + n].cpu().numpy() for a, n in secs])


def test_forward_identical_across_gradient_rules():
    """The forward never reads the gradient rule: O, scores and row statistics
    are bitwise equal under all five rules (P1's forward is detach's)."""
    print("[case] c2 forward identity across rules", flush=True)
    ref_o, ref_st = _fwd("c2", P(K=32, grad_rule="full"))
    for rule in ("detach", "max_only", "min_only", "p1"):
        o, st = _fwd("c2", P(K=32, grad_rule=rule))
        assert np.array_equal(o.view(np.uint32), ref_o.view(np.uint32)), rule
        assert np.array_equal(st, ref_st), rule


@pytest.mark.parametrize("cal", ["minmax", "fwm"])
def test_forward_identical_across_surrogates(cal):
    """Weight-STE and Prob-STE share one hard forward: O and the shared state
    are bitwise equal (Prob-STE only adds its LERP extras)."""
    print(f"[case] c3 forward identity across surrogates ({cal})", flush=True)
    o1, st1 = _fwd("c3", P(K=4, calibration=cal, reconstruction="nearest", surrogate="weight"))
    o2, st2 = _fwd("c3", P(K=4, calibration=cal, reconstruction="nearest", surrogate="prob"))
    assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32))
    assert np.array_equal(st1, st2)


def _fwd_bwd(q, k, v, do, params):
    import torch
    import quantized_softmax_attention_amd as kia
    dev = torch.device("cuda:0")
    tq, tk, tv, tdo = (torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in (q, k, v, do))
    o, st = kia.kia_forward(tq, tk, tv, params)
    dq, dk, dv, _ = kia.kia_backward(tq, tk, tv, o, tdo, st, params)
    torch.cuda.synchronize()
    return [x.cpu().numpy() for x in (o, dq, dk, dv)]


def test_repeatable_and_batch_invariant():
    """Two identical calls give identical bits, and a (b, h) slice gives the
    same bits whether it runs alone or inside the batch."""
    print("[case] c2 determinism and batch invariance", flush=True)
    q, k, v, do = inputs("c2")
    p = P(K=32)
    a = _fwd_bwd(q, k, v, do, p)
    b = _fwd_bwd(q, k, v, do, p)
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))
    bi, hi = 5, 9
    one = _fwd_bwd(*(x[bi: bi + 1, hi: hi + 1] for x in (q, k, v, do)), p)
    for x, y in zip(a, one):
        assert np.array_equal(x[bi, hi].view(np.uint32), y[0, 0].view(np.uint32))


# ---------------------------------------------------------------------------
# constructed edge cases
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("d,rec,ste,T", [
    (64, "lerp", "weight", 70),      # interleaved sweep order: kept copies in registers
    (128, "lerp", "weight", 70),     # serial order (d = 128): kept copies in LDS
    (64, "nearest", "prob", 70),     # serial order (Prob-STE)
    (64, "lerp", "weight", 1100),    # serial order (rows past 32 tiles)
])
def test_exact_ties_pick_lowest_key(d, rec, ste, T):
    """Duplicated keys give bitwise-equal scores; the row max and min are
    attributed to the smallest key index (as in the oracle), in both ways the
    forward keeps the scores of an extreme's tile."""
    import oracle as O
    rng = np.random.default_rng(11)
    q = rng.standard_normal((1, 1, T, d)).astype(np.float32)
    k = rng.standard_normal((1, 1, T, d)).astype(np.float32)
    v = rng.standard_normal((1, 1, T, d)).astype(np.float32)
    do = rng.standard_normal((1, 1, T, d)).astype(np.float32)
    k[0, 0, 45] = k[0, 0, 7]      # keys 7 and 45 identical
    k[0, 0, 60] = k[0, 0, 33]     # keys 33 and 60 identical
    expect_a, expect_b = {}, {}
    for t in range(46, T):        # rows whose max is the 7 / 45 pair
        q[0, 0, t] = 4.0 * k[0, 0, 7] + 0.05 * q[0, 0, t]
        expect_a[t] = 7
    for t in range(61, T):        # and whose min is the 33 / 60 pair
        q[0, 0, t] -= 4.0 * k[0, 0, 33]
        expect_b[t] = 33
    params = P(K=8, reconstruction=rec, surrogate=ste)
    print(f"[case] exact ties d={d} {rec}/{ste} T={T}", flush=True)
    g = run_gpu(q, k, v, do, params, want_dense=True, want_idx=False)
    a = g["a"][0, 0].cpu().numpy()
    b = g["b"][0, 0].cpu().numpy()
    s = g["S"][0, 0].cpu().numpy()
    for t, j in expect_a.items():
        assert s[t, 7] == s[t, 45] and s[t, :t + 1].max() == s[t, 7]
        assert a[t] == j, (t, a[t])
        assert O.calibrate(O.row_scores(q[0, 0, t], k[0, 0, : t + 1]), to_oracle_params(params)).a == j
    for t, j in expect_b.items():
        if s[t, :t + 1].min() == s[t, 33]:
            assert b[t] == j, (t, b[t])


def test_nan_row_stays_contained():
    """A NaN query row makes only its own outputs non-finite (no special
    handling); every other row of O and dQ keeps the bits of the clean run."""
    rng = np.random.default_rng(5)
    T, d = 96, 64
    q, k, v, do = (rng.standard_normal((1, 2, T, d)).astype(np.float32) for _ in range(4))
    p = P(K=16)
    print("[case] NaN query row", flush=True)
    clean = _fwd_bwd(q, k, v, do, p)
    q2 = q.copy()
    q2[0, 1, 40] = np.nan
    dirty = _fwd_bwd(q2, k, v, do, p)
    o_c, dq_c = clean[0], clean[1]
    o_d, dq_d = dirty[0], dirty[1]
    assert not np.isfinite(o_d[0, 1, 40]).any()
    others = np.ones(T, dtype=bool)
    others[40] = False
    assert np.array_equal(o_d[0, 1, others].view(np.uint32), o_c[0, 1, others].view(np.uint32))
    assert np.array_equal(o_d[0, 0].view(np.uint32), o_c[0, 0].view(np.uint32))
    assert np.array_equal(dq_d[0, 1, others].view(np.uint32), dq_c[0, 1, others].view(np.uint32))

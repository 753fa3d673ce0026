"""CPU checks of the seeded input recipes (no GPU, no operator arithmetic).

The generators promise a fixed draw order (Q, K, V, dO from PCG64, then each
workload's structural draws) and a score geometry: a query scale, a per-head
temperature, or one key per chosen row placed a fixed number of nats above
the runner-up.  These tests re-draw the raw stream independently and check
each promise on small copies of the measured workloads, in fp64 on the fp32
tensors the library and the oracle both receive.
"""
import numpy as np
import pytest

from workloads import WORKLOADS, Workload, make_inputs, spike_rows
from workloads.synth import _spike_gamma


def raw_draws(w):
    rng = np.random.default_rng(w.seed)
    draws = [rng.standard_normal(w.shape()) for _ in range(4)]
    return rng, draws


def scores(q, k, b, h, t, d):
    """fp64 scaled dot products of query row t against keys 0..t."""
    return k[b, h, : t + 1].astype(np.float64) @ q[b, h, t].astype(np.float64) / np.sqrt(d)


def margins(q, k, b, h, t, js, d):
    s = scores(q, k, b, h, t, d)
    return s[js] - np.delete(s, js).max(), int(np.argmax(s))


def test_draw_order_plain():
    w = WORKLOADS["c1"].scaled(T=40, d=16)
    _, (rq, rk, rv, rdo) = raw_draws(w)
    q, k, v, do = make_inputs(w)
    for got, want in ((q, rq), (k, rk), (v, rv), (do, rdo)):
        assert got.dtype == np.float32 and got.shape == w.shape()
        assert np.array_equal(got, want.astype(np.float32))


def test_scaled_multiplies_queries_only():
    w = WORKLOADS["c2"].scaled(B=1, H=2, T=33)
    _, (rq, rk, rv, rdo) = raw_draws(w)
    q, k, v, do = make_inputs(w)
    assert w.q_scale == 2.0
    assert np.array_equal(q, (rq * 2.0).astype(np.float32))
    assert np.array_equal(k, rk.astype(np.float32))
    assert np.array_equal(v, rv.astype(np.float32))
    assert np.array_equal(do, rdo.astype(np.float32))


def test_head_temperature_is_one_factor_per_head():
    w = WORKLOADS["c4"].scaled(B=2, H=5, T=24, d=32)
    rng, (rq, rk, _, _) = raw_draws(w)
    c = rng.uniform(w.lo, w.hi, size=w.H)
    q, k, _, _ = make_inputs(w)
    assert np.all((c >= 0.5) & (c <= 3.0))
    assert np.array_equal(q, (rq * c[None, :, None, None]).astype(np.float32))
    assert np.array_equal(k, rk.astype(np.float32))
    # the factor is shared by every row of a head and differs across heads
    ratio = q.astype(np.float64) / rq
    for h in range(w.H):
        np.testing.assert_allclose(ratio[:, h], c[h], rtol=1e-6)
    assert len(set(np.round(c, 6))) == w.H


def test_spike_all_puts_one_key_gap_nats_above_the_rest():
    w = WORKLOADS["c3"].scaled(B=2, H=2, T=80)
    _, (rq, rk, _, _) = raw_draws(w)
    q, k, _, _ = make_inputs(w)
    rows = spike_rows(w)
    # every row but the first of each (b, h) carries a spike
    assert [(b, h, t) for b, h, t, _ in rows] == [
        (b, h, t) for b in range(w.B) for h in range(w.H) for t in range(1, w.T)]
    for b, h, t, js in rows:
        assert 0 <= js <= t
        m, amax = margins(q, k, b, h, t, js, w.d)
        assert amax == js
        # the construction takes the smallest shift that meets every margin,
        # so the closest competitor sits exactly ``gap`` below (fp32 cast aside)
        assert abs(m - 20.0) < 1e-4, (b, h, t, js, m)
    # row 0 has one key only and keeps its scaled draw
    assert np.array_equal(q[:, :, 0], (rq[:, :, 0] * 11.0).astype(np.float32))
    assert np.array_equal(k, rk.astype(np.float32))


def test_spike_shift_is_along_the_chosen_key():
    w = WORKLOADS["c3"].scaled(B=1, H=1, T=24)
    _, (rq, rk, _, _) = raw_draws(w)
    q, _, _, _ = make_inputs(w)
    for b, h, t, js in spike_rows(w):
        delta = q[b, h, t].astype(np.float64) - rq[b, h, t] * w.q_scale
        g = float(delta @ rk[b, h, js]) / float(rk[b, h, js] @ rk[b, h, js])
        np.testing.assert_allclose(delta, g * rk[b, h, js], atol=1e-5 * max(1.0, abs(g)))
        assert g > 0


def test_spike_frac_picks_that_share_of_rows():
    w = WORKLOADS["c5"].scaled(B=2, H=3, T=200)
    rng, (rq, rk, _, _) = raw_draws(w)
    q, k, _, _ = make_inputs(w)
    rows = spike_rows(w)
    n_rows = w.B * w.H * (w.T - 1)
    assert len(rows) == round(0.01 * n_rows) == 12
    picked = {(b, h, t) for b, h, t, _ in rows}
    assert len(picked) == len(rows)
    assert all(t >= 1 for _, _, t in picked)
    for b, h, t, js in rows:
        m, amax = margins(q, k, b, h, t, js, w.d)
        assert amax == js
        assert abs(m - 40.0) < 1e-4, (b, h, t, js, m)
    # the other rows keep their (unscaled) draws
    for b in range(w.B):
        for h in range(w.H):
            for t in range(w.T):
                if (b, h, t) not in picked:
                    assert np.array_equal(q[b, h, t], rq[b, h, t].astype(np.float32))


def test_spike_rows_follow_the_drawn_stream():
    # the row choice and j* come from the stream after the four tensors
    w = WORKLOADS["c5"].scaled(B=1, H=2, T=300, seed=7)
    rng, _ = raw_draws(w)
    flat = np.array([h * w.T + t for h in range(w.H) for t in range(1, w.T)], dtype=np.int64)
    pick = np.sort(rng.choice(flat, size=int(round(w.frac * flat.size)), replace=False))
    want = [(0, int(f // w.T), int(f % w.T)) for f in pick]
    jst = [int(rng.integers(0, t + 1)) for _, _, t in want]
    assert spike_rows(w) == [(b, h, t, j) for (b, h, t), j in zip(want, jst)]


def test_seeds_are_deterministic_and_distinct():
    w = WORKLOADS["c3"].scaled(B=1, H=1, T=32)
    a = make_inputs(w)
    b = make_inputs(w)
    c = make_inputs(w.scaled(seed=1))
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    assert not np.array_equal(a[0], c[0])


def test_plain_workload_has_no_structural_rows():
    assert spike_rows(WORKLOADS["c1"]) == []
    assert spike_rows(WORKLOADS["c2"]) == []


def test_pairs_counts_causal_entries():
    w = Workload("x", 2, 3, 5, 8)
    assert w.pairs() == 2 * 3 * 15
    assert WORKLOADS["c2"].pairs() == 8 * 12 * 1024 * 1025 // 2


def test_measured_shapes():
    assert WORKLOADS["c2"].shape() == (8, 12, 1024, 64)
    assert WORKLOADS["c3"].shape() == (8, 12, 1024, 64)
    assert WORKLOADS["c4"].shape() == (4, 16, 2048, 128)
    assert WORKLOADS["c5"].shape() == (1, 12, 8192, 64)


def test_spike_gamma_rejects_a_parallel_key():
    keys = np.array([[1.0, 0.0], [2.0, 0.0]])
    with pytest.raises(ValueError):
        _spike_gamma(np.array([0.3, 0.1]), keys, 0, 5.0, 1.0)


def test_spike_gamma_single_key_needs_no_shift():
    assert _spike_gamma(np.array([0.3, 0.1]), np.array([[1.0, 2.0]]), 0, 5.0, 1.0) == 0.0


def test_unknown_kind_rejected():
    with pytest.raises(ValueError):
        make_inputs(Workload("x", 1, 1, 4, 4, "nope"))

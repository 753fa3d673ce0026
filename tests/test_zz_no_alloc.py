"""kia_backward_noalloc (the backward that allocates nothing, for callers
that cannot allocate) against kia_backward on the same forward state: equal
bits on consecutive calls of shrinking size, across the scratch's slice
groups, and the refusal of a slice larger than the scratch."""
import numpy as np
import pytest

from workloads import WORKLOADS, Workload, make_inputs

pytestmark = pytest.mark.gpu


def _run_both(w, params):
    import torch
    import quantized_softmax_attention_amd as kia
    dev = torch.device("cuda:0")
    q, k, v, do = (torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in make_inputs(w))
    o, stats = kia.kia_forward(q, k, v, params)
    ref = kia.kia_backward(q, k, v, o, do, stats, params)[:3]
    # outputs prefilled with NaN: every element must be written
    out = tuple(torch.full_like(q, float("nan")) for _ in range(3))
    got = kia.kia_backward_noalloc(q, k, v, o, do, stats, params, *out)
    torch.cuda.synchronize()
    return ref, got


CALLS = [
    # 64 slices of 17 MB of workspace: groups of 15 slices, Prob-STE extras and d = 128
    (WORKLOADS["c4"], dict(K=16, tau=6.0, calibration="fwm", reconstruction="nearest", surrogate="prob")),
    # smaller: 96 slices of 4.3 MB, two groups, P1's prefix sums in the workspace
    (WORKLOADS["c2"], dict(K=32, grad_rule="p1")),
    # smaller still: one group
    (Workload("noalloc_small", 1, 3, 200, 64, "scaled", q_scale=2.0), dict(K=8, reconstruction="nearest")),
]


def test_noalloc_backward_matches_backward_on_consecutive_calls():
    from quantized_softmax_attention_amd import Params
    for w, kw in CALLS:
        params = Params(**kw)
        print(f"[case] noalloc {w.name} B{w.B} H{w.H} T{w.T} d{w.d} {params}", flush=True)
        ref, got = _run_both(w, params)
        for name, a, b in zip(("dQ", "dK", "dV"), ref, got):
            assert bool(b.isfinite().all()), name
            assert np.array_equal(a.cpu().numpy().view(np.uint32), b.cpu().numpy().view(np.uint32)), name


def test_noalloc_refuses_a_slice_larger_than_its_scratch():
    import torch
    import quantized_softmax_attention_amd as kia
    from quantized_softmax_attention_amd import KiaError, Params
    dev = torch.device("cuda:0")
    T, d = 8192, 64
    q = torch.zeros((1, 1, T, d), dtype=torch.float32, device=dev)
    params = Params(K=4)
    stats = torch.empty(kia.kia_stats_bytes(params, 1, 1, T, d), dtype=torch.uint8, device=dev)
    with pytest.raises(KiaError) as e:
        kia.kia_backward_noalloc(q, q, q, q, q, stats, params)
    assert e.value.status == 7

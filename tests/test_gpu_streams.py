"""The library on a caller's stream, under HIP graph capture, and through
the autograd wrapper kia_attention.

The C ABI launches only on the stream it is given, never allocates and never
synchronises, so a forward + backward can run on any stream and be captured
into a graph.  Results are deterministic (no atomics), so every check here is
bitwise: a side stream against the current stream, and every replay of a
captured step against the eager step on the same inputs.  Between replays
the test runs other eager work (a step on different inputs) and synchronises,
and it checks each replay, not only the last.
"""
import numpy as np
import pytest

from workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu

W = Workload("streams", 2, 3, 200, 64, "scaled", q_scale=2.0)
W128 = Workload("streams_d128", 1, 2, 150, 128, "head_temp", lo=0.5, hi=3.0)


def _params(**kw):
    from quantized_softmax_attention_amd import Params
    return Params(**kw)


def _tensors(seed_shift=0, w=W):
    import torch
    q, k, v, do = make_inputs(w)
    if seed_shift:
        q = np.roll(q, seed_shift, axis=2)
    dev = torch.device("cuda:0")
    return tuple(torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in (q, k, v, do))


def _step(kia, x, p, out, stream=None):
    q, k, v, do = x
    o, st, dq, dk, dv, ws = out
    kia.kia_forward(q, k, v, p, o=o, stats=st, stream=stream)
    kia.kia_backward(q, k, v, o, do, st, p, dq=dq, dk=dk, dv=dv, ws=ws, stream=stream)


def _alloc(kia, x, p):
    import torch
    q = x[0]
    B, H, T, d = q.shape
    st = torch.empty(kia.kia_stats_bytes(p, B, H, T, d), dtype=torch.uint8, device=q.device)
    ws = torch.empty(kia.kia_workspace_bytes(p, B, H, T, d), dtype=torch.uint8, device=q.device)
    return (torch.empty_like(q), st, torch.empty_like(q), torch.empty_like(q), torch.empty_like(q), ws)


VARIANTS = [dict(K=32), dict(K=4, calibration="fwm", reconstruction="nearest", surrogate="prob"),
            dict(K=4, grad_rule="p1"), dict(K=1, reconstruction="exp_fp8"), dict(K=16, d128=True),
            dict(K=4, calibration="fwm", reconstruction="nearest", surrogate="prob", grad_rule="p1", d128=True)]


def _variant(kw):
    """Params and workload of a variant (d128 selects the d = 128 workload)."""
    kw = dict(kw)
    return _params(**{k: v for k, v in kw.items() if k != "d128"}), (W128 if kw.get("d128") else W)


@pytest.mark.parametrize("kw", VARIANTS, ids=lambda kw: "-".join(f"{k}={v}" for k, v in kw.items()))
def test_side_stream_matches_current_stream(kw):
    import torch
    import quantized_softmax_attention_amd as kia
    p, w = _variant(kw)
    x = _tensors(w=w)
    a, b = _alloc(kia, x, p), _alloc(kia, x, p)
    print(f"[case] side stream {p}", flush=True)
    _step(kia, x, p, a)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    _step(kia, x, p, b, stream=s)
    torch.cuda.synchronize()
    for name, ga, gb in zip(("o", "dq", "dk", "dv"), (a[0], a[2], a[3], a[4]), (b[0], b[2], b[3], b[4])):
        assert torch.equal(ga, gb), name


@pytest.mark.parametrize("kw", VARIANTS, ids=lambda kw: "-".join(f"{k}={v}" for k, v in kw.items()))
def test_graph_replays_match_eager(kw):
    import torch
    import quantized_softmax_attention_amd as kia
    p, w = _variant(kw)
    x = _tensors(w=w)
    other = _tensors(seed_shift=17, w=w)
    eager = _alloc(kia, x, p)
    print(f"[case] graph capture {p}", flush=True)
    _step(kia, x, p, eager)
    torch.cuda.synchronize()
    want = [t.clone() for t in (eager[0], eager[2], eager[3], eager[4])]

    cap = _alloc(kia, x, p)
    side = _alloc(kia, other, p)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        _step(kia, x, p, cap)             # warm the stream before capture
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            _step(kia, x, p, cap)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (cap[0], cap[2], cap[3], cap[4]):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        _step(kia, other, p, side)        # other eager work between replays
        torch.cuda.synchronize()
        for name, got, ref in zip(("o", "dq", "dk", "dv"), (cap[0], cap[2], cap[3], cap[4]), want):
            assert torch.equal(got, ref), (rep, name)


@pytest.mark.parametrize("kw", VARIANTS, ids=lambda kw: "-".join(f"{k}={v}" for k, v in kw.items()))
def test_autograd_op_matches_direct_calls(kw):
    """kia_attention (the autograd wrapper) returns kia_forward's O and, from
    torch.autograd, exactly kia_backward's dQ, dK, dV."""
    import torch
    import quantized_softmax_attention_amd as kia
    p, w = _variant(kw)
    q, k, v, do = _tensors(w=w)
    print(f"[case] autograd op {p}", flush=True)
    o_ref, st = kia.kia_forward(q, k, v, p)
    dq_ref, dk_ref, dv_ref, _ = kia.kia_backward(q, k, v, o_ref, do, st, p)
    qa, ka, va = (t.clone().requires_grad_(True) for t in (q, k, v))
    o = kia.kia_attention(qa, ka, va, p)
    dq, dk, dv = torch.autograd.grad(o, (qa, ka, va), grad_outputs=do)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), o_ref)
    for name, got, ref in (("dq", dq, dq_ref), ("dk", dk, dk_ref), ("dv", dv, dv_ref)):
        assert torch.equal(got, ref), name


TABLE_VARIANTS = [dict(K=32), dict(K=32, reconstruction="nearest"),
                  dict(K=4, calibration="fwm", reconstruction="nearest", surrogate="prob"),
                  dict(K=16, calibration="fwm", grad_rule="detach"), dict(K=16, d128=True),
                  dict(K=4, calibration="fwm", reconstruction="nearest", surrogate="prob", grad_rule="p1", d128=True)]


@pytest.mark.parametrize("kw", TABLE_VARIANTS, ids=lambda kw: "-".join(f"{k}={v}" for k, v in kw.items()))
def test_grid_table_matches_per_score_exponential(kw, monkeypatch):
    """The row kernel's per-row grid table holds exactly the values the
    per-score exponential computes (same expression, same inputs), so the
    backward with KIA_GRID_TABLE=0 is bitwise the same."""
    import torch
    import quantized_softmax_attention_amd as kia
    p, w = _variant(kw)
    x = _tensors(w=w)
    with_table, without = _alloc(kia, x, p), _alloc(kia, x, p)
    print(f"[case] grid table on / off {p}", flush=True)
    monkeypatch.delenv("KIA_GRID_TABLE", raising=False)
    _step(kia, x, p, with_table)
    monkeypatch.setenv("KIA_GRID_TABLE", "0")
    _step(kia, x, p, without)
    monkeypatch.delenv("KIA_GRID_TABLE")
    torch.cuda.synchronize()
    for name, ga, gb in zip(("o", "dq", "dk", "dv"), (with_table[0], with_table[2], with_table[3], with_table[4]),
                            (without[0], without[2], without[3], without[4])):
        assert torch.equal(ga, gb), name
    # the stored P and dS tiles too
    B, H, T, _ = x[0].shape
    WL = kia.kia_workspace_layout_query(p, *x[0].shape)
    for off in (WL.probs, WL.dscores):
        ta = kia.kia_tiles_to_dense(B, H, T, with_table[5][off:], True)
        tb = kia.kia_tiles_to_dense(B, H, T, without[5][off:], True)
        assert torch.equal(ta, tb)


@pytest.mark.parametrize("kw", VARIANTS, ids=lambda kw: "-".join(f"{k}={v}" for k, v in kw.items()))
def test_prepared_step_matches_direct_calls(kw):
    """kia.Step (buffers checked once, then the C ABI called with stored
    arguments) computes exactly what kia_forward + kia_backward compute."""
    import torch
    import quantized_softmax_attention_amd as kia
    p, w = _variant(kw)
    x = _tensors(w=w)
    direct, prepared = _alloc(kia, x, p), _alloc(kia, x, p)
    print(f"[case] prepared step {p}", flush=True)
    _step(kia, x, p, direct)
    q, k, v, do = x
    o, st, dq, dk, dv, ws = prepared
    step = kia.Step(q, k, v, do, p, o, st, dq, dk, dv, ws)
    for t in (o, dq, dk, dv):
        t.fill_(float("nan"))
    step()
    torch.cuda.synchronize()
    for name, ga, gb in zip(("o", "dq", "dk", "dv"), (direct[0], direct[2], direct[3], direct[4]), (o, dq, dk, dv)):
        assert torch.equal(ga, gb), name

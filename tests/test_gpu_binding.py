"""The Python binding checks every buffer a caller passes (device, dtype,
shape, byte size) before the library sees it, and sizes buffers of any
dtype by bytes."""
import numpy as np
import pytest

from workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu

W = Workload("binding", 1, 2, 100, 64, "scaled", q_scale=2.0)


def _inputs():
    import torch
    dev = torch.device("cuda:0")
    return tuple(torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in make_inputs(W))


def test_bad_buffers_rejected():
    import torch
    import quantized_softmax_attention_amd as kia
    print("[case] binding buffer checks", flush=True)
    q, k, v, do = _inputs()
    p = kia.Params(K=8)
    o, st = kia.kia_forward(q, k, v, p)
    with pytest.raises(ValueError, match="shape"):
        kia.kia_forward(q, k, v, p, o=torch.empty(1, 2, 99, 64, device=q.device))
    with pytest.raises(ValueError, match="bytes"):
        kia.kia_forward(q, k, v, p, stats=st[: st.numel() // 2])
    with pytest.raises(ValueError, match="shape"):
        kia.kia_backward(q, k, v, o, do, st, p, dq=torch.empty(1, 2, 100, 32, device=q.device))
    with pytest.raises(ValueError, match="bytes"):
        kia.kia_backward(q, k, v, o, do, st[:1024], p)
    ws_bytes = kia.kia_workspace_bytes(p, 1, 2, 100, 64)
    with pytest.raises(ValueError, match="bytes"):
        kia.kia_backward(q, k, v, o, do, st, p, ws=torch.empty(ws_bytes - 1, dtype=torch.uint8, device=q.device))
    with pytest.raises(ValueError, match="float32"):
        kia.kia_backward(q, k, v, o, do.double(), st, p)
    with pytest.raises(ValueError, match="shape"):
        kia.kia_geometry(q, k, st, p, geo=torch.empty(8, 1, 2, 99, device=q.device))
    with pytest.raises(ValueError, match="bytes"):
        kia.kia_tiles_to_dense(1, 2, 100, st[:4096], False)
    torch.cuda.synchronize()


def test_buffers_sized_by_bytes():
    """A float32 workspace and stats buffer of the right byte size give the
    same bits as the uint8 buffers the binding allocates."""
    import torch
    import quantized_softmax_attention_amd as kia
    print("[case] binding byte-sized buffers", flush=True)
    q, k, v, do = _inputs()
    p = kia.Params(K=8)
    o, st = kia.kia_forward(q, k, v, p)
    dq, dk, dv, _ = kia.kia_backward(q, k, v, o, do, st, p)
    sb = kia.kia_stats_bytes(p, 1, 2, 100, 64)
    wb = kia.kia_workspace_bytes(p, 1, 2, 100, 64)
    st4 = torch.empty((sb + 3) // 4, dtype=torch.float32, device=q.device)
    ws4 = torch.empty((wb + 3) // 4, dtype=torch.float32, device=q.device)
    o2, _ = kia.kia_forward(q, k, v, p, stats=st4)
    dq2, dk2, dv2, _ = kia.kia_backward(q, k, v, o2, do, st4, p, ws=ws4)
    torch.cuda.synchronize()
    for a, b in ((o, o2), (dq, dq2), (dk, dk2), (dv, dv2)):
        assert torch.equal(a, b)

"""The Python binding rejects tensors it cannot hand to the library before
any call reaches it (no GPU needed: CPU tensors are never GPU tensors)."""
import pytest

torch = pytest.importorskip("torch")


def _kia():
    import quantized_softmax_attention_amd as kia
    return kia


def test_cpu_tensors_rejected():
    kia = _kia()
    q = torch.zeros(1, 1, 8, 64)
    p = kia.Params(K=4)
    with pytest.raises(ValueError, match="GPU tensor"):
        kia.kia_forward(q, q, q, p)
    with pytest.raises(ValueError, match="GPU tensor"):
        kia.kia_backward(q, q, q, q, q, torch.zeros(16, dtype=torch.uint8), p)
    with pytest.raises(ValueError, match="GPU tensor"):
        kia.kia_geometry(q, q, torch.zeros(16, dtype=torch.uint8), p)
    with pytest.raises(ValueError, match="GPU tensor"):
        kia.kia_tiles_to_dense(1, 1, 8, torch.zeros(4096, dtype=torch.uint8), False)


def test_rank_checked():
    kia = _kia()
    with pytest.raises(ValueError, match=r"\[B, H, T, d\]"):
        kia.kia_forward(torch.zeros(8, 64), torch.zeros(8, 64), torch.zeros(8, 64), kia.Params(K=4))

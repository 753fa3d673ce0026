"""Host-side tests of libkia: it loads, exports every function include/kia.h
declares, sizes its buffers, and rejects bad arguments before any launch.

No kernel is launched here (no GPU in the CPU suite): every call below either
is a pure size query or returns an error status before its first launch.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kia.h")


def _lib():
    from quantized_softmax_attention_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libkia.so not built (run __graft_entry__.build())")
    return _lib.load(), _lib


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(kia_\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_documented_entry_points():
    names = declared_functions()
    for must in ("kia_forward", "kia_backward", "kia_stats_bytes", "kia_workspace_bytes",
                 "kia_forward_ext", "kia_backward_ext", "kia_status_str"):
        assert must in names


def test_library_exports_every_declared_symbol():
    lib, mod = _lib()
    names = declared_functions()
    assert names, "no declarations parsed"
    for name in names:
        assert hasattr(lib, name), f"libkia.so does not export {name}"
        assert name in mod.SIGNATURES, f"binding has no signature for {name}"
    assert set(mod.SIGNATURES) == set(names)
    assert lib.kia_abi_version() == 4


def _params(mod, K=4, tau=6.0, cal=0, rec=0, ste=0, rule=0):
    return mod.KiaParams(K, tau, cal, rec, ste, rule)


def test_size_queries():
    lib, mod = _lib()
    p = _params(mod)
    B, H, T, d = 2, 3, 100, 64
    n_t = (T + 31) // 32
    tiles = B * H * n_t * (n_t + 1) // 2 * 1024 * 4
    sb = lib.kia_stats_bytes(ctypes.byref(p), B, H, T, d)
    wb = lib.kia_workspace_bytes(ctypes.byref(p), B, H, T, d)
    assert sb >= tiles + 6 * B * H * T * 4
    assert wb >= 2 * tiles + 2 * B * H * T * 4
    L = mod.KiaStatsLayout()
    assert lib.kia_stats_layout_query(ctypes.byref(p), B, H, T, d, ctypes.byref(L)) == 0
    assert L.total_bytes == sb and L.tiles_per_head == n_t * (n_t + 1) // 2 and L.o_lerp == 0
    offs = [L.scores, L.row_m, L.row_n, L.row_a, L.row_b, L.row_w, L.row_wl]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    # Prob-STE keeps the LERP-probability output as well
    pp = _params(mod, rec=1, ste=1)
    Lp = mod.KiaStatsLayout()
    assert lib.kia_stats_layout_query(ctypes.byref(pp), B, H, T, d, ctypes.byref(Lp)) == 0
    assert Lp.o_lerp > 0 and Lp.total_bytes >= sb + B * H * T * d * 4
    W = mod.KiaWorkspaceLayout()
    assert lib.kia_workspace_layout_query(ctypes.byref(p), B, H, T, d, ctypes.byref(W)) == 0
    assert W.total_bytes == wb and W.dscores >= W.probs + tiles
    assert W.prefix_k == 0 and W.chunk_k == 0
    # P1 adds the causal prefix sums of K and their chunk sums
    p1 = _params(mod, rule=4)
    W1 = mod.KiaWorkspaceLayout()
    assert lib.kia_workspace_layout_query(ctypes.byref(p1), B, H, T, d, ctypes.byref(W1)) == 0
    assert W1.prefix_k >= W1.row_cn + B * H * T * 4 and W1.chunk_k >= W1.prefix_k + B * H * T * d * 4
    assert W1.total_bytes >= W1.chunk_k + B * H * n_t * d * 4
    # invalid arguments size to zero
    assert lib.kia_stats_bytes(ctypes.byref(p), B, H, T, 96) == 0
    assert lib.kia_stats_bytes(ctypes.byref(_params(mod, K=0)), B, H, T, d) == 0
    assert lib.kia_stats_bytes(None, B, H, T, d) == 0


# fake, 16-byte aligned "device" addresses: never dereferenced because every
# call below fails its checks before launching
A = 0x7000_0000_0000


def _fwd(lib, p, B=1, H=1, T=8, d=64, q=A, k=A, v=A, o=A, stats=A, nbytes=1 << 40):
    return lib.kia_forward(ctypes.byref(p) if p is not None else None, B, H, T, d, q, k, v, o, stats, nbytes, None)


def _bwd(lib, p, ptrs=None, nbytes=1 << 40, wbytes=1 << 40, T=8, d=64):
    ptrs = ptrs or [A] * 10
    q, k, v, o, do, st, dq, dk, dv, ws = ptrs
    return lib.kia_backward(ctypes.byref(p), 1, 1, T, d, q, k, v, o, do, st, nbytes, dq, dk, dv, ws, wbytes, None)


@pytest.mark.parametrize("field,value", [("n_intervals", 0), ("n_intervals", 65537), ("calibration", 3),
                                         ("reconstruction", -1), ("reconstruction", 5), ("surrogate", 3),
                                         ("grad_rule", 5)])
def test_bad_params_rejected(field, value):
    lib, mod = _lib()
    p = _params(mod)
    setattr(p, field, value)
    assert _fwd(lib, p) == 3
    assert _bwd(lib, p) == 3


@pytest.mark.parametrize("tau", [0.0, -1.0, float("inf"), float("nan")])
def test_bad_tau_rejected_under_fwm_only(tau):
    lib, mod = _lib()
    assert _fwd(lib, _params(mod, tau=tau, cal=1)) == 3
    # MinMax ignores tau; with a too-small stats buffer it fails on the buffer instead
    assert _fwd(lib, _params(mod, tau=tau, cal=0), nbytes=16) == 5


def test_bad_shapes_rejected():
    lib, mod = _lib()
    p = _params(mod)
    for B, H, T, d in [(0, 1, 8, 64), (1, 0, 8, 64), (1, 1, 0, 64), (1, 1, 8, 32), (1, 1, 8, 96), (1, 1, -5, 64)]:
        assert _fwd(lib, p, B=B, H=H, T=T, d=d) == 2


@pytest.mark.parametrize("B,H,T", [(1 << 16, 1 << 16, 8),           # B*H past int32 (grid index)
                                   (1 << 16, 1 << 10, 1 << 11),     # B*H*n_t workgroups past int32
                                   (1 << 15, 1 << 15, 1 << 20)])    # score tiles past 9e18 bytes
def test_oversized_shapes_rejected(B, H, T):
    """Shapes whose grid or tile buffer would overflow the library's index
    types are refused by every entry point, and size to zero."""
    lib, mod = _lib()
    p = _params(mod)
    assert _fwd(lib, p, B=B, H=H, T=T) == 2
    assert lib.kia_stats_bytes(ctypes.byref(p), B, H, T, 64) == 0
    assert lib.kia_workspace_bytes(ctypes.byref(p), B, H, T, 64) == 0
    ptrs = [A] * 10
    q, k, v, o, do, st, dq, dk, dv, ws = ptrs
    assert lib.kia_backward(ctypes.byref(p), B, H, T, 64, q, k, v, o, do, st, 1 << 40, dq, dk, dv, ws,
                            1 << 40, None) == 2


def test_null_misaligned_and_small_buffers_rejected():
    lib, mod = _lib()
    p = _params(mod)
    assert _fwd(lib, None) == 1
    assert _fwd(lib, p, q=0) == 1
    assert _fwd(lib, p, stats=0) == 1
    assert _fwd(lib, p, k=A + 4) == 4
    assert _fwd(lib, p, nbytes=1024) == 5
    ptrs = [A] * 10
    for i in range(10):
        bad = list(ptrs)
        bad[i] = 0
        assert _bwd(lib, p, bad) == 1
        bad[i] = A + 8
        assert _bwd(lib, p, bad) == 4
    assert _bwd(lib, p, wbytes=64) == 5
    assert _bwd(lib, p, nbytes=64) == 5


def test_geometry_probe_size_and_argument_checks():
    lib, mod = _lib()
    p = _params(mod)
    assert lib.kia_geometry_bytes(2, 3, 100) == 8 * 2 * 3 * 100 * 4
    assert lib.kia_geometry_bytes(0, 3, 100) == 0
    B, H, T, d = 1, 2, 40, 64
    nbytes = lib.kia_stats_bytes(p, B, H, T, d)
    gbytes = lib.kia_geometry_bytes(B, H, T)

    def geo(p=p, q=A, k=A, stats=A, sb=nbytes, g=A, gb=gbytes, T=T, d=d):
        return lib.kia_geometry(p, B, H, T, d, q, k, stats, sb, g, gb, None)

    assert geo(p=None) == 1
    assert geo(q=0) == 1 and geo(k=0) == 1 and geo(stats=0) == 1 and geo(g=0) == 1
    assert geo(g=A + 4) == 4 and geo(stats=A + 8) == 4
    assert geo(sb=nbytes - 1) == 5
    assert geo(gb=gbytes - 4) == 5
    assert geo(d=96) == 2 and geo(T=0) == 2
    assert geo(p=_params(mod, cal=1, tau=0.0)) == 3


def test_status_strings():
    lib, _ = _lib()
    for s in range(8):
        assert lib.kia_status_str(s)
    assert b"unknown" in lib.kia_status_str(99)


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    from quantized_softmax_attention_amd import _lib as mod
    monkeypatch.setattr(mod, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(mod, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        mod.load()


def test_noalloc_backward_argument_checks():
    """kia_backward_noalloc validates like kia_backward and refuses, before any
    launch, a shape whose single slice needs more workspace than its scratch
    (T = 8192: 32,896 tiles of P and dS, 270 MB > 256 MiB)."""
    lib, mod = _lib()
    p = _params(mod)
    B, H, T, d = 2, 3, 100, 64
    nbytes = lib.kia_stats_bytes(p, B, H, T, d)

    def call(p=p, ptrs=None, sb=nbytes, T=T, d=d):
        q, k, v, o, do, st, dq, dk, dv = ptrs or [A] * 9
        return lib.kia_backward_noalloc(p, B, H, T, d, q, k, v, o, do, st, sb, dq, dk, dv, None)

    assert call(p=None) == 1
    for i in range(9):
        bad = [A] * 9
        bad[i] = 0
        assert call(ptrs=bad) == 1
        bad[i] = A + 8
        assert call(ptrs=bad) == 4
    assert call(sb=nbytes - 1) == 5
    assert call(d=96) == 2 and call(T=0) == 2
    assert call(p=_params(mod, cal=1, tau=0.0)) == 3
    big = lib.kia_stats_bytes(p, B, H, 8192, d)
    assert call(sb=big, T=8192) == 7
    assert lib.kia_workspace_bytes(p, 1, 1, 8192, d) > 256 << 20
    assert lib.kia_workspace_bytes(p, 1, 1, 4096, d) <= 256 << 20

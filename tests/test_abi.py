"""The C-ABI library loads and exports what include/ringag.h declares (CPU only: no device calls
beyond the argument checks that come before any HIP call)."""
import ctypes

import pytest

from ring_all_gather_amd import binding as B


def test_header_declares_the_boundary():
    names = B.declared_functions()
    for f in ("rag_create", "rag_destroy", "rag_set_option", "ag_gemm", "gemm_rs", "rag_check",
              "rag_kernel_times", "rag_last_error", "rag_version", "rag_ag_kernel_name",
              "rag_rs_kernel_name", "gemm_rs_ring", "linear_allreduce",
              "ag_gemm_ex"):
        assert f in names


def test_library_exports_every_declared_symbol():
    L = B.lib()
    missing = [f for f in B.declared_functions() if not hasattr(L, f)]
    assert not missing, f"not exported: {missing}"
    assert L.rag_version() == 100


def test_argument_errors_before_any_device_call():
    L = B.lib()
    h = ctypes.c_void_p()
    assert L.rag_create(ctypes.byref(h), 0, 0, 0) == B.RAG_EINVAL
    assert "max_tp" in B.last_error()
    assert L.rag_create(ctypes.byref(h), 0, B.RAG_MAX_TP + 1, 0) == B.RAG_EINVAL
    assert L.rag_create(ctypes.byref(h), 0, 4, 1) == B.RAG_EINVAL
    assert "flags" in B.last_error()
    assert L.rag_create(None, 0, 4, 0) == B.RAG_EINVAL
    assert L.rag_destroy(None) == B.RAG_OK
    assert L.rag_set_option(None, B.RAG_OPT_TILE, 0) == B.RAG_EINVAL
    assert L.rag_check(None) == B.RAG_EINVAL
    assert L.rag_kernel_times(None, None, 0) == B.RAG_EINVAL
    ptrs = (ctypes.c_void_p * 1)(None)
    assert L.ag_gemm(None, None, 1, 64, ptrs, 1, 1, 0, None, None, 0, None, None, 0,
                     None) == B.RAG_EINVAL
    assert "ctx is NULL" in B.last_error()
    assert L.gemm_rs(None, None, 1, 64, None, 1, None, 1, 1, 0, None, None, 0,
                     None) == B.RAG_EINVAL


def test_no_device_is_reported_not_crashed():
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    h = ctypes.c_void_p()
    rc = B.lib().rag_create(ctypes.byref(h), 0, 4, 0)
    assert rc in (B.RAG_EHIP, B.RAG_EINVAL)
    assert B.last_error()


def test_binding_refuses_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        B.lib()

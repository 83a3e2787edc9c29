"""The C-ABI library loads and exports every symbol the header declares
(CPU only: no compute call is made)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("rskv.h", "rskv_retrieval.h", "rskv_window.h")]
LIB = os.path.join(ROOT, "routed_sparse_kv_amd", "lib", "librskv.so")


def declared_symbols():
    text = "".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rskv_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    syms = declared_symbols()
    for s in ("rskv_build_spans", "rskv_decode_step", "rskv_append_kv", "rskv_append_token",
              "rskv_cache_export",
              "rskv_cache_import", "rskv_cache_destroy", "rskv_last_error",
              "rskv_retrieval_build", "rskv_retrieval_decode", "rskv_retrieval_export",
              "rskv_retrieval_trace_get", "rskv_retrieval_destroy",
              "rskv_window_build", "rskv_window_decode", "rskv_window_info_get",
              "rskv_window_state_get", "rskv_window_profile_enable", "rskv_window_profile_read",
              "rskv_window_destroy"):
        assert s in syms


@pytest.mark.skipif(not os.path.exists(LIB), reason="librskv.so not built")
def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(LIB)
    missing = [s for s in declared_symbols() if not hasattr(lib, s)]
    assert not missing, missing


@pytest.mark.skipif(not os.path.exists(LIB), reason="librskv.so not built")
def test_version_and_error_strings_without_gpu():
    lib = ctypes.CDLL(LIB)
    lib.rskv_version.restype = ctypes.c_char_p
    lib.rskv_last_error.restype = ctypes.c_char_p
    assert lib.rskv_version().startswith(b"rskv")
    # invalid handle: rejected on the host before any HIP call
    lib.rskv_append_kv.argtypes = [ctypes.c_void_p] * 4
    assert lib.rskv_append_kv(None, None, None, None) == -6
    assert b"invalid cache handle" in lib.rskv_last_error()
    lib.rskv_append_token.argtypes = [ctypes.c_void_p] * 5
    assert lib.rskv_append_token(None, None, None, None, None) == -6
    lib.rskv_retrieval_decode.argtypes = [ctypes.c_void_p] * 5
    assert lib.rskv_retrieval_decode(None, None, None, None, None) == -6
    assert b"invalid retrieval handle" in lib.rskv_last_error()
    lib.rskv_window_decode.argtypes = [ctypes.c_void_p] * 4
    assert lib.rskv_window_decode(None, None, None, None) == -6
    assert b"invalid window cache handle" in lib.rskv_last_error()
    lib.rskv_window_build.argtypes = [ctypes.c_void_p] * 5
    out = ctypes.c_void_p(1)
    assert lib.rskv_window_build(None, None, None, None, ctypes.byref(out)) == -1
    assert out.value is None


def test_binding_fails_loudly_without_library(monkeypatch):
    from routed_sparse_kv_amd import binding
    monkeypatch.setattr(binding, "LIB_PATH", os.path.join(ROOT, "nonexistent.so"))
    monkeypatch.setattr(binding, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        binding.lib()

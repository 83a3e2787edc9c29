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


def _c_layout(structs):
    """sizeof and field offsets of header structs, from a C program that
    gcc compiles against the headers (host code only)."""
    import shutil
    import subprocess
    import tempfile
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    lines = ['#include <stddef.h>', '#include <stdio.h>', '#include "rskv.h"',
             '#include "rskv_window.h"', '#include "rskv_retrieval.h"', "int main(void) {"]
    for name, fields in structs.items():
        lines.append(f'printf("{name} size %zu\\n", sizeof({name}));')
        for f in fields:
            lines.append(f'printf("{name} {f} %zu\\n", offsetof({name}, {f}));')
    lines += ["return 0;", "}"]
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "layout.c"), os.path.join(d, "layout")
        open(src, "w").write("\n".join(lines))
        subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), src, "-o", exe],
                       check=True)
        out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout
    res = {}
    for line in out.splitlines():
        name, field, val = line.split()
        res[(name, field)] = int(val)
    return res


def test_ctypes_structs_match_the_headers():
    """Every option/info struct the binding passes has the header's size and
    field offsets (the allocator hook included)."""
    from routed_sparse_kv_amd import binding, retrieval, window
    pairs = {"rskv_build_opts": binding.BuildOpts, "rskv_cache_info": binding.CacheInfo,
             "rskv_host_arrays": binding.HostArrays, "rskv_profile": binding.Profile,
             "rskv_allocator": binding.Allocator, "rskv_window_opts": window.WindowOpts,
             "rskv_window_info": window.WindowInfo, "rskv_window_state": window.WindowState,
             "rskv_window_profile": window.WindowProfile,
             "rskv_retrieval_opts": retrieval.RetrievalOpts,
             "rskv_retrieval_info": retrieval.RetrievalInfo,
             "rskv_retrieval_host": retrieval.RetrievalHost,
             "rskv_retrieval_trace": retrieval.RetrievalTrace,
             "rskv_retrieval_profile": retrieval.RetrievalProfile}
    fields = {n: [f for f, _ in cls._fields_ if not f.endswith("_")] for n, cls in pairs.items()}
    lay = _c_layout(fields)
    for name, cls in pairs.items():
        assert lay[(name, "size")] == ctypes.sizeof(cls), name
        for f in fields[name]:
            assert lay[(name, f)] == getattr(cls, f).offset, (name, f)


@pytest.mark.skipif(not os.path.exists(LIB), reason="librskv.so not built")
def test_half_allocator_hook_is_rejected_before_any_device_call():
    from routed_sparse_kv_amd import binding
    lib = binding.lib()
    hook = binding.HookAllocator(lambda n, s: 0, lambda p, s: None)
    opts = binding.BuildOpts(batch=1, n_q_heads=1, n_kv_heads=1, head_dim=64, context_len=8,
                             dtype=0, anchor_frac=0.5, alpha=8.0, tail_capacity=0, k_max_cap=0,
                             factor_tier=0)
    opts.allocator.alloc = hook.struct.alloc  # free left NULL
    out = ctypes.c_void_p(1)
    rc = lib.rskv_build_spans(ctypes.c_void_p(16), ctypes.c_void_p(16), ctypes.c_void_p(16), 4,
                              ctypes.byref(opts), None, ctypes.byref(out))
    assert rc == -1 and b"allocator" in lib.rskv_last_error()
    assert out.value is None


@pytest.mark.skipif(not os.path.exists(LIB), reason="librskv.so not built")
def test_query_group_above_16_is_rejected_before_any_device_call():
    from routed_sparse_kv_amd import binding
    lib = binding.lib()
    opts = binding.BuildOpts(batch=1, n_q_heads=17, n_kv_heads=1, head_dim=64, context_len=8,
                             dtype=0, anchor_frac=0.5, alpha=8.0, tail_capacity=0, k_max_cap=0,
                             factor_tier=0)
    out = ctypes.c_void_p(1)
    rc = lib.rskv_build_spans(ctypes.c_void_p(16), ctypes.c_void_p(16), ctypes.c_void_p(16), 4,
                              ctypes.byref(opts), None, ctypes.byref(out))
    assert rc == -1 and b"above 16" in lib.rskv_last_error()
    assert out.value is None

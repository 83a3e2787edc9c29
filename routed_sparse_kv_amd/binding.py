"""ctypes binding of librskv.so (argument marshalling only).

Every computation runs in the HIP library; this module checks tensor
shapes/dtypes/devices, passes ``data_ptr()`` and the current HIP stream, and
raises ``RskvError`` with the library's message on failure.  There is no
fallback: if the shared library is missing, every call raises.
"""
from __future__ import annotations

import atexit
import ctypes as C
import os
import weakref
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "librskv.so")

F32, BF16 = 0, 1
DTYPE_NAMES = {F32: "f32", BF16: "bf16"}
TIERS = {"hbm": 0, "host": 1}  # where the span factors live


class RskvError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"rskv error {code}: {msg}")
        self.code = code


ALLOC_FN = C.CFUNCTYPE(C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p)
FREE_FN = C.CFUNCTYPE(None, C.c_void_p, C.c_void_p, C.c_void_p)


class Allocator(C.Structure):
    """rskv_allocator: device-memory hook of a cache (zeroed: hipMalloc)."""
    _fields_ = [("alloc", ALLOC_FN), ("free", FREE_FN), ("ctx", C.c_void_p)]


class HookAllocator:
    """A device allocator hook from two Python callables:
    ``alloc(nbytes, stream) -> int`` (device pointer, 0 on failure) and
    ``free(ptr, stream)``; ``stream`` is the hipStream_t as an int.  The
    object must outlive every cache built with it (the caches keep a
    reference)."""

    def __init__(self, alloc, free):
        self._alloc_py, self._free_py = alloc, free
        self._alloc_c = ALLOC_FN(self._on_alloc)
        self._free_c = FREE_FN(self._on_free)
        self.struct = Allocator(self._alloc_c, self._free_c, None)

    def _on_alloc(self, ctx, nbytes, stream):
        try:
            return self._alloc_py(int(nbytes), int(stream or 0)) or None
        except Exception:  # an exception must not cross the C boundary
            return None

    def _on_free(self, ctx, ptr, stream):
        try:
            self._free_py(int(ptr), int(stream or 0))
        except Exception:
            pass


_torch_hook = None


def torch_allocator() -> HookAllocator:
    """The hook that takes cache memory from torch's caching allocator on
    the stream of the allocating call (the binding's default)."""
    global _torch_hook
    if _torch_hook is None:
        torch = _torch()

        def alloc(nbytes, stream):
            return torch.cuda.caching_allocator_alloc(nbytes, stream=stream)

        def free(ptr, stream):
            torch.cuda.caching_allocator_delete(ptr)
        _torch_hook = HookAllocator(alloc, free)
    return _torch_hook


def resolve_allocator(allocator):
    """"torch" (default), "hip" (hipMalloc) or a HookAllocator ->
    (struct, object to keep alive)."""
    if allocator is None or allocator == "hip":
        return Allocator(), None
    if allocator == "torch":
        allocator = torch_allocator()
    if not isinstance(allocator, HookAllocator):
        raise TypeError("allocator must be 'torch', 'hip' or a HookAllocator")
    return allocator.struct, allocator


# Handles still open at interpreter exit are closed while torch (whose
# allocator the default hook calls) is still alive.
_live = weakref.WeakSet()


@atexit.register
def _close_live():
    for h in list(_live):
        try:
            h.close()
        except Exception:
            pass


class BuildOpts(C.Structure):
    _fields_ = [("batch", C.c_int32), ("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("context_len", C.c_int32), ("dtype", C.c_int32),
                ("anchor_frac", C.c_double), ("alpha", C.c_float), ("proj", C.c_void_p),
                ("n_proj", C.c_int32), ("tail_capacity", C.c_int32), ("k_max_cap", C.c_int32),
                ("factor_tier", C.c_int32), ("allocator", Allocator)]


class CacheInfo(C.Structure):
    _fields_ = [("batch", C.c_int32), ("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("context_len", C.c_int32), ("rank", C.c_int32),
                ("dtype", C.c_int32), ("n_spans_max", C.c_int32), ("n_full_cap", C.c_int32),
                ("n_span_tokens_max", C.c_int32), ("tail_capacity", C.c_int32),
                ("appended", C.c_int32), ("k_max_cap", C.c_int32), ("alpha", C.c_float),
                ("device_bytes", C.c_size_t), ("factor_tier", C.c_int32),
                ("host_bytes", C.c_size_t)]


_ARRAY_FIELDS = ["n_anchor", "n_spans", "n_full", "n_span_tokens", "span_id", "span_start",
                 "span_len", "full_pos", "summary", "vmean", "log_len", "k_full", "v_full",
                 "a_k", "a_v", "w_k", "w_v", "h_full", "theta", "last_anchor"]
_INT_FIELDS = ("n_anchor", "n_spans", "n_full", "n_span_tokens", "span_id", "span_start",
               "span_len", "full_pos", "last_anchor")
_F32_FIELDS = ("log_len", "h_full", "theta")


class HostArrays(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in _ARRAY_FIELDS]


class Profile(C.Structure):
    _fields_ = [("steps", C.c_int64), ("route_ms", C.c_double), ("topk_ms", C.c_double),
                ("attend_ms", C.c_double), ("merge_ms", C.c_double), ("appends", C.c_int64),
                ("close_ms", C.c_double), ("append_ms", C.c_double)]


_lib = None


def lib():
    """Load librskv.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = C.CDLL(LIB_PATH)
        vp, i32 = C.c_void_p, C.c_int32
        L.rskv_build_spans.argtypes = [vp, vp, vp, i32, C.POINTER(BuildOpts), vp, C.POINTER(vp)]
        L.rskv_decode_step.argtypes = [vp, vp, C.c_float, i32, vp, vp, vp, vp]
        L.rskv_append_kv.argtypes = [vp, vp, vp, vp]
        L.rskv_append_token.argtypes = [vp, vp, vp, vp, vp]
        L.rskv_cache_info_get.argtypes = [vp, C.POINTER(CacheInfo)]
        L.rskv_cache_export.argtypes = [vp, C.POINTER(HostArrays)]
        L.rskv_cache_import.argtypes = [C.POINTER(HostArrays), C.POINTER(BuildOpts), i32, i32,
                                        i32, i32, vp, C.POINTER(vp)]
        L.rskv_cache_destroy.argtypes = [vp]
        L.rskv_cache_destroy.restype = None
        L.rskv_decode_scores.argtypes = [vp, vp, vp]
        L.rskv_decode_step_static.argtypes = [vp, vp, C.c_float, i32, vp, vp, vp, vp]
        L.rskv_decode_static_capacity.restype = C.c_size_t
        L.rskv_profile_enable.argtypes = [vp, i32]
        L.rskv_profile_read.argtypes = [vp, C.POINTER(Profile)]
        L.rskv_last_error.restype = C.c_char_p
        L.rskv_version.restype = C.c_char_p
        for fn in ("rskv_build_spans", "rskv_decode_step", "rskv_decode_step_static",
                   "rskv_decode_scores", "rskv_append_kv",
                   "rskv_append_token",
                   "rskv_cache_info_get", "rskv_cache_export", "rskv_cache_import",
                   "rskv_profile_enable", "rskv_profile_read"):
            getattr(L, fn).restype = C.c_int
        _lib = L
    return _lib


def _check(rc: int):
    if rc != 0:
        raise RskvError(rc, lib().rskv_last_error().decode())


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(t, name, shape=None, dtype=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    return C.c_void_p(t.data_ptr())


def _stream():
    return C.c_void_p(_torch().cuda.current_stream().cuda_stream)


class Cache:
    """Owner of an rskv_cache handle."""

    def __init__(self, handle: C.c_void_p, keep=None):
        self._h = handle
        self._keep = keep  # the allocator hook, alive while the cache is
        self.info = self._info()
        _live.add(self)

    @property
    def handle(self):
        if not self._h:
            raise RskvError(-6, "cache already destroyed")
        return self._h

    def _info(self) -> dict:
        ci = CacheInfo()
        _check(lib().rskv_cache_info_get(self.handle, C.byref(ci)))
        return {n: getattr(ci, n) for n, _ in CacheInfo._fields_}

    def refresh(self) -> dict:
        self.info = self._info()
        return self.info

    @property
    def torch_dtype(self):
        torch = _torch()
        return torch.bfloat16 if self.info["dtype"] == BF16 else torch.float32

    def close(self):
        if self._h:
            lib().rskv_cache_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ------------------------------------------------------------ export
    def export(self) -> dict:
        """Every stored array, canonical layout (bf16 as uint16 bits)."""
        i = self.refresh()
        B, Hkv, d, T, r = i["batch"], i["n_kv_heads"], i["head_dim"], i["context_len"], i["rank"]
        S, F, N = i["n_spans_max"], i["n_full_cap"], i["n_span_tokens_max"]
        et = np.uint16 if i["dtype"] == BF16 else np.float32
        shapes = dict(n_anchor=((B,), np.int32), n_spans=((B,), np.int32),
                      n_full=((B,), np.int32), n_span_tokens=((B,), np.int32),
                      span_id=((B, T), np.int32), span_start=((B, S), np.int32),
                      span_len=((B, S), np.int32), full_pos=((B, F), np.int32),
                      summary=((B, Hkv, S, d), et), vmean=((B, Hkv, S, d), et),
                      log_len=((B, S), np.float32), k_full=((B, Hkv, F, d), et),
                      v_full=((B, Hkv, F, d), et), a_k=((B, Hkv, N, r), et),
                      a_v=((B, Hkv, N, r), et), w_k=((B, Hkv, S, r, d), et),
                      w_v=((B, Hkv, S, r, d), et), h_full=((B, F), np.float32),
                      theta=((B,), np.float32), last_anchor=((B,), np.int32))
        out = {k: np.zeros(sh, dt) for k, (sh, dt) in shapes.items()}
        ha = HostArrays(**{k: v.ctypes.data for k, v in out.items()})
        _check(lib().rskv_cache_export(self.handle, C.byref(ha)))
        out["info"] = dict(i)
        return out

    def scores(self):
        """(z [B][Hkv][S] fp64, n_spans [B]) of the last decode step."""
        i = self.info
        z = np.zeros((i["batch"], i["n_kv_heads"], i["n_spans_max"]), np.float64)
        ns = np.zeros(i["batch"], np.int32)
        _check(lib().rskv_decode_scores(self.handle, C.c_void_p(z.ctypes.data),
                                        C.c_void_p(ns.ctypes.data)))
        return z, ns

    # ------------------------------------------------------------ profile
    def profile_enable(self, on: bool = True):
        _check(lib().rskv_profile_enable(self.handle, 1 if on else 0))

    def profile_read(self) -> dict:
        p = Profile()
        _check(lib().rskv_profile_read(self.handle, C.byref(p)))
        return {n: getattr(p, n) for n, _ in Profile._fields_}


def build_spans(surprisal, K, V, rank: int, anchor_frac: float, n_q_heads: Optional[int] = None,
                alpha: float = 8.0, proj=None, tail_capacity: int = 0,
                k_max_cap: int = 0, factor_tier: str = "hbm", allocator="torch") -> Cache:
    """Build a cache.  surprisal [B][T] fp32; K, V [B][Hkv][T][d] (fp32 or
    bf16) on the GPU; proj [1 or Hkv][d][d] fp32 on the GPU or None;
    factor_tier "hbm" or "host" (span factors in pinned host memory);
    allocator "torch" (torch's caching allocator), "hip" (hipMalloc) or a
    HookAllocator."""
    torch = _torch()
    B, Hkv, T, d = K.shape
    dt = _dtype_code(K)
    hook, keep = resolve_allocator(allocator)
    opts = BuildOpts(batch=B, n_q_heads=n_q_heads or Hkv, n_kv_heads=Hkv, head_dim=d,
                     context_len=T, dtype=dt, anchor_frac=float(anchor_frac), alpha=float(alpha),
                     proj=None, n_proj=0, tail_capacity=int(tail_capacity),
                     k_max_cap=int(k_max_cap), factor_tier=TIERS[factor_tier], allocator=hook)
    args = [_dev(surprisal, "surprisal", (B, T), torch.float32),
            _dev(K, "K", (B, Hkv, T, d)), _dev(V, "V", (B, Hkv, T, d), K.dtype)]
    if proj is not None:
        opts.proj = _dev(proj, "proj", dtype=torch.float32).value
        opts.n_proj = proj.shape[0]
    h = C.c_void_p()
    _check(lib().rskv_build_spans(args[0], args[1], args[2], int(rank), C.byref(opts),
                                  _stream(), C.byref(h)))
    return Cache(h, keep)


def decode_step(cache: Cache, q, tau: float, k_max: int, out=None, sel=None, n_sel=None):
    """One decode step; returns ``out`` [B][Hq][d] fp32 (sel/n_sel filled if
    given: int32 [B][Hkv][k_max] and [B][Hkv])."""
    torch = _torch()
    i = cache.info
    B, Hq, Hkv, d = i["batch"], i["n_q_heads"], i["n_kv_heads"], i["head_dim"]
    qp = _dev(q, "q", (B, Hq, d), cache.torch_dtype)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    op = _dev(out, "out", (B, Hq, d), torch.float32)
    sp = _dev(sel, "sel", (B, Hkv, k_max), torch.int32) if sel is not None else None
    np_ = _dev(n_sel, "n_sel", (B, Hkv), torch.int32) if n_sel is not None else None
    _check(lib().rskv_decode_step(cache.handle, qp, C.c_float(tau), int(k_max), op, sp, np_,
                                  _stream()))
    return out


def decode_step_static(cache: Cache, q, tau: float, k_max: int, out, sel=None, n_sel=None):
    """decode_step through rskv_decode_step_static: the decode workspace is
    the library's static device array (no allocation); ``out`` must be
    given."""
    torch = _torch()
    i = cache.info
    B, Hq, Hkv, d = i["batch"], i["n_q_heads"], i["n_kv_heads"], i["head_dim"]
    qp = _dev(q, "q", (B, Hq, d), cache.torch_dtype)
    op = _dev(out, "out", (B, Hq, d), torch.float32)
    sp = _dev(sel, "sel", (B, Hkv, k_max), torch.int32) if sel is not None else None
    np_ = _dev(n_sel, "n_sel", (B, Hkv), torch.int32) if n_sel is not None else None
    _check(lib().rskv_decode_step_static(cache.handle, qp, C.c_float(tau), int(k_max), op, sp,
                                         np_, _stream()))
    return out


def decode_static_capacity() -> int:
    """Bytes of the static decode workspace of one GPU."""
    return int(lib().rskv_decode_static_capacity())


def append_kv(cache: Cache, k, v):
    """Append one token per sequence: k, v [B][Hkv][d] in the cache dtype
    (no surprisal: the token is never an anchor)."""
    i = cache.info
    shape = (i["batch"], i["n_kv_heads"], i["head_dim"])
    _check(lib().rskv_append_kv(cache.handle, _dev(k, "k", shape, cache.torch_dtype),
                                _dev(v, "v", shape, cache.torch_dtype), _stream()))
    cache.info["appended"] += 1


def append_token(cache: Cache, k, v, h=None):
    """Append one token per sequence with streaming segmentation: k, v
    [B][Hkv][d] in the cache dtype, h [B] fp32 surprisal on the GPU (or
    None: surprisal 0, never an anchor)."""
    torch = _torch()
    i = cache.info
    shape = (i["batch"], i["n_kv_heads"], i["head_dim"])
    hp = _dev(h, "h", (i["batch"],), torch.float32) if h is not None else None
    _check(lib().rskv_append_token(cache.handle, _dev(k, "k", shape, cache.torch_dtype),
                                   _dev(v, "v", shape, cache.torch_dtype), hp, _stream()))
    cache.info["appended"] += 1


def cache_import(arrays: dict, n_q_heads: int, rank: int, dtype: str, context_len: int,
                 alpha: float = 8.0, proj: Optional[np.ndarray] = None,
                 tail_capacity: int = 0, k_max_cap: int = 0, factor_tier: str = "hbm",
                 allocator="torch") -> Cache:
    """Create a cache from host arrays in the canonical (export) layout."""
    dt = BF16 if dtype == "bf16" else F32
    et = np.uint16 if dt == BF16 else np.float32
    keep = {}
    for k in _ARRAY_FIELDS:
        if k not in arrays:
            continue
        want = np.int32 if k in _INT_FIELDS else (np.float32 if k in _F32_FIELDS else et)
        keep[k] = np.ascontiguousarray(arrays[k], dtype=want)
    B, Hkv, S, d = keep["summary"].shape
    F = keep["k_full"].shape[2]
    N = keep["a_k"].shape[2]
    hook, hook_ref = resolve_allocator(allocator)
    opts = BuildOpts(batch=B, n_q_heads=n_q_heads, n_kv_heads=Hkv, head_dim=d,
                     context_len=context_len, dtype=dt, anchor_frac=0.0, alpha=float(alpha),
                     proj=None, n_proj=0, tail_capacity=int(tail_capacity),
                     k_max_cap=int(k_max_cap), factor_tier=TIERS[factor_tier], allocator=hook)
    if proj is not None:
        keep["_proj"] = np.ascontiguousarray(proj, dtype=np.float32)
        opts.proj = keep["_proj"].ctypes.data
        opts.n_proj = keep["_proj"].shape[0]
    ha = HostArrays(**{k: v.ctypes.data for k, v in keep.items() if k in _ARRAY_FIELDS})
    h = C.c_void_p()
    _check(lib().rskv_cache_import(C.byref(ha), C.byref(opts), int(rank), S, F, N, _stream(),
                                   C.byref(h)))
    return Cache(h, hook_ref)


def version() -> str:
    return lib().rskv_version().decode()

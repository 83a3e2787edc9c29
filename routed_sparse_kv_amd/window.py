"""ctypes binding of the window-routed three-tier cache (include/rskv_window.h).

Argument marshalling only: every step of the build and of the decode runs
in librskv.so; there is no fallback, a missing library raises.
"""
from __future__ import annotations

import ctypes as C
import numpy as np

from .binding import (BF16, F32, Allocator, RskvError, _check, _dev, _dtype_code, _live, _stream,
                      _torch, lib, resolve_allocator)

ROWS = 64    #: positions per window
GROUP = 64   #: coordinates per INT2 scale group
FULL, INT2, EVICTED = 0, 1, 2


class WindowOpts(C.Structure):
    _fields_ = [(n, C.c_int32) for n in
                ("batch", "n_q_heads", "n_kv_heads", "head_dim", "context_len", "dtype", "n_full",
                 "n_quant", "route_every")] + [("allocator", Allocator)]


class WindowInfo(C.Structure):
    _fields_ = [(n, C.c_int32) for n in
                ("batch", "n_q_heads", "n_kv_heads", "head_dim", "context_len", "dtype", "n_full",
                 "n_quant", "route_every", "n_windows")] + \
               [("step", C.c_int64)] + \
               [(n, C.c_int32) for n in ("next_full", "next_quant", "next_splits", "full_bytes",
                                         "quant_bytes")] + \
               [("device_bytes", C.c_size_t)]


class WindowState(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in
                ("tier", "score", "mass", "has_code", "code_k", "code_v", "scale_k", "min_k",
                 "scale_v", "min_v", "k", "v")]


class WindowProfile(C.Structure):
    _fields_ = [("steps", C.c_int64), ("events", C.c_int64), ("ms", C.c_double * 5)]


#: Names of the decode launches, in the order of WindowProfile.ms.
KERNELS = ("attend_full", "attend_int2", "merge", "route", "transition")

_ready = False


def _lib():
    global _ready
    L = lib()
    if not _ready:
        vp, i32 = C.c_void_p, C.c_int32
        L.rskv_window_build.argtypes = [vp, vp, C.POINTER(WindowOpts), vp, C.POINTER(vp)]
        L.rskv_window_decode.argtypes = [vp, vp, vp, vp]
        L.rskv_window_info_get.argtypes = [vp, C.POINTER(WindowInfo)]
        L.rskv_window_state_get.argtypes = [vp, C.POINTER(WindowState)]
        L.rskv_window_profile_enable.argtypes = [vp, i32]
        L.rskv_window_profile_read.argtypes = [vp, C.POINTER(WindowProfile)]
        L.rskv_window_destroy.argtypes = [vp]
        L.rskv_window_destroy.restype = None
        for fn in ("rskv_window_build", "rskv_window_decode", "rskv_window_info_get",
                   "rskv_window_state_get", "rskv_window_profile_enable",
                   "rskv_window_profile_read"):
            getattr(L, fn).restype = C.c_int
        _ready = True
    return L


class WindowCache:
    """Owner of an rskv_window handle."""

    def __init__(self, handle: C.c_void_p, keep=None):
        self._h = handle
        self._keep = keep  # the allocator hook, alive while the cache is
        _live.add(self)

    @property
    def handle(self):
        if not self._h:
            raise RskvError(-6, "window cache already destroyed")
        return self._h

    @property
    def info(self) -> dict:
        wi = WindowInfo()
        _check(_lib().rskv_window_info_get(self.handle, C.byref(wi)))
        return {n: getattr(wi, n) for n, _ in WindowInfo._fields_}

    @property
    def torch_dtype(self):
        torch = _torch()
        return torch.bfloat16 if self.info["dtype"] == BF16 else torch.float32

    def close(self):
        if self._h:
            _lib().rskv_window_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def decode(self, q, out=None):
        """One decode step: q [B][Hq][d] (cache dtype) -> out [B][Hq][d] fp32."""
        torch = _torch()
        i = self.info
        B, Hq, d = i["batch"], i["n_q_heads"], i["head_dim"]
        qp = _dev(q, "q", (B, Hq, d), self.torch_dtype)
        if out is None:
            out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
        op = _dev(out, "out", (B, Hq, d), torch.float32)
        _check(_lib().rskv_window_decode(self.handle, qp, op, _stream()))
        return out

    def state(self, ledger: bool = True, store: bool = False) -> dict:
        """Host copies of tiers, scores, masses, ledger flags and (optionally)
        the ledger and the full-precision store (row-major)."""
        i = self.info
        U, nW, d = i["batch"] * i["n_kv_heads"], i["n_windows"], i["head_dim"]
        ng = d // GROUP
        out = dict(tier=np.zeros((U, nW), np.int8), score=np.zeros((U, nW)),
                   mass=np.zeros((U, nW)), has_code=np.zeros((U, nW), np.uint8))
        if ledger:
            out.update(code_k=np.zeros((U, nW, ROWS, d), np.uint8),
                       code_v=np.zeros((U, nW, ROWS, d), np.uint8),
                       scale_k=np.zeros((U, nW, ROWS, ng), np.float32),
                       min_k=np.zeros((U, nW, ROWS, ng), np.float32),
                       scale_v=np.zeros((U, nW, ROWS, ng), np.float32),
                       min_v=np.zeros((U, nW, ROWS, ng), np.float32))
        if store:
            dt = np.uint16 if i["dtype"] == BF16 else np.float32
            out.update(k=np.zeros((U, nW * ROWS, d), dt), v=np.zeros((U, nW * ROWS, d), dt))
        s = WindowState(**{k: v.ctypes.data for k, v in out.items()})
        _check(_lib().rskv_window_state_get(self.handle, C.byref(s)))
        return out

    def profile_enable(self, on: bool = True):
        _check(_lib().rskv_window_profile_enable(self.handle, 1 if on else 0))

    def profile_read(self) -> dict:
        p = WindowProfile()
        _check(_lib().rskv_window_profile_read(self.handle, C.byref(p)))
        return dict(steps=p.steps, events=p.events, **{f"{k}_ms": p.ms[j] for j, k in enumerate(KERNELS)})


def build_window(K, V, n_q_heads: int, n_full: int, n_quant: int, route_every: int = 1,
                 allocator="torch") -> WindowCache:
    """Build a window cache.  K, V [B][Hkv][T][d] (fp32 or bf16) on the GPU;
    allocator as in build_spans."""
    B, Hkv, T, d = K.shape
    dt = _dtype_code(K)
    hook, keep = resolve_allocator(allocator)
    opts = WindowOpts(batch=B, n_q_heads=int(n_q_heads), n_kv_heads=Hkv, head_dim=d,
                      context_len=T, dtype=dt, n_full=int(n_full), n_quant=int(n_quant),
                      route_every=int(route_every), allocator=hook)
    h = C.c_void_p()
    _check(_lib().rskv_window_build(_dev(K, "K", (B, Hkv, T, d)), _dev(V, "V", (B, Hkv, T, d), K.dtype),
                                    C.byref(opts), _stream(), C.byref(h)))
    return WindowCache(h, keep)


def window_decode(cache: WindowCache, q, out=None):
    """Module-level form of WindowCache.decode."""
    return cache.decode(q, out=out)


__all__ = ["WindowCache", "build_window", "window_decode", "KERNELS", "ROWS", "GROUP", "FULL",
           "INT2", "EVICTED", "F32", "BF16"]

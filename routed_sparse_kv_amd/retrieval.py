"""ctypes binding of the token-retrieval router (include/rskv_retrieval.h).

Argument marshalling only: every step of the build and of the decode runs
in librskv.so; there is no fallback, a missing library raises.
"""
from __future__ import annotations

import ctypes as C
import numpy as np

from .binding import (BF16, F32, TIERS, Allocator, RskvError, _check, _dev, _dtype_code, _live,
                      _stream, _torch, lib, resolve_allocator)


class RetrievalOpts(C.Structure):
    _fields_ = [("batch", C.c_int32), ("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("context_len", C.c_int32), ("dtype", C.c_int32),
                ("m", C.c_int32), ("rho", C.c_int32), ("cand_frac", C.c_double),
                ("k_ret", C.c_int32), ("n_sink", C.c_int32), ("n_local", C.c_int32),
                ("kv_tier", C.c_int32), ("allocator", Allocator)]


class RetrievalInfo(C.Structure):
    _fields_ = [(n, C.c_int32) for n in
                ("batch", "n_q_heads", "n_kv_heads", "head_dim", "context_len", "dtype", "m",
                 "rho", "k_ret", "n_sink", "local_start", "n_retrieval", "n_cand", "n_sel",
                 "n_attend", "record_bytes", "kv_tier")] + \
               [("cand_frac", C.c_double), ("device_bytes", C.c_size_t),
                ("host_bytes", C.c_size_t)]


class RetrievalHost(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("buckets", "codes", "w", "beta", "lambda_")]


class RetrievalTrace(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in
                ("q_rot", "q_norm", "votes", "scores", "threshold", "cand", "est", "retrieved")]


class RetrievalProfile(C.Structure):
    _fields_ = [("steps", C.c_int64), ("ms", C.c_double * 10)]


#: Names of the ten decode launches, in the order of RetrievalProfile.ms.
KERNELS = ("query", "vote", "compact", "rerank", "histogram", "crossing", "threshold", "output",
           "attend", "merge")

_ready = False


def _lib():
    global _ready
    L = lib()
    if not _ready:
        vp, i32 = C.c_void_p, C.c_int32
        L.rskv_retrieval_build.argtypes = [vp, vp, vp, C.POINTER(RetrievalOpts), vp, C.POINTER(vp)]
        L.rskv_retrieval_decode.argtypes = [vp, vp, vp, vp, vp]
        L.rskv_retrieval_info_get.argtypes = [vp, C.POINTER(RetrievalInfo)]
        L.rskv_retrieval_export.argtypes = [vp, C.POINTER(RetrievalHost)]
        L.rskv_retrieval_trace_get.argtypes = [vp, C.POINTER(RetrievalTrace)]
        L.rskv_retrieval_profile_enable.argtypes = [vp, i32]
        L.rskv_retrieval_profile_read.argtypes = [vp, C.POINTER(RetrievalProfile)]
        L.rskv_retrieval_destroy.argtypes = [vp]
        L.rskv_retrieval_destroy.restype = None
        for fn in ("rskv_retrieval_build", "rskv_retrieval_decode", "rskv_retrieval_info_get",
                   "rskv_retrieval_export", "rskv_retrieval_trace_get",
                   "rskv_retrieval_profile_enable", "rskv_retrieval_profile_read"):
            getattr(L, fn).restype = C.c_int
        _ready = True
    return L


class Retrieval:
    """Owner of an rskv_retrieval handle."""

    def __init__(self, handle: C.c_void_p, keep=None):
        self._h = handle
        self._keep = keep  # the allocator hook, alive while the index is
        _live.add(self)
        ri = RetrievalInfo()
        _check(_lib().rskv_retrieval_info_get(self.handle, C.byref(ri)))
        self.info = {n: getattr(ri, n) for n, _ in RetrievalInfo._fields_}

    @property
    def handle(self):
        if not self._h:
            raise RskvError(-6, "retrieval index already destroyed")
        return self._h

    @property
    def torch_dtype(self):
        torch = _torch()
        return torch.bfloat16 if self.info["dtype"] == BF16 else torch.float32

    @property
    def units(self) -> int:
        return self.info["batch"] * self.info["n_kv_heads"]

    def close(self):
        if self._h:
            _lib().rskv_retrieval_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def decode(self, q, out=None, retrieved=None):
        """One decode step: q [B][Hq][d] (index dtype) -> out [B][Hq][d] fp32;
        ``retrieved`` (int32 [B][Hkv][k_ret]) receives the positions."""
        torch = _torch()
        i = self.info
        B, Hq, Hkv, d = i["batch"], i["n_q_heads"], i["n_kv_heads"], i["head_dim"]
        qp = _dev(q, "q", (B, Hq, d), self.torch_dtype)
        if out is None:
            out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
        op = _dev(out, "out", (B, Hq, d), torch.float32)
        rp = (_dev(retrieved, "retrieved", (B, Hkv, i["k_ret"]), torch.int32)
              if retrieved is not None else None)
        _check(_lib().rskv_retrieval_decode(self.handle, qp, op, rp, _stream()))
        return out

    def export(self) -> dict:
        """Buckets, codes, calibrations and the codebook (host copies)."""
        i = self.info
        U, N, d = self.units, i["n_retrieval"], i["head_dim"]
        out = dict(buckets=np.zeros((U, N, d // 8), np.uint8),
                   codes=np.zeros((U, N, d // 2), np.uint8),
                   w=np.zeros((U, N, d // 8), np.float32),
                   beta=np.zeros(9), lambda_=np.zeros(8))
        h = RetrievalHost(**{k: v.ctypes.data for k, v in out.items()})
        _check(_lib().rskv_retrieval_export(self.handle, C.byref(h)))
        return out

    def trace(self) -> dict:
        """Intermediates of the last decode step (host copies)."""
        i = self.info
        U, N, d, Cn, ns = self.units, i["n_retrieval"], i["head_dim"], i["n_cand"], i["n_sel"]
        out = dict(q_rot=np.zeros((U, d)), q_norm=np.zeros(U),
                   votes=np.zeros((U, d // 8, 256), np.uint8),
                   scores=np.zeros((U, N), np.uint16), threshold=np.zeros((U, 2), np.int32),
                   cand=np.zeros((U, Cn), np.int32), est=np.zeros((U, Cn), np.float32),
                   retrieved=np.zeros((U, ns), np.int32))
        t = RetrievalTrace(**{k: v.ctypes.data for k, v in out.items()})
        _check(_lib().rskv_retrieval_trace_get(self.handle, C.byref(t)))
        return out

    def profile_enable(self, on: bool = True):
        _check(_lib().rskv_retrieval_profile_enable(self.handle, 1 if on else 0))

    def profile_read(self) -> dict:
        p = RetrievalProfile()
        _check(_lib().rskv_retrieval_profile_read(self.handle, C.byref(p)))
        return dict(steps=p.steps, **{f"{k}_ms": p.ms[j] for j, k in enumerate(KERNELS)})


def build_retrieval(K, V, signs, n_q_heads: int, m: int = 8, rho: int = 16,
                    cand_frac: float = 0.05, k_ret: int = 1024, n_sink: int = 16,
                    n_local: int = 512, kv_tier: str = "hbm", allocator="torch") -> Retrieval:
    """Build a retrieval index.  K, V [B][Hkv][T][d] (fp32 or bf16) on the
    GPU; signs: d entries +-1 (host, any integer array); allocator as in
    build_spans."""
    B, Hkv, T, d = K.shape
    dt = _dtype_code(K)
    s = np.ascontiguousarray(np.asarray(signs), dtype=np.int8)
    if s.shape != (d,):
        raise ValueError(f"signs must have shape ({d},)")
    hook, keep = resolve_allocator(allocator)
    opts = RetrievalOpts(batch=B, n_q_heads=int(n_q_heads), n_kv_heads=Hkv, head_dim=d,
                         context_len=T, dtype=dt, m=int(m), rho=int(rho),
                         cand_frac=float(cand_frac), k_ret=int(k_ret), n_sink=int(n_sink),
                         n_local=int(n_local), kv_tier=TIERS[kv_tier], allocator=hook)
    h = C.c_void_p()
    _check(_lib().rskv_retrieval_build(_dev(K, "K", (B, Hkv, T, d)),
                                       _dev(V, "V", (B, Hkv, T, d), K.dtype),
                                       C.c_void_p(s.ctypes.data), C.byref(opts), _stream(),
                                       C.byref(h)))
    return Retrieval(h, keep)


def retrieval_decode(index: Retrieval, q, out=None, retrieved=None):
    """Module-level form of Retrieval.decode."""
    return index.decode(q, out=out, retrieved=retrieved)


__all__ = ["Retrieval", "build_retrieval", "retrieval_decode", "KERNELS", "F32", "BF16"]

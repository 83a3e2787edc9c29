"""Span-routed mixed-resolution KV-cache decode for AMD MI355X (gfx950).

The compute path is the HIP library ``lib/librskv.so`` (C ABI declared in
``include/rskv.h`` for the span router, ``include/rskv_retrieval.h`` for
the token-retrieval router and ``include/rskv_window.h`` for the
window-routed three-tier cache); this package only marshals arguments to
it.
"""
from .binding import (BF16, F32, Cache, RskvError, append_kv, append_token, build_spans,  # noqa: F401
                      cache_import,
                      decode_step, lib, version)
from .retrieval import Retrieval, build_retrieval, retrieval_decode  # noqa: F401
from .window import WindowCache, build_window, window_decode  # noqa: F401

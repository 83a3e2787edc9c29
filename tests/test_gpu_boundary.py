"""The C-ABI boundary's contracts beyond the arithmetic (GPU).

  * Allocator hook: every device block of a cache, its build temporaries
    and its workspace come from the caller's hook; a hook that fails on its
    n-th call makes the build return RSKV_ENOMEM, and every block handed out
    before is returned (for the span cache, an imported cache, the window
    cache and the retrieval index).
  * Graph capture: rskv_decode_step captured once in a HIP graph and
    replayed gives outputs and selections bit-identical to eager calls, on
    both selection paths (fused in the attention kernel, separate top-k
    kernel), with eager decodes and synchronisations between the replays.
  * Destroy waits for the cache's last stream only: work queued on another
    stream is still running when it returns.
"""
import gc
import time

import numpy as np
import pytest
import torch

import routed_sparse_kv_amd as rskv
from gpu_helpers import dev_tensor, gpu_build, say
from routed_sparse_kv_amd import binding
from routed_sparse_kv_amd import workloads as W

pytestmark = pytest.mark.gpu


class CountingHook:
    """torch-backed allocator hook that counts, tracks live blocks and can
    fail on its n-th call."""

    def __init__(self, fail_at=None):
        self.fail_at = fail_at
        self.calls = 0
        self.live = set()
        self.freed = 0
        self.hook = binding.HookAllocator(self._alloc, self._free)

    def _alloc(self, nbytes, stream):
        self.calls += 1
        if self.fail_at is not None and self.calls == self.fail_at:
            return 0
        p = torch.cuda.caching_allocator_alloc(nbytes, stream=stream)
        assert p % 256 == 0
        self.live.add(p)
        return p

    def _free(self, p, stream):
        self.live.remove(p)  # raises (and the test fails) on a foreign pointer
        torch.cuda.caching_allocator_delete(p)
        self.freed += 1


def _span_builder(wl):
    cfg = wl.cfg
    H = torch.from_numpy(wl.H).cuda()
    K, V = dev_tensor(wl.K, wl.dtype), dev_tensor(wl.V, wl.dtype)

    def build(hook):
        return rskv.build_spans(H, K, V, cfg["rank"], cfg["anchor_frac"], n_q_heads=cfg["Hq"],
                                tail_capacity=cfg["tail_capacity"], allocator=hook)
    return build


def _import_builder(wl):
    cache = gpu_build(wl)
    ex = cache.export()
    cache.close()
    cfg = wl.cfg
    arrays = {k: v for k, v in ex.items() if k != "info"}

    def build(hook):
        return rskv.cache_import(arrays, n_q_heads=cfg["Hq"], rank=cfg["rank"], dtype=wl.dtype,
                                 context_len=cfg["T"], allocator=hook)
    return build


def _window_builder(wl):
    K, V = dev_tensor(wl.K, wl.dtype), dev_tensor(wl.V, wl.dtype)

    def build(hook):
        return rskv.build_window(K, V, wl.cfg["Hq"], 4, 8, 2, allocator=hook)
    return build


def _retrieval_builder(wl):
    K, V = dev_tensor(wl.K, wl.dtype), dev_tensor(wl.V, wl.dtype)
    signs = W.srht_signs(wl.cfg)

    def build(hook):
        return rskv.build_retrieval(K, V, signs, wl.cfg["Hq"], k_ret=64, n_sink=8, n_local=64,
                                    allocator=hook)
    return build


BUILDERS = {"spans": _span_builder, "import": _import_builder, "window": _window_builder,
            "retrieval": _retrieval_builder}


@pytest.mark.parametrize("kind", sorted(BUILDERS))
def test_allocator_hook_failure_returns_enomem_and_frees(kind):
    # spans longer than 48 tokens: the build allocates its long-span item list
    wl = W.generate("long_128k_bf16", B=2, Hq=8, Hkv=2, T=8192, steps=1)
    build = BUILDERS[kind](wl)
    # earlier tests' tensors must not be released while the baseline holds
    gc.collect()
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    ok = CountingHook()
    obj = build(ok.hook)
    n = ok.calls
    assert n >= 3 and len(ok.live) > 0
    obj.close()
    assert not ok.live and ok.freed == n, (kind, ok.freed, n)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == base
    say(f"[hook {kind}] {n} allocations through the hook, all returned by destroy")
    for fail_at in sorted({1, 2, n // 2, n - 1, n}):
        h = CountingHook(fail_at)
        with pytest.raises(rskv.RskvError) as ei:
            build(h.hook)
        assert ei.value.code == -3, (kind, fail_at, str(ei.value))
        assert h.calls == fail_at, (kind, fail_at, h.calls)
        assert not h.live and h.freed == fail_at - 1, (kind, fail_at, h.freed)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == base


def _decode_into(cache, q, tau, k_max, out, sel, nsel):
    rskv.decode_step(cache, q, tau, k_max, out=out, sel=sel, n_sel=nsel)


GRAPH_CASES = {
    # a unit's spans fit in LDS: selection fused into the attention kernel
    "fused": ("gqa_32k_bf16", dict(T=4099, steps=4)),
    # more than 4096 spans per unit: the separate top-k kernel
    "topk_kernel": ("million_1m_bf16", dict(Hq=8, Hkv=2, T=262144, steps=4)),
}


@pytest.mark.parametrize("case", sorted(GRAPH_CASES))
def test_decode_step_graph_replay_is_bit_identical(case):
    name, over = GRAPH_CASES[case]
    wl = W.generate(name, **over)
    cfg = wl.cfg
    cache = gpu_build(wl)
    ns = int(cache.export()["n_spans"].max())
    assert (ns > 4096) == (case == "topk_kernel"), ns
    B, Hq, Hkv, d = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["d"]
    tau, k_max = cfg["tau"], cfg["k_max"]
    qs = [dev_tensor(q, wl.dtype) for q in wl.queries]
    q_buf = torch.empty_like(qs[0])
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    sel = torch.empty((B, Hkv, k_max), dtype=torch.int32, device="cuda")
    nsel = torch.empty((B, Hkv), dtype=torch.int32, device="cuda")
    eager = []
    for q in qs:
        q_buf.copy_(q)
        _decode_into(cache, q_buf, tau, k_max, out, sel, nsel)
        torch.cuda.synchronize()
        eager.append((out.clone(), sel.clone(), nsel.clone()))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _decode_into(cache, q_buf, tau, k_max, out, sel, nsel)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _decode_into(cache, q_buf, tau, k_max, out, sel, nsel)
    torch.cuda.synchronize()
    other = torch.empty_like(out)
    for rep in range(3):
        for i, q in enumerate(qs):
            q_buf.copy_(q)
            out.fill_(float("nan"))
            sel.fill_(-7)
            nsel.fill_(-7)
            g.replay()
            torch.cuda.synchronize()
            eo, es, en = eager[i]
            assert torch.equal(out, eo), (case, rep, i)
            assert torch.equal(sel, es) and torch.equal(nsel, en), (case, rep, i)
            # eager work on the same cache between replays
            _decode_into(cache, qs[(i + 1) % len(qs)], tau, k_max, other, None, None)
            torch.cuda.synchronize()
            assert torch.equal(other, eager[(i + 1) % len(qs)][0]), (case, rep, i)
    say(f"[graph {case}] {3 * len(qs)} replays bit-identical to eager decode ({ns} spans)")
    del g
    cache.close()


def test_destroy_waits_only_for_the_cache_stream():
    wl = W.generate("gqa_32k_bf16", T=4099, steps=1)
    cfg = wl.cfg
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    with torch.cuda.stream(s1):
        cache = gpu_build(wl)
        q = dev_tensor(wl.queries[0], wl.dtype)
        rskv.decode_step(cache, q, cfg["tau"], cfg["k_max"])
    s1.synchronize()
    start, done = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(s2):
        start.record(s2)
        torch.cuda._sleep(1_000_000_000)
        done.record(s2)
    t0 = time.perf_counter()
    cache.close()
    t_close = time.perf_counter() - t0
    still_running = not done.query()
    torch.cuda.synchronize()
    busy_ms = start.elapsed_time(done)
    say(f"[destroy] close took {1e3 * t_close:.2f} ms while the other stream ran "
        f"{busy_ms:.1f} ms; still running at return: {still_running}")
    assert still_running and 1e3 * t_close < busy_ms

"""rskv_decode_step_static (decode workspace in the library's static device
array) against rskv_decode_step on the same caches (GPU).

The two entry points run the same kernels on the same inputs, so outputs,
selections and counts must be bit-identical.  Calls come in a row from the
largest workspace to smaller ones, so each later call runs over what the
earlier one left in the shared array: the separate top-k kernel path (more
than 4096 spans per unit), then a smaller cache whose selection is fused
into the attention kernel, then a small fp32 cache (the VALU attention
path), then the first cache again.  A cache whose workspace exceeds the
array is rejected with RSKV_ECAPACITY and still decodes through
rskv_decode_step.
"""
import numpy as np
import pytest
import torch

import routed_sparse_kv_amd as rskv
from gpu_helpers import dev_tensor, gpu_build, say
from routed_sparse_kv_amd import binding
from routed_sparse_kv_amd import workloads as W

pytestmark = pytest.mark.gpu

CASES = [  # largest workspace first
    ("topk_kernel", "million_1m_bf16", dict(Hq=8, Hkv=2, T=262144, steps=2)),
    ("fused", "gqa_32k_bf16", dict(T=4099, steps=2)),
    ("valu_fp32", "tiny_fp32_2k", dict(B=2, Hq=4, Hkv=2, d=128, T=3001, rank=6, k_max=5,
                                       query="uniform", steps=2)),
]


def _both(cache, q, tau, k_max):
    i = cache.info
    B, Hq, Hkv, d = i["batch"], i["n_q_heads"], i["n_kv_heads"], i["head_dim"]
    res = []
    for fn in (rskv.decode_step, binding.decode_step_static):
        out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
        sel = torch.full((B, Hkv, k_max), -7, dtype=torch.int32, device="cuda")
        nsel = torch.full((B, Hkv), -7, dtype=torch.int32, device="cuda")
        fn(cache, q, tau, k_max, out=out, sel=sel, n_sel=nsel)
        torch.cuda.synchronize()
        res.append((out, sel, nsel))
    return res


def test_static_workspace_decode_matches_decode_step():
    cap = binding.decode_static_capacity()
    assert cap == 32 << 20
    built = []
    for name, wname, over in CASES:
        wl = W.generate(wname, **over)
        cache = gpu_build(wl)
        built.append((name, wl, cache))
    sizes = []
    for name, wl, cache in built + built[:1]:
        cfg = wl.cfg
        for s, qn in enumerate(wl.queries):
            say(f"[static {name}] step {s}")
            q = dev_tensor(qn, wl.dtype)
            (o1, s1, n1), (o2, s2, n2) = _both(cache, q, cfg["tau"], cfg["k_max"])
            assert not torch.isnan(o1).any()
            assert torch.equal(o1, o2), f"{name} step {s}: outputs differ"
            assert torch.equal(s1, s2) and torch.equal(n1, n2), f"{name} step {s}: selections"
        sizes.append(name)
    say(f"[static] bit-identical to rskv_decode_step in the order {sizes}")
    for _, _, cache in built:
        cache.close()


def test_static_workspace_rejects_a_cache_above_the_capacity():
    # about 1e5 one- and two-token spans per unit, 8 units of 8 query heads:
    # z, summary logits and span descriptors alone need about 48 MB
    B, Hkv, G, T, d = 1, 8, 8, 400_000, 128
    gen = torch.Generator(device="cuda").manual_seed(7)
    H = torch.rand((B, T), generator=gen, device="cuda")
    K = torch.randn((B, Hkv, T, d), generator=gen, device="cuda").to(torch.bfloat16)
    V = torch.randn((B, Hkv, T, d), generator=gen, device="cuda").to(torch.bfloat16)
    cache = rskv.build_spans(H, K, V, 8, 0.5, n_q_heads=Hkv * G)
    del K, V
    q = torch.randn((B, Hkv * G, d), generator=gen, device="cuda").to(torch.bfloat16)
    out = torch.empty((B, Hkv * G, d), dtype=torch.float32, device="cuda")
    with pytest.raises(rskv.RskvError) as ei:
        binding.decode_step_static(cache, q, 0.0, 64, out=out)
    assert ei.value.code == -4 and "static scratch" in str(ei.value)
    rskv.decode_step(cache, q, 0.0, 64, out=out)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    say(f"[static] rejected: {ei.value}")
    cache.close()

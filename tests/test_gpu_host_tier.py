"""Host-resident factor tier (GPU).

With factor_tier="host" the span factors live in pinned host memory and the
kernels read the expanded spans' factors over the host link.  Nothing else
changes, so a host-tier cache must hold exactly the arrays of an HBM-tier
cache built from the same inputs, and decode (with appends whose decoded
anchors close spans, i.e. factors written to host memory) must give
bit-identical outputs and selections.  One step is also checked against the
oracle on the host-tier export, and the full 128K workload is decoded in
both tiers.
"""
import numpy as np
import pytest

from gpu_helpers import compare_decode, decode_gpu, dev_tensor, gpu_build, oracle_view, say
from routed_sparse_kv_amd import workloads as W

pytestmark = pytest.mark.gpu

CASES = {
    "serving_bf16": ("serving_b16_bf16", dict(B=3, T=2053, steps=12, tail_capacity=12)),
    "tiny_fp32": ("tiny_fp32_2k", dict(B=2, Hq=4, Hkv=2, T=1500, steps=6, tail_capacity=6,
                                       append=True, query="uniform")),
}


def _same_exports(ea, eb, what):
    for k in ea:
        if k == "info":
            continue
        assert np.array_equal(ea[k], eb[k]), f"{what}: array {k} differs between tiers"


@pytest.mark.parametrize("case", sorted(CASES))
def test_host_tier_matches_hbm_tier(case):
    import torch

    import routed_sparse_kv_amd as rskv
    name, over = CASES[case]
    wl = W.generate(name, **over)
    cfg, dt = wl.cfg, wl.dtype
    say(f"[host tier {case}] build both tiers")
    ch = gpu_build(wl)
    cx = gpu_build(wl, factor_tier="host")
    ih, ix = ch.info, cx.info
    assert ih["factor_tier"] == 0 and ix["factor_tier"] == 1
    assert ih["host_bytes"] == 0 and ix["host_bytes"] > 0
    assert ix["device_bytes"] < ih["device_bytes"]
    say(f"[host tier {case}] HBM {ih['device_bytes'] / 1e6:.2f} MB -> "
        f"{ix['device_bytes'] / 1e6:.2f} MB + host {ix['host_bytes'] / 1e6:.2f} MB")
    e0 = ch.export()
    _same_exports(e0, cx.export(), f"{case} build")
    # anchors every third append so that spans close into host memory
    theta = e0["theta"]
    for s in range(cfg["steps"]):
        k, v = wl.appends[s]
        h = np.where(s % 3 == 2, 2 * theta + 1, theta / 2).astype(np.float32)
        for c in (ch, cx):
            rskv.append_token(c, dev_tensor(k, dt), dev_tensor(v, dt), torch.from_numpy(h).cuda())
        q = wl.queries[s]
        oh, sh = decode_gpu(ch, q, cfg["tau"], cfg["k_max"])
        ox, sx = decode_gpu(cx, q, cfg["tau"], cfg["k_max"])
        assert np.array_equal(oh, ox), f"{case} step {s}: outputs differ between tiers"
        for b in range(cfg["B"]):
            for hh in range(cfg["Hkv"]):
                assert np.array_equal(sh[b][hh], sx[b][hh]), f"{case} step {s}: selections differ"
    ex = cx.export()
    _same_exports(ch.export(), ex, f"{case} after appends")
    assert (ex["n_spans"] > e0["n_spans"]).all(), "decoded anchors closed no span"
    q = wl.queries[-1]
    out, sels = decode_gpu(cx, q, cfg["tau"], cfg["k_max"])
    err, _ = compare_decode(oracle_view(ex), q, out, sels, cfg["tau"], cfg["k_max"], cfg["alpha"],
                            wl.P, dt, what=f"{case} host tier")
    say(f"[host tier {case}] oracle max abs err {err:.2e}")
    ch.close()
    cx.close()


@pytest.mark.timeout(900)
def test_host_tier_full_size():
    """128K context, 4 sequences, 8 KV heads: both tiers decode the same."""
    name = "long_128k_bf16"
    say(f"[host tier full] generate {name}")
    wl = W.generate(name, steps=2)
    cfg = wl.cfg
    ch = gpu_build(wl)
    cx = gpu_build(wl, factor_tier="host")
    say(f"[host tier full] HBM {ch.info['device_bytes'] / 1e9:.2f} GB -> "
        f"{cx.info['device_bytes'] / 1e9:.2f} GB + host {cx.info['host_bytes'] / 1e9:.2f} GB")
    for s, q in enumerate(wl.queries):
        oh, sh = decode_gpu(ch, q, cfg["tau"], cfg["k_max"])
        ox, sx = decode_gpu(cx, q, cfg["tau"], cfg["k_max"])
        assert np.array_equal(oh, ox), f"step {s}: outputs differ between tiers"
        assert all(np.array_equal(a, b) for ra, rb in zip(sh, sx) for a, b in zip(ra, rb))
    ch.close()
    cx.close()

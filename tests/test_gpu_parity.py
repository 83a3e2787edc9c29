"""HIP path against the fp64 oracle on the same seeded inputs (GPU).

Integer outputs (span ids, span tables, full-resolution positions,
selections) are compared bit-exactly; selections may differ only for spans
whose z lies within 1e-5 of tau (or of the k-th largest z), and those are
counted.  Stored floating values are compared within one storage ulp,
factors through their products (the SVD basis is unique only up to sign),
outputs within 1e-5 (fp32 caches) and 1e-2 (bf16 caches) max-abs, on the
same exported cache with the GPU's selection forced where the band excuses
a difference.
"""
import numpy as np
import pytest

import oracle
from gpu_helpers import (check_factor_products, check_full_rows, check_segmentation_tables,
                         check_summaries,
                         check_selection, compare_decode, decode_gpu, dev_tensor, gpu_build,
                         oracle_view, say)
from routed_sparse_kv_amd import workloads as W

pytestmark = pytest.mark.gpu

# Small variants of the five workloads: several tiles, ragged tails.
SMALL = {
    "tiny_fp32": ("tiny_fp32_2k", {}),
    "tiny_fp32_gqa_d128": ("tiny_fp32_2k", dict(B=2, Hq=4, Hkv=2, d=128, T=3001, rank=6,
                                                k_max=5, query="uniform")),
    "gqa_bf16": ("gqa_32k_bf16", dict(T=4099, steps=3)),
    "long_bf16": ("long_128k_bf16", dict(B=2, Hq=8, Hkv=2, T=8192, k_max=24, steps=2)),
    "serving_bf16": ("serving_b16_bf16", dict(B=3, T=2053, steps=4, tail_capacity=6)),
    "drift_bf16": ("million_1m_bf16", dict(Hq=8, Hkv=2, T=16384, steps=2)),
    # query groups of 16 heads (the MFMA tiles' full width; G d = 2048 outputs
    # per workgroup on the fp32 path)
    "tiny_fp32_g16": ("tiny_fp32_2k", dict(Hq=16, Hkv=1, d=128, T=2051, query="uniform")),
    "gqa_bf16_g16": ("gqa_32k_bf16", dict(Hq=32, Hkv=2, T=4099, steps=2)),
}


@pytest.fixture(scope="module", params=sorted(SMALL))
def built(request):
    name, over = SMALL[request.param]
    say(f"[case {request.param}] generate {name} {over}")
    wl = W.generate(name, **over)
    say(f"[case {request.param}] build_spans on GPU")
    cache = gpu_build(wl)
    yield request.param, wl, cache
    cache.close()


def _input_f64(wl):
    return W.as_f64(wl.K, wl.dtype), W.as_f64(wl.V, wl.dtype)


def test_segmentation_exact(built):
    case, wl, cache = built
    if wl.appends is not None and cache.info["appended"] > 0:
        pytest.skip("tables already changed by appends")
    check_segmentation_tables(cache.export(), wl.H, wl.cfg["anchor_frac"], case)


def test_full_rows_exact(built):
    case, wl, cache = built
    if wl.appends is not None and cache.info["appended"] > 0:
        pytest.skip("rows already changed by appends")
    ex = cache.export()
    for b in range(wl.cfg["B"]):
        for h in range(wl.cfg["Hkv"]):
            check_full_rows(ex, wl.K, wl.V, b, h, case)


def test_summaries_within_one_ulp(built):
    case, wl, cache = built
    ex = cache.export()
    Kf, Vf = _input_f64(wl)
    rng = np.random.default_rng(0)
    for b in range(wl.cfg["B"]):
        ns = int(ex["n_spans"][b])
        if ns == 0:
            continue
        js = np.sort(rng.choice(ns, size=min(ns, 40), replace=False))
        for h in range(wl.cfg["Hkv"]):
            check_summaries(ex, wl.H, Kf[b, h], Vf[b, h], b, h, js, wl.dtype, case)


def test_factor_products(built):
    """A W rebuilds the best rank-r_j approximation (Eckart-Young residual)
    and matches the oracle's factors' product."""
    case, wl, cache = built
    ex = cache.export()
    Kf, Vf = _input_f64(wl)
    rng = np.random.default_rng(1)
    for b in range(wl.cfg["B"]):
        ns = int(ex["n_spans"][b])
        if ns == 0:
            continue
        for h in range(wl.cfg["Hkv"]):
            js = rng.choice(ns, size=min(ns, 12), replace=False)
            check_factor_products(ex, Kf[b, h], Vf[b, h], b, h, js, wl.dtype, wl.cfg["rank"], case)


def test_decode_parity_on_same_cache(built):
    case, wl, cache = built
    cfg = wl.cfg
    dt = wl.dtype
    P = wl.P
    worst, excused = 0.0, 0
    for s, q in enumerate(wl.queries):
        if wl.appends is not None:
            import routed_sparse_kv_amd as rskv
            k, v = wl.appends[s]
            if cache.info["appended"] < cfg["tail_capacity"]:
                rskv.append_kv(cache, dev_tensor(k, dt), dev_tensor(v, dt))
        say(f"[case {case}] decode step {s}")
        out, sels = decode_gpu(cache, q, cfg["tau"], cfg["k_max"])
        oc = oracle_view(cache.export())
        err, ex_ = compare_decode(oc, q, out, sels, cfg["tau"], cfg["k_max"], cfg["alpha"], P, dt,
                                  what=f"{case} step {s}")
        worst = max(worst, err)
        excused += ex_
    say(f"[case {case}] max abs err {worst:.3e}, excused selections {excused}")


def test_appended_rows(built):
    case, wl, cache = built
    if wl.appends is None:
        pytest.skip("no appends in this workload")
    ex = cache.export()
    a = ex["info"]["appended"]
    assert a >= 1
    n_a = oracle.n_anchors(wl.cfg["T"], wl.cfg["anchor_frac"])
    for b in range(wl.cfg["B"]):
        nf0 = len(oracle.segment(wl.H[b], n_a)["fr_pos"])
        assert ex["n_full"][b] == nf0 + a
        assert ex["full_pos"][b, nf0:nf0 + a].tolist() == [wl.cfg["T"] + i for i in range(a)]
        for i in range(a):
            k, v = wl.appends[i]
            assert np.array_equal(ex["k_full"][b, :, nf0 + i], k[b])
            assert np.array_equal(ex["v_full"][b, :, nf0 + i], v[b])


def test_tiny_end_to_end():
    """fp32 workload gated end to end: GPU build + decode against the
    oracle's own build + decode from the same inputs."""
    wl = W.generate("tiny_fp32_2k")
    cfg = wl.cfg
    cache = gpu_build(wl)
    Kf, Vf = _input_f64(wl)
    oc = oracle.build_cache(wl.H, Kf, Vf, cfg["rank"], cfg["anchor_frac"], "f32", Hq=cfg["Hq"])
    q = wl.queries[0]
    out, sels = decode_gpu(cache, q, cfg["tau"], cfg["k_max"])
    res = oracle.decode_step(oc, oracle.from_stored(q, "f32"), cfg["tau"], cfg["k_max"], cfg["alpha"])
    rt = res["routes"][(0, 0)]
    assert check_selection(rt, sels[0][0], cfg["tau"], cfg["k_max"]) == 0
    assert len(sels[0][0]) == cfg["k_max"]
    err = float(np.max(np.abs(out - res["out"])))
    say(f"tiny end-to-end: selection {sels[0][0].tolist()} err {err:.2e}")
    assert err <= 1e-5
    cache.close()

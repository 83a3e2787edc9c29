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
import math

import numpy as np
import pytest

import oracle
from gpu_helpers import (TOL, check_selection, compare_decode, decode_gpu, dev_tensor, gpu_build,
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
    ex = cache.export()
    n_a = oracle.n_anchors(wl.cfg["T"], wl.cfg["anchor_frac"])
    for b in range(wl.cfg["B"]):
        sg = oracle.segment(wl.H[b], n_a)
        ns = len(sg["span_len"])
        assert ex["n_anchor"][b] == sg["n_a"]
        assert ex["n_spans"][b] == ns
        assert np.array_equal(ex["span_id"][b], sg["span_id"]), case
        assert np.array_equal(ex["span_start"][b, :ns], sg["span_start"])
        assert np.array_equal(ex["span_len"][b, :ns], sg["span_len"])
        nf = len(sg["fr_pos"])
        assert ex["n_full"][b] == nf
        assert np.array_equal(ex["full_pos"][b, :nf], sg["fr_pos"])
        assert ex["n_span_tokens"][b] == sg["span_len"].sum()


def _ulps(a, b, dtype):
    """Distance in units of the last stored place of b."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    mant = 8 if dtype == "bf16" else 24
    _, e = np.frexp(np.where(b == 0, 1.0, np.abs(b)))
    ulp = np.ldexp(1.0, e - mant)
    return np.abs(a - b) / ulp


def test_summaries_within_one_ulp(built):
    case, wl, cache = built
    dt = wl.dtype
    ex = cache.export()
    oc = oracle_view(ex)
    Kf, Vf = _input_f64(wl)
    rng = np.random.default_rng(0)
    worst = 0.0
    for b in range(wl.cfg["B"]):
        ns = int(oc["n_s"][b])
        if ns == 0:
            continue
        js = rng.choice(ns, size=min(ns, 40), replace=False)
        ell_ref = np.log(oc["span_len"][b, js].astype(np.float64)).astype(np.float32)
        assert np.array_equal(ex["log_len"][b, js], ell_ref)
        for h in range(wl.cfg["Hkv"]):
            for j in js:
                st, ln = int(oc["span_start"][b, j]), int(oc["span_len"][b, j])
                s_ref = oracle.round_stored(oracle.span_summary(wl.H[b, st:st + ln], Kf[b, h, st:st + ln]), dt)
                v_ref = oracle.round_stored(oracle.span_value_mean(Vf[b, h, st:st + ln]), dt)
                worst = max(worst, _ulps(oc["s"][b, h, j], s_ref, dt).max(),
                            _ulps(oc["vbar"][b, h, j], v_ref, dt).max())
    assert worst <= 1.0, f"{case}: summaries differ by {worst} ulp"


def test_factor_products(built):
    """A W rebuilds the best rank-r_j approximation (Eckart-Young residual)
    and matches the oracle's factors' product."""
    case, wl, cache = built
    dt = wl.dtype
    ex = cache.export()
    oc = oracle_view(ex)
    Kf, Vf = _input_f64(wl)
    r = wl.cfg["rank"]
    rng = np.random.default_rng(1)
    # storage rounding of A and W bounds the product error
    rel = 2e-6 if dt == "f32" else 3 * 2.0 ** -8
    for b in range(wl.cfg["B"]):
        ns = int(oc["n_s"][b])
        offs = np.concatenate([[0], np.cumsum(oc["span_len"][b, :ns])])
        for h in range(wl.cfg["Hkv"]):
            for j in rng.choice(ns, size=min(ns, 12), replace=False):
                st, ln = int(oc["span_start"][b, j]), int(oc["span_len"][b, j])
                for X, Akey, Wkey in ((Kf[b, h, st:st + ln], "AK", "BK"),
                                      (Vf[b, h, st:st + ln], "AV", "BV")):
                    A = oc[Akey][b, h, offs[j]:offs[j + 1]]
                    Wt = oc[Wkey][b, h, j]
                    P_gpu = A @ Wt
                    Ao, Wo = oracle.truncated_svd(X, r)
                    P_ref = Ao @ Wo
                    nx = np.linalg.norm(X)
                    err = np.linalg.norm(P_gpu - P_ref) / nx
                    sig = np.linalg.svd(X, compute_uv=False)
                    rj = min(r, ln, X.shape[1])
                    gap = (sig[rj - 1] - sig[rj]) / sig[0] if rj < len(sig) else 1.0
                    if gap < 1e-6:
                        continue  # truncation not unique
                    assert err <= rel * math.sqrt(r), f"{case} span {j}: product err {err:.2e}"
                    res = np.linalg.norm(X - P_gpu) ** 2
                    assert res <= np.sum(sig[rj:] ** 2) + (2 * rel * nx) ** 2 + 1e-9 * nx ** 2


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

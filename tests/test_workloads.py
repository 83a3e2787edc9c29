"""Self-checks of the seeded input generators (CPU only)."""
import numpy as np
import pytest

import oracle
from routed_sparse_kv_amd import workloads as W


def test_tiny_shapes_and_anchor_count():
    wl = W.generate("tiny_fp32_2k")
    assert wl.H.shape == (1, 2048) and wl.K.shape == (1, 1, 2048, 64)
    assert wl.K.dtype == np.float32
    assert len(wl.anchor_pos[0]) == 102
    # the generator's anchors are exactly the oracle's top-n_a surprisal set
    mask = oracle.select_anchors(wl.H[0], 102)
    assert np.flatnonzero(mask).tolist() == wl.anchor_pos[0].tolist()
    q = wl.queries[0]
    assert abs(np.linalg.norm(q[0, 0]) - 1.0) < 1e-6


def test_deterministic_and_worker_independent():
    a = W.generate("long_128k_bf16", B=2, T=4096, Hkv=2, Hq=8, workers=1)
    b = W.generate("long_128k_bf16", B=2, T=4096, Hkv=2, Hq=8, workers=3)
    assert np.array_equal(a.K, b.K) and np.array_equal(a.V, b.V)
    assert np.array_equal(a.H, b.H)
    assert all(np.array_equal(x, y) for x, y in zip(a.queries, b.queries))


def test_clustered_gap_bounds_and_needles():
    wl = W.generate("long_128k_bf16", B=1, T=16384, Hkv=1, Hq=4)
    apos = wl.anchor_pos[0]
    n_a = W.n_anchors(16384, 0.03)
    assert len(apos) == n_a
    gaps = np.diff(np.concatenate([[-1], apos, [16384]])) - 1
    assert gaps.min() >= 8 and gaps.max() <= 256
    assert gaps.sum() == 16384 - n_a
    assert len(wl.needles[0]) == 5 and len(set(wl.needles[0].tolist())) == 5
    assert np.array_equal(np.flatnonzero(oracle.select_anchors(wl.H[0], n_a)), apos)


def test_bf16_storage_roundtrip():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 0.0], np.float32)
    b = W.f32_to_bf16_bits(x)
    assert W.bf16_bits_to_f32(b).tolist() == [1.0, 1.0, 1.0 + 2 ** -6, -2.5, 0.0]


@pytest.mark.parametrize("name", ["gqa_32k_bf16", "serving_b16_bf16", "million_1m_bf16"])
def test_small_variants(name):
    wl = W.generate(name, B=2, T=4096)
    cfg = wl.cfg
    assert wl.K.shape == (2, cfg["Hkv"], 4096, cfg["d"]) and wl.K.dtype == np.uint16
    assert len(wl.queries) == cfg["steps"]
    if cfg.get("append"):
        assert len(wl.appends) == cfg["steps"]
    if cfg["P"] == "gauss":
        assert wl.P.shape == (1, cfg["d"], cfg["d"])


def test_window_budget_counts():
    """The window tiers fill the byte budget: n_full is the full share of
    the budget in whole windows; n_quant INT2 windows (codes, and an fp32
    scale and minimum per row and 64-column group, for K and V) fit in the
    rest; one more INT2 window would exceed it."""
    from routed_sparse_kv_amd import workloads as W
    for T, d, dt, budget, share in ((131072, 128, "bf16", 0.2, 0.5), (32768, 128, "bf16", 0.05, 0.5),
                                    (2065, 64, "f32", 0.2, 0.5), (5000, 64, "bf16", 0.1, 0.25)):
        nw = -(-T // 64)
        full_b = 2 * 64 * d * (2 if dt == "bf16" else 4)
        quant_b = 2 * 64 * d // 4 + 2 * 64 * (d // 64) * 8
        nf, nq = W.window_tiers(T, d, dt, budget, share)
        assert nf == int(share * budget * nw)
        total = budget * nw * full_b
        assert nf * full_b + nq * quant_b <= total + 1e-9
        assert nf * full_b + (nq + 1) * quant_b > total
    assert W.window_tiers(100, 128, "bf16", 0.0, 0.5) == (1, 0)
    assert W.window_tiers(131072, 128, "bf16", 0.2, 0.5) == (204, 1096)

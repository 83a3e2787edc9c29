"""Capacity bound that the library's cache sizing relies on (CPU).

With a tail capacity t, streaming segmentation adds at most ceil(t/2) spans
to a sequence (a closing needs a decoded anchor, and two closings need a
decoded non-anchor between them), holding at most the prefill tail run plus
the t decoded tokens.  Checked on the oracle over random anchor patterns,
including the worst case (anchor, non-anchor, anchor, ...).
"""
import numpy as np
import pytest

import oracle


def _cache(rng, T=40, n_a=6, d=8, t=9):
    H = rng.random((1, T)).astype(np.float32)
    K = rng.standard_normal((1, 1, T, d))
    V = rng.standard_normal((1, 1, T, d))
    return oracle.build_cache(H, K, V, 3, 0.0, "f64", tail_capacity=t, n_anchor=n_a)


@pytest.mark.parametrize("seed", range(12))
def test_closings_within_capacity(seed):
    rng = np.random.default_rng(seed)
    t = int(rng.integers(1, 12))
    c = _cache(rng, t=t)
    ns0, nt0 = int(c["n_s"][0]), int(c["nt"][0])
    trail = int(c["n_F"][0] - c["la"][0] - 1)
    theta = float(c["theta"][0])
    if seed < 3:
        pattern = [i % 2 == 0 for i in range(t)]  # anchor, non-anchor, anchor, ...
    else:
        pattern = list(rng.random(t) < rng.random())
    for is_anchor in pattern:
        h = np.array([theta + 1.0 if is_anchor else theta], np.float32)
        oracle.append_kv(c, rng.standard_normal((1, 1, 8)), rng.standard_normal((1, 1, 8)), h)
    assert c["n_s"][0] - ns0 <= (t + 1) // 2
    assert c["nt"][0] - nt0 <= trail + t
    if seed < 3 and trail > 0:
        assert c["n_s"][0] - ns0 == (t + 1) // 2  # the bound is reached

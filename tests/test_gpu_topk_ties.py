"""Top-k cap on tied and tightly clustered routing scores (GPU).

Crafted bf16 caches are imported through rskv_cache_import so that the
routing scores z = alpha <qbar, s> take chosen values: the query is
(1, 2^-8, 0, ...) and span j's summary (s0_j, s1_j, 0, ...), so
z_j = 8 (s0_j + s1_j / 256) is exact in fp64 on both sides and every
selection must equal the oracle's exactly (no ambiguity band is needed).

  * tied block: 600 spans share one score and k_max ends inside the block,
    so the k-th largest value is tied and the lower span indices win;
  * dense cluster: 512 distinct scores packed into a window under 1/4000 of
    the score range, so the bin of a 1024-bin histogram over the range that
    holds the k-th largest value holds more than 256 values and the search
    must narrow the range again.

Each runs with 1000 spans (selection fused into the attention kernel) and
with 5000 spans (the separate top-k kernel).  Outputs are compared with the
oracle's decode on the same stored cache as well.
"""
import math

import numpy as np
import pytest

import oracle
import routed_sparse_kv_amd as rskv
from gpu_helpers import check_selection, compare_decode, decode_gpu, oracle_view, say
from routed_sparse_kv_amd import workloads as W

pytestmark = pytest.mark.gpu

D, RANK, G = 128, 16, 4


def _bf16(x):
    return W.f32_to_bf16_bits(np.asarray(x, np.float32))


def _crafted(s0, s1, seed):
    """One-unit bf16 cache with spans of 1-3 tokens whose summaries are
    (s0_j, s1_j, 0, ...); everything else random."""
    rng = np.random.default_rng(seed)
    S = len(s0)
    F = 96
    lens = rng.integers(1, 4, S)
    N = int(lens.sum())
    T = F + N
    summ = np.zeros((1, 1, S, D), np.float32)
    summ[0, 0, :, 0] = s0
    summ[0, 0, :, 1] = s1
    assert np.array_equal(W.bf16_bits_to_f32(_bf16(summ)), summ), "scores must be bf16-exact"
    arr = dict(
        n_anchor=np.array([F], np.int32), n_spans=np.array([S], np.int32),
        n_full=np.array([F], np.int32), n_span_tokens=np.array([N], np.int32),
        span_start=(F + np.concatenate([[0], np.cumsum(lens)[:-1]]))[None].astype(np.int32),
        span_len=lens[None].astype(np.int32), full_pos=np.arange(F, dtype=np.int32)[None],
        summary=_bf16(summ), vmean=_bf16(rng.standard_normal((1, 1, S, D))),
        log_len=np.log(lens.astype(np.float64)).astype(np.float32)[None],
        k_full=_bf16(rng.standard_normal((1, 1, F, D))),
        v_full=_bf16(rng.standard_normal((1, 1, F, D))),
        a_k=_bf16(rng.standard_normal((1, 1, N, RANK)) * 0.3),
        a_v=_bf16(rng.standard_normal((1, 1, N, RANK)) * 0.3),
        w_k=_bf16(rng.standard_normal((1, 1, S, RANK, D)) * 0.1),
        w_v=_bf16(rng.standard_normal((1, 1, S, RANK, D)) * 0.1))
    cache = rskv.cache_import(arr, n_q_heads=G, rank=RANK, dtype="bf16", context_len=T)
    q = np.zeros((1, G, D), np.float32)
    q[0, :, 0] = 1.0
    q[0, :, 1] = 2.0 ** -8
    return cache, _bf16(q)


def _scores_tied(S, rng):
    """100 spans above, 600 tied at z = 8, the rest below (some negative)."""
    idx = rng.permutation(S)
    s0 = np.zeros(S, np.float32)
    s1 = np.zeros(S, np.float32)
    above, tied = idx[:100], idx[100:700]
    s0[above] = rng.integers(3, 200, len(above))          # z in [24, 1600)
    s0[tied] = 1.0                                         # z = 8 exactly
    rest = idx[700:]
    s0[rest] = rng.integers(-200, 1, len(rest)) / 4.0       # z in (-400, 0]
    return s0, s1, 100 + 250, 0.0


def _scores_cluster(S, rng):
    """Scores over [-2048, 2048]; 512 distinct ones packed in [1.03, 2)
    (s1 from 4 binades of bf16 values); 100 above the cluster."""
    idx = rng.permutation(S)
    s0 = np.zeros(S, np.float32)
    s1 = np.zeros(S, np.float32)
    ends, above, clus = idx[:2], idx[2:102], idx[102:614]
    s0[ends] = [256.0, -256.0]                             # z = +-2048: the range
    s0[above] = rng.integers(1, 250, len(above))           # z in [8, 2000)
    c = np.concatenate([(1.0 + np.arange(128) / 128.0) * 2.0 ** e for e in range(4)])
    s0[clus] = 0.125                                       # z = 1 + s1 / 32
    s1[clus] = rng.permutation(c)
    rest = idx[614:]
    s0[rest] = -rng.integers(1, 250, len(rest)).astype(np.float32)
    return s0, s1, 100 + 200, -math.inf


@pytest.mark.parametrize("S", [1000, 5000])
@pytest.mark.parametrize("kind", ["tied", "cluster"])
def test_topk_ties_and_clusters(kind, S):
    rng = np.random.default_rng(S + (0 if kind == "tied" else 1))
    s0, s1, k_max, tau = (_scores_tied if kind == "tied" else _scores_cluster)(S, rng)
    say(f"[topk {kind} S={S}] k_max={k_max} tau={tau}")
    cache, q = _crafted(s0, s1, seed=S)
    out, sels = decode_gpu(cache, q, tau, k_max)
    oc = oracle_view(cache.export())
    rt = oracle.route_unit(oc["s"][0, 0, :S], oracle.from_stored(q, "bf16")[0], tau, k_max, 8.0)
    z = rt["z"]
    if kind == "tied":
        assert np.sum(z == 8.0) == 600 and rt["rank_tie"]
    else:
        inside = (z > 1.0) & (z < 2.0)
        assert inside.sum() == 512 and len(np.unique(z[inside])) == 512
    assert check_selection(rt, sels[0][0], tau, k_max, f"{kind} S={S}") == 0
    assert np.array_equal(sels[0][0], rt["E"])
    err, _ = compare_decode(oc, q, out, sels, tau, k_max, 8.0, None, "bf16",
                            what=f"{kind} S={S}")
    say(f"[topk {kind} S={S}] selection exact ({len(rt['E'])} spans), max abs err {err:.2e}")
    cache.close()

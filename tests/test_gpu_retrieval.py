"""Token-retrieval router on the GPU against the oracle (GPU).

Each case builds the index on the GPU from a seeded workload and compares,
unit by unit, with oracle.paris run on the same stored K/V:
  * the export: buckets bit-exact (the rotation's signs are exact on both
    sides); codes exact except a coordinate within 1e-12 of a magnitude-bin
    boundary; calibrations w within one fp32 ulp; the codebook within 1e-12;
  * the trace of each decode step: rotated query, vote table, vote totals,
    threshold and candidates exact; estimates within one fp32 ulp of the
    oracle's fp32 decision values; the retrieved set exact except
    candidates whose decision value sits within one fp32 ulp of the k-th
    (reported), and the -1 padding of the caller's buffer;
  * the output: within 1e-5 (fp32) / 1e-2 (bf16) max-abs of the oracle's
    attention over Sink, the GPU's retrieved set (validated above) and
    Local.
Sizes span several 4096-key chunks with a ragged last one; the edge cases
cover an empty retrieval region, k_ret = 0, cand_frac = 0, retrieval of
every candidate, dense retrieval (everything), no Sink/Local, zero keys and a
zero query (every stage's tie rule).
"""
import numpy as np
import pytest

from gpu_helpers import TOL, dev_tensor, say
from oracle import paris as P
from routed_sparse_kv_amd import workloads as W

pytestmark = pytest.mark.gpu

CODE_BAND = 1e-12
VOTE_BAND = 1e-12

# case -> (workload, overrides, retrieval parameters, decode steps)
CASES = {
    "bf16_g4_d128": ("gqa_32k_bf16", dict(B=2, T=9001, steps=3),
                     dict(rho=16, cand_frac=0.05, k_ret=64, n_sink=16, n_local=128)),
    "f32_g3_d64": ("tiny_fp32_2k", dict(Hq=3, T=5000, steps=2),
                   dict(rho=8, cand_frac=0.1, k_ret=100, n_sink=4, n_local=60)),
    "bf16_g7_serving": ("serving_b16_bf16", dict(B=2, T=4500, steps=2),
                        dict(rho=4, cand_frac=0.08, k_ret=50, n_sink=8, n_local=64)),
    "bf16_clustered": ("long_128k_bf16", dict(B=1, T=12000, steps=2),
                       dict(rho=16, cand_frac=0.05, k_ret=128, n_sink=16, n_local=256)),
    "bf16_drift": ("million_1m_bf16", dict(T=20000, Hkv=2, Hq=8, steps=2),
                   dict(rho=16, cand_frac=0.07, k_ret=256, n_sink=16, n_local=512)),
    # edge cases
    "all_candidates": ("tiny_fp32_2k", dict(T=3000, steps=1),
                       dict(rho=16, cand_frac=0.02, k_ret=500, n_sink=2, n_local=10)),
    "dense": ("tiny_fp32_2k", dict(Hq=2, Hkv=1, T=700, steps=1),
              dict(rho=2, cand_frac=1.0, k_ret=700, n_sink=3, n_local=5)),
    "no_retrieval_region": ("tiny_fp32_2k", dict(T=300, steps=1),
                            dict(rho=8, cand_frac=0.5, k_ret=10, n_sink=200, n_local=200)),
    "k_ret_zero": ("gqa_32k_bf16", dict(T=5000, Hkv=2, Hq=4, steps=1),
                   dict(rho=16, cand_frac=0.05, k_ret=0, n_sink=16, n_local=64)),
    "cand_frac_zero": ("tiny_fp32_2k", dict(T=1000, steps=1),
                       dict(rho=16, cand_frac=0.0, k_ret=20, n_sink=4, n_local=4)),
    "no_sink_local": ("gqa_32k_bf16", dict(T=6000, Hkv=1, Hq=4, steps=2),
                      dict(rho=1, cand_frac=0.03, k_ret=40, n_sink=0, n_local=0)),
    # more candidates than the top-k kernel keeps in registers (1024 x 64)
    "select_from_memory": ("tiny_fp32_2k", dict(T=70100, steps=1),
                           dict(rho=16, cand_frac=1.0, k_ret=300, n_sink=50, n_local=50)),
}


def unpack_codes(codes):
    """[.., d/2] bytes -> (sign bits, magnitude bins), each [.., d]."""
    nib = np.stack([codes & 15, codes >> 4], axis=-1).reshape(*codes.shape[:-1], -1)
    return ((nib >> 3) & 1).astype(np.int64), (nib & 7).astype(np.int64)


def gpu_index(K, V, signs, Hq, dt, **params):
    import routed_sparse_kv_amd as rskv
    Kd, Vd = dev_tensor(K, dt), dev_tensor(V, dt)
    idx = rskv.build_retrieval(Kd, Vd, signs, Hq, **params)
    del Kd, Vd
    return idx


def check_codebook(ex, cb):
    assert np.max(np.abs(ex["beta"] - cb[0])) <= 1e-12, "bin boundaries"
    assert np.max(np.abs(ex["lambda_"] - cb[1])) <= 1e-12, "bin means"


def check_encoding(buckets, codes, w, enc, what):
    """GPU rows (buckets, packed codes, w) against oracle.encode_keys."""
    assert np.array_equal(buckets, enc["buckets"]), f"{what}: buckets"
    neg, mag = unpack_codes(codes)
    assert np.array_equal(neg, enc["neg"]), f"{what}: sign bits"
    bad = mag != enc["mag"]
    n_bad = int(bad.sum())
    if n_bad:
        a = np.abs(enc["u"][bad])
        dist = np.min(np.abs(a[:, None] - enc["beta"][None, 1:8]), axis=1)
        assert (dist <= CODE_BAND).all(), f"{what}: magnitude bins differ away from a boundary"
    B = w.shape[-1]
    m = enc["neg"].shape[-1] // B
    sub_bad = bad.reshape(bad.shape[0], B, m).any(axis=2)
    wo = enc["w"].astype(np.float32)
    ok = np.abs(w.astype(np.float64) - wo) <= np.spacing(np.abs(wo)).astype(np.float64)
    assert (ok | sub_bad).all(), f"{what}: calibration beyond one fp32 ulp"
    return n_bad


def vote_ambiguous(qt, m, rho):
    """Subspaces whose top rho + 1 pattern scores hold a near-tie (two
    correct implementations may rank them differently)."""
    out = []
    for b in range(len(qt) // m):
        sc = np.sort(P.pattern_matrix(m) @ qt[b * m:(b + 1) * m])[::-1][:rho + 1]
        gaps = np.abs(np.diff(sc))
        if ((gaps <= VOTE_BAND * max(1e-300, np.abs(sc).max())) & (gaps > 0)).any():
            out.append(b)
    return out


def check_retrieved(g_ret, res, n_sel, first, what):
    """GPU retrieved positions against the oracle's; a difference is excused
    only for candidates whose fp32 decision value ties the k-th within one
    ulp.  Returns the number of excused positions."""
    o_ret = res["retrieved"]
    assert len(g_ret) == len(o_ret) == n_sel, f"{what}: retrieved count"
    assert (np.diff(g_ret) > 0).all(), f"{what}: retrieved not ascending"
    if np.array_equal(g_ret, o_ret):
        return 0
    dec = P.as_decision(res["est"]).astype(np.float64)
    kth = np.sort(dec)[::-1][n_sel - 1]
    pos_to_cand = {int(first + c): j for j, c in enumerate(res["cand"])}
    diff = np.setxor1d(g_ret, o_ret)
    for p in diff:
        assert int(p) in pos_to_cand, f"{what}: position {p} is not a candidate"
        v = dec[pos_to_cand[int(p)]]
        assert abs(v - kth) <= np.spacing(np.float32(abs(kth))), \
            f"{what}: retrieved sets differ away from the cut ({v} vs k-th {kth})"
    return int(len(diff))


def check_step(tr, res, enc, u, info, what):
    n_sel, first = info["n_sel"], info["n_sink"]
    assert np.max(np.abs(tr["q_rot"][u] - res["qt"])) <= 1e-14, f"{what}: rotated query"
    assert abs(tr["q_norm"][u] - res["qnorm"]) <= 1e-13 * max(1.0, res["qnorm"]), f"{what}: |q|"
    amb = vote_ambiguous(res["qt"], 8, info["rho"])
    if amb:
        say(f"  {what}: near-tied pattern scores in subspaces {amb}; exact checks skipped")
        return 0
    assert np.array_equal(tr["votes"][u].astype(np.int64), res["table"]), f"{what}: vote table"
    assert np.array_equal(tr["scores"][u].astype(np.int64), res["scores"]), f"{what}: vote totals"
    C = info["n_cand"]
    s_sorted = np.sort(res["scores"])[::-1]
    s_star = int(s_sorted[C - 1])
    quota = C - int((res["scores"] > s_star).sum())
    assert tr["threshold"][u].tolist() == [s_star, quota], f"{what}: threshold"
    assert np.array_equal(tr["cand"][u], res["cand"]), f"{what}: candidates"
    dec = P.as_decision(res["est"])
    d_ulp = np.abs(tr["est"][u].astype(np.float64) - dec.astype(np.float64))
    assert (d_ulp <= np.spacing(np.abs(dec)).astype(np.float64)).all(), f"{what}: estimates"
    return check_retrieved(tr["retrieved"][u], res, n_sel, first, what)


def run_case(wl, params, kv_tier="hbm", zero_keys=False, zero_query=False, dup_keys=0):
    import torch
    cfg = wl.cfg
    dt, B, Hq, Hkv = wl.dtype, cfg["B"], cfg["Hq"], cfg["Hkv"]
    G = Hq // Hkv
    K, V = wl.K.copy(), wl.V
    signs = W.srht_signs(cfg)
    if zero_keys:
        # zero keys, and keys whose rotation is exactly e_0 + e_9 (k = sigma
        # (H e_0 + H e_9) / d, entries 0 and +-2/d): zero coordinates and
        # zero subspaces after the rotation
        d = cfg["d"]
        h9 = np.array([-1.0 if bin(i & 9).count("1") % 2 else 1.0 for i in range(d)])
        K[:, :, 5::97] = W.store(np.zeros(d, np.float32), dt)
        K[:, :, 11::101] = W.store((signs * (1.0 + h9) / d).astype(np.float32), dt)
    if dup_keys:
        # one key repeated at many positions, aligned with the first query's
        # group mean: its copies share one estimate, and more of them than
        # k_ret rank at the top, so the cut falls inside an exact tie
        G_ = Hq // Hkv
        q0 = W.as_f64(wl.queries[0], dt)
        for b in range(B):
            for h in range(Hkv):
                qb = q0[b, h * G_:(h + 1) * G_].mean(axis=0)
                K[b, h, 100::dup_keys] = W.store((3.0 * qb / np.linalg.norm(qb)).astype(np.float32), dt)
    idx = gpu_index(K, V, signs, Hq, dt, kv_tier=kv_tier, **params)
    info = idx.info
    say(f"  N={info['n_retrieval']} C={info['n_cand']} n_sel={info['n_sel']} "
        f"n_attend={info['n_attend']} tier={kv_tier}")
    ex = idx.export()
    cb = P.magnitude_codebook(8)
    check_codebook(ex, cb)
    Kf, Vf = W.as_f64(K, dt), W.as_f64(V, dt)
    encs, n_bad = {}, 0
    for b in range(B):
        for h in range(Hkv):
            u = b * Hkv + h
            encs[u] = P.encode_unit(Kf[b, h], signs, 8, params["n_sink"], params["n_local"], cb)
            if info["n_retrieval"]:
                n_bad += check_encoding(ex["buckets"][u], ex["codes"][u], ex["w"][u], encs[u],
                                        f"unit {u}")
    worst, excused = 0.0, 0
    for s in range(cfg["steps"]):
        qn = wl.queries[s]
        if zero_query:
            qn = np.zeros_like(qn)
        q = dev_tensor(qn, dt)
        ret = torch.full((B, Hkv, params["k_ret"]), -7, dtype=torch.int32, device="cuda")
        out = idx.decode(q, retrieved=ret)
        torch.cuda.synchronize()
        tr = idx.trace() if info["n_sel"] else None
        gret = ret.cpu().numpy()
        out = out.cpu().numpy().astype(np.float64)
        qf = W.as_f64(qn, dt)
        for b in range(B):
            for h in range(Hkv):
                u = b * Hkv + h
                what = f"step {s} unit {u}"
                g = gret[b, h]
                assert (g[info["n_sel"]:] == -1).all(), f"{what}: padding"
                g = g[:info["n_sel"]].astype(np.int64)
                res = P.decode_unit(encs[u], Kf[b, h], Vf[b, h], qf[b, h * G:(h + 1) * G],
                                    signs, params["rho"], params["cand_frac"], params["k_ret"],
                                    params["n_sink"], params["n_local"])
                if tr is not None:
                    excused += check_step(tr, res, encs[u], u, info, what)
                    assert np.array_equal(tr["retrieved"][u], g), f"{what}: caller buffer"
                else:
                    assert len(g) == 0
                ref = P.decode_unit(encs[u], Kf[b, h], Vf[b, h], qf[b, h * G:(h + 1) * G],
                                    signs, params["rho"], params["cand_frac"], params["k_ret"],
                                    params["n_sink"], params["n_local"], forced=g)
                err = float(np.max(np.abs(out[b, h * G:(h + 1) * G] - ref["out"])))
                worst = max(worst, err)
                assert err <= TOL[dt], f"{what}: max abs err {err:.3e}"
    idx.close()
    say(f"  max abs err {worst:.2e}, codes at a boundary {n_bad}, excused retrievals {excused}")
    return info


@pytest.mark.timeout(600)
@pytest.mark.parametrize("case", list(CASES))
def test_retrieval_parity(case):
    name, over, params = CASES[case]
    say(f"[retrieval {case}] {name} {over} {params}")
    wl = W.generate(name, **over)
    info = run_case(wl, params)
    if case == "no_retrieval_region":
        assert info["n_retrieval"] == 0
    if case == "dense":
        assert info["n_attend"] == wl.cfg["T"]
    if case == "all_candidates":
        assert info["n_sel"] == info["n_cand"]


def test_retrieval_zero_keys_and_query():
    """Zero keys (bucket 0, code 0, w 0) and a zero query (all pattern scores
    tie, every estimate is 0): every stage falls back to its tie rule."""
    wl = W.generate("gqa_32k_bf16", B=1, Hkv=2, Hq=4, T=6000, steps=1)
    say("[retrieval zero keys]")
    run_case(wl, dict(rho=16, cand_frac=0.05, k_ret=40, n_sink=4, n_local=16), zero_keys=True)
    say("[retrieval zero query]")
    run_case(wl, dict(rho=16, cand_frac=0.05, k_ret=40, n_sink=4, n_local=16), zero_query=True)


@pytest.mark.parametrize("stride", [37, 2])
def test_retrieval_tied_estimates(stride):
    """The k_ret-th estimate is shared by many equal keys (a key copied to
    every stride-th position): the retrieved copies are the ones at the
    lowest positions.  With stride 2 the top-k's crossing bin holds more
    members than it ranks in LDS (the refinement path)."""
    wl = W.generate("gqa_32k_bf16", B=1, Hkv=2, Hq=8, T=9001, steps=1)
    say(f"[retrieval tied estimates, stride {stride}]")
    params = dict(rho=16, cand_frac=0.05 if stride > 2 else 0.9, k_ret=64, n_sink=16,
                  n_local=128)
    run_case(wl, params, dup_keys=stride)


def test_retrieval_host_tier_matches_hbm():
    """K/V of the retrieval region in pinned host memory: identical results."""
    import torch
    wl = W.generate("gqa_32k_bf16", B=1, T=9001, steps=2)
    params = dict(rho=16, cand_frac=0.05, k_ret=64, n_sink=16, n_local=128)
    say("[retrieval host tier]")
    info = run_case(wl, params, kv_tier="host")
    assert info["kv_tier"] == 1
    signs = W.srht_signs(wl.cfg)
    a = gpu_index(wl.K, wl.V, signs, wl.cfg["Hq"], wl.dtype, **params)
    b = gpu_index(wl.K, wl.V, signs, wl.cfg["Hq"], wl.dtype, kv_tier="host", **params)
    assert b.info["host_bytes"] > 0 and a.info["host_bytes"] == 0
    for s in range(2):
        q = dev_tensor(wl.queries[s], wl.dtype)
        oa, ob = a.decode(q), b.decode(q)
        torch.cuda.synchronize()
        assert torch.equal(oa, ob), "host tier output differs"
        assert np.array_equal(a.trace()["retrieved"], b.trace()["retrieved"])
    a.close()
    b.close()


def test_retrieval_argument_errors():
    import torch

    import routed_sparse_kv_amd as rskv
    from routed_sparse_kv_amd.binding import RskvError
    K = torch.zeros((1, 1, 64, 64), dtype=torch.float32, device="cuda")
    s = np.ones(64, np.int8)
    with pytest.raises(RskvError, match="rho"):
        rskv.build_retrieval(K, K, s, 1, rho=0)
    with pytest.raises(RskvError, match="cand_frac"):
        rskv.build_retrieval(K, K, s, 1, cand_frac=1.5)
    with pytest.raises(RskvError, match="signs"):
        rskv.build_retrieval(K, K, np.zeros(64, np.int8), 1)
    with pytest.raises(RskvError, match="nothing to attend"):
        rskv.build_retrieval(K, K, s, 1, k_ret=0, n_sink=0, n_local=0)
    idx = rskv.build_retrieval(K, K, s, 1, k_ret=4, n_sink=1, n_local=1)
    with pytest.raises(ValueError):
        idx.decode(torch.zeros((1, 2, 64), device="cuda"))
    idx.close()
    with pytest.raises(RskvError):
        idx.decode(torch.zeros((1, 1, 64), device="cuda"))


@pytest.mark.timeout(900)
def test_retrieval_full_size():
    """The million-token workload at its real shape (8 KV heads, 1M tokens)
    in the configuration bench.py times.  The oracle checks what it can
    compute one by one: 2048 sampled keys of every unit (buckets, codes, w),
    every unit's rotated query and vote table, 512 sampled candidates'
    estimates, and three units' outputs; and properties at full size: the
    vote totals are the oracle's table applied to the (sample-checked)
    buckets, the candidates are the oracle's top ceil(gamma N) of those
    totals, the retrieved set is the oracle's top k_ret of the GPU's fp32
    estimates."""
    import torch
    say("[retrieval full] generate million_1m_bf16")
    wl = W.generate("million_1m_bf16")
    cfg = wl.cfg
    dt, B, Hkv = wl.dtype, cfg["B"], cfg["Hkv"]
    G = cfg["Hq"] // Hkv
    params = W.retrieval_params()
    signs = W.srht_signs(cfg)
    say("[retrieval full] build")
    idx = gpu_index(wl.K, wl.V, signs, cfg["Hq"], dt, **params)
    info = idx.info
    N, C, n_sel, first = info["n_retrieval"], info["n_cand"], info["n_sel"], info["n_sink"]
    say(f"  N={N} C={C} n_sel={n_sel} n_attend={info['n_attend']}")
    ex = idx.export()
    cb = P.magnitude_codebook(8)
    check_codebook(ex, cb)
    rng = np.random.default_rng(7)
    U = B * Hkv
    for u in range(U):
        b, h = divmod(u, Hkv)
        rows = np.sort(rng.choice(N, 2048, replace=False))
        enc = P.encode_keys(W.as_f64(wl.K[b, h, first + rows], dt), signs, 8, cb)
        check_encoding(ex["buckets"][u, rows], ex["codes"][u, rows], ex["w"][u, rows], enc,
                       f"unit {u} sampled keys")
    worst = 0.0
    for s in range(2):
        qn = wl.queries[s]
        ret = torch.full((B, Hkv, params["k_ret"]), -7, dtype=torch.int32, device="cuda")
        say(f"[retrieval full] decode step {s}")
        out = idx.decode(dev_tensor(qn, dt), retrieved=ret)
        torch.cuda.synchronize()
        tr = idx.trace()
        gret = ret.cpu().numpy()
        out = out.cpu().numpy().astype(np.float64)
        qf = W.as_f64(qn, dt)
        for u in range(U):
            b, h = divmod(u, Hkv)
            what = f"step {s} unit {u}"
            qg = qf[b, h * G:(h + 1) * G]
            qbar = qg.sum(axis=0) / G
            qt = P.srht(qbar, signs)[0]
            qnorm = float(np.linalg.norm(qbar))
            assert np.max(np.abs(tr["q_rot"][u] - qt)) <= 1e-14, f"{what}: rotated query"
            assert abs(tr["q_norm"][u] - qnorm) <= 1e-13 * max(1.0, qnorm), f"{what}: |q|"
            assert not vote_ambiguous(qt, 8, params["rho"]), f"{what}: near-tied pattern scores"
            table = P.vote_table(qt, 8, params["rho"])
            assert np.array_equal(tr["votes"][u].astype(np.int64), table), f"{what}: votes"
            sc = P.coarse_scores(ex["buckets"][u].astype(np.int64), table)
            assert np.array_equal(tr["scores"][u].astype(np.int64), sc), f"{what}: totals"
            cand = P.top_by_score(sc, C)
            assert np.array_equal(tr["cand"][u], cand), f"{what}: candidates"
            pick = np.sort(rng.choice(C, 512, replace=False))
            enc = P.encode_keys(W.as_f64(wl.K[b, h, first + cand[pick]], dt), signs, 8, cb)
            dec = P.as_decision(P.estimate(enc, np.arange(512), qt, qnorm))
            d_ulp = np.abs(tr["est"][u, pick].astype(np.float64) - dec.astype(np.float64))
            assert (d_ulp <= np.spacing(np.abs(dec)).astype(np.float64)).all(), \
                f"{what}: sampled estimates"
            want = first + cand[P.top_by_value(tr["est"][u], n_sel)]
            assert np.array_equal(tr["retrieved"][u], want), f"{what}: retrieved set"
            assert np.array_equal(gret[b, h, :n_sel], want) and (gret[b, h, n_sel:] == -1).all()
        for u in sorted({0, U - 1, int(rng.integers(U))}):
            b, h = divmod(u, Hkv)
            T = cfg["T"]
            sink, _, local = P.regions(T, params["n_sink"], params["n_local"])
            use = np.concatenate([sink, gret[b, h, :n_sel], local])
            ref = P.attend(W.as_f64(wl.K[b, h], dt), W.as_f64(wl.V[b, h], dt),
                           qf[b, h * G:(h + 1) * G], use)
            err = float(np.max(np.abs(out[b, h * G:(h + 1) * G] - ref)))
            worst = max(worst, err)
            assert err <= TOL[dt], f"step {s} unit {u}: max abs err {err:.3e}"
    idx.close()
    say(f"[retrieval full] max abs err {worst:.2e}")

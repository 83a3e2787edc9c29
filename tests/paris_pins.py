"""Pins that fix the ParisKV-style retrieval oracle independently of itself.

Each ``pin_*`` takes the oracle module (oracle.paris) and raises
AssertionError when it disagrees with something the page or the mathematics
fixes: a worked example, the Hadamard matrix's closed form, a brute-force
definition enumerated with plain loops, the codebook's closed forms and a
Monte-Carlo draw of the law it quantises, the estimate's exactness along a
key's own direction, and torch's fp64 attention on the retrieved subset.
The helpers here rebuild what they need (Hadamard entries from bit
parities, centroids from itertools) instead of calling the oracle's own.

test_paris_mutants.py runs the same pins on mutated copies of the oracle.
"""
from __future__ import annotations

import itertools
import math

import numpy as np
import torch
import torch.nn.functional as F


def _close(a, b, tol, what=""):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


def _had_entry(i, j):
    """Sylvester Hadamard entry: (-1)^popcount(i & j)."""
    return -1.0 if bin(i & j).count("1") % 2 else 1.0


def _rot_loop(x, signs):
    """H diag(sigma) x / (||x|| sqrt(d)) with explicit loops."""
    d = len(x)
    n = math.sqrt(sum(float(v) * float(v) for v in x))
    if n == 0:
        return np.zeros(d)
    return np.array([sum(_had_entry(i, j) * signs[j] * float(x[j]) for j in range(d))
                     for i in range(d)]) / (n * math.sqrt(d))


def _patterns(m):
    """All centroids as (index, vector): bit i of the index set <=> entry i < 0."""
    out = []
    for bits in itertools.product((0, 1), repeat=m):
        idx = sum(b << i for i, b in enumerate(bits))
        out.append((idx, np.array([-1.0 if b else 1.0 for b in bits]) / math.sqrt(m)))
    return sorted(out)


def _rank_select(values, k):
    """Indices i with #{j: v_j > v_i or (v_j == v_i and j < i)} < k."""
    v = [float(x) for x in values]
    n = len(v)
    return np.array([i for i in range(n)
                     if sum(1 for j in range(n) if v[j] > v[i] or (v[j] == v[i] and j < i)) < k],
                    np.int64)


def _codebook_closed_m8():
    """Octiles and bin means of |y| for m = 8 in closed form.  With t = sin(th)
    the density (1-t^2)^(5/2) dt becomes cos^6(th) dth, whose integral from 0
    is 5 th/16 + 15 sin(2th)/64 + 3 sin(4th)/64 + sin(6th)/192 (5 pi/32 at
    pi/2); the first moment integrates to (1 - (1-t^2)^(7/2)) / 7."""
    def I(t):
        th = math.asin(t)
        return 5 * th / 16 + 15 * math.sin(2 * th) / 64 + 3 * math.sin(4 * th) / 64 + \
            math.sin(6 * th) / 192
    Z = 5 * math.pi / 32
    beta = [0.0]
    for j in range(1, 8):
        lo, hi = 0.0, 1.0
        for _ in range(200):
            mid = 0.5 * (lo + hi)
            lo, hi = (mid, hi) if I(mid) / Z < j / 8 else (lo, mid)
        beta.append(0.5 * (lo + hi))
    beta.append(1.0)
    M = lambda t: (1.0 - (1.0 - t * t) ** 3.5) / 7.0  # noqa: E731
    lam = [(M(beta[j + 1]) - M(beta[j])) / (I(beta[j + 1]) - I(beta[j])) for j in range(8)]
    return np.array(beta), np.array(lam)


# ------------------------------------------------------------------ rotation

def pin_hadamard_closed_form(P):
    for d in (1, 2, 8, 32):
        H = P.hadamard(d)
        ref = np.array([[_had_entry(i, j) for j in range(d)] for i in range(d)])
        assert np.array_equal(H, ref), f"Sylvester entries, d={d}"
        assert np.array_equal(H @ H.T, d * np.eye(d)), f"orthogonality, d={d}"


def pin_srht_worked_example(P):
    # x = (1, 2, 3, 4), sigma = (+, -, +, -): sigma x = (1, -2, 3, -4);
    # H_4 sigma x = (-2, 10, 0, -4); ||x|| sqrt(4) = 2 sqrt(30)
    x = np.array([1.0, 2.0, 3.0, 4.0])
    s = np.array([1.0, -1.0, 1.0, -1.0])
    _close(P.srht(x, s)[0], np.array([-1.0, 5.0, 0.0, -2.0]) / math.sqrt(30), 1e-15, "srht")
    _close(P.rotate(x, s)[0], [-2.0, 10.0, 0.0, -4.0], 0, "rotate")
    assert np.array_equal(P.srht(np.zeros(4), s)[0], np.zeros(4)), "zero vector"


def pin_srht_isometry(P):
    rng = np.random.default_rng(11)
    d = 64
    s = rng.choice([-1.0, 1.0], d)
    X = rng.standard_normal((5, d)) * rng.uniform(0.1, 10, (5, 1))
    Xt = P.srht(X, s)
    _close(np.linalg.norm(Xt, axis=1), np.ones(5), 1e-14, "unit rows")
    U = X / np.linalg.norm(X, axis=1, keepdims=True)
    _close(Xt @ Xt.T, U @ U.T, 1e-14, "angles kept")
    _close(Xt[2], _rot_loop(X[2], s), 1e-14, "loop form")


# ------------------------------------------------------------------ centroids

def pin_bucket_bruteforce(P):
    rng = np.random.default_rng(12)
    pats = _patterns(8)
    for trial in range(20):
        xb = rng.standard_normal(8)
        if trial % 4 == 0:
            xb[rng.integers(8)] = 0.0  # a zero coordinate counts as positive
        scores = [(float(v @ xb), idx) for idx, v in pats]
        best = max(scores, key=lambda t: (t[0], -t[1]))[1]
        assert P.bucket_of(xb) == best, "nearest centroid"
        assert best == sum(1 << i for i in range(8) if xb[i] < 0), "sign pattern"


def pin_encode_buckets(P):
    rng = np.random.default_rng(13)
    d, m = 32, 8
    s = rng.choice([-1.0, 1.0], d)
    K = rng.standard_normal((6, d)).astype(np.float32).astype(np.float64)
    K[5] = 0.0
    enc = P.encode_keys(K, s, m)
    for i in range(6):
        xt = _rot_loop(K[i], s)
        for b in range(d // m):
            want = sum(1 << t for t in range(m) if xt[b * m + t] < 0)
            assert enc["buckets"][i, b] == want, f"key {i} subspace {b}"
    assert (enc["w"][5] == 0).all() and (enc["mag"][5] == 0).all() and (enc["neg"][5] == 0).all()


# ------------------------------------------------------------------ query ranking

def pin_query_ranks_bruteforce(P):
    rng = np.random.default_rng(14)
    pats = _patterns(8)
    for trial in range(6):
        qb = rng.standard_normal(8)
        if trial == 5:
            qb = np.zeros(8)  # every pattern ties: the lowest indices win
        rho = [1, 3, 16, 40, 256, 5][trial]
        scored = sorted(((-float(v @ qb), idx) for idx, v in pats))
        want = [idx for _, idx in scored[:rho]]
        assert list(P.query_ranks(qb, rho)) == want, f"trial {trial}"
        if trial < 5:
            # flip-cost form: the best pattern is the sign pattern; the second
            # flips the coordinate of smallest magnitude
            sign_pat = sum(1 << i for i in range(8) if qb[i] < 0)
            assert want[0] == sign_pat
            if rho > 1:
                assert want[1] == sign_pat ^ (1 << int(np.argmin(np.abs(qb))))


def pin_votes_hand(P):
    # m = 2, d = 4: subspace 0 has q~ = (0.3, -0.1): <q, c_p> sqrt(2) is
    # 0.2, -0.4, 0.4, -0.2 for p = 0..3, ranks p2, p0, p3, p1; subspace 1 has
    # q~ = (-0.5, 0.2): -0.3, 0.7, -0.7, 0.3, ranks p1, p3, p0, p2.  rho = 2.
    qt = np.array([0.3, -0.1, -0.5, 0.2])
    T = P.vote_table(qt, 2, 2)
    assert T.tolist() == [[1, 0, 2, 0], [0, 2, 0, 1]], T.tolist()
    buckets = np.array([[2, 1], [0, 3], [1, 2], [2, 3], [3, 0]])
    assert P.coarse_scores(buckets, T).tolist() == [4, 2, 0, 3, 0]
    T3 = P.vote_table(qt, 2, 3)
    assert T3.tolist() == [[2, 0, 3, 1], [1, 3, 0, 2]], T3.tolist()


def pin_candidates_bruteforce(P):
    rng = np.random.default_rng(15)
    for trial in range(8):
        n = int(rng.integers(1, 40))
        sc = rng.integers(0, 5, n)  # many ties
        C = int(rng.integers(0, n + 2))
        assert np.array_equal(P.top_by_score(sc, min(C, n)), _rank_select(sc, C)), trial
    for N, g, want in ((100, 0.05, 5), (101, 0.05, 6), (7, 1.0, 7), (7, 0.0, 0), (7, 3.0, 7),
                       (20, 0.1, 2), (1, 0.01, 1)):
        assert P.n_candidates(N, g) == want, (N, g)


def pin_top_by_value_bruteforce(P):
    rng = np.random.default_rng(16)
    for trial in range(8):
        n = int(rng.integers(1, 40))
        v = rng.integers(-3, 3, n).astype(np.float32) * np.float32(0.5)
        k = int(rng.integers(0, n + 2))
        assert np.array_equal(P.top_by_value(v, min(k, n)), _rank_select(v, k)), trial
    # the decision precision is fp32: values equal in fp32 tie
    e = np.array([1.0 + 1e-12, 1.0, 0.5])
    assert P.as_decision(e).dtype == np.float32
    assert P.top_by_value(P.as_decision(e), 1).tolist() == [0]
    assert P.top_by_value(P.as_decision(e[::-1].copy()), 1).tolist() == [1]


# ------------------------------------------------------------------ codebook

def pin_codebook_m3(P):
    # m = 3: |y| is uniform on [0, 1], octiles j/8, bin means (2j+1)/16
    beta, lam = P.magnitude_codebook(3)
    _close(beta, np.arange(9) / 8, 1e-13, "m=3 octiles")
    _close(lam, (2 * np.arange(8) + 1) / 16, 1e-13, "m=3 means")


def pin_codebook_m8_closed_form(P):
    beta, lam = P.magnitude_codebook(8)
    rb, rl = _codebook_closed_m8()
    _close(beta, rb, 1e-12, "m=8 octiles")
    _close(lam, rl, 1e-12, "m=8 bin means")


def pin_codebook_m8_monte_carlo(P):
    """The law quantised is that of one coordinate of a uniform unit vector."""
    beta, lam = P.magnitude_codebook(8)
    rng = np.random.default_rng(17)
    Y = rng.standard_normal((200000, 8))
    y = np.abs(Y[:, 0] / np.linalg.norm(Y, axis=1))
    j = np.searchsorted(beta[1:8], y, side="right")
    frac = np.bincount(j, minlength=8) / len(y)
    _close(frac, np.full(8, 0.125), 0.004, "octile mass")
    means = np.array([y[j == i].mean() for i in range(8)])
    _close(means, lam, 0.003, "bin means")


# ------------------------------------------------------------------ codes and estimate

def pin_codes_and_estimate_bruteforce(P):
    rng = np.random.default_rng(18)
    d, m = 32, 8
    s = rng.choice([-1.0, 1.0], d)
    K = rng.standard_normal((5, d)).astype(np.float32).astype(np.float64)
    beta, lam = P.magnitude_codebook(m)
    enc = P.encode_keys(K, s, m, (beta, lam))
    q = rng.standard_normal(d)
    qt = _rot_loop(q, s)
    qn = float(np.linalg.norm(q))
    est = P.estimate(enc, np.arange(5), qt, qn)
    for i in range(5):
        xt = _rot_loop(K[i], s)
        total = 0.0
        for b in range(d // m):
            xb = xt[b * m:(b + 1) * m]
            nb = math.sqrt(float(xb @ xb))
            u = xb / nb
            dot_vu, dot_vq = 0.0, 0.0
            for t in range(m):
                c = b * m + t
                jb = enc["mag"][i, c]
                assert beta[jb] <= abs(u[t]) < beta[jb + 1], "magnitude bin"
                assert enc["neg"][i, c] == (1 if u[t] < 0 else 0), "sign bit"
                v = -lam[jb] if u[t] < 0 else lam[jb]
                dot_vu += v * u[t]
                dot_vq += v * qt[c]
            w = np.linalg.norm(K[i]) * nb / dot_vu
            assert enc["w"][i, b] == float(np.float32(w)), "stored calibration"
            total += float(np.float32(w)) * dot_vq
        _close(est[i], qn * total, 1e-12 * max(1.0, abs(qn * total)), f"estimate {i}")


def pin_estimate_exact_on_own_direction(P):
    """With q = k the calibration makes the estimate exact: ||k||^2."""
    rng = np.random.default_rng(19)
    d, m = 128, 8
    s = rng.choice([-1.0, 1.0], d)
    K = rng.standard_normal((8, d)) * rng.uniform(0.5, 4, (8, 1))
    enc = P.encode_keys(K, s, m)
    for i in range(8):
        qt = P.srht(K[i], s)[0]
        e = P.estimate(enc, [i], qt, float(np.linalg.norm(K[i])))[0]
        _close(e, float(K[i] @ K[i]), 2e-6 * float(K[i] @ K[i]), f"key {i}")


def pin_estimate_accuracy(P):
    """4-bit codes keep the inner products: correlation and scale."""
    rng = np.random.default_rng(20)
    d, m = 128, 8
    s = rng.choice([-1.0, 1.0], d)
    K = rng.standard_normal((2000, d))
    q = rng.standard_normal(d)
    enc = P.encode_keys(K, s, m)
    est = P.estimate(enc, np.arange(2000), P.srht(q, s)[0], float(np.linalg.norm(q)))
    ex = K @ q
    assert np.corrcoef(est, ex)[0, 1] > 0.99
    slope = float(est @ ex / (ex @ ex))
    assert abs(slope - 1.0) < 0.03, slope


# ------------------------------------------------------------------ decode

def _sdpa(qg, K, V):
    q = torch.from_numpy(np.ascontiguousarray(qg))[None, :, None, :]
    k = torch.from_numpy(np.ascontiguousarray(K))[None, None].expand(1, qg.shape[0], -1, -1)
    v = torch.from_numpy(np.ascontiguousarray(V))[None, None].expand(1, qg.shape[0], -1, -1)
    return F.scaled_dot_product_attention(q, k, v)[0, :, 0].numpy()


def pin_regions(P):
    for T, ns, nl, want in ((10, 2, 3, ([0, 1], [2, 3, 4, 5, 6], [7, 8, 9])),
                            (4, 2, 3, ([0, 1], [], [2, 3])),
                            (4, 6, 3, ([0, 1, 2, 3], [], [])),
                            (5, 0, 0, ([], [0, 1, 2, 3, 4], []))):
        got = [r.tolist() for r in P.regions(T, ns, nl)]
        assert got == [list(w) for w in want], (T, ns, nl, got)


def _decode_bruteforce(P, K, V, qg, s, m, rho, gamma, k_ret, ns, nl):
    T, d = K.shape
    sink, ret, local = list(range(min(ns, T))), [], []
    l0 = max(len(sink), T - nl)
    ret = list(range(len(sink), l0))
    local = list(range(l0, T))
    qbar = qg.mean(axis=0)
    qt = _rot_loop(qbar, s)
    qn = float(np.linalg.norm(qbar))
    B = d // m
    pats = _patterns(m)
    votes = []
    for b in range(B):
        qb = qt[b * m:(b + 1) * m]
        ranked = [idx for _, idx in sorted((-float(v @ qb), idx) for idx, v in pats)][:rho]
        votes.append({p: rho - r for r, p in enumerate(ranked)})
    beta, lam = P.magnitude_codebook(m)
    scores, est = [], {}
    for i, pos in enumerate(ret):
        xt = _rot_loop(K[pos], s)
        sc = 0
        for b in range(B):
            xb = xt[b * m:(b + 1) * m]
            sc += votes[b].get(sum(1 << t for t in range(m) if xb[t] < 0), 0)
        scores.append(sc)
    C = min(len(ret), math.ceil(gamma * len(ret)))
    cand = _rank_select(scores, C) if ret else np.zeros(0, np.int64)
    ests = []
    for i in cand:
        xt = _rot_loop(K[ret[i]], s)
        tot = 0.0
        for b in range(B):
            xb = xt[b * m:(b + 1) * m]
            nb = math.sqrt(float(xb @ xb))
            vu = vq = 0.0
            for t in range(m):
                jb = int(np.searchsorted(beta[1:8], abs(xb[t] / nb), side="right"))
                v = -lam[jb] if xb[t] < 0 else lam[jb]
                vu += v * xb[t] / nb
                vq += v * qt[b * m + t]
            tot += float(np.float32(np.linalg.norm(K[ret[i]]) * nb / vu)) * vq
        ests.append(np.float32(qn * tot))
    pick = [ret[cand[j]] for j in _rank_select(ests, k_ret)] if len(cand) else []
    use = sink + sorted(pick) + local
    return np.array(sorted(pick), np.int64), _sdpa(qg, K[use], V[use])


def pin_decode_bruteforce(P):
    rng = np.random.default_rng(21)
    for trial, (T, d, G, rho, gamma, k_ret, ns, nl) in enumerate(
            ((60, 16, 2, 4, 0.25, 5, 3, 6), (45, 32, 3, 16, 0.5, 40, 0, 5),
             (30, 16, 1, 1, 1.0, 4, 4, 0), (9, 16, 2, 4, 0.5, 3, 5, 5))):
        s = rng.choice([-1.0, 1.0], d)
        K = rng.standard_normal((T, d)).astype(np.float32).astype(np.float64)
        V = rng.standard_normal((T, d))
        qg = rng.standard_normal((G, d)) + 2 * K[T // 2]
        enc = P.encode_unit(K, s, 8, ns, nl)
        res = P.decode_unit(enc, K, V, qg, s, rho, gamma, k_ret, ns, nl)
        pick, out = _decode_bruteforce(P, K, V, qg, s, 8, rho, gamma, k_ret, ns, nl)
        assert np.array_equal(res["retrieved"], pick), f"trial {trial}: retrieved"
        _close(res["out"], out, 1e-13, f"trial {trial}: out")


def pin_decode_full_retrieval_is_dense(P):
    """gamma = 1 and k_ret >= N retrieve every token: dense attention."""
    rng = np.random.default_rng(22)
    T, d, G = 50, 32, 4
    s = rng.choice([-1.0, 1.0], d)
    K, V = rng.standard_normal((T, d)), rng.standard_normal((T, d))
    qg = rng.standard_normal((G, d))
    enc = P.encode_unit(K, s, 8, 3, 7)
    res = P.decode_unit(enc, K, V, qg, s, 8, 1.0, T, 3, 7)
    assert res["retrieved"].tolist() == list(range(3, 43))
    _close(res["out"], _sdpa(qg, K, V), 1e-13, "dense")


def pin_decode_group_mean(P):
    """Retrieval sees only the mean of the group's query heads."""
    rng = np.random.default_rng(23)
    T, d = 80, 32
    s = rng.choice([-1.0, 1.0], d)
    K, V = rng.standard_normal((T, d)), rng.standard_normal((T, d))
    qg = rng.standard_normal((3, d)) * 2
    enc = P.encode_unit(K, s, 8, 2, 4)
    a = P.decode_unit(enc, K, V, qg, s, 4, 0.3, 6, 2, 4)
    qm = np.repeat(qg.mean(axis=0, keepdims=True), 3, axis=0)
    b = P.decode_unit(enc, K, V, qm, s, 4, 0.3, 6, 2, 4)
    assert np.array_equal(a["table"], b["table"]) and np.array_equal(a["retrieved"], b["retrieved"])
    c = P.decode_unit(enc, K, V, qg[:1].repeat(3, 0), s, 4, 0.3, 6, 2, 4)
    assert not np.array_equal(a["table"], c["table"]), "table must depend on the mean"


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]

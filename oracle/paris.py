"""fp64 CPU oracle of ParisKV-style token retrieval (test infrastructure).

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the test-suite,
the smoke check and the bench's CPU-baseline leg use it, and it shares no
code, table or constant generator with the HIP library.

Page followed throughout: "ParisKV: Fast and Drift-Robust KV-Cache Retrieval
for Long-Context LLMs" (gist.science, paper 2602.07721, Italian edition),
section "Metodologia: Il Framework ParisKV":
  * "Centroidi Analitici Robusti al Drift": keys and queries are
    l2-normalised and rotated by one shared random orthogonal transform (an
    SRHT) onto the unit sphere; the centroids are fixed sign patterns with
    entries +-1/sqrt(m), independent of the data.
  * "Pipeline di Recupero Nativa su GPU in Due Stadi": the rotated keys are
    cut into B subspaces and each subspace direction goes to its nearest
    analytic centroid; the query's top-rho centroids of every subspace hand
    tiered votes to the keys in those buckets; the integer vote total prunes
    the keys to a small candidate set (the page's example: the top 5-10 %);
    the candidates are reranked by RSQ-IP, a calibrated inner-product
    estimate built from a 4-bit code of every subspace direction (1 sign and
    3 magnitude bits, from the Beta law that the rotation induces on a
    coordinate), a per-key, per-subspace scale w_{i,b} computed at prefill,
    and the estimate ||q||_2 sum_b w_{i,b} <v_{i,b}, q~_b>.
  * "Meccanismo di Aggiornamento a Finestra Scorrevole" (system level): the
    Sink and Local regions stay resident and are always attended; retrieval
    serves the older tokens.

Readings taken where the page leaves a step open (each the plainest one the
rest of it supports):
  P1  SRHT: x~ = H diag(sigma) x / (||x|| sqrt(d)), H the d x d Sylvester
      Hadamard matrix, sigma a vector of random signs given as input
      (x = 0 gives x~ = 0).  The Hadamard sum is formed before the scaling:
      for keys stored in bf16 or fp32 it is then exact in fp64, so every
      sign below is exact.
  P2  B = d/m subspaces of m contiguous coordinates; m = 8 by default.
  P3  Centroid of pattern p in {0 .. 2^m - 1}: c_p[i] = (-1)^(bit i of p) /
      sqrt(m).  A key's bucket in subspace b is argmax_p <x~_b, c_p>, the
      first maximum on ties; that is its sign pattern, a zero coordinate
      counting as positive.
  P4  Retrieval runs once per KV head, on the mean q-bar of its G query
      heads.  Per subspace the 2^m patterns are ranked by <q~_b, c_p>,
      descending, ties to the lower pattern index.
  P5  Tiered votes: a key whose bucket in subspace b is the query's rank-r
      pattern (r < rho) receives rho - r votes; its coarse score is the sum
      over the subspaces.
  P6  Candidates: the C = min(N, ceil(gamma N)) keys of the retrieval region
      (N keys) with the largest coarse score, ties to the lower position.
  P7  4-bit code of a key's subspace direction u = x~_b / ||x~_b||: per
      coordinate a sign bit (set for u_t < 0) and a 3-bit magnitude bin j,
      beta_j <= |u_t| < beta_{j+1}, where beta_0 = 0 < ... < beta_8 = 1 are
      the octiles of |y| for y one coordinate of a uniform random unit
      vector of R^m (|y| has density proportional to (1 - y^2)^((m-3)/2)
      on [0, 1], i.e. y^2 ~ Beta(1/2, (m-1)/2)).  The dequantised
      coordinate is +-lambda_j, the mean of |y| over bin j; v_b is the
      dequantised direction.  A zero subspace (x~_b = 0) has code 0.
  P8  Calibration: w_b = ||k|| ||x~_b|| / <v_b, u_b> (0 for a zero
      subspace), the scale that makes the estimate exact along the key's own
      subspace direction; it is stored in fp32.
  P9  Estimate of <k, q-bar>: ||q-bar|| sum_b w_b <v_b, q~_b> (fp64, with the
      stored w), q~ the rotated unit q-bar.
  P10 The k_ret candidates of largest estimate are retrieved; the estimate
      is rounded to fp32 for this decision, ties to the lower position.
  P11 Regions: Sink = the first n_sink positions, Local = the last n_local,
      Retrieval = the rest.  With no decode-time appends the page's Update
      Buffer is empty.
  P12 Attention per query head: one exact softmax over the Sink, Local and
      retrieved tokens with their stored K/V, logits <q, k> / sqrt(d).

Pinning status (tests/paris_pins.py): the Hadamard matrix and the rotation
(orthogonality, norms, a worked example), the centroid assignment (brute
force over all patterns and the sign-pattern closed form), the query ranking
(brute force and the flip-cost closed form), the votes and scores (hand-worked
example), the codebook (the m = 3 closed form, a Monte-Carlo check of the
octiles at m = 8, the conditional means), the estimate (exact along the key's
own direction; unbiased in expectation; brute force), the selections (brute
force on tiny inputs) and the attention (torch's fp64 softmax attention on
the retrieved subset).  Parity unpinned: P4-P8 and P10-P11 are readings (the
vote tiers, rho, gamma, the octile codebook, the form of w, the fp32
decision, the region sizes); the pins fix the arithmetic of each step, not
the choice.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np
from scipy import integrate, optimize

__all__ = [
    "hadamard", "rotate", "srht", "pattern_matrix", "bucket_of", "query_ranks",
    "vote_table", "coarse_scores", "n_candidates", "top_by_score", "magnitude_codebook",
    "encode_keys", "estimate", "as_decision", "top_by_value", "regions", "encode_unit",
    "decode_unit", "attend", "ESTIMATE_BAND",
]

#: Relative band inside which two correct implementations may order values
#: differently (fp64 rounding of different summation orders).
ESTIMATE_BAND = 1e-9


# --------------------------------------------------------------------------
# rotation and analytic centroids ("Centroidi Analitici Robusti al Drift")
# --------------------------------------------------------------------------

def hadamard(d: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order d (a power of two), entries +-1."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    H = np.ones((1, 1))
    while H.shape[0] < d:
        H = np.block([[H, H], [H, -H]])
    return H


def rotate(X: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """P1 before scaling: rows of H diag(sigma) x (exact for bf16/fp32 input)."""
    X = np.atleast_2d(np.asarray(X, np.float64))
    return (X * np.asarray(signs, np.float64)[None, :]) @ hadamard(X.shape[1]).T


def srht(X: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """P1: x~ = H diag(sigma) x / (||x|| sqrt(d)) for every row (0 for x = 0)."""
    X = np.atleast_2d(np.asarray(X, np.float64))
    R = rotate(X, signs)
    scale = np.linalg.norm(X, axis=1, keepdims=True) * math.sqrt(X.shape[1])
    return np.divide(R, scale, out=np.zeros_like(R), where=scale > 0)


def pattern_matrix(m: int) -> np.ndarray:
    """P3: [2^m][m] centroids; row p is (-1)^(bit i of p) / sqrt(m)."""
    p = np.arange(1 << m)[:, None]
    bits = (p >> np.arange(m)[None, :]) & 1
    return (1.0 - 2.0 * bits) / math.sqrt(m)


def bucket_of(xb: np.ndarray) -> int:
    """P3: the centroid nearest to one subspace direction (largest inner
    product, first maximum).  Any positive multiple of x~_b gives the same."""
    scores = pattern_matrix(len(xb)) @ np.asarray(xb, np.float64)
    return int(np.argmax(scores))


def query_ranks(qb: np.ndarray, rho: int) -> np.ndarray:
    """P4: the rho patterns of largest <q~_b, c_p>, ties to the lower index."""
    scores = pattern_matrix(len(qb)) @ np.asarray(qb, np.float64)
    order = np.lexsort((np.arange(len(scores)), -scores))
    return order[:rho]


def vote_table(qt: np.ndarray, m: int, rho: int) -> np.ndarray:
    """P5: votes[b][p] = rho - (rank of p in subspace b), 0 when unranked."""
    B = len(qt) // m
    T = np.zeros((B, 1 << m), np.int64)
    for b in range(B):
        for r, p in enumerate(query_ranks(qt[b * m:(b + 1) * m], rho)):
            T[b, p] = rho - r
    return T


def coarse_scores(buckets: np.ndarray, table: np.ndarray) -> np.ndarray:
    """P5: vote total of every key; buckets [N][B]."""
    B = table.shape[0]
    return table[np.arange(B)[None, :], buckets].sum(axis=1)


def n_candidates(N: int, gamma: float) -> int:
    """P6: C = min(N, ceil(gamma N)) (gamma N formed in fp64)."""
    return min(N, int(math.ceil(float(gamma) * N)))


def top_by_score(scores: np.ndarray, C: int) -> np.ndarray:
    """P6: indices of the C largest integer scores, ties to the lower index,
    returned in index order."""
    scores = np.asarray(scores)
    order = np.lexsort((np.arange(len(scores)), -scores))
    return np.sort(order[:C])


# --------------------------------------------------------------------------
# RSQ-IP codes and estimate ("Reranking dei Candidati (RSQ-IP)")
# --------------------------------------------------------------------------

_QUAD = dict(epsabs=1e-15, epsrel=1e-13, limit=200)


def magnitude_codebook(m: int):
    """P7: octile boundaries beta[0..8] and bin means lambda[0..7] of |y|, y a
    coordinate of a uniform unit vector of R^m.  The density of |y| is
    proportional to f(t) = (1 - t^2)^((m-3)/2) on [0, 1]; the CDF and the bin
    means are integrated numerically (scipy quad) and each octile is found
    by bracketing root search on the CDF."""
    a = (m - 3) / 2.0

    def f(t):
        return (1.0 - t * t) ** a

    Z = integrate.quad(f, 0.0, 1.0, **_QUAD)[0]

    def cdf(t):
        return integrate.quad(f, 0.0, t, **_QUAD)[0] / Z

    beta = np.zeros(9)
    beta[8] = 1.0
    for j in range(1, 8):
        beta[j] = optimize.brentq(lambda t: cdf(t) - j / 8.0, 0.0, 1.0, xtol=1e-16, rtol=1e-15)
    lam = np.zeros(8)
    for j in range(8):
        num = integrate.quad(lambda t: t * f(t), beta[j], beta[j + 1], **_QUAD)[0]
        den = integrate.quad(f, beta[j], beta[j + 1], **_QUAD)[0]
        lam[j] = num / den
    return beta, lam


def encode_keys(K: np.ndarray, signs: np.ndarray, m: int, codebook=None) -> dict:
    """Buckets (P3), 4-bit codes (P7) and stored calibration (P8) of the rows
    of K [N][d] (fp64 values of the stored keys).

    Returns buckets [N][B], u [N][d] (unit subspace directions), neg [N][d]
    (sign bits), mag [N][d] (bins), w [N][B] (fp32 values, as stored) and
    w64 (before storage rounding)."""
    K = np.atleast_2d(np.asarray(K, np.float64))
    N, d = K.shape
    B = d // m
    beta, lam = codebook if codebook is not None else magnitude_codebook(m)
    R = rotate(K, signs).reshape(N, B, m)       # rotated, not yet scaled
    knorm = np.linalg.norm(K, axis=1)
    scale = knorm * math.sqrt(d)
    Xt = np.divide(R, scale[:, None, None], out=np.zeros_like(R),
                   where=scale[:, None, None] > 0)  # x~ per subspace
    cent = pattern_matrix(m)
    buckets = np.zeros((N, B), np.int64)
    for i0 in range(0, N, 2048):                  # nearest centroid, in chunks
        buckets[i0:i0 + 2048] = np.argmax(R[i0:i0 + 2048] @ cent.T, axis=2)
    xn = np.linalg.norm(Xt, axis=2)               # ||x~_b||
    live = xn > 0
    U = np.divide(Xt, xn[:, :, None], out=np.zeros_like(Xt), where=live[:, :, None])
    neg = (U < 0) & live[:, :, None]
    mag = np.where(live[:, :, None], np.searchsorted(beta[1:8], np.abs(U), side="right"), 0)
    Vq = np.where(neg, -lam[mag], lam[mag])
    den = (Vq * U).sum(axis=2)
    w64 = np.divide(knorm[:, None] * xn, den, out=np.zeros_like(xn), where=live & (den != 0))
    return dict(buckets=buckets, u=U.reshape(N, d), neg=neg.reshape(N, d).astype(np.int64),
                mag=mag.reshape(N, d).astype(np.int64),
                w=w64.astype(np.float32).astype(np.float64), w64=w64, m=m, lam=lam, beta=beta)


def estimate(enc: dict, rows: np.ndarray, qt: np.ndarray, qnorm: float) -> np.ndarray:
    """P9: ||q|| sum_b w_b <v_b, q~_b> for the given key rows (fp64)."""
    m, lam = enc["m"], enc["lam"]
    rows = np.asarray(rows, np.int64)
    mag = enc["mag"][rows]
    V = np.where(enc["neg"][rows] == 1, -lam[mag], lam[mag])
    B = V.shape[1] // m
    dots = (V * np.asarray(qt, np.float64)[None, :]).reshape(len(rows), B, m).sum(axis=2)
    return qnorm * (enc["w"][rows] * dots).sum(axis=1)


def as_decision(est: np.ndarray) -> np.ndarray:
    """P10: the precision in which the retrieval decision is taken (fp32)."""
    return np.asarray(est, np.float64).astype(np.float32)


def top_by_value(values: np.ndarray, k: int) -> np.ndarray:
    """P10: indices of the k largest values, ties to the lower index, in
    index order."""
    values = np.asarray(values)
    order = np.lexsort((np.arange(len(values)), -values.astype(np.float64)))
    return np.sort(order[:k])


# --------------------------------------------------------------------------
# regions and decode ("Meccanismo di Aggiornamento a Finestra Scorrevole")
# --------------------------------------------------------------------------

def regions(T: int, n_sink: int, n_local: int):
    """P11: (sink, retrieval, local) position ranges of a T-token context."""
    s = min(n_sink, T)
    l0 = max(s, T - n_local)
    return np.arange(s), np.arange(s, l0), np.arange(l0, T)


def encode_unit(K: np.ndarray, signs: np.ndarray, m: int, n_sink: int, n_local: int,
                codebook=None) -> dict:
    """Encoding of the retrieval region of one unit; K [T][d] fp64 values of
    the stored keys.  Rows of the result are indexed by position - n_sink."""
    T = K.shape[0]
    _, ret, _ = regions(T, n_sink, n_local)
    enc = encode_keys(np.asarray(K, np.float64)[ret], signs, m, codebook)
    enc["first"] = int(ret[0]) if len(ret) else min(n_sink, T)
    return enc


def decode_unit(enc: dict, K: np.ndarray, V: np.ndarray, q_group: np.ndarray,
                signs: np.ndarray, rho: int, gamma: float, k_ret: int, n_sink: int,
                n_local: int, forced: Optional[np.ndarray] = None) -> dict:
    """Retrieval and attention of one unit (a sequence's KV head).

    K, V [T][d] and q_group [G][d] are fp64 values of the stored tensors.
    Returns the vote table, coarse scores, candidates (retrieval-region
    indices), their estimates, the retrieved positions (absolute, ascending)
    and out [G][d].  `forced` (absolute positions) replaces the retrieved
    set in the attention, for comparing outputs where a different retrieval
    is equally correct."""
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    q_group = np.asarray(q_group, np.float64)
    T, d = K.shape
    m = enc["m"]
    sink, ret, local = regions(T, n_sink, n_local)
    qbar = q_group.sum(axis=0) / q_group.shape[0]
    qnorm = float(np.linalg.norm(qbar))
    qt = srht(qbar, signs)[0]
    res = dict(qt=qt, qnorm=qnorm, table=vote_table(qt, m, rho))
    retrieved = np.zeros(0, np.int64)
    if len(ret):
        sc = coarse_scores(enc["buckets"], res["table"])
        cand = top_by_score(sc, n_candidates(len(ret), gamma))
        est = estimate(enc, cand, qt, qnorm)
        pick = cand[top_by_value(as_decision(est), min(k_ret, len(cand)))]
        res.update(scores=sc, cand=cand, est=est)
        retrieved = ret[pick]
    res["retrieved"] = retrieved
    use = np.concatenate([sink, retrieved if forced is None else np.asarray(forced), local])
    res["out"] = attend(K, V, q_group, use)
    return res


def attend(K: np.ndarray, V: np.ndarray, q_group: np.ndarray, positions: np.ndarray) -> np.ndarray:
    """P12: one exact softmax per query head over the given positions of the
    stored K/V, logits <q, k> / sqrt(d); returns [G][d]."""
    K = np.asarray(K, np.float64)
    idx = np.asarray(positions, np.int64)
    logits = np.asarray(q_group, np.float64) @ K[idx].T / math.sqrt(K.shape[1])
    p = np.exp(logits - logits.max(axis=1, keepdims=True))
    return (p @ np.asarray(V, np.float64)[idx]) / p.sum(axis=1, keepdims=True)

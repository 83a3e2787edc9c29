"""Plain fp64 implementation of SEKV's build and decode (test infrastructure).

Page cited throughout: "SEKV - KV Cache Adattiva alla Risoluzione con
Memoria Semantica Gerarchica" (gist.science, paper 2606.31145, Italian
edition; the Korean edition of the same paper agrees section by section).

Sections used:
  * Metodologia 1, "Segmentazione degli Span Guidata dall'Entropia":
    high-surprisal tokens are anchors kept at full resolution; the tokens
    between two neighbouring anchors form a span S.
  * Metodologia 2, "Rappresentazione dello Span a Doppia Risoluzione":
    each span has a normalised, surprisal-weighted summary of its keys and a
    low-rank SVD basis from which token-level K/V can be rebuilt.
  * Metodologia 3, "Meccanismo di Zoom-In": the query is projected into the
    routing space, a sigmoid gate scores each span, a threshold decides
    expansion, and attention runs over anchors (full K/V), expanded spans
    (rebuilt tokens) and unexpanded spans (summary with a size correction).

Readings taken where the pages leave a step open (each is the plainest one
the rest of the text supports):
  R1  n_a = floor(p*T) anchors: the tokens with the largest surprisal,
      ties going to the lower position.
  R2  spans are the non-empty runs with an anchor on both sides; the run
      before the first anchor and the run after the last anchor stay at full
      resolution with the anchors (adjacent anchors make no empty span).
  R3  summary s = u/||u||, u = sum_t H_t k_t over the span (raw surprisal as
      weight, the span's cached keys); s = 0 when ||u|| = 0.
  R4  the value of an unexpanded span is the arithmetic mean of its values;
      its key is s with logit <q, s>/sqrt(d) + ln|S| (the size correction).
  R5  factors: X = U S W^T per span and per K/V, rank r_j = min(r, |S|, d),
      A = U_r S_r (|S| x r_j), W_r (d x r_j); stored zero-padded to r.
  R6  routing per KV head: rho = P (1/G sum of the group's queries),
      z_j = alpha <rho, s_j>, gate g_j = sigmoid(z_j - tau); a span is a
      candidate iff z_j > tau (g_j > 1/2).  If more than k_max candidates,
      the k_max largest z are kept, ties to the lower span index.
  R7  stored values (s, v-bar, A, W, full-resolution K/V) are rounded to the
      cache dtype (bf16 round-to-nearest-even, or fp32); ln|S| is fp32.  An
      extra "f64" storage mode (no rounding at all) exists for the pins.
  R8  decode-time appends join the trailing full-resolution run before the
      step's attention and are not routed.
  R11 streaming segmentation: an appended token is an anchor iff its
      surprisal exceeds the sequence's threshold theta, the smallest
      surprisal among the prefill anchors (+inf without anchors); the
      full-resolution run after the previous anchor then becomes a span
      (closed with the build's summary, mean, ln|S| and factors).  A token
      appended without a surprisal value counts as surprisal 0.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

__all__ = [
    "n_anchors", "select_anchors", "segment", "span_summary", "span_value_mean",
    "truncated_svd", "round_stored", "from_stored", "build_cache", "append_kv", "close_span",
    "route_unit", "attend_unit", "decode_step", "AMBIGUITY_BAND",
]

#: Width of the band (in z units) inside which a selection may legitimately
#: differ between two correct implementations (rounding of the fp64 z).
AMBIGUITY_BAND = 1e-5


# --------------------------------------------------------------------------
# storage rounding (reading R7)
# --------------------------------------------------------------------------

def _round_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to the nearest bf16 value, ties to even.

    bf16 keeps 7 explicit mantissa bits; an fp64 keeps 52, so the low 45 bits
    are rounded away on the fp64 bit pattern (carries propagate into the
    exponent, as they should).  Values below the bf16 normal range are not
    expected in this workload and are not treated specially.
    """
    x = np.ascontiguousarray(x, dtype=np.float64)
    bits = x.view(np.uint64)
    lsb = (bits >> np.uint64(45)) & np.uint64(1)
    half = np.uint64((1 << 44) - 1)
    keep = ~np.uint64((1 << 45) - 1)
    return ((bits + half + lsb) & keep).view(np.float64)


def round_stored(x: np.ndarray, dtype: str) -> np.ndarray:
    """Value that the cache holds for ``x`` in storage ``dtype`` (fp64 array)."""
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        return _round_bf16(x)
    raise ValueError(dtype)


def from_stored(raw: np.ndarray, dtype: str) -> np.ndarray:
    """fp64 value of a raw stored array (bf16 given as uint16 bit patterns)."""
    if dtype in ("f32", "f64"):
        return np.asarray(raw).astype(np.float64)
    if dtype == "bf16":
        u = np.asarray(raw).astype(np.uint16).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


# --------------------------------------------------------------------------
# segmentation: Metodologia 1 (readings R1, R2)
# --------------------------------------------------------------------------

def n_anchors(T: int, anchor_frac: float) -> int:
    """Number of anchors, floor(p*T) with the product taken in fp64 (R1)."""
    return int(math.floor(float(anchor_frac) * float(T)))


def select_anchors(H: np.ndarray, n_a: int) -> np.ndarray:
    """Boolean anchor mask: the n_a tokens of largest surprisal H_t.

    Metodologia 1: high-surprisal tokens mark span boundaries and are kept at
    full resolution.  Order is (H descending, position ascending) (R1).
    """
    H = np.asarray(H, dtype=np.float32)
    if np.isnan(H).any():
        raise ValueError("surprisal holds NaN")
    T = H.shape[0]
    order = np.lexsort((np.arange(T), -H.astype(np.float64)))
    mask = np.zeros(T, dtype=bool)
    mask[order[:n_a]] = True
    return mask


def segment(H: np.ndarray, n_a: int) -> dict:
    """Anchors, spans and full-resolution tokens of one sequence.

    Returns span_id[t] (j for span j, -1 for anchors, -2 for the lead/tail
    runs kept at full resolution), span starts and lengths in position
    order, and the positions of all full-resolution tokens (anchors and the
    lead/tail runs) in position order.  Metodologia 1, R2.
    """
    T = len(H)
    anchor = select_anchors(H, n_a)
    span_id = np.full(T, -2, dtype=np.int32)
    span_id[anchor] = -1
    pos = np.flatnonzero(anchor)
    starts, lens = [], []
    for left, right in zip(pos[:-1], pos[1:]):
        if right - left > 1:
            starts.append(left + 1)
            lens.append(right - left - 1)
    for j, (st, ln) in enumerate(zip(starts, lens)):
        span_id[st:st + ln] = j
    fr_pos = np.flatnonzero(span_id < 0)
    return dict(span_id=span_id,
                span_start=np.array(starts, dtype=np.int64),
                span_len=np.array(lens, dtype=np.int64),
                fr_pos=fr_pos.astype(np.int64),
                n_a=int(anchor.sum()))


# --------------------------------------------------------------------------
# dual-resolution span store: Metodologia 2 (readings R3, R4, R5)
# --------------------------------------------------------------------------

def span_summary(H_span: np.ndarray, K_span: np.ndarray) -> np.ndarray:
    """Normalised, surprisal-weighted sum of a span's keys (R3), fp64."""
    u = (np.asarray(H_span, np.float64)[:, None] * np.asarray(K_span, np.float64)).sum(axis=0)
    n = math.sqrt(float(u @ u))
    if n == 0.0:
        return np.zeros_like(u)
    return u / n


def span_value_mean(V_span: np.ndarray) -> np.ndarray:
    """Value carried by an unexpanded span: mean of its value rows (R4)."""
    V_span = np.asarray(V_span, np.float64)
    return V_span.sum(axis=0) / V_span.shape[0]


def truncated_svd(X: np.ndarray, r: int):
    """Rank-r_j factors of X (|S| x d): A = U_r S_r, W_r, r_j = min(r,|S|,d).

    Metodologia 2: the token-level structure of a span is encoded by a
    low-rank SVD basis.  Returned A is |S| x r and Wt is r x d, zero-padded
    beyond r_j, so that A @ Wt is the best rank-r_j approximation of X.
    The SVD itself is LAPACK's (numpy), in fp64.
    """
    X = np.asarray(X, np.float64)
    n, d = X.shape
    rj = min(r, n, d)
    U, S, Wt = np.linalg.svd(X, full_matrices=False)
    A = np.zeros((n, r))
    W = np.zeros((r, d))
    A[:, :rj] = U[:, :rj] * S[:rj]
    W[:rj] = Wt[:rj]
    return A, W


def build_cache(H, K, V, rank: int, anchor_frac: float, dtype: str,
                Hq: Optional[int] = None, tail_capacity: int = 0,
                n_anchor: Optional[int] = None) -> dict:
    """Segment, summarise and factor a batch of prefilled contexts.

    H: [B][T] surprisal (fp32 values); K, V: [B][Hkv][T][d] fp64 values of the
    stored inputs.  Returns the canonical cache dictionary: every stored
    array as fp64 values already rounded to ``dtype`` (R7), zero-padded to
    the batch maxima, with per-sequence counts.  ``n_anchor`` replaces
    floor(p*T) when given.  For streaming segmentation (R11) the cache also
    keeps the surprisal of every full-resolution row (HF), the anchor
    threshold of each sequence (theta: the smallest anchor surprisal, +inf
    without anchors) and the full-resolution row of its last anchor (la, -1
    without anchors).
    """
    H = np.asarray(H, np.float32)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    B, T = H.shape
    Hkv, d = K.shape[1], K.shape[3]
    n_a = n_anchors(T, anchor_frac) if n_anchor is None else int(n_anchor)
    segs = [segment(H[b], n_a) for b in range(B)]
    n_s = np.array([len(sg["span_len"]) for sg in segs], dtype=np.int64)
    n_F = np.array([len(sg["fr_pos"]) for sg in segs], dtype=np.int64)
    nt = np.array([int(sg["span_len"].sum()) for sg in segs], dtype=np.int64)
    S = max(1, int(n_s.max()))
    F = max(1, int(n_F.max()) + tail_capacity)
    N = max(1, int(nt.max()))
    c = dict(B=B, Hq=Hq if Hq is not None else Hkv, Hkv=Hkv, d=d, T=T,
             rank=rank, dtype=dtype, tail_capacity=tail_capacity,
             n_a=np.array([sg["n_a"] for sg in segs], dtype=np.int64),
             n_s=n_s, n_F=n_F.copy(), nt=nt, appended=0,
             span_id=np.stack([sg["span_id"] for sg in segs]),
             span_start=np.zeros((B, S), np.int64),
             span_len=np.zeros((B, S), np.int64),
             fr_pos=np.full((B, F), -1, np.int64),
             s=np.zeros((B, Hkv, S, d)), vbar=np.zeros((B, Hkv, S, d)),
             ell=np.zeros((B, S)),
             KF=np.zeros((B, Hkv, F, d)), VF=np.zeros((B, Hkv, F, d)),
             AK=np.zeros((B, Hkv, N, rank)), AV=np.zeros((B, Hkv, N, rank)),
             BK=np.zeros((B, Hkv, S, rank, d)), BV=np.zeros((B, Hkv, S, rank, d)),
             HF=np.zeros((B, F)), theta=np.full(B, np.inf), la=np.full(B, -1, np.int64))
    for b, sg in enumerate(segs):
        ns, nf = int(n_s[b]), int(n_F[b])
        c["span_start"][b, :ns] = sg["span_start"]
        c["span_len"][b, :ns] = sg["span_len"]
        c["fr_pos"][b, :nf] = sg["fr_pos"]
        c["HF"][b, :nf] = H[b, sg["fr_pos"]].astype(np.float64)
        anchors = np.flatnonzero(sg["span_id"] == -1)
        if len(anchors):
            c["theta"][b] = float(H[b, anchors].min())
            c["la"][b] = int(np.searchsorted(sg["fr_pos"], anchors[-1]))
        # ln|S| is kept in fp32 (R7); the oracle-only "f64" mode keeps fp64
        ell = np.log(sg["span_len"].astype(np.float64))
        c["ell"][b, :ns] = ell if dtype == "f64" else ell.astype(np.float32)
        for h in range(Hkv):
            c["KF"][b, h, :nf] = round_stored(K[b, h, sg["fr_pos"]], dtype)
            c["VF"][b, h, :nf] = round_stored(V[b, h, sg["fr_pos"]], dtype)
            off = 0
            for j in range(ns):
                st, ln = int(sg["span_start"][j]), int(sg["span_len"][j])
                ks, vs = K[b, h, st:st + ln], V[b, h, st:st + ln]
                c["s"][b, h, j] = round_stored(span_summary(H[b, st:st + ln], ks), dtype)
                c["vbar"][b, h, j] = round_stored(span_value_mean(vs), dtype)
                for kind, X in (("K", ks), ("V", vs)):
                    A, W = truncated_svd(X, rank)
                    c["A" + kind][b, h, off:off + ln] = round_stored(A, dtype)
                    c["B" + kind][b, h, j] = round_stored(W, dtype)
                off += ln
    return c


def _grow(cache: dict, key: str, axis: int, size: int) -> None:
    """Zero-pad cache[key] along ``axis`` to at least ``size`` entries."""
    a = cache[key]
    if a.shape[axis] >= size:
        return
    pad = [(0, 0)] * a.ndim
    pad[axis] = (0, size - a.shape[axis])
    cache[key] = np.pad(a, pad)


def close_span(cache: dict, b: int) -> None:
    """Streaming segmentation (R11): turn the run of full-resolution rows
    after the last anchor of sequence b into a new span, exactly as the
    build would for a run with an anchor on both sides (Metodologia 1 and
    2): summary, value mean, ln|S| and factors from the stored rows, which
    then leave the full-resolution set.  No-op when there is no anchor or
    the run is empty."""
    la, nf = int(cache["la"][b]), int(cache["n_F"][b])
    ln = nf - la - 1
    if la < 0 or ln <= 0:
        return
    dtype, rank = cache["dtype"], cache["rank"]
    j, off = int(cache["n_s"][b]), int(cache["nt"][b])
    _grow(cache, "span_start", 1, j + 1)
    _grow(cache, "span_len", 1, j + 1)
    _grow(cache, "ell", 1, j + 1)
    for key in ("s", "vbar", "BK", "BV"):
        _grow(cache, key, 2, j + 1)
    for key in ("AK", "AV"):
        _grow(cache, key, 2, off + ln)
    rows = slice(la + 1, nf)
    st = int(cache["fr_pos"][b, la + 1])
    cache["span_start"][b, j] = st
    cache["span_len"][b, j] = ln
    ell = math.log(ln)
    cache["ell"][b, j] = ell if dtype == "f64" else float(np.float32(ell))
    for h in range(cache["Hkv"]):
        ks, vs = cache["KF"][b, h, rows], cache["VF"][b, h, rows]
        cache["s"][b, h, j] = round_stored(span_summary(cache["HF"][b, rows], ks), dtype)
        cache["vbar"][b, h, j] = round_stored(span_value_mean(vs), dtype)
        for kind, X in (("K", ks), ("V", vs)):
            A, W = truncated_svd(X, rank)
            cache["A" + kind][b, h, off:off + ln] = round_stored(A, dtype)
            cache["B" + kind][b, h, j] = round_stored(W, dtype)
    T = cache["T"]
    if st < T:
        cache["span_id"][b, st:min(st + ln, T)] = j
    cache["n_s"][b] = j + 1
    cache["nt"][b] = off + ln
    cache["KF"][b, :, rows] = 0.0
    cache["VF"][b, :, rows] = 0.0
    cache["HF"][b, rows] = 0.0
    cache["fr_pos"][b, rows] = -1
    cache["n_F"][b] = la + 1


def append_kv(cache: dict, k: np.ndarray, v: np.ndarray, h: Optional[np.ndarray] = None) -> None:
    """Append one decoded token per sequence (R8).  k, v: [B][Hkv][d] fp64
    values of the stored token; h: [B] its surprisal (fp32 values) or None.

    Streaming segmentation (R11): a token whose surprisal exceeds the
    sequence's anchor threshold (strictly; an earlier anchor keeps ties) is
    a new anchor; the full-resolution run before it, after the previous
    anchor, is first closed into a span (close_span).  A token without a
    surprisal is never an anchor and weighs 0 in a later span summary.
    """
    B = cache["B"]
    if cache["appended"] >= cache["tail_capacity"]:
        raise ValueError("tail capacity exhausted")
    for b in range(B):
        hb = 0.0 if h is None else float(np.float32(h[b]))
        anchor = h is not None and hb > cache["theta"][b]
        if anchor:
            close_span(cache, b)
        i = int(cache["n_F"][b])
        if i >= cache["KF"].shape[2]:
            raise ValueError("tail capacity exhausted")
        cache["KF"][b, :, i] = round_stored(k[b], cache["dtype"])
        cache["VF"][b, :, i] = round_stored(v[b], cache["dtype"])
        cache["HF"][b, i] = hb
        cache["fr_pos"][b, i] = cache["T"] + cache["appended"]
        cache["n_F"][b] = i + 1
        if anchor:
            cache["la"][b] = i
    cache["appended"] += 1


# --------------------------------------------------------------------------
# zoom-in routing and mixed-resolution attention: Metodologia 3 (R4, R6)
# --------------------------------------------------------------------------

def route_unit(s_rows: np.ndarray, q_group: np.ndarray, tau: float, k_max: int,
               alpha: float = 8.0, P: Optional[np.ndarray] = None) -> dict:
    """Routing decision of one KV head (R6).

    s_rows: [n_s][d] stored summaries; q_group: [G][d] the group's queries.
    Returns z, the gate, the sorted expansion set E and an ambiguity report:
    spans whose z lies within AMBIGUITY_BAND of tau, and whether the k-th and
    (k+1)-th largest candidate z are that close.
    """
    q_group = np.asarray(q_group, np.float64)
    qbar = q_group.sum(axis=0) / q_group.shape[0]
    rho = np.asarray(P, np.float64) @ qbar if P is not None else qbar
    z = alpha * (np.asarray(s_rows, np.float64) @ rho)
    with np.errstate(over="ignore"):
        gate = 1.0 / (1.0 + np.exp(-(z - tau)))
    cand = np.flatnonzero(z > tau)
    rank_tie = False
    if len(cand) > k_max:
        order = np.lexsort((cand, -z[cand]))
        E = np.sort(cand[order[:k_max]])
        if k_max > 0:
            zs = z[cand[order]]
            rank_tie = bool(zs[k_max - 1] - zs[k_max] <= AMBIGUITY_BAND)
    else:
        E = cand
    near = np.flatnonzero(np.abs(z - tau) <= AMBIGUITY_BAND)
    return dict(z=z, gate=gate, E=E.astype(np.int64), near_tau=near,
                rank_tie=rank_tie, n_cand=len(cand))


def attend_unit(cache: dict, b: int, h: int, q_group: np.ndarray,
                E: np.ndarray) -> np.ndarray:
    """Mixed-resolution attention of one KV head's query group (R4).

    Three sources enter one softmax: full-resolution tokens (anchors, lead,
    tail and appended tokens) with their exact K/V; every token of an
    expanded span with K-hat = A_K W_K and V-hat = A_V W_V; every other span
    as a single entry with key s (plus ln|S| on the logit) and value v-bar.
    Returns [G][d].
    """
    d = cache["d"]
    scale = 1.0 / math.sqrt(d)
    nf, ns = int(cache["n_F"][b]), int(cache["n_s"][b])
    lens = cache["span_len"][b, :ns].astype(np.int64)
    offs = np.concatenate([[0], np.cumsum(lens)])
    keys = [cache["KF"][b, h, :nf]]
    vals = [cache["VF"][b, h, :nf]]
    bias = [np.zeros(nf)]
    expanded = np.zeros(ns, dtype=bool)
    expanded[np.asarray(E, np.int64)] = True
    for j in np.flatnonzero(expanded):
        rows = slice(int(offs[j]), int(offs[j + 1]))
        keys.append(cache["AK"][b, h, rows] @ cache["BK"][b, h, j])
        vals.append(cache["AV"][b, h, rows] @ cache["BV"][b, h, j])
        bias.append(np.zeros(int(lens[j])))
    rest = np.flatnonzero(~expanded)
    keys.append(cache["s"][b, h, rest])
    vals.append(cache["vbar"][b, h, rest])
    bias.append(cache["ell"][b, rest].astype(np.float64))
    Kall = np.concatenate(keys)
    Vall = np.concatenate(vals)
    ball = np.concatenate(bias)
    out = np.empty((q_group.shape[0], d))
    for g, q in enumerate(np.asarray(q_group, np.float64)):
        logit = (Kall @ q) * scale + ball
        w = np.exp(logit - logit.max())
        out[g] = (w @ Vall) / w.sum()
    return out


def decode_step(cache: dict, q: np.ndarray, tau: float, k_max: int,
                alpha: float = 8.0, P: Optional[np.ndarray] = None,
                forced_sel: Optional[list] = None, units=None) -> dict:
    """One decode step for every (sequence, KV head) unit.

    q: [B][Hq][d] fp64 query values; P: [1 or Hkv][d][d] or None (identity).
    ``forced_sel[b][h]`` replaces the routed expansion set (used to compare
    outputs where a selection legitimately differs).  ``units`` restricts the
    work to a list of (b, h) pairs; other outputs stay NaN.
    Returns out [B][Hq][d], per-unit routing results and the selections.
    """
    B, Hkv = cache["B"], cache["Hkv"]
    q = np.asarray(q, np.float64)
    Hq = q.shape[1]
    G = Hq // Hkv
    out = np.full((B, Hq, cache["d"]), np.nan)
    routes = {}
    todo = units if units is not None else [(b, h) for b in range(B) for h in range(Hkv)]
    for b, h in todo:
        ns = int(cache["n_s"][b])
        Ph = None
        if P is not None:
            P = np.asarray(P)
            Ph = P[0] if P.shape[0] == 1 else P[h]
        qg = q[b, h * G:(h + 1) * G]
        rt = route_unit(cache["s"][b, h, :ns], qg, tau, k_max, alpha, Ph)
        E = rt["E"] if forced_sel is None else np.asarray(forced_sel[b][h], np.int64)
        out[b, h * G:(h + 1) * G] = attend_unit(cache, b, h, qg, E)
        routes[(b, h)] = rt
    return dict(out=out, routes=routes)

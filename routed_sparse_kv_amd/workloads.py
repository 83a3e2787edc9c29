"""Seeded synthetic inputs for span-routed mixed-resolution KV decode.

This module only *constructs* inputs: surprisal, keys, values, queries, the
routing projection and decode-time appends.  It holds none of the method's
arithmetic (no segmentation, summaries, factors, routing or attention), so
the fp64 oracle and the HIP path can both be fed from it without sharing any
of the computation they are compared on.

Recipes follow the workload descriptions of the SEKV summary ("Segmentazione
degli Span Guidata dall'Entropia": surprisal-marked anchors; spans between
neighbouring anchors) and the five decode configurations the library is
measured on.  No benchmark item (NIAH, RULER, LongBench, ...) is used: needle
depths in the long-context workload are only a placement pattern.

Construction rule shared by every recipe: the generator first picks the anchor
positions, then draws T surprisal values from the configuration's law and
hands the n_a largest ones to the anchor positions (in random order) and the
rest to the other positions (in random order).  For i.i.d. draws this is the
same distribution as drawing i.i.d. and taking the top n_a, but it lets the
generator know the runs between anchors without computing any quantile.
A draw whose n_a-th and (n_a+1)-th largest values tie in fp32 is redrawn.

Storage convention: fp32 arrays are ``np.float32``; bf16 arrays are raw bf16
bit patterns in ``np.uint16`` (round-to-nearest-even from fp32).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np

# --------------------------------------------------------------------------
# configuration table
# --------------------------------------------------------------------------

#: Named decode workloads.  ``recipe`` selects the key/value construction.
CONFIGS: Dict[str, dict] = {
    # 1 KV head, d=64, 2K context, fp32, per-run mean directions (norm 2).
    "tiny_fp32_2k": dict(
        B=1, Hq=1, Hkv=1, d=64, T=2048, dtype="f32", anchor_frac=0.05,
        rank=8, alpha=8.0, tau=0.0, k_max=8, steps=1, recipe="runs",
        h_law=("exp", 1.0), P=None, seed=0, tail_capacity=16,
        query="three_spans"),
    # Llama-3-8B-shaped layer: 32q/8kv, d=128, 32K, bf16, random projection.
    "gqa_32k_bf16": dict(
        B=1, Hq=32, Hkv=8, d=128, T=32768, dtype="bf16", anchor_frac=0.04,
        rank=16, alpha=8.0, tau=1.0, k_max=64, steps=16, recipe="runs",
        h_law=("lognormal", 0.0, 1.0), P="gauss", seed=2000,
        tail_capacity=16, query="uniform"),
    # Long context: B=4, 128K, spans of 8..256 tokens, clustered keys, needles.
    "long_128k_bf16": dict(
        B=4, Hq=32, Hkv=8, d=128, T=131072, dtype="bf16", anchor_frac=0.03,
        rank=16, alpha=8.0, tau=0.0, k_max=393, steps=5, recipe="clustered",
        h_law=("lognormal", 0.0, 1.2), P=None, seed=3000, tail_capacity=16,
        gap_min=8, gap_max=256, n_centres=512, noise=0.5, query="needles"),
    # Batched serving: B=16, 28q/4kv (G=7), 32K, appends every step.
    "serving_b16_bf16": dict(
        B=16, Hq=28, Hkv=4, d=128, T=32768, dtype="bf16", anchor_frac=0.05,
        rank=8, alpha=8.0, tau=0.5, k_max=128, steps=32, recipe="runs",
        h_law=("lognormal", 0.0, 1.0), P=None, seed=4000, tail_capacity=64,
        query="uniform", append=True),
    # One million tokens, drifting key mixture.
    "million_1m_bf16": dict(
        B=1, Hq=32, Hkv=8, d=128, T=1048576, dtype="bf16", anchor_frac=0.02,
        rank=16, alpha=8.0, tau=0.0, k_max=256, steps=4, recipe="drift",
        h_law=("lognormal", 0.0, 1.0), P=None, seed=5000, tail_capacity=16,
        n_centres=512, noise=0.5, query="drift"),
}


#: Token-retrieval router parameters (ParisKV page, "Pipeline di Recupero
#: Nativa su GPU in Due Stadi" and the sliding-window regions): subspace
#: width m, centroids voted per subspace rho, candidate fraction (the page's
#: example range is 5-10 %), tokens retrieved, Sink and Local sizes.  These
#: are parameters of the input, not arithmetic of the method.
RETRIEVAL_DEFAULTS = dict(m=8, rho=16, cand_frac=0.05, k_ret=1024, n_sink=16, n_local=512)


def retrieval_params(**overrides) -> dict:
    """Copy of RETRIEVAL_DEFAULTS with ``overrides`` applied."""
    out = dict(RETRIEVAL_DEFAULTS)
    for k, v in overrides.items():
        if k not in out:
            raise KeyError(f"unknown retrieval parameter {k!r}")
        out[k] = v
    return out


#: Window-routed cache parameters (QEvict page, "Metodologia: QEvict" and
#: the LongBench results): the memory budget as a fraction of the
#: full-precision cache (the page reports budgets of 20 % and 5 %), the
#: share of that budget held by the full-precision tier, and the routing
#: period R in decode steps.  Parameters of the input, not arithmetic of the
#: method.
WINDOW_DEFAULTS = dict(budget=0.2, full_share=0.5, route_every=4)

WINDOW_ROWS = 64
WINDOW_GROUP = 64


def window_params(**overrides) -> dict:
    """Copy of WINDOW_DEFAULTS with ``overrides`` applied."""
    out = dict(WINDOW_DEFAULTS)
    for k, v in overrides.items():
        if k not in out:
            raise KeyError(f"unknown window parameter {k!r}")
        out[k] = v
    return out


def window_tiers(T: int, d: int, dtype: str, budget: float, full_share: float):
    """Window counts (n_full, n_quant) per KV head that fit a byte budget of
    ``budget`` times the full-precision cache: ``full_share`` of the budget
    (rounded down to whole windows) at full precision, the rest in INT2
    windows (2-bit codes plus an fp32 scale and minimum per row and group
    of 64 coordinates, for K and V).  At least one window is kept."""
    n_w = (T + WINDOW_ROWS - 1) // WINDOW_ROWS
    full_b = 2 * WINDOW_ROWS * d * (2 if dtype == "bf16" else 4)
    quant_b = 2 * WINDOW_ROWS * (d // 4) + 2 * WINDOW_ROWS * (d // WINDOW_GROUP) * 2 * 4
    total = budget * n_w * full_b
    n_full = int(math.floor(full_share * budget * n_w))
    n_quant = int(max(0.0, total - n_full * full_b) // quant_b)
    if n_full + n_quant < 1:
        n_full = 1
    return n_full, n_quant


def srht_signs(cfg: dict) -> np.ndarray:
    """The d random signs of the retrieval router's rotation (int8, +-1),
    drawn from ``default_rng([seed, 2**24])`` of the configuration."""
    r = np.random.default_rng([int(cfg["seed"]), 1 << 24])
    return np.where(r.integers(0, 2, int(cfg["d"])) == 1, 1, -1).astype(np.int8)


def config(name: str, **overrides) -> dict:
    """Return a copy of a named configuration with ``overrides`` applied."""
    if name not in CONFIGS:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(CONFIGS)}")
    cfg = dict(CONFIGS[name])
    cfg.update(overrides)
    cfg["name"] = name
    if cfg["Hq"] % cfg["Hkv"]:
        raise ValueError("Hq must be a multiple of Hkv")
    return cfg


# --------------------------------------------------------------------------
# storage helpers (input preparation only)
# --------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); return raw bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    r = (b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen raw bf16 bits to fp32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def store(x: np.ndarray, dtype: str) -> np.ndarray:
    """Cast fp32 input values to the storage representation of ``dtype``."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(dtype)


def as_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 value of a stored input array."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    raise ValueError(dtype)


def n_anchors(T: int, anchor_frac: float) -> int:
    """Anchor count floor(p*T), with p*T evaluated in fp64."""
    return int(math.floor(float(anchor_frac) * float(T)))


# --------------------------------------------------------------------------
# random building blocks
# --------------------------------------------------------------------------

def _unit(rng, n, d):
    x = rng.standard_normal((n, d))
    return x / np.linalg.norm(x, axis=1, keepdims=True)


def _unit_perp(rng, u):
    """Random unit vector orthogonal to unit vector ``u``."""
    x = rng.standard_normal(u.shape[0])
    x -= (x @ u) * u
    return x / np.linalg.norm(x)


def _draw_h(rng, law, n):
    if law[0] == "exp":
        return rng.exponential(law[1], n)
    if law[0] == "lognormal":
        return rng.lognormal(law[1], law[2], n)
    raise ValueError(law)


def _assign_surprisal(rng, law, T, anchor_pos):
    """Give the n_a largest of T draws to ``anchor_pos`` (strictly larger)."""
    n_a = len(anchor_pos)
    for _ in range(100):
        vals = _draw_h(rng, law, T).astype(np.float32)
        srt = np.sort(vals)[::-1]
        if 0 < n_a < T and not srt[n_a - 1] > srt[n_a]:
            continue
        H = np.empty(T, np.float32)
        is_a = np.zeros(T, bool)
        is_a[anchor_pos] = True
        H[anchor_pos] = rng.permutation(srt[:n_a])
        H[~is_a] = rng.permutation(srt[n_a:])
        return H
    raise RuntimeError("could not draw untied surprisal")


def _runs_from_anchors(T, anchor_pos):
    """(start, length) of every maximal non-anchor run, lead and tail included."""
    edges = np.concatenate([[-1], np.sort(anchor_pos), [T]])
    starts = edges[:-1] + 1
    lens = edges[1:] - starts
    return starts, lens


def _gap_lengths(rng, n_runs, total, lo, hi):
    """n_runs lengths in [lo, hi] summing to ``total`` (8 + geometric law)."""
    if not (n_runs * lo <= total <= n_runs * hi):
        raise ValueError("gap bounds cannot reach the requested total")
    mean_extra = total / n_runs - lo
    p = 1.0 / (mean_extra + 1.0) if mean_extra > 0 else 1.0
    g = lo + rng.geometric(p, n_runs) - 1
    bad = g > hi
    while bad.any():
        g[bad] = lo + rng.geometric(p, int(bad.sum())) - 1
        bad = g > hi
    diff = int(g.sum()) - total
    while diff != 0:
        i = int(rng.integers(n_runs))
        if diff > 0 and g[i] > lo:
            g[i] -= 1
            diff -= 1
        elif diff < 0 and g[i] < hi:
            g[i] += 1
            diff += 1
    return g


# --------------------------------------------------------------------------
# workload object
# --------------------------------------------------------------------------

@dataclasses.dataclass
class Workload:
    cfg: dict
    H: np.ndarray                 # [B][T] fp32 surprisal
    K: np.ndarray                 # [B][Hkv][T][d] stored dtype
    V: np.ndarray                 # [B][Hkv][T][d] stored dtype
    queries: List[np.ndarray]     # per step [B][Hq][d] stored dtype
    appends: Optional[List[tuple]]  # per step (k, v) [B][Hkv][d] or None
    append_h: Optional[List[np.ndarray]]  # per step [B] fp32 surprisal of the appends
    P: Optional[np.ndarray]       # [1][d][d] fp32 or None
    anchor_pos: List[np.ndarray]  # per b, sorted anchor positions
    needles: Optional[List[np.ndarray]] = None  # per b, needle span starts

    @property
    def dtype(self) -> str:
        return self.cfg["dtype"]


def generate(name: str, workers: Optional[int] = None, **overrides) -> Workload:
    """Build the seeded workload ``name`` (see ``CONFIGS``).

    Streams: sequence structure (anchors, surprisal, run directions, needles)
    comes from ``default_rng([seed, b])``; the token noise of KV head h of
    sequence b from ``default_rng([seed, b, h])``; queries and appends from
    ``default_rng([seed, b, 2**21])``; the surprisal of the appended tokens,
    drawn from the configuration's law, from ``default_rng([seed, b, 2**23])``.
    Units are generated on a thread pool;
    the result does not depend on the number of workers.
    """
    cfg = config(name, **overrides)
    B, Hq, Hkv, d, T = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["d"], cfg["T"]
    G = Hq // Hkv
    dt = cfg["dtype"]
    n_a = n_anchors(T, cfg["anchor_frac"])
    steps = cfg["steps"]
    recipe = cfg["recipe"]
    seed = int(cfg["seed"])

    H = np.empty((B, T), np.float32)
    kd = np.float32 if dt == "f32" else np.uint16
    K = np.empty((B, Hkv, T, d), kd)
    V = np.empty((B, Hkv, T, d), kd)
    q_all = np.zeros((steps, B, Hq, d), np.float32)
    app_k = np.zeros((steps, B, Hkv, d), np.float32) if cfg.get("append") else None
    app_v = np.zeros((steps, B, Hkv, d), np.float32) if cfg.get("append") else None
    app_h = np.zeros((steps, B), np.float32) if cfg.get("append") else None
    anchors, needles = [], []

    P = None
    if cfg.get("P") == "gauss":
        prng = np.random.default_rng([seed, 1 << 20])
        P = (prng.standard_normal((1, d, d)) / math.sqrt(d)).astype(np.float32)

    jobs = []
    for b in range(B):
        rng = np.random.default_rng([seed, b])
        # ---- anchor positions, surprisal and runs
        if recipe == "clustered" and n_a >= 2:
            lens = _gap_lengths(rng, n_a + 1, T - n_a, cfg["gap_min"], cfg["gap_max"])
            # anchor i sits after runs 0..i and the i anchors before it
            apos = (np.cumsum(lens[:-1]) + np.arange(n_a)).astype(np.int64)
        else:
            apos = np.sort(rng.choice(T, n_a, replace=False)).astype(np.int64)
        anchors.append(apos)
        H[b] = _assign_surprisal(rng, cfg["h_law"], T, apos)
        starts, lens = _runs_from_anchors(T, apos)
        n_runs = len(starts)
        interior = np.arange(1, n_runs - 1)
        interior = interior[lens[interior] > 0]
        # per-token row into a table of [run rows | anchor rows]
        amask = _anchor_mask(T, apos)
        tok_row = np.empty(T, np.int64)
        tok_row[~amask] = np.repeat(np.arange(n_runs), lens)
        tok_row[amask] = n_runs + np.arange(n_a)

        needle_runs, u_needle = None, None
        if recipe == "clustered":
            needle_runs = _pick_needles(starts, lens, interior, T)
            needles.append(starts[needle_runs])
            u_needle = _unit(rng, len(needle_runs), d)
        tables = []
        for h in range(Hkv):
            if recipe == "runs":
                mK = _unit(rng, n_runs, d)
                mV = _unit(rng, n_runs, d)
                zK = np.zeros((n_a, d))
                tables.append((np.vstack([2.0 * mK, zK]).astype(np.float32),
                               np.vstack([2.0 * mV, zK]).astype(np.float32), mK, mV))
            elif recipe == "clustered":
                cen = _unit(rng, cfg["n_centres"], d)
                rows = np.vstack([cen[rng.integers(cfg["n_centres"], size=n_runs)],
                                  cen[rng.integers(cfg["n_centres"], size=n_a)]])
                rows[needle_runs] = u_needle
                tables.append((rows.astype(np.float32), None, None, None))
            elif recipe == "drift":
                comp = rng.integers(cfg["n_centres"], size=n_runs + n_a)
                tables.append((comp, None, None, None))
            else:
                raise ValueError(recipe)
            jobs.append((b, h, tok_row, tables[-1]))

        # ---- queries (unit norm before storage rounding) and appends
        qrng = np.random.default_rng([seed, b, 1 << 21])
        for s in range(steps):
            if cfg["query"] == "three_spans":
                # q = 0.6*u + 0.8*xi, u the normalised sum of the mean key
                # directions of three random spans, xi a unit vector _|_ u.
                chosen = qrng.choice(interior, size=min(3, len(interior)), replace=False)
                u = tables[0][2][chosen].sum(axis=0)
                u /= np.linalg.norm(u)
                for hq in range(Hq):
                    q_all[s, b, hq] = 0.6 * u + 0.8 * _unit_perp(qrng, u)
            elif cfg["query"] == "uniform":
                q_all[s, b] = _unit(qrng, Hq, d)
            elif cfg["query"] == "needles":
                u = u_needle[s % len(u_needle)]
                for hq in range(Hq):
                    q_all[s, b, hq] = 0.6 * u + 0.8 * _unit_perp(qrng, u)
            elif cfg["query"] == "drift":
                for hq in range(Hq):
                    u = _drift_query_dir(cfg, qrng, b, hq // G, d)
                    q_all[s, b, hq] = 0.6 * u + 0.8 * _unit_perp(qrng, u)
            else:
                raise ValueError(cfg["query"])
        if app_k is not None:
            hrng = np.random.default_rng([seed, b, 1 << 23])
            app_h[:, b] = _draw_h(hrng, cfg["h_law"], steps).astype(np.float32)
            for h in range(Hkv):
                mK, mV = tables[h][2], tables[h][3]
                app_k[:, b, h] = qrng.standard_normal((steps, d)) + 2.0 * mK[-1]
                app_v[:, b, h] = qrng.standard_normal((steps, d)) + 2.0 * mV[-1]

    def unit_job(job):
        b, h, tok_row, tab = job
        r = np.random.default_rng([seed, b, h])
        step = 1 << 14
        for t0 in range(0, T, step):
            t1 = min(T, t0 + step)
            n = t1 - t0
            nk = r.standard_normal((n, d), dtype=np.float32)
            nv = r.standard_normal((n, d), dtype=np.float32)
            rows = tok_row[t0:t1]
            if recipe == "runs":
                nk += tab[0][rows]
                nv += tab[1][rows]
            elif recipe == "clustered":
                nk *= np.float32(cfg["noise"])
                nk += tab[0][rows]
            else:  # drift
                nk *= np.float32(cfg["noise"])
                nk += _drift_mean_chunk(cfg, b, h, d, tab[0][rows], t0, t1, T)
            K[b, h, t0:t1] = store(nk, dt)
            V[b, h, t0:t1] = store(nv, dt)

    import concurrent.futures as cf
    import os
    nw = workers or min(16, os.cpu_count() or 1)
    if nw <= 1 or len(jobs) == 1:
        for jb in jobs:
            unit_job(jb)
    else:
        with cf.ThreadPoolExecutor(nw) as ex:
            list(ex.map(unit_job, jobs))

    queries = [store(q_all[s], dt) for s in range(steps)]
    appends, append_h = None, None
    if app_k is not None:
        appends = [(store(app_k[s], dt), store(app_v[s], dt)) for s in range(steps)]
        append_h = [app_h[s].copy() for s in range(steps)]
    return Workload(cfg=cfg, H=H, K=K, V=V, queries=queries, appends=appends, append_h=append_h,
                    P=P, anchor_pos=anchors,
                    needles=needles if recipe == "clustered" else None)


def _anchor_mask(T, apos):
    m = np.zeros(T, bool)
    m[apos] = True
    return m


def _pick_needles(starts, lens, interior, T):
    """Interior runs holding positions floor(f*T), f in {.1,.3,.5,.7,.9}.

    If the position is an anchor or lies in the lead/tail run, the next
    interior run to the right is used instead.
    """
    out = []
    for f in (0.1, 0.3, 0.5, 0.7, 0.9):
        pos = int(math.floor(f * T))
        cand = interior[(starts[interior] + lens[interior] > pos)]
        inside = cand[starts[cand] <= pos]
        ri = int(inside[0]) if len(inside) else int(cand[0])
        if ri in out:
            later = cand[cand > ri]
            ri = int(later[0])
        out.append(ri)
    return np.array(out, np.int64)


def _drift_centres(cfg, b, h, d):
    r = np.random.default_rng([int(cfg["seed"]), b, h, 1 << 22])
    return _unit(r, cfg["n_centres"], d), _unit(r, cfg["n_centres"], d)


def _drift_mean_chunk(cfg, b, h, d, comp, t0, t1, T):
    """mu_c(t) = normalise((1 - t/T) a_c + (t/T) b_c) for tokens t0..t1-1."""
    a, bb = _drift_centres(cfg, b, h, d)
    a = a.astype(np.float32)
    bb = bb.astype(np.float32)
    f = (np.arange(t0, t1, dtype=np.float64) / T).astype(np.float32)[:, None]
    m = (1.0 - f) * a[comp] + f * bb[comp]
    m /= np.linalg.norm(m, axis=1, keepdims=True)
    return m


def _drift_query_dir(cfg, qrng, b, h, d):
    a, bb = _drift_centres(cfg, b, h, d)
    c = int(qrng.integers(cfg["n_centres"]))
    return bb[c]  # mu_c(T): t/T = 1 leaves the unit vector b_c

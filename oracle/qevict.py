"""fp64 CPU oracle of the window-routed three-tier cache (test infrastructure).

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the test-suite,
the smoke check and the bench's CPU-baseline leg use it, and it shares no
code, table or constant generator with the HIP library.

Page followed: "QEvict" technical summary (gist.science, paper 2608.05326,
Italian edition), section "Metodologia: QEvict" and its "Meccanismi
Chiave": the cached history is cut into contiguous windows; under a fixed
memory budget each window is routed to one of three tiers (full precision;
a recoverable low-bit tier, INT2 in the experiments, still attended and
promotable; evicted for good); a window's importance is its attention mass
accumulated over time; a full-precision window whose importance falls is
demoted, a quantised one whose score rises is dequantised and promoted; a
window is quantised once, at its first demotion, into a write-once ledger
that every later promotion and demotion reuses; attention is computed
materially at routing events to update the scores.

Readings taken where the page leaves a step open (each the plainest one the
rest of it supports):
  W1  Windows of w contiguous positions (w = 64), window j covering
      [j w, (j+1) w); the last one may be shorter.
  W2  The tier sizes are given as window counts n_full (full precision) and
      n_quant (INT2); the caller derives them from a byte budget.  Before
      the first routing event every window is at full precision (the
      prefilled cache).
  W3  Score of a window = its attention mass summed over the routing events
      so far: at an event, the softmax probabilities of the group's query
      heads over the resident tokens, summed over the heads and over the
      window's positions.  Evicted windows receive nothing.
  W4  Routing events happen at decode steps 0, R, 2R, ...  At an event the
      step attends with the tiers in force, adds the masses to the scores,
      then re-tiers for the following steps.
  W5  Re-tiering ranks the windows that are not evicted by score,
      descending, ties to the lower window index: the first n_full are full
      precision, the next n_quant INT2, the rest evicted for good.
  W6  INT2 code of a window (K and V alike): per position and group of g =
      64 consecutive coordinates, mn = min, scale = (max - min) / 3,
      code = clamp(rint((x - mn) / scale), 0, 3) (code 0 when scale = 0),
      all in fp32; the dequantised value is mn + code * scale (fp32, the
      product and the sum each rounded).  It is computed at the window's
      first demotion from the window's values then and kept (write-once).
  W7  Promotion replaces the window's full-precision values by its
      dequantised values rounded to the cache dtype.
  W8  Attention per query head: one softmax over the positions of the full
      windows (their values) and of the INT2 windows (dequantised values),
      logits <q, k> / sqrt(d).  One tiering per KV head (GQA).

Pinning status (tests/qevict_pins.py): the quantiser (a hand-worked group,
constant groups, ties rounding to even, the error bound scale / 2, the
value range), attention (torch's fp64 attention when every window is full,
over the dequantised cache when every window is INT2; masses summing to the
number of query heads; masses against brute force), routing (a hand-worked
ranking with ties, permanence of eviction, the event schedule), the
write-once ledger (demote, promote, demote keeps the codes; promotion
restores the dequantised values) and the full-budget case (dense attention
at every step).  Parity unpinned: W1-W8 are readings (window size, group
size, scale form, score rule, event rule, tier order).
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

from .sekv import round_stored

__all__ = ["window_count", "quantize_int2", "dequantize_int2", "new_unit", "attend_unit",
           "route_unit", "decode_unit", "MASS_BAND"]

#: Relative band inside which two correct implementations may rank window
#: scores differently (fp32 attention probabilities against fp64).
MASS_BAND = 1e-5

FULL, QUANT, EVICTED = 0, 1, 2


def window_count(T: int, w: int) -> int:
    """W1: number of windows of a T-position context."""
    return (T + w - 1) // w


def quantize_int2(X: np.ndarray, g: int):
    """W6: INT2 codes of the rows of X [n][d] in groups of g coordinates, in
    fp32 arithmetic.  Returns codes [n][d] (uint8 0..3), scale and mn
    [n][d/g] (fp32)."""
    X = np.asarray(X, np.float64).astype(np.float32)
    n, d = X.shape
    Xg = X.reshape(n, d // g, g)
    mn = Xg.min(axis=2)
    mx = Xg.max(axis=2)
    scale = (mx - mn) / np.float32(3.0)
    safe = np.where(scale > 0, scale, np.float32(1.0))
    codes = np.rint((Xg - mn[:, :, None]) / safe[:, :, None])
    codes = np.clip(codes, 0, 3).astype(np.uint8)
    codes[scale == 0] = 0
    return codes.reshape(n, d), scale.astype(np.float32), mn.astype(np.float32)


def dequantize_int2(codes: np.ndarray, scale: np.ndarray, mn: np.ndarray, g: int) -> np.ndarray:
    """W6: mn + code * scale in fp32 (two roundings); returned as fp64."""
    n, d = codes.shape
    c = codes.reshape(n, d // g, g).astype(np.float32)
    prod = (c * scale[:, :, None]).astype(np.float32)
    return (mn[:, :, None] + prod).astype(np.float32).reshape(n, d).astype(np.float64)


def new_unit(K: np.ndarray, V: np.ndarray, w: int) -> dict:
    """State of one unit (a sequence's KV head) after prefill (W2): K, V
    [T][d] fp64 values of the stored cache, every window full precision."""
    T = K.shape[0]
    nW = window_count(T, w)
    return dict(K=np.array(K, np.float64), V=np.array(V, np.float64), w=w, T=T,
                tier=np.zeros(nW, np.int64), score=np.zeros(nW), ledger={})


def _window_rows(st: dict, j: int) -> slice:
    w = st["w"]
    return slice(j * w, min((j + 1) * w, st["T"]))


def _resident(st: dict, g: int):
    """Positions attended and their K/V values (W8)."""
    K, V = st["K"].copy(), st["V"].copy()
    keep = np.zeros(st["T"], bool)
    for j, tier in enumerate(st["tier"]):
        rows = _window_rows(st, j)
        if tier == FULL:
            keep[rows] = True
        elif tier == QUANT:
            ck, sk, mk, cv, sv, mv = st["ledger"][j]
            K[rows] = dequantize_int2(ck, sk, mk, g)
            V[rows] = dequantize_int2(cv, sv, mv, g)
            keep[rows] = True
    pos = np.flatnonzero(keep)
    return pos, K[pos], V[pos]


def attend_unit(st: dict, q_group: np.ndarray, g: int):
    """W8 and W3: out [G][d] and the attention mass of every window (summed
    over the G query heads; 0 for evicted windows)."""
    q_group = np.asarray(q_group, np.float64)
    pos, K, V = _resident(st, g)
    logits = q_group @ K.T / math.sqrt(K.shape[1])
    p = np.exp(logits - logits.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    out = p @ V
    mass = np.zeros(len(st["tier"]))
    np.add.at(mass, pos // st["w"], p.sum(axis=0))
    return out, mass


def route_unit(st: dict, mass: np.ndarray, n_full: int, n_quant: int, g: int, dtype: str,
               forced: Optional[np.ndarray] = None) -> np.ndarray:
    """W3, W5-W7: add the masses, re-tier, quantise first demotions into the
    ledger, restore promoted windows.  Returns the new tiers.  `forced`
    imposes a tier vector (for comparing runs where a different ranking of
    near-equal scores is equally correct)."""
    st["score"] = st["score"] + mass
    old = st["tier"].copy()
    live = np.flatnonzero(old != EVICTED)
    order = live[np.lexsort((live, -st["score"][live]))]
    new = np.full(len(old), EVICTED, np.int64)
    new[order[:n_full]] = FULL
    new[order[n_full:n_full + n_quant]] = QUANT
    if forced is not None:
        new = np.asarray(forced, np.int64).copy()
    for j in range(len(old)):
        rows = _window_rows(st, j)
        if new[j] == QUANT and old[j] == FULL and j not in st["ledger"]:
            st["ledger"][j] = (*quantize_int2(st["K"][rows], g), *quantize_int2(st["V"][rows], g))
        if new[j] == FULL and old[j] == QUANT:
            ck, sk, mk, cv, sv, mv = st["ledger"][j]
            st["K"][rows] = round_stored(dequantize_int2(ck, sk, mk, g), dtype)
            st["V"][rows] = round_stored(dequantize_int2(cv, sv, mv, g), dtype)
    st["tier"] = new
    return new


def decode_unit(st: dict, q_group: np.ndarray, step: int, R: int, n_full: int, n_quant: int,
                g: int, dtype: str):
    """One decode step of a unit (W4): attention with the tiers in force;
    at a routing event, score update and re-tiering afterwards.  Returns
    out [G][d], the masses and whether the step was an event."""
    out, mass = attend_unit(st, q_group, g)
    event = step % R == 0
    if event:
        route_unit(st, mass, n_full, n_quant, g, dtype)
    return out, mass, event

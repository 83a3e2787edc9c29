"""Full-size parity (GPU): every workload at its real shape, built and
decoded by the library in its default launch configuration (the one
bench.py times).

Build: every sequence's segmentation (span ids, span starts and lengths,
full-resolution positions, anchor count, anchor threshold, last anchor) is
compared bit-exactly with the oracle's segmentation of the same surprisal;
for the checked units the packed full-resolution rows are the input rows
bit for bit, 40 sampled spans' summaries and value means are within one
stored ulp of the oracle's, ln|S| is exact, and their factor products match
the oracle's factors within the storage-rounding bound (plus the
Eckart-Young residual).

Decode: selections of every (sequence, KV head) unit are compared with the
oracle's routing on the stored summaries (exact outside the 1e-5 ambiguity
band); outputs of the checked units with the oracle's decode of those units
on the same stored cache (GPU selection forced where the band excuses a
difference), within 1e-2 max-abs for bf16 caches.  The oracle converts and
decodes one unit at a time, so the check stays within seconds per unit at
a million tokens.
"""
import numpy as np
import pytest

import oracle
from gpu_helpers import (TOL, check_factor_products, check_full_rows, check_segmentation_tables,
                         check_selection, check_summaries, decode_gpu, dev_tensor, gpu_build, say,
                         unit_view)
from routed_sparse_kv_amd import workloads as W

pytestmark = pytest.mark.gpu

# workload -> decode steps checked (appends run before every step)
STEPS = {"gqa_32k_bf16": 3, "long_128k_bf16": 2, "serving_b16_bf16": 32, "million_1m_bf16": 2}
# steps whose decode is checked when not all are (serving: 32 appends with
# their surprisal, so decoded anchors close spans; decode checked every 8th)
CHECK_EVERY = {"serving_b16_bf16": 8}
# units whose build (rows, summaries, factors) is checked against the oracle
BUILD_UNITS = 4
SPANS_PER_UNIT = 40


def _sampled_units(B, Hkv, seed, n):
    rng = np.random.default_rng(seed)
    u = {(0, 0), (B - 1, Hkv - 1)}
    while len(u) < min(n, B * Hkv):
        u.add((int(rng.integers(B)), int(rng.integers(Hkv))))
    return sorted(u)


class _Rows:
    """fp64 values of a stored [T][d] array, converted slice by slice (a
    million-token unit is never converted whole)."""

    def __init__(self, raw, dtype):
        self.raw, self.dtype = raw, dtype

    def __getitem__(self, rows):
        return W.as_f64(self.raw[rows], self.dtype)


def _check_build(wl, ex, name):
    """Build-time parity of a full-size cache against the oracle."""
    cfg = wl.cfg
    dt = wl.dtype
    check_segmentation_tables(ex, wl.H, cfg["anchor_frac"], name)
    rng = np.random.default_rng(cfg["seed"] + 7)
    worst, checked = 0.0, 0
    for b, h in _sampled_units(cfg["B"], cfg["Hkv"], cfg["seed"] + 1, BUILD_UNITS):
        check_full_rows(ex, wl.K, wl.V, b, h, name)
        ns = int(ex["n_spans"][b])
        if ns == 0:
            continue
        js = np.sort(rng.choice(ns, size=min(ns, SPANS_PER_UNIT), replace=False))
        Kf, Vf = _Rows(wl.K[b, h], dt), _Rows(wl.V[b, h], dt)
        worst = max(worst, check_summaries(ex, wl.H, Kf, Vf, b, h, js, dt, name))
        checked += check_factor_products(ex, Kf, Vf, b, h, js, dt, cfg["rank"], name)
    say(f"[full {name}] build: tables of {cfg['B']} sequences exact; summaries within "
        f"{worst:.2f} ulp, {checked} factor products checked")


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("name", sorted(STEPS))
def test_full_size_parity(name):
    import routed_sparse_kv_amd as rskv
    say(f"[full {name}] generate")
    wl = W.generate(name)
    cfg = wl.cfg
    dt, tau, k_max, alpha = wl.dtype, cfg["tau"], cfg["k_max"], cfg["alpha"]
    B, Hkv, G = cfg["B"], cfg["Hkv"], cfg["Hq"] // cfg["Hkv"]
    say(f"[full {name}] build_spans on GPU")
    cache = gpu_build(wl)
    ex = cache.export()
    say(f"[full {name}] build against the oracle")
    _check_build(wl, ex, name)
    units = [(b, h) for b in range(B) for h in range(Hkv)]
    views = {u: unit_view(ex, *u) for u in units}
    if wl.append_h is not None:
        n_anc = [sum(float(h[b]) > float(ex["theta"][b]) for h in wl.append_h[:STEPS[name]])
                 for b in range(B)]
        say(f"[full {name}] decoded anchors per sequence: {n_anc}")
    P = wl.P
    worst, excused = 0.0, 0
    for s in range(STEPS[name]):
        if wl.appends is not None:
            import torch
            k, v = wl.appends[s]
            hs = wl.append_h[s]
            rskv.append_token(cache, dev_tensor(k, dt), dev_tensor(v, dt),
                              torch.from_numpy(hs).cuda())
            kf, vf = W.as_f64(k, dt), W.as_f64(v, dt)
            for (b, h), view in views.items():
                oracle.append_kv(view, kf[b:b + 1, h:h + 1], vf[b:b + 1, h:h + 1], hs[b:b + 1])
        if s % CHECK_EVERY.get(name, 1) != CHECK_EVERY.get(name, 1) - 1 and s != 0:
            continue
        ex = cache.export() if wl.appends is not None else ex
        q = wl.queries[s % len(wl.queries)]
        say(f"[full {name}] decode step {s}")
        out, sels = decode_gpu(cache, q, tau, k_max)
        qf = oracle.from_stored(q, dt)
        # every unit's selection against the oracle's routing
        for b in range(B):
            ns = int(ex["n_spans"][b])
            for h in range(Hkv):
                srows = oracle.from_stored(ex["summary"][b, h, :ns], dt)
                Ph = None if P is None else (P[0] if P.shape[0] == 1 else P[h])
                rt = oracle.route_unit(srows, qf[b, h * G:(h + 1) * G], tau, k_max, alpha, Ph)
                excused += check_selection(rt, sels[b][h], tau, k_max,
                                           f"{name} step {s} unit {(b, h)}")
        # streamed state of every unit: tables exact, then outputs
        for (b, h), view in views.items():
            ns = int(view["n_s"][0])
            assert ex["n_spans"][b] == ns and ex["n_full"][b] == view["n_F"][0], (name, s, b)
            assert ex["last_anchor"][b] == view["la"][0], (name, s, b)
            assert np.array_equal(ex["span_len"][b, :ns], view["span_len"][0, :ns]), (name, s, b)
            assert np.array_equal(ex["full_pos"][b], view["fr_pos"][0]), (name, s, b)
        for (b, h), view in views.items():
            Pu = None if P is None else (P[0:1] if P.shape[0] == 1 else P[h:h + 1])
            ref = oracle.decode_step(view, qf[b:b + 1, h * G:(h + 1) * G], tau, k_max, alpha, Pu,
                                     forced_sel=[[sels[b][h]]])
            err = float(np.max(np.abs(out[b, h * G:(h + 1) * G] - ref["out"][0])))
            worst = max(worst, err)
            assert err <= TOL[dt], f"{name} step {s} unit {(b, h)}: max abs err {err:.3e}"
    say(f"[full {name}] max abs err {worst:.3e} over all {len(units)} units, "
        f"excused selections {excused}")
    cache.close()

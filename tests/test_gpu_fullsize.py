"""Full-size parity (GPU): every workload at its real shape, decoded by the
library in its default launch configuration (the one bench.py times).

Selections of every (sequence, KV head) unit are compared with the oracle's
routing on the stored summaries (exact outside the 1e-5 ambiguity band);
outputs of sampled units with the oracle's decode of those units on the
same stored cache (GPU selection forced where the band excuses a
difference), within 1e-2 max-abs for bf16 caches.  The oracle converts and
decodes only the sampled units, so the check stays within seconds at a
million tokens.
"""
import numpy as np
import pytest

import oracle
from gpu_helpers import TOL, check_selection, decode_gpu, dev_tensor, gpu_build, say, unit_view
from routed_sparse_kv_amd import workloads as W

pytestmark = pytest.mark.gpu

# workload -> decode steps checked (appends run before every step)
STEPS = {"gqa_32k_bf16": 3, "long_128k_bf16": 2, "serving_b16_bf16": 32, "million_1m_bf16": 2}
# steps whose decode is checked when not all are (serving: 32 appends with
# their surprisal, so decoded anchors close spans; decode checked every 8th)
CHECK_EVERY = {"serving_b16_bf16": 8}


def _sampled_units(B, Hkv, seed):
    rng = np.random.default_rng(seed)
    u = {(0, 0), (B - 1, Hkv - 1), (int(rng.integers(B)), int(rng.integers(Hkv)))}
    return sorted(u)


@pytest.mark.timeout(900)
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
    units = _sampled_units(B, Hkv, cfg["seed"])
    if wl.append_h is not None:
        # also sample the sequence with the most decoded anchors
        n_anc = [sum(float(h[b]) > float(ex["theta"][b]) for h in wl.append_h[:STEPS[name]])
                 for b in range(B)]
        units = sorted(set(units) | {(int(np.argmax(n_anc)), Hkv // 2)})
        say(f"[full {name}] decoded anchors per sequence: {n_anc}")
    views = {u: unit_view(ex, *u) for u in units}
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
        # sampled units' streamed state: tables exact, then outputs
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
    say(f"[full {name}] max abs err {worst:.3e} over units {units}, excused selections {excused}")
    cache.close()

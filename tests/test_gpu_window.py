"""Window-routed three-tier cache on the GPU against the oracle (GPU).

Each case builds the cache on the GPU from a seeded workload and runs a
sequence of decode steps, unit by unit beside oracle.qevict on the same
stored K/V and queries.  After every step:
  * the output is within 1e-5 (fp32) / 1e-2 (bf16) max-abs of the oracle's
    attention over the same tiers;
  * on routing events: the masses agree to a relative 1e-5 (fp32 softmax
    statistics against fp64); the new tiers are exact, except windows whose
    oracle scores lie within the relative band of a window across a tier
    boundary (both orders are correct; counted, and the oracle then follows
    the GPU's tiers); evicted windows stay evicted; the tier counts are the
    budget's; the ledger flags match, and every ledger entry (codes, scales,
    minima) is bit-exact;
  * at the end of a case, the full-precision store (promoted windows
    included) is bit-exact.
Sizes span many windows with a ragged last one; the cases cover fp32 / bf16,
d = 64 / 128, query groups of 1 to 16, a budget holding every window at full
precision, an INT2-only budget, a single surviving window, routing at every
step (promotions and re-demotions), a context shorter than one window and
the 128K-token workload at full size (sampled units).
"""
import numpy as np
import pytest

from gpu_helpers import TOL, dev_tensor, say
from oracle import qevict as Q
from oracle.sekv import from_stored
from routed_sparse_kv_amd import workloads as W

pytestmark = pytest.mark.gpu

BAND = Q.MASS_BAND

# case -> (workload, overrides, (budget, full_share) or explicit (n_full, n_quant), R, steps)
CASES = {
    "f32_g1_d64": ("tiny_fp32_2k", dict(T=2048 + 17, steps=6), dict(budget=(0.2, 0.5)), 2, 6),
    "bf16_g4_d128": ("gqa_32k_bf16", dict(B=1, Hq=8, Hkv=2, T=4096 + 37, steps=7),
                     dict(budget=(0.2, 0.5)), 3, 7),
    "f32_g3_d128": ("gqa_32k_bf16", dict(B=1, Hq=3, Hkv=1, T=3000, dtype="f32", steps=5),
                    dict(budget=(0.3, 0.4)), 2, 5),
    "bf16_g7_serving": ("serving_b16_bf16", dict(B=2, T=3100, steps=4), dict(budget=(0.2, 0.5)),
                        2, 4),
    "bf16_d64_clustered": ("long_128k_bf16", dict(B=1, Hq=4, Hkv=2, d=64, T=5000, steps=5),
                           dict(budget=(0.1, 0.5)), 2, 5),
    # edge cases
    "full_budget": ("gqa_32k_bf16", dict(B=1, Hq=4, Hkv=1, T=1000, steps=3), dict(counts=(100, 0)),
                    1, 3),
    "int2_only": ("gqa_32k_bf16", dict(B=1, Hq=4, Hkv=1, T=2000, steps=4), dict(counts=(0, 20)), 2,
                  4),
    "single_window": ("tiny_fp32_2k", dict(T=700, steps=3), dict(counts=(1, 0)), 1, 3),
    "route_every_step": ("gqa_32k_bf16", dict(B=1, Hq=8, Hkv=2, T=1500, steps=10),
                         dict(counts=(3, 6)), 1, 10),
    "short_context": ("tiny_fp32_2k", dict(T=40, Hq=2, steps=3), dict(counts=(0, 1)), 1, 3),
    # the largest query group the kernels take (16 heads per KV head)
    "bf16_g16": ("gqa_32k_bf16", dict(B=1, Hq=16, Hkv=1, T=1500, steps=3), dict(counts=(5, 10)), 1,
                 3),
    "f32_g16": ("tiny_fp32_2k", dict(Hq=16, T=1100, steps=3), dict(counts=(4, 6)), 1, 3),
    # every window holds the same K/V: all masses tie exactly and the
    # ranking falls back to the window index
    "tied_windows": ("gqa_32k_bf16", dict(B=1, Hq=4, Hkv=1, T=1024, steps=3), dict(counts=(4, 5),
                                                                                  tile=64), 1, 3),
}


def tiers_for(cfg, spec):
    if "counts" in spec:
        return spec["counts"]
    budget, share = spec["budget"]
    return W.window_tiers(cfg["T"], cfg["d"], cfg["dtype"], budget, share)


def validate_tiers(new, old, scores, n_full, n_quant, what):
    """GPU tiers against the oracle's new scores: evicted windows stay
    evicted, the counts are the budget's, and no window sits in a lower tier
    than a window with a clearly smaller score.  Returns the number of
    windows placed differently from the strict ranking (ties within BAND)."""
    live = np.flatnonzero(old != Q.EVICTED)
    assert (new[old == Q.EVICTED] == Q.EVICTED).all(), f"{what}: an evicted window came back"
    nf = min(n_full, len(live))
    nq = min(n_quant, len(live) - nf)
    assert (new == Q.FULL).sum() == nf and (new == Q.QUANT).sum() == nq, f"{what}: tier counts"
    rank = {Q.FULL: 0, Q.QUANT: 1, Q.EVICTED: 2}
    s = scores[live]
    t = np.array([rank[int(x)] for x in new[live]])
    for a in range(3):
        for b in range(a + 1, 3):
            hi, lo = s[t == a], s[t == b]
            if hi.size and lo.size:
                worst = hi.min() - lo.max()
                scale = max(abs(hi.min()), abs(lo.max()), 1e-300)
                assert worst >= -BAND * scale, f"{what}: tier {a} holds a score {worst:.3e} below tier {b}"
    order = live[np.lexsort((live, -scores[live]))]
    strict = np.full(len(new), Q.EVICTED)
    strict[order[:nf]] = Q.FULL
    strict[order[nf:nf + nq]] = Q.QUANT
    return int((strict != new).sum())


def run_case(wl, n_full, n_quant, R, steps, units=None, check_store=True):
    import torch

    import routed_sparse_kv_amd as rskv
    cfg = wl.cfg
    dt = cfg["dtype"]
    B, Hq, Hkv, d, T = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["d"], cfg["T"]
    G = Hq // Hkv
    U = B * Hkv
    units = list(range(U)) if units is None else units
    Kd, Vd = dev_tensor(wl.K, dt), dev_tensor(wl.V, dt)
    cache = rskv.build_window(Kd, Vd, Hq, n_full, n_quant, R)
    del Kd, Vd
    st = {u: Q.new_unit(from_stored(wl.K[u // Hkv, u % Hkv], dt), from_stored(wl.V[u // Hkv, u % Hkv], dt),
                        64) for u in units}
    excused = 0
    worst = 0.0
    for step in range(steps):
        qn = wl.queries[step % len(wl.queries)]
        q = dev_tensor(qn, dt)
        out = cache.decode(q).cpu().numpy()
        q64 = from_stored(qn, dt)
        event = step % R == 0
        gs = cache.state(ledger=event, store=False)
        for u in units:
            b, h = divmod(u, Hkv)
            o_out, o_mass = Q.attend_unit(st[u], q64[b, h * G:(h + 1) * G], 64)
            err = float(np.max(np.abs(out[b, h * G:(h + 1) * G] - o_out)))
            worst = max(worst, err)
            assert err <= TOL[dt], f"step {step} unit {u}: output error {err:.3e}"
            if not event:
                continue
            gm = gs["mass"][u]
            merr = np.abs(gm - o_mass) / np.maximum(np.abs(o_mass), 1e-30)
            assert (merr <= 1e-5).all(), f"step {step} unit {u}: mass error {merr.max():.3e}"
            old = st[u]["tier"].copy()
            new = gs["tier"][u].astype(np.int64)
            excused += validate_tiers(new, old, st[u]["score"] + o_mass, n_full, n_quant,
                                      f"step {step} unit {u}")
            Q.route_unit(st[u], o_mass, n_full, n_quant, 64, dt, forced=new)
            gsc = gs["score"][u]
            assert np.allclose(gsc, st[u]["score"], rtol=1e-5, atol=1e-30), f"unit {u}: scores"
            has = np.array([j in st[u]["ledger"] for j in range(len(new))])
            assert np.array_equal(gs["has_code"][u].astype(bool), has), f"step {step} unit {u}: ledger flags"
            for j in np.flatnonzero(has):
                ck, sk, mk, cv, sv, mv = st[u]["ledger"][j]
                n = ck.shape[0]
                for name, o_arr in (("code_k", ck), ("scale_k", sk), ("min_k", mk), ("code_v", cv),
                                    ("scale_v", sv), ("min_v", mv)):
                    g_arr = gs[name][u, j, :n]
                    assert np.array_equal(g_arr.astype(np.float64), o_arr.astype(np.float64)), \
                        f"step {step} unit {u} window {j}: ledger {name}"
        say(f"  step {step}{' (event)' if event else ''}: max err {worst:.2e}, excused {excused}")
    if check_store:
        gs = cache.state(ledger=False, store=True)
        for u in units:
            gk = from_stored(gs["k"][u, :T], dt)
            gv = from_stored(gs["v"][u, :T], dt)
            for name, g_arr, o_arr in (("keys", gk, st[u]["K"]), ("values", gv, st[u]["V"])):
                bad = np.argwhere(g_arr != o_arr)
                if len(bad):
                    wins = sorted(set(int(r) // 64 for r in bad[:, 0]))
                    r0, c0 = bad[0]
                    raise AssertionError(
                        f"unit {u}: full-precision {name} differ in windows {wins[:10]} "
                        f"(tiers {[int(st[u]['tier'][j]) for j in wins[:10]]}, {len(bad)} values); "
                        f"first at row {r0} col {c0}: gpu {g_arr[r0, c0]!r} oracle {o_arr[r0, c0]!r}")
    info = cache.info
    cache.close()
    torch.cuda.synchronize()
    return worst, excused, info


@pytest.mark.parametrize("case", sorted(CASES))
def test_window_parity(case):
    name, over, spec, R, steps = CASES[case]
    wl = W.generate(name, **over)
    if "tile" in spec:  # repeat the first `tile` positions over the whole context
        t = spec["tile"]
        reps = -(-wl.cfg["T"] // t)
        wl.K[...] = np.tile(wl.K[:, :, :t], (1, 1, reps, 1))[:, :, :wl.cfg["T"]]
        wl.V[...] = np.tile(wl.V[:, :, :t], (1, 1, reps, 1))[:, :, :wl.cfg["T"]]
    n_full, n_quant = tiers_for(wl.cfg, spec)
    say(f"case {case}: T={wl.cfg['T']} d={wl.cfg['d']} G={wl.cfg['Hq'] // wl.cfg['Hkv']} "
        f"n_full={n_full} n_quant={n_quant} R={R}")
    worst, excused, info = run_case(wl, n_full, n_quant, R, steps)
    assert info["step"] == steps
    say(f"case {case}: worst {worst:.2e}, excused {excused}")


def test_window_full_size():
    """The 128K-token workload at full size (B=4, 32q/8kv, d=128, 20 % budget,
    R=4) in the launch configuration the bench times; the oracle follows
    four sampled units through two routing events."""
    wl = W.generate("long_128k_bf16", steps=5)
    p = W.window_params()
    n_full, n_quant = W.window_tiers(wl.cfg["T"], wl.cfg["d"], "bf16", p["budget"], p["full_share"])
    say(f"full size: n_full={n_full} n_quant={n_quant}")
    worst, excused, info = run_case(wl, n_full, n_quant, p["route_every"], 5, units=[0, 9, 18, 31],
                                    check_store=False)
    assert info["next_full"] == n_full and info["next_quant"] == n_quant
    say(f"full size: worst {worst:.2e}, excused {excused}")


def test_window_argument_errors():
    import torch

    import routed_sparse_kv_amd as rskv
    from routed_sparse_kv_amd.binding import RskvError
    K = torch.zeros((1, 1, 100, 64), dtype=torch.float32, device="cuda")
    for bad in (dict(n_full=0, n_quant=0), dict(n_full=-1, n_quant=2), dict(route_every=0)):
        kw = dict(n_full=1, n_quant=1, route_every=1)
        kw.update(bad)
        with pytest.raises(RskvError):
            rskv.build_window(K, K, 1, **kw)
    with pytest.raises(RskvError):
        rskv.build_window(K, K, 17 * 1, 1, 1)  # group above 16 (17 heads on 1 KV head)
    K2 = torch.zeros((1, 1, 100, 96), dtype=torch.float32, device="cuda")
    with pytest.raises(RskvError):
        rskv.build_window(K2, K2, 1, 1, 1)

"""Pins that fix the window-routed (QEvict-form) oracle independently of itself.

Each ``pin_*`` takes the oracle module (oracle.qevict) and raises
AssertionError when it disagrees with something the page or the mathematics
fixes: hand-worked quantiser groups, the nearest-level definition of a
2-bit uniform quantiser enumerated level by level, exact reconstruction of
groups that sit on a representable grid, torch's fp64 attention over the
full cache and over a cache rebuilt level by level, masses summed position
by position, a hand-worked ranking with ties, the permanence of eviction,
the write-once ledger followed through demote / promote / demote, and the
routing-event schedule.  The helpers here rebuild what they need with plain
loops instead of calling the oracle's own.

test_qevict_mutants.py runs the same pins on mutated copies of the oracle.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
import torch
import torch.nn.functional as F

FULL, QUANT, EVICTED = 0, 1, 2


def _f32(x):
    return np.float32(x)


def _bf16(x):
    """bf16 rounding (ties to even) through torch."""
    return torch.tensor(np.asarray(x, np.float64), dtype=torch.float64).to(torch.bfloat16) \
        .to(torch.float64).numpy()


def _levels(group):
    """The four fp32 levels mn + fl(k * scale) of one group, with mn, scale."""
    g = [_f32(v) for v in group]
    mn, mx = min(g), max(g)
    scale = _f32(_f32(mx - mn) / _f32(3.0))
    return [_f32(mn + _f32(_f32(k) * scale)) for k in range(4)], mn, scale


def _nearest_rebuild(X, g):
    """Brute force: every coordinate replaced by the level of its group whose
    exact value mn + k (mx - mn) / 3 is nearest (exact rational arithmetic on
    the fp32 values, ties to the even k as rounding to nearest even does);
    the value is that level's fp32 form mn + fl(k * scale)."""
    X = np.asarray(X, np.float64)
    out = np.zeros_like(X)
    for r in range(X.shape[0]):
        for s in range(0, X.shape[1], g):
            lv, mn, _ = _levels(X[r, s:s + g])
            span = Fraction(float(max(_f32(v) for v in X[r, s:s + g]))) - Fraction(float(mn))
            for c in range(s, s + g):
                x = Fraction(float(_f32(X[r, c])))
                k = 0 if span == 0 else min(3, max(0, round(3 * (x - Fraction(float(mn))) / span)))
                out[r, c] = float(lv[k])
    return out


def _sdpa(q, K, V):
    q = torch.tensor(np.asarray(q, np.float64))
    K = torch.tensor(np.asarray(K, np.float64))
    V = torch.tensor(np.asarray(V, np.float64))
    return F.scaled_dot_product_attention(q[None, :, None, :], K[None, None].expand(1, q.shape[0], -1, -1),
                                          V[None, None].expand(1, q.shape[0], -1, -1))[0, :, 0].numpy()


def _probs(q, K):
    """Softmax probabilities [G][n] by plain loops over positions."""
    d = K.shape[1]
    P = np.zeros((q.shape[0], K.shape[0]))
    for h in range(q.shape[0]):
        lg = [sum(float(q[h, c]) * float(K[i, c]) for c in range(d)) / math.sqrt(d)
              for i in range(K.shape[0])]
        m = max(lg)
        e = [math.exp(v - m) for v in lg]
        s = sum(e)
        P[h] = [v / s for v in e]
    return P


def _close(a, b, tol, what=""):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


def _unit(qe, T, d, w, seed, dtype="f32"):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((T, d))
    V = rng.standard_normal((T, d))
    if dtype == "bf16":
        K, V = _bf16(K), _bf16(V)
    else:
        K = K.astype(np.float32).astype(np.float64)
        V = V.astype(np.float32).astype(np.float64)
    return qe.new_unit(K, V, w), K, V, rng


# ---------------------------------------------------------------- quantiser


def pin_quantize_hand(qe):
    """Hand-worked groups of 4: levels on the integers, a half-way value that
    rounds to the even level, one that rounds down to even, and a scaled
    group."""
    X = np.array([[0.0, 1.0, 2.0, 3.0],
                  [-1.5, 0.0, 0.25, 1.5],
                  [0.0, 0.5, 2.5, 3.0],
                  [2.0, 8.0, 5.0, 6.0]])
    codes, scale, mn = qe.quantize_int2(X, 4)
    assert codes.tolist() == [[0, 1, 2, 3], [0, 2, 2, 3], [0, 0, 2, 3], [0, 3, 2, 2]], codes.tolist()
    assert scale.ravel().tolist() == [1.0, 1.0, 1.0, 2.0], scale.ravel().tolist()
    assert mn.ravel().tolist() == [0.0, -1.5, 0.0, 2.0], mn.ravel().tolist()
    deq = qe.dequantize_int2(codes, scale, mn, 4)
    assert deq.tolist() == [[0, 1, 2, 3], [-1.5, 0.5, 0.5, 1.5], [0, 0, 2, 3], [2, 8, 6, 6]], deq.tolist()


def pin_quantize_constant(qe):
    """A constant group has scale 0, code 0 everywhere and is rebuilt exactly."""
    X = np.full((3, 8), 0.7)
    X[1] = -2.25
    X[2, 4:] = 5.0
    codes, scale, mn = qe.quantize_int2(X, 4)
    assert (codes == 0).all()
    assert (scale == 0).all()
    _close(qe.dequantize_int2(codes, scale, mn, 4), X.astype(np.float32), 0.0, "constant groups")


def pin_quantize_nearest(qe):
    """Each code picks the nearest of its group's four levels (random data,
    where ties have probability zero), the levels span [min, max] and every
    coordinate is within half a step of its level."""
    rng = np.random.default_rng(11)
    X = rng.standard_normal((9, 128)) * rng.uniform(0.1, 3.0, (9, 1))
    codes, scale, mn = qe.quantize_int2(X, 64)
    assert codes.dtype == np.uint8 and codes.min() >= 0 and codes.max() <= 3
    deq = qe.dequantize_int2(codes, scale, mn, 64)
    _close(deq, _nearest_rebuild(X, 64), 0.0, "nearest level")
    for r in range(9):
        for s in (0, 64):
            lv, m0, sc = _levels(X[r, s:s + 64])
            assert mn[r, s // 64] == m0 and scale[r, s // 64] == sc
            assert (np.abs(X[r, s:s + 64].astype(np.float32) - deq[r, s:s + 64])
                    <= float(sc) / 2 * (1 + 1e-6)).all()


def pin_dequantize_grid(qe):
    """Groups already on a grid mn + k * 2^-e (k in 0..3, all four present)
    are rebuilt exactly."""
    rng = np.random.default_rng(5)
    X = np.zeros((6, 64))
    for r in range(6):
        m0, step = float(rng.integers(-40, 40)) / 8.0, 2.0 ** -int(rng.integers(0, 6))
        ks = np.concatenate([np.arange(4), rng.integers(0, 4, 60)])
        X[r] = m0 + step * ks[rng.permutation(64)]
    codes, scale, mn = qe.quantize_int2(X, 64)
    _close(qe.dequantize_int2(codes, scale, mn, 64), X, 0.0, "grid groups")


# ---------------------------------------------------------------- attention


def pin_windows(qe):
    """Window counts round up; the last window of a ragged context is short."""
    assert [qe.window_count(T, 64) for T in (1, 64, 65, 128, 130)] == [1, 1, 2, 2, 3]
    st, K, V, rng = _unit(qe, 130, 16, 64, 3)
    assert len(st["tier"]) == 3 and (st["tier"] == FULL).all()
    q = rng.standard_normal((2, 16))
    _, mass = qe.attend_unit(st, q, 8)
    P = _probs(q, K)
    _close(mass, [P[:, :64].sum(), P[:, 64:128].sum(), P[:, 128:].sum()], 1e-12, "window masses")


def pin_attend_full(qe):
    """With every window at full precision the step is dense attention, and
    the masses of the G heads add up to G."""
    st, K, V, rng = _unit(qe, 200, 32, 64, 4)
    q = rng.standard_normal((3, 32)) * 0.7
    out, mass = qe.attend_unit(st, q, 16)
    _close(out, _sdpa(q, K, V), 1e-12, "all-full attention")
    _close(mass.sum(), 3.0, 1e-12, "mass total")
    P = _probs(q, K)
    _close(mass, [P[:, j * 64:(j + 1) * 64].sum() for j in range(4)], 1e-12, "masses")


def pin_attend_quant(qe):
    """With every window INT2 the step is dense attention over the cache
    rebuilt level by level (K and V alike)."""
    st, K, V, rng = _unit(qe, 192, 64, 64, 6)
    nW = 3
    qe.route_unit(st, np.zeros(nW), 0, nW, 64, "f32")
    assert (st["tier"] == QUANT).all()
    q = rng.standard_normal((2, 64))
    out, mass = qe.attend_unit(st, q, 64)
    Kq, Vq = _nearest_rebuild(K, 64), _nearest_rebuild(V, 64)
    _close(out, _sdpa(q, Kq, Vq), 1e-12, "all-INT2 attention")
    P = _probs(q, Kq)
    _close(mass, [P[:, j * 64:(j + 1) * 64].sum() for j in range(nW)], 1e-12, "INT2 masses")


def pin_attend_mixed(qe):
    """Full, INT2 and evicted windows together: evicted positions are left
    out of the softmax and get no mass."""
    st, K, V, rng = _unit(qe, 256, 64, 64, 7)
    qe.route_unit(st, np.array([0.4, 0.1, 0.3, 0.2]), 1, 2, 64, "f32")
    assert st["tier"].tolist() == [FULL, EVICTED, QUANT, QUANT]
    q = rng.standard_normal((2, 64))
    out, mass = qe.attend_unit(st, q, 64)
    Kr = np.concatenate([K[:64], _nearest_rebuild(K[128:], 64)])
    Vr = np.concatenate([V[:64], _nearest_rebuild(V[128:], 64)])
    _close(out, _sdpa(q, Kr, Vr), 1e-12, "mixed attention")
    P = _probs(q, Kr)
    _close(mass, [P[:, :64].sum(), 0.0, P[:, 64:128].sum(), P[:, 128:].sum()], 1e-12, "mixed masses")


# ---------------------------------------------------------------- routing


def pin_route_hand(qe):
    """Hand-worked ranking: scores 0.1 0.5 0.5 0.2 0 0.3 with two full and
    two INT2 slots give full {1, 2} (tie to the lower window), INT2 {5, 3},
    evicted {0, 4}.  Scores accumulate over events; an evicted window stays
    evicted whatever mass it is later credited with."""
    st, K, V, _ = _unit(qe, 6 * 8, 8, 8, 8)
    new = qe.route_unit(st, np.array([0.1, 0.5, 0.5, 0.2, 0.0, 0.3]), 2, 2, 8, "f32")
    assert new.tolist() == [EVICTED, FULL, FULL, QUANT, EVICTED, QUANT], new.tolist()
    _close(st["score"], [0.1, 0.5, 0.5, 0.2, 0.0, 0.3], 0.0, "scores")
    new = qe.route_unit(st, np.array([5.0, 0.0, 0.0, 0.45, 9.0, 0.0]), 2, 2, 8, "f32")
    assert new.tolist() == [EVICTED, FULL, QUANT, FULL, EVICTED, QUANT], new.tolist()
    _close(st["score"], [5.1, 0.5, 0.5, 0.65, 9.0, 0.3], 1e-15, "cumulative scores")
    new = qe.route_unit(st, np.zeros(6), 1, 1, 8, "f32")
    assert new.tolist() == [EVICTED, QUANT, EVICTED, FULL, EVICTED, EVICTED], new.tolist()


def pin_route_brute(qe):
    """Random tie-heavy scores over several events: each event's tiers equal
    the brute-force definition (a live window's rank = the live windows with
    a larger cumulative score, or an equal one and a lower index; ranks
    below n_full full, the next n_quant INT2, the rest evicted; evicted
    windows stay evicted)."""
    rng = np.random.default_rng(21)
    for trial in range(6):
        nW = int(rng.integers(3, 12))
        st, K, V, _ = _unit(qe, nW * 4, 4, 4, 100 + trial)
        nf, nq = int(rng.integers(0, nW)), int(rng.integers(0, nW))
        if nf + nq == 0:
            nf = 1
        total = np.zeros(nW)
        tiers = np.zeros(nW, np.int64)
        for ev in range(4):
            mass = rng.integers(0, 3, nW) * 0.25  # many exact ties
            mass[tiers == EVICTED] = 0.0
            total = total + mass
            live = [j for j in range(nW) if tiers[j] != EVICTED]
            want = np.full(nW, EVICTED)
            for j in live:
                rank = sum(1 for i in live if total[i] > total[j] or (total[i] == total[j] and i < j))
                want[j] = FULL if rank < nf else QUANT if rank < nf + nq else EVICTED
            got = qe.route_unit(st, mass, nf, nq, 4, "f32")
            assert got.tolist() == want.tolist(), (trial, ev, got.tolist(), want.tolist())
            tiers = want


def pin_write_once(qe):
    """Demote, promote, demote: the ledger keeps the codes of the first
    demotion (taken from the prefilled values), promotion writes the
    dequantised values rounded to the cache dtype, and the second demotion
    quantises nothing again."""
    st, K, V, _ = _unit(qe, 128, 64, 64, 9, "bf16")
    qe.route_unit(st, np.array([1.0, 0.0]), 1, 1, 64, "bf16")
    assert st["tier"].tolist() == [FULL, QUANT]
    first = [np.array(a).copy() for a in st["ledger"][1]]
    _close(qe.dequantize_int2(first[0], first[1], first[2], 64), _nearest_rebuild(K[64:], 64), 0.0,
           "ledger K from the prefilled values")
    _close(qe.dequantize_int2(first[3], first[4], first[5], 64), _nearest_rebuild(V[64:], 64), 0.0,
           "ledger V from the prefilled values")
    qe.route_unit(st, np.array([0.0, 2.0]), 1, 1, 64, "bf16")
    assert st["tier"].tolist() == [QUANT, FULL]
    _close(st["K"][64:], _bf16(_nearest_rebuild(K[64:], 64)), 0.0, "promoted K")
    _close(st["V"][64:], _bf16(_nearest_rebuild(V[64:], 64)), 0.0, "promoted V")
    _close(st["K"][:64], K[:64], 0.0, "window 0 full values kept")
    # whatever the full store holds when the window is demoted again, the
    # ledger is not rewritten
    st["K"][64:] = st["K"][64:] * 2.0 + 1.0
    st["V"][64:] = -st["V"][64:]
    qe.route_unit(st, np.array([5.0, 0.0]), 1, 1, 64, "bf16")
    assert st["tier"].tolist() == [FULL, QUANT]
    for a, b in zip(first, st["ledger"][1]):
        assert np.array_equal(a, b), "ledger rewritten at a later demotion"
    _close(st["K"][:64], _bf16(_nearest_rebuild(K[:64], 64)), 0.0, "window 0 promoted")


def pin_schedule(qe):
    """Routing events at steps 0, R, 2R: scores change only there, by the
    masses of the step's own attention."""
    st, K, V, rng = _unit(qe, 320, 16, 64, 10)
    R = 3
    for step in range(7):
        q = rng.standard_normal((2, 16))
        before = st["score"].copy()
        tiers = st["tier"].copy()
        out, mass, event = qe.decode_unit(st, q, step, R, 2, 2, 16, "f32")
        assert event == (step in (0, 3, 6)), (step, event)
        if event:
            _close(st["score"] - before, mass, 1e-15, f"score update at step {step}")
        else:
            _close(st["score"], before, 0.0, f"scores at step {step}")
            assert np.array_equal(st["tier"], tiers)
    assert (st["tier"] == FULL).sum() == 2 and (st["tier"] == QUANT).sum() == 2


def pin_full_budget(qe):
    """A budget that holds every window at full precision keeps the cache
    exact: every step is dense attention and nothing is quantised."""
    st, K, V, rng = _unit(qe, 150, 32, 64, 12)
    for step in range(5):
        q = rng.standard_normal((2, 32))
        out, _, _ = qe.decode_unit(st, q, step, 2, 3, 1, 16, "f32")
        _close(out, _sdpa(q, K, V), 1e-12, f"step {step}")
    assert not st["ledger"]


ALL_PINS = [pin_quantize_hand, pin_quantize_constant, pin_quantize_nearest, pin_dequantize_grid,
            pin_windows, pin_attend_full, pin_attend_quant, pin_attend_mixed, pin_route_hand,
            pin_route_brute, pin_write_once, pin_schedule, pin_full_budget]

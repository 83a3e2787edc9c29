"""Streaming segmentation on the GPU against the oracle (GPU).

A cache is built on the GPU; its export (checked against the oracle's own
build in the parity tests) seeds the oracle's state.  Tokens are then
appended with surprisal values chosen to make some of them anchors, ties
with the threshold included.  After every append the GPU cache's export is
compared with the oracle's state after the same append (oracle.append_kv):
the integer tables (span count, starts, lengths, token count, span ids,
full-resolution count and positions, last anchor), the full-resolution rows
and their surprisal bit-exactly; the summaries and value means of the new
spans within one storage ulp; their factors through their products (the
SVD basis is unique only up to sign).  A decode step on the GPU cache is
then compared with the oracle's decode of its export, as in the parity
tests.
"""
import math

import numpy as np
import pytest

import oracle
from gpu_helpers import compare_decode, decode_gpu, dev_tensor, gpu_build, oracle_view, say
from routed_sparse_kv_amd import workloads as W

pytestmark = pytest.mark.gpu

# Per-sequence patterns, one character per append:
#   a  anchor (surprisal 2 theta + 1),  b  below the threshold (theta / 2),
#   t  exactly the threshold (not an anchor: the comparison is strict),
#   w  the workload's own draw,  n  the whole step appends without surprisal.
CASES = {
    # bf16, d = 128: a run of 63 rows closes through the global Jacobi slab
    "bf16_d128": ("serving_b16_bf16", dict(B=3, T=2053, tail_capacity=72, steps=72),
                  ["a" + "b" * 62 + "abtbaa" + "bab",
                   "w" * 72,
                   "bbaab" + "n" + "tbabbbtaab" + "b" * 40 + "a" + "b" * 15]),
    # fp32, d = 64, one sequence
    "f32_d64": ("tiny_fp32_2k", dict(tail_capacity=14, steps=14, append=True),
                ["abbaabtbabnbba"]),
}


def _fix_none_steps(patterns):
    """A step marked n in one sequence appends without surprisal for all."""
    steps = len(patterns[0])
    none = [any(p[s] == "n" for p in patterns) for s in range(steps)]
    return [["n" if none[s] else p[s] for s in range(steps)] for p in patterns], none


def _h_values(pattern, theta, drawn):
    h = np.zeros(len(pattern), np.float32)
    for b, ch in enumerate(pattern):
        th = float(theta[b])
        h[b] = {"a": 2 * th + 1, "b": th / 2, "t": th, "w": drawn[b], "n": 0.0}[ch]
    return h


def _ulps(a, b, dtype):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    mant = 8 if dtype == "bf16" else 24
    _, e = np.frexp(np.where(b == 0, 1.0, np.abs(b)))
    return np.abs(a - b) / np.ldexp(1.0, e - mant)


def _check_build_state(wl, ex):
    """Threshold, last-anchor row and row surprisal of the GPU build."""
    n_a = oracle.n_anchors(wl.cfg["T"], wl.cfg["anchor_frac"])
    for b in range(wl.cfg["B"]):
        sg = oracle.segment(wl.H[b], n_a)
        anchors = np.flatnonzero(sg["span_id"] == -1)
        nf = len(sg["fr_pos"])
        if len(anchors):
            assert ex["theta"][b] == wl.H[b, anchors].min()
            assert ex["last_anchor"][b] == np.searchsorted(sg["fr_pos"], anchors[-1])
        else:
            assert np.isinf(ex["theta"][b]) and ex["theta"][b] > 0
            assert ex["last_anchor"][b] == -1
        assert np.array_equal(ex["h_full"][b, :nf], wl.H[b, sg["fr_pos"]])
        assert (ex["h_full"][b, nf:] == 0).all()


def _compare_state(ex, ref, ns0, closed_x, dt, rank, what):
    """GPU export against the oracle's streamed state (see module doc)."""
    B, Hkv = ref["B"], ref["Hkv"]
    conv = {}

    def f(k):
        if k not in conv:
            conv[k] = oracle.from_stored(ex[k], dt)
        return conv[k]

    for b in range(B):
        ns, nf = int(ref["n_s"][b]), int(ref["n_F"][b])
        assert ex["n_spans"][b] == ns, f"{what} b={b}: n_spans {ex['n_spans'][b]} != {ns}"
        assert ex["n_full"][b] == nf, f"{what} b={b}: n_full"
        assert ex["n_span_tokens"][b] == ref["nt"][b], f"{what} b={b}: n_span_tokens"
        assert ex["last_anchor"][b] == ref["la"][b], f"{what} b={b}: last_anchor"
        assert np.array_equal(ex["span_start"][b, :ns], ref["span_start"][b, :ns]), what
        assert np.array_equal(ex["span_len"][b, :ns], ref["span_len"][b, :ns]), what
        assert np.array_equal(ex["span_id"][b], ref["span_id"][b]), f"{what} b={b}: span_id"
        assert np.array_equal(ex["full_pos"][b], ref["fr_pos"][b]), f"{what} b={b}: full_pos"
        assert np.array_equal(ex["h_full"][b].astype(np.float64), ref["HF"][b]), what
        assert np.array_equal(ex["log_len"][b, :ns].astype(np.float64), ref["ell"][b, :ns]), what
    assert np.array_equal(f("k_full"), ref["KF"]), f"{what}: full-resolution keys"
    assert np.array_equal(f("v_full"), ref["VF"]), f"{what}: full-resolution values"
    s_gpu, v_gpu = f("summary"), f("vmean")
    for b in range(B):
        ns = int(ref["n_s"][b])
        # spans that existed before the appends are untouched
        assert np.array_equal(s_gpu[b, :, :ns0[b]], ref["s"][b, :, :ns0[b]]), what
        if ns > ns0[b]:
            assert _ulps(s_gpu[b, :, ns0[b]:ns], ref["s"][b, :, ns0[b]:ns], dt).max() <= 1.0, \
                f"{what} b={b}: summary of a closed span"
            assert _ulps(v_gpu[b, :, ns0[b]:ns], ref["vbar"][b, :, ns0[b]:ns], dt).max() <= 1.0, \
                f"{what} b={b}: value mean of a closed span"
    rel = 2e-6 if dt == "f32" else 3 * 2.0 ** -8
    for (b, j), (xk, xv, off) in closed_x.items():
        ln = xk.shape[1]
        for h in range(Hkv):
            for X, akey, wkey, ak, wk in ((xk[h], "a_k", "w_k", "AK", "BK"),
                                          (xv[h], "a_v", "w_v", "AV", "BV")):
                P_gpu = f(akey)[b, h, off:off + ln] @ f(wkey)[b, h, j]
                P_ref = ref[ak][b, h, off:off + ln] @ ref[wk][b, h, j]
                sig = np.linalg.svd(X, compute_uv=False)
                rj = min(rank, ln, X.shape[1])
                gap = (sig[rj - 1] - sig[rj]) / sig[0] if rj < len(sig) else 1.0
                if sig[0] == 0 or gap < 1e-6:
                    continue  # truncation not unique
                nx = np.linalg.norm(X)
                err = np.linalg.norm(P_gpu - P_ref) / nx
                assert err <= rel * math.sqrt(rank), f"{what} span {(b, j)}: product err {err:.2e}"


def _run_stream(wl, patterns, decode_every=1):
    import torch

    import routed_sparse_kv_amd as rskv
    cfg = wl.cfg
    dt = wl.dtype
    cache = gpu_build(wl)
    ex = cache.export()
    _check_build_state(wl, ex)
    ref = oracle_view(ex)
    ns0 = ref["n_s"].copy()
    pats, none = _fix_none_steps(patterns)
    closed_x, n_closed = {}, 0
    steps = len(pats[0])
    for s in range(steps):
        k, v = wl.appends[s]
        kf, vf = W.as_f64(k, dt), W.as_f64(v, dt)
        col = "".join(p[s] for p in pats)
        if none[s]:
            rskv.append_kv(cache, dev_tensor(k, dt), dev_tensor(v, dt))
            h = None
        else:
            h = _h_values(col, ref["theta"], wl.append_h[s])
            rskv.append_token(cache, dev_tensor(k, dt), dev_tensor(v, dt),
                              torch.from_numpy(h).cuda())
        # rows the oracle is about to close, for the factor check
        for b in range(ref["B"]):
            la, nf = int(ref["la"][b]), int(ref["n_F"][b])
            if h is not None and h[b] > ref["theta"][b] and la >= 0 and nf - la - 1 > 0:
                j, off = int(ref["n_s"][b]), int(ref["nt"][b])
                closed_x[(b, j)] = (ref["KF"][b, :, la + 1:nf].copy(),
                                    ref["VF"][b, :, la + 1:nf].copy(), off)
                n_closed += 1
                say(f"  step {s}: sequence {b} closes span {j} of {nf - la - 1} rows")
        oracle.append_kv(ref, kf, vf, h)
        ex = cache.export()
        _compare_state(ex, ref, ns0, closed_x, dt, cfg["rank"], f"step {s} ({col})")
        if s % decode_every == 0 or s == steps - 1:
            q = wl.queries[s % len(wl.queries)]
            out, sels = decode_gpu(cache, q, cfg["tau"], cfg["k_max"])
            compare_decode(oracle_view(ex), q, out, sels, cfg["tau"], cfg["k_max"], cfg["alpha"],
                           wl.P, dt, what=f"step {s}")
    cache.close()
    return n_closed


@pytest.mark.timeout(600)
@pytest.mark.parametrize("case", sorted(CASES))
def test_streaming_segmentation(case):
    name, over, patterns = CASES[case]
    say(f"[stream {case}] generate {name} {over}")
    wl = W.generate(name, **over)
    n_closed = _run_stream(wl, patterns, decode_every=4)
    say(f"[stream {case}] {n_closed} spans closed")
    assert n_closed >= 3


def test_streaming_without_anchors():
    """No prefill anchor: theta is +inf and no decoded token is an anchor."""
    import torch

    import routed_sparse_kv_amd as rskv
    wl = W.generate("tiny_fp32_2k", B=2, T=300, anchor_frac=0.0, tail_capacity=4, steps=4,
                    append=True, query="uniform")
    cache = gpu_build(wl)
    ex = cache.export()
    _check_build_state(wl, ex)
    for s in range(4):
        k, v = wl.appends[s]
        h = torch.full((2,), 1e30, dtype=torch.float32, device="cuda")
        rskv.append_token(cache, dev_tensor(k, "f32"), dev_tensor(v, "f32"), h)
    ex = cache.export()
    assert (ex["n_spans"] == 0).all() and (ex["n_full"] == 304).all()
    assert (ex["last_anchor"] == -1).all()
    assert ex["full_pos"][:, 300:304].tolist() == [[300, 301, 302, 303]] * 2
    cache.close()


def test_streaming_anchor_at_the_end():
    """The prefill ends on an anchor (empty tail run): a first decoded anchor
    closes nothing, the next one closes the decoded tokens between them."""
    wl = W.generate("tiny_fp32_2k", B=2, T=700, tail_capacity=8, steps=8, append=True)
    wl.H[:, -1] = wl.H.max() + 1.0  # the last position becomes an anchor
    n_closed = _run_stream(wl, ["abbbaabt", "bbabbbab"])
    assert n_closed == 3


def _run_patterns(runs_per_seq):
    """Append patterns that close runs of the given lengths in each sequence
    (one anchor first, to close the prefill tail), padded to equal length."""
    pats = ["a" + "".join("b" * n + "a" for n in runs) for runs in runs_per_seq]
    steps = max(len(p) for p in pats)
    return [p + "b" * (steps - len(p)) for p in pats], steps


# Closed runs across the closing kernel's forms: the Gram matrix is X X^T
# (n x n) up to n = d rows and X^T X (d x d) beyond; ranks above 16 take
# the eigenvector tiles of eight lanes per vector.
LONG_RUNS = {
    "bf16_d128": ("serving_b16_bf16", 2, [[128, 150], [64, 1, 2, 17, 100]], {}),
    "f32_d64": ("tiny_fp32_2k", 1, [[64, 90, 5]], {}),
    "bf16_d128_r32": ("serving_b16_bf16", 2, [[40, 128], [33, 70, 150]], {"rank": 32}),
    "f32_d64_r24": ("tiny_fp32_2k", 1, [[48, 90, 20, 12]], {"rank": 24}),
    # two batches of eigenvectors with 16 lanes per vector (12 and 16 kept)
    "bf16_d128_r12": ("serving_b16_bf16", 2, [[40, 128], [33, 70, 150]], {"rank": 12}),
    "bf16_d128_r16": ("serving_b16_bf16", 2, [[40, 128], [33, 70, 150]], {"rank": 16}),
}


@pytest.mark.timeout(900)
@pytest.mark.parametrize("case", sorted(LONG_RUNS))
def test_streaming_long_runs(case):
    name, B, runs, extra = LONG_RUNS[case]
    pats, steps = _run_patterns(runs)
    over = dict(B=B, T=700, tail_capacity=steps + 8, steps=steps, **extra)
    if name == "tiny_fp32_2k":
        over["append"] = True
    say(f"[stream long {case}] {steps} appends closing runs {runs}")
    wl = W.generate(name, **over)
    n_closed = _run_stream(wl, pats, decode_every=64)
    assert n_closed >= sum(len(r) for r in runs)


def test_streaming_equal_singular_values():
    """Runs whose key rows are orthogonal with equal norms (every singular
    value equal): with n <= r the truncation keeps all of them and the
    product must give the rows back; with n > r it is not unique and only
    the tables, summaries and decode are compared."""
    runs = [[6], [12]]
    pats, steps = _run_patterns(runs)
    wl = W.generate("serving_b16_bf16", B=2, T=700, tail_capacity=steps + 8, steps=steps)
    dt = wl.dtype
    # appends 1 .. n of each sequence: key rows 2 e_i in every KV head
    for b, rr in enumerate(runs):
        for i in range(rr[0]):
            k, v = wl.appends[1 + i]
            k = k.copy()
            row = np.zeros(wl.cfg["d"], np.float32)
            row[i] = 2.0
            k[b, :] = W.store(row, dt)
            wl.appends[1 + i] = (k, v)
    n_closed = _run_stream(wl, pats, decode_every=4)
    assert n_closed == 4

"""Helpers for the GPU parity tests: device transfer, export -> oracle view,
selection comparison with the ambiguity band."""
from __future__ import annotations

import sys

import numpy as np

import oracle

TOL = {"f32": 1e-5, "bf16": 1e-2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_tensor(arr, dtype_name, device="cuda"):
    import torch
    if dtype_name == "bf16" and arr.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(arr)).to(device)


def gpu_build(wl, device="cuda", **over):
    import torch

    import routed_sparse_kv_amd as rskv
    cfg = dict(wl.cfg)
    cfg.update(over)
    dt = cfg["dtype"]
    H = torch.from_numpy(wl.H).to(device)
    K = dev_tensor(wl.K, dt, device)
    V = dev_tensor(wl.V, dt, device)
    P = torch.from_numpy(wl.P).to(device) if wl.P is not None else None
    cache = rskv.build_spans(H, K, V, cfg["rank"], cfg["anchor_frac"], n_q_heads=cfg["Hq"],
                             alpha=cfg["alpha"], proj=P, tail_capacity=cfg["tail_capacity"],
                             k_max_cap=cfg.get("k_max_cap", 0),
                             factor_tier=cfg.get("factor_tier", "hbm"))
    del K, V
    return cache


def oracle_view(ex):
    """Canonical export -> the oracle's cache dictionary (fp64 values)."""
    info = ex["info"]
    dt = "bf16" if info["dtype"] == 1 else "f32"
    f = lambda k: oracle.from_stored(ex[k], dt)  # noqa: E731
    return dict(B=info["batch"], Hq=info["n_q_heads"], Hkv=info["n_kv_heads"],
                d=info["head_dim"], T=info["context_len"], rank=info["rank"], dtype=dt,
                tail_capacity=info["tail_capacity"], appended=info["appended"],
                n_s=ex["n_spans"].astype(np.int64), n_F=ex["n_full"].astype(np.int64),
                n_a=ex["n_anchor"].astype(np.int64), nt=ex["n_span_tokens"].astype(np.int64),
                span_id=ex["span_id"], span_start=ex["span_start"].astype(np.int64),
                span_len=ex["span_len"].astype(np.int64), fr_pos=ex["full_pos"].astype(np.int64),
                s=f("summary"), vbar=f("vmean"), ell=ex["log_len"].astype(np.float64),
                KF=f("k_full"), VF=f("v_full"), AK=f("a_k"), AV=f("a_v"), BK=f("w_k"),
                BV=f("w_v"), HF=ex["h_full"].astype(np.float64),
                theta=ex["theta"].astype(np.float64), la=ex["last_anchor"].astype(np.int64))


def unit_view(ex, b, h):
    """Oracle cache dictionary holding the single unit (sequence b, KV head
    h) of a canonical export (B = Hkv = 1; converts only that unit)."""
    info = ex["info"]
    dt = "bf16" if info["dtype"] == 1 else "f32"
    f = lambda k: oracle.from_stored(ex[k][b:b + 1, h:h + 1], dt)  # noqa: E731
    return dict(B=1, Hq=info["n_q_heads"] // info["n_kv_heads"], Hkv=1, d=info["head_dim"],
                T=info["context_len"], rank=info["rank"], dtype=dt,
                tail_capacity=info["tail_capacity"], appended=info["appended"],
                n_s=ex["n_spans"][b:b + 1].astype(np.int64),
                n_F=ex["n_full"][b:b + 1].astype(np.int64).copy(),
                span_len=ex["span_len"][b:b + 1].astype(np.int64),
                fr_pos=ex["full_pos"][b:b + 1].astype(np.int64).copy(),
                s=f("summary"), vbar=f("vmean"), ell=ex["log_len"][b:b + 1].astype(np.float64),
                KF=f("k_full"), VF=f("v_full"), AK=f("a_k"), AV=f("a_v"), BK=f("w_k"),
                BV=f("w_v"), HF=ex["h_full"][b:b + 1].astype(np.float64),
                theta=ex["theta"][b:b + 1].astype(np.float64),
                la=ex["last_anchor"][b:b + 1].astype(np.int64), span_id=ex["span_id"][b:b + 1].copy(),
                span_start=ex["span_start"][b:b + 1].astype(np.int64),
                nt=ex["n_span_tokens"][b:b + 1].astype(np.int64))


def decode_gpu(cache, q_np, tau, k_max, device="cuda"):
    """Returns (out [B][Hq][d] fp64, sel lists [b][h])."""
    import torch

    import routed_sparse_kv_amd as rskv
    i = cache.info
    B, Hkv = i["batch"], i["n_kv_heads"]
    dt = "bf16" if i["dtype"] == 1 else "f32"
    q = dev_tensor(q_np, dt, device)
    sel = torch.full((B, Hkv, k_max), -7, dtype=torch.int32, device=device) if k_max > 0 else None
    nsel = torch.full((B, Hkv), -7, dtype=torch.int32, device=device)
    out = rskv.decode_step(cache, q, tau, k_max, sel=sel, n_sel=nsel)
    torch.cuda.synchronize()
    s = sel.cpu().numpy() if sel is not None else np.zeros((B, Hkv, 0), np.int32)
    n = nsel.cpu().numpy()
    sels = [[s[b, h, :n[b, h]].astype(np.int64) for h in range(Hkv)] for b in range(B)]
    if k_max > 0:
        for b in range(B):
            for h in range(Hkv):
                assert (s[b, h, n[b, h]:k_max] == -1).all(), "sel padding must be -1"
    return out.cpu().numpy().astype(np.float64), sels


def check_selection(rt, gsel, tau, k_max, what=""):
    """GPU selection equals the oracle's, except spans inside the ambiguity
    band (|z - tau| <= band, or tied with the k-th largest within the band).
    Returns the number of excused spans."""
    E = rt["E"]
    if np.array_equal(E, gsel):
        return 0
    z = rt["z"]
    diff = np.setxor1d(E, gsel)
    band = oracle.AMBIGUITY_BAND
    ok = np.abs(z[diff] - tau) <= band
    if rt["rank_tie"] or len(E) == k_max:
        cand = np.flatnonzero(z > tau)
        zs = np.sort(z[cand])[::-1]
        if k_max > 0 and len(zs) >= k_max:
            ok |= np.abs(z[diff] - zs[k_max - 1]) <= band
    assert ok.all(), (f"{what}: selections differ outside the ambiguity band: "
                      f"oracle-only {np.setdiff1d(E, gsel)[:10]}, gpu-only "
                      f"{np.setdiff1d(gsel, E)[:10]}")
    assert len(gsel) == len(E) or k_max == 0, f"{what}: selection sizes differ"
    return int(len(diff))


def compare_decode(oc, q_np, out_gpu, sels, tau, k_max, alpha, P, dtype, units=None, what=""):
    """Oracle decode on the exported cache; selections exact (band aside),
    outputs within the dtype tolerance with the GPU selection forced."""
    q = oracle.from_stored(q_np, dtype)
    res = oracle.decode_step(oc, q, tau, k_max, alpha, P, units=units)
    excused = 0
    for (b, h), rt in res["routes"].items():
        excused += check_selection(rt, sels[b][h], tau, k_max, f"{what} unit {(b, h)}")
    forced = [[sels[b][h] for h in range(oc["Hkv"])] for b in range(oc["B"])]
    ref = oracle.decode_step(oc, q, tau, k_max, alpha, P, forced_sel=forced, units=units)
    G = oc["Hq"] // oc["Hkv"]
    todo = units if units is not None else [(b, h) for b in range(oc["B"]) for h in range(oc["Hkv"])]
    err = 0.0
    for b, h in todo:
        sl = slice(h * G, (h + 1) * G)
        err = max(err, float(np.max(np.abs(out_gpu[b, sl] - ref["out"][b, sl]))))
    assert err <= TOL[dtype], f"{what}: max abs err {err:.3e} > {TOL[dtype]}"
    return err, excused


def ulps(a, b, dtype):
    """Distance of a from b in units of the last stored place of b."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    mant = 8 if dtype == "bf16" else 24
    _, e = np.frexp(np.where(b == 0, 1.0, np.abs(b)))
    ulp = np.ldexp(1.0, e - mant)
    return np.abs(a - b) / ulp


def check_segmentation_tables(ex, H, anchor_frac, what=""):
    """Every sequence's segmentation in a GPU export against oracle.segment
    on the same surprisal, bit-exact: anchor count, span ids, span starts and
    lengths, full-resolution positions, and the streaming state (anchor
    threshold theta = smallest anchor surprisal, full-resolution row of the
    last anchor).  Only build-time tables: call before any append."""
    B, T = H.shape
    n_a = oracle.n_anchors(T, anchor_frac)
    for b in range(B):
        sg = oracle.segment(H[b], n_a)
        ns, nf = len(sg["span_len"]), len(sg["fr_pos"])
        w = f"{what} sequence {b}"
        assert ex["n_anchor"][b] == sg["n_a"], w
        assert ex["n_spans"][b] == ns, w
        assert ex["n_full"][b] == nf, w
        assert ex["n_span_tokens"][b] == int(sg["span_len"].sum()), w
        assert np.array_equal(ex["span_id"][b], sg["span_id"]), w
        assert np.array_equal(ex["span_start"][b, :ns], sg["span_start"]), w
        assert np.array_equal(ex["span_len"][b, :ns], sg["span_len"]), w
        assert np.array_equal(ex["full_pos"][b, :nf], sg["fr_pos"]), w
        assert (ex["full_pos"][b, nf:] == -1).all(), w
        anchors = np.flatnonzero(sg["span_id"] == -1)
        if len(anchors):
            assert ex["theta"][b] == np.float32(H[b, anchors].min()), w
            assert ex["last_anchor"][b] == int(np.searchsorted(sg["fr_pos"], anchors[-1])), w
        else:
            assert np.isinf(ex["theta"][b]) and ex["last_anchor"][b] == -1, w
    return n_a


def check_full_rows(ex, K, V, b, h, what=""):
    """Packed full-resolution rows of unit (b, h) are the input rows at the
    exported positions, bit for bit (stored dtype)."""
    nf = int(ex["n_full"][b])
    pos = ex["full_pos"][b, :nf].astype(np.int64)
    assert np.array_equal(ex["k_full"][b, h, :nf], K[b, h, pos]), f"{what} K rows {(b, h)}"
    assert np.array_equal(ex["v_full"][b, h, :nf], V[b, h, pos]), f"{what} V rows {(b, h)}"


def check_summaries(ex, H, Kf, Vf, b, h, js, dtype, what=""):
    """Summaries and value means of spans js of unit (b, h) within one
    stored ulp of the oracle's (from the same input rows), ln|S| exact.
    Returns the largest distance in ulp."""
    worst = 0.0
    lens = ex["span_len"][b, js].astype(np.float64)
    assert np.array_equal(ex["log_len"][b, js], np.log(lens).astype(np.float32)), what
    s = oracle.from_stored(ex["summary"][b, h, js], dtype)
    vb = oracle.from_stored(ex["vmean"][b, h, js], dtype)
    for i, j in enumerate(js):
        st, ln = int(ex["span_start"][b, j]), int(ex["span_len"][b, j])
        s_ref = oracle.round_stored(oracle.span_summary(H[b, st:st + ln], Kf[st:st + ln]), dtype)
        v_ref = oracle.round_stored(oracle.span_value_mean(Vf[st:st + ln]), dtype)
        worst = max(worst, ulps(s[i], s_ref, dtype).max(), ulps(vb[i], v_ref, dtype).max())
    assert worst <= 1.0, f"{what} unit {(b, h)}: summaries differ by {worst} ulp"
    return worst


def check_factor_products(ex, Kf, Vf, b, h, js, dtype, rank, what=""):
    """A W of spans js of unit (b, h) against the oracle's factors of the
    same input rows (relative Frobenius error bounded by the storage
    rounding of A and W), and the Eckart-Young residual.  Spans whose
    rank-r truncation is not unique (sigma_r = sigma_{r+1} to 1e-6) are
    skipped.  Returns the number of spans checked."""
    rel = 2e-6 if dtype == "f32" else 3 * 2.0 ** -8
    ns = int(ex["n_spans"][b])
    offs = np.concatenate([[0], np.cumsum(ex["span_len"][b, :ns].astype(np.int64))])
    checked = 0
    for j in js:
        st, ln = int(ex["span_start"][b, j]), int(ex["span_len"][b, j])
        for X, akey, wkey in ((Kf[st:st + ln], "a_k", "w_k"), (Vf[st:st + ln], "a_v", "w_v")):
            A = oracle.from_stored(ex[akey][b, h, offs[j]:offs[j + 1]], dtype)
            Wt = oracle.from_stored(ex[wkey][b, h, j], dtype)
            prod = A @ Wt
            sig = np.linalg.svd(X, compute_uv=False)
            rj = min(rank, ln, X.shape[1])
            gap = (sig[rj - 1] - sig[rj]) / sig[0] if rj < len(sig) else 1.0
            if gap < 1e-6:
                continue  # truncation not unique
            Ao, Wo = oracle.truncated_svd(X, rank)
            nx = np.linalg.norm(X)
            err = np.linalg.norm(prod - Ao @ Wo) / nx
            assert err <= rel * np.sqrt(rank), f"{what} unit {(b, h)} span {j}: product err {err:.2e}"
            res = np.linalg.norm(X - prod) ** 2
            assert res <= np.sum(sig[rj:] ** 2) + (2 * rel * nx) ** 2 + 1e-9 * nx ** 2, \
                f"{what} unit {(b, h)} span {j}: residual above Eckart-Young"
            checked += 1
    return checked

"""Plant plausible mistakes in copies of the oracle; some pin must fail.

Each mutation edits one line of the oracle's source text, loads the edited
text as a throw-away module and runs the pins against it.  A mutation that
no pin notices means the pins leave that part of the oracle unchecked.
"""
import os
import types

import pytest

from oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "sekv.py")

MUTATIONS = {
    "drop size bias": ('bias.append(cache["ell"][b, rest].astype(np.float64))',
                       'bias.append(0.0 * cache["ell"][b, rest])'),
    "scale 1/d": ("scale = 1.0 / math.sqrt(d)", "scale = 1.0 / d"),
    "biased mean": ("return V_span.sum(axis=0) / V_span.shape[0]",
                    "return V_span.sum(axis=0) / max(1, V_span.shape[0] - 1)"),
    "tie to higher position": ("order = np.lexsort((np.arange(T), -H.astype(np.float64)))",
                               "order = np.lexsort((-np.arange(T), -H.astype(np.float64)))"),
    "span starts on anchor": ("starts.append(left + 1)", "starts.append(left)"),
    "one anchor short": ("mask[order[:n_a]] = True", "mask[order[:max(0, n_a - 1)]] = True"),
    "lead/tail dropped": ("fr_pos = np.flatnonzero(span_id < 0)",
                          "fr_pos = np.flatnonzero(span_id == -1)"),
    "non-strict gate": ("cand = np.flatnonzero(z > tau)", "cand = np.flatnonzero(z >= tau)"),
    "rank tie to higher j": ("order = np.lexsort((cand, -z[cand]))",
                             "order = np.lexsort((-cand, -z[cand]))"),
    "first query routes": ("qbar = q_group.sum(axis=0) / q_group.shape[0]", "qbar = q_group[0]"),
    "transposed projection": ("rho = np.asarray(P, np.float64) @ qbar",
                              "rho = np.asarray(P, np.float64).T @ qbar"),
    "alpha dropped": ("z = alpha * (np.asarray(s_rows, np.float64) @ rho)",
                      "z = (np.asarray(s_rows, np.float64) @ rho)"),
    "unweighted summary": ("u = (np.asarray(H_span, np.float64)[:, None] *",
                           "u = (0 * np.asarray(H_span, np.float64)[:, None] + 1 *"),
    "summary not normalised": ("    return u / n", "    return u"),
    "wrong factor operand": ('keys.append(cache["AK"][b, h, rows] @ cache["BK"][b, h, j])',
                             'keys.append(cache["AV"][b, h, rows] @ cache["BK"][b, h, j])'),
    "singular values dropped": ("A[:, :rj] = U[:, :rj] * S[:rj]", "A[:, :rj] = U[:, :rj]"),
    "rank one short": ("rj = min(r, n, d)", "rj = max(1, min(r, n, d) - 1)"),
    "expanded spans also summarised": ("rest = np.flatnonzero(~expanded)", "rest = np.arange(ns)"),
    "bf16 ties away": ("half = np.uint64((1 << 44) - 1)", "half = np.uint64(1 << 44)"),
    "append invisible": ('cache["n_F"][b] = i + 1', 'cache["n_F"][b] = i'),
    "streaming anchor at the threshold": ('anchor = h is not None and hb > cache["theta"][b]',
                                          'anchor = h is not None and hb >= cache["theta"][b]'),
    "threshold from the strongest anchor": ('c["theta"][b] = float(H[b, anchors].min())',
                                            'c["theta"][b] = float(H[b, anchors].max())'),
    "closed span keeps the anchor": ("    rows = slice(la + 1, nf)\n    st = int(cache[\"fr_pos\"][b, la + 1])",
                                     "    rows = slice(la, nf)\n    st = int(cache[\"fr_pos\"][b, la])"),
    "new anchor forgotten": ('            cache["la"][b] = i\n', '            cache["la"][b] = i - 1\n'),
}


def _mutant(old, new):
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation anchor not found once: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(text.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutant_is_caught(name):
    mod = _mutant(*MUTATIONS[name])
    caught = []
    for pin in ALL_PINS:
        try:
            pin(mod)
        except Exception:  # AssertionError or a crash both count
            caught.append(pin.__name__)
            break
    assert caught, f"no pin notices mutation {name!r}"

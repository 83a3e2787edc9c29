"""Plant plausible mistakes in copies of the window-routed oracle; a pin must fail.

Each mutation edits one passage of oracle/qevict.py's source text, loads the
edited text as a throw-away module of the oracle package and runs the pins
against it.
"""
import os
import types

import pytest

from qevict_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "qevict.py")

MUTATIONS = {
    "last window dropped": ("return (T + w - 1) // w", "return max(1, T // w)"),
    "scale over four levels": ("scale = (mx - mn) / np.float32(3.0)",
                               "scale = (mx - mn) / np.float32(4.0)"),
    "codes truncated": ("codes = np.rint((Xg - mn[:, :, None])", "codes = np.floor((Xg - mn[:, :, None])"),
    "codes from the max": ("codes = np.rint((Xg - mn[:, :, None]) / safe[:, :, None])",
                           "codes = 3 - np.rint((mx[:, :, None] - Xg) / safe[:, :, None])"),
    "dequantise without offset": ("return (mn[:, :, None] + prod)", "return (0 * mn[:, :, None] + prod)"),
    "dequantise fused in fp64": (
        "prod = (c * scale[:, :, None]).astype(np.float32)",
        "prod = c.astype(np.float64) * scale[:, :, None].astype(np.float64)"),
    "INT2 values not dequantised": ("            V[rows] = dequantize_int2(cv, sv, mv, g)\n", ""),
    "INT2 windows not attended": ("            keep[rows] = True\n    pos", "            pass\n    pos"),
    "logit scale 1/d": ("q_group @ K.T / math.sqrt(K.shape[1])", "q_group @ K.T / K.shape[1]"),
    "mass of the first head only": ("p.sum(axis=0))", "p[0])"),
    "scores not cumulative": ('st["score"] = st["score"] + mass', 'st["score"] = 0 * st["score"] + mass'),
    "ascending scores": ('np.lexsort((live, -st["score"][live]))', 'np.lexsort((live, st["score"][live]))'),
    "ties to the higher window": ('np.lexsort((live, -st["score"][live]))',
                                  'np.lexsort((-live, -st["score"][live]))'),
    "eviction not permanent": ("live = np.flatnonzero(old != EVICTED)", "live = np.arange(len(old))"),
    "tiers swapped": ("new[order[:n_full]] = FULL", "new[order[:n_full]] = QUANT"),
    "re-quantised at every demotion": (' and j not in st["ledger"]:', ":"),
    "promotion keeps the old values": (
        '            st["K"][rows] = round_stored(dequantize_int2(ck, sk, mk, g), dtype)\n', ""),
    "promotion not rounded to the cache": (
        'st["V"][rows] = round_stored(dequantize_int2(cv, sv, mv, g), dtype)',
        'st["V"][rows] = dequantize_int2(cv, sv, mv, g)'),
    "event one step late": ("event = step % R == 0", "event = step % R == 1 % R"),
    "re-tier before attending": (
        "    out, mass = attend_unit(st, q_group, g)\n    event = step % R == 0\n    if event:\n"
        "        route_unit(st, mass, n_full, n_quant, g, dtype)\n",
        "    event = step % R == 0\n    if event:\n"
        "        route_unit(st, attend_unit(st, q_group, g)[1], n_full, n_quant, g, dtype)\n"
        "    out, mass = attend_unit(st, q_group, g)\n"),
}


def _mutant(old, new):
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation anchor not found once: {old!r}"
    mod = types.ModuleType("oracle.qevict_mutant")
    mod.__package__ = "oracle"
    exec(compile(text.replace(old, new), "qevict_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutant_is_caught(name):
    mod = _mutant(*MUTATIONS[name])
    for pin in ALL_PINS:
        try:
            pin(mod)
        except Exception:  # AssertionError or a crash both count
            return
    pytest.fail(f"no pin notices mutation {name!r}")

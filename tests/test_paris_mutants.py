"""Plant plausible mistakes in copies of the retrieval oracle; a pin must fail.

Each mutation edits one passage of oracle/paris.py's source text, loads the
edited text as a throw-away module and runs the pins against it.
"""
import os
import types

import pytest

from paris_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "paris.py")

MUTATIONS = {
    "hadamard blocks swapped": ("H = np.block([[H, H], [H, -H]])",
                                "H = np.block([[H, H], [-H, H]])"),
    "signs ignored": ("return (X * np.asarray(signs, np.float64)[None, :]) @",
                      "return (X * 1.0) @"),
    "scale by d": ("np.linalg.norm(X, axis=1, keepdims=True) * math.sqrt(X.shape[1])",
                   "np.linalg.norm(X, axis=1, keepdims=True) * X.shape[1]"),
    "centroid sign flipped": ("return (1.0 - 2.0 * bits) / math.sqrt(m)",
                              "return (2.0 * bits - 1.0) / math.sqrt(m)"),
    "rank ties to higher pattern": (
        "    order = np.lexsort((np.arange(len(scores)), -scores))\n    return order[:rho]",
        "    order = np.lexsort((-np.arange(len(scores)), -scores))\n    return order[:rho]"),
    "flat votes": ("T[b, p] = rho - r", "T[b, p] = 1"),
    "votes one short": ("T[b, p] = rho - r", "T[b, p] = rho - r - 1"),
    "candidate ties to higher index": (
        "    order = np.lexsort((np.arange(len(scores)), -scores))\n    return np.sort(order[:C])",
        "    order = np.lexsort((-np.arange(len(scores)), -scores))\n    return np.sort(order[:C])"),
    "floor candidates": ("return min(N, int(math.ceil(float(gamma) * N)))",
                         "return min(N, int(math.floor(float(gamma) * N)))"),
    "wrong Beta exponent": ("a = (m - 3) / 2.0", "a = (m - 2) / 2.0"),
    "bin midpoints": ("lam[j] = num / den", "lam[j] = 0.5 * (beta[j] + beta[j + 1])"),
    "sign bit inverted": ("neg = (U < 0) & live[:, :, None]", "neg = (U > 0) & live[:, :, None]"),
    "calibration without key norm": ("w64 = np.divide(knorm[:, None] * xn, den,",
                                     "w64 = np.divide(xn, den,"),
    "calibration not divided": ("w64 = np.divide(knorm[:, None] * xn, den,",
                                "w64 = np.divide(knorm[:, None] * xn, 1.0 + 0 * den,"),
    "estimate without query norm": ("return qnorm * (enc[\"w\"][rows] * dots).sum(axis=1)",
                                    "return (enc[\"w\"][rows] * dots).sum(axis=1)"),
    "estimate without calibration": ("return qnorm * (enc[\"w\"][rows] * dots).sum(axis=1)",
                                     "return qnorm * dots.sum(axis=1)"),
    "retrieval tie to higher index": (
        "    order = np.lexsort((np.arange(len(values)), -values.astype(np.float64)))",
        "    order = np.lexsort((-np.arange(len(values)), -values.astype(np.float64)))"),
    "local region one short": ("l0 = max(s, T - n_local)", "l0 = max(s, T - n_local + 1)"),
    "sink dropped": ("use = np.concatenate([sink, retrieved", "use = np.concatenate([sink[:0], retrieved"),
    "first query routes": ("qbar = q_group.sum(axis=0) / q_group.shape[0]", "qbar = q_group[0]"),
    "logit scale 1/d": ("K[idx].T / math.sqrt(K.shape[1])", "K[idx].T / K.shape[1]"),
    "calibration kept in fp64": ("w=w64.astype(np.float32).astype(np.float64)", "w=w64"),
}


def _mutant(old, new):
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation anchor not found once: {old!r}"
    mod = types.ModuleType("paris_mutant")
    exec(compile(text.replace(old, new), "paris_mutant", "exec"), mod.__dict__)
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

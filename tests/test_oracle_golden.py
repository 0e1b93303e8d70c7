"""The oracle reproduces the hand-worked single-line cases in
tests/golden/hand_worked.json (each derived step by step, not by running
code; see the 'derivation' entries there)."""
import json
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")
CASES = json.load(open(GOLD))["cases"]


def _unpack(q: np.ndarray, n: int) -> list:
    out = []
    for i in range(n):
        b = int(q[i // 2])
        out.append((b >> 4) if i & 1 else (b & 0xF))
    return out


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_hand_worked(case):
    x = np.array(case["x"], dtype=np.float32)
    n = x.size
    for var in case["variants"]:
        bound = var["bound"]
        q, s = oracle.quantize_rowwise(x[None, :], oracle.MODE_LINE, [case["amax"]], bound)
        assert s[0].tolist() == var["scales"], (bound, s[0].tolist())
        assert _unpack(q[0], n) == var["codes"], (bound, _unpack(q[0], n))
        if "packed" in var:
            assert q[0].tobytes().hex() == var["packed"]
        y = oracle.dequantize(q, s, 1, n, oracle.MODE_LINE, [case["amax"]], bound)[0]
        if "dequant" in var:
            want = np.array(var["dequant"], dtype=np.float32)
            assert np.array_equal(y.view(np.uint32), want.view(np.uint32)), y
        if "dequant_first_bits" in var:
            assert int(y.view(np.uint32)[0]) == var["dequant_first_bits"]
        # the same line through the column direction gives the same bytes
        qc, sc = oracle.quantize_colwise(x[:, None], oracle.MODE_LINE, [case["amax"]], bound)
        assert np.array_equal(qc, q) and np.array_equal(sc, s)

"""Pins of the oracle's four-over-six block scaling (a reading: the pages name
the four-over-six quantizer, its MSE choice and its bound 256, and define
nothing more; the oracle keeps, per block, whichever of the max-6 and max-4
scales dequantizes with the smaller squared error).

* hand-worked blocks (tests/golden/four_over_six.json, each argued step by
  step);
* an independent re-derivation of both candidates with numpy binary32
  arithmetic, torch's float8_e4m3fn conversion and a threshold-rule E2M1
  encoder, with the squared errors compared exactly (fractions): the oracle
  keeps the candidate with the smaller exact error, and where its binary64
  sums could disagree (exact errors within 1e-9 relative) either candidate
  is accepted;
* a block that keeps the max-6 scale is byte-identical to the standard 1x16
  quantization, and every kept block dequantizes with no more squared error
  than the standard one;
* the transposed copy is the rowwise copy of the transpose; scaling a row by
  a power of two leaves its codes and scales unchanged.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "four_over_six.json")))
GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _unpack(q, n):
    return [(int(q[i // 2]) >> 4) if i & 1 else (int(q[i // 2]) & 0xF) for i in range(n)]


@pytest.mark.parametrize("case", GOLD["cases"], ids=[c["name"] for c in GOLD["cases"]])
def test_hand_worked(case):
    x = np.array(case["x"], dtype=np.float32)
    q, s = oracle.quantize_line_46(x, [case["amax"]], case["bound"])
    assert s.tolist() == case["scales"]
    assert _unpack(q, x.size) == case["codes"]


# ----------------------------------------------------- independent candidates
def _e4m3(v: np.float32) -> int:
    t = torch.tensor([min(float(v), 448.0)], dtype=torch.float32).to(torch.float8_e4m3fn)
    return int(t.view(torch.uint8)[0])


def _e4m3_value(b: int) -> np.float32:
    return np.float32(torch.tensor([b], dtype=torch.uint8).view(torch.float8_e4m3fn).float()[0])


def _e2m1(v: np.float32) -> int:
    m = abs(float(v))
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    c = 0
    for k, t in enumerate(mids):
        if m > t or (m == t and (k + 1) % 2 == 0):
            c += 1
    c = min(c, 7)
    return c | (8 if np.signbit(v) else 0)


def _candidate(x, a, bound, top):
    f = np.float32(bound) * np.float32(6.0)
    f_inv = np.float32(1.0) / f
    s_enc = np.float32(1.0) if a == 0 else np.float32(min(np.float32(f / np.float32(a)), np.finfo(np.float32).max))
    bamax = np.float32(np.max(np.abs(x)))
    s32 = np.float32(np.float32(bamax / np.float32(top)) * s_enc)
    b = _e4m3(s32)
    d = np.float32(np.float32(_e4m3_value(b) * np.float32(a)) * f_inv)
    enc = np.float32(0.0) if d == 0 else np.float32(min(np.float32(np.float32(1.0) / d), np.finfo(np.float32).max))
    codes = [_e2m1(np.float32(v * enc)) for v in x]
    y = [np.float32(np.float32(-GRID[c & 7] if c & 8 else GRID[c & 7]) * d) for c in codes]
    err = sum((Fraction(float(v)) - Fraction(float(w))) ** 2 for v, w in zip(x, y))
    return b, codes, err


def _blocks(n_blocks, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n_blocks):
        kind = i % 4
        if kind == 0:
            x = rng.standard_normal(16)
        elif kind == 1:  # heavy tail
            x = rng.standard_t(2, 16)
        elif kind == 2:  # values near the top of the block
            x = rng.uniform(0.6, 1.0, 16) * rng.choice([-1, 1], 16)
        else:  # a few large values among small ones
            x = rng.standard_normal(16) * 0.05
            x[rng.integers(0, 16, 3)] = rng.uniform(0.5, 1.0, 3)
        x = (x * 10.0 ** rng.uniform(-3, 3)).astype(np.float32)
        out.append(x)
    return out


@pytest.mark.parametrize("bound", [256.0, 448.0])
def test_matches_independent_candidates(bound):
    kept = {4: 0, 6: 0}
    for x in _blocks(400, 5 if bound == 256.0 else 6):
        a = float(np.max(np.abs(x))) * (1.0 if np.random.default_rng(int(x[0] * 1e3) & 0xFFFF).random() < 0.5 else 1.7)
        a = float(np.float32(a))
        b6, c6, e6 = _candidate(x, a, bound, 6.0)
        b4, c4, e4 = _candidate(x, a, bound, 4.0)
        q, s = oracle.quantize_line_46(x, [a], bound)
        got = (int(s[0]), _unpack(q, 16))
        close = abs(e4 - e6) <= Fraction(1, 10 ** 9) * max(e4, e6, Fraction(1, 10 ** 300))
        if close:
            assert got in ((b6, c6), (b4, c4))
        elif e4 < e6:
            assert got == (b4, c4)
            kept[4] += 1
        else:
            assert got == (b6, c6)
            kept[6] += 1
    assert kept[4] > 20 and kept[6] > 20, kept  # both branches exercised


def test_max6_blocks_are_the_standard_quantization_and_error_never_grows():
    rng = np.random.default_rng(9)
    X = (rng.standard_normal((64, 256)) * 10.0 ** rng.uniform(-2, 2, (64, 1))).astype(np.float32)
    ra = oracle.amax_rows(X)
    q46, s46 = oracle.quantize_rowwise_46(X, oracle.MODE_LINE, ra, 256.0)
    q, s = oracle.quantize_rowwise(X, oracle.MODE_LINE, ra, 256.0)
    y46 = oracle.dequantize(q46, s46, 64, 256, oracle.MODE_LINE, ra, 256.0).astype(np.float64)
    y = oracle.dequantize(q, s, 64, 256, oracle.MODE_LINE, ra, 256.0).astype(np.float64)
    same = s46 == s
    for i in range(64):
        for b in range(16):
            sl = slice(16 * b, 16 * b + 16)
            if same[i, b]:
                assert np.array_equal(q46[i, 8 * b:8 * b + 8], q[i, 8 * b:8 * b + 8])
            e46 = np.sum((X[i, sl].astype(np.float64) - y46[i, sl]) ** 2)
            e6 = np.sum((X[i, sl].astype(np.float64) - y[i, sl]) ** 2)
            assert e46 <= e6 * (1 + 1e-9) + 1e-300
    assert 0.05 < np.mean(~same) < 0.95  # both choices occur


def test_transposed_copy_and_power_of_two_rows():
    rng = np.random.default_rng(10)
    X = (rng.standard_normal((48, 80)) * 10.0 ** rng.uniform(-2, 2, (48, 1))).astype(np.float32)
    ca = oracle.amax_cols(X)
    qc, sc = oracle.quantize_colwise_46(X, oracle.MODE_LINE, ca, 256.0)
    qt, st = oracle.quantize_rowwise_46(np.ascontiguousarray(X.T), oracle.MODE_LINE, ca, 256.0)
    assert np.array_equal(qc, qt) and np.array_equal(sc, st)
    ra = oracle.amax_rows(X)
    q, s = oracle.quantize_rowwise_46(X, oracle.MODE_LINE, ra, 256.0)
    X2 = X * np.float32(2.0 ** 7)
    q2, s2 = oracle.quantize_rowwise_46(X2, oracle.MODE_LINE, oracle.amax_rows(X2), 256.0)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)

"""Pins of the oracle's element formats against things other than itself.

E2M1: the oracle finds the nearest of the 8 grid magnitudes by distance. It is
checked against (a) the closed form of a 2-bit-exponent / 1-bit-mantissa float
with bias 1, (b) an independent threshold rule built from the 7 midpoints of
the grid with ties to the even code, over every BF16 bit pattern, fp32 values
around every midpoint and a random fp32 sample, and (c) exact rational
arithmetic (fractions) on a sample.

E4M3: the oracle scans the 127 finite non-negative values. It is checked
against torch's float8_e4m3fn conversion (a library routine: round-to-nearest-
even, non-saturating, hence the clamp to 448 first) over a sweep of the fp32
range, every midpoint, and the full byte range for decode.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _e2m1_closed_form(code: int) -> float:
    e = (code >> 1) & 3
    m = code & 1
    mag = (m * 0.5) if e == 0 else (2.0 ** (e - 1)) * (1.0 + m / 2.0)
    return -mag if code & 8 else mag


def test_e2m1_decode_closed_form():
    for c in range(16):
        v = oracle.e2m1_value(c)
        assert v == _e2m1_closed_form(c)
        assert np.signbit(np.float32(v)) == bool(c & 8)


def _e2m1_by_thresholds(v: np.ndarray) -> np.ndarray:
    """Count the grid midpoints below |v|; a value exactly on a midpoint goes
    to whichever neighbour has the even code."""
    v = v.astype(np.float32)
    m = np.abs(v)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float32)
    code = np.zeros(v.shape, dtype=np.int32)
    for k, t in enumerate(mids):
        code += (m > t).astype(np.int32)
        if (k + 1) % 2 == 0:  # upper neighbour k+1 is even -> a tie rounds up
            code += (m == t).astype(np.int32)
    code = np.minimum(code, 7)
    return (code | (np.signbit(v).astype(np.int32) << 3)).astype(np.uint8)


def _fp32_probe_set():
    bf = np.arange(65536, dtype=np.uint32) << 16
    vals = bf.view(np.float32)
    vals = vals[np.isfinite(vals)]
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 0.5, 1.0], dtype=np.float32)
    near = []
    for t in mids:
        b = np.array([t], dtype=np.float32).view(np.uint32)[0]
        for d in range(-4, 5):
            near.append(np.uint32(int(b) + d))
    near = np.array(near, dtype=np.uint32).view(np.float32)
    near = np.concatenate([near, -near])
    rng = np.random.default_rng(123)
    rnd = rng.integers(0, 2**32, size=400_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    rnd = rnd[np.isfinite(rnd)]
    small = (rng.standard_normal(200_000) * 4).astype(np.float32)
    special = np.array([0.0, -0.0, np.inf, -np.inf, np.finfo(np.float32).max,
                        -np.finfo(np.float32).max, 1e-45, -1e-45, 1e-39], dtype=np.float32)
    return np.concatenate([vals, near, rnd, small, special]).astype(np.float32)


def test_e2m1_encode_matches_threshold_rule():
    v = _fp32_probe_set()
    got = oracle.e2m1_encode(v)
    want = _e2m1_by_thresholds(v)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"first mismatch v={v[bad[0]]!r} got={got[bad[0]]} want={want[bad[0]]}"


def test_e2m1_encode_exact_rationals():
    rng = np.random.default_rng(7)
    v = np.concatenate([(rng.standard_normal(3000) * 3).astype(np.float32),
                        np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float32)])
    got = oracle.e2m1_encode(v)
    grid = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2),
            Fraction(3), Fraction(4), Fraction(6)]
    for x, c in zip(v.tolist(), got.tolist()):
        m = abs(Fraction(x))
        dists = [abs(m - g) for g in grid]
        best = min(dists)
        cands = [k for k, d in enumerate(dists) if d == best]
        k = cands[0] if len(cands) == 1 else [k for k in cands if k % 2 == 0][0]
        assert (c & 7) == k, (x, c, k)
        assert (c >> 3) == (1 if np.signbit(np.float32(x)) else 0)


def test_e2m1_worked_ties():
    # every tie of the grid, and both signs
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float32)
    assert oracle.e2m1_encode(ties).tolist() == [0, 2, 2, 4, 4, 6, 6]
    assert oracle.e2m1_encode(-ties).tolist() == [8, 10, 10, 12, 12, 14, 14]
    sat = np.array([6.0, 7.0, 1e30, np.inf, -1e30], dtype=np.float32)
    assert oracle.e2m1_encode(sat).tolist() == [7, 7, 7, 7, 15]
    assert oracle.e2m1_encode(np.array([0.0, -0.0, -1e-30], dtype=np.float32)).tolist() == [0, 8, 8]


def test_e4m3_decode_matches_torch():
    b = np.arange(256, dtype=np.uint8)
    t = torch.from_numpy(b).view(torch.float8_e4m3fn).float().numpy()
    for byte in range(256):
        if (byte & 0x7F) == 0x7F:
            continue  # NaN encodings are never produced
        assert oracle.e4m3_value(byte) == t[byte], byte


def _torch_e4m3(s: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(s.astype(np.float32)).clamp(max=448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encode_matches_torch_sweep():
    # every 2003rd non-negative fp32 pattern up to +inf, plus every E4M3 value
    # and the fp32 neighbours of every midpoint between consecutive values
    pats = np.arange(0, 0x7F800001, 2003, dtype=np.uint64).astype(np.uint32)
    s = pats.view(np.float32)
    vals = np.array([oracle.e4m3_value(b) for b in range(127)], dtype=np.float32)
    mids = ((vals[:-1].astype(np.float64) + vals[1:]) / 2).astype(np.float32)
    mb = mids.view(np.uint32)
    near = np.concatenate([mb.astype(np.int64) + d for d in range(-3, 4)]).astype(np.uint32).view(np.float32)
    s = np.concatenate([s, vals, near, np.array([448.0, 464.0, 465.0, 1e30, np.inf], np.float32)])
    s = s[np.isfinite(s) | np.isinf(s)]
    got = oracle.e4m3_encode(s)
    finite = np.isfinite(s)
    want = np.where(finite, _torch_e4m3(np.where(finite, s, 0)), 0x7E).astype(np.uint8)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"first mismatch s={s[bad[0]]!r} got={got[bad[0]]} want={want[bad[0]]}"


def test_e4m3_roundtrip_and_ties():
    vals = np.array([oracle.e4m3_value(b) for b in range(127)], dtype=np.float32)
    assert oracle.e4m3_encode(vals).tolist() == list(range(127))
    # subnormal ties: m * 2^-9 with m + 1/2 goes to the even m
    ties = np.array([(m + 0.5) * 2.0 ** -9 for m in range(8)], dtype=np.float32)
    assert oracle.e4m3_encode(ties).tolist() == [0, 2, 2, 4, 4, 6, 6, 8]
    assert oracle.e4m3_encode(np.array([2.0 ** -10], np.float32)).tolist() == [0]
    assert oracle.e4m3_encode(np.array([448.0, 460.0, 1e38], np.float32)).tolist() == [0x7E] * 3

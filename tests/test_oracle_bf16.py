"""The oracle's BF16 output rounding (backward-overrides PR description: the
dequantize writes BF16 or FP32) against two statements of round-to-nearest-
even that share nothing with it:

* the nearest-value rule in exact rational arithmetic: the BF16 grid spacing
  at x's binade, the grid points on either side, the nearer one, the even
  grid point on a tie, infinity past the largest finite BF16;
* the integer carry rule on the bit pattern, (b + 0x7FFF + bit16(b)) >> 16.

The rational rule covers every upper half (every BF16 value and its sign)
with the tie and its two neighbouring lower halves; the integer rule covers
every upper half with all lower halves within 4 of the tie, both ends of
the lower-half range, and a random sample of patterns."""
from fractions import Fraction
import math
import struct

import numpy as np

import oracle

FINITE_UPPER = np.array([u for u in range(1 << 16) if (u & 0x7F80) != 0x7F80], dtype=np.uint32)


def _patterns(lowers) -> np.ndarray:
    return (FINITE_UPPER[:, None] << 16 | np.asarray(lowers, dtype=np.uint32)[None, :]).ravel()


def _oracle_bits(bits: np.ndarray) -> np.ndarray:
    return oracle.to_bf16_bits(np.ascontiguousarray(bits, dtype=np.uint32).view(np.float32))


def _nearest_bf16(x: float) -> int:
    """RNE to BF16 (8 significant bits, exponent >= -126, no upper bound
    until rounding) from the exact value of x, as a 16-bit pattern."""
    if x == 0.0:
        return 0x8000 if math.copysign(1.0, x) < 0 else 0
    sign = 0x8000 if x < 0 else 0
    v = Fraction(abs(x))
    e = math.frexp(abs(x))[1] - 1          # 2^e <= |x| < 2^(e+1)
    q = Fraction(2) ** (max(e, -126) - 7)  # BF16 spacing in that binade
    k = v // q                             # lo = k q <= v < (k + 1) q
    r = v - k * q
    if r * 2 > q or (r * 2 == q and k % 2 == 1):
        k += 1
    y = k * q
    if y >= Fraction(2) ** 128:
        return sign | 0x7F80
    return sign | (struct.unpack("<I", struct.pack("<f", float(y)))[0] >> 16)


def test_nearest_value_rule_at_every_tie():
    bits = _patterns([0x7FFF, 0x8000, 0x8001])
    got = _oracle_bits(bits)
    x = bits.view(np.float32)
    want = np.array([_nearest_bf16(float(v)) for v in x], dtype=np.uint16)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} mismatches, first {bits[bad[0]]:#010x}"


def test_integer_carry_rule_near_ties_and_at_range_ends():
    lowers = list(range(0x7FFC, 0x8005)) + [0x0000, 0x0001, 0xFFFE, 0xFFFF]
    bits = _patterns(lowers)
    rng = np.random.default_rng(5)
    sample = rng.integers(0, 1 << 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    sample = sample[(sample & 0x7F800000) != 0x7F800000]
    bits = np.concatenate([bits, sample])
    want = ((bits.astype(np.uint64) + 0x7FFF + ((bits >> 16) & 1)) >> 16).astype(np.uint16)
    got = _oracle_bits(bits)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} mismatches, first {bits[bad[0]]:#010x}"


def test_special_values():
    f = lambda v: int(oracle.to_bf16_bits(np.array([v], dtype=np.float32))[0])
    assert f(0.0) == 0x0000 and f(-0.0) == 0x8000
    assert f(np.inf) == 0x7F80 and f(-np.inf) == 0xFF80
    assert f(1.0) == 0x3F80 and f(-2.0) == 0xC000
    # largest finite BF16, the midpoint above it (ties to the even, infinite,
    # pattern) and FLT_MAX
    big = struct.unpack("<f", struct.pack("<I", 0x7F7F7FFF))[0]
    mid = struct.unpack("<f", struct.pack("<I", 0x7F7F8000))[0]
    assert f(big) == 0x7F7F and f(mid) == 0x7F80 and f(np.finfo(np.float32).max) == 0x7F80
    # smallest subnormals: 2^-149 rounds to 0 (far below half of 2^-133)
    assert f(np.float32(2.0 ** -149)) == 0 and f(np.float32(2.0 ** -133)) == 0x0001
    # the pattern run form gives the same bits
    run = oracle.bf16_round_bits(0x3F7F7FF0, 64)
    assert np.array_equal(run, _oracle_bits(np.arange(0x3F7F7FF0, 0x3F7F8030, dtype=np.uint32)))

"""The cast kernel's branch-free block-scale chain replaces two IEEE
operations with cheaper forms that it uses only inside a checked range:

* RN(x / 6) as fma(x, H, RN(x * L)) with H = RN(1/6), L = RN(1/6 - H), for
  x >= 2^-121 (outside that range the kernel takes the IEEE division).

These tests check that identity with exactly emulated binary32 arithmetic:
the fma's exact sum x*H + c fits in a binary64 significand (x*H has 48
significant bits and c lies 24 binary places below its top), so one
binary64 addition followed by the rounding to binary32 is the fma. They
sweep every BF16 magnitude and every binary32 significand at the edges of
the range, and confirm that the range really ends there (the form fails
just below 2^-121)."""
import numpy as np

H = np.float32(1.0 / 6.0)
L = np.float32(np.float64(1.0) / 6.0 - np.float64(H))


def _two_term(x: np.ndarray) -> np.ndarray:
    c = (x * L).astype(np.float32)
    return (x.astype(np.float64) * np.float64(H) + c.astype(np.float64)).astype(np.float32)


def _ieee(x: np.ndarray) -> np.ndarray:
    # x / 6 in binary64 is within 2^-53 relative of the quotient, far from
    # every binary32 rounding midpoint (x / 6 never lies within a sixth of a
    # binary32 ulp of one), so rounding it to binary32 is RN(x / 6)
    return (x.astype(np.float64) / 6.0).astype(np.float32)


def _significands(exp: int) -> np.ndarray:
    bits = (np.uint32((exp + 127) << 23) + np.arange(1 << 23, dtype=np.uint32)).astype(np.uint32)
    return bits.view(np.float32)


def test_constants():
    assert H.view(np.uint32) == 0x3E2AAAAB
    assert L.view(np.uint32) == 0xB1AAAAAB
    assert L == np.float32(-float.fromhex("0x1.555556p-28"))


def test_every_bf16_magnitude_in_range():
    bits = (np.arange(1 << 15, dtype=np.uint32) << 16).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x) & (x >= np.float32(2.0 ** -121))]
    assert np.array_equal(_two_term(x), _ieee(x))


def test_every_significand_at_the_range_edges():
    for e in (-121, -120, 0, 1, 126, 127):
        x = _significands(e)
        x = x[np.isfinite(x)]
        bad = np.nonzero(_two_term(x) != _ieee(x))[0]
        assert bad.size == 0, f"2^{e}: first failure at {x[bad[0]]!r}"


def test_the_range_ends_below_2_pow_minus_121():
    fails = [np.count_nonzero(_two_term(x) != _ieee(x)) for x in map(_significands, (-123, -122))]
    assert all(f > 0 for f in fails)


# ----------------------------------------------------------------------------
# Exact emulation of fma(a, b, c) = RN32(a*b + c) for binary32 a, b, c whose
# exact sum is within a few ulps of c: a*b is exact in binary64 (48 bits). The
# part of it at or above u = ulp(c)/8 is added to c exactly in binary64; the
# part below u only matters through its sign (every binary32 grid point and
# midpoint near c, also one binade down, is a multiple of u), so it is
# replaced by u/2 when non-zero.
def _ulp32(c: np.ndarray) -> np.ndarray:
    e = ((c.view(np.uint32) >> 23) & 0xFF).astype(np.int64)
    return np.ldexp(1.0, np.maximum(e, 1) - 150)


def _fma_near(a: np.ndarray, b: np.ndarray, c: np.ndarray) -> np.ndarray:
    t = a.astype(np.float64) * b.astype(np.float64)
    u = _ulp32(c) / 8.0
    t_hi = np.floor(t / u) * u
    s = c.astype(np.float64) + t_hi + np.where(t != t_hi, u / 2.0, 0.0)
    return s.astype(np.float32)


def _fma_exact_small(a: np.ndarray, b: np.ndarray, c: np.ndarray) -> np.ndarray:
    """RN32(a*b + c) when a*b + c is exact in binary64 (few enough bits)."""
    return (a.astype(np.float64) * b.astype(np.float64) + c.astype(np.float64)).astype(np.float32)


# ---- RN(x / 6) in div6_rn: q = RN(x * R6), c = fma(-q, 6, x), fma(c, R6, q)
def _div6_corrected(x: np.ndarray) -> np.ndarray:
    q = (x.astype(np.float64) * np.float64(H)).astype(np.float32)  # 48-bit product, one rounding
    c = _fma_exact_small(-q, np.full_like(q, 6.0), x)               # x - 6q: exact in binary64
    return _fma_near(c, np.full_like(q, H), q)


def test_div6_correction_form_every_bf16_magnitude():
    bits = (np.arange(1 << 15, dtype=np.uint32) << 16).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x) & (x >= np.float32(2.0 ** -125))]
    assert np.array_equal(_div6_corrected(x), _ieee(x))


def test_div6_correction_form_edge_significands():
    for e in (-125, -124, -1, 0, 1, 126, 127):
        x = _significands(e)
        x = x[np.isfinite(x)]
        bad = np.nonzero(_div6_corrected(x) != _ieee(x))[0]
        assert bad.size == 0, f"2^{e}: first failure at {x[bad[0]]!r}"


# ---- RN(1 / d) in recip_rn: one Newton step fma(fma(-d, r, 1), r, r) from a
# hardware reciprocal r within an ulp of 1/d, i.e. either float neighbour of
# 1/d. The step is invariant under d -> d 2^k (r -> r 2^-k) while everything
# stays normal, so d in [1, 2) with every significand covers [2^-126, 2^126).
def _neighbours_of_recip(d: np.ndarray):
    rn = (1.0 / d.astype(np.float64)).astype(np.float32)  # RN32(1/d): no double rounding here
    above = d.astype(np.float64) * rn.astype(np.float64) > 1.0  # exact 48-bit product
    up = np.nextafter(rn, np.float32(np.inf))
    dn = np.nextafter(rn, np.float32(0.0))
    lo = np.where(above, dn, rn)
    hi = np.where(above, rn, up)
    return rn, lo, hi


def _newton(d: np.ndarray, r: np.ndarray) -> np.ndarray:
    e = _fma_exact_small(-d, r, np.ones_like(d))  # 1 - d r: 26 bits at most, exact
    return _fma_near(e, r, r)


def test_newton_step_from_both_neighbours():
    d = _significands(0)
    rn, lo, hi = _neighbours_of_recip(d)
    exact = d.astype(np.float64) * rn.astype(np.float64) == 1.0
    bad_lo = np.nonzero((_newton(d, lo) != rn) & ~exact)[0]
    bad_hi = np.nonzero((_newton(d, hi) != rn) & ~exact)[0]
    # from the upper neighbour the step is always RN(1/d)
    assert bad_hi.size == 0
    # from the lower neighbour it fails at exactly one significand: d = 2 - 2^-23,
    # where 1/d is 2^-48 relative above the midpoint between 2^-1 and its
    # successor and the step lands on the midpoint itself (ties to even, 2^-1)
    allones = (d.view(np.uint32) & 0x7FFFFF) == 0x7FFFFF
    assert bad_lo.tolist() == np.nonzero(allones)[0].tolist()
    i = int(bad_lo[0])
    assert lo[i] == np.float32(0.5) and rn[i].view(np.uint32) == 0x3F000001
    assert _newton(d[i:i + 1], lo[i:i + 1])[0] == np.float32(0.5)
    # at d = 1 (exact reciprocal) both neighbours of 1 step back to 1
    one = np.ones(1, dtype=np.float32)
    for r in (np.nextafter(one, np.float32(0)), np.nextafter(one, np.float32(2))):
        assert _newton(one, r)[0] == np.float32(1.0)


def test_reciprocal_guard_excludes_exactly_the_failing_significand():
    """The kernels take the IEEE division when D's significand is all ones
    (the guard on the bit pattern); every other significand is exact from
    either neighbour, so the encode factor never depends on which one the
    hardware returns."""
    d = _significands(0)
    guarded = (d.view(np.uint32) & 0x7FFFFF) == 0x7FFFFF
    rn, lo, hi = _neighbours_of_recip(d)
    ok = ~guarded
    assert np.array_equal(_newton(d[ok], lo[ok]), rn[ok])
    assert np.array_equal(_newton(d[ok], hi[ok]), rn[ok])
    assert int(guarded.sum()) == 1

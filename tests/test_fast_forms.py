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

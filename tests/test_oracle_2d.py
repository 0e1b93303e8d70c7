"""Pins of the oracle's 2-D (16 x 16 tile) quantization.

The pages name TE's 2-D weight blocks only through the switch that turns them
off (the 1x16 weight option of the backward-overrides PR), so the tile rule is
a reading: one scale per 16 x 16 tile from the tile's max magnitude, through
the same steps as a 1x16 block, under one per-tensor amax. These tests tie it
to the 1x16 path, which is pinned on its own:
  - every element's code and its tile's scale equal the 1x16 result for a
    two-element line holding the tile max and that element;
  - a matrix whose row blocks (or column blocks) all reach their tile's max
    quantizes exactly as the 1x16 per-tensor rowwise (or columnwise) copy;
  - the transposed copy is the nibble-level transpose of the rowwise copy;
  - tiles are independent, and partial edge tiles use only what exists.
"""
import numpy as np
import pytest

import oracle


def _matrix(M, K, seed):
    g = np.random.RandomState(seed)
    x = g.standard_normal((M, K)) * 10.0 ** g.uniform(-2, 2, size=(M, 1))
    return x.astype(np.float32)


def _codes(q, n):
    """Unpack [L][ceil(n/2)] packed codes into [L][n] nibbles."""
    lo, hi = q & 0xF, q >> 4
    out = np.empty((q.shape[0], 2 * q.shape[1]), dtype=np.uint8)
    out[:, 0::2], out[:, 1::2] = lo, hi
    return out[:, :n]


def _tile_max(x):
    M, K = x.shape
    t = np.zeros_like(x)
    for i in range(0, M, 16):
        for j in range(0, K, 16):
            t[i:i + 16, j:j + 16] = np.abs(x[i:i + 16, j:j + 16]).max()
    return t


@pytest.mark.parametrize("M,K,bound", [(16, 16, 448.0), (37, 53, 448.0), (48, 80, 256.0), (5, 3, 448.0)])
def test_every_element_matches_a_two_element_line(M, K, bound):
    x = _matrix(M, K, seed=M * K)
    a = np.float32(np.abs(x).max())
    q_row, s_row, q_col, s_col = oracle.quantize_2d(x, a, bound)
    tm = _tile_max(x)
    # line [tile max, element]: its block max is the tile max, so its scale
    # and the element's code are the 2-D ones
    lines = np.stack([tm.ravel(), x.ravel()], axis=1)
    q1, s1 = oracle.quantize_rowwise(lines, oracle.MODE_TENSOR, [a], bound)
    want_codes = (q1[:, 0] >> 4).reshape(M, K)
    want_scale = s1[:, 0].reshape(M, K)
    assert np.array_equal(_codes(q_row, K), want_codes)
    assert np.array_equal(np.repeat(s_row, 16, axis=1)[:, :K], want_scale)
    assert np.array_equal(np.repeat(s_col, 16, axis=1)[:, :M], want_scale.T)


@pytest.mark.parametrize("M,K", [(32, 64), (40, 45)])
def test_reduces_to_1x16_when_every_block_reaches_the_tile_max(M, K):
    g = np.random.RandomState(M + K)
    x = _matrix(M, K, seed=7)
    a = np.float32(np.abs(x).max() * 2)
    # rowwise: put the tile max (with a random sign) into every 1x16 row block
    xr = x.copy()
    tm = _tile_max(x)
    for r in range(M):
        for j in range(0, K, 16):
            c = j + g.randint(0, min(16, K - j))
            xr[r, c] = tm[r, c] * (1 if g.rand() < 0.5 else -1)
    q_row, s_row, _, _ = oracle.quantize_2d(xr, a)
    q1, s1 = oracle.quantize_rowwise(xr, oracle.MODE_TENSOR, [a])
    assert np.array_equal(q_row, q1) and np.array_equal(s_row, s1)
    # columnwise: the tile max in every column block
    xc = x.copy()
    for c in range(K):
        for i in range(0, M, 16):
            r = i + g.randint(0, min(16, M - i))
            xc[r, c] = tm[r, c] * (1 if g.rand() < 0.5 else -1)
    _, _, q_col, s_col = oracle.quantize_2d(xc, a)
    q2, s2 = oracle.quantize_colwise(xc, oracle.MODE_TENSOR, [a])
    assert np.array_equal(q_col, q2) and np.array_equal(s_col, s2)


@pytest.mark.parametrize("M,K", [(16, 16), (33, 47), (64, 32)])
def test_transposed_copy_is_the_exact_transpose(M, K):
    x = _matrix(M, K, seed=3)
    a = np.float32(np.abs(x).max())
    q_row, s_row, q_col, s_col = oracle.quantize_2d(x, a)
    assert np.array_equal(_codes(q_col, M), _codes(q_row, K).T)
    qt_row, st_row, qt_col, st_col = oracle.quantize_2d(np.ascontiguousarray(x.T), a)
    assert np.array_equal(qt_row, q_col) and np.array_equal(st_row, s_col)
    assert np.array_equal(qt_col, q_row) and np.array_equal(st_col, s_row)


def test_tiles_are_independent_and_zero_tiles_are_zero():
    x = _matrix(48, 48, seed=5)
    x[16:32, 16:32] = 0.0
    a = np.float32(np.abs(x).max())
    base = oracle.quantize_2d(x, a)
    c = _codes(base[0], 48)
    assert not c[16:32, 16:32].any() and not base[1][16:32, 1].any()
    y = x.copy()
    y[3, 40] *= 0.5  # tile (0, 2) only
    other = oracle.quantize_2d(y, a)
    cy = _codes(other[0], 48)
    mask = np.ones((48, 48), dtype=bool)
    mask[0:16, 32:48] = False
    assert np.array_equal(c[mask], cy[mask])
    assert np.array_equal(np.delete(base[1], 2, axis=1), np.delete(other[1], 2, axis=1))

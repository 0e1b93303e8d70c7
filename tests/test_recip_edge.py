"""Blocks whose decode scale D has an all-ones significand, D = (2 - 2^-23) 2^(j-1).

There RN(1/D) = 2^-j (1 + 2^-23), while a reciprocal one ulp low, 2^-j, is
what a Newton step from the lower neighbour of 1/D gives (tests in
test_fast_forms.py). Elements x = t 2^j with t on an E2M1 tie that rounds to
the even code below (0.25, 1.25, 2.5, 5) turn that one ulp into a different
code: x * 2^-j is the tie itself (rounds down), x * RN(1/D) lies above it
(rounds up). Every code of such a block therefore depends on the encode
factor being correctly rounded (backward-overrides PR description: FP32
decode with a correctly rounded reciprocal).

Lines: for exponents j from -100 to 100, a line amax a just below 6 * 2^j
makes D = RN(RN(sq * a) * F_inv) all-ones with the block's scale byte at the
bound (448 -> 0x7E, 256 -> 0x78). FP32 inputs hold a itself (the true line
max); BF16 inputs hold the BF16 value 5.96875 * 2^j as the block max and
pass a as the caller's line amax (mode LINE). The matrix is symmetric, so
every crafted row block is also a column block of the transposed copy with
the same amax.

The CPU tests check the construction itself (D's significand, and that a
reciprocal one ulp low changes codes: a mistake planted in a copy of the
oracle's step on the CPU); the GPU tests compare every byte with the oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle

EXPS = (-100, -40, -10, -3, 0, 3, 10, 40, 100)
TIES = (0.25, 1.25, 2.5, 5.0)
BF16_MAX_ELEM = 5.96875  # BF16 1.0111111b x 4, just below 6


def _f32(v) -> np.float32:
    return np.float32(v)


def _decode_scale(sq: float, a: np.float32, bound: float) -> np.float32:
    f_inv = _f32(1.0) / _f32(bound * 6.0)
    return (_f32(sq) * a) * f_inv


def _amax_for(j: int, bound: float) -> np.float32:
    """The float32 a just below 6 * 2^j (searched downwards) whose decode
    scale with the bound's top byte has an all-ones significand."""
    a = _f32(6.0 * 2.0 ** j)
    for _ in range(256):
        a = np.nextafter(a, _f32(0.0))
        d = _decode_scale(min(bound, 448.0), a, bound)
        if (int(d.view(np.uint32)) & 0x7FFFFF) == 0x7FFFFF:
            return a
    raise AssertionError(f"no all-ones decode scale near 6*2^{j} (bound {bound})")


def crafted_matrix(n: int, dtype: torch.dtype, bound: float, seed: int = 21):
    """Symmetric n x n matrix (n >= 176) and the line amax vector to quantize
    it with (the same for rows and columns). Crafted lines are rows/columns
    8 .. 8 + len(EXPS) - 1; line 8 + m has its crafted block at columns
    16 (2 + m) .. 16 (2 + m) + 15, away from every crafted line. Returns
    (x [n][n] as dtype, amax float32 [n], list of (line, block, j))."""
    assert n >= 16 * (2 + len(EXPS))
    g = torch.Generator().manual_seed(seed)
    r = torch.randn(n, n, generator=g) * 2.0 ** -3
    base = r + r.T  # symmetric
    x = base.clone()
    lines = [8 + m for m in range(len(EXPS))]
    for i, j in zip(lines, EXPS):
        # the rest of line i at a small scale, so that the block max and the
        # line amax are the crafted ones
        x[i, :] = base[i, :] * 2.0 ** (j - 6)
        x[:, i] = x[i, :]
    idx = torch.tensor(lines)
    x[idx[:, None], idx[None, :]] = 0.0  # crafted lines meet at zeros
    sites = []
    amax_line = {}
    for m, (i, j) in enumerate(zip(lines, EXPS)):
        b = 2 + m
        a = _amax_for(j, bound)
        top = float(a) if dtype == torch.float32 else BF16_MAX_ELEM * 2.0 ** j
        vals = [top] + [s * t * 2.0 ** j for t in TIES for s in (1.0, -1.0)]
        vals += [0.75 * 2.0 ** j, 2.0 ** (j - 30)]
        vals += [0.0] * (16 - len(vals))
        for k, v in enumerate(vals):
            x[i, 16 * b + k] = v
            x[16 * b + k, i] = v
        sites.append((i, b, j))
        amax_line[i] = a
    x = x.to(dtype)
    assert torch.equal(x, x.T) and torch.isfinite(x.float()).all()
    xf = x.float().numpy()
    amax = oracle.amax_rows(xf)
    for i, a in amax_line.items():
        if dtype == torch.float32:
            assert amax[i] == a  # the true line max is the crafted amax itself
        amax[i] = a
    return x, amax.astype(np.float32), sites


def _codes_with_enc(xb: np.ndarray, enc: np.float32) -> np.ndarray:
    return oracle.e2m1_encode((xb.astype(np.float32) * enc).astype(np.float32))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("bound", [448.0, 256.0])
def test_construction_hits_allones_and_is_sensitive(dtype, bound):
    x, amax, sites = crafted_matrix(192, dtype, bound)
    xf = x.float().numpy()
    q, s = oracle.quantize_rowwise(xf, oracle.MODE_LINE, amax, bound)
    for i, b, j in sites:
        byte = int(s[i, b])
        assert byte == (0x7E if bound == 448.0 else 0x78)
        sq = float(oracle.e4m3_value(byte))
        d = _decode_scale(sq, amax[i], bound)
        assert (int(d.view(np.uint32)) & 0x7FFFFF) == 0x7FFFFF
        enc = _f32(1.0) / d
        assert enc.view(np.uint32) == (_f32(2.0 ** -j).view(np.uint32) + 1)
        blk = xf[i, 16 * b:16 * b + 16]
        got = np.concatenate([[w & 0xF, w >> 4] for w in q[i, 8 * b:8 * b + 8]])
        assert np.array_equal(got, _codes_with_enc(blk, enc))
        # planted mistake: a reciprocal one ulp low changes every tie element
        wrong = _codes_with_enc(blk, _f32(2.0 ** -j))
        assert int((wrong != got).sum()) == 2 * len(TIES)
    # the transposed copy sees the same blocks (symmetric matrix, same amax)
    qc, sc = oracle.quantize_colwise(xf, oracle.MODE_LINE, amax, bound)
    assert np.array_equal(qc, q) and np.array_equal(sc, s)


# ----------------------------------------------------------------- GPU parity
SHAPES = [256, 263]  # the macro-tile kernel (n % 256 == 0) and the checked kernel


@pytest.mark.gpu
@pytest.mark.parametrize("n", SHAPES)
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("bound", [448.0, 256.0])
def test_gpu_quantize_transpose_allones(n, dtype, bound):
    import precision_quantization_row_amd as p
    from parity_utils import assert_same, gpu_quantize, say, to_np

    say(f"[gpu] all-ones decode scale: quantize_transpose {n}x{n} {dtype} bound {bound}")
    dev = torch.device("cuda:0")
    x, amax, _ = crafted_matrix(n, dtype, bound)
    xd = x.to(dev)
    ad = torch.from_numpy(amax).to(dev)
    out = gpu_quantize(xd, p.NVFP4_AMAX_LINE, ad, p.NVFP4_AMAX_LINE, ad, bound)
    xf = x.float().numpy()
    qr, sr = oracle.quantize_rowwise(xf, oracle.MODE_LINE, amax, bound)
    qc, sc = oracle.quantize_colwise(xf, oracle.MODE_LINE, amax, bound)
    assert_same("q_row", to_np(out["q_row"]), qr)
    assert_same("s_row", to_np(out["s_row"]), sr)
    assert_same("q_col", to_np(out["q_col"]), qc)
    assert_same("s_col", to_np(out["s_col"]), sc)
    if dtype == torch.float32:
        # the amax pass finds the crafted amaxes as the true line maxima
        ra = torch.empty(n, device=dev)
        ca = torch.empty(n, device=dev)
        p.nvfp4_amax_rowcol(xd, ra, ca)
        assert_same("row_amax", to_np(ra).view(np.uint32), amax.view(np.uint32))
        assert_same("col_amax", to_np(ca).view(np.uint32), amax.view(np.uint32))


@pytest.mark.gpu
@pytest.mark.parametrize("n", SHAPES)
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_gpu_quantize_dequantize_allones(n, dtype):
    import precision_quantization_row_amd as p
    from parity_utils import assert_same, say, to_np

    say(f"[gpu] all-ones decode scale: quantize_dequantize {n}x{n} {dtype}")
    dev = torch.device("cuda:0")
    x, amax, _ = crafted_matrix(n, dtype, 448.0)
    xd = x.to(dev)
    ad = torch.from_numpy(amax).to(dev)
    q = torch.empty(n, (n + 1) // 2, dtype=torch.uint8, device=dev)
    s = torch.empty(n, (n + 15) // 16, dtype=torch.uint8, device=dev)
    y = torch.empty(n, n, dtype=torch.float32, device=dev)
    p.nvfp4_quantize_dequantize(xd, p.NVFP4_AMAX_LINE, ad, 448.0, y, q, s)
    q_o, s_o, y_o = oracle.quantize_dequantize(x.float().numpy(), oracle.MODE_LINE, amax, 448.0)
    assert_same("q", to_np(q), q_o)
    assert_same("s", to_np(s), s_o)
    assert_same("y", to_np(y).view(np.uint32), y_o.view(np.uint32))


@pytest.mark.gpu
@pytest.mark.parametrize("n", SHAPES)
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_gpu_2d_allones(n, dtype):
    """2-D tiles under one per-tensor amax: the crafted amax of the largest
    exponent as the tensor amax (the true tensor max for FP32) gives the tile
    holding that line's crafted block the top byte and an all-ones decode
    scale."""
    import precision_quantization_row_amd as p
    from parity_utils import assert_same, say, to_np

    say(f"[gpu] all-ones decode scale: 2-D tiles {n}x{n} {dtype}")
    dev = torch.device("cuda:0")
    x, amax, sites = crafted_matrix(n, dtype, 448.0)
    xf = x.float().numpy()
    ta = np.array([amax[sites[-1][0]]], dtype=np.float32)
    assert np.abs(xf).max() <= ta[0]
    out = p.empty_outputs(n, n, dev)
    p.nvfp4_quantize_2d(x.to(dev), torch.from_numpy(ta).to(dev), 448.0, out["q_row"],
                        out["s_row"], out["q_col"], out["s_col"])
    qr, sr, qc, sc = oracle.quantize_2d(xf, float(ta[0]), 448.0)
    assert_same("q_row", to_np(out["q_row"]), qr)
    assert_same("s_row", to_np(out["s_row"]), sr)
    assert_same("q_col", to_np(out["q_col"]), qc)
    assert_same("s_col", to_np(out["s_col"]), sc)

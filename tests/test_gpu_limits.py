"""GPU parity at the size limits of the fast paths.

The interior cast kernel addresses a 32-row band of X with 31-bit offsets, so
it takes only rows with 32 * K * sizeof(element) < 2^31; longer rows go to the
checked edge kernel. These matrices cross that limit (4 GB of input). The
oracle checks sampled rows and columns one line at a time: the amax of the
line, its codes and scales, and the dequantized rowwise copy of a sampled row.
"""
import numpy as np
import pytest
import torch

import oracle
import precision_quantization_row_amd as p

from parity_utils import assert_same, f32_bits, say, to_np

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    p.load_library()


def _wide_matrix(M, K, dtype, seed):
    """N(0,1) times a per-row factor 10^U(-2,2), drawn on the device (seeded)."""
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    scale = torch.pow(10.0, -2.0 + 4.0 * torch.rand(M, 1, generator=g, device=DEV))
    x = torch.empty(M, K, dtype=dtype, device=DEV)
    step = 1 << 22
    for c in range(0, K, step):
        w = min(step, K - c)
        x[:, c:c + w] = (torch.randn(M, w, generator=g, device=DEV) * scale).to(dtype)
    return x


@pytest.mark.parametrize("dtype,K", [(torch.bfloat16, (1 << 25) + 256), (torch.float32, (1 << 24) + 256)])
def test_rows_past_the_interior_offset_limit(dtype, K):
    M = 64
    size = 2 if dtype == torch.bfloat16 else 4
    assert 32 * K * size >= 1 << 31  # the interior kernel cannot take these rows
    say(f"[gpu] limits: {M}x{K} {dtype} (interior offset limit crossed)")
    x = _wide_matrix(M, K, dtype, seed=21 if size == 2 else 22)
    ra = torch.full((M,), -7.0, device=DEV)
    ca = torch.full((K,), -7.0, device=DEV)
    p.nvfp4_amax_rowcol(x, ra, ca)
    out = p.empty_outputs(M, K, DEV)
    for v in out.values():
        v.fill_(0xA5)
    p.nvfp4_quantize_transpose(x, p.NVFP4_AMAX_LINE, ra, p.NVFP4_AMAX_LINE, ca, 448.0,
                               out["q_row"], out["s_row"], out["q_col"], out["s_col"])
    y = torch.empty(2, K, dtype=torch.bfloat16, device=DEV)
    p.nvfp4_dequantize(out["q_row"][:2].contiguous(), out["s_row"][:2].contiguous(), 2, K,
                       p.NVFP4_AMAX_LINE, ra[:2].contiguous(), 448.0, y)
    torch.cuda.synchronize()

    rows = [0, 1, 37, M - 1]
    for r in rows:
        xr = x[r:r + 1].float().cpu().numpy()
        a = oracle.amax_rows(xr)
        assert_same(f"row_amax[{r}]", f32_bits(ra[r:r + 1]), a.view(np.uint32))
        q, s = oracle.quantize_rowwise(xr, oracle.MODE_LINE, a, 448.0)
        assert_same(f"q_row[{r}]", to_np(out["q_row"][r:r + 1]), q)
        assert_same(f"s_row[{r}]", to_np(out["s_row"][r:r + 1]), s)
        if r < 2:
            yo = oracle.dequantize(q, s, 1, K, oracle.MODE_LINE, a, 448.0)
            assert_same(f"dequant[{r}]", y[r:r + 1].view(torch.int16).cpu().numpy().view(np.uint16),
                        oracle.to_bf16_bits(yo))
    cols = [0, 1, 255, 256, (1 << 20) + 3, K // 2, K - 257, K - 256, K - 1]
    xc = x[:, cols].float().cpu().numpy()            # [M][len(cols)]
    ac = oracle.amax_cols(xc)
    assert_same("col_amax[sampled]", f32_bits(ca[cols]), ac.view(np.uint32))
    qc, sc = oracle.quantize_colwise(xc, oracle.MODE_LINE, ac, 448.0)
    assert_same("q_col[sampled]", to_np(out["q_col"][cols]), qc)
    assert_same("s_col[sampled]", to_np(out["s_col"][cols]), sc)


@pytest.mark.parametrize("dtype,K", [(torch.bfloat16, (1 << 25) + 256), (torch.float32, (1 << 24) + 256)])
def test_2d_and_quantize_dequantize_past_the_offset_limit(dtype, K):
    """The 2-D tile cast and the one-pass quantize + dequantize on the same
    wide rows: sampled 16 x 16 tiles and whole sampled rows against the oracle."""
    M = 64
    say(f"[gpu] limits 2-D / qdq: {M}x{K} {dtype}")
    x = _wide_matrix(M, K, dtype, seed=23 if dtype == torch.bfloat16 else 24)
    ta = torch.empty(1, device=DEV)
    p.nvfp4_amax_rowcol(x, None, None, ta)
    out = p.empty_outputs(M, K, DEV)
    for v in out.values():
        v.fill_(0xA5)
    p.nvfp4_quantize_2d(x, ta, 448.0, out["q_row"], out["s_row"], out["q_col"], out["s_col"])
    torch.cuda.synchronize()
    a = np.float32(ta.item())
    for r0, c0 in [(0, 0), (16, 1 << 20), (48, K - 256), (32, K - 16)]:
        xt = x[r0:r0 + 16, c0:c0 + 16].float().cpu().numpy()
        q, s, qc, sc = oracle.quantize_2d(xt, a, 448.0)
        assert_same(f"2d q_row tile ({r0},{c0})", to_np(out["q_row"][r0:r0 + 16, c0 // 2:c0 // 2 + 8]), q)
        assert_same(f"2d s_row tile ({r0},{c0})", to_np(out["s_row"][r0:r0 + 16, c0 // 16:c0 // 16 + 1]), s)
        assert_same(f"2d q_col tile ({r0},{c0})", to_np(out["q_col"][c0:c0 + 16, r0 // 2:r0 // 2 + 8]), qc)
        assert_same(f"2d s_col tile ({r0},{c0})", to_np(out["s_col"][c0:c0 + 16, r0 // 16:r0 // 16 + 1]), sc)
    del out
    ra = torch.empty(M, device=DEV)
    p.nvfp4_amax_rowcol(x, ra)
    y = torch.empty(M, K, dtype=torch.bfloat16, device=DEV)
    qr = torch.empty(M, (K + 1) // 2, dtype=torch.uint8, device=DEV)
    sr = torch.empty(M, (K + 15) // 16, dtype=torch.uint8, device=DEV)
    p.nvfp4_quantize_dequantize(x, p.NVFP4_AMAX_LINE, ra, 448.0, y, qr, sr)
    torch.cuda.synchronize()
    for r in (1, M - 1):
        xr = x[r:r + 1].float().cpu().numpy()
        ar = oracle.amax_rows(xr)
        wq, ws, wy = oracle.quantize_dequantize(xr, oracle.MODE_LINE, ar, 448.0)
        assert_same(f"qdq q_row[{r}]", to_np(qr[r:r + 1]), wq)
        assert_same(f"qdq s_row[{r}]", to_np(sr[r:r + 1]), ws)
        assert_same(f"qdq y[{r}]", y[r:r + 1].view(torch.int16).cpu().numpy().view(np.uint16),
                    oracle.to_bf16_bits(wy))

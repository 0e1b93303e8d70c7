"""GPU parity of 2-D (16 x 16 tile) quantization against the oracle.

Both copies, byte for byte, on shapes that take the macro-tile kernel and on
shapes that take the checked edge kernel (partial tiles, odd sizes), both
input dtypes, both scale bounds, one copy at a time, noop, and the
dequantized copies. The full 8192 x 28672 matrix is checked on sampled
16-row bands (whole tiles), which the oracle quantizes on their own.
"""
import numpy as np
import pytest
import torch

import oracle
import precision_quantization_row_amd as p
from precision_quantization_row_amd import workloads

from parity_utils import assert_same, f32_bits, say, to_np

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    p.load_library()


def _matrix(M, K, dtype, seed):
    g = torch.Generator()
    g.manual_seed(seed)
    scale = torch.pow(10.0, -2.0 + 4.0 * torch.rand(M, 1, generator=g, dtype=torch.float64))
    x = torch.randn(M, K, generator=g, dtype=torch.float32)
    return (x.double() * scale).float().to(dtype)


def _run(xd, ta, bound, rowwise=True, colwise=True, noop=None, fill=0xA5):
    M, K = xd.shape
    out = p.empty_outputs(M, K, DEV, rowwise, colwise)
    for v in out.values():
        v.fill_(fill)
    p.nvfp4_quantize_2d(xd, ta, bound, out.get("q_row"), out.get("s_row"), out.get("q_col"),
                        out.get("s_col"), noop=noop)
    torch.cuda.synchronize()
    return out


def _check(tag, x, bound=448.0, rowwise=True, colwise=True):
    M, K = x.shape
    say(f"[gpu] 2d {tag}: {M}x{K} {x.dtype} bound={bound} row={rowwise} col={colwise}")
    xd = x.to(DEV)
    ta = torch.empty(1, device=DEV)
    p.nvfp4_amax_rowcol(xd, None, None, ta)
    out = _run(xd, ta, bound, rowwise, colwise)
    a = oracle.amax_tensor(x.float().numpy())
    assert_same(f"{tag} tensor amax", f32_bits(ta), np.asarray([a], np.float32).view(np.uint32))
    wq, ws, wqc, wsc = oracle.quantize_2d(x.float().numpy(), a, bound)
    if rowwise:
        assert_same(f"{tag} q_row", to_np(out["q_row"]), wq)
        assert_same(f"{tag} s_row", to_np(out["s_row"]), ws)
    if colwise:
        assert_same(f"{tag} q_col", to_np(out["q_col"]), wqc)
        assert_same(f"{tag} s_col", to_np(out["s_col"]), wsc)
    return ta, out, a


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("M,K", [
    (256, 256), (512, 768), (384, 512),    # macro tiles, a half macro row
    (320, 256),                            # macro tiles + edge rows
    (37, 53), (16, 16), (1, 7), (100, 130), (64, 300), (129, 1029),
])
def test_2d_matches_oracle(dtype, M, K):
    x = _matrix(M, K, dtype, seed=M * 131 + K)
    _check("shape", x)


@pytest.mark.parametrize("bound", [256.0, 6.0])
def test_2d_bounds_and_single_copies(bound):
    x = _matrix(256, 512, torch.bfloat16, seed=int(bound))
    _check("bound", x, bound)
    _check("rowwise", x, bound, colwise=False)
    _check("colwise", x, bound, rowwise=False)
    y = _matrix(50, 90, torch.float32, seed=3)
    _check("edge rowwise", y, bound, colwise=False)
    _check("edge colwise", y, bound, rowwise=False)


def test_2d_planted_structure():
    """Zero tiles, subnormal tiles, a tile holding one huge value."""
    w = workloads.make("fp32_edge", (96, 512))
    _check("fp32_edge", w.x)


def test_2d_noop_leaves_outputs_untouched():
    x = _matrix(256, 256, torch.bfloat16, seed=9).to(DEV)
    ta = torch.ones(1, device=DEV)
    out = _run(x, ta, 448.0, noop=torch.ones(1, device=DEV), fill=0x5A)
    for k, v in out.items():
        assert (v == 0x5A).all(), k


@pytest.mark.parametrize("od", [torch.bfloat16, torch.float32])
def test_2d_copies_dequantize_like_the_oracle(od):
    x = _matrix(256, 272, torch.bfloat16, seed=11)
    ta, out, a = _check("dequant", x)
    M, K = x.shape
    for name, R, C in (("row", M, K), ("col", K, M)):
        y = torch.empty(R, C, dtype=od, device=DEV)
        p.nvfp4_dequantize(out["q_" + name], out["s_" + name], R, C, p.NVFP4_AMAX_TENSOR, ta, 448.0, y)
        torch.cuda.synchronize()
        want = oracle.dequantize(to_np(out["q_" + name]), to_np(out["s_" + name]), R, C,
                                 oracle.MODE_TENSOR, [a], 448.0)
        if od == torch.bfloat16:
            got = y.view(torch.int16).cpu().numpy().view(np.uint16)
            assert_same(f"dequant {name}", got, oracle.to_bf16_bits(want))
        else:
            assert_same(f"dequant {name}", f32_bits(y), want.view(np.uint32))


def test_2d_full_size_sampled_bands():
    w = workloads.make("llm_mlp")
    M, K = w.shape
    say(f"[gpu] 2d full size {M}x{K}")
    xd = w.x.to(DEV)
    ta = torch.empty(1, device=DEV)
    p.nvfp4_amax_rowcol(xd, None, None, ta)
    out = _run(xd, ta, 448.0)
    xf = w.x[:, :].float()
    a = np.float32(xf.abs().max().item())
    assert_same("tensor amax", f32_bits(ta), np.asarray([a], np.float32).view(np.uint32))
    for band in (0, 1, 255, 256, M // 16 - 1):
        r0 = 16 * band
        xb = xf[r0:r0 + 16].numpy()
        wq, ws, wqc, wsc = oracle.quantize_2d(xb, a, 448.0)
        assert_same(f"q_row band {band}", to_np(out["q_row"][r0:r0 + 16]), wq)
        assert_same(f"s_row band {band}", to_np(out["s_row"][r0:r0 + 16]), ws)
        assert_same(f"q_col band {band}", to_np(out["q_col"][:, r0 // 2:r0 // 2 + 8]), wqc)
        assert_same(f"s_col band {band}", to_np(out["s_col"][:, band:band + 1]), wsc)


def test_2d_two_full_rounds_every_byte():
    """8192 x 8192 BF16: 128 macro tiles per XCD's strips, two full rounds of
    the resident grid on a 256-CU GPU (no split last round), so every
    workgroup carries its next tile's rows, loaded ahead, across a tile
    boundary. Every byte of both copies against the oracle."""
    _check("two rounds", _matrix(8192, 8192, torch.bfloat16, seed=88))


@pytest.mark.parametrize("M,K", [(256, 320), (512, 2880)])
def test_2d_columns_past_the_last_strip(M, K):
    _check("partial strip", _matrix(M, K, torch.bfloat16, seed=M + K))

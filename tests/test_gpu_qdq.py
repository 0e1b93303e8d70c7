"""GPU parity of the one-pass rowwise quantize + dequantize (the dequantized
backward operand) against the oracle's composition of the two steps.

Codes, scales and the dequantized values are compared bit for bit: vector
and general paths (K % 16, misaligned rows), BF16 and FP32 in and out,
per-tensor and per-row amax, both scale bounds, no codes requested, noop,
planted extremes and subnormals, and sampled rows of the 8192 x 28672 matrix.
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


def _shifted(shape, dtype, shift):
    """A contiguous device tensor whose data starts `shift` elements into its
    buffer (so its rows lose 16-byte alignment when shift > 0)."""
    n = int(np.prod(shape))
    buf = torch.empty(n + 8, dtype=dtype, device=DEV)
    return buf[shift:shift + n].view(*shape)


def _y_bits(y):
    if y.dtype == torch.bfloat16:
        return y.view(torch.int16).cpu().numpy().view(np.uint16)
    return f32_bits(y)


def _want_y_bits(y32, od):
    return oracle.to_bf16_bits(y32) if od == torch.bfloat16 else y32.view(np.uint32)


def _check(tag, x, mode, od, bound=448.0, codes=True, xshift=0, yshift=0):
    M, K = x.shape
    say(f"[gpu] qdq {tag}: {M}x{K} {x.dtype}->{od} mode={mode} bound={bound} codes={codes} "
        f"shift={xshift},{yshift}")
    xd = _shifted((M, K), x.dtype, xshift)
    xd.copy_(x.to(DEV))
    xf = x.float().numpy()
    if mode == p.NVFP4_AMAX_TENSOR:
        a_o = np.asarray([oracle.amax_tensor(xf)], np.float32)
    else:
        a_o = oracle.amax_rows(xf)
    a = torch.from_numpy(a_o).to(DEV)
    y = _shifted((M, K), od, yshift)
    y.fill_(7.0)
    q = torch.full((M, (K + 1) // 2), 0xA5, dtype=torch.uint8, device=DEV) if codes else None
    s = torch.full((M, (K + 15) // 16), 0xA5, dtype=torch.uint8, device=DEV) if codes else None
    p.nvfp4_quantize_dequantize(xd, mode, a, bound, y, q, s)
    torch.cuda.synchronize()
    wq, ws, wy = oracle.quantize_dequantize(xf, mode, a_o, bound)
    if codes:
        assert_same(f"{tag} q_row", to_np(q), wq)
        assert_same(f"{tag} s_row", to_np(s), ws)
    assert_same(f"{tag} y", _y_bits(y), _want_y_bits(wy, od))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("od", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("mode", [p.NVFP4_AMAX_TENSOR, p.NVFP4_AMAX_LINE])
@pytest.mark.parametrize("M,K", [(160, 272), (33, 2064), (7, 4112), (50, 37), (19, 150)])
def test_qdq_matches_oracle(dtype, od, mode, M, K):
    _check("shape", _matrix(M, K, dtype, seed=M + K), mode, od)


@pytest.mark.parametrize("bound", [256.0, 6.0])
def test_qdq_bounds_and_no_codes(bound):
    x = _matrix(64, 4096, torch.bfloat16, seed=int(bound))
    _check("bound", x, p.NVFP4_AMAX_LINE, torch.bfloat16, bound)
    _check("no codes", x, p.NVFP4_AMAX_LINE, torch.bfloat16, bound, codes=False)
    _check("no codes general", _matrix(9, 45, torch.float32, 1), p.NVFP4_AMAX_LINE,
           torch.float32, bound, codes=False)


@pytest.mark.parametrize("xshift,yshift", [(1, 0), (0, 1), (3, 5)])
def test_qdq_misaligned_rows(xshift, yshift):
    _check("misaligned", _matrix(24, 512, torch.bfloat16, seed=xshift), p.NVFP4_AMAX_LINE,
           torch.bfloat16, xshift=xshift, yshift=yshift)


def test_qdq_planted_structure():
    w = workloads.make("fp32_edge", (97, 160))
    _check("fp32_edge", w.x, p.NVFP4_AMAX_LINE, torch.float32)
    _check("fp32_edge bf16 out", w.x, p.NVFP4_AMAX_LINE, torch.bfloat16)


def test_qdq_noop_leaves_outputs_untouched():
    x = _matrix(32, 256, torch.bfloat16, seed=2).to(DEV)
    a = torch.ones(32, device=DEV)
    y = torch.full((32, 256), 3.0, dtype=torch.bfloat16, device=DEV)
    q = torch.full((32, 128), 0x5A, dtype=torch.uint8, device=DEV)
    s = torch.full((32, 16), 0x5A, dtype=torch.uint8, device=DEV)
    p.nvfp4_quantize_dequantize(x, p.NVFP4_AMAX_LINE, a, 448.0, y, q, s, noop=torch.ones(1, device=DEV))
    torch.cuda.synchronize()
    assert (y == 3.0).all() and (q == 0x5A).all() and (s == 0x5A).all()


def test_qdq_full_size_sampled_rows():
    w = workloads.make("llm_mlp")
    M, K = w.shape
    say(f"[gpu] qdq full size {M}x{K}")
    xd = w.x.to(DEV)
    ra = torch.empty(M, device=DEV)
    p.nvfp4_amax_rowcol(xd, ra)
    y = torch.empty(M, K, dtype=torch.bfloat16, device=DEV)
    q = torch.empty(M, K // 2, dtype=torch.uint8, device=DEV)
    s = torch.empty(M, K // 16, dtype=torch.uint8, device=DEV)
    p.nvfp4_quantize_dequantize(xd, p.NVFP4_AMAX_LINE, ra, 448.0, y, q, s)
    torch.cuda.synchronize()
    for r in (0, 1, 4095, M - 1):
        xr = w.x[r:r + 1].float().numpy()
        a = oracle.amax_rows(xr)
        assert_same(f"row_amax[{r}]", f32_bits(ra[r:r + 1]), a.view(np.uint32))
        wq, ws, wy = oracle.quantize_dequantize(xr, oracle.MODE_LINE, a, 448.0)
        assert_same(f"q_row[{r}]", to_np(q[r:r + 1]), wq)
        assert_same(f"s_row[{r}]", to_np(s[r:r + 1]), ws)
        assert_same(f"y[{r}]", _y_bits(y[r:r + 1]), oracle.to_bf16_bits(wy))

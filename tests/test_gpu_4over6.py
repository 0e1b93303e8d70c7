"""GPU parity of four-over-six block scaling (nvfp4_quantize_4over6) with the
oracle's quantize_rowwise_46 / quantize_colwise_46, byte for byte: both
copies and each alone, bounds 256 and 448, per-row, per-tensor and
group-expanded amaxes, aligned and ragged shapes, BF16 and FP32; the output
decodes with the plain dequantize; noop leaves every buffer untouched."""
import numpy as np
import pytest
import torch

import oracle
import precision_quantization_row_amd as p
from precision_quantization_row_amd import workloads

from parity_utils import (assert_same, bf16_exponent_sweep, dequant_bits, gpu_amax, gpu_dequant,
                          oracle_dequant_bits, say, to_np)

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    p.load_library()


def _run(x, row_mode, ra, col_mode, ca, bound, rowwise=True, colwise=True, noop=None):
    M, K = x.shape
    out = p.empty_outputs(M, K, x.device, rowwise, colwise)
    for v in out.values():
        v.fill_(0xA5)
    p.nvfp4_quantize_4over6(x, row_mode, ra if rowwise else None, col_mode, ca if colwise else None,
                            bound, out.get("q_row"), out.get("s_row"), out.get("q_col"),
                            out.get("s_col"), noop=noop)
    torch.cuda.synchronize()
    return out


def _check(x_cpu, bound, label, rowwise=True, colwise=True):
    M, K = x_cpu.shape
    say(f"[gpu] 4over6 {label} {M}x{K} {x_cpu.dtype} bound={bound} rw={rowwise} cw={colwise}")
    x = x_cpu.to(DEV)
    xf = x_cpu.float().numpy()
    ra, ca, _ = gpu_amax(x)
    out = _run(x, p.NVFP4_AMAX_LINE, ra, p.NVFP4_AMAX_LINE, ca, bound, rowwise, colwise)
    ra_o, ca_o = oracle.amax_rows(xf), oracle.amax_cols(xf)
    if rowwise:
        q, s = oracle.quantize_rowwise_46(xf, oracle.MODE_LINE, ra_o, bound)
        assert_same(f"{label} q_row", to_np(out["q_row"]), q)
        assert_same(f"{label} s_row", to_np(out["s_row"]), s)
    if colwise:
        q, s = oracle.quantize_colwise_46(xf, oracle.MODE_LINE, ca_o, bound)
        assert_same(f"{label} q_col", to_np(out["q_col"]), q)
        assert_same(f"{label} s_col", to_np(out["s_col"]), s)
    return x, ra, ca, out


SHAPES = [
    ("llm_mlp", (256, 512), torch.bfloat16),
    ("llm_mlp", (129, 1000), torch.bfloat16),   # ragged rows and blocks
    ("outliers", (384, 640), torch.bfloat16),
    ("fp32_edge", (97, 160), torch.float32),    # subnormal patches, extremes
    ("fp32_edge", (33, 47), torch.float32),     # odd sizes, short last blocks
]


@pytest.mark.parametrize("bound", [256.0, 448.0])
@pytest.mark.parametrize("name,shape,dtype", SHAPES, ids=[f"{n}-{s}" for n, s, _ in SHAPES])
def test_row_scaled_both_copies(name, shape, dtype, bound):
    x_cpu = workloads.make(name, shape).x.to(dtype)
    _check(x_cpu, bound, name)


@pytest.mark.parametrize("rowwise,colwise", [(True, False), (False, True)])
def test_single_copies(rowwise, colwise):
    x_cpu = workloads.make("llm_mlp", (200, 520)).x
    _check(x_cpu, 256.0, "single copy", rowwise, colwise)


def test_whole_bf16_exponent_range():
    _check(bf16_exponent_sweep(256, 512, seed=13), 256.0, "exponent sweep")


def test_per_tensor_and_group_amax_and_dequantize():
    w = workloads.make("moe_groups", None)
    # a slice of the grouped workload: 2 whole groups' worth of padded rows
    ge = w.group_end.numpy()
    M = int(ge[1])
    x_cpu = w.x[:M, :512].contiguous()
    x = x_cpu.to(DEV)
    xf = x_cpu.float().numpy()
    say(f"[gpu] 4over6 per-tensor and row-group amax {M}x512")
    ta = torch.empty(1, device=DEV)
    p.nvfp4_amax_rowcol(x, None, None, tensor_amax=ta)
    out = _run(x, p.NVFP4_AMAX_TENSOR, ta, p.NVFP4_AMAX_TENSOR, ta, 256.0)
    a = [oracle.amax_tensor(xf)]
    q, s = oracle.quantize_rowwise_46(xf, oracle.MODE_TENSOR, a, 256.0)
    assert_same("q_row tensor", to_np(out["q_row"]), q)
    assert_same("s_row tensor", to_np(out["s_row"]), s)
    qc, sc = oracle.quantize_colwise_46(xf, oracle.MODE_TENSOR, a, 256.0)
    assert_same("q_col tensor", to_np(out["q_col"]), qc)
    assert_same("s_col tensor", to_np(out["s_col"]), sc)
    # the plain dequantize decodes the result
    y = gpu_dequant(out["q_row"], out["s_row"], M, 512, p.NVFP4_AMAX_TENSOR, ta, 256.0, torch.float32)
    assert_same("dequant", dequant_bits(y), oracle_dequant_bits(q, s, M, 512, oracle.MODE_TENSOR, a,
                                                                 256.0, torch.float32))
    # group amax expanded over the rows, transposed blocks by row group
    ra = torch.empty(M, device=DEV)
    p.nvfp4_amax_rowcol(x, ra)
    ge_d = w.group_end[:2].to(DEV)
    p.nvfp4_group_amax_expand(ra, ge_d)
    out = _run(x, p.NVFP4_AMAX_LINE, ra, p.NVFP4_AMAX_ROWGROUP, ra, 256.0)
    ga = oracle.group_amax_expand(oracle.amax_rows(xf), w.group_end[:2].numpy())
    q, s = oracle.quantize_rowwise_46(xf, oracle.MODE_LINE, ga, 256.0)
    qc, sc = oracle.quantize_colwise_46(xf, oracle.MODE_ROWGROUP, ga, 256.0)
    assert_same("q_row group", to_np(out["q_row"]), q)
    assert_same("s_row group", to_np(out["s_row"]), s)
    assert_same("q_col rowgroup", to_np(out["q_col"]), qc)
    assert_same("s_col rowgroup", to_np(out["s_col"]), sc)


def test_noop_leaves_buffers():
    x = workloads.make("llm_mlp", (64, 128)).x.to(DEV)
    ra, ca, _ = gpu_amax(x)
    out = _run(x, 1, ra, 1, ca, 256.0, noop=torch.ones(1, device=DEV))
    for k, v in out.items():
        assert bool((v == 0xA5).all()), k


def test_medium_llm_shape():
    x_cpu = workloads.make("llm_mlp", (2048, 4096)).x
    _check(x_cpu, 256.0, "medium")

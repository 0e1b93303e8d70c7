"""GPU parity on the five workloads at their full sizes, in the launch
configuration the bench times. Every output element is compared with the
oracle (the oracle finishes the largest, 8192 x 28672, in seconds)."""
import numpy as np
import pytest
import torch

import oracle
import precision_quantization_row_amd as p
from precision_quantization_row_amd import workloads

from parity_utils import (assert_same, check_row_scaled, dequant_bits, f32_bits, gpu_amax,
                          gpu_dequant, gpu_quantize, oracle_dequant_bits, say, to_np)

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    p.load_library()


def test_tiny_rowscale_full():
    check_row_scaled(workloads.make("tiny_rowscale").x, bounds=(448.0, 256.0), label="256x256")


def test_outliers_full_row_scaled_and_per_tensor():
    w = workloads.make("outliers")
    x, ra, ca = check_row_scaled(w.x, bounds=(448.0,), label="4096x4096")
    xf = w.x.float().numpy()
    say("[gpu] outliers per-tensor")
    _, _, ta = gpu_amax(x, row=False, col=False, tensor=True)
    ta_o = oracle.amax_tensor(xf)
    assert f32_bits(ta)[0] == np.float32(ta_o).view(np.uint32)
    out = gpu_quantize(x, p.NVFP4_AMAX_TENSOR, ta, p.NVFP4_AMAX_TENSOR, ta, 448.0)
    qr, sr = oracle.quantize_rowwise(xf, oracle.MODE_TENSOR, [ta_o], 448.0)
    qc, sc = oracle.quantize_colwise(xf, oracle.MODE_TENSOR, [ta_o], 448.0)
    assert_same("q_row", to_np(out["q_row"]), qr)
    assert_same("s_row", to_np(out["s_row"]), sr)
    assert_same("q_col", to_np(out["q_col"]), qc)
    assert_same("s_col", to_np(out["s_col"]), sc)


def test_llm_mlp_full_with_noop():
    w = workloads.make("llm_mlp")
    M, K = w.shape
    say(f"[gpu] llm_mlp {M}x{K}: fused amax vs two-kernel")
    x = w.x.to(DEV)
    assert p.nvfp4_amax_path(p.NVFP4_BF16, M, K, 1, 1, 0) == 1
    ra, ca, _ = gpu_amax(x)
    ra2, ca2, _ = gpu_amax(x, flags=p.NVFP4_FLAG_FORCE_TWO_KERNEL)
    assert_same("fused vs two-kernel row", f32_bits(ra), f32_bits(ra2))
    assert_same("fused vs two-kernel col", f32_bits(ca), f32_bits(ca2))
    del ra2, ca2
    xf = w.x.float().numpy()
    ra_o, ca_o = oracle.amax_rows(xf), oracle.amax_cols(xf)
    assert_same("row_amax", f32_bits(ra), ra_o.view(np.uint32))
    assert_same("col_amax", f32_bits(ca), ca_o.view(np.uint32))
    say("[gpu] llm_mlp quantize both directions")
    out = gpu_quantize(x, 1, ra, 1, ca, 448.0)
    qr, sr = oracle.quantize_rowwise(xf, 1, ra_o, 448.0)
    assert_same("q_row", to_np(out["q_row"]), qr)
    assert_same("s_row", to_np(out["s_row"]), sr)
    del qr, sr
    qc, sc = oracle.quantize_colwise(xf, 1, ca_o, 448.0)
    assert_same("q_col", to_np(out["q_col"]), qc)
    assert_same("s_col", to_np(out["s_col"]), sc)
    del qc, sc
    say("[gpu] llm_mlp noop=1 preserves amax and outputs")
    noop = torch.ones(1, device=DEV)
    keep = [t.clone() for t in (ra, ca)]
    p.nvfp4_amax_rowcol(x, ra, ca, noop=noop)
    snap = {k: v.clone() for k, v in out.items()}
    p.nvfp4_quantize_transpose(x, 1, ra, 1, ca, 448.0, out["q_row"], out["s_row"],
                               out["q_col"], out["s_col"], noop=noop)
    torch.cuda.synchronize()
    assert torch.equal(keep[0], ra) and torch.equal(keep[1], ca)
    for k in out:
        assert torch.equal(snap[k], out[k]), k


def test_moe_groups_full():
    """Grouped-GEMM PR description: per-group amax expanded to rows; one call
    equals quantizing each split; padded rows give zero codes."""
    w = workloads.make("moe_groups")
    M, K = w.shape
    say(f"[gpu] moe_groups {M}x{K}, {w.group_end.numel()} groups")
    x = w.x.to(DEV)
    ge = w.group_end.to(DEV)
    ra, _, _ = gpu_amax(x, col=False)
    p.nvfp4_group_amax_expand(ra, ge)
    xf = w.x.float().numpy()
    ex_o = oracle.group_amax_expand(oracle.amax_rows(xf), w.group_end.numpy())
    assert_same("expanded amax", f32_bits(ra), ex_o.view(np.uint32))
    out = gpu_quantize(x, p.NVFP4_AMAX_LINE, ra, p.NVFP4_AMAX_ROWGROUP, ra, 448.0)
    qr, sr = oracle.quantize_rowwise(xf, oracle.MODE_LINE, ex_o, 448.0)
    qc, sc = oracle.quantize_colwise(xf, oracle.MODE_ROWGROUP, ex_o, 448.0)
    assert_same("q_row", to_np(out["q_row"]), qr)
    assert_same("s_row", to_np(out["s_row"]), sr)
    assert_same("q_col", to_np(out["q_col"]), qc)
    assert_same("s_col", to_np(out["s_col"]), sc)
    # padded rows are zero codes and zero scales in both copies
    start = 0
    q_row, s_row = to_np(out["q_row"]), to_np(out["s_row"])
    q_col, s_col = to_np(out["q_col"]), to_np(out["s_col"])
    for g, end in enumerate(w.group_end.tolist()):
        real = start + int(w.group_rows[g])
        assert not q_row[real:end].any() and not s_row[real:end].any()
        if end > real:
            lo, hi = (real + 15) // 16, end // 16  # whole padded 16-row blocks
            assert not s_col[:, lo:hi].any() and not q_col[:, lo * 8:hi * 8].any()
        start = end
    # one call == each split quantized alone (per-tensor) on the GPU too
    start = 0
    for g, end in enumerate(w.group_end.tolist()[:4]):
        if end > start:
            xs = x[start:end].contiguous()
            _, _, ta = gpu_amax(xs, row=False, col=False, tensor=True)
            o = gpu_quantize(xs, 0, ta, 0, ta, 448.0)
            assert torch.equal(o["q_row"], out["q_row"][start:end])
            assert torch.equal(o["q_col"], out["q_col"][:, start // 2:end // 2])
            assert torch.equal(o["s_col"], out["s_col"][:, start // 16:end // 16])
        start = end
    # dequantize the transposed copy with the group amax of each block
    y = gpu_dequant(out["q_col"], out["s_col"], K, M, p.NVFP4_AMAX_ROWGROUP, ra, 448.0, torch.bfloat16)
    assert_same("dequant col", dequant_bits(y),
                oracle_dequant_bits(qc, sc, K, M, oracle.MODE_ROWGROUP, ex_o, 448.0, torch.bfloat16))


@pytest.mark.parametrize("flags", [0, p.NVFP4_FLAG_FORCE_TWO_KERNEL])
def test_fp32_edge_full(flags):
    """FP32 4097 x 2880 with its planted structure, both bounds, through the
    one-pass amax (the default for 16-byte rows) and through the two-kernel
    amax path."""
    w = workloads.make("fp32_edge")
    M, K = w.shape
    assert p.nvfp4_amax_path(p.NVFP4_FP32, M, K, 1, 1, flags) == (2 if flags else 1)
    x, ra, ca = check_row_scaled(w.x, bounds=(448.0, 256.0), flags=flags, label="fp32_edge")
    zr = w.notes["zero_row"]
    out = gpu_quantize(x, 1, ra, 1, ca, 448.0)
    assert not out["q_row"][zr].any() and not out["s_row"][zr].any()

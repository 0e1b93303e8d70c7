"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI
binding, run the CPU oracle on the same seeded input, compare bit for bit."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import precision_quantization_row_amd as p

MODE_NAMES = {0: "tensor", 1: "line", 2: "rowgroup"}


def say(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def assert_same(name: str, got: np.ndarray, want: np.ndarray) -> None:
    assert got.shape == want.shape, f"{name}: shape {got.shape} != {want.shape}"
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        i = tuple(bad[0])
        raise AssertionError(f"{name}: {len(bad)} mismatches, first at {i}: got {got[i]!r} "
                             f"want {want[i]!r}")


def f32_bits(t) -> np.ndarray:
    a = t.detach().cpu().numpy() if isinstance(t, torch.Tensor) else np.asarray(t)
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def gpu_amax(x: torch.Tensor, row=True, col=True, tensor=False, flags=0, noop=None):
    M, K = x.shape
    dev = x.device
    ra = torch.full((M,), -7.0, device=dev) if row else None
    ca = torch.full((K,), -7.0, device=dev) if col else None
    ta = torch.full((1,), -7.0, device=dev) if tensor else None
    p.nvfp4_amax_rowcol(x, ra, ca, ta, noop=noop, flags=flags)
    return ra, ca, ta


def gpu_quantize(x: torch.Tensor, row_mode, row_amax, col_mode, col_amax, bound,
                 rowwise=True, colwise=True, noop=None):
    M, K = x.shape
    out = p.empty_outputs(M, K, x.device, rowwise, colwise)
    for v in out.values():
        v.fill_(0xA5)  # sentinel: every byte must be overwritten
    p.nvfp4_quantize_transpose(x, row_mode, row_amax if rowwise else None, col_mode,
                               col_amax if colwise else None, bound, out.get("q_row"),
                               out.get("s_row"), out.get("q_col"), out.get("s_col"), noop=noop)
    return out


def gpu_dequant(q, s, R, C, mode, amax, bound, out_dtype):
    y = torch.empty(R, C, dtype=out_dtype, device=q.device)
    p.nvfp4_dequantize(q, s, R, C, mode, amax, bound, y)
    return y


def dequant_bits(y: torch.Tensor) -> np.ndarray:
    if y.dtype == torch.bfloat16:
        return y.view(torch.int16).cpu().numpy().view(np.uint16)
    return f32_bits(y)


def oracle_dequant_bits(q, s, R, C, mode, amax, bound, out_dtype) -> np.ndarray:
    y = oracle.dequantize(q, s, R, C, mode, amax, bound)
    return oracle.to_bf16_bits(y) if out_dtype == torch.bfloat16 else y.view(np.uint32)


def check_row_scaled(x_cpu: torch.Tensor, bounds=(448.0,), flags=0, dequant=True, label=""):
    """Row-scaled NVFP4 in both directions through the HIP path vs the oracle:
    amax vectors, codes, scales, and (optionally) both dequantized copies."""
    dev = torch.device("cuda:0")
    M, K = x_cpu.shape
    say(f"[gpu] row-scaled {label} {M}x{K} {x_cpu.dtype} flags={flags}")
    x = x_cpu.to(dev)
    xf = x_cpu.float().numpy()
    ra, ca, _ = gpu_amax(x, flags=flags)
    ra_o, ca_o = oracle.amax_rows(xf), oracle.amax_cols(xf)
    assert_same("row_amax", f32_bits(ra), ra_o.view(np.uint32))
    assert_same("col_amax", f32_bits(ca), ca_o.view(np.uint32))
    for bound in bounds:
        out = gpu_quantize(x, p.NVFP4_AMAX_LINE, ra, p.NVFP4_AMAX_LINE, ca, bound)
        qr, sr = oracle.quantize_rowwise(xf, oracle.MODE_LINE, ra_o, bound)
        qc, sc = oracle.quantize_colwise(xf, oracle.MODE_LINE, ca_o, bound)
        assert_same(f"q_row b={bound}", to_np(out["q_row"]), qr)
        assert_same(f"s_row b={bound}", to_np(out["s_row"]), sr)
        assert_same(f"q_col b={bound}", to_np(out["q_col"]), qc)
        assert_same(f"s_col b={bound}", to_np(out["s_col"]), sc)
        if dequant:
            for od in (torch.bfloat16, torch.float32):
                y = gpu_dequant(out["q_row"], out["s_row"], M, K, p.NVFP4_AMAX_LINE, ra, bound, od)
                assert_same(f"dequant row {od} b={bound}", dequant_bits(y),
                            oracle_dequant_bits(qr, sr, M, K, oracle.MODE_LINE, ra_o, bound, od))
                y = gpu_dequant(out["q_col"], out["s_col"], K, M, p.NVFP4_AMAX_LINE, ca, bound, od)
                assert_same(f"dequant col {od} b={bound}", dequant_bits(y),
                            oracle_dequant_bits(qc, sc, K, M, oracle.MODE_LINE, ca_o, bound, od))
    return x, ra, ca


def bf16_exponent_sweep(M: int, K: int, seed: int = 11) -> torch.Tensor:
    """N(0,1) rows scaled by 2^e with e swept over the BF16 range (subnormal
    rows included), plus planted elements: single magnitudes in [2^121,
    2^126] inside ordinary rows, a row of exactly 2^121, a row of BF16
    subnormals and an all-zero row. Magnitudes of 2^121 and above are the
    patterns that read as f16 infinities or NaNs."""
    g = torch.Generator().manual_seed(seed)
    z = torch.randn(M, K, generator=g)
    e = torch.linspace(-140.0, 124.0, M).round()
    x = z * torch.pow(2.0, e)[:, None]
    idx = torch.randperm(M * K, generator=g)[: M * K // 997]
    x.view(-1)[idx] = torch.pow(2.0, torch.randint(121, 127, (idx.numel(),), generator=g).float()) * \
        torch.where(torch.rand(idx.numel(), generator=g) < 0.5, -1.0, 1.0)
    x[M // 3] = 2.0 ** 121
    x[M // 2] = torch.where(torch.rand(K, generator=g) < 0.5, -1.0, 1.0) * 2.0 ** -130
    x[M // 5] = 0.0
    xb = x.to(torch.bfloat16)
    assert torch.isfinite(xb.float()).all()
    return xb

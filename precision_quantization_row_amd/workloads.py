"""Seeded synthetic inputs shaped like the LLM / MoE workloads of row-scaled
NVFP4 quantization.

This module holds no NVFP4 arithmetic: it only draws random matrices (with
torch's CPU generator, so the same seed gives the same bits on every host)
and lays out grouped tokens. Tests and the bench feed the same tensors to the
HIP library and to the CPU oracle.

Workloads (name: shape, dtype, distribution):
  tiny_rowscale   256 x 256 BF16, N(0,1) times a per-row factor 10^U(-3,3)
  outliers        4096 x 4096 BF16, N(0,1) with 0.1 % of the elements replaced
                  by +-U(100, 1000) at random positions
  llm_mlp         8192 x 28672 BF16, N(0,1) times a per-row factor 10^U(-2,2)
  moe_groups      16 expert groups, token counts multinomial over 16384 tokens,
                  K = 4096, BF16 N(0,1), each group zero-padded to a multiple
                  of 128 rows
  fp32_edge       4097 x 2880 FP32, N(0,1) plus planted structure: an all-zero
                  row, a column with a single nonzero value, 16x16 patches of
                  subnormal magnitude (and one all-subnormal row), and rows /
                  blocks with magnitudes in [0.5, 0.99] * FLT_MAX / 448
Every generator takes an optional shape override so tests can draw the same
distribution at a size the oracle finishes in seconds.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import torch

FLT_MAX = float(torch.finfo(torch.float32).max)

NAMES = ("tiny_rowscale", "outliers", "llm_mlp", "moe_groups", "fp32_edge")
SEEDS = {"tiny_rowscale": 1, "outliers": 2, "llm_mlp": 3, "moe_groups": 4, "fp32_edge": 5}
SHAPES = {
    "tiny_rowscale": (256, 256),
    "outliers": (4096, 4096),
    "llm_mlp": (8192, 28672),
    "moe_groups": (16384, 4096),  # (total real tokens, K)
    "fp32_edge": (4097, 2880),
}


@dataclass
class Workload:
    name: str
    x: torch.Tensor                       # [M, K] CPU, bfloat16 or float32
    group_end: Optional[torch.Tensor] = None   # int64 [G], padded row offsets
    group_rows: Optional[torch.Tensor] = None  # int64 [G], real rows per group
    notes: dict = field(default_factory=dict)

    @property
    def shape(self):
        return tuple(self.x.shape)


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator()
    g.manual_seed(seed)
    return g


def _row_log_uniform(g, M: int, lo: float, hi: float) -> torch.Tensor:
    u = torch.rand(M, 1, generator=g, dtype=torch.float64)
    return torch.pow(10.0, lo + (hi - lo) * u)


def tiny_rowscale(shape=None) -> Workload:
    M, K = shape or SHAPES["tiny_rowscale"]
    g = _gen(SEEDS["tiny_rowscale"])
    x = torch.randn(M, K, generator=g, dtype=torch.float32)
    x = (x.double() * _row_log_uniform(g, M, -3.0, 3.0)).float()
    return Workload("tiny_rowscale", x.to(torch.bfloat16))


def outliers(shape=None) -> Workload:
    M, K = shape or SHAPES["outliers"]
    g = _gen(SEEDS["outliers"])
    x = torch.randn(M * K, generator=g, dtype=torch.float32)
    n_out = max(1, (M * K) // 1000)
    pos = torch.randperm(M * K, generator=g)[:n_out]
    mag = 100.0 + 900.0 * torch.rand(n_out, generator=g, dtype=torch.float32)
    sign = torch.where(torch.rand(n_out, generator=g) < 0.5, -1.0, 1.0)
    x[pos] = mag * sign
    return Workload("outliers", x.view(M, K).to(torch.bfloat16), notes={"n_outliers": n_out})


def llm_mlp(shape=None) -> Workload:
    M, K = shape or SHAPES["llm_mlp"]
    g = _gen(SEEDS["llm_mlp"])
    scale = _row_log_uniform(g, M, -2.0, 2.0).float()
    x = torch.empty(M, K, dtype=torch.bfloat16)
    step = 512  # draw in row chunks to bound host memory at full size
    for r in range(0, M, step):
        blk = torch.randn(min(step, M - r), K, generator=g, dtype=torch.float32)
        x[r:r + step] = (blk * scale[r:r + step]).to(torch.bfloat16)
    return Workload("llm_mlp", x)


def moe_groups(shape=None, n_groups: int = 16, align: int = 128) -> Workload:
    T, K = shape or SHAPES["moe_groups"]
    g = _gen(SEEDS["moe_groups"])
    pick = torch.multinomial(torch.ones(n_groups), T, replacement=True, generator=g)
    rows = torch.bincount(pick, minlength=n_groups).to(torch.int64)
    padded = ((rows + align - 1) // align) * align
    group_end = torch.cumsum(padded, 0)
    M = int(group_end[-1]) if n_groups else 0
    x = torch.zeros(M, K, dtype=torch.bfloat16)
    start = 0
    for gi in range(n_groups):
        n = int(rows[gi])
        if n:
            x[start:start + n] = torch.randn(n, K, generator=g, dtype=torch.float32).to(torch.bfloat16)
        start += int(padded[gi])
    return Workload("moe_groups", x, group_end=group_end, group_rows=rows,
                    notes={"tokens": T, "align": align})


def fp32_edge(shape=None) -> Workload:
    M, K = shape or SHAPES["fp32_edge"]
    g = _gen(SEEDS["fp32_edge"])
    x = torch.randn(M, K, generator=g, dtype=torch.float32)
    notes = {}

    def rnd(n):
        return torch.rand(n, generator=g, dtype=torch.float64)

    def signs(n):
        return torch.where(torch.rand(n, generator=g) < 0.5, -1.0, 1.0).double()

    # subnormal-magnitude 16x16 patches inside normal rows, |x| ~ 1e-39
    n_patch = max(1, min(8, (M // 16) * (K // 16) // 4))
    patches = []
    for _ in range(n_patch):
        r = int(torch.randint(0, max(1, M - 16), (1,), generator=g))
        c = int(torch.randint(0, max(1, K - 16), (1,), generator=g))
        h, w = min(16, M - r), min(16, K - c)
        v = (0.2 + 1.6 * rnd(h * w)) * 1e-39 * signs(h * w)
        x[r:r + h, c:c + w] = v.float().view(h, w)
        patches.append((r, c))
    notes["subnormal_patches"] = patches
    # extreme magnitudes near FLT_MAX / 448: one full row and a few blocks
    lim = FLT_MAX / 448.0
    rows_ext = [int(M * 0.73) % M]
    for r in rows_ext:
        v = (0.5 + 0.49 * rnd(K)) * lim * signs(K)
        x[r] = v.float()
    blocks_ext = []
    for _ in range(3):
        r = int(torch.randint(0, M, (1,), generator=g))
        c = int(torch.randint(0, max(1, K - 16), (1,), generator=g)) // 16 * 16
        w = min(16, K - c)
        x[r, c:c + w] = ((0.5 + 0.49 * rnd(w)) * lim * signs(w)).float()
        blocks_ext.append((r, c))
    notes["extreme_rows"] = rows_ext
    notes["extreme_blocks"] = blocks_ext
    # one row made entirely of subnormal magnitudes
    r_sub = (M // 2 + 1) % M
    x[r_sub] = ((0.2 + 1.6 * rnd(K)) * 1e-39 * signs(K)).float()
    notes["subnormal_row"] = r_sub
    # an all-zero row
    r_zero = 7 % M
    x[r_zero] = 0.0
    notes["zero_row"] = r_zero
    # a column holding a single nonzero value
    c_one = 13 % K
    x[:, c_one] = 0.0
    r_one = (M // 3) % M
    if r_one == r_zero:
        r_one = (r_one + 1) % M
    x[r_one, c_one] = 3.25
    notes["single_nonzero_col"] = (c_one, r_one)
    return Workload("fp32_edge", x, notes=notes)


GENERATORS = {
    "tiny_rowscale": tiny_rowscale,
    "outliers": outliers,
    "llm_mlp": llm_mlp,
    "moe_groups": moe_groups,
    "fp32_edge": fp32_edge,
}


def make(name: str, shape=None) -> Workload:
    return GENERATORS[name](shape)


def algorithmic_bytes(M: int, K: int, in_bytes: int, rowwise: bool = True,
                      colwise: bool = True, row_amax: bool = True,
                      col_amax: bool = True, tensor_amax: bool = False) -> int:
    """Bytes the two-pass method must move: X read by the amax pass and again
    by the cast pass, each amax vector written once and read once, each code
    and scale copy written once."""
    x = M * K * in_bytes
    amax = 4 * ((M if row_amax else 0) + (K if col_amax else 0) + (1 if tensor_amax else 0))
    out = 0
    if rowwise:
        out += M * ((K + 1) // 2) + M * ((K + 15) // 16)
    if colwise:
        out += K * ((M + 1) // 2) + K * ((M + 15) // 16)
    return 2 * x + 2 * amax + out

"""GPU parity of grouped-token quantization with padding on the way in.

The HIP entry point takes the token rows of G ragged groups and the group
sizes (on the device), and writes the padded layout: per-group amax expanded
over each padded group, rowwise and transposed codes and scales. Every case is
compared byte for byte with the oracle's quantize_grouped on the same input;
the full-size grouped workload is checked on sampled lines, and as a whole
against padding the matrix first and quantizing it with the plain entry points.
"""
import numpy as np
import pytest
import torch

import oracle
import precision_quantization_row_amd as p
from precision_quantization_row_amd import workloads

from parity_utils import assert_same, bf16_exponent_sweep, f32_bits, say, to_np

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    p.load_library()


def _tokens(T, K, dtype, seed):
    """N(0,1) times a per-row factor 10^U(-2,2) (seeded, CPU)."""
    g = torch.Generator()
    g.manual_seed(seed)
    scale = torch.pow(10.0, -2.0 + 4.0 * torch.rand(max(T, 1), 1, generator=g, dtype=torch.float64))
    x = torch.randn(max(T, 1), K, generator=g, dtype=torch.float32)
    return (x.double() * scale).float()[:T].to(dtype).contiguous()


def _run(x, group_rows, align, m_out, bound=448.0, rowwise=True, colwise=True, noop=None,
         fill=0xA5):
    K = x.shape[1]
    xd = x.to(DEV)
    gr = torch.tensor(group_rows, dtype=torch.int64, device=DEV)
    ra = torch.full((m_out,), -7.0, device=DEV)
    out = p.empty_outputs(m_out, K, DEV, rowwise, colwise)
    for v in out.values():
        v.fill_(fill)
    p.nvfp4_quantize_grouped(xd, gr, align, m_out, bound, ra, out.get("q_row"), out.get("s_row"),
                             out.get("q_col"), out.get("s_col"), noop=noop)
    torch.cuda.synchronize()
    return ra, out


def _check(tag, x, group_rows, align, m_out, bound=448.0, rowwise=True, colwise=True):
    say(f"[gpu] grouped {tag}: T={x.shape[0]} K={x.shape[1]} {x.dtype} groups={list(group_rows)} "
        f"align={align} M_out={m_out} bound={bound}")
    ra, out = _run(x, group_rows, align, m_out, bound, rowwise, colwise)
    # the header's reading of negative sizes: they count as empty groups
    sizes = np.maximum(np.asarray(group_rows, dtype=np.int64), 0)
    wa, wq, ws, wqc, wsc = oracle.quantize_grouped(x.float().numpy(), sizes, align, m_out, bound)
    assert_same(f"{tag} row_amax", f32_bits(ra), wa.view(np.uint32))
    if rowwise:
        assert_same(f"{tag} q_row", to_np(out["q_row"]), wq)
        assert_same(f"{tag} s_row", to_np(out["s_row"]), ws)
    if colwise:
        assert_same(f"{tag} q_col", to_np(out["q_col"]), wqc)
        assert_same(f"{tag} s_col", to_np(out["s_col"]), wsc)
    return ra, out


def _full_rows(group_rows, align):
    return int(oracle.padded_group_end(group_rows, align, 1 << 40)[-1])


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("group_rows,align,K", [
    ([20, 0, 30, 7], 16, 64),          # an empty group, ragged groups
    ([1, 33, 16, 0, 0, 5], 32, 48),    # two empty groups in a row, K of 3 blocks
    ([300], 128, 256),                 # one group (G = 1)
    ([0, 0, 3], 16, 37),               # leading empty groups, odd K
    ([129, 127, 128, 1, 255], 128, 512),
    ([17] * 40, 16, 96),               # many small groups
])
def test_grouped_matches_oracle(dtype, group_rows, align, K):
    T = sum(group_rows)
    x = _tokens(T, K, dtype, seed=T + K + align)
    m_out = _full_rows(group_rows, align)
    _check("exact", x, group_rows, align, m_out)


@pytest.mark.parametrize("extra", [16, 40, 301])
def test_rows_past_the_groups_are_zero(extra):
    group_rows = [50, 0, 14]
    x = _tokens(64, 80, torch.bfloat16, seed=extra)
    m_out = _full_rows(group_rows, 16) + extra
    ra, out = _check(f"+{extra}", x, group_rows, 16, m_out)
    last = _full_rows(group_rows, 16)
    assert not ra[last:].any()


@pytest.mark.parametrize("m_out", [1, 15, 40, 72, 100])
def test_truncated_layout(m_out):
    """M_out smaller than the padded total: rows that do not fit are dropped
    and take no part in their group's amax."""
    group_rows = [50, 0, 14, 30]
    x = _tokens(94, 64, torch.float32, seed=m_out)
    _check(f"truncated to {m_out}", x, group_rows, 16, m_out)


def test_tokens_beyond_the_groups_and_short_x():
    # T larger than the groups need: the extra token rows are ignored
    x = _tokens(100, 64, torch.bfloat16, seed=5)
    x[60:] = 1000.0  # would change the amax if read
    _check("extra tokens", x, [20, 40], 32, 96)
    # groups claim more rows than x holds: the missing rows read as zero
    _check("short x", _tokens(30, 64, torch.bfloat16, seed=6), [20, 40], 32, 96)


def test_negative_sizes_count_as_empty():
    x = _tokens(40, 32, torch.bfloat16, seed=8)
    _check("negative", x, [10, -5, 30], 16, 64)


@pytest.mark.parametrize("bound", [448.0, 256.0, 6.0])
def test_bounds_and_single_directions(bound):
    group_rows = [33, 70, 0, 9]
    x = _tokens(112, 128, torch.bfloat16, seed=int(bound))
    m_out = _full_rows(group_rows, 16)
    _check("both", x, group_rows, 16, m_out, bound)
    _check("rowwise", x, group_rows, 16, m_out, bound, colwise=False)
    _check("colwise", x, group_rows, 16, m_out, bound, rowwise=False)


def test_maximum_group_count_and_alignment():
    rng = np.random.RandomState(11)
    group_rows = rng.randint(0, 9, size=p.NVFP4_GROUPS_MAX).tolist()
    x = _tokens(sum(group_rows), 32, torch.bfloat16, seed=11)
    _check("256 groups", x, group_rows, 16, _full_rows(group_rows, 16))
    group_rows = [5000, 100]
    x = _tokens(5100, 16, torch.float32, seed=12)
    _check("align 4096", x, group_rows, 4096, _full_rows(group_rows, 4096))


def test_noop_leaves_every_buffer_untouched():
    group_rows = [20, 12]
    x = _tokens(32, 64, torch.bfloat16, seed=13)
    noop = torch.ones(1, device=DEV)
    ra, out = _run(x, group_rows, 16, 48, noop=noop, fill=0x3C)
    assert (ra == -7.0).all()
    for k, v in out.items():
        assert (v == 0x3C).all(), k


def _round64(n):
    return -(-n // 64) * 64


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("case", ["mixed", "large_align", "short_x", "truncated", "many", "past",
                                  "partial_strip"])
def test_macro_tile_layouts(dtype, case):
    """Layouts that take the macro-tile path (K a multiple of 256, M_out of 64):
    16-row blocks that end a group mid-block, next to padding, empty groups,
    token rows missing at the end of x, truncation, 256 groups, and rows past
    the last group."""
    K, align, T = 256, 16, None
    if case == "mixed":
        group_rows = [5, 0, 300, 17, 64, 1]
    elif case == "large_align":
        group_rows, align, K = [1000, 3, 250], 128, 512
    elif case == "short_x":
        group_rows, align, T = [200, 200], 32, 150
    elif case == "truncated":
        group_rows = [300, 300]
    elif case == "partial_strip":
        group_rows, K = [100, 37, 0, 60], 320
    elif case == "many":
        group_rows = np.random.RandomState(17).randint(0, 41, size=p.NVFP4_GROUPS_MAX).tolist()
    else:
        group_rows = [40, 90]
    T = sum(group_rows) if T is None else T
    x = _tokens(T, K, dtype, seed=len(case) + K)
    # M_out a multiple of 64 (the last macro-tile sub-step half full) and of
    # 128 (every sub-step full)
    for rnd in (64, 128):
        m_out = -(-_full_rows(group_rows, align) // rnd) * rnd
        if case == "truncated":
            m_out = 512 - 64 * (rnd == 64)
        if case == "past":
            m_out += 256
        _check(f"{case} M_out {m_out}", x, group_rows, align, m_out)
    if case == "mixed" and dtype == torch.bfloat16:
        _check("mixed rowwise", x, group_rows, align, m_out, colwise=False)
        _check("mixed colwise", x, group_rows, align, m_out, rowwise=False)


def test_transposed_copy_dequantizes_like_the_oracle():
    group_rows = [40, 0, 25]
    align = 32
    x = _tokens(65, 96, torch.bfloat16, seed=14)
    m_out = _full_rows(group_rows, align)
    ra, out = _check("dequant", x, group_rows, align, m_out)
    y = torch.empty(96, m_out, dtype=torch.float32, device=DEV)
    p.nvfp4_dequantize(out["q_col"], out["s_col"], 96, m_out, p.NVFP4_AMAX_ROWGROUP, ra, 448.0, y)
    torch.cuda.synchronize()
    want = oracle.dequantize(to_np(out["q_col"]), to_np(out["s_col"]), 96, m_out,
                             oracle.MODE_ROWGROUP, ra.cpu().numpy(), 448.0)
    assert_same("dequant q_col", f32_bits(y), np.asarray(want, dtype=np.float32).view(np.uint32))


def test_full_size_grouped_workload():
    """16 groups over 16384 tokens, K = 4096, 128-row alignment: sampled lines
    against the oracle, and the whole output against padding first and then
    quantizing with the plain entry points."""
    w = workloads.make("moe_groups")
    xp = w.x                                   # padded [M, K], built by the generator
    M, K = xp.shape
    rows = w.group_rows
    starts = torch.cat([torch.zeros(1, dtype=torch.int64), w.group_end[:-1]])
    tokens = torch.cat([xp[int(s):int(s) + int(n)] for s, n in zip(starts, rows)])
    say(f"[gpu] grouped full size: T={tokens.shape[0]} K={K} M_out={M}")
    ra, out = _run(tokens, rows.tolist(), 128, M)

    # whole output: the padded matrix through amax + expand + quantize
    xd = xp.to(DEV)
    ra2 = torch.empty(M, device=DEV)
    p.nvfp4_amax_rowcol(xd, ra2)
    p.nvfp4_group_amax_expand(ra2, w.group_end.to(DEV))
    out2 = p.empty_outputs(M, K, DEV)
    p.nvfp4_quantize_transpose(xd, 1, ra2, 2, ra2, 448.0, out2["q_row"], out2["s_row"],
                               out2["q_col"], out2["s_col"])
    torch.cuda.synchronize()
    assert torch.equal(ra, ra2)
    for k in out:
        assert torch.equal(out[k], out2[k]), k

    # sampled lines against the oracle
    xf = xp.float().numpy()
    ge = w.group_end.numpy()
    for g in (0, 7, 15):
        s, e = int(starts[g]), int(ge[g])
        ga = np.float32(np.abs(xf[s:e]).max())
        assert_same(f"group {g} amax", f32_bits(ra[s:e]), np.full(e - s, ga, np.float32).view(np.uint32))
    for r in (0, int(rows[0]) - 1, int(rows[0]), int(starts[9]) + 3, M - 1):
        a = np.asarray([ra[r].item()], dtype=np.float32)
        q, sc = oracle.quantize_rowwise(xf[r:r + 1], oracle.MODE_LINE, a, 448.0)
        assert_same(f"q_row[{r}]", to_np(out["q_row"][r:r + 1]), q)
        assert_same(f"s_row[{r}]", to_np(out["s_row"][r:r + 1]), sc)
    cols = [0, 1, 15, 16, 2047, K - 1]
    xc = np.ascontiguousarray(xf[:, cols])
    qc, scc = oracle.quantize_colwise(xc, oracle.MODE_ROWGROUP, ra.cpu().numpy(), 448.0)
    assert_same("q_col[sampled]", to_np(out["q_col"][cols]), qc)
    assert_same("s_col[sampled]", to_np(out["s_col"][cols]), scc)


def test_grouped_bf16_whole_exponent_range():
    """Token rows with BF16 magnitudes from subnormal to 2^126 (the patterns
    that read as f16 infinities or NaNs included) through the grouped
    macro-tile kernel, byte for byte against the oracle."""
    x = bf16_exponent_sweep(427, 512, seed=12)
    group_rows = [200, 77, 0, 150]
    _check("exponent sweep", x, group_rows, 128, _full_rows(group_rows, 128))

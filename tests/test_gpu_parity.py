"""GPU parity: every output of the HIP path, called through the C ABI, is
compared element by element with the CPU oracle on the same seeded input.
The bar is bit-exact for amax floats, E4M3 scale bytes, packed E2M1 code
bytes (padding nibbles included) and dequantized FP32 / BF16 bits."""
import numpy as np
import pytest
import torch

import oracle
import precision_quantization_row_amd as p
from precision_quantization_row_amd import workloads

from parity_utils import (assert_same, bf16_exponent_sweep, check_row_scaled, dequant_bits,
                          f32_bits, gpu_amax, gpu_dequant, gpu_quantize, oracle_dequant_bits, say,
                          to_np)

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    p.load_library()


# ------------------------------------------------------- small shapes, full
SMALL = [
    ("tiny_rowscale", None),          # 256 x 256 BF16, fused amax
    ("outliers", (384, 640)),         # BF16, fused amax, several tiles
    ("llm_mlp", (512, 1152)),         # BF16, fused, partial 512-column strip
    ("llm_mlp", (200, 520)),          # BF16 unaligned: two-kernel amax, ragged tiles
    ("llm_mlp", (129, 1000)),         # BF16, M % 16 != 0, K % 16 != 0
    ("fp32_edge", (97, 160)),         # FP32 ragged rows
    ("fp32_edge", (33, 47)),          # FP32 odd sizes, odd line lengths
    ("tiny_rowscale", (1, 1)),
    ("tiny_rowscale", (1, 17)),
    ("tiny_rowscale", (17, 1)),
    ("tiny_rowscale", (2, 33)),
]


@pytest.mark.parametrize("name,shape", SMALL, ids=[f"{n}-{s}" for n, s in SMALL])
def test_small_row_scaled(name, shape):
    w = workloads.make(name, shape)
    check_row_scaled(w.x, bounds=(448.0, 256.0), label=name)


@pytest.mark.parametrize("shape", [(256, 256), (384, 640)])
def test_small_forced_two_kernel(shape):
    w = workloads.make("outliers", shape)
    check_row_scaled(w.x, flags=p.NVFP4_FLAG_FORCE_TWO_KERNEL, dequant=False, label="two-kernel")


@pytest.mark.parametrize("M,K", [(128, 128), (384, 640), (1152, 2304), (4224, 1024), (8192, 128),
                                 (4224, 24576)])
def test_fused_amax_tile_heights(M, K):
    """The fused amax picks its tile height per shape, 256 rows down to 32:
    32-row tiles for the small shapes here (with a partial last column tile
    when K is not a multiple of 512), 128-row tiles for 4224 x 24576. The
    full-size workload tests cover 256 (8192 x 28672) and 64 (grouped
    tokens). Every choice gives the exact maxima."""
    say(f"[gpu] fused amax tile heights {M}x{K}")
    g = torch.Generator().manual_seed(M + K)
    x = (torch.randn(M, K, generator=g) * torch.exp(torch.randn(M, 1, generator=g) * 3)).to(torch.bfloat16)
    assert p.nvfp4_amax_path(p.NVFP4_BF16, M, K, 1, 1, 0) == 1
    ra, ca, _ = gpu_amax(x.to(DEV))
    xf = x.float().numpy()
    assert_same("row_amax", f32_bits(ra), oracle.amax_rows(xf).view(np.uint32))
    assert_same("col_amax", f32_bits(ca), oracle.amax_cols(xf).view(np.uint32))


@pytest.mark.parametrize("dtype,M,K", [
    (torch.float32, 4097, 2880), (torch.float32, 1, 4), (torch.float32, 17, 260),
    (torch.float32, 300, 1028), (torch.float32, 33, 65540 // 4 * 4), (torch.float32, 1000, 12),
    (torch.bfloat16, 1, 8), (torch.bfloat16, 257, 520), (torch.bfloat16, 129, 4104),
    (torch.bfloat16, 4097, 2888), (torch.bfloat16, 70, 24),
    # the 128-column tiles of medium matrices, with a cut last chunk
    (torch.bfloat16, 2000, 4104), (torch.float32, 3000, 5000)])
def test_fused_amax_ragged_and_fp32(dtype, M, K):
    """The one-pass amax on shapes outside the 128-aligned BF16 case: FP32,
    ragged M, and K that ends inside a chunk or a tile (only whole 16-byte
    row vectors are required). Values over the whole exponent range of the
    type (FP32 subnormals and magnitudes up to FLT_MAX / 448 included); exact
    maxima, identical to the two-kernel path."""
    say(f"[gpu] fused amax {M}x{K} {dtype}")
    g = torch.Generator().manual_seed(M * 7 + K)
    e = torch.randint(-140, 120, (M, 1), generator=g).float() if dtype == torch.float32 else \
        torch.randint(-130, 120, (M, 1), generator=g).float()
    x = (torch.randn(M, K, generator=g) * torch.pow(2.0, e)).to(dtype)
    x[torch.rand(M, K, generator=g) < 0.01] = 0.0
    assert torch.isfinite(x.float()).all()
    assert p.nvfp4_amax_path(p.NVFP4_BF16 if dtype == torch.bfloat16 else p.NVFP4_FP32,
                             M, K, 1, 1, 0) == 1
    xd = x.to(DEV)
    ra, ca, _ = gpu_amax(xd)
    xf = x.float().numpy()
    assert_same("row_amax", f32_bits(ra), oracle.amax_rows(xf).view(np.uint32))
    assert_same("col_amax", f32_bits(ca), oracle.amax_cols(xf).view(np.uint32))
    ra2, ca2, _ = gpu_amax(xd, flags=p.NVFP4_FLAG_FORCE_TWO_KERNEL)
    assert_same("row two-kernel", f32_bits(ra2), f32_bits(ra))
    assert_same("col two-kernel", f32_bits(ca2), f32_bits(ca))


# Shapes the general macro-tile variant takes in one launch: ragged M (odd
# counts included, so transposed code rows have an odd number of bytes),
# K % 16 == 0 but not a multiple of 256 (a cut last strip), tiny matrices,
# and M % 128 == 64 (formerly the macro tiles plus a checked launch).
GENERAL = [
    (torch.float32, 4097, 2880), (torch.bfloat16, 4097, 2880), (torch.bfloat16, 1, 16),
    (torch.float32, 1, 16), (torch.bfloat16, 17, 48), (torch.float32, 255, 272),
    (torch.bfloat16, 257, 4112), (torch.bfloat16, 300, 1040), (torch.float32, 129, 512),
    (torch.bfloat16, 8256, 512), (torch.float32, 1000, 2000), (torch.bfloat16, 33, 4000),
    (torch.float32, 383, 784), (torch.bfloat16, 2049, 1296),
]


@pytest.mark.parametrize("dtype,M,K", GENERAL, ids=[f"{d}-{m}x{k}" for d, m, k in GENERAL])
def test_general_shapes_row_scaled(dtype, M, K):
    """Row-scaled, both copies, both bounds, dequantized both ways: every byte
    and bit against the oracle. Values over a wide exponent range (FP32
    subnormals included), with zero rows and columns planted."""
    g = torch.Generator().manual_seed(M * 31 + K)
    e = torch.randint(-135 if dtype == torch.float32 else -125, 100, (M, 1), generator=g).float()
    x = torch.randn(M, K, generator=g) * torch.pow(2.0, e)
    x[M // 2] = 0.0
    x[:, K // 3] = 0.0
    x = x.to(dtype)
    assert torch.isfinite(x.float()).all()
    check_row_scaled(x, bounds=(448.0, 256.0), label=f"general {M}x{K}")


@pytest.mark.parametrize("dtype,M,K", [(torch.float32, 4097, 2880), (torch.bfloat16, 257, 1040),
                                       (torch.bfloat16, 129, 48)])
@pytest.mark.parametrize("rowwise,colwise", [(True, False), (False, True)])
def test_general_shapes_one_direction(dtype, M, K, rowwise, colwise):
    say(f"[gpu] general {M}x{K} {dtype} rowwise={rowwise} colwise={colwise}")
    g = torch.Generator().manual_seed(M + 3 * K)
    x = (torch.randn(M, K, generator=g) * torch.exp(torch.randn(M, 1, generator=g) * 4)).to(dtype)
    xf = x.float().numpy()
    xd = x.to(DEV)
    ra, ca, _ = gpu_amax(xd)
    out = gpu_quantize(xd, 1, ra, 1, ca, 448.0, rowwise=rowwise, colwise=colwise)
    if rowwise:
        qr, sr = oracle.quantize_rowwise(xf, oracle.MODE_LINE, oracle.amax_rows(xf), 448.0)
        assert_same("q_row", to_np(out["q_row"]), qr)
        assert_same("s_row", to_np(out["s_row"]), sr)
    else:
        qc, sc = oracle.quantize_colwise(xf, oracle.MODE_LINE, oracle.amax_cols(xf), 448.0)
        assert_same("q_col", to_np(out["q_col"]), qc)
        assert_same("s_col", to_np(out["s_col"]), sc)


@pytest.mark.parametrize("dtype,M,K", [(torch.float32, 4097, 2880), (torch.bfloat16, 401, 528)])
def test_general_shapes_tensor_and_rowgroup_modes(dtype, M, K):
    """Per-tensor amax in both directions, and the row-group column mode
    (block b of a column takes amax[16 b]) with cut blocks at the bottom."""
    say(f"[gpu] general {M}x{K} {dtype} tensor / rowgroup modes")
    g = torch.Generator().manual_seed(M + K + 1)
    x = (torch.randn(M, K, generator=g) * 10.0).to(dtype)
    xf = x.float().numpy()
    xd = x.to(DEV)
    _, _, ta = gpu_amax(xd, row=False, col=False, tensor=True)
    out = gpu_quantize(xd, 0, ta, 0, ta, 256.0)
    t = float(oracle.amax_tensor(xf))
    qr, sr = oracle.quantize_rowwise(xf, oracle.MODE_TENSOR, t, 256.0)
    qc, sc = oracle.quantize_colwise(xf, oracle.MODE_TENSOR, t, 256.0)
    for name, got, want in (("q_row", out["q_row"], qr), ("s_row", out["s_row"], sr),
                            ("q_col", out["q_col"], qc), ("s_col", out["s_col"], sc)):
        assert_same(name, to_np(got), want)
    ends = np.array([16 * 5, 16 * 9, M], dtype=np.int64)
    ga = oracle.group_amax_expand(oracle.amax_rows(xf), ends)
    gad = torch.from_numpy(ga).to(DEV)
    out = gpu_quantize(xd, 1, gad, 2, gad, 448.0)
    qr, sr = oracle.quantize_rowwise(xf, oracle.MODE_LINE, ga, 448.0)
    qc, sc = oracle.quantize_colwise(xf, oracle.MODE_ROWGROUP, ga, 448.0)
    for name, got, want in (("q_row", out["q_row"], qr), ("s_row", out["s_row"], sr),
                            ("q_col", out["q_col"], qc), ("s_col", out["s_col"], sc)):
        assert_same(name + " rowgroup", to_np(got), want)


@pytest.mark.parametrize("shift", [1, 2, 3, 5])
def test_general_shapes_outputs_at_odd_offsets(shift):
    """Transposed codes and both scale copies starting at odd byte offsets
    (views into larger buffers): every row start has another alignment, and
    nothing outside the outputs' bytes is written."""
    M, K = 259, 528
    say(f"[gpu] general {M}x{K} outputs shifted by {shift} bytes")
    g = torch.Generator().manual_seed(shift)
    x = (torch.randn(M, K, generator=g) * 3.0).to(torch.bfloat16)
    xf = x.float().numpy()
    xd = x.to(DEV)
    ra, ca, _ = gpu_amax(xd)
    sizes = {"q_row": M * (K // 2), "s_row": M * (K // 16), "q_col": K * ((M + 1) // 2),
             "s_col": K * ((M + 15) // 16)}
    bufs, views = {}, {}
    for name, n in sizes.items():
        sh = 4 * shift if name == "q_row" else shift  # rowwise codes: dword-aligned rows
        bufs[name] = torch.full((n + 64,), 0xA5, dtype=torch.uint8, device=DEV)
        views[name] = bufs[name][sh:sh + n]
    p.nvfp4_quantize_transpose(xd, 1, ra, 1, ca, 448.0, views["q_row"], views["s_row"],
                               views["q_col"], views["s_col"])
    qr, sr = oracle.quantize_rowwise(xf, oracle.MODE_LINE, oracle.amax_rows(xf), 448.0)
    qc, sc = oracle.quantize_colwise(xf, oracle.MODE_LINE, oracle.amax_cols(xf), 448.0)
    for name, want in (("q_row", qr), ("s_row", sr), ("q_col", qc), ("s_col", sc)):
        b = to_np(bufs[name])
        sh = 4 * shift if name == "q_row" else shift
        assert_same(name, b[sh:sh + sizes[name]], want.ravel())
        assert (b[:sh] == 0xA5).all() and (b[sh + sizes[name]:] == 0xA5).all(), name


@pytest.mark.parametrize("M,K", [(128, 256), (384, 768), (640, 256), (192, 512), (448, 512)])
def test_interior_half_macro_tiles(M, K):
    """M % 256 = 128 or 192: the interior kernel's last macro row is a 128-row
    half tile (flushed after one sub-step), and for 192 the last 64 rows go to
    the edge kernel."""
    g = torch.Generator().manual_seed(3 * M + K)
    x = (torch.randn(M, K, generator=g) * torch.pow(10.0, torch.rand(M, 1, generator=g) * 4 - 2))
    check_row_scaled(x.to(torch.bfloat16), bounds=(448.0,), label=f"half tiles {M}x{K}")


def test_fused_equals_two_kernel_bytes():
    """Fused-amax PR, description: an exact max does not depend on the
    order of evaluation, so the one-pass and the two-kernel amax must agree
    in every bit."""
    w = workloads.make("llm_mlp", (1024, 2048))
    x = w.x.to(DEV)
    assert p.nvfp4_amax_path(p.NVFP4_BF16, 1024, 2048, 1, 1, 0) == 1
    ra1, ca1, _ = gpu_amax(x)
    ra2, ca2, _ = gpu_amax(x, flags=p.NVFP4_FLAG_FORCE_TWO_KERNEL)
    assert_same("row", f32_bits(ra1), f32_bits(ra2))
    assert_same("col", f32_bits(ca1), f32_bits(ca2))


@pytest.mark.parametrize("M,K", [(256, 512), (1024, 2048)])
def test_misaligned_x_takes_the_two_kernel_amax(M, K):
    """A BF16 view two bytes past a 16-byte boundary: the fused pass reads
    16-byte vectors, so the call sends it to the two-kernel path, with the
    oracle's bits either way."""
    w = workloads.make("llm_mlp", (M, K))
    base = torch.empty(M * K + 8, dtype=torch.bfloat16, device=DEV)
    x = base[1:1 + M * K].view(M, K)
    x.copy_(w.x.to(DEV))
    assert x.data_ptr() % 16 == 2 and x.is_contiguous()
    xf = w.x.float().numpy()
    ra, ca, _ = gpu_amax(x)
    assert_same("row", f32_bits(ra), oracle.amax_rows(xf).view(np.uint32))
    assert_same("col", f32_bits(ca), oracle.amax_cols(xf).view(np.uint32))
    out = gpu_quantize(x, 1, ra, 1, ca, 448.0)
    qr, sr = oracle.quantize_rowwise(xf, oracle.MODE_LINE, oracle.amax_rows(xf), 448.0)
    assert_same("q_row", to_np(out["q_row"]), qr)
    assert_same("s_row", to_np(out["s_row"]), sr)


def test_tensor_amax_and_per_tensor_quantize():
    w = workloads.make("outliers", (300, 200))
    x = w.x.to(DEV)
    xf = w.x.float().numpy()
    _, _, ta = gpu_amax(x, row=False, col=False, tensor=True)
    ta_o = oracle.amax_tensor(xf)
    assert f32_bits(ta)[0] == np.float32(ta_o).view(np.uint32)
    for bound in (448.0, 256.0):
        out = gpu_quantize(x, p.NVFP4_AMAX_TENSOR, ta, p.NVFP4_AMAX_TENSOR, ta, bound)
        qr, sr = oracle.quantize_rowwise(xf, oracle.MODE_TENSOR, [ta_o], bound)
        qc, sc = oracle.quantize_colwise(xf, oracle.MODE_TENSOR, [ta_o], bound)
        assert_same("q_row", to_np(out["q_row"]), qr)
        assert_same("s_row", to_np(out["s_row"]), sr)
        assert_same("q_col", to_np(out["q_col"]), qc)
        assert_same("s_col", to_np(out["s_col"]), sc)


@pytest.mark.parametrize("rowwise,colwise", [(True, False), (False, True)])
def test_single_direction(rowwise, colwise):
    w = workloads.make("tiny_rowscale", (96, 80))
    x = w.x.to(DEV)
    xf = w.x.float().numpy()
    ra, ca, _ = gpu_amax(x, row=rowwise, col=colwise)
    out = gpu_quantize(x, 1, ra, 1, ca, 448.0, rowwise=rowwise, colwise=colwise)
    if rowwise:
        q, s = oracle.quantize_rowwise(xf, 1, oracle.amax_rows(xf), 448.0)
        assert_same("q_row", to_np(out["q_row"]), q)
        assert_same("s_row", to_np(out["s_row"]), s)
    else:
        q, s = oracle.quantize_colwise(xf, 1, oracle.amax_cols(xf), 448.0)
        assert_same("q_col", to_np(out["q_col"]), q)
        assert_same("s_col", to_np(out["s_col"]), s)


# ------------------------------------------------------------ dequant matrix
@pytest.mark.parametrize("bound", [448.0, 256.0])
@pytest.mark.parametrize("mode", [p.NVFP4_AMAX_TENSOR, p.NVFP4_AMAX_LINE])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_dequant_matrix(bound, mode, out_dtype):
    """Backward-overrides PR validation: 256/448 x per-tensor/row-scaled x
    bf16/fp32 output."""
    w = workloads.make("tiny_rowscale", (160, 272))
    x = w.x.to(DEV)
    xf = w.x.float().numpy()
    M, K = xf.shape
    if mode == p.NVFP4_AMAX_TENSOR:
        _, _, a = gpu_amax(x, row=False, col=False, tensor=True)
        a_o = np.array([oracle.amax_tensor(xf)], dtype=np.float32)
    else:
        a, _, _ = gpu_amax(x, col=False)
        a_o = oracle.amax_rows(xf)
    out = gpu_quantize(x, mode, a, mode, a, bound, colwise=False)
    q, s = oracle.quantize_rowwise(xf, mode, a_o, bound)
    assert_same("q_row", to_np(out["q_row"]), q)
    y = gpu_dequant(out["q_row"], out["s_row"], M, K, mode, a, bound, out_dtype)
    assert_same("dequant", dequant_bits(y), oracle_dequant_bits(q, s, M, K, mode, a_o, bound, out_dtype))


def test_dequant_random_codes_all_bytes():
    """Every code nibble and every finite non-negative scale byte."""
    R, C = 127, 160
    g = torch.Generator().manual_seed(9)
    q = torch.randint(0, 256, (R, C // 2), generator=g, dtype=torch.uint8)
    s = torch.randint(0, 127, (R, C // 16), generator=g, dtype=torch.uint8)
    s.view(-1)[:127] = torch.arange(127, dtype=torch.uint8)
    a = (torch.rand(R, generator=g) * 100).float()
    for od in (torch.bfloat16, torch.float32):
        y = gpu_dequant(q.to(DEV), s.to(DEV), R, C, p.NVFP4_AMAX_LINE, a.to(DEV), 448.0, od)
        assert_same(f"dequant {od}", dequant_bits(y),
                    oracle_dequant_bits(q.numpy(), s.numpy(), R, C, 1, a.numpy(), 448.0, od))


@pytest.mark.parametrize("R,C,shift", [(33, 4112, 0), (33, 4112, 1), (19, 150, 0), (5, 2064, 0)])
@pytest.mark.parametrize("od", [torch.bfloat16, torch.float32])
def test_dequant_signed_scales_chunks_and_alignment(R, C, shift, od):
    """Scale bytes with the sign bit set decode to negative scales; lines that
    span several vector chunks with a ragged last one (C = 4112, 2064), an
    output that starts off a 16-byte boundary (shift = 1 element: the general
    kernel) and a line length that is not a whole number of blocks (C = 150)."""
    g = torch.Generator().manual_seed(11 + R + C + shift)
    qrs, nb = (C + 1) // 2, (C + 15) // 16
    q = torch.randint(0, 256, (R, qrs), generator=g, dtype=torch.uint8)
    s = torch.randint(0, 127, (R, nb), generator=g, dtype=torch.uint8)
    s = torch.where(torch.rand(R, nb, generator=g) < 0.5, s, s | 0x80)  # 0x80..0xFE
    a = (torch.rand(R, generator=g) * 100).float()
    dev = torch.device("cuda:0")
    say(f"[gpu] dequant signed scales {R}x{C} shift={shift} {od}")
    base = torch.empty(R * C + 8, dtype=od, device=dev)
    y = base[shift:shift + R * C].view(R, C)
    p.nvfp4_dequantize(q.to(dev), s.to(dev), R, C, p.NVFP4_AMAX_LINE, a.to(dev), 448.0, y)
    assert_same(f"dequant {od}", dequant_bits(y.clone()),
                oracle_dequant_bits(q.numpy(), s.numpy(), R, C, 1, a.numpy(), 448.0, od))


# ---------------------------------------------------------------- noop
def test_noop_leaves_every_buffer_untouched():
    """Fused-amax PR review: a call skipped by noop must not erase the
    preserved amax state -- nor any other output."""
    w = workloads.make("outliers", (256, 512))
    x = w.x.to(DEV)
    noop = torch.ones(1, device=DEV)
    for flags in (0, p.NVFP4_FLAG_FORCE_TWO_KERNEL):
        ra, ca, ta = gpu_amax(x, tensor=True, flags=flags, noop=noop)
        torch.cuda.synchronize()
        assert (ra == -7.0).all() and (ca == -7.0).all() and (ta == -7.0).all()
    ra, ca, _ = gpu_amax(x)
    before = [t.clone() for t in (ra, ca)]
    p.nvfp4_amax_rowcol(x, ra, ca, noop=noop)
    assert all(torch.equal(a, b) for a, b in zip(before, (ra, ca)))
    out = gpu_quantize(x, 1, ra, 1, ca, 448.0, noop=noop)
    torch.cuda.synchronize()
    for k, v in out.items():
        assert (v == 0xA5).all(), k
    y = torch.full((256, 512), 3.0, device=DEV)
    q = torch.zeros(256, 256, dtype=torch.uint8, device=DEV)
    s = torch.zeros(256, 32, dtype=torch.uint8, device=DEV)
    p.nvfp4_dequantize(q, s, 256, 512, 1, ra, 448.0, y, noop=noop)
    ge = torch.tensor([100, 256], dtype=torch.int64, device=DEV)
    r2 = ra.clone()
    p.nvfp4_group_amax_expand(r2, ge, noop=noop)
    torch.cuda.synchronize()
    assert (y == 3.0).all() and torch.equal(r2, ra)


@pytest.mark.parametrize("val", [0.0, 2.0, -1.0])
def test_noop_other_values_run(val):
    w = workloads.make("tiny_rowscale", (64, 64))
    x = w.x.to(DEV)
    noop = torch.full((1,), val, device=DEV)
    ra, ca, _ = gpu_amax(x, noop=noop)
    xf = w.x.float().numpy()
    assert_same("row", f32_bits(ra), oracle.amax_rows(xf).view(np.uint32))


# --------------------------------------------------------- grouped tokens
def test_group_expand_matches_oracle():
    g = torch.Generator().manual_seed(3)
    ra = torch.rand(1000, generator=g) * 10
    ge = torch.tensor([0, 128, 128, 384, 1000], dtype=torch.int64)
    r = ra.to(DEV)
    p.nvfp4_group_amax_expand(r, ge.to(DEV))
    want = oracle.group_amax_expand(ra.numpy(), ge.numpy())
    assert_same("expanded", f32_bits(r), want.view(np.uint32))


@pytest.mark.parametrize("ends,first_bad", [
    ([0, 128, 128, 384, 1000], 0),       # valid: the last end (M) need not be aligned
    ([16, 40, 1000], 2),                 # group 1 ends (group 2 starts) at row 40
    ([128, 64, 1000], 2),                # decreasing
    ([128, 1001], 2),                    # past M
    ([-16, 1000], 1),
    ([992], 0),                          # rows past the last group: allowed when aligned
    ([995], 1),                          # ... not when the last end is not a multiple of 16
])
def test_group_expand_validates_on_device(ends, first_bad):
    """With a status buffer the ends are checked on the device: status 0 and
    the expansion when every end lies in [0, M], in order, and is a multiple
    of 16 unless it equals M; otherwise 1 + the first offending group and
    row_amax untouched (the host reads nothing: the caller reads status)."""
    g = torch.Generator().manual_seed(5)
    ra = torch.rand(1000, generator=g) * 10
    r = ra.to(DEV)
    ge = torch.tensor(ends, dtype=torch.int64)
    st = torch.full((1,), -5, dtype=torch.int32, device=DEV)
    p.nvfp4_group_amax_expand(r, ge.to(DEV), status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == first_bad
    if first_bad == 0:
        # rows past the last group keep their values
        want = ra.numpy().copy()
        last = int(ends[-1])
        want[:last] = oracle.group_amax_expand(want[:last], ge.numpy())
        assert_same("expanded", f32_bits(r), want.view(np.uint32))
        # the host-held form of the same ends passes the host check and expands
        r2 = ra.to(DEV)
        p.nvfp4_group_amax_expand(r2, ge)
        assert_same("expanded (host ends)", f32_bits(r2), want.view(np.uint32))
    else:
        assert torch.equal(r.cpu(), ra)
        with pytest.raises(p.Nvfp4Error):
            p.nvfp4_group_amax_expand(ra.to(DEV), ge)  # host ends: rejected before any launch
    # noop = 1: neither the status nor the amax vector is written
    st.fill_(-5)
    r3 = ra.to(DEV)
    p.nvfp4_group_amax_expand(r3, ge.to(DEV), status=st, noop=torch.ones(1, device=DEV))
    torch.cuda.synchronize()
    assert int(st.item()) == -5 and torch.equal(r3.cpu(), ra)


def test_other_stream():
    w = workloads.make("llm_mlp", (256, 1024))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        x = w.x.to(DEV)
        ra, ca, _ = gpu_amax(x)
        out = gpu_quantize(x, 1, ra, 1, ca, 448.0)
    s.synchronize()
    xf = w.x.float().numpy()
    q, sc = oracle.quantize_colwise(xf, 1, oracle.amax_cols(xf), 448.0)
    assert_same("q_col", to_np(out["q_col"]), q)


# ------------------------------------ macro tiles with a partial last strip
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("M,K", [(256, 320), (512, 2880), (320, 576), (384, 1088)])
def test_interior_with_columns_past_the_last_strip(dtype, M, K):
    """K % 256 != 0 (K % 64 == 0): the macro-tile kernel takes the whole
    256-column strips and the edge kernel the remaining columns (and the
    rows below the last macro tile); every output byte against the oracle,
    both directions and each direction alone, per-row and per-tensor."""
    w = workloads.make("llm_mlp", (M, K))
    x_cpu = w.x.to(dtype)
    check_row_scaled(x_cpu, bounds=(448.0,), dequant=False, label="partial strip")
    x = x_cpu.to(DEV)
    xf = x_cpu.float().numpy()
    ra, ca, ta = gpu_amax(x, tensor=True)
    for rw, cw in ((True, False), (False, True)):
        out = gpu_quantize(x, p.NVFP4_AMAX_LINE, ra, p.NVFP4_AMAX_LINE, ca, 256.0, rowwise=rw, colwise=cw)
        if rw:
            q, s = oracle.quantize_rowwise(xf, oracle.MODE_LINE, oracle.amax_rows(xf), 256.0)
            assert_same("q_row", to_np(out["q_row"]), q)
            assert_same("s_row", to_np(out["s_row"]), s)
        if cw:
            q, s = oracle.quantize_colwise(xf, oracle.MODE_LINE, oracle.amax_cols(xf), 256.0)
            assert_same("q_col", to_np(out["q_col"]), q)
            assert_same("s_col", to_np(out["s_col"]), s)
    a = [oracle.amax_tensor(xf)]
    out = gpu_quantize(x, p.NVFP4_AMAX_TENSOR, ta, p.NVFP4_AMAX_TENSOR, ta, 448.0)
    q, s = oracle.quantize_rowwise(xf, oracle.MODE_TENSOR, a, 448.0)
    qc, sc = oracle.quantize_colwise(xf, oracle.MODE_TENSOR, a, 448.0)
    assert_same("q_row tensor", to_np(out["q_row"]), q)
    assert_same("s_row tensor", to_np(out["s_row"]), s)
    assert_same("q_col tensor", to_np(out["q_col"]), qc)
    assert_same("s_col tensor", to_np(out["s_col"]), sc)


# ------------------------------------- BF16 magnitudes over the whole range
@pytest.mark.parametrize("M,K", [(512, 512), (256, 768)])
def test_bf16_whole_exponent_range(M, K):
    """Every output byte against the oracle for BF16 magnitudes from
    subnormal to 2^126, through the macro-tile kernel: both directions and
    each alone, bounds 448 and 256 (dequantize is left out: decode scales
    overflow for amaxes past FLT_MAX / 448)."""
    x_cpu = bf16_exponent_sweep(M, K)
    x, ra, ca = check_row_scaled(x_cpu, bounds=(448.0, 256.0), dequant=False, label="exponent sweep")
    xf = x_cpu.float().numpy()
    for rw, cw in ((True, False), (False, True)):
        out = gpu_quantize(x, p.NVFP4_AMAX_LINE, ra, p.NVFP4_AMAX_LINE, ca, 448.0, rowwise=rw, colwise=cw)
        if rw:
            q, s = oracle.quantize_rowwise(xf, oracle.MODE_LINE, oracle.amax_rows(xf), 448.0)
            assert_same("q_row", to_np(out["q_row"]), q)
            assert_same("s_row", to_np(out["s_row"]), s)
        if cw:
            q, s = oracle.quantize_colwise(xf, oracle.MODE_LINE, oracle.amax_cols(xf), 448.0)
            assert_same("q_col", to_np(out["q_col"]), q)
            assert_same("s_col", to_np(out["s_col"]), s)

"""The one-call row-scaled quantize, nvfp4_quantize_rowcol: the amax pass and
both copies (row-scaled backward PR, sequence diagram: the amax pass, then the
cast writing both copies; fused-amax PR, "Performance": the full quantize).

Every case compares the amax vectors and all four outputs with the oracle,
byte for byte, on shapes that take each of the cast's launch plans (one
macro tile, split halves, several rounds, the general variant with odd M,
FP32, and the checked kernel for K % 16 != 0). The 8192 x 28672 workload is
compared with the two separate calls everywhere and with the oracle on
sampled rows and columns. Also: noop = 1 (no buffer changes, amax vectors
included) and HIP graph capture with new data written into the captured
input between replays."""
from __future__ import annotations

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


def _outputs(M, K):
    out = p.empty_outputs(M, K, DEV)
    for v in out.values():
        v.fill_(0xA5)  # every byte must be overwritten
    ra = torch.full((M,), -7.0, device=DEV)
    ca = torch.full((K,), -7.0, device=DEV)
    return ra, ca, out


def _rowcol(x, bound=448.0, noop=None):
    M, K = x.shape
    ra, ca, out = _outputs(M, K)
    p.nvfp4_quantize_rowcol(x, ra, ca, bound, out["q_row"], out["s_row"], out["q_col"],
                            out["s_col"], noop=noop)
    return ra, ca, out


def _check_oracle(label, x_cpu, ra, ca, out, bound=448.0):
    xf = x_cpu.float().numpy()
    ra_o, ca_o = oracle.amax_rows(xf), oracle.amax_cols(xf)
    assert_same(f"{label} row_amax", f32_bits(ra), ra_o.view(np.uint32))
    assert_same(f"{label} col_amax", f32_bits(ca), ca_o.view(np.uint32))
    qr, sr = oracle.quantize_rowwise(xf, oracle.MODE_LINE, ra_o, bound)
    qc, sc = oracle.quantize_colwise(xf, oracle.MODE_LINE, ca_o, bound)
    assert_same(f"{label} q_row", to_np(out["q_row"]), qr)
    assert_same(f"{label} s_row", to_np(out["s_row"]), sr)
    assert_same(f"{label} q_col", to_np(out["q_col"]), qc)
    assert_same(f"{label} s_col", to_np(out["s_col"]), sc)


def _rows_scale(M, K, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    scale = torch.pow(10.0, -2.0 + 4.0 * torch.rand(M, 1, generator=g))
    return (torch.randn(M, K, generator=g) * scale).to(dtype)


CASES = [
    ("bf16 256x256", 256, 256, torch.bfloat16, 448.0),
    ("bf16 1024x2048", 1024, 2048, torch.bfloat16, 448.0),
    ("bf16 2304x768 bound 256", 2304, 768, torch.bfloat16, 256.0),
    ("bf16 1000x2064 (general)", 1000, 2064, torch.bfloat16, 448.0),
    ("bf16 333x1040 (general, odd M)", 333, 1040, torch.bfloat16, 448.0),
    ("fp32 512x1024", 512, 1024, torch.float32, 448.0),
    ("fp32 777x1552 (general, odd M)", 777, 1552, torch.float32, 448.0),
    ("bf16 300x264 (checked kernel)", 300, 264, torch.bfloat16, 448.0),
    ("fp32 45x7 (checked kernel, two-kernel amax)", 45, 7, torch.float32, 448.0),
]


@pytest.mark.parametrize("label,M,K,dtype,bound", CASES, ids=[c[0] for c in CASES])
def test_rowcol_matches_oracle(label, M, K, dtype, bound):
    x_cpu = _rows_scale(M, K, dtype, seed=M + K)
    say(f"[gpu] quantize_rowcol {label}")
    ra, ca, out = _rowcol(x_cpu.to(DEV), bound)
    torch.cuda.synchronize()
    _check_oracle(label, x_cpu, ra, ca, out, bound)


@pytest.mark.parametrize("name", ["tiny_rowscale", "outliers", "fp32_edge"])
def test_rowcol_workloads(name):
    w = workloads.make(name)
    say(f"[gpu] quantize_rowcol workload {name} {tuple(w.shape)}")
    ra, ca, out = _rowcol(w.x.to(DEV))
    torch.cuda.synchronize()
    _check_oracle(name, w.x, ra, ca, out)


def _sampled_oracle(label, x_cpu, ra, ca, out, rows, cols, bound=448.0):
    """Rows and columns of the outputs against the oracle run on those lines
    alone (a line's codes depend only on the line and its amax)."""
    xf = x_cpu.float().numpy()
    xr = np.ascontiguousarray(xf[rows])
    xc = np.ascontiguousarray(xf[:, cols])
    ra_o = oracle.amax_rows(xr)
    ca_o = oracle.amax_cols(xc)
    assert_same(f"{label} row_amax sample", f32_bits(ra)[rows], ra_o.view(np.uint32))
    assert_same(f"{label} col_amax sample", f32_bits(ca)[cols], ca_o.view(np.uint32))
    qr, sr = oracle.quantize_rowwise(xr, oracle.MODE_LINE, ra_o, bound)
    qc, sc = oracle.quantize_colwise(xc, oracle.MODE_LINE, ca_o, bound)
    assert_same(f"{label} q_row sample", to_np(out["q_row"])[rows], qr)
    assert_same(f"{label} s_row sample", to_np(out["s_row"])[rows], sr)
    assert_same(f"{label} q_col sample", to_np(out["q_col"])[cols], qc)
    assert_same(f"{label} s_col sample", to_np(out["s_col"])[cols], sc)


def test_rowcol_headline_shape():
    """8192 x 28672 BF16 (the LLM MLP workload): the one call against the two
    separate calls on every byte, and against the oracle on sampled lines."""
    w = workloads.make("llm_mlp")
    x = w.x.to(DEV)
    M, K = w.shape
    say("[gpu] quantize_rowcol 8192x28672 bf16")
    ra, ca, out = _rowcol(x)
    ra2, ca2, out2 = _outputs(M, K)
    p.nvfp4_amax_rowcol(x, ra2, ca2)
    p.nvfp4_quantize_transpose(x, p.NVFP4_AMAX_LINE, ra2, p.NVFP4_AMAX_LINE, ca2, 448.0,
                               out2["q_row"], out2["s_row"], out2["q_col"], out2["s_col"])
    torch.cuda.synchronize()
    assert torch.equal(ra, ra2) and torch.equal(ca, ca2)
    for k in out:
        assert torch.equal(out[k], out2[k]), f"{k} differs from the two separate calls"
    g = np.random.RandomState(5)
    rows = np.sort(g.choice(M, 24, replace=False))
    cols = np.sort(g.choice(K, 24, replace=False))
    _sampled_oracle("llm_mlp", w.x, ra, ca, out, rows, cols)


def test_rowcol_noop():
    x = _rows_scale(1024, 2048, torch.bfloat16, 6).to(DEV)
    noop = torch.ones(1, device=DEV)
    ra, ca, out = _rowcol(x, noop=noop)
    torch.cuda.synchronize()
    assert bool((ra == -7.0).all()) and bool((ca == -7.0).all())
    for k, v in out.items():
        assert bool((v == 0xA5).all()), f"noop call wrote {k}"


def test_rowcol_rejects_before_enqueueing():
    x = _rows_scale(256, 256, torch.bfloat16, 7).to(DEV)
    ra, ca, out = _outputs(256, 256)
    lib = p.load_library()
    import ctypes
    vp = lambda t: ctypes.c_void_p(t.data_ptr())
    st = torch.cuda.current_stream(DEV).cuda_stream
    # bound out of range, then a missing copy: NVFP4_ERR_ARG, nothing written
    assert lib.nvfp4_quantize_rowcol(vp(x), p.NVFP4_BF16, 256, 256, ctypes.c_float(500.0), vp(ra),
                                     vp(ca), vp(out["q_row"]), vp(out["s_row"]), vp(out["q_col"]),
                                     vp(out["s_col"]), None, ctypes.c_void_p(st)) == p.NVFP4_ERR_ARG
    assert lib.nvfp4_quantize_rowcol(vp(x), p.NVFP4_BF16, 256, 256, ctypes.c_float(448.0), vp(ra),
                                     vp(ca), vp(out["q_row"]), vp(out["s_row"]), None,
                                     vp(out["s_col"]), None, ctypes.c_void_p(st)) == p.NVFP4_ERR_ARG
    torch.cuda.synchronize()
    assert bool((ra == -7.0).all()) and bool((ca == -7.0).all())
    for k, v in out.items():
        assert bool((v == 0xA5).all()), f"rejected call wrote {k}"


def test_rowcol_graph_replays():
    M, K = 2048, 2048
    x = torch.empty(M, K, dtype=torch.bfloat16, device=DEV)
    ra = torch.empty(M, device=DEV)
    ca = torch.empty(K, device=DEV)
    out = p.empty_outputs(M, K, DEV)

    def step():
        p.nvfp4_quantize_rowcol(x, ra, ca, 448.0, out["q_row"], out["s_row"], out["q_col"],
                                out["s_col"])

    x.copy_(_rows_scale(M, K, torch.bfloat16, 30).to(DEV))
    s = torch.cuda.Stream(DEV)
    s.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream(DEV).wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep, seed in enumerate((31, 32, 33)):
        say(f"[gpu] quantize_rowcol graph replay {rep}")
        xc = _rows_scale(M, K, torch.bfloat16, seed)
        x.copy_(xc.to(DEV))
        for v in out.values():
            v.fill_(0xA5)
        ra.fill_(-7.0)
        ca.fill_(-7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _check_oracle(f"graph replay {rep}", xc, ra, ca, out)

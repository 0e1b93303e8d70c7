"""The path under HIP graph capture (row-scaled backward PR, maintainer
comment: grouped tensors so that the path is CUDA-graph safe; fused-amax PR
review summary: the noop flag exists for calls a replayed graph skips).

Every call only enqueues kernels on the caller's stream, keeps its sizes and
group offsets on the device and clears its own amax state with a kernel, so
a captured sequence can be replayed with new data written in place:

* amax pass + quantize-transpose on a 4096 x 4096 BF16 matrix (row-scaled,
  both copies, fused amax path): three replays, each after writing a new X
  into the captured input, each compared byte for byte with the oracle; then
  a replay with noop = 1, after which every buffer (amax vectors included)
  holds the bytes it held before;
* the one-call grouped quantize: replays after writing new token rows and
  new group sizes into the captured tensors, each compared with the oracle's
  grouped quantize; then a noop replay.

Between replays the program does its own eager work (writing inputs, reading
results) and synchronizes."""
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


def _capture(fn):
    """Warm up fn on a side stream (first-call host caches), then capture it."""
    s = torch.cuda.Stream(DEV)
    s.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream(DEV).wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _snapshot(bufs: dict) -> dict:
    return {k: v.clone() for k, v in bufs.items()}


def _assert_unchanged(before: dict, after: dict) -> None:
    for k in before:
        assert torch.equal(before[k].view(torch.uint8), after[k].view(torch.uint8)), \
            f"noop replay changed {k}"


def _outliers(seed: int, M: int = 4096, K: int = 4096) -> torch.Tensor:
    """The outliers recipe (N(0,1), 0.1 % of the positions set to
    +-U(100, 1000)) with another seed per replay."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(M * K, generator=g)
    idx = torch.randperm(M * K, generator=g)[: (M * K) // 1000]
    sign = torch.where(torch.rand(idx.numel(), generator=g) < 0.5, -1.0, 1.0)
    x[idx] = sign * (100.0 + 900.0 * torch.rand(idx.numel(), generator=g))
    return x.view(M, K).to(torch.bfloat16)


def test_graph_row_scaled_amax_and_quantize():
    M = K = 4096
    x = torch.empty(M, K, dtype=torch.bfloat16, device=DEV)
    ra = torch.empty(M, device=DEV)
    ca = torch.empty(K, device=DEV)
    noop = torch.zeros(1, device=DEV)
    out = p.empty_outputs(M, K, DEV)
    assert p.nvfp4_amax_path(p.NVFP4_BF16, M, K, True, True) == 1

    def step():
        p.nvfp4_amax_rowcol(x, ra, ca, noop=noop)
        p.nvfp4_quantize_transpose(x, p.NVFP4_AMAX_LINE, ra, p.NVFP4_AMAX_LINE, ca, 448.0,
                                   out["q_row"], out["s_row"], out["q_col"], out["s_col"],
                                   noop=noop)

    x.copy_(_outliers(2).to(DEV))
    g = _capture(step)
    for rep, seed in enumerate((7, 8, 9)):
        say(f"[gpu] graph replay {rep}: amax + quantize_transpose 4096x4096 bf16 seed {seed}")
        xc = _outliers(seed)
        x.copy_(xc.to(DEV))
        for v in out.values():
            v.fill_(0xA5)
        ra.fill_(-7.0)
        ca.fill_(-7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        xf = xc.float().numpy()
        ra_o, ca_o = oracle.amax_rows(xf), oracle.amax_cols(xf)
        assert_same("row_amax", f32_bits(ra), ra_o.view(np.uint32))
        assert_same("col_amax", f32_bits(ca), ca_o.view(np.uint32))
        qr, sr = oracle.quantize_rowwise(xf, oracle.MODE_LINE, ra_o, 448.0)
        qc, sc = oracle.quantize_colwise(xf, oracle.MODE_LINE, ca_o, 448.0)
        assert_same("q_row", to_np(out["q_row"]), qr)
        assert_same("s_row", to_np(out["s_row"]), sr)
        assert_same("q_col", to_np(out["q_col"]), qc)
        assert_same("s_col", to_np(out["s_col"]), sc)
    # noop = 1: a replay after new input leaves every buffer as it was
    say("[gpu] graph replay with noop = 1")
    x.copy_(_outliers(10).to(DEV))
    noop.fill_(1.0)
    torch.cuda.synchronize()
    before = _snapshot({"ra": ra, "ca": ca, **out})
    g.replay()
    torch.cuda.synchronize()
    _assert_unchanged(before, {"ra": ra, "ca": ca, **out})
    # and noop = 0 again runs
    noop.fill_(0.0)
    g.replay()
    torch.cuda.synchronize()
    xf = _outliers(10).float().numpy()
    assert_same("row_amax after noop", f32_bits(ra), oracle.amax_rows(xf).view(np.uint32))


def _tokens(T, K, seed):
    g = torch.Generator().manual_seed(seed)
    scale = torch.pow(10.0, -2.0 + 4.0 * torch.rand(T, 1, generator=g))
    return (torch.randn(T, K, generator=g) * scale).to(torch.bfloat16)


def test_graph_grouped_quantize():
    T, K, G, align = 3000, 512, 8, 128
    m_out = p.padded_rows_max(T, G, align)
    x = torch.empty(T, K, dtype=torch.bfloat16, device=DEV)
    rows = torch.empty(G, dtype=torch.int64, device=DEV)
    noop = torch.zeros(1, device=DEV)
    ra = torch.empty(m_out, device=DEV)
    out = p.empty_outputs(m_out, K, DEV)

    def step():
        p.nvfp4_quantize_grouped(x, rows, align, m_out, 448.0, ra, out["q_row"], out["s_row"],
                                 out["q_col"], out["s_col"], noop=noop)

    rng = np.random.RandomState(4)
    x.copy_(_tokens(T, K, 40).to(DEV))
    rows.copy_(torch.from_numpy(rng.multinomial(T, np.ones(G) / G).astype(np.int64)))
    g = _capture(step)
    # ragged sizes, an empty group, a group holding every token
    cases = [rng.multinomial(T, np.ones(G) / G), np.array([0, 700, 1, 0, 1299, 500, 0, 500]),
             np.array([0, 0, 0, T, 0, 0, 0, 0])]
    for rep, sizes in enumerate(cases):
        sizes = sizes.astype(np.int64)
        say(f"[gpu] graph replay {rep}: grouped quantize T={T} K={K} sizes={sizes.tolist()}")
        xc = _tokens(T, K, 41 + rep)
        x.copy_(xc.to(DEV))
        rows.copy_(torch.from_numpy(sizes))
        for v in out.values():
            v.fill_(0xA5)
        ra.fill_(-7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ra_o, qr, sr, qc, sc = oracle.quantize_grouped(xc.float().numpy(), sizes, align, m_out)
        assert_same("row_amax", f32_bits(ra), ra_o.view(np.uint32))
        assert_same("q_row", to_np(out["q_row"]), qr)
        assert_same("s_row", to_np(out["s_row"]), sr)
        assert_same("q_col", to_np(out["q_col"]), qc)
        assert_same("s_col", to_np(out["s_col"]), sc)
    say("[gpu] graph replay with noop = 1 (grouped)")
    x.copy_(_tokens(T, K, 50).to(DEV))
    rows.copy_(torch.from_numpy(rng.multinomial(T, np.ones(G) / G).astype(np.int64)))
    noop.fill_(1.0)
    torch.cuda.synchronize()
    before = _snapshot({"ra": ra, **out})
    g.replay()
    torch.cuda.synchronize()
    _assert_unchanged(before, {"ra": ra, **out})

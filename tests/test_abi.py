"""The C ABI library loads on the host and exports every entry point that
include/nvfp4.h declares; host-side validation and the fused-amax gate work
without a GPU (no call here enqueues device work: each is rejected before any
HIP call, or is the host-only gate query)."""
import ctypes
import os
import re

import pytest

import precision_quantization_row_amd as p

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nvfp4_\w+)\s*\(", text)))


def test_header_and_binding_agree():
    assert _declared() == sorted(p.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = p.load_library()
    for name in _declared():
        assert hasattr(lib, name), name
        assert hasattr(p, name), name  # the binding has the same names


def test_status_strings():
    assert p.status_string(p.NVFP4_OK) == "ok"
    assert p.status_string(p.NVFP4_ERR_ARG) == "invalid argument"
    assert p.status_string(p.NVFP4_ERR_HIP) == "HIP launch failure"


@pytest.mark.parametrize("dtype,M,K,row,col,flags,want", [
    (p.NVFP4_BF16, 256, 512, 1, 1, 0, 1),
    (p.NVFP4_BF16, 8192, 28672, 1, 1, 0, 1),
    (p.NVFP4_FP32, 256, 512, 1, 1, 0, 1),      # FP32 too
    (p.NVFP4_FP32, 4097, 2880, 1, 1, 0, 1),    # ragged M and K with 16-byte rows
    (p.NVFP4_BF16, 257, 520, 1, 1, 0, 1),
    (p.NVFP4_BF16, 256, 524, 1, 1, 0, 2),      # rows that are not whole 16-byte vectors
    (p.NVFP4_FP32, 256, 514, 1, 1, 0, 2),
    (p.NVFP4_BF16, 256, 512, 1, 0, 0, 2),      # one direction only
    (p.NVFP4_BF16, 256, 512, 0, 1, 0, 2),
    (p.NVFP4_BF16, 256, 512, 1, 1, p.NVFP4_FLAG_FORCE_TWO_KERNEL, 2),
    (p.NVFP4_BF16, 256, 512, 0, 0, 0, 0),
])
def test_fused_amax_gate(dtype, M, K, row, col, flags, want):
    assert p.nvfp4_amax_path(dtype, M, K, row, col, flags) == want


def test_fused_amax_kill_switch(monkeypatch):
    monkeypatch.setenv("NVFP4_FUSED_AMAX", "0")
    assert p.nvfp4_amax_path(p.NVFP4_BF16, 256, 512, 1, 1, 0) == 2
    monkeypatch.setenv("NVFP4_FUSED_AMAX", "1")
    assert p.nvfp4_amax_path(p.NVFP4_BF16, 256, 512, 1, 1, 0) == 1


def _fake(addr=0x1000):
    return ctypes.c_void_p(addr)  # never dereferenced: every call below is rejected first


def test_validation_rejects_before_launch():
    lib = p.load_library()
    f = ctypes.c_float
    E = p.NVFP4_ERR_ARG
    # amax: null input, bad sizes, bad dtype, no output, unknown flag
    assert lib.nvfp4_amax_rowcol(None, 0, 4, 4, _fake(), None, None, None, 0, None) == E
    assert lib.nvfp4_amax_rowcol(_fake(), 0, 0, 4, _fake(), None, None, None, 0, None) == E
    assert lib.nvfp4_amax_rowcol(_fake(), 0, 4, -1, _fake(), None, None, None, 0, None) == E
    assert lib.nvfp4_amax_rowcol(_fake(), 7, 4, 4, _fake(), None, None, None, 0, None) == E
    assert lib.nvfp4_amax_rowcol(_fake(), 0, 4, 4, None, None, None, None, 0, None) == E
    assert lib.nvfp4_amax_rowcol(_fake(), 0, 4, 4, _fake(), None, None, None, 8, None) == E
    # quantize: bounds outside (0, 448], NaN, missing buffers, bad modes
    q = lambda bound, rm=1, cm=1, qr=_fake(), sr=_fake(), qc=_fake(), sc=_fake(), ra=_fake(), ca=_fake(): \
        lib.nvfp4_quantize_transpose(_fake(), 0, 32, 32, rm, ra, cm, ca, f(bound), qr, sr, qc, sc, None, None)
    for bad in (0.0, -1.0, 449.0, float("nan"), float("inf")):
        assert q(bad) == E
    assert q(448.0, qr=None, sr=None, qc=None, sc=None) == E
    assert q(448.0, sr=None) == E
    assert q(448.0, sc=None) == E
    assert q(448.0, ra=None) == E
    assert q(448.0, rm=2) == E      # ROWGROUP is for the transposed copy only
    assert q(448.0, cm=3) == E
    # empty matrices are rejected, not launched
    for M, K in ((0, 32), (32, 0), (-1, 32)):
        assert lib.nvfp4_quantize_transpose(_fake(), 0, M, K, 1, _fake(), 1, _fake(), f(448.0),
                                            _fake(), _fake(), _fake(), _fake(), None, None) == E
    # four-over-six: the same validation as the plain quantize
    q46 = lambda bound, M=32, rm=1, cm=1, qr=_fake(), sr=_fake(), qc=_fake(), sc=_fake(), \
        ra=_fake(), ca=_fake(), x=_fake(), dt=0: lib.nvfp4_quantize_4over6(
            x, dt, M, 32, rm, ra, cm, ca, f(bound), qr, sr, qc, sc, None, None)
    for bad in (0.0, -1.0, 449.0, float("nan")):
        assert q46(bad) == E
    for kw in (dict(M=0), dict(x=None), dict(dt=4), dict(qr=None, sr=None, qc=None, sc=None),
               dict(sr=None), dict(ca=None), dict(rm=2), dict(cm=3)):
        assert q46(256.0, **kw) == E, kw
    # dequantize
    d = lambda mode=1, out=0, bound=448.0, R=4, C=16: lib.nvfp4_dequantize(
        _fake(), _fake(), R, C, mode, _fake(), f(bound), _fake(), out, None, None)
    assert d(mode=5) == E
    assert d(out=2) == E
    assert d(bound=500.0) == E
    assert d(R=0) == E
    assert d(C=0) == E
    # quantize-dequantize: missing input / amax / output, half a copy, modes, dtypes
    qd = lambda M=32, K=32, x=_fake(), ra=_fake(), y=_fake(), qr=_fake(), sr=_fake(), mode=1, \
        dt=0, od=0, bound=448.0: lib.nvfp4_quantize_dequantize(x, dt, M, K, mode, ra, f(bound), qr,
                                                                sr, y, od, None, None)
    for kw in (dict(M=0), dict(K=0), dict(x=None), dict(ra=None), dict(y=None), dict(sr=None),
               dict(qr=None), dict(mode=2), dict(dt=5), dict(od=5), dict(bound=-1.0)):
        assert qd(**kw) == E, kw
    # 2-D blocks: missing amax / buffers, sizes, bound, dtype
    t = lambda M=32, K=32, ta=_fake(), bound=448.0, qr=_fake(), sr=_fake(), qc=_fake(), sc=_fake(), \
        dt=0, x=_fake(): lib.nvfp4_quantize_2d(x, dt, M, K, ta, f(bound), qr, sr, qc, sc, None, None)
    for kw in (dict(M=0), dict(K=0), dict(ta=None), dict(x=None), dict(bound=0.0), dict(bound=449.0),
               dict(dt=2), dict(qr=None, sr=None, qc=None, sc=None), dict(sr=None), dict(sc=None)):
        assert t(**kw) == E, kw
    # grouped tokens: sizes, group count, alignment, bound, missing buffers
    g = lambda T=64, K=32, G=4, align=16, M=128, bound=448.0, x=_fake(), gr=_fake(), ra=_fake(), \
        qr=_fake(), sr=_fake(), qc=_fake(), sc=_fake(), dt=0: lib.nvfp4_quantize_grouped(
            x, dt, T, K, gr, G, align, M, f(bound), ra, qr, sr, qc, sc, None, None)
    for kw in (dict(T=0), dict(K=0), dict(M=0), dict(G=0), dict(align=8), dict(align=24),
               dict(align=8192), dict(bound=0.0), dict(bound=500.0), dict(x=None), dict(gr=None),
               dict(ra=None), dict(dt=3), dict(qr=None, sr=None, qc=None, sc=None),
               dict(sr=None), dict(qc=None)):
        assert g(**kw) == E, kw
    assert g(G=p.NVFP4_GROUPS_MAX + 1) == p.NVFP4_ERR_UNSUPPORTED
    assert g(T=1 << 31) == p.NVFP4_ERR_UNSUPPORTED
    assert g(M=(1 << 31) - 1) == p.NVFP4_ERR_UNSUPPORTED
    # group expansion
    assert lib.nvfp4_group_amax_expand(_fake(), 16, _fake(), 0, None, None, None) == E
    assert lib.nvfp4_group_amax_expand(None, 16, _fake(), 2, None, None, None) == E


def test_host_group_end_check():
    """Group ends held on the host are validated before anything is enqueued:
    in [0, M], non-decreasing, and a multiple of 16 unless equal to M (so no
    1x16 block of the transposed copy straddles a group boundary in mode
    ROWGROUP; row-scaled backward PR review: a clear error rather than
    silently wrong results)."""
    import torch
    ok, E = p.NVFP4_OK, p.NVFP4_ERR_ARG
    chk = lambda ends, M: p.nvfp4_check_group_end(torch.tensor(ends, dtype=torch.int64), M)
    assert chk([16, 32, 100], 100) == ok      # last end == M need not be aligned
    assert chk([0, 0, 48, 48], 64) == ok      # empty groups
    assert chk([64], 64) == ok
    assert chk([16, 40, 100], 100) == E       # group 2 starts at row 40
    assert chk([17], 64) == E                 # last end short of M, not aligned
    assert chk([32, 16], 64) == E             # decreasing
    assert chk([-16, 32], 64) == E
    assert chk([16, 80], 64) == E             # past M
    assert p.load_library().nvfp4_check_group_end(None, 2, 64) == E
    assert chk([16], 0) == E
    with pytest.raises(TypeError):
        p.nvfp4_check_group_end(torch.tensor([16], dtype=torch.int32), 16)


def test_binding_rejects_host_tensors():
    import torch
    x = torch.zeros(16, 16, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        p.nvfp4_amax_rowcol(x, torch.zeros(16))


def test_padded_rows_max_bounds_every_layout():
    """The binding's worst-case M_out for grouped tokens covers every split of
    T tokens into G groups (the header's sizing rule)."""
    import numpy as np
    import oracle
    rng = np.random.RandomState(3)
    for _ in range(200):
        G = int(rng.randint(1, 20))
        align = 16 * int(rng.randint(1, 9))
        rows = rng.multinomial(int(rng.randint(0, 500)), np.ones(G) / G)
        T = int(rows.sum())
        need = int(oracle.padded_group_end(rows, align, 1 << 40)[-1])
        bound = p.padded_rows_max(T, G, align)
        assert need <= bound and bound % align == 0
    # the bound is reached: every group one row past a multiple of align
    assert p.padded_rows_max(3 * 17, 3, 16) == int(oracle.padded_group_end([17, 17, 17], 16, 1 << 40)[-1])

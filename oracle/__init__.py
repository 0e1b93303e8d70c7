"""CPU oracle for row-scaled NVFP4 quantize-transpose -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product path (the HIP library and
its Python binding) never imports it, and it imports nothing from the
product. It wraps the scalar C implementation in ``nvfp4_oracle.c`` (every
floating-point step one IEEE binary32 operation, see that file for the
definitions and the page passages they follow) with numpy arrays.

Modes of the second-level amax (same numbering as the C file):
  TENSOR   -- one amax for the whole tensor (per-tensor NVFP4)
  LINE     -- one amax per line (row-scaled: per row, or per column for the
              transposed copy)
  ROWGROUP -- block b of a line uses amax[16*b] (per-group amax expanded along
              the rows, used for the transposed copy of grouped tokens)
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .build import build_oracle, library_path

MODE_TENSOR = 0
MODE_LINE = 1
MODE_ROWGROUP = 2

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        build_oracle()
    lib = ctypes.CDLL(path)
    f32p = ctypes.POINTER(ctypes.c_float)
    u8p = ctypes.POINTER(ctypes.c_uint8)
    i64 = ctypes.c_int64
    i64p = ctypes.POINTER(ctypes.c_int64)
    c_int = ctypes.c_int
    c_f = ctypes.c_float
    sigs = {
        "orc_e2m1_value": (c_f, [c_int]),
        "orc_e2m1_encode": (ctypes.c_uint8, [c_f]),
        "orc_e4m3_value": (c_f, [c_int]),
        "orc_e4m3_encode": (ctypes.c_uint8, [c_f]),
        "orc_factor": (c_f, [c_f]),
        "orc_factor_inv": (c_f, [c_f]),
        "orc_global_encode_scale": (c_f, [c_f, c_f]),
        "orc_quantize_line": (None, [f32p, i64, i64, f32p, c_f, u8p, u8p]),
        "orc_quantize_rowwise": (None, [f32p, i64, i64, c_int, f32p, c_f, u8p, u8p]),
        "orc_quantize_colwise": (None, [f32p, i64, i64, c_int, f32p, c_f, u8p, u8p]),
        "orc_quantize_line_46": (None, [f32p, i64, i64, f32p, c_f, u8p, u8p]),
        "orc_quantize_rowwise_46": (None, [f32p, i64, i64, c_int, f32p, c_f, u8p, u8p]),
        "orc_quantize_colwise_46": (None, [f32p, i64, i64, c_int, f32p, c_f, u8p, u8p]),
        "orc_dequantize": (None, [u8p, u8p, i64, i64, c_int, f32p, c_f, f32p]),
        "orc_quantize_2d": (None, [f32p, i64, i64, c_f, c_f, u8p, u8p, u8p, u8p]),
        "orc_amax_rows": (None, [f32p, i64, i64, f32p]),
        "orc_amax_cols": (None, [f32p, i64, i64, f32p]),
        "orc_amax_tensor": (c_f, [f32p, i64]),
        "orc_group_amax_expand": (None, [f32p, i64p, i64, f32p]),
        "orc_e2m1_encode_array": (None, [f32p, i64, u8p]),
        "orc_e4m3_encode_array": (None, [f32p, i64, u8p]),
        "orc_bf16_round": (ctypes.c_uint16, [c_f]),
        "orc_bf16_round_array": (None, [f32p, i64, ctypes.POINTER(ctypes.c_uint16)]),
        "orc_e2m1_encode_bits": (None, [ctypes.c_uint32, i64, u8p]),
        "orc_e4m3_encode_bits": (None, [ctypes.c_uint32, i64, u8p]),
        "orc_bf16_round_bits": (None, [ctypes.c_uint32, i64, ctypes.POINTER(ctypes.c_uint16)]),
        "orc_div6_bits": (None, [ctypes.c_uint32, i64, f32p]),
        "orc_recip_bits": (None, [ctypes.c_uint32, i64, f32p]),
        "orc_max_threads": (c_int, []),
        "orc_set_threads": (None, [c_int]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _f32(a) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    if not np.isfinite(a).all():
        raise ValueError("oracle inputs must be finite (NaN/inf are outside the contract)")
    return a


def _p(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def set_threads(n: int) -> None:
    """Threads the OpenMP loops over lines use from now on (the bits do not
    depend on it)."""
    _load().orc_set_threads(int(n))


def max_threads() -> int:
    """OpenMP threads the oracle's line loops use."""
    return int(_load().orc_max_threads())


# --------------------------------------------------------------------------- formats
def e2m1_value(code: int) -> float:
    return float(_load().orc_e2m1_value(int(code)))


def e4m3_value(byte: int) -> float:
    return float(_load().orc_e4m3_value(int(byte)))


def e2m1_encode(v) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    if np.isnan(v).any():
        raise ValueError("NaN is outside the contract")
    out = np.empty(v.shape, dtype=np.uint8)
    _load().orc_e2m1_encode_array(_p(v, ctypes.c_float), v.size, _p(out, ctypes.c_uint8))
    return out


def e4m3_encode(s) -> np.ndarray:
    s = np.ascontiguousarray(s, dtype=np.float32)
    if np.isnan(s).any() or (s < 0).any():
        raise ValueError("scales are non-negative and not NaN")
    out = np.empty(s.shape, dtype=np.uint8)
    _load().orc_e4m3_encode_array(_p(s, ctypes.c_float), s.size, _p(out, ctypes.c_uint8))
    return out


def factor_inv(bound: float) -> float:
    return float(_load().orc_factor_inv(float(bound)))


def global_encode_scale(a: float, bound: float) -> float:
    return float(_load().orc_global_encode_scale(float(a), float(bound)))


# --------------------------------------------------------------------------- amax
def amax_rows(X) -> np.ndarray:
    X = _f32(X)
    M, K = X.shape
    out = np.empty(M, dtype=np.float32)
    _load().orc_amax_rows(_p(X, ctypes.c_float), M, K, _p(out, ctypes.c_float))
    return out


def amax_cols(X) -> np.ndarray:
    X = _f32(X)
    M, K = X.shape
    out = np.empty(K, dtype=np.float32)
    _load().orc_amax_cols(_p(X, ctypes.c_float), M, K, _p(out, ctypes.c_float))
    return out


def amax_tensor(X) -> np.float32:
    X = _f32(X)
    return np.float32(_load().orc_amax_tensor(_p(X, ctypes.c_float), X.size))


def group_amax_expand(row_amax, group_end) -> np.ndarray:
    ra = np.ascontiguousarray(row_amax, dtype=np.float32)
    ge = np.ascontiguousarray(group_end, dtype=np.int64)
    if ge.size and (ge[-1] != ra.size or (np.diff(ge) < 0).any() or ge[0] < 0):
        raise ValueError("group_end must be non-decreasing and end at the row count")
    out = np.zeros_like(ra)
    _load().orc_group_amax_expand(_p(ra, ctypes.c_float), _p(ge, ctypes.c_int64), ge.size,
                                  _p(out, ctypes.c_float))
    return out


# --------------------------------------------------------------------------- quantize
def _amax_arg(mode: int, amax, n_lines: int, line_len: int) -> np.ndarray:
    a = np.ascontiguousarray(np.atleast_1d(np.asarray(amax, dtype=np.float32)))
    need = {MODE_TENSOR: 1, MODE_LINE: n_lines, MODE_ROWGROUP: line_len}[mode]
    if a.size != need:
        raise ValueError(f"amax for mode {mode} needs {need} entries, got {a.size}")
    return a


def quantize_rowwise(X, mode: int, amax, bound: float = 448.0):
    """Row i of X -> (codes [M][ceil(K/2)] u8, scales [M][ceil(K/16)] u8)."""
    X = _f32(X)
    M, K = X.shape
    a = _amax_arg(mode, amax, M, K)
    q = np.zeros((M, (K + 1) // 2), dtype=np.uint8)
    s = np.zeros((M, (K + 15) // 16), dtype=np.uint8)
    _load().orc_quantize_rowwise(_p(X, ctypes.c_float), M, K, mode, _p(a, ctypes.c_float),
                                 float(bound), _p(q, ctypes.c_uint8), _p(s, ctypes.c_uint8))
    return q, s


def quantize_colwise(X, mode: int, amax, bound: float = 448.0):
    """Column j of X -> (codes [K][ceil(M/2)] u8, scales [K][ceil(M/16)] u8)."""
    X = _f32(X)
    M, K = X.shape
    a = _amax_arg(mode, amax, K, M)
    q = np.zeros((K, (M + 1) // 2), dtype=np.uint8)
    s = np.zeros((K, (M + 15) // 16), dtype=np.uint8)
    _load().orc_quantize_colwise(_p(X, ctypes.c_float), M, K, mode, _p(a, ctypes.c_float),
                                 float(bound), _p(q, ctypes.c_uint8), _p(s, ctypes.c_uint8))
    return q, s


def quantize_rowwise_46(X, mode: int, amax, bound: float = 256.0):
    """quantize_rowwise with four-over-six block scales: per block, the scale
    that maps the block max to 6 or the one that maps it to 4, whichever
    dequantizes with the smaller squared error (see the C file)."""
    X = _f32(X)
    M, K = X.shape
    a = _amax_arg(mode, amax, M, K)
    q = np.zeros((M, (K + 1) // 2), dtype=np.uint8)
    s = np.zeros((M, (K + 15) // 16), dtype=np.uint8)
    _load().orc_quantize_rowwise_46(_p(X, ctypes.c_float), M, K, mode, _p(a, ctypes.c_float),
                                    float(bound), _p(q, ctypes.c_uint8), _p(s, ctypes.c_uint8))
    return q, s


def quantize_colwise_46(X, mode: int, amax, bound: float = 256.0):
    """quantize_colwise with four-over-six block scales."""
    X = _f32(X)
    M, K = X.shape
    a = _amax_arg(mode, amax, K, M)
    q = np.zeros((K, (M + 1) // 2), dtype=np.uint8)
    s = np.zeros((K, (M + 15) // 16), dtype=np.uint8)
    _load().orc_quantize_colwise_46(_p(X, ctypes.c_float), M, K, mode, _p(a, ctypes.c_float),
                                    float(bound), _p(q, ctypes.c_uint8), _p(s, ctypes.c_uint8))
    return q, s


def quantize_line_46(x, block_amax, bound: float = 256.0):
    """One line with four-over-six block scales and an explicit second-level
    amax per 16-element block."""
    x = _f32(x).ravel()
    n = x.size
    ba = np.ascontiguousarray(block_amax, dtype=np.float32).ravel()
    if ba.size != (n + 15) // 16:
        raise ValueError("one amax per block is required")
    q = np.zeros((n + 1) // 2, dtype=np.uint8)
    s = np.zeros((n + 15) // 16, dtype=np.uint8)
    _load().orc_quantize_line_46(_p(x, ctypes.c_float), n, 1, _p(ba, ctypes.c_float), float(bound),
                                 _p(q, ctypes.c_uint8), _p(s, ctypes.c_uint8))
    return q, s


def quantize_line(x, block_amax, bound: float = 448.0):
    """One line with an explicit second-level amax per 16-element block."""
    x = _f32(x).ravel()
    n = x.size
    ba = np.ascontiguousarray(block_amax, dtype=np.float32).ravel()
    if ba.size != (n + 15) // 16:
        raise ValueError("one amax per block is required")
    q = np.zeros((n + 1) // 2, dtype=np.uint8)
    s = np.zeros((n + 15) // 16, dtype=np.uint8)
    _load().orc_quantize_line(_p(x, ctypes.c_float), n, 1, _p(ba, ctypes.c_float), float(bound),
                              _p(q, ctypes.c_uint8), _p(s, ctypes.c_uint8))
    return q, s


def quantize_2d(X, amax: float, bound: float = 448.0):
    """2-D 16x16 blocks under one per-tensor amax (a reading: the pages name
    TE's 2-D weight blocks only through the switch that turns them off).
    Returns (q_row, s_row, q_col, s_col) in the 1x16 layouts, each tile's
    scale byte repeated on its 16 rows and 16 columns."""
    X = _f32(X)
    M, K = X.shape
    q_row = np.zeros((M, (K + 1) // 2), dtype=np.uint8)
    s_row = np.zeros((M, (K + 15) // 16), dtype=np.uint8)
    q_col = np.zeros((K, (M + 1) // 2), dtype=np.uint8)
    s_col = np.zeros((K, (M + 15) // 16), dtype=np.uint8)
    _load().orc_quantize_2d(_p(X, ctypes.c_float), M, K, float(np.float32(amax)), float(bound),
                            _p(q_row, ctypes.c_uint8), _p(s_row, ctypes.c_uint8),
                            _p(q_col, ctypes.c_uint8), _p(s_col, ctypes.c_uint8))
    return q_row, s_row, q_col, s_col


def dequantize(q, s, R: int, C: int, mode: int, amax, bound: float = 448.0) -> np.ndarray:
    """Codes [R][ceil(C/2)] + scales [R][ceil(C/16)] -> FP32 [R][C]."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    s = np.ascontiguousarray(s, dtype=np.uint8)
    if q.size != R * ((C + 1) // 2) or s.size != R * ((C + 15) // 16):
        raise ValueError("code/scale buffer sizes do not match R x C")
    a = _amax_arg(mode, amax, R, C)
    y = np.empty((R, C), dtype=np.float32)
    _load().orc_dequantize(_p(q, ctypes.c_uint8), _p(s, ctypes.c_uint8), R, C, mode,
                           _p(a, ctypes.c_float), float(bound), _p(y, ctypes.c_float))
    return y


def quantize_dequantize(X, mode: int, amax, bound: float = 448.0):
    """Backward-overrides PR description, "dequantized" policy: the rowwise
    fprop codes and scales are kept and the backward GEMMs run in BF16 on
    their dequantization. This is the rowwise quantize followed by the
    dequantize of that copy, nothing else (both steps pinned on their own).
    Returns (q [M][ceil(K/2)], s [M][ceil(K/16)], y FP32 [M][K])."""
    X = _f32(X)
    M, K = X.shape
    q, s = quantize_rowwise(X, mode, amax, bound)
    return q, s, dequantize(q, s, M, K, mode, amax, bound)


def to_bf16_bits(y: np.ndarray) -> np.ndarray:
    """Backward-overrides PR description (BF16 output of the dequantize): the
    nearest BF16 value to each FP32 value, ties to the even pattern, as uint16
    bit patterns (``orc_bf16_round`` in the C file)."""
    y = np.ascontiguousarray(y, dtype=np.float32)
    out = np.empty(y.shape, dtype=np.uint16)
    _load().orc_bf16_round_array(_p(y, ctypes.c_float), y.size, _p(out, ctypes.c_uint16))
    return out


# ------------------------------------------- runs of binary32 bit patterns
# For exhaustive comparisons of hardware converters and arithmetic shortcuts
# with the definitions: each returns the oracle's result for the patterns
# start, start + 1, ..., start + n - 1 (start + n <= 2^32). Patterns outside
# a function's domain carry a marker (see the C file) that callers mask out.
def _check_run(start: int, n: int) -> None:
    if not (0 <= start and n >= 0 and start + n <= 1 << 32):
        raise ValueError("pattern run outside [0, 2^32)")


def e2m1_encode_bits(start: int, n: int) -> np.ndarray:
    _check_run(start, n)
    out = np.empty(n, dtype=np.uint8)
    _load().orc_e2m1_encode_bits(start, n, _p(out, ctypes.c_uint8))
    return out


def e4m3_encode_bits(start: int, n: int) -> np.ndarray:
    _check_run(start, n)
    out = np.empty(n, dtype=np.uint8)
    _load().orc_e4m3_encode_bits(start, n, _p(out, ctypes.c_uint8))
    return out


def bf16_round_bits(start: int, n: int) -> np.ndarray:
    _check_run(start, n)
    out = np.empty(n, dtype=np.uint16)
    _load().orc_bf16_round_bits(start, n, _p(out, ctypes.c_uint16))
    return out


def div6_bits(start: int, n: int) -> np.ndarray:
    """RN(x / 6) (the block-scale step with top 6), as float32."""
    _check_run(start, n)
    out = np.empty(n, dtype=np.float32)
    _load().orc_div6_bits(start, n, _p(out, ctypes.c_float))
    return out


def recip_bits(start: int, n: int) -> np.ndarray:
    """min(RN(1 / D), FLT_MAX) for D > 0 (the encode-factor step), float32."""
    _check_run(start, n)
    out = np.empty(n, dtype=np.float32)
    _load().orc_recip_bits(start, n, _p(out, ctypes.c_float))
    return out


# ------------------------------------------------------------ grouped tokens
def pad_groups(x_tokens, group_rows, align: int, m_out: int) -> np.ndarray:
    """Grouped-GEMM PR description (ragged token groups zero-padded to 128-row
    alignment before quantization): the G groups of x_tokens [T][K] (group g
    holds group_rows[g] consecutive rows) laid out in an [m_out][K] matrix,
    group g starting at the sum of the earlier groups' sizes rounded up to
    `align`, every other row zero. Rows that do not fit in m_out are
    dropped; token rows past T read as zero."""
    x = _f32(x_tokens)
    T, K = x.shape
    out = np.zeros((m_out, K), dtype=np.float32)
    p = t = 0
    for n in np.asarray(group_rows, dtype=np.int64).tolist():
        for r in range(n):
            if p + r < m_out and t + r < T:
                out[p + r] = x[t + r]
        t += n
        p += -(-n // align) * align
    return out


def padded_group_end(group_rows, align: int, m_out: int) -> np.ndarray:
    """End row (exclusive) of every padded group, clipped to m_out."""
    ends, p = [], 0
    for n in np.asarray(group_rows, dtype=np.int64).tolist():
        p += -(-n // align) * align
        ends.append(min(p, m_out))
    return np.asarray(ends, dtype=np.int64)


def quantize_grouped(x_tokens, group_rows, align: int, m_out: int, bound: float = 448.0):
    """Grouped tokens, padded on the way in: per-group amax expanded over each
    padded group (rows past the last group get 0), rowwise codes with that
    per-row amax, transposed codes with the group amax of each 16-row block
    (grouped-GEMM PR description: equal to quantizing each split on its own).
    Returns (row_amax [m_out], q_row, s_row, q_col, s_col)."""
    xp = pad_groups(x_tokens, group_rows, align, m_out)
    ends = padded_group_end(group_rows, align, m_out)
    last = int(ends[-1]) if ends.size else 0
    ra = np.zeros(m_out, dtype=np.float32)
    if last:
        ra[:last] = group_amax_expand(amax_rows(xp[:last]), ends)
    q_row, s_row = quantize_rowwise(xp, MODE_LINE, ra, bound)
    q_col, s_col = quantize_colwise(xp, MODE_ROWGROUP, ra, bound)
    return ra, q_row, s_row, q_col, s_col

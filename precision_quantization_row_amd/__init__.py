"""Row-scaled NVFP4 quantize-transpose for AMD Instinct MI355X (gfx950).

A thin ctypes binding over ``libnvfp4.so`` (the C ABI declared in
``include/nvfp4.h``). Every function here has the name of the C entry point
it calls and only marshals arguments: it checks dtypes, shapes, contiguity
and devices of torch tensors, passes their device pointers and the current
HIP stream, and raises on a non-zero status. All computation runs in the HIP
kernels; there is no CPU fallback, and importing a function whose library is
missing raises.

Layouts (row-major, packed, no pitch):
  x      [M, K] bfloat16 or float32
  q_row  [M, ceil(K/2)] uint8   s_row [M, ceil(K/16)] uint8 (or float8_e4m3fn)
  q_col  [K, ceil(M/2)] uint8   s_col [K, ceil(M/16)] uint8 (or float8_e4m3fn)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

from .build import library_path

NVFP4_OK = 0
NVFP4_ERR_ARG = -1
NVFP4_ERR_UNSUPPORTED = -2
NVFP4_ERR_HIP = -3

NVFP4_BF16 = 0
NVFP4_FP32 = 1

NVFP4_AMAX_TENSOR = 0
NVFP4_AMAX_LINE = 1
NVFP4_AMAX_ROWGROUP = 2

NVFP4_FLAG_FORCE_TWO_KERNEL = 1

# Every entry point include/nvfp4.h declares.
EXPORTED = ("nvfp4_amax_path", "nvfp4_amax_rowcol", "nvfp4_group_amax_expand",
            "nvfp4_check_group_end",
            "nvfp4_quantize_transpose", "nvfp4_quantize_rowcol", "nvfp4_quantize_4over6",
            "nvfp4_quantize_2d",
            "nvfp4_quantize_grouped",
            "nvfp4_quantize_dequantize", "nvfp4_dequantize",
            "nvfp4_status_string")

NVFP4_GROUPS_MAX = 256

_lib = None


class Nvfp4Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status_string(status)} ({status})")
        self.status = status


def load_library():
    """Load libnvfp4.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with __graft_entry__.build() "
                          "(the HIP library is required; there is no fallback)")
    lib = ctypes.CDLL(path)
    vp, f32p, u8p, i64p = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
    i64, c_int, c_uint, c_f = ctypes.c_int64, ctypes.c_int, ctypes.c_uint, ctypes.c_float
    lib.nvfp4_status_string.restype = ctypes.c_char_p
    lib.nvfp4_status_string.argtypes = [c_int]
    lib.nvfp4_amax_path.restype = c_int
    lib.nvfp4_amax_path.argtypes = [c_int, i64, i64, c_int, c_int, c_uint]
    lib.nvfp4_amax_rowcol.restype = c_int
    lib.nvfp4_amax_rowcol.argtypes = [vp, c_int, i64, i64, f32p, f32p, f32p, f32p, c_uint, vp]
    lib.nvfp4_group_amax_expand.restype = c_int
    lib.nvfp4_group_amax_expand.argtypes = [f32p, i64, i64p, i64, vp, f32p, vp]
    lib.nvfp4_check_group_end.restype = c_int
    lib.nvfp4_check_group_end.argtypes = [i64p, i64, i64]
    lib.nvfp4_quantize_transpose.restype = c_int
    lib.nvfp4_quantize_transpose.argtypes = [vp, c_int, i64, i64, c_int, f32p, c_int, f32p, c_f,
                                             u8p, u8p, u8p, u8p, f32p, vp]
    lib.nvfp4_quantize_4over6.restype = c_int
    lib.nvfp4_quantize_rowcol.restype = c_int
    lib.nvfp4_quantize_rowcol.argtypes = [vp, c_int, i64, i64, c_f, f32p, f32p, u8p, u8p, u8p, u8p,
                                          f32p, vp]
    lib.nvfp4_quantize_4over6.argtypes = [vp, c_int, i64, i64, c_int, f32p, c_int, f32p, c_f,
                                          u8p, u8p, u8p, u8p, f32p, vp]
    lib.nvfp4_quantize_2d.restype = c_int
    lib.nvfp4_quantize_2d.argtypes = [vp, c_int, i64, i64, f32p, c_f, u8p, u8p, u8p, u8p, f32p, vp]
    lib.nvfp4_quantize_grouped.restype = c_int
    lib.nvfp4_quantize_grouped.argtypes = [vp, c_int, i64, i64, i64p, i64, i64, i64, c_f, f32p,
                                           u8p, u8p, u8p, u8p, f32p, vp]
    lib.nvfp4_quantize_dequantize.restype = c_int
    lib.nvfp4_quantize_dequantize.argtypes = [vp, c_int, i64, i64, c_int, f32p, c_f, u8p, u8p, vp,
                                              c_int, f32p, vp]
    lib.nvfp4_dequantize.restype = c_int
    lib.nvfp4_dequantize.argtypes = [u8p, u8p, i64, i64, c_int, f32p, c_f, vp, c_int, f32p, vp]
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().nvfp4_status_string(int(status)).decode()


def nvfp4_status_string(status: int) -> str:
    return status_string(status)


# ----------------------------------------------------------------- marshalling
def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return NVFP4_BF16
    if t.dtype == torch.float32:
        return NVFP4_FP32
    raise TypeError(f"expected bfloat16 or float32, got {t.dtype}")


def _dev(t: Optional[torch.Tensor], name: str, dtypes, numel: Optional[int] = None,
         device: Optional[torch.device] = None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must have {numel} entries, got {t.numel()}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return t


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, device) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


_SCALE_DTYPES = (torch.uint8, torch.float8_e4m3fn)
_F32 = (torch.float32,)


def _check(fn: str, status: int):
    if status != NVFP4_OK:
        raise Nvfp4Error(fn, status)


# ------------------------------------------------------------------ entry points
def nvfp4_amax_path(in_dtype: int, M: int, K: int, want_row: bool, want_col: bool,
                    flags: int = 0) -> int:
    return int(load_library().nvfp4_amax_path(in_dtype, M, K, int(want_row), int(want_col), flags))


def nvfp4_amax_rowcol(x: torch.Tensor, row_amax: Optional[torch.Tensor] = None,
                      col_amax: Optional[torch.Tensor] = None,
                      tensor_amax: Optional[torch.Tensor] = None,
                      noop: Optional[torch.Tensor] = None, flags: int = 0, stream=None) -> None:
    """row_amax [M], col_amax [K], tensor_amax [1] (float32, any subset)."""
    lib = load_library()
    if x.dim() != 2:
        raise ValueError("x must be 2-D [M, K]")
    _dev(x, "x", (torch.bfloat16, torch.float32))
    M, K = x.shape
    dev = x.device
    _dev(row_amax, "row_amax", _F32, M, dev)
    _dev(col_amax, "col_amax", _F32, K, dev)
    _dev(tensor_amax, "tensor_amax", _F32, 1, dev)
    _dev(noop, "noop", _F32, 1, dev)
    st = lib.nvfp4_amax_rowcol(_ptr(x), _dtype_code(x), M, K, _ptr(row_amax), _ptr(col_amax),
                               _ptr(tensor_amax), _ptr(noop), flags, _stream(stream, dev))
    _check("nvfp4_amax_rowcol", st)


def nvfp4_check_group_end(group_end: torch.Tensor, M: int) -> int:
    """Host-side validation of group ends held in host memory (int64 CPU
    tensor); returns the C status (NVFP4_OK or NVFP4_ERR_ARG)."""
    if not isinstance(group_end, torch.Tensor) or group_end.is_cuda:
        raise ValueError("group_end must be a host (CPU) tensor")
    if group_end.dtype != torch.int64 or not group_end.is_contiguous():
        raise TypeError("group_end must be a contiguous int64 tensor")
    return int(load_library().nvfp4_check_group_end(ctypes.c_void_p(group_end.data_ptr()),
                                                    group_end.numel(), int(M)))


def nvfp4_group_amax_expand(row_amax: torch.Tensor, group_end: torch.Tensor,
                            status: Optional[torch.Tensor] = None,
                            noop: Optional[torch.Tensor] = None, stream=None) -> None:
    """group_end: an int64 device tensor (validated on the device when a
    status [1] int32 device tensor is given), or an int64 CPU tensor, which
    is validated on the host (Nvfp4Error with NVFP4_ERR_ARG when a group
    boundary is misaligned) and then copied to the device."""
    lib = load_library()
    _dev(row_amax, "row_amax", _F32)
    dev = row_amax.device
    if isinstance(group_end, torch.Tensor) and not group_end.is_cuda:
        _check("nvfp4_check_group_end", nvfp4_check_group_end(group_end, row_amax.numel()))
        group_end = group_end.to(dev)
    _dev(group_end, "group_end", (torch.int64,), None, dev)
    _dev(status, "status", (torch.int32,), 1, dev)
    _dev(noop, "noop", _F32, 1, dev)
    st = lib.nvfp4_group_amax_expand(_ptr(row_amax), row_amax.numel(), _ptr(group_end),
                                     group_end.numel(), _ptr(status), _ptr(noop),
                                     _stream(stream, dev))
    _check("nvfp4_group_amax_expand", st)


def _amax_numel(mode: int, lines: int, length: int) -> int:
    return {NVFP4_AMAX_TENSOR: 1, NVFP4_AMAX_LINE: lines, NVFP4_AMAX_ROWGROUP: length}.get(mode, -1)


def nvfp4_quantize_transpose(x: torch.Tensor, row_mode: int, row_amax: Optional[torch.Tensor],
                             col_mode: int, col_amax: Optional[torch.Tensor], bound: float,
                             q_row: Optional[torch.Tensor], s_row: Optional[torch.Tensor],
                             q_col: Optional[torch.Tensor], s_col: Optional[torch.Tensor],
                             noop: Optional[torch.Tensor] = None, stream=None) -> None:
    _quantize("nvfp4_quantize_transpose", x, row_mode, row_amax, col_mode, col_amax, bound,
              q_row, s_row, q_col, s_col, noop, stream)


def nvfp4_quantize_rowcol(x: torch.Tensor, row_amax: torch.Tensor, col_amax: torch.Tensor,
                          bound: float, q_row: torch.Tensor, s_row: torch.Tensor,
                          q_col: torch.Tensor, s_col: torch.Tensor,
                          noop: Optional[torch.Tensor] = None, stream=None) -> None:
    """The whole row-scaled quantize in one call: row_amax [M] and col_amax
    [K] are written, then both copies (mode LINE)."""
    lib = load_library()
    if x.dim() != 2:
        raise ValueError("x must be 2-D [M, K]")
    _dev(x, "x", (torch.bfloat16, torch.float32))
    M, K = x.shape
    dev = x.device
    _dev(row_amax, "row_amax", _F32, M, dev)
    _dev(col_amax, "col_amax", _F32, K, dev)
    _dev(q_row, "q_row", (torch.uint8,), M * ((K + 1) // 2), dev)
    _dev(s_row, "s_row", _SCALE_DTYPES, M * ((K + 15) // 16), dev)
    _dev(q_col, "q_col", (torch.uint8,), K * ((M + 1) // 2), dev)
    _dev(s_col, "s_col", _SCALE_DTYPES, K * ((M + 15) // 16), dev)
    _dev(noop, "noop", _F32, 1, dev)
    st = lib.nvfp4_quantize_rowcol(_ptr(x), _dtype_code(x), M, K, ctypes.c_float(bound),
                                   _ptr(row_amax), _ptr(col_amax), _ptr(q_row), _ptr(s_row),
                                   _ptr(q_col), _ptr(s_col), _ptr(noop), _stream(stream, dev))
    _check("nvfp4_quantize_rowcol", st)


def nvfp4_quantize_4over6(x: torch.Tensor, row_mode: int, row_amax: Optional[torch.Tensor],
                          col_mode: int, col_amax: Optional[torch.Tensor], bound: float,
                          q_row: Optional[torch.Tensor], s_row: Optional[torch.Tensor],
                          q_col: Optional[torch.Tensor], s_col: Optional[torch.Tensor],
                          noop: Optional[torch.Tensor] = None, stream=None) -> None:
    """nvfp4_quantize_transpose with four-over-six block scales."""
    _quantize("nvfp4_quantize_4over6", x, row_mode, row_amax, col_mode, col_amax, bound,
              q_row, s_row, q_col, s_col, noop, stream)


def _quantize(name, x, row_mode, row_amax, col_mode, col_amax, bound, q_row, s_row, q_col, s_col,
              noop, stream) -> None:
    lib = load_library()
    if x.dim() != 2:
        raise ValueError("x must be 2-D [M, K]")
    _dev(x, "x", (torch.bfloat16, torch.float32))
    M, K = x.shape
    dev = x.device
    if q_row is not None:
        _dev(row_amax, "row_amax", _F32, _amax_numel(row_mode, M, K), dev)
        _dev(q_row, "q_row", (torch.uint8,), M * ((K + 1) // 2), dev)
        _dev(s_row, "s_row", _SCALE_DTYPES, M * ((K + 15) // 16), dev)
    if q_col is not None:
        # ROWGROUP: the transposed lines' blocks index an [M] per-row vector
        _dev(col_amax, "col_amax", _F32, _amax_numel(col_mode, K, M), dev)
        _dev(q_col, "q_col", (torch.uint8,), K * ((M + 1) // 2), dev)
        _dev(s_col, "s_col", _SCALE_DTYPES, K * ((M + 15) // 16), dev)
    _dev(noop, "noop", _F32, 1, dev)
    st = getattr(lib, name)(_ptr(x), _dtype_code(x), M, K, row_mode, _ptr(row_amax), col_mode,
                            _ptr(col_amax), ctypes.c_float(bound), _ptr(q_row), _ptr(s_row),
                            _ptr(q_col), _ptr(s_col), _ptr(noop), _stream(stream, dev))
    _check(name, st)


def nvfp4_quantize_2d(x: torch.Tensor, tensor_amax: torch.Tensor, bound: float,
                      q_row: Optional[torch.Tensor], s_row: Optional[torch.Tensor],
                      q_col: Optional[torch.Tensor], s_col: Optional[torch.Tensor],
                      noop: Optional[torch.Tensor] = None, stream=None) -> None:
    """x [M, K] with 16 x 16 tile scales under the per-tensor amax tensor_amax [1]."""
    lib = load_library()
    if x.dim() != 2:
        raise ValueError("x must be 2-D [M, K]")
    _dev(x, "x", (torch.bfloat16, torch.float32))
    M, K = x.shape
    dev = x.device
    _dev(tensor_amax, "tensor_amax", _F32, 1, dev)
    if q_row is not None:
        _dev(q_row, "q_row", (torch.uint8,), M * ((K + 1) // 2), dev)
        _dev(s_row, "s_row", _SCALE_DTYPES, M * ((K + 15) // 16), dev)
    if q_col is not None:
        _dev(q_col, "q_col", (torch.uint8,), K * ((M + 1) // 2), dev)
        _dev(s_col, "s_col", _SCALE_DTYPES, K * ((M + 15) // 16), dev)
    _dev(noop, "noop", _F32, 1, dev)
    st = lib.nvfp4_quantize_2d(_ptr(x), _dtype_code(x), M, K, _ptr(tensor_amax),
                               ctypes.c_float(bound), _ptr(q_row), _ptr(s_row), _ptr(q_col),
                               _ptr(s_col), _ptr(noop), _stream(stream, dev))
    _check("nvfp4_quantize_2d", st)


def padded_rows_max(T: int, G: int, align: int) -> int:
    """Rows the padded layout of T tokens in G groups can need at most."""
    return -(-(T + G * (align - 1)) // align) * align


def nvfp4_quantize_grouped(x: torch.Tensor, group_rows: torch.Tensor, align: int, M_out: int,
                           bound: float, row_amax: torch.Tensor,
                           q_row: Optional[torch.Tensor], s_row: Optional[torch.Tensor],
                           q_col: Optional[torch.Tensor], s_col: Optional[torch.Tensor],
                           noop: Optional[torch.Tensor] = None, stream=None) -> None:
    """Grouped tokens x [T, K] (group sizes in the device int64 tensor
    group_rows [G]) quantized into the padded [M_out, K] layout."""
    lib = load_library()
    if x.dim() != 2:
        raise ValueError("x must be 2-D [T, K]")
    _dev(x, "x", (torch.bfloat16, torch.float32))
    T, K = x.shape
    dev = x.device
    _dev(group_rows, "group_rows", (torch.int64,), None, dev)
    _dev(row_amax, "row_amax", _F32, M_out, dev)
    if q_row is not None:
        _dev(q_row, "q_row", (torch.uint8,), M_out * ((K + 1) // 2), dev)
        _dev(s_row, "s_row", _SCALE_DTYPES, M_out * ((K + 15) // 16), dev)
    if q_col is not None:
        _dev(q_col, "q_col", (torch.uint8,), K * ((M_out + 1) // 2), dev)
        _dev(s_col, "s_col", _SCALE_DTYPES, K * ((M_out + 15) // 16), dev)
    _dev(noop, "noop", _F32, 1, dev)
    st = lib.nvfp4_quantize_grouped(_ptr(x), _dtype_code(x), T, K, _ptr(group_rows),
                                    group_rows.numel(), int(align), int(M_out),
                                    ctypes.c_float(bound), _ptr(row_amax), _ptr(q_row),
                                    _ptr(s_row), _ptr(q_col), _ptr(s_col), _ptr(noop),
                                    _stream(stream, dev))
    _check("nvfp4_quantize_grouped", st)


def nvfp4_quantize_dequantize(x: torch.Tensor, row_mode: int, row_amax: torch.Tensor,
                              bound: float, y: torch.Tensor, q_row: Optional[torch.Tensor] = None,
                              s_row: Optional[torch.Tensor] = None,
                              noop: Optional[torch.Tensor] = None, stream=None) -> None:
    """Rowwise codes of x [M, K] (optional) and their dequantization y [M, K]
    (bfloat16 or float32) in one pass."""
    lib = load_library()
    if x.dim() != 2:
        raise ValueError("x must be 2-D [M, K]")
    _dev(x, "x", (torch.bfloat16, torch.float32))
    M, K = x.shape
    dev = x.device
    _dev(row_amax, "row_amax", _F32, _amax_numel(row_mode, M, K), dev)
    _dev(y, "y", (torch.bfloat16, torch.float32), M * K, dev)
    if q_row is not None:
        _dev(q_row, "q_row", (torch.uint8,), M * ((K + 1) // 2), dev)
        _dev(s_row, "s_row", _SCALE_DTYPES, M * ((K + 15) // 16), dev)
    _dev(noop, "noop", _F32, 1, dev)
    st = lib.nvfp4_quantize_dequantize(_ptr(x), _dtype_code(x), M, K, row_mode, _ptr(row_amax),
                                       ctypes.c_float(bound), _ptr(q_row), _ptr(s_row), _ptr(y),
                                       _dtype_code(y), _ptr(noop), _stream(stream, dev))
    _check("nvfp4_quantize_dequantize", st)


def nvfp4_dequantize(q: torch.Tensor, sc: torch.Tensor, R: int, C: int, amax_mode: int,
                     amax: torch.Tensor, bound: float, y: torch.Tensor,
                     noop: Optional[torch.Tensor] = None, stream=None) -> None:
    lib = load_library()
    _dev(q, "q", (torch.uint8,), R * ((C + 1) // 2))
    dev = q.device
    _dev(sc, "sc", _SCALE_DTYPES, R * ((C + 15) // 16), dev)
    _dev(amax, "amax", _F32, _amax_numel(amax_mode, R, C), dev)
    _dev(y, "y", (torch.bfloat16, torch.float32), R * C, dev)
    _dev(noop, "noop", _F32, 1, dev)
    st = lib.nvfp4_dequantize(_ptr(q), _ptr(sc), R, C, amax_mode, _ptr(amax),
                              ctypes.c_float(bound), _ptr(y), _dtype_code(y), _ptr(noop),
                              _stream(stream, dev))
    _check("nvfp4_dequantize", st)


# --------------------------------------------------------------- conveniences
def empty_outputs(M: int, K: int, device, rowwise: bool = True, colwise: bool = True) -> dict:
    """Allocate the packed output buffers for an M x K input."""
    out = {}
    if rowwise:
        out["q_row"] = torch.empty(M, (K + 1) // 2, dtype=torch.uint8, device=device)
        out["s_row"] = torch.empty(M, (K + 15) // 16, dtype=torch.uint8, device=device)
    if colwise:
        out["q_col"] = torch.empty(K, (M + 1) // 2, dtype=torch.uint8, device=device)
        out["s_col"] = torch.empty(K, (M + 15) // 16, dtype=torch.uint8, device=device)
    return out

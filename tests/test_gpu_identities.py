"""Every hardware converter and arithmetic shortcut the kernels rely on,
against the oracle's definitions over its whole input range (backward-
overrides PR description: FP32 decode with a correctly rounded reciprocal;
fused-amax PR "Reproduce": codes and scales that match exactly).

The probes (tests/hw/nvfp4_identities.hip, built by __graft_entry__.build())
run the inline device functions of the library's nvfp4_device.h, compiled
with the library's flags, over runs of inputs; each run is compared with
the CPU oracle on the host, and a test stops at the first run that differs:

* e2m1_pack8 (v_cvt_scalef32_pk_fp4_f32, scale 1): every binary32 pattern
  except NaN, against the nearest-of-eight E2M1 encoder;
* v_cvt_pk_fp8_f32 in both operand forms the scale chains use: every scale
  in [0, 448], against the nearest-of-127 E4M3 encoder;
* v_cvt_f32_fp8, e4m3_value, fp4x2_decode (v_cvt_scalef32_pk_f32_fp4) and
  e2m1_value: every byte and code, against the decode tables;
* bf16x2_rne (v_cvt_pk_bf16_f32) and bf16_rne: every pattern except NaN,
  against the oracle's BF16 rounding;
* recip_rn: every positive finite D, against min(RN(1/D), FLT_MAX); the bare
  Newton form recip_newton wherever the kernels use it (recip_fast_ok);
* div6_rn: every finite x >= 0, and the two-term div6_two_term for
  x >= 2^-121, against RN(x / 6);
* the scaled form of the E2M1 converter with arbitrary scales s: it encodes
  x / 2^floor(log2 s), so it takes the scale's exponent only and cannot fold
  a block's encode factor into the conversion (the kernels multiply first and
  convert with scale 1)."""
from __future__ import annotations

import ctypes
import os

import numpy as np
import pytest
import torch

import oracle
from parity_utils import say

pytestmark = pytest.mark.gpu

HW = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hw")
CHUNK = 1 << 27
DEV = torch.device("cuda:0")

_lib = None


def _probes():
    global _lib
    if _lib is None:
        path = os.path.join(HW, "libnvfp4_identities.so")
        if not os.path.exists(path):
            raise ImportError(f"{path} is missing: build it with __graft_entry__.build()")
        lib = ctypes.CDLL(path)
        u32, i64, vp = ctypes.c_uint32, ctypes.c_int64, ctypes.c_void_p
        for name, args in (("probe_fp4_encode", [u32, i64, vp, vp]),
                           ("probe_fp8_encode", [u32, i64, vp, vp, vp]),
                           ("probe_decode", [vp, vp, vp, vp, vp]),
                           ("probe_bf16", [u32, i64, vp, vp, vp]),
                           ("probe_recip", [u32, i64, vp, vp, vp]),
                           ("probe_div6", [u32, i64, vp, vp, vp]),
                           ("probe_fp4_scaled", [vp, vp, i64, vp, vp])):
            fn = getattr(lib, name)
            fn.restype = ctypes.c_int
            fn.argtypes = args
        _lib = lib
    return _lib


def _ptr(t: torch.Tensor) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr())


def _stream() -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream)


def _runs(lo: int, hi: int):
    """[lo, hi) in runs of at most CHUNK patterns (lo a multiple of 8)."""
    s = lo
    while s < hi:
        n = min(CHUNK, hi - s)
        yield s, n
        s += n


def _same(name: str, start: int, got: np.ndarray, want: np.ndarray, mask=None) -> None:
    bad = got != want
    if mask is not None:
        bad &= mask
    if bad.any():
        i = int(np.argmax(bad))
        raise AssertionError(f"{name}: {int(bad.sum())} mismatches in the run at {start:#010x}; "
                             f"first pattern {start + i:#010x}: got {got[i]!r} want {want[i]!r}")


def test_e2m1_encode_every_pattern():
    lib = _probes()
    out = torch.empty(CHUNK // 2, dtype=torch.uint8, device=DEV)
    say("[gpu] identities: E2M1 encode over 2^32 patterns")
    for start, n in _runs(0, 1 << 32):
        assert lib.probe_fp4_encode(start, n, _ptr(out), _stream()) == 0
        b = out[: n // 2].cpu().numpy()
        got = np.empty(n, dtype=np.uint8)
        got[0::2] = b & 0xF
        got[1::2] = b >> 4
        want = oracle.e2m1_encode_bits(start, n)
        _same("e2m1_pack8", start, got, want, want != 0xFF)


def test_e4m3_encode_every_scale():
    lib = _probes()
    hi = int(np.float32(448.0).view(np.uint32)) + 1
    a = torch.empty(CHUNK, dtype=torch.uint8, device=DEV)
    b = torch.empty(CHUNK, dtype=torch.uint8, device=DEV)
    say(f"[gpu] identities: E4M3 encode over [0, 448] ({hi} patterns)")
    for start, n in _runs(0, hi):
        assert lib.probe_fp8_encode(start, n, _ptr(a), _ptr(b), _stream()) == 0
        want = oracle.e4m3_encode_bits(start, n)
        _same("cvt_pk_fp8_f32 (zero operand)", start, a[:n].cpu().numpy(), want)
        _same("cvt_pk_fp8_f32 (own bits)", start, b[:n].cpu().numpy(), want)


def test_decoders_every_byte_and_code():
    lib = _probes()
    fp8_hw = torch.empty(4 * 256, device=DEV)
    fp8_sw = torch.empty(256, device=DEV)
    fp4_hw = torch.empty(4 * 256 * 2, device=DEV)
    fp4_sw = torch.empty(16, device=DEV)
    assert lib.probe_decode(_ptr(fp8_hw), _ptr(fp8_sw), _ptr(fp4_hw), _ptr(fp4_sw), _stream()) == 0
    e4 = np.array([oracle.e4m3_value(b) for b in range(256)], dtype=np.float32)
    e2 = np.array([oracle.e2m1_value(c) for c in range(16)], dtype=np.float32)
    bits = lambda t: t.cpu().numpy().view(np.uint32)
    finite = np.array([(b & 0x7F) != 0x7F for b in range(256)])  # 0x7F / 0xFF: the NaN bytes
    for f in range(4):
        _same(f"cvt_f32_fp8 fill {f}", 0, bits(fp8_hw)[256 * f:256 * (f + 1)], e4.view(np.uint32),
              finite)
    _same("e4m3_value", 0, bits(fp8_sw), e4.view(np.uint32))
    want = np.stack([e2[np.arange(256) & 0xF], e2[np.arange(256) >> 4]], axis=1).ravel()
    for sel in range(4):
        _same(f"fp4x2_decode<{sel}>", 0, bits(fp4_hw)[512 * sel:512 * (sel + 1)],
              want.view(np.uint32))
    _same("e2m1_value", 0, bits(fp4_sw), e2.view(np.uint32))


def test_bf16_round_every_pattern():
    lib = _probes()
    hw = torch.empty(CHUNK // 2, dtype=torch.int32, device=DEV)
    sw = torch.empty(CHUNK, dtype=torch.int16, device=DEV)
    say("[gpu] identities: FP32 -> BF16 over 2^32 patterns")
    for start, n in _runs(0, 1 << 32):
        assert lib.probe_bf16(start, n, _ptr(hw), _ptr(sw), _stream()) == 0
        want = oracle.bf16_round_bits(start, n)
        # NaN inputs (outside the contract) are the patterns the oracle maps
        # to a NaN; no other input does
        not_nan = ((want & 0x7F80) != 0x7F80) | ((want & 0x007F) == 0)
        _same("bf16x2_rne", start, hw[: n // 2].cpu().numpy().view(np.uint16), want, not_nan)
        _same("bf16_rne", start, sw[:n].cpu().numpy().view(np.uint16), want, not_nan)


def test_reciprocal_every_decode_scale():
    lib = _probes()
    rn = torch.empty(CHUNK, device=DEV)
    nw = torch.empty(CHUNK, device=DEV)
    hi = int(np.finfo(np.float32).max.view(np.uint32)) + 1
    say(f"[gpu] identities: RN(1/D) over every positive finite D ({hi - 1} patterns)")
    allones_off = 0
    for start, n in _runs(0, hi):
        assert lib.probe_recip(start, n, _ptr(rn), _ptr(nw), _stream()) == 0
        want = oracle.recip_bits(start, n).view(np.uint32)
        pat = np.arange(start, start + n, dtype=np.uint32)
        pos = pat != 0
        _same("recip_rn", start, rn[:n].cpu().numpy().view(np.uint32), want, pos)
        newton = nw[:n].cpu().numpy().view(np.uint32)
        in_range = (pat >= 0x00800000) & (pat < 0x7E800000)
        allones = (pat & 0x7FFFFF) == 0x7FFFFF
        _same("recip_newton where the kernels use it", start, newton, want, in_range & ~allones)
        allones_off += int(((newton != want) & in_range & allones).sum())
    # informational: the bare Newton form at the all-ones significands, which
    # the kernels send to the IEEE division (exact from the upper neighbour of
    # 1/D, a tie from the lower one)
    say(f"[gpu] identities: recip_newton differs at {allones_off} of 252 all-ones significands")


def test_div6_every_magnitude():
    lib = _probes()
    rn = torch.empty(CHUNK, device=DEV)
    tt = torch.empty(CHUNK, device=DEV)
    hi = int(np.finfo(np.float32).max.view(np.uint32)) + 1
    say(f"[gpu] identities: RN(x/6) over every finite x >= 0 ({hi} patterns)")
    for start, n in _runs(0, hi):
        assert lib.probe_div6(start, n, _ptr(rn), _ptr(tt), _stream()) == 0
        want = oracle.div6_bits(start, n).view(np.uint32)
        _same("div6_rn", start, rn[:n].cpu().numpy().view(np.uint32), want)
        pat = np.arange(start, start + n, dtype=np.uint32)
        _same("div6_two_term (x >= 2^-121)", start, tt[:n].cpu().numpy().view(np.uint32), want,
              pat >= 0x03000000)


def test_scaled_fp4_converter_takes_only_the_scale_exponent():
    lib = _probes()
    g = np.random.RandomState(12)
    n = 1 << 20
    e = g.randint(-20, 21, n)
    m = np.where(g.rand(n) < 0.1, 1.0, 1.0 + g.rand(n))  # mostly not a power of two
    s = (m * np.exp2(e)).astype(np.float32)
    # random magnitudes around the E2M1 range, and values at and beside its
    # rounding ties, all relative to 2^e
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    t = np.where(g.rand(n) < 0.5, g.randn(n) * 3.0,
                 ties[g.randint(0, len(ties), n)] * (1.0 + g.choice([-1e-6, 0.0, 1e-6], n))
                 * np.where(g.rand(n) < 0.5, -1.0, 1.0))
    x = (t * np.exp2(e)).astype(np.float32)
    xd = torch.from_numpy(x).to(DEV)
    sd = torch.from_numpy(s).to(DEV)
    out = torch.empty(n, dtype=torch.uint8, device=DEV)
    say("[gpu] identities: scaled E2M1 converter over 2^20 random (x, s)")
    assert lib.probe_fp4_scaled(_ptr(xd), _ptr(sd), n, _ptr(out), _stream()) == 0
    hw = out.cpu().numpy() & 0xF
    scaled = (x / np.exp2(e).astype(np.float32)).astype(np.float32)  # exact: a power of two
    _same("cvt_scalef32_pk_fp4_f32 vs E2M1(x / 2^floor(log2 s))", 0, hw, oracle.e2m1_encode(scaled))
    # a plain division by s gives other codes on a good part of these inputs
    by_s = oracle.e2m1_encode((x / s).astype(np.float32))
    assert float((hw != by_s).mean()) > 0.05

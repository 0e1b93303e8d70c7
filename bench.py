"""Throughput of row-scaled NVFP4 quantize-transpose on one MI355X.

One step = the whole quantize path on one 8192 x 28672 BF16 matrix (the MLP
activation / weight shape, N(0,1) times a per-row factor 10^U(-2,2)):
  1. noop-aware zeroing of the amax vectors          (amax-init kernel)
  2. fused per-row + per-column amax, one read of X   (fused amax kernel)
  3. both NVFP4 copies (rowwise + transposed), one more read of X (cast kernel)
The input is resident in HBM before timing starts. value = algorithmic bytes
of the step (X read twice, amax vectors written and read once, all codes and
scales written once) / step time, in GB/s.

The headline region holds K whole steps with HIP events only at its two ends,
queued right after 50 untimed steps (so that a short region does not start on
a GPU still ramping up from an idle wait).
The roofline figure is the cast kernel's duration where it runs in the step:
a second region of K steps records an event pair around each cast (after its
amax pass), and the pairs' average gives the roofline fraction (algorithmic
bytes of one cast launch / that duration, against 8 TB/s). Two more regions of
K back-to-back launches of one kernel each (amax pass, cast pass) are reported
beside it; a cast right after another cast also pays for the previous cast's
write-back, so that figure runs higher and varies more from GPU to GPU. A
bounded spin kernel queued ahead of each timed region lets the host enqueue
the whole region before the GPU reaches it. Also reported: the dequantize
kernel's bandwidth, the other kernels of the path on the workloads they serve
(two-kernel and per-tensor amax, 2-D tiles, four-over-six, quantize +
dequantize, the FP32 edge matrix, grouped tokens, and the two small matrices
cold and warm; the 2-D tile cast also as a whole step, per-tensor amax pass
then cast, timed like the headline step), the fused-amax PR's comparison (whole quantize with the fused
amax against the separate row and column amax kernels, medians), what plain
streaming kernels sustain on the same GPU (read, write, copy), and the CPU
oracle timed on a bounded sample of the same workload on the host cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
       python bench.py --copy-calibration   (plain torch copy, for counter scaling)
       python bench.py --case 2d [--case grouped ...]   (those rows alone, for profiling)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, AMD published peak
# Untimed steps (about 10 ms of the same work) queued right before each
# headline region: after an idle wait the GPU needs about that long to reach
# its steady clock. The first 20-step region of a fresh process read 206-215 us
# per step with 0-20 such steps and 200.5-202.5 us with 50 (same GPU).
RUN_IN = 50
METRIC = "row-scaled NVFP4 quantize-transpose GB/s (in+out) and % of HBM peak, 1 GPU"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "cast_llm_mlp_traffic.json")


def source_digest() -> str:
    """Digest of the kernel sources: counter-derived traffic is only reported
    for the kernel build it was measured on."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "precision_quantization_row_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    if not os.path.exists(TRAFFIC_FILE):
        return None
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("source_digest") != source_digest():
        return None
    return rec.get("cast_hbm_bytes_per_launch")


def cpu_model() -> str:
    """The host CPU as /proc/cpuinfo (what lscpu reads) names it: model name,
    then family / model / stepping (a virtualized host may report only a
    generic model name, which the numbers still identify)."""
    info = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if ":" not in line:
                    if info:
                        break  # the first processor's block is enough
                    continue
                k, v = (t.strip() for t in line.split(":", 1))
                info.setdefault(k, v)
    except OSError:
        pass
    if "model name" not in info:
        import platform
        return platform.processor() or "unknown"
    ids = ", ".join(f"{k} {info[k]}" for k in ("cpu family", "model", "stepping") if k in info)
    return f"{info['model name']} ({ids})" if ids else info["model name"]


class StreamRef:
    """Plain streaming kernels (16-byte non-temporal loads / stores, nothing
    else per byte) from bench_ref/libstream_ref.so: the HBM ceiling the
    quantize path is set against, and a read-only pass that evicts the
    memory-side cache between cold repetitions without leaving dirty lines
    behind (a fill would leave its writes to drain into the timed call)."""

    def __init__(self, torch, dev):
        import ctypes

        from precision_quantization_row_amd.build import stream_ref_path

        self.torch, self.dev, self.ct = torch, dev, ctypes
        lib = ctypes.CDLL(stream_ref_path())
        vp, i64, c_int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        for name, args in (("stream_read", [vp, i64, vp, c_int, c_int, vp]),
                           ("stream_write", [vp, i64, c_int, vp]),
                           ("stream_copy", [vp, vp, i64, c_int, vp]),
                           ("stream_pieces", [vp, i64, c_int, c_int, c_int, vp])):
            fn = getattr(lib, name)
            fn.restype = c_int
            fn.argtypes = args
        self.lib = lib
        self.sink = torch.zeros(4, dtype=torch.int32, device=dev)
        self.flush_buf = None

    def _st(self):
        return self.ct.c_void_p(self.torch.cuda.current_stream(self.dev).cuda_stream)

    def read(self, t, grid=4096, cached=False):
        assert self.lib.stream_read(t.data_ptr(), t.numel() * t.element_size(),
                                    self.sink.data_ptr(), grid, int(cached), self._st()) == 0

    def write(self, t, grid=4096):
        assert self.lib.stream_write(t.data_ptr(), t.numel() * t.element_size(), grid,
                                     self._st()) == 0

    def copy(self, a, b, grid=4096):
        assert self.lib.stream_copy(a.data_ptr(), b.data_ptr(), a.numel() * a.element_size(), grid,
                                    self._st()) == 0

    def pieces(self, t, piece, nt, grid=4096):
        """Write t in `piece`-byte pieces of scattered 128-byte lines."""
        assert self.lib.stream_pieces(t.data_ptr(), t.numel() * t.element_size(), piece, int(nt),
                                      grid, self._st()) == 0

    def flush(self):
        """Read 512 MB (twice the memory-side cache) with ordinary, caching
        loads: the caches end up holding clean lines of this buffer."""
        if self.flush_buf is None:
            self.flush_buf = self.torch.ones(512 << 20, dtype=self.torch.uint8, device=self.dev)
        self.read(self.flush_buf, cached=True)

    def ceiling(self, timed):
        torch = self.torch
        nbytes = 1 << 30
        a = torch.ones(nbytes, dtype=torch.uint8, device=self.dev)
        b = torch.empty_like(a)
        best = {"read": (0.0, 0), "write": (0.0, 0), "copy": (0.0, 0)}
        for grid in (512, 1024, 2048, 4096, 8192, 16384):
            for kind, fn, moved in (("read", lambda i: self.read(a, grid), nbytes),
                                    ("write", lambda i: self.write(b, grid), nbytes),
                                    ("copy", lambda i: self.copy(a, b, grid), 2 * nbytes)):
                fn(0)
                gbs = moved / (timed(fn, 10) * 1e-3) / 1e9
                if gbs > best[kind][0]:
                    best[kind] = (gbs, grid)
        del a, b
        return {"read_GBs": round(best["read"][0], 1), "write_GBs": round(best["write"][0], 1),
                "copy_GBs": round(best["copy"][0], 1),
                "grids": {k: v[1] for k, v in best.items()},
                "how": "1 GiB buffers, plain 16-byte non-temporal loads/stores (4 in flight per "
                       "thread, 1 KB contiguous per wave instruction), 10 back-to-back launches "
                       "per point, best over grids of 512-16384 workgroups of 256 threads; copy "
                       "counts bytes read + written"}


def _row(us, nbytes, what):
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"us": round(us, 2), "bytes": nbytes, "GBs": round(gbs, 1),
            "frac": round(gbs / HBM_PEAK_GBS, 4), "bytes_are": what}


def cold_warm(torch, ref, fn, nbytes, hold, calls=2, reps=20):
    """Medians of reps single calls of fn (calls API calls), each between its
    own event pair: cold (a read-only pass over 512 MB with caching loads
    evicts the memory-side cache first) and warm (the call right after the
    same call). A spin kernel queued ahead of the event pair keeps the GPU
    busy while the host enqueues the call, so launch latency is not timed."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    fn()
    med = {}
    for kind in ("cold", "warm"):
        ts = []
        for _ in range(reps):
            if kind == "cold":
                ref.flush()
            else:
                fn()
            hold(calls)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        ts.sort()
        med[kind] = 0.5 * (ts[(reps - 1) // 2] + ts[reps // 2])
    out = {"bytes": nbytes, "bytes_are": "X read by the amax and the cast passes, both copies "
                                          "written (algorithmic)"}
    for kind, us in med.items():
        gbs = nbytes / (us * 1e-6) / 1e9
        out[f"{kind}_us"] = round(us, 2)
        out[f"{kind}_GBs"] = round(gbs, 1)
        out[f"{kind}_frac"] = round(gbs / HBM_PEAK_GBS, 4)
    out["how"] = (f"median of {reps} single calls each, a spin kernel queued ahead of each: "
                  "cold after a 512 MB read-only pass with caching loads, warm right after the "
                  "same call")
    return out


class Ctx:
    """What every case below needs: the package, torch, the device, the two
    copies of the headline matrix, the timers and the streaming reference."""

    def __init__(self, p, workloads, torch, dev, xs, timed, bound, ref, hold):
        self.p, self.workloads, self.torch, self.dev = p, workloads, torch, dev
        self.xs, self.timed, self.bound, self.ref, self.hold = xs, timed, bound, ref, hold

    def events(self, n):
        ev = self.torch.cuda.Event
        return [(ev(enable_timing=True), ev(enable_timing=True)) for _ in range(n)]


N_ROW = 20  # launches (or steps) per region in the cases below


def case_amax(c):
    """Two-kernel and per-tensor amax on the headline matrix."""
    p, torch, dev, xs = c.p, c.torch, c.dev, c.xs
    M, K = xs[0].shape
    ra = torch.empty(M, dtype=torch.float32, device=dev)
    ca = torch.empty(K, dtype=torch.float32, device=dev)
    ta = torch.empty(1, dtype=torch.float32, device=dev)
    xb = M * K * 2
    res = {}
    f2 = lambda i: p.nvfp4_amax_rowcol(xs[i & 1], ra, ca, flags=p.NVFP4_FLAG_FORCE_TWO_KERNEL)
    f2(0)
    res["two_kernel_amax_bf16_8192x28672"] = _row(c.timed(f2, N_ROW) * 1e3, 2 * xb + 4 * (M + K),
                                                  "X read by each of the two kernels, vectors written")
    ft = lambda i: p.nvfp4_amax_rowcol(xs[i & 1], None, None, tensor_amax=ta)
    ft(0)
    res["tensor_amax_bf16_8192x28672"] = _row(c.timed(ft, N_ROW) * 1e3, xb + 4, "X read once")
    return res


def case_2d(c):
    """2-D 16 x 16 tile scales, both copies, on the headline matrix: the cast
    back to back, and the whole 2-D quantize step (per-tensor amax pass, then
    the cast) measured like the headline step."""
    p, torch, dev, xs = c.p, c.torch, c.dev, c.xs
    M, K = xs[0].shape
    xb = M * K * 2
    ta = torch.empty(1, dtype=torch.float32, device=dev)
    out = p.empty_outputs(M, K, dev)
    amax = lambda i: p.nvfp4_amax_rowcol(xs[i & 1], None, None, tensor_amax=ta)
    f2d = lambda i: p.nvfp4_quantize_2d(xs[i & 1], ta, c.bound, out["q_row"], out["s_row"],
                                        out["q_col"], out["s_col"])
    amax(0)
    f2d(0)
    cb2 = xb + 4 + 2 * (M * (K // 2) + M * (K // 16))
    res = {"quantize_2d_bf16_8192x28672": _row(
        c.timed(f2d, N_ROW) * 1e3, cb2,
        "X read once, both copies written; back to back, each launch also absorbing the previous "
        "launch's write-back")}
    # the step: whole steps with events at the region's ends (200 of them: a
    # region pays a fixed cost where it starts), then the same steps with an
    # event pair around each cast
    n = 200
    step_ms = c.timed(lambda i: (amax(i), f2d(i)), n, 2, lead=RUN_IN)
    ev = c.events(n)
    torch.cuda.synchronize()
    c.hold(4 * n + 2 * RUN_IN)
    for i in range(RUN_IN):
        amax(i)
        f2d(i)
    for i in range(n):
        amax(i)
        ev[i][0].record()
        f2d(i)
        ev[i][1].record()
    torch.cuda.synchronize()
    cast_ms = sum(a.elapsed_time(b) for a, b in ev) / n
    row = _row(step_ms * 1e3, xb + 4 + cb2,
               "X read by the per-tensor amax pass and the cast, both copies written")
    cast = _row(cast_ms * 1e3, cb2, "the cast launch inside the step, event pair around it")
    row.update({"cast_in_step_us": cast["us"], "cast_in_step_GBs": cast["GBs"],
                "cast_in_step_frac": cast["frac"]})
    res["quantize_2d_step_bf16_8192x28672"] = row
    return res


def case_4over6(c):
    """Four-over-six block scales, both copies (row and column amax given; one
    launch per direction, so X is read twice)."""
    p, torch, dev, xs = c.p, c.torch, c.dev, c.xs
    M, K = xs[0].shape
    xb = M * K * 2
    ra = torch.empty(M, dtype=torch.float32, device=dev)
    ca = torch.empty(K, dtype=torch.float32, device=dev)
    p.nvfp4_amax_rowcol(xs[0], ra, ca)
    out = p.empty_outputs(M, K, dev)
    f46 = lambda i: p.nvfp4_quantize_4over6(xs[i & 1], p.NVFP4_AMAX_LINE, ra, p.NVFP4_AMAX_LINE, ca,
                                            256.0, out["q_row"], out["s_row"], out["q_col"],
                                            out["s_col"])
    f46(0)
    return {"quantize_4over6_bf16_8192x28672": _row(
        c.timed(f46, 5) * 1e3, 2 * xb + 4 * (M + K) + 2 * (M * (K // 2) + M * (K // 16)),
        "X read once per direction, both copies written")}


def case_qdq(c):
    """Rowwise codes and their BF16 dequantization in one pass (row amax given)."""
    p, torch, dev, xs = c.p, c.torch, c.dev, c.xs
    M, K = xs[0].shape
    ra = torch.empty(M, dtype=torch.float32, device=dev)
    p.nvfp4_amax_rowcol(xs[0], ra)
    qr = torch.empty(M, K // 2, dtype=torch.uint8, device=dev)
    sr = torch.empty(M, K // 16, dtype=torch.uint8, device=dev)
    yq = torch.empty(M, K, dtype=torch.bfloat16, device=dev)
    fq = lambda i: p.nvfp4_quantize_dequantize(xs[i & 1], p.NVFP4_AMAX_LINE, ra, c.bound, yq, qr, sr)
    fq(0)
    return {"quantize_dequantize_bf16_8192x28672": _row(
        c.timed(fq, N_ROW) * 1e3, M * K * 2 + 4 * M + M * (K // 2) + M * (K // 16) + M * K * 2,
        "X read once, rowwise codes + scales and the BF16 operand written")}


def case_fp32_edge(c):
    """The FP32 4097 x 2880 matrix: amax (one-pass and two-kernel), cast, and
    the whole quantize back to back, cold and warm."""
    p, torch, dev, wl = c.p, c.torch, c.dev, c.workloads
    w = wl.make("fp32_edge")
    M, K = w.shape
    x = w.x.to(dev)
    ra = torch.empty(M, dtype=torch.float32, device=dev)
    ca = torch.empty(K, dtype=torch.float32, device=dev)
    out = p.empty_outputs(M, K, dev)
    fa = lambda i: p.nvfp4_amax_rowcol(x, ra, ca)
    fa2 = lambda i: p.nvfp4_amax_rowcol(x, ra, ca, flags=p.NVFP4_FLAG_FORCE_TWO_KERNEL)
    fc = lambda i: p.nvfp4_quantize_transpose(x, 1, ra, 1, ca, c.bound, out["q_row"], out["s_row"],
                                              out["q_col"], out["s_col"])
    fa(0); fa2(0); fc(0)
    assert p.nvfp4_amax_path(p.NVFP4_FP32, M, K, 1, 1, 0) == 1  # one-pass amax
    cb = M * K * 4 + 4 * (M + K) + M * ((K + 1) // 2) + M * ((K + 15) // 16) + K * ((M + 1) // 2) \
        + K * ((M + 15) // 16)
    res = {}
    res["fp32_4097x2880_amax"] = _row(c.timed(fa, N_ROW) * 1e3, M * K * 4 + 4 * (M + K),
                                      "one-pass row + column amax: X read once, vectors written")
    res["fp32_4097x2880_two_kernel_amax"] = _row(c.timed(fa2, N_ROW) * 1e3,
                                                 2 * M * K * 4 + 4 * (M + K),
                                                 "X read by each of the two kernels (forced)")
    res["fp32_4097x2880_cast"] = _row(c.timed(fc, N_ROW) * 1e3, cb, "X read once, both copies written")
    fac = lambda i: (fa(i), fc(i))
    res["fp32_4097x2880_amax_and_cast"] = _row(
        c.timed(fac, N_ROW, 2) * 1e3, wl.algorithmic_bytes(M, K, 4),
        "the whole quantize (one-pass amax, then cast), back to back; algorithmic bytes "
        "(X counted twice)")
    res["fp32_4097x2880_amax_and_cast"].update(
        cold_warm(torch, c.ref, lambda: fac(0), wl.algorithmic_bytes(M, K, 4), c.hold))
    return res


def case_grouped(c):
    """Grouped tokens (16 groups of about 1024 rows x 4096, padded to 128
    rows): the three-call sequence on the padded layout, and the one-call
    grouped quantize from the token rows."""
    p, torch, dev = c.p, c.torch, c.dev
    w = c.workloads.make("moe_groups")
    M, K = w.shape
    x = w.x.to(dev)
    ge = w.group_end.to(dev)
    ra = torch.empty(M, dtype=torch.float32, device=dev)
    out = p.empty_outputs(M, K, dev)

    def moe(i):
        # per-group amax: row amax expanded over each group, colwise blocks use
        # the group amax of their rows
        p.nvfp4_amax_rowcol(x, ra)
        p.nvfp4_group_amax_expand(ra, ge)
        p.nvfp4_quantize_transpose(x, 1, ra, 2, ra, c.bound, out["q_row"], out["s_row"],
                                   out["q_col"], out["s_col"])

    moe(0)
    mb = 2 * M * K * 2 + 4 * 4 * M + 8 * ge.numel() + M * ((K + 1) // 2) + M * ((K + 15) // 16) \
        + K * ((M + 1) // 2) + K * ((M + 15) // 16)
    res = {"moe_%dx%d_amax_expand_cast" % (M, K): _row(c.timed(moe, N_ROW, 3) * 1e3, mb,
                                                        "X read by the amax and the cast passes")}
    del x
    # the same groups as token rows, padded on the way in by one call
    starts = torch.cat([torch.zeros(1, dtype=torch.int64), w.group_end[:-1]])
    tok = torch.cat([w.x[int(s):int(s) + int(r)] for s, r in zip(starts, w.group_rows)]).to(dev)
    T = tok.shape[0]
    gr = w.group_rows.to(dev)

    def grouped(i):
        p.nvfp4_quantize_grouped(tok, gr, 128, M, c.bound, ra, out["q_row"], out["s_row"],
                                 out["q_col"], out["s_col"])

    grouped(0)
    gb = 2 * T * K * 2 + 4 * M + 8 * gr.numel() + M * ((K + 1) // 2) + M * ((K + 15) // 16) \
        + K * ((M + 1) // 2) + K * ((M + 15) // 16)
    res["moe_%dtok_x%d_quantize_grouped" % (T, K)] = _row(
        c.timed(grouped, N_ROW) * 1e3, gb,
        "token rows read by the amax and the cast, padded layout written")
    cw = cold_warm(torch, c.ref, lambda: grouped(0), gb, c.hold, calls=3)
    cw.pop("bytes_are")
    res["moe_%dtok_x%d_quantize_grouped" % (T, K)].update(cw)
    return res


def case_small(c):
    """The two small matrices, one whole quantize each (amax pass + cast):
    median of 20 cold repetitions (the memory-side cache evicted by a
    read-only pass before each) and of 20 warm ones (the same call again right
    after itself); the 256 x 256 case is launch-bound."""
    p, torch, dev, wl = c.p, c.torch, c.dev, c.workloads
    res = {}
    for name in ("tiny_rowscale", "outliers"):
        w = wl.make(name)
        M, K = w.shape
        x = w.x.to(dev)
        ra = torch.empty(M, dtype=torch.float32, device=dev)
        ca = torch.empty(K, dtype=torch.float32, device=dev)
        ta = torch.empty(1, dtype=torch.float32, device=dev)
        out = p.empty_outputs(M, K, dev)

        def row_scaled():
            p.nvfp4_amax_rowcol(x, ra, ca)
            p.nvfp4_quantize_transpose(x, 1, ra, 1, ca, c.bound, out["q_row"], out["s_row"],
                                       out["q_col"], out["s_col"])

        def per_tensor():
            p.nvfp4_amax_rowcol(x, None, None, tensor_amax=ta)
            p.nvfp4_quantize_transpose(x, 0, ta, 0, ta, c.bound, out["q_row"], out["s_row"],
                                       out["q_col"], out["s_col"])

        res["%s_%dx%d_row_scaled" % (name, M, K)] = cold_warm(
            torch, c.ref, row_scaled, wl.algorithmic_bytes(M, K, 2), c.hold)
        if name == "outliers":
            res["%s_%dx%d_per_tensor" % (name, M, K)] = cold_warm(
                torch, c.ref, per_tensor,
                wl.algorithmic_bytes(M, K, 2, row_amax=False, col_amax=False,
                                     tensor_amax=True), c.hold)
        del x, out
    return res


def case_hw(c):
    """The write-path probes (bench_ref/stream_ref.hip), not part of the
    default line: 117 MB (the size of one copy's codes at 8192 x 28672)
    written as scattered pieces of 128, 64, 32 or 16 bytes per 128-byte line,
    with non-temporal or ordinary stores, each write followed by a 470 MB
    non-temporal read (the size of X), which absorbs the write-back of the
    lines the write left dirty in the memory-side cache. Medians of 10
    repetitions, an event pair around each kernel; each repetition starts
    after a read of its own, so no dirty line is left from the one before."""
    torch, ref, dev = c.torch, c.ref, c.dev
    nw, nr = 117440512, 469762048
    wbuf = torch.empty(nw, dtype=torch.uint8, device=dev)
    rbuf = torch.ones(nr, dtype=torch.uint8, device=dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def med(v):
        v = sorted(v)
        return 0.5 * (v[(len(v) - 1) // 2] + v[len(v) // 2])

    def pair(write):
        tw, tr = [], []
        for _ in range(10):
            ref.read(rbuf)
            torch.cuda.synchronize()
            e0, e1, e2 = ev(), ev(), ev()
            c.hold(3)
            e0.record()
            write()
            e1.record()
            ref.read(rbuf)
            e2.record()
            torch.cuda.synchronize()
            tw.append(e0.elapsed_time(e1) * 1e3)
            tr.append(e1.elapsed_time(e2) * 1e3)
        return med(tw), med(tr)

    res = {}
    _, r0 = pair(lambda: ref.read(wbuf))  # a read in place of the write: the read alone
    res["read_470MB_after_a_read"] = {"us": round(r0, 2)}
    for piece in (128, 64, 32, 16):
        for nt in (True, False):
            w_us, r_us = pair(lambda: ref.pieces(wbuf, piece, nt))
            res[f"write_117MB_{piece}B_pieces_{'nt' if nt else 'cached'}"] = {
                "write_us": round(w_us, 2), "read_470MB_after_us": round(r_us, 2),
                "sum_us": round(w_us + r_us, 2),
                "write_plus_drain_us": round(w_us + r_us - r0, 2)}
    return res


CASES = {"amax": case_amax, "2d": case_2d, "4over6": case_4over6, "qdq": case_qdq,
         "fp32_edge": case_fp32_edge, "grouped": case_grouped, "small": case_small,
         "hw": case_hw}
DEFAULT_CASES = ("amax", "2d", "4over6", "qdq", "fp32_edge", "grouped", "small")


def other_rows(ctx, names=None):
    """The remaining kernels of the path, each on the workload it serves.
    Back-to-back regions have events at their ends only; bytes are those each
    launch actually has to move (the two-kernel amax reads X twice)."""
    res = {}
    for name in (names or DEFAULT_CASES):
        res.update(CASES[name](ctx))
    return res


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # 1000 steps take about 0.2 s; a region of 100 reads 1-2 % slower per
    # step (a fixed cost of a few hundred microseconds where a region starts)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-rows", action="store_true",
                    help="skip the other kernels of the path (two-kernel amax, per-tensor "
                         "amax, FP32 and grouped-token workloads)")
    ap.add_argument("--cpu-rows", type=int, default=8192,
                    help="rows of the workload the CPU oracle is timed on")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="wall time the CPU oracle is run for (whole passes)")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--case", action="append", choices=sorted(CASES),
                    help="run only this case of the other rows (repeatable), after the warm-up; "
                         "prints their rows alone")
    ap.add_argument("--hold-ms", type=float, default=None,
                    help="length of the spin kernel queued ahead of each timed region "
                         "(default: 1 ms + 1.5 x the host's measured time to enqueue it)")
    return ap.parse_args()


def copy_calibration():
    import torch

    n = 1 << 28  # 1 GiB of float32 read + 1 GiB written per copy
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "launches": 3}))


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}, WORLD_SIZE {world}): "
              "the quantize path has no cross-GPU step in this build", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    import numpy as np
    import torch

    import precision_quantization_row_amd as p
    from precision_quantization_row_amd import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    p.load_library()
    w = workloads.make("llm_mlp")
    M, K = w.shape
    # Two device copies of the same matrix, used by alternate steps: a step
    # never finds its input in a cache because the previous step read it (the
    # second read inside a step, amax pass then cast pass, is the method's own).
    xs = [w.x.to(dev), w.x.to(dev)]
    ra = torch.empty(M, dtype=torch.float32, device=dev)
    ca = torch.empty(K, dtype=torch.float32, device=dev)
    out = p.empty_outputs(M, K, dev)
    bound = 448.0
    assert p.nvfp4_amax_path(p.NVFP4_BF16, M, K, 1, 1, 0) == 1  # fused amax runs

    def amax(i):
        p.nvfp4_amax_rowcol(xs[i & 1], ra, ca)

    def cast(i):
        p.nvfp4_quantize_transpose(xs[i & 1], p.NVFP4_AMAX_LINE, ra, p.NVFP4_AMAX_LINE, ca, bound,
                                   out["q_row"], out["s_row"], out["q_col"], out["s_col"])

    # A bounded spin kernel at the head of the stream keeps the GPU busy
    # while the host enqueues a whole timed region, so the region's kernels
    # run back to back from the queue with no launch gaps, also when a
    # profiler slows every host-side launch. Its length follows the host's
    # measured cost per launch (a longer wait than needed idles the GPU, which
    # then starts the region at a lower clock).
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(1000)
    torch.cuda.synchronize()
    e0.record()
    torch.cuda._sleep(1 << 20)
    e1.record()
    torch.cuda.synchronize()
    sleep_cycles_per_ms = (1 << 20) / max(e0.elapsed_time(e1), 1e-3)

    host_ms_per_call = [0.05]  # refined by the warm-up below

    def hold_queue(n_calls):
        ms = args.hold_ms if args.hold_ms is not None else 1.0 + 1.5 * n_calls * host_ms_per_call[0]
        torch.cuda._sleep(int(ms * sleep_cycles_per_ms))

    def timed(fn, n, calls_per_fn=1, lead=0):
        """Average time of fn(0..n-1) launched back to back, HIP events on the
        launch stream at the two ends of the region only (an event between two
        kernels would add a gap of its own). lead: untimed launches of fn
        queued between the spin kernel and the first event, so that the timed
        region starts on a GPU that is already running the same work (a
        region that starts right after the idle wait can read a few percent
        slower when it is short)."""
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        hold_queue((n + lead) * calls_per_fn)
        for i in range(lead):
            fn(i)
        e0.record()
        for i in range(n):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    for i in range(args.warmup):
        amax(i)
        cast(i)
    torch.cuda.synchronize()
    # the host's cost per launch, from a few more (untimed) steps enqueued
    # after the warm-up
    t_host = time.perf_counter()
    for i in range(4):
        amax(i)
        cast(i)
    host_ms_per_call[0] = (time.perf_counter() - t_host) * 1e3 / 8
    torch.cuda.synchronize()

    if args.case:
        # only the named cases (for a profiler run): no headline, no streaming
        # reference, no CPU baseline
        ctx = Ctx(p, workloads, torch, dev, xs, timed, bound, StreamRef(torch, dev), hold_queue)
        print(json.dumps({"cases": args.case, "rows": other_rows(ctx, args.case),
                          "source_digest": source_digest(),
                          "library": os.path.relpath(p.library_path(), ROOT)}))
        return

    K_steps = args.steps
    step_bytes = workloads.algorithmic_bytes(M, K, 2)
    # headline: K whole steps (after RUN_IN untimed ones in the same queue)
    ms_per_step = timed(lambda i: (amax(i), cast(i)), K_steps, 2, lead=RUN_IN)
    # per-kernel regions: the same launches, one kind at a time
    # the cast inside the step: an event pair around each cast, after its amax
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(K_steps)]
    torch.cuda.synchronize()
    hold_queue(4 * K_steps + 2 * RUN_IN)
    for i in range(RUN_IN):
        amax(i)
        cast(i)
    for i in range(K_steps):
        amax(i)
        ev[i][0].record()
        cast(i)
        ev[i][1].record()
    torch.cuda.synchronize()
    cast_step = sum(a.elapsed_time(b) for a, b in ev) / K_steps
    cast_avg = timed(cast, K_steps, lead=RUN_IN)
    amax_avg = timed(amax, K_steps, lead=RUN_IN)
    cast_bytes = M * K * 2 + 4 * (M + K) + (M * ((K + 1) // 2) + M * ((K + 15) // 16)
                                            + K * ((M + 1) // 2) + K * ((M + 15) // 16))
    amax_bytes = M * K * 2 + 4 * (M + K)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    cast_gbs = cast_bytes / (cast_step * 1e-3) / 1e9

    # The fused-amax PR's own comparison ("Performance"): the median latency
    # of the whole quantize with the fused amax pass against the same quantize
    # with the separate row and column amax kernels. Regions of 100 steps of
    # each kind alternate, and the median of the region means is reported.
    def amax2(i):
        p.nvfp4_amax_rowcol(xs[i & 1], ra, ca, flags=p.NVFP4_FLAG_FORCE_TWO_KERNEL)

    for i in range(4):
        amax2(i)
        cast(i)
    fused_r, two_r = [], []
    n_cmp = min(100, K_steps)  # shorter regions when a profiler run asks for few steps
    for _ in range(11):
        fused_r.append(timed(lambda i: (amax(i), cast(i)), n_cmp, 2))
        two_r.append(timed(lambda i: (amax2(i), cast(i)), n_cmp, 2))
    fused_r.sort()
    two_r.sort()
    fused_med, two_med = fused_r[5] * 1e3, two_r[5] * 1e3
    full_cmp = {
        "fused_amax_then_cast_us": round(fused_med, 2),
        "row_amax_col_amax_then_cast_us": round(two_med, 2),
        "speedup": round(two_med / fused_med, 3),
        "fused_GBs": round(step_bytes / (fused_med * 1e-6) / 1e9, 1),
        "how": f"median of 11 region means, each region {n_cmp} whole quantizes (amax init + "
               "amax kernels + cast) back to back; fused and two-kernel regions alternate",
        "pages": "fused-amax PR 'Performance': full-quantize median latency, fused amax + cast "
                 "against row amax + column amax + cast, on one Blackwell SM100 (GB200); its "
                 "values did not survive the text extraction, so there is no number to set "
                 "these against",
    }

    ref = StreamRef(torch, dev)
    ceiling = ref.ceiling(timed)

    # dequantize the rowwise copy to BF16 (reported beside the step, not in it)
    y = torch.empty(M, K, dtype=torch.bfloat16, device=dev)
    dq = lambda i: p.nvfp4_dequantize(out["q_row"], out["s_row"], M, K, 1, ra, bound, y)
    for i in range(3):
        dq(i)
    dq_ms = timed(dq, 10)
    dq_bytes = M * ((K + 1) // 2) + M * ((K + 15) // 16) + 4 * M + M * K * 2
    del y

    row_meas = {} if args.no_rows else other_rows(
        Ctx(p, workloads, torch, dev, xs, timed, bound, ref, hold_queue))

    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        rows = min(args.cpu_rows, M)
        x_host = w.x[:rows].float().numpy()
        # whole passes (amax both directions, then both quantize directions)
        # until about cpu_seconds of wall time have been spent
        reps = 0
        t0 = time.perf_counter()
        while reps == 0 or (time.perf_counter() - t0 < args.cpu_seconds and reps < 100):
            ra_o, ca_o = oracle.amax_rows(x_host), oracle.amax_cols(x_host)
            oracle.quantize_rowwise(x_host, oracle.MODE_LINE, ra_o, bound)
            oracle.quantize_colwise(x_host, oracle.MODE_LINE, ca_o, bound)
            reps += 1
        dt = time.perf_counter() - t0
        threads = oracle.max_threads()
        # the same pass on one thread, over a sixteenth of the rows
        rows1 = max(16, rows // 16)
        x1 = np.ascontiguousarray(x_host[:rows1])
        oracle.set_threads(1)
        t1 = time.perf_counter()
        ra_o, ca_o = oracle.amax_rows(x1), oracle.amax_cols(x1)
        oracle.quantize_rowwise(x1, oracle.MODE_LINE, ra_o, bound)
        oracle.quantize_colwise(x1, oracle.MODE_LINE, ca_o, bound)
        dt1 = time.perf_counter() - t1
        oracle.set_threads(threads)
        cpu = {"value": round(reps * workloads.algorithmic_bytes(rows, K, 2) / dt / 1e9, 4),
               "unit": "GB/s", "cores": threads, "kind": "oracle", "cpu_model": cpu_model(),
               "host_cpus_available": len(os.sched_getaffinity(0)),
               "sample": f"{reps} pass(es) over the first {rows} rows x {K} columns of the same "
                         f"matrix (as its own {rows}x{K} input): amax rows+cols, then both "
                         f"quantize directions; {dt:.1f} s wall",
               "value_1_thread": round(workloads.algorithmic_bytes(rows1, K, 2) / dt1 / 1e9, 4),
               "sample_1_thread": f"one pass over the first {rows1} rows x {K} columns on 1 "
                                  f"thread; {dt1:.1f} s wall"}

    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K_steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "llm_mlp: 8192x28672 BF16, N(0,1) x per-row 10^U(-2,2), "
                               "row-scaled NVFP4 both directions, 1x16 blocks, bound 448",
                   "M": M, "K": K, "input_dtype": "bf16", "step_bytes": step_bytes,
                   "parallelism": "none (1 GPU)"},
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "roofline": {"bound": "hbm", "achieved": round(cast_gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(cast_gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(), "kernel": "cast_kernel (quantize-transpose)",
                     "bytes_per_launch": cast_bytes, "avg_us": round(cast_step * 1e3, 2),
                     "avg_of": "cast dispatches inside the steps, event pair around each"},
        "kernels_us": {"amax_init+fused_amax": round(amax_avg * 1e3, 2),
                       "cast_in_step": round(cast_step * 1e3, 2),
                       "cast_back_to_back": round(cast_avg * 1e3, 2),
                       "amax_GBs": round(amax_bytes / (amax_avg * 1e-3) / 1e9, 1),
                       "how": "each kind launched alone, back to back, same inputs"},
        "full_quantize_fused_vs_two_kernel": full_cmp,
        "hbm_measured": dict(ceiling, step_frac_of_copy=round(value / ceiling["copy_GBs"], 4),
                             cast_frac_of_copy=round(cast_gbs / ceiling["copy_GBs"], 4)),
        "dequant_rowwise_bf16": {"us": round(dq_ms * 1e3, 2),
                                 "GBs": round(dq_bytes / (dq_ms * 1e-3) / 1e9, 1),
                                 "frac": round(dq_bytes / (dq_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "other_rows": row_meas,
        "cpu_baseline": cpu,
        "source_digest": source_digest(),
        "library": os.path.relpath(p.library_path(), ROOT),
    }
    print(json.dumps(rec))


if __name__ == "__main__":
    main()

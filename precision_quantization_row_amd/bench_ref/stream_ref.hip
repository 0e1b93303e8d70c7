// stream_ref.hip -- reference streaming kernels for measuring what this GPU's
// HBM sustains (the achievable ceiling printed next to the quantize path's
// bandwidth). Not part of the NVFP4 library: plain 16-byte non-temporal reads,
// writes and copies over a buffer, grid-stride, with nothing else per byte,
// and a writer of scattered partial lines (the store-pattern probe).
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

template <bool NT>
__device__ __forceinline__ u32x4 load16(const u32x4* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

// Every kernel walks the buffer in chunks of kUnroll * 256 vectors (16 KB):
// workgroup b takes chunks b, b + grid, b + 2 grid, ...; in a chunk, load u
// of thread t is vector u * 256 + t, so each instruction of a wave covers
// 1 KB of contiguous memory and a thread keeps kUnroll loads in flight.

// Reads every 16-byte vector once and folds it into a register; the fold is
// stored only if it equals a value the caller can never arrange for all
// lanes (`never`), so no load can be removed. NT: non-temporal loads (the
// ceiling); otherwise ordinary loads, which allocate in the caches (the
// read-only cache flush).
template <bool NT>
__global__ void __launch_bounds__(kThreads) read_kernel(const u32x4* __restrict__ x, int64_t n,
                                                        uint32_t never, uint32_t* sink) {
  constexpr int64_t kChunk = (int64_t)kThreads * kUnroll;
  uint32_t acc = 0u;
  for (int64_t c = blockIdx.x; c * kChunk < n; c += gridDim.x) {
    const int64_t b = c * kChunk + threadIdx.x;
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = b + u * kThreads;
      v[u] = i < n ? load16<NT>(x + i) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == never) sink[0] = acc;
}

__global__ void __launch_bounds__(kThreads) write_kernel(u32x4* __restrict__ y, int64_t n,
                                                         uint32_t v) {
  constexpr int64_t kChunk = (int64_t)kThreads * kUnroll;
  const u32x4 w = {v, v, v, v};
  for (int64_t c = blockIdx.x; c * kChunk < n; c += gridDim.x) {
    const int64_t b = c * kChunk + threadIdx.x;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = b + u * kThreads;
      if (i < n) __builtin_nontemporal_store(w, y + i);
    }
  }
}

__global__ void __launch_bounds__(kThreads) copy_kernel(const u32x4* __restrict__ x,
                                                        u32x4* __restrict__ y, int64_t n) {
  constexpr int64_t kChunk = (int64_t)kThreads * kUnroll;
  for (int64_t c = blockIdx.x; c * kChunk < n; c += gridDim.x) {
    const int64_t b = c * kChunk + threadIdx.x;
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = b + u * kThreads;
      if (i < n) v[u] = __builtin_nontemporal_load(x + i);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = b + u * kThreads;
      if (i < n) __builtin_nontemporal_store(v[u], y + i);
    }
  }
}

// Writes a buffer of `lines` 128-byte lines in pieces of `piece` bytes (16,
// 32, 64 or 128), one 16-byte store per thread and step. Consecutive threads
// fill a piece (piece / 16 of them), and the next group of threads writes the
// same part of the next line: piece q goes to line q % lines at offset
// (q / lines) * piece. So one wave instruction writes 64 * 16 / piece pieces
// in as many consecutive lines (piece 128: 1 KB of whole lines), and a line's
// other pieces come from instructions much later -- the pattern of scattered
// partial lines. NT: non-temporal stores; otherwise ordinary ones.
template <bool NT>
__global__ void __launch_bounds__(kThreads) piece_write_kernel(u32x4* __restrict__ y, int64_t lines,
                                                               int piece, uint32_t v) {
  const int per = piece / 16;  // threads (16-byte stores) per piece
  const int64_t units = lines * 8;
  const u32x4 w = {v, v, v, v};
  for (int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x; u < units;
       u += (int64_t)gridDim.x * kThreads) {
    const int64_t q = u / per;
    const int k = (int)(u - q * per);
    const int64_t line = q % lines, part = q / lines;
    u32x4* d = y + line * 8 + part * per + k;
    if constexpr (NT) __builtin_nontemporal_store(w, d);
    else *d = w;
  }
}

bool ok(const void* p, int64_t bytes) {
  return p != nullptr && bytes > 0 && bytes % 16 == 0 && (reinterpret_cast<uintptr_t>(p) & 15) == 0;
}

int done() { return hipGetLastError() == hipSuccess ? 0 : -3; }

}  // namespace

extern "C" {

// Each returns -1 for a bad argument (NULL, size not a positive multiple of
// 16, pointer not 16-byte aligned, grid < 1), else 0 or -3 after enqueuing
// one kernel of `grid` workgroups of 256 threads on `stream`.
// cached != 0: ordinary loads (they allocate in the caches) instead of
// non-temporal ones.
int stream_read(const void* x, int64_t bytes, uint32_t* sink, int grid, int cached, void* stream) {
  if (!ok(x, bytes) || sink == nullptr || grid < 1) return -1;
  if (cached)
    hipLaunchKernelGGL(read_kernel<false>, dim3((unsigned)grid), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4*>(x), bytes / 16,
                       0xC0FFEE11u, sink);
  else
    hipLaunchKernelGGL(read_kernel<true>, dim3((unsigned)grid), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4*>(x), bytes / 16,
                       0xC0FFEE11u, sink);
  return done();
}

int stream_write(void* y, int64_t bytes, int grid, void* stream) {
  if (!ok(y, bytes) || grid < 1) return -1;
  hipLaunchKernelGGL(write_kernel, dim3((unsigned)grid), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<u32x4*>(y), bytes / 16, 0u);
  return done();
}

int stream_copy(const void* x, void* y, int64_t bytes, int grid, void* stream) {
  if (!ok(x, bytes) || !ok(y, bytes) || grid < 1) return -1;
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)grid), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(x),
                     static_cast<u32x4*>(y), bytes / 16);
  return done();
}

// bytes: a positive multiple of 128; piece: 16, 32, 64 or 128; nt != 0:
// non-temporal stores. -1 for a bad argument, else 0 or -3 after enqueuing
// one kernel of `grid` workgroups on `stream`.
int stream_pieces(void* y, int64_t bytes, int piece, int nt, int grid, void* stream) {
  if (!ok(y, bytes) || bytes % 128 != 0 || grid < 1 ||
      (piece != 16 && piece != 32 && piece != 64 && piece != 128))
    return -1;
  if (nt)
    hipLaunchKernelGGL(piece_write_kernel<true>, dim3((unsigned)grid), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<u32x4*>(y), bytes / 128, piece,
                       0u);
  else
    hipLaunchKernelGGL(piece_write_kernel<false>, dim3((unsigned)grid), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<u32x4*>(y), bytes / 128, piece,
                       0u);
  return done();
}

}  // extern "C"

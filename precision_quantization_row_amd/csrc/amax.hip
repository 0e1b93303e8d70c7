// amax.hip -- the amax pre-pass of row-scaled NVFP4 (gfx950).
//
// The two-pass design (TransformerEngine row-scaled backward PR, sequence
// diagram: row amax [M] and column amax [K] are computed before the cast) and
// its fused form (fused-amax PR commit message: one pass computes both
// directions, so the column reduction never reads global memory
// column-strided). amax is an exact max, so every kernel here produces the
// same bits whatever the reduction order; the fused and the separate kernels
// are interchangeable (fused-amax PR description).
//
// Publication: a magnitude's fp32 bit pattern orders like the magnitude, so
// partial maxima are published with 32-bit unsigned atomic max onto buffers a
// noop-aware kernel has zeroed on the device (never a host memset: the
// fused-amax PR review found that clearing before a skipped call destroys the
// preserved amax state).
#include "nvfp4_device.h"
#include "nvfp4_launch.h"

#include <algorithm>

namespace nvfp4 {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bool skip(const float* noop) { return noop != nullptr && *noop == 1.0f; }

// ------------------------------------------------------------------ init
__global__ void __launch_bounds__(256) amax_init_kernel(float* ra, int64_t M, float* ca, int64_t K,
                                                        float* ta, const float* noop) {
  if (skip(noop)) return;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t t0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (ra)
    for (int64_t i = t0; i < M; i += stride) ra[i] = 0.0f;
  if (ca)
    for (int64_t i = t0; i < K; i += stride) ca[i] = 0.0f;
  if (ta && t0 == 0) ta[0] = 0.0f;
}

// ------------------------------------------------------------------ fused
// Workgroup = 4 waves; a wave's 16-lane DPP row g reads 16 x 16 B of one row
// per load (128 BF16 or 64 FP32 columns: a "chunk"), so every load
// instruction fetches 4 full 256-byte row segments. The tile is tr rows x
// FUSED_NC chunks (tr = 256, or fewer for small matrices so that the grid
// still fills the GPU); the 16 (wave, row-group) slots take rows slot,
// slot + 16, ... Each lane keeps the running column max of its columns in
// registers (BF16: packed u16 magnitudes, v_pk_max_u16; FP32: one magnitude
// per dword), so the column reduction is a register reduction over rows --
// no strided global read and no LDS staging of the tile. Row maxima are
// reduced across the 16 lanes with DPP; column maxima of the 16 slots meet
// once in LDS; both are published with atomic max at the end of the tile,
// one per row and one per column.
//
// Any M, and any K whose rows are whole 16-byte vectors (K % 8 == 0 for
// BF16, K % 4 == 0 for FP32) with a 16-byte aligned X: a lane's 16-byte
// vector lies wholly inside the row or wholly past its end (then it reads
// nothing and counts as zeros), and rows past M are skipped.
constexpr int FUSED_TR = 256;  // rows per tile (largest)

// NC chunks per tile (the tile width), RU rows per slot per loop iteration:
// NC * RU 16-byte loads in flight per lane.
template <typename T, int NC>
struct FusedGeom {
  static constexpr int V = 16 / sizeof(T);  // elements per 16-byte vector
  static constexpr int CH = 16 * V;         // columns per chunk
  static constexpr int TC = CH * NC;        // columns per tile
};

// Magnitude bits of one dword's elements, maxed into acc (BF16: two packed
// u16 magnitudes; FP32: one).
template <typename T>
__device__ __forceinline__ uint32_t mag_max(uint32_t acc, uint32_t w) {
  if constexpr (sizeof(T) == 2) return pk_max_u16(acc, w & kAbsBf16x2);
  else return max(acc, w & kAbsF32);
}

// The FP32 bit pattern of the largest magnitude held in acc.
template <typename T>
__device__ __forceinline__ uint32_t mag_bits(uint32_t acc) {
  if constexpr (sizeof(T) == 2) return max(acc & 0xFFFFu, acc >> 16) << 16;
  else return acc;
}

template <typename T, int FUSED_NC, int FUSED_RU>
__global__ void __launch_bounds__(256) fused_amax_kernel(const T* __restrict__ x, int64_t M,
                                                         int64_t K, float* __restrict__ ra,
                                                         float* __restrict__ ca,
                                                         const float* noop, int64_t tiles_c,
                                                         int64_t tr) {
  if (skip(noop)) return;
  using G = FusedGeom<T, FUSED_NC>;
  __shared__ uint32_t colmax_s[16][FUSED_NC * 64 + 1];
  __shared__ uint32_t rowmax_s[FUSED_TR];  // the tile's row maxima, published at the end
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int q = lane & 15;           // lane within the DPP row
  const int slot = (tid >> 6) * 4 + (lane >> 4);  // 0..15
  const int64_t tile = blockIdx.x;
  const int64_t r0 = (tile / tiles_c) * tr;
  const int64_t c0 = (tile % tiles_c) * G::TC;

  uint32_t cm[FUSED_NC][4];
#pragma unroll
  for (int j = 0; j < FUSED_NC; ++j)
#pragma unroll
    for (int d = 0; d < 4; ++d) cm[j][d] = 0u;

  // the lane's vector of chunk j: inside the row or wholly past its end
  bool colok[FUSED_NC];
#pragma unroll
  for (int j = 0; j < FUSED_NC; ++j) colok[j] = (c0 + G::CH * j + G::V * q) < K;

  const int64_t rend = min(r0 + tr, M);
  // FUSED_RU rows per slot and iteration, all loads issued before any use
  // (rows past rend are skipped).
  //
  // The first half of the tile's rows is read with non-temporal loads, the
  // second half with ordinary ones: X is read again by the cast right after
  // this pass, and what this pass reads last is what the caches still hold
  // then. Measured on 8192 x 28672 BF16 (same GPU, step = this pass + the
  // cast): streamed fraction 0: 217 us, 1/4: 209, 3/8: 207, 1/2: 205-207,
  // 5/8: 207, 3/4: 208-209 (this pass alone: 87 us with none streamed, 79.6
  // with half).
  const int64_t r_stream = r0 + tr / 2;
  for (int64_t rb = r0 + slot; rb < rend; rb += 16 * FUSED_RU) {
    uint4 v[FUSED_RU][FUSED_NC];
    const bool stream = rb < r_stream;
#pragma unroll
    for (int u = 0; u < FUSED_RU; ++u) {
      const int64_t r = rb + 16 * u;
      const uint4* rowp = reinterpret_cast<const uint4*>(x + r * K + c0) + q;
#pragma unroll
      for (int j = 0; j < FUSED_NC; ++j) {
        if (colok[j] && r < rend) {
          if (stream) {
            const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(rowp + 16 * j));
            v[u][j] = make_uint4(t.x, t.y, t.z, t.w);
          } else {
            v[u][j] = rowp[16 * j];
          }
        } else {
          v[u][j] = make_uint4(0, 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < FUSED_RU; ++u) {
      const int64_t r = rb + 16 * u;
      uint32_t rm = 0u;
#pragma unroll
      for (int j = 0; j < FUSED_NC; ++j) {
        cm[j][0] = mag_max<T>(cm[j][0], v[u][j].x);
        cm[j][1] = mag_max<T>(cm[j][1], v[u][j].y);
        cm[j][2] = mag_max<T>(cm[j][2], v[u][j].z);
        cm[j][3] = mag_max<T>(cm[j][3], v[u][j].w);
        rm = mag_max<T>(mag_max<T>(mag_max<T>(mag_max<T>(rm, v[u][j].x), v[u][j].y), v[u][j].z),
                        v[u][j].w);
      }
      uint32_t rbits = row16_max(mag_bits<T>(rm));
      if (q == 0 && r < rend) rowmax_s[r - r0] = rbits;  // row r has one writer in the tile
    }
  }

  // column maxima: the 16 slots meet in LDS, one atomic per column per tile
#pragma unroll
  for (int j = 0; j < FUSED_NC; ++j)
#pragma unroll
    for (int d = 0; d < 4; ++d) colmax_s[slot][j * 64 + q * 4 + d] = cm[j][d];
  __syncthreads();
  // Row maxima are published here rather than inside the load loop: a
  // memory atomic there sits in the same in-order counter as the loads and
  // holds up the waits for the next rows.
  if (tid < rend - r0) atomicMax(reinterpret_cast<unsigned int*>(ra + r0 + tid), rowmax_s[tid]);
  // 256 threads, FUSED_NC * 64 dwords (BF16: two columns each, FP32: one)
  for (int e = tid; e < FUSED_NC * 64; e += 256) {
    uint32_t m = 0u;
#pragma unroll
    for (int s = 0; s < 16; ++s) m = mag_max<T>(m, colmax_s[s][e]);  // magnitudes already
    const int j = e / 64, w = e % 64;  // w = q * 4 + d
    if constexpr (sizeof(T) == 2) {
      const int64_t col = c0 + G::CH * j + 2 * w;  // columns 8q + 2d, +1
      if (col < K) {
        atomicMax(reinterpret_cast<unsigned int*>(ca + col), (m & 0xFFFFu) << 16);
        atomicMax(reinterpret_cast<unsigned int*>(ca + col + 1), m & 0xFFFF0000u);
      }
    } else {
      const int64_t col = c0 + G::CH * j + w;  // column 4q + d
      if (col < K) atomicMax(reinterpret_cast<unsigned int*>(ca + col), m);
    }
  }
}

// Magnitude bits of the largest element in one 16-byte vector (BF16: the
// larger half shifted into fp32 position).
template <typename T>
__device__ __forceinline__ uint32_t vec_max_bits(const uint4 v) {
  if constexpr (sizeof(T) == 2) {
    const uint32_t t = pk_max_u16(pk_max_u16(v.x & kAbsBf16x2, v.y & kAbsBf16x2),
                                  pk_max_u16(v.z & kAbsBf16x2, v.w & kAbsBf16x2));
    return max(t & 0xFFFFu, t >> 16) << 16;
  } else {
    return max(max(v.x & kAbsF32, v.y & kAbsF32), max(v.z & kAbsF32, v.w & kAbsF32));
  }
}

// The lane's share of a row max over nv 16-byte vectors (lane, lane + 64, ...):
// four independent loads in flight per iteration, so a wave that owns a row
// keeps 4 KB of it on the way instead of 1 KB.
template <typename T>
__device__ __forceinline__ uint32_t lane_row_max(const uint4* __restrict__ rv, int64_t nv, int lane) {
  uint32_t m0 = 0u, m1 = 0u;
  int64_t i = lane;
  for (; i + 192 < nv; i += 256) {
    const uint4 a = rv[i], b = rv[i + 64], c = rv[i + 128], d = rv[i + 192];
    m0 = max(m0, max(vec_max_bits<T>(a), vec_max_bits<T>(b)));
    m1 = max(m1, max(vec_max_bits<T>(c), vec_max_bits<T>(d)));
  }
  for (; i < nv; i += 64) m0 = max(m0, vec_max_bits<T>(rv[i]));
  return max(m0, m1);
}

// -------------------------------------------------------------- row amax
// One wave per row (grid-stride over rows); lanes stride the row with 16-byte
// vectors when every row starts 16-byte aligned, else with scalar loads. The
// wave owns its row, so the result is stored directly.
template <typename T, bool VEC>
__global__ void __launch_bounds__(256) row_amax_kernel(const T* __restrict__ x, int64_t M,
                                                       int64_t K, float* __restrict__ ra,
                                                       const float* noop) {
  if (skip(noop)) return;
  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
  constexpr int V = 16 / sizeof(T);
  for (int64_t r = wave; r < M; r += nwaves) {
    const T* row = x + r * K;
    uint32_t m = 0u;
    if (VEC) {
      const int64_t nv = K / V;
      m = lane_row_max<T>(reinterpret_cast<const uint4*>(row), nv, lane);
      for (int64_t i = nv * V + lane; i < K; i += 64) {  // K % V tail (never with VEC rows)
        if constexpr (sizeof(T) == 2)
          m = max(m, (uint32_t)(reinterpret_cast<const uint16_t*>(row)[i] & 0x7FFFu) << 16);
        else
          m = max(m, reinterpret_cast<const uint32_t*>(row)[i] & kAbsF32);
      }
    } else {
      for (int64_t i = lane; i < K; i += 64) {
        if constexpr (sizeof(T) == 2)
          m = max(m, (uint32_t)(reinterpret_cast<const uint16_t*>(row)[i] & 0x7FFFu) << 16);
        else
          m = max(m, reinterpret_cast<const uint32_t*>(row)[i] & kAbsF32);
      }
    }
    // wave max
    for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
    if (lane == 0) ra[r] = __uint_as_float(m);
  }
}

// ----------------------------------------------------------- column amax
// Workgroup = 4 waves over one strip of columns; lane l owns columns
// c0 + V*l .. +V (16-byte vector when rows are 16-byte aligned) or column
// c0 + l (scalar). Each wave walks a quarter of the workgroup's row segment,
// reading whole row segments (coalesced), and keeps the column max in
// registers; the 4 waves meet in LDS and publish one atomic max per column.
template <typename T, bool VEC>
__global__ void __launch_bounds__(256) col_amax_kernel(const T* __restrict__ x, int64_t M,
                                                       int64_t K, float* __restrict__ ca,
                                                       const float* noop, int64_t rows_per_wg) {
  if (skip(noop)) return;
  constexpr int V = VEC ? (16 / sizeof(T)) : 1;
  __shared__ uint32_t part[4][64 * V];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int64_t c0 = (int64_t)blockIdx.x * 64 * V;
  const int64_t rs = (int64_t)blockIdx.y * rows_per_wg;
  const int64_t re = min(rs + rows_per_wg, M);
  uint32_t m[V];
#pragma unroll
  for (int k = 0; k < V; ++k) m[k] = 0u;
  const int64_t c = c0 + (int64_t)lane * V;
  // one 16-byte vector of a row into the lane's running column maxima
  auto take = [&](const uint4 v) {
    if constexpr (VEC) {
      const uint32_t dw[4] = {v.x, v.y, v.z, v.w};
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          m[2 * d] = max(m[2 * d], (dw[d] & 0x7FFFu) << 16);
          m[2 * d + 1] = max(m[2 * d + 1], dw[d] & 0x7FFF0000u);
        }
      } else {
#pragma unroll
        for (int d = 0; d < 4; ++d) m[d] = max(m[d], dw[d] & kAbsF32);
      }
    }
  };
  if (c < K) {
    int64_t r = rs + w;
    if constexpr (VEC) {  // four rows in flight per wave
      for (; r + 12 < re; r += 16) {
        const uint4 a = *reinterpret_cast<const uint4*>(x + r * K + c);
        const uint4 b = *reinterpret_cast<const uint4*>(x + (r + 4) * K + c);
        const uint4 d = *reinterpret_cast<const uint4*>(x + (r + 8) * K + c);
        const uint4 e = *reinterpret_cast<const uint4*>(x + (r + 12) * K + c);
        take(a);
        take(b);
        take(d);
        take(e);
      }
    }
    for (; r < re; r += 4) {
      const T* p = x + r * K + c;
      if constexpr (VEC) {
        take(*reinterpret_cast<const uint4*>(p));
      } else {
        if constexpr (sizeof(T) == 2)
          m[0] = max(m[0], (uint32_t)(*reinterpret_cast<const uint16_t*>(p) & 0x7FFFu) << 16);
        else
          m[0] = max(m[0], *reinterpret_cast<const uint32_t*>(p) & kAbsF32);
      }
    }
  }
#pragma unroll
  for (int k = 0; k < V; ++k) part[w][lane * V + k] = m[k];
  __syncthreads();
  for (int e = threadIdx.x; e < 64 * V; e += 256) {
    const uint32_t v = max(max(part[0][e], part[1][e]), max(part[2][e], part[3][e]));
    const int64_t col = c0 + e;
    if (col < K) atomicMax(reinterpret_cast<unsigned int*>(ca + col), v);
  }
}

// ------------------------------------------------------------ tensor amax
// A persistent grid of at most one 16-wave workgroup per CU: each wave keeps
// four 1 KB loads in flight, and only one atomic per workgroup reaches the
// result word (same-word atomics from thousands of workgroups serialize).
constexpr int TENSOR_THREADS = 1024;
template <typename T, bool VEC>
__global__ void __launch_bounds__(TENSOR_THREADS) tensor_amax_kernel(const T* __restrict__ x, int64_t n,
                                                          float* __restrict__ ta,
                                                          const float* noop) {
  if (skip(noop)) return;
  __shared__ uint32_t red[TENSOR_THREADS / 64];
  constexpr int V = 16 / sizeof(T);
  const int64_t t0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  uint32_t m = 0u;
  int64_t done = 0;
  if (VEC) {
    const uint4* xv = reinterpret_cast<const uint4*>(x);
    const int64_t nv = n / V;
    // a wave reads 64 x 16 B per load; four loads of consecutive 1 KB pieces
    // are in flight per wave and iteration. The first two pieces stream past
    // the caches (non-temporal) and the last two are read normally, so the
    // cast that reads X next finds half of it in the memory-side cache
    // without this pass evicting that half. Measured on 8192 x 28672 BF16
    // (same GPU, per-tensor amax + 2-D cast per step): all pieces cached
    // 208.0 us per step (this pass alone 80.6 us), all streamed 207.2 (72.7),
    // half and half 194.3 (74.1).
    const int64_t lane = threadIdx.x & 63, wave = t0 >> 6, nwaves = stride >> 6;
    int64_t i = wave * 256 + lane;
    for (; i + 192 < nv; i += nwaves * 256) {
      const u32x4 sa = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(xv + i));
      const u32x4 sb = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(xv + i + 64));
      const uint4 a = make_uint4(sa.x, sa.y, sa.z, sa.w), b = make_uint4(sb.x, sb.y, sb.z, sb.w);
      const uint4 c = xv[i + 128], d = xv[i + 192];
      m = max(m, max(max(vec_max_bits<T>(a), vec_max_bits<T>(b)),
                     max(vec_max_bits<T>(c), vec_max_bits<T>(d))));
    }
    // a lane stops early only in the last, partial group: the rest of it
    for (; i < nv; i += 64) m = max(m, vec_max_bits<T>(xv[i]));
    done = nv * V;
  }
  for (int64_t i = done + t0; i < n; i += stride) {
    if constexpr (sizeof(T) == 2)
      m = max(m, (uint32_t)(reinterpret_cast<const uint16_t*>(x)[i] & 0x7FFFu) << 16);
    else
      m = max(m, reinterpret_cast<const uint32_t*>(x)[i] & kAbsF32);
  }
  for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t v = 0u;
#pragma unroll
    for (int r = 0; r < TENSOR_THREADS / 64; ++r) v = max(v, red[r]);
    atomicMax(reinterpret_cast<unsigned int*>(ta), v);
  }
}

// ----------------------------------------------------- group expansion
// One workgroup per group: max over the group's rows, then every row of the
// group receives it. Groups are disjoint, so the in-place update is safe.
// Validity of the group ends for the transposed copy's per-group blocks:
// every entry within [0, M], non-decreasing, and a multiple of 16 unless it
// equals M (a 1x16 column block must not straddle a group boundary). One
// workgroup; *status = 0 when valid, else 1 + the first g whose end breaks a
// rule.
__global__ void __launch_bounds__(256) group_check_kernel(const int64_t* __restrict__ group_end,
                                                          int64_t G, int64_t M, int32_t* status,
                                                          const float* noop) {
  if (skip(noop)) return;
  __shared__ int64_t first[4];
  int64_t bad = G;  // smallest bad g seen by this thread (G: none)
  for (int64_t g = threadIdx.x; g < G && g < bad; g += 256) {
    const int64_t e = group_end[g];
    const int64_t b = g == 0 ? 0 : group_end[g - 1];
    if (e < 0 || e > M || e < b || (e != M && e % 16 != 0)) bad = g;
  }
  for (int off = 32; off > 0; off >>= 1) bad = min(bad, (int64_t)__shfl_xor(bad, off));
  if ((threadIdx.x & 63) == 0) first[threadIdx.x >> 6] = bad;
  __syncthreads();
  if (threadIdx.x == 0) {
    const int64_t f = min(min(first[0], first[1]), min(first[2], first[3]));
    *status = f < G ? (int32_t)min(f + 1, (int64_t)0x7FFFFFFF) : 0;
  }
}

// status == nullptr: expand whatever the ends are (clamped); otherwise only
// when group_check_kernel found them valid, so misaligned groups leave ra
// unchanged.
__global__ void __launch_bounds__(256) group_expand_kernel(float* __restrict__ ra, int64_t M,
                                                           const int64_t* __restrict__ group_end,
                                                           const int32_t* status,
                                                           const float* noop) {
  if (skip(noop)) return;
  if (status != nullptr && *status != 0) return;
  __shared__ uint32_t red[4];
  const int64_t g = blockIdx.x;
  int64_t s = g == 0 ? 0 : group_end[g - 1];
  int64_t e = group_end[g];
  s = min(max(s, (int64_t)0), M);
  e = min(max(e, (int64_t)0), M);
  uint32_t m = 0u;
  for (int64_t i = s + threadIdx.x; i < e; i += 256) m = max(m, __float_as_uint(ra[i]) & kAbsF32);
  for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  const float v = __uint_as_float(max(max(red[0], red[1]), max(red[2], red[3])));
  for (int64_t i = s + threadIdx.x; i < e; i += 256) ra[i] = v;
}

// ------------------------------------------------------- grouped tokens
// Grouped tokens with padding on the way in (grouped-GEMM PR description:
// per-group global scales from the group amax, expanded to every row of the
// padded group). Pass 1: one wave per token row writes the row's max into the
// padded row the token lands in (a row that does not fit in M_out is
// skipped). Pass 2: one workgroup per group reduces those row maxima and
// writes the group max over the group's padded rows; the workgroups past the
// last group write 0 over the rows past it. Every row of [0, M_out) is
// written once, so nothing has to be zeroed first. T, M_out < 2^31.
template <typename T, bool VEC>
__global__ void __launch_bounds__(256) grouped_row_amax_kernel(const T* __restrict__ x,
                                                               int64_t T_rows, int64_t K,
                                                               const int64_t* grows, int G,
                                                               int64_t align, int64_t M_out,
                                                               float* __restrict__ ra,
                                                               const float* noop) {
  if (skip(noop)) return;
  const int lane = threadIdx.x & 63;
  const LaneEnds e = lane_group_ends(grows, G, align, lane);
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
  constexpr int V = 16 / sizeof(T);
  for (int64_t r = wave; r < T_rows; r += nwaves) {
    // the row's loads go out first; its place in the padded layout is looked
    // up while they are in flight (a row past the groups is read and dropped)
    const T* row = x + r * K;
    uint32_t m = 0u;
    if (VEC) {
      m = lane_row_max<T>(reinterpret_cast<const uint4*>(row), K / V, lane);
    } else {
      for (int64_t i = lane; i < K; i += 64) {
        if constexpr (sizeof(T) == 2)
          m = max(m, (uint32_t)(reinterpret_cast<const uint16_t*>(row)[i] & 0x7FFFu) << 16);
        else
          m = max(m, reinterpret_cast<const uint32_t*>(row)[i] & kAbsF32);
      }
    }
    for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
    const uint32_t g = groups_ending_by(e.tok, (uint32_t)r);
    if (g >= (uint32_t)G) break;  // this and every later row lie past the groups
    const uint32_t t0 = g ? group_end_at(e.tok, g - 1) : 0u;
    const uint32_t p0 = g ? group_end_at(e.pad, g - 1) : 0u;
    const int64_t pr = (int64_t)p0 + (r - (int64_t)t0);
    if (lane == 0 && pr < M_out) ra[pr] = __uint_as_float(m);
  }
}

// Workgroup g < G: group g. Its token rows that exist (below T) and fit in
// M_out carry their row maxima from pass 1; their max goes over every padded
// row of the group that fits. Workgroups G .. grid - 1: zeros over
// [P_G, M_out), P_G = the padded end of the last group.
__global__ void __launch_bounds__(256) grouped_expand_kernel(float* __restrict__ ra,
                                                             const int64_t* grows, int G,
                                                             int64_t align, int64_t T_rows,
                                                             int64_t M_out, const float* noop) {
  if (skip(noop)) return;
  __shared__ uint32_t wmax[4];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const LaneEnds e = lane_group_ends(grows, G, align, lane);
  const int64_t PG = group_end_at(e.pad, (uint32_t)G - 1);
  if ((int)blockIdx.x >= G) {
    const int64_t n = (int64_t)gridDim.x - G;
    for (int64_t i = PG + ((int64_t)blockIdx.x - G) * 256 + tid; i < M_out; i += n * 256) ra[i] = 0.0f;
    return;
  }
  const uint32_t g = blockIdx.x;
  const int64_t t0 = g ? group_end_at(e.tok, g - 1) : 0u, t1 = group_end_at(e.tok, g);
  const int64_t p0 = g ? group_end_at(e.pad, g - 1) : 0u, p1 = group_end_at(e.pad, g);
  const int64_t pe = min(p1, M_out);
  if (p0 >= pe) return;  // empty group, or past M_out (uniform per workgroup)
  // rows of the group written by pass 1
  const int64_t n = min(min(t1, T_rows) - t0, pe - p0);
  uint32_t m = 0u;
  for (int64_t i = tid; i < n; i += 256) m = max(m, __float_as_uint(ra[p0 + i]));
  for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  if (lane == 0) wmax[wv] = m;
  __syncthreads();
  const float v = __uint_as_float(max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3])));
  for (int64_t i = p0 + tid; i < pe; i += 256) ra[i] = v;
}

// ================================================================ launchers

int launch_amax_init(float* ra, int64_t M, float* ca, int64_t K, float* ta, const float* noop,
                     hipStream_t s) {
  const int64_t n = max(ra ? M : 0, ca ? K : 0);
  const int blocks = (int)std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, 1024));
  hipLaunchKernelGGL(amax_init_kernel, dim3(blocks), dim3(256), 0, s, ra, M, ca, K, ta, noop);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

template <typename T, int NC, int RU>
static int launch_fused_nc(const void* x, int64_t M, int64_t K, float* ra, float* ca,
                           const float* noop, hipStream_t s, int64_t tr_min) {
  const int64_t tiles_c = (K + FusedGeom<T, NC>::TC - 1) / FusedGeom<T, NC>::TC;
  // Tall tiles publish fewer column maxima; short ones give more workgroups.
  // Take the tallest tile (256 .. tr_min rows) that still gives about 6
  // workgroups per CU.
  int64_t tr = FUSED_TR;
  while (tr > tr_min && ((M + tr - 1) / tr) * tiles_c < (int64_t)num_cus() * 6) tr /= 2;
  const int64_t tiles_r = (M + tr - 1) / tr;
  hipLaunchKernelGGL((fused_amax_kernel<T, NC, RU>), dim3((unsigned)(tiles_r * tiles_c)),
                     dim3(256), 0, s, static_cast<const T*>(x), M, K, ra, ca, noop, tiles_c, tr);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

// Tile shape per matrix. Large matrices (256-row tiles of 4 chunks already
// give 6 workgroups per CU) and tiny ones keep 4-chunk tiles. In between,
// 128-column tiles of 128 rows or more (1 BF16 / 2 FP32 chunks, 8 loads in
// flight per lane) publish about half as many atomics as 512-column tiles cut
// to 32 rows for the same workgroup count: 4096 x 4096 BF16 7.2 us against
// 10.1 (amax pass back to back), FP32 4097 x 2880 the same or better.
template <typename T>
static int launch_fused_t(const void* x, int64_t M, int64_t K, float* ra, float* ca,
                          const float* noop, hipStream_t s) {
  const int64_t cus = num_cus();
  const int64_t t4 = (K + FusedGeom<T, 4>::TC - 1) / FusedGeom<T, 4>::TC;
  if (((M + FUSED_TR - 1) / FUSED_TR) * t4 >= cus * 6)
    return launch_fused_nc<T, 4, 2>(x, M, K, ra, ca, noop, s, 32);
  constexpr int NN = sizeof(T) == 2 ? 1 : 2, RN = 8 / NN;
  const int64_t tn = (K + FusedGeom<T, NN>::TC - 1) / FusedGeom<T, NN>::TC;
  if (((M + 127) / 128) * tn >= cus * 2) return launch_fused_nc<T, NN, RN>(x, M, K, ra, ca, noop, s, 128);
  return launch_fused_nc<T, 4, 2>(x, M, K, ra, ca, noop, s, 32);
}

int launch_fused_amax(const void* x, int in_dtype, int64_t M, int64_t K, float* ra, float* ca,
                      const float* noop, hipStream_t s) {
  return in_dtype == 0 ? launch_fused_t<uint16_t>(x, M, K, ra, ca, noop, s)
                       : launch_fused_t<float>(x, M, K, ra, ca, noop, s);
}

template <typename T>
static int launch_row_col_t(const void* xv, int64_t M, int64_t K, float* ra, float* ca,
                            const float* noop, hipStream_t s) {
  const T* x = static_cast<const T*>(xv);
  constexpr int V = 16 / sizeof(T);
  const bool vec = ((K % V) == 0) && ((reinterpret_cast<uintptr_t>(x) & 15) == 0);
  if (ra) {
    const int64_t blocks = std::min<int64_t>((M + 3) / 4, (int64_t)num_cus() * 16);
    if (vec)
      hipLaunchKernelGGL((row_amax_kernel<T, true>), dim3((unsigned)blocks), dim3(256), 0, s, x, M, K, ra, noop);
    else
      hipLaunchKernelGGL((row_amax_kernel<T, false>), dim3((unsigned)blocks), dim3(256), 0, s, x, M, K, ra, noop);
    if (hipGetLastError() != hipSuccess) return -3;
  }
  if (ca) {
    const int64_t cols_per_wg = vec ? 64 * V : 64;
    const int64_t strips = (K + cols_per_wg - 1) / cols_per_wg;
    // enough row segments for ~8 workgroups per CU, at least 64 rows each
    int64_t segs = std::max<int64_t>(1, ((int64_t)num_cus() * 8 + strips - 1) / strips);
    segs = std::min<int64_t>(segs, std::max<int64_t>(1, (M + 63) / 64));
    segs = std::min<int64_t>(segs, 65535);
    const int64_t rows_per_wg = (M + segs - 1) / segs;
    segs = (M + rows_per_wg - 1) / rows_per_wg;
    dim3 grid((unsigned)strips, (unsigned)segs);
    if (vec)
      hipLaunchKernelGGL((col_amax_kernel<T, true>), grid, dim3(256), 0, s, x, M, K, ca, noop, rows_per_wg);
    else
      hipLaunchKernelGGL((col_amax_kernel<T, false>), grid, dim3(256), 0, s, x, M, K, ca, noop, rows_per_wg);
    if (hipGetLastError() != hipSuccess) return -3;
  }
  return 0;
}

int launch_row_col_amax(const void* x, int in_dtype, int64_t M, int64_t K, float* ra, float* ca,
                        const float* noop, hipStream_t s) {
  return in_dtype == 0 ? launch_row_col_t<uint16_t>(x, M, K, ra, ca, noop, s)
                       : launch_row_col_t<float>(x, M, K, ra, ca, noop, s);
}

template <typename T>
static int launch_tensor_t(const void* xv, int64_t n, float* ta, const float* noop, hipStream_t s) {
  const T* x = static_cast<const T*>(xv);
  const bool vec = (reinterpret_cast<uintptr_t>(x) & 15) == 0;
  constexpr int V = 16 / sizeof(T);
  // one workgroup of 16 waves per CU at most: every workgroup ends with an
  // atomic on the same word, and those queue behind each other
  const int64_t blocks = std::max<int64_t>(
      1, std::min<int64_t>((n / V + 4 * TENSOR_THREADS - 1) / (4 * TENSOR_THREADS), (int64_t)num_cus()));
  if (vec)
    hipLaunchKernelGGL((tensor_amax_kernel<T, true>), dim3((unsigned)blocks), dim3(TENSOR_THREADS), 0, s,
                       x, n, ta, noop);
  else
    hipLaunchKernelGGL((tensor_amax_kernel<T, false>), dim3((unsigned)blocks), dim3(TENSOR_THREADS), 0, s,
                       x, n, ta, noop);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

int launch_tensor_amax(const void* x, int in_dtype, int64_t n, float* ta, const float* noop,
                       hipStream_t s) {
  return in_dtype == 0 ? launch_tensor_t<uint16_t>(x, n, ta, noop, s)
                       : launch_tensor_t<float>(x, n, ta, noop, s);
}

int launch_group_expand(float* ra, int64_t M, const int64_t* group_end, int64_t G,
                        int32_t* status, const float* noop, hipStream_t s) {
  if (status != nullptr) {
    hipLaunchKernelGGL(group_check_kernel, dim3(1), dim3(256), 0, s, group_end, G, M, status, noop);
    if (hipGetLastError() != hipSuccess) return -3;
  }
  hipLaunchKernelGGL(group_expand_kernel, dim3((unsigned)G), dim3(256), 0, s, ra, M, group_end,
                     status, noop);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // namespace nvfp4

namespace nvfp4 {

int launch_grouped_amax(const void* x, int in_dtype, int64_t T, int64_t K, const int64_t* grows,
                        int64_t G, int64_t align, int64_t M_out, float* ra, const float* noop,
                        hipStream_t s) {
  // a few rows per wave, so that its group-table setup is shared
  const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>((T + 3) / 4, (int64_t)num_cus() * 4));
  const bool vec16 = ((reinterpret_cast<uintptr_t>(x) & 15) == 0);
  const int g = (int)G;
  if (in_dtype == 0) {
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    if (vec16 && K % 8 == 0)
      hipLaunchKernelGGL((grouped_row_amax_kernel<uint16_t, true>), dim3((unsigned)blocks), dim3(256),
                         0, s, xb, T, K, grows, g, align, M_out, ra, noop);
    else
      hipLaunchKernelGGL((grouped_row_amax_kernel<uint16_t, false>), dim3((unsigned)blocks), dim3(256),
                         0, s, xb, T, K, grows, g, align, M_out, ra, noop);
  } else {
    const float* xf = static_cast<const float*>(x);
    if (vec16 && K % 4 == 0)
      hipLaunchKernelGGL((grouped_row_amax_kernel<float, true>), dim3((unsigned)blocks), dim3(256), 0,
                         s, xf, T, K, grows, g, align, M_out, ra, noop);
    else
      hipLaunchKernelGGL((grouped_row_amax_kernel<float, false>), dim3((unsigned)blocks), dim3(256), 0,
                         s, xf, T, K, grows, g, align, M_out, ra, noop);
  }
  if (hipGetLastError() != hipSuccess) return -3;
  // G group workgroups + enough for the zero tail (at most M_out rows)
  const int64_t tail = std::min<int64_t>((M_out + 255) / 256, (int64_t)num_cus() * 2);
  hipLaunchKernelGGL(grouped_expand_kernel, dim3((unsigned)(G + tail)), dim3(256), 0, s, ra, grows, g,
                     align, T, M_out, noop);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // namespace nvfp4

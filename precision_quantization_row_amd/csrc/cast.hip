// cast.hip -- the quantize-transpose pass of row-scaled NVFP4 (gfx950).
//
// One read of X produces both copies (TransformerEngine row-scaled backward
// PR summary: the columnwise / transposed output is emitted in the same kernel
// pass as the rowwise one, each direction with its own second-level amax).
//
// Geometry. A workgroup is 4 waves and owns a strip of 512 columns over a
// segment of rows; it walks the segment 64 rows at a time. In one step lane
// (wave w, DPP row g, lane-in-row q) holds a 16 x 8 register block of X:
// rows r0 + 16g .. +16, columns c0 + 128w + 8q .. +8. Each 16-lane DPP row
// loads 16 x 16 B of one row per BF16 load instruction (two for FP32), i.e.
// whole 256-byte (512-byte) row segments: loads are coalesced and X is never
// read column-strided. The transpose happens in registers:
//   rowwise   -- a 16-element row block spans the lane pair (q, q^1); their
//                8-element maxima meet through one DPP swap. The pair splits
//                the 16 block-scale computations (even lane: even rows, odd
//                lane: odd rows) and DPP broadcasts hand each row's encode
//                factor to both lanes.
//   columnwise-- each of the lane's 8 columns has all 16 rows of a column
//                block in the lane itself: the block max is a register
//                reduction (packed u16 max for BF16), no data exchange.
// Stores: a DPP row writes 64 contiguous bytes of rowwise codes per row (the 4
// waves of the workgroup fill 256 contiguous bytes); the 4 DPP rows of a wave
// write 4 x 8 contiguous bytes of one transposed line, and the workgroup's
// consecutive steps extend those lines, so partial lines meet in L2 before
// they are written back.
//
// Interior workgroups (the whole strip inside K, whole 64-row steps, aligned
// rows) use buffer loads and stores whose per-row offsets are uniform scalar
// values, so addressing costs no vector ALU; edge workgroups take a checked
// path with per-element bounds.
#include "nvfp4_device.h"
#include "nvfp4_launch.h"

#include <algorithm>

namespace nvfp4 {

constexpr int CAST_STEP_ROWS = 64;
constexpr int CAST_STRIP_COLS = 512;
constexpr int CAST_MAX_ROWS_PER_WG = 1024;
constexpr int kBufWord3 = 0x00020000;  // raw buffer, 32-bit data format (gfx9 family)

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

struct CastK {
  const void* x;
  int64_t M, K;
  int row_mode;
  const float* row_amax;
  int col_mode;
  const float* col_amax;
  float F, F_inv;
  uint8_t *q_row, *s_row, *q_col, *s_col;
  const float* noop;
  int vec_load;    // rows start 16-byte aligned
  int row_store4;  // K % 8 == 0: rowwise code rows are dword aligned
  int col_store8;  // M % 16 == 0: transposed code rows are 8-byte aligned
  // interior kernel: tiles of 64 rows x 512 columns in the first n_isteps
  // steps and n_istrips strips
  int64_t n_istrips, n_isteps;
  // edge kernel: rows [rstart, rend) in segments of rows_per_wg (a multiple of
  // CAST_STEP_ROWS, <= CAST_MAX_ROWS_PER_WG); workgroup b takes segment
  // seg0 + b / nstrips of strip strip0 + b % nstrips
  int64_t rstart, rend, rows_per_wg;
  int64_t seg0, strip0, nstrips;
};

// Lane block storage: NW dwords per row. BF16: 4 dwords = 8 values (element
// 2d in the low half of dword d). FP32: 8 dwords = 8 values.
template <typename T>
struct Blk {
  static constexpr int NW = sizeof(T) == 2 ? 4 : 8;
};

template <typename T>
__device__ __forceinline__ float elem(const uint32_t (&w)[16][Blk<T>::NW], int i, int k) {
  if constexpr (sizeof(T) == 2)
    return (k & 1) ? bf16_hi(w[i][k >> 1]) : bf16_lo(w[i][k >> 1]);
  else
    return __uint_as_float(w[i][k]);
}

// The same element through v_perm_b32 (the BF16 value's two bytes into the high
// half, zeros below; selector bytes 4..7 pick bytes of the first source, 0x0C
// gives zero). Used by the columnwise direction so that the compiler does not
// keep the rowwise direction's 128 unpacked values alive for reuse.
template <typename T>
__device__ __forceinline__ float elem_c(const uint32_t (&w)[16][Blk<T>::NW], int i, int k) {
  if constexpr (sizeof(T) == 2) {
    uint32_t r;
    if (k & 1)
      asm("v_perm_b32 %0, %1, 0, %2" : "=v"(r) : "v"(w[i][k >> 1]), "s"(0x07060c0cu));
    else
      asm("v_perm_b32 %0, %1, 0, %2" : "=v"(r) : "v"(w[i][k >> 1]), "s"(0x05040c0cu));
    return __uint_as_float(r);
  } else {
    return __uint_as_float(w[i][k]);
  }
}

// DPP quad_perm [0,0,2,2] / [1,1,3,3]: both lanes of a pair get the even /
// the odd lane's value.
__device__ __forceinline__ float bcast_even(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xA0, 0xF, 0xF, false));
}
__device__ __forceinline__ float bcast_odd(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xF5, 0xF, 0xF, false));
}

// ------------------------------------------------------------------ loads
template <typename T>
__device__ __forceinline__ void load_row_checked(const T* __restrict__ x, int64_t M, int64_t K,
                                                 int64_t r, int64_t c, bool vec,
                                                 uint32_t (&out)[Blk<T>::NW]) {
  constexpr int NW = Blk<T>::NW;
#pragma unroll
  for (int d = 0; d < NW; ++d) out[d] = 0u;
  if (r >= M || c >= K) return;
  const T* p = x + r * K + c;
  if constexpr (sizeof(T) == 2) {
    if (vec && c + 8 <= K) {
      const uint4 v = *reinterpret_cast<const uint4*>(p);
      out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
    } else {
      const uint16_t* h = reinterpret_cast<const uint16_t*>(p);
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (c + k < K) out[k >> 1] |= (uint32_t)h[k] << (16 * (k & 1));
    }
  } else {
    const uint32_t* f = reinterpret_cast<const uint32_t*>(p);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (vec && c + 4 * h + 4 <= K) {
        const uint4 v = *reinterpret_cast<const uint4*>(f + 4 * h);
        out[4 * h + 0] = v.x; out[4 * h + 1] = v.y; out[4 * h + 2] = v.z; out[4 * h + 3] = v.w;
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (c + 4 * h + k < K) out[4 * h + k] = f[4 * h + k];
      }
    }
  }
}

template <typename T>
__device__ __forceinline__ void load_row_buf(__amdgpu_buffer_rsrc_t rx, uint32_t vo, uint32_t so,
                                             uint32_t (&out)[Blk<T>::NW]) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)vo, (int)so, 0);
  out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
  if constexpr (sizeof(T) == 4) {
    const u32x4 u = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)(vo + 16u), (int)so, 0);
    out[4] = u.x; out[5] = u.y; out[6] = u.z; out[7] = u.w;
  }
}

// ------------------------------------------------------------------ stores
// Interior: buffer stores, lane offsets fixed per workgroup, row / column
// offsets uniform.
struct StoreFast {
  __amdgpu_buffer_rsrc_t qr, sr, qc, sc;
  uint32_t vo_qr, vo_sr, vo_qc, vo_sc;  // per lane
  uint32_t so_qr, so_sr, so_qc, so_sc;  // per step (uniform)
  uint32_t qrs, srs, qcs, scs;
  __device__ __forceinline__ void row_codes(int i, uint32_t word) const {
    __builtin_amdgcn_raw_buffer_store_b32(word, qr, (int)vo_qr, (int)(so_qr + i * qrs), 0);
  }
  // the scale of row 2j + par of the lane pair's block
  __device__ __forceinline__ void row_scale(int j, uint32_t byte) const {
    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)byte, sr, (int)vo_sr, (int)(so_sr + 2 * j * srs), 0);
  }
  __device__ __forceinline__ void col(int k, uint32_t w0, uint32_t w1, uint32_t byte) const {
    const u32x2 v = {w0, w1};
    __builtin_amdgcn_raw_buffer_store_b64(v, qc, (int)vo_qc, (int)(so_qc + k * qcs), 0);
    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)byte, sc, (int)vo_sc, (int)(so_sc + k * scs), 0);
  }
};

// Edge: global stores with bounds and alignment checks per element.
struct StoreChecked {
  uint8_t *q_row, *s_row, *q_col, *s_col;
  int64_t rb0, re, c, cb, K;
  int64_t qrs, srs, qcs, scs;
  int par;
  bool row4, col8;
  __device__ __forceinline__ void row_codes(int i, uint32_t word) const {
    const int64_t r = rb0 + i;
    if (r >= re || c >= K) return;
    uint8_t* dst = q_row + r * qrs + c / 2;
    if (row4 && c + 8 <= K) {
      *reinterpret_cast<uint32_t*>(dst) = word;
    } else {
#pragma unroll
      for (int b = 0; b < 4; ++b)
        if (c + 2 * b < K) dst[b] = (uint8_t)(word >> (8 * b));
    }
  }
  __device__ __forceinline__ void row_scale(int j, uint32_t byte) const {
    const int64_t r = rb0 + 2 * j + par;
    if (r < re && cb < K) s_row[r * srs + cb / 16] = (uint8_t)byte;
  }
  __device__ __forceinline__ void col(int k, uint32_t w0, uint32_t w1, uint32_t byte) const {
    const int64_t cc = c + k;
    if (rb0 >= re || cc >= K) return;
    s_col[cc * scs + rb0 / 16] = (uint8_t)byte;
    uint8_t* dst = q_col + cc * qcs + rb0 / 2;
    if (col8 && rb0 + 16 <= re) {
      *reinterpret_cast<uint2*>(dst) = make_uint2(w0, w1);
    } else {
#pragma unroll
      for (int b = 0; b < 8; ++b)
        if (rb0 + 2 * b < re) dst[b] = (uint8_t)((b < 4 ? w0 : w1) >> (8 * (b & 3)));
    }
  }
};

// ---------------------------------------------------------------- compute
// Both directions of one 64-row step from the lane's 16 x 8 register block.
//   row_a / row_s: amax and S_enc of the step's 64 rows (index: row - r0)
//   col_a / col_s: amax and S_enc of the lane's 8 columns (index k)
// Row pairs are encoded as soon as their block scales exist, so only the
// data block and the 4-register running column max stay live.
template <typename T, bool ROWW, bool COLW, class Store, class RowTab, class ColTab>
__device__ __forceinline__ void process_block(const uint32_t (&w)[16][Blk<T>::NW],
                                              const Store& st, int g, int par, const RowTab& row,
                                              const ColTab& col, float f_inv) {
  constexpr int NW = Blk<T>::NW;
  uint32_t cm[NW];
#pragma unroll
  for (int d = 0; d < NW; ++d) cm[d] = 0u;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t h[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int i = 2 * j + e;
      if constexpr (sizeof(T) == 2) {
        const uint32_t a0 = w[i][0] & kAbsBf16x2, a1 = w[i][1] & kAbsBf16x2;
        const uint32_t a2 = w[i][2] & kAbsBf16x2, a3 = w[i][3] & kAbsBf16x2;
        if constexpr (COLW) {
          cm[0] = pk_max_u16(cm[0], a0);
          cm[1] = pk_max_u16(cm[1], a1);
          cm[2] = pk_max_u16(cm[2], a2);
          cm[3] = pk_max_u16(cm[3], a3);
        }
        const uint32_t t = pk_max_u16(pk_max_u16(a0, a1), pk_max_u16(a2, a3));
        h[e] = max(t & 0xFFFFu, t >> 16) << 16;
      } else {
        uint32_t m = 0u;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const uint32_t av = w[i][k] & kAbsF32;
          if constexpr (COLW) cm[k] = max(cm[k], av);
          m = max(m, av);
        }
        h[e] = m;
      }
    }
    if constexpr (ROWW) {
      const uint32_t b0 = max(h[0], dpp_swap1(h[0]));
      const uint32_t b1 = max(h[1], dpp_swap1(h[1]));
      const uint32_t bsel = par ? b1 : b0;  // this lane's row: 2j + par
      const int lr = 16 * g + 2 * j + par;
      uint32_t byte;
      float enc;
      block_scale(__uint_as_float(bsel), row.a(lr), row.s(lr), f_inv, &byte, &enc);
      st.row_scale(j, byte);
      const float e0 = bcast_even(enc), e1 = bcast_odd(enc);
      st.row_codes(2 * j, e2m1_pack8(elem<T>(w, 2 * j, 0) * e0, elem<T>(w, 2 * j, 1) * e0,
                                     elem<T>(w, 2 * j, 2) * e0, elem<T>(w, 2 * j, 3) * e0,
                                     elem<T>(w, 2 * j, 4) * e0, elem<T>(w, 2 * j, 5) * e0,
                                     elem<T>(w, 2 * j, 6) * e0, elem<T>(w, 2 * j, 7) * e0));
      st.row_codes(2 * j + 1,
                   e2m1_pack8(elem<T>(w, 2 * j + 1, 0) * e1, elem<T>(w, 2 * j + 1, 1) * e1,
                              elem<T>(w, 2 * j + 1, 2) * e1, elem<T>(w, 2 * j + 1, 3) * e1,
                              elem<T>(w, 2 * j + 1, 4) * e1, elem<T>(w, 2 * j + 1, 5) * e1,
                              elem<T>(w, 2 * j + 1, 6) * e1, elem<T>(w, 2 * j + 1, 7) * e1));
    }
  }

  if constexpr (COLW) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      uint32_t cb;
      if constexpr (sizeof(T) == 2)
        cb = (k & 1) ? (cm[k >> 1] & 0xFFFF0000u) : (cm[k >> 1] << 16);
      else
        cb = cm[k];
      uint32_t byte;
      float enc;
      block_scale(__uint_as_float(cb), col.a(k), col.s(k), f_inv, &byte, &enc);
      // rows 0..7 -> w0 (row i in nibble i), rows 8..15 -> w1
      const uint32_t w0 = e2m1_pack8(elem_c<T>(w, 0, k) * enc, elem_c<T>(w, 1, k) * enc,
                                     elem_c<T>(w, 2, k) * enc, elem_c<T>(w, 3, k) * enc,
                                     elem_c<T>(w, 4, k) * enc, elem_c<T>(w, 5, k) * enc,
                                     elem_c<T>(w, 6, k) * enc, elem_c<T>(w, 7, k) * enc);
      const uint32_t w1 = e2m1_pack8(elem_c<T>(w, 8, k) * enc, elem_c<T>(w, 9, k) * enc,
                                     elem_c<T>(w, 10, k) * enc, elem_c<T>(w, 11, k) * enc,
                                     elem_c<T>(w, 12, k) * enc, elem_c<T>(w, 13, k) * enc,
                                     elem_c<T>(w, 14, k) * enc, elem_c<T>(w, 15, k) * enc);
      st.col(k, w0, w1, byte);
    }
  }
}

// Row / column tables in LDS (a pointer and a base index).
struct LdsTab {
  const float* pa;
  const float* ps;
  int base;
  __device__ __forceinline__ float a(int i) const { return pa[base + i]; }
  __device__ __forceinline__ float s(int i) const { return ps[base + i]; }
};
// The lane's 8 column values held in registers (edge kernel).
struct ColRegs {
  const float (&va)[8];
  const float (&vs)[8];
  __device__ __forceinline__ float a(int k) const { return va[k]; }
  __device__ __forceinline__ float s(int k) const { return vs[k]; }
};
// One value for every entry (per-tensor / group amax modes).
struct UniformTab {
  float va, vs;
  __device__ __forceinline__ float a(int) const { return va; }
  __device__ __forceinline__ float s(int) const { return vs; }
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = (int)(bytes < 0x7FFFFFFF ? bytes : 0x7FFFFFFF);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, kBufWord3);
}

// --------------------------------------------------------- interior kernel
// Interior tiles are 64 rows x 512 columns. A workgroup is 4 waves; wave w
// holds rows r0 + 16w .. +16 of the tile and all 512 columns, lane l a 16 x 8
// block at columns c0 + 8l, so every load instruction reads 1 KB of one row
// and every rowwise-code store writes 256 contiguous bytes of one row.
//
// Schedule. On this GPU write bandwidth depends on how long the contiguous
// runs that reach memory at about the same time are, far more than read
// bandwidth does. The persistent workgroups therefore advance in lockstep
// "super-steps": workgroup b runs on XCD x = b % 8 as its j = b / 8-th of
// P = grid / 8 workgroups there, and in super-step u it takes strip
// 8 * (u / nh) + x and tile row P * (u % nh) + j (nh = tile rows / P, rounded
// up). At any moment the P (64 on MI355X) workgroups of an XCD cover P
// consecutive tiles of one strip and the 8 XCDs cover 8 adjacent strips, so
//   rowwise codes      -- one row gets 8 x 256 B = 2 KB in the same window
//   transposed codes   -- one column gets 64 x 32 B = 2 KB, all from one XCD,
//                         so its lines fill up in that XCD's L2
//   scales             -- 256 B runs in both directions
// Within a tile the transposed codes (32 B per column), transposed scales
// (4 B per column) and rowwise scales (32 B per row) are gathered in LDS
// (double buffered) and stored 16 bytes per lane where the run allows it.
constexpr int T6_ROWS = 64;
constexpr int T6_COLS = CAST_STRIP_COLS;  // 512
constexpr int T6_XCDS = 8;

struct T6Smem {
  // transposed codes: [buf][column][4 waves x 8 B], wave w's slot at w ^ ((column >> 3) & 3)
  uint8_t qc[2][T6_COLS][32];
  // transposed scales: [buf][column][4 waves x 1 B]
  uint8_t sc[2][T6_COLS][4];
  // rowwise scales: [buf][row][32 B]
  uint8_t sr[2][T6_ROWS][32];
  // per-wave row amax / S_enc of the wave's 16 rows
  float ra[4][16], rs[4][16];
};

struct StoreT6 {
  __amdgpu_buffer_rsrc_t qr;  // rowwise codes of this tile
  uint32_t vo_qr, qrs;
  uint8_t* sr;
  uint8_t* qc;
  uint8_t* sc;
  int wv, lane, par;
  __device__ __forceinline__ void row_codes(int i, uint32_t word) const {
    __builtin_amdgcn_raw_buffer_store_b32(word, qr, (int)vo_qr, (int)(i * qrs), 0);
  }
  __device__ __forceinline__ void row_scale(int j, uint32_t byte) const {
    sr[(16 * wv + 2 * j + par) * 32 + (lane >> 1)] = (uint8_t)byte;
  }
  __device__ __forceinline__ void col(int k, uint32_t w0, uint32_t w1, uint32_t byte) const {
    const int c = 8 * lane + k;
    *reinterpret_cast<uint2*>(qc + c * 32 + 8 * (wv ^ (lane & 3))) = make_uint2(w0, w1);
    sc[c * 4 + wv] = (uint8_t)byte;
  }
};

template <typename T, bool ROWW, bool COLW>
__global__ void __launch_bounds__(256) cast_interior_kernel(const CastK p) {
  if (p.noop != nullptr && *p.noop == 1.0f) return;
  constexpr int NW = Blk<T>::NW;
  __shared__ __attribute__((aligned(16))) T6Smem sm;
  const T* __restrict__ x = static_cast<const T*>(p.x);
  const int tid = threadIdx.x;
  const int wv = tid >> 6;
  const int lane = tid & 63;
  const int par = lane & 1;
  const int64_t K = p.K;

  const int64_t G = gridDim.x;  // T6_XCDS * per_xcd workgroups
  const int64_t per_xcd = G / T6_XCDS;  // tiles of one strip an XCD covers per super-step
  const int64_t xcd = blockIdx.x % T6_XCDS, jw = blockIdx.x / T6_XCDS;
  const int64_t nstrips = p.n_istrips, ntrows = p.n_isteps;  // tile rows per strip
  const int64_t nh = (ntrows + per_xcd - 1) / per_xcd;
  const int64_t ng = (nstrips + T6_XCDS - 1) / T6_XCDS;

  const uint32_t rowbytes = (uint32_t)(K * (int64_t)sizeof(T));
  const int64_t qrs = (K + 1) / 2, srs = (K + 15) / 16;
  const int64_t qcs = (p.M + 1) / 2, scs = (p.M + 15) / 16;

  int buf = 0;
  for (int64_t u = 0; u < ng * nh; ++u) {
    const int64_t strip = T6_XCDS * (u / nh) + xcd;
    if (strip >= nstrips) continue;  // uniform per workgroup
    {
      const int64_t trow = per_xcd * (u % nh) + jw;
      if (trow >= ntrows) continue;  // uniform per workgroup
      const int64_t r0 = trow * T6_ROWS, c0 = strip * T6_COLS;

      // column amax / S_enc of the lane's 8 columns
      float acol[8], scol[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        float a = 0.0f;
        if constexpr (COLW) {
          if (p.col_mode == 0) a = p.col_amax[0];
          else if (p.col_mode == 1) a = p.col_amax[c0 + 8 * lane + k];
          else a = p.col_amax[r0 + 16 * wv];
        }
        acol[k] = a;
        scol[k] = COLW ? global_encode_scale(a, p.F) : 1.0f;
      }
      // row amax / S_enc of the wave's 16 rows
      if constexpr (ROWW) {
        if (lane < 16) {
          const float a = (p.row_mode == 0) ? p.row_amax[0] : p.row_amax[r0 + 16 * wv + lane];
          sm.ra[wv][lane] = a;
          sm.rs[wv][lane] = global_encode_scale(a, p.F);
        }
        __builtin_amdgcn_wave_barrier();
      }
      uint32_t w[16][NW];
      {
        const __amdgpu_buffer_rsrc_t rx =
            make_rsrc(x + (r0 + 16 * wv) * K + c0, (int64_t)16 * K * (int64_t)sizeof(T));
        const uint32_t vo = (uint32_t)(8 * lane * sizeof(T));
#pragma unroll
        for (int i = 0; i < 16; ++i) load_row_buf<T>(rx, vo, (uint32_t)i * rowbytes, w[i]);
      }
      StoreT6 st;
      st.wv = wv;
      st.lane = lane;
      st.par = par;
      st.qrs = (uint32_t)qrs;
      st.sr = &sm.sr[buf][0][0];
      st.qc = &sm.qc[buf][0][0];
      st.sc = &sm.sc[buf][0][0];
      if constexpr (ROWW) {
        st.qr = make_rsrc(p.q_row + (r0 + 16 * wv) * qrs + c0 / 2, (int64_t)16 * qrs);
        st.vo_qr = (uint32_t)(4 * lane);
      }
      process_block<T, ROWW, COLW>(w, st, 0, par, LdsTab{sm.ra[wv], sm.rs[wv], 0},
                                   ColRegs{acol, scol}, p.F_inv);
      __syncthreads();  // the tile's staged outputs are complete

      if constexpr (ROWW) {  // 64 rows x 32 B: two lanes per row, 16 B each
        if (tid < 2 * T6_ROWS) {
          const int row = tid >> 1, half = tid & 1;
          *reinterpret_cast<uint4*>(p.s_row + (r0 + row) * srs + c0 / 16 + 16 * half) =
              *reinterpret_cast<const uint4*>(&sm.sr[buf][row][16 * half]);
        }
      }
      if constexpr (COLW) {
        // 512 columns x 32 B: two lanes per column, 16 B each (wave slots
        // restored to row order)
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const int pidx = tid + 256 * it;
          const int c = pidx >> 1, half = pidx & 1;
          const int xsw = (c >> 3) & 3;
          const uint8_t* base = &sm.qc[buf][c][0];
          const uint2 lo = *reinterpret_cast<const uint2*>(base + 8 * ((2 * half) ^ xsw));
          const uint2 hi = *reinterpret_cast<const uint2*>(base + 8 * ((2 * half + 1) ^ xsw));
          *reinterpret_cast<uint4*>(p.q_col + (c0 + c) * qcs + r0 / 2 + 16 * half) =
              make_uint4(lo.x, lo.y, hi.x, hi.y);
        }
        // 512 columns x 4 B
#pragma unroll
        for (int it = 0; it < 2; ++it) {
          const int c = tid + 256 * it;
          *reinterpret_cast<uint32_t*>(p.s_col + (c0 + c) * scs + r0 / 16) =
              *reinterpret_cast<const uint32_t*>(&sm.sc[buf][c][0]);
        }
      }
      buf ^= 1;
    }
  }
}

// ------------------------------------------------------------- edge kernel
// Tiles outside the interior: the partial last strip, the partial last
// 64-row step, or every tile of a shape the buffer path cannot take. One
// workgroup per segment of rows_per_wg rows of one strip, checked loads and
// stores. Launched over a rectangle: segment seg0 + b / nstrips of the row
// range [rstart, rend), strip strip0 + b % nstrips.
template <typename T, bool ROWW, bool COLW>
__global__ void __launch_bounds__(256) cast_edge_kernel(const CastK p) {
  if (p.noop != nullptr && *p.noop == 1.0f) return;
  constexpr int NW = Blk<T>::NW;
  __shared__ float row_a_s[CAST_MAX_ROWS_PER_WG];
  __shared__ float row_se_s[CAST_MAX_ROWS_PER_WG];
  const T* __restrict__ x = static_cast<const T*>(p.x);
  const int tid = threadIdx.x;
  const int wv = tid >> 6;
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int q = lane & 15;
  const int par = q & 1;
  const int64_t M = p.M, K = p.K;

  const int64_t b = (int64_t)blockIdx.x;
  const int64_t strip = p.strip0 + b % p.nstrips;
  const int64_t seg = p.seg0 + b / p.nstrips;
  const int64_t c0 = strip * CAST_STRIP_COLS;
  const int64_t c = c0 + 128 * wv + 8 * q;  // lane's first column
  const int64_t rs = p.rstart + seg * p.rows_per_wg;
  const int64_t re = min(rs + p.rows_per_wg, p.rend);

  if constexpr (ROWW) {
    for (int i = tid; i < (int)p.rows_per_wg; i += 256) {
      float a = 0.0f;
      if (rs + i < re) a = (p.row_mode == 0) ? p.row_amax[0] : p.row_amax[rs + i];
      row_a_s[i] = a;
      row_se_s[i] = global_encode_scale(a, p.F);
    }
    __syncthreads();
  }

  float acol[8], scol[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    float a = 0.0f;
    if constexpr (COLW) {
      if (p.col_mode == 0) a = p.col_amax[0];
      else if (p.col_mode == 1 && c + k < K) a = p.col_amax[c + k];
    }
    acol[k] = a;
    scol[k] = COLW ? global_encode_scale(a, p.F) : 1.0f;
  }

  StoreChecked st;
  st.q_row = p.q_row;
  st.s_row = p.s_row;
  st.q_col = p.q_col;
  st.s_col = p.s_col;
  st.re = re;
  st.c = c;
  st.cb = c - 8 * par;
  st.K = K;
  st.qrs = (K + 1) / 2;
  st.srs = (K + 15) / 16;
  st.qcs = (M + 1) / 2;
  st.scs = (M + 15) / 16;
  st.par = par;
  st.row4 = p.row_store4 != 0;
  st.col8 = p.col_store8 != 0;
  const bool vec = p.vec_load != 0;
  for (int64_t r0 = rs; r0 < re; r0 += CAST_STEP_ROWS) {
    const int64_t rb0 = r0 + 16 * g;
    uint32_t w[16][NW];
#pragma unroll
    for (int i = 0; i < 16; ++i) load_row_checked<T>(x, re, K, rb0 + i, c, vec, w[i]);
    st.rb0 = rb0;
    if constexpr (COLW) {
      if (p.col_mode == 2) {
        const float ga = rb0 < re ? p.col_amax[rb0] : 0.0f;
        const float gse = global_encode_scale(ga, p.F);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          acol[k] = ga;
          scol[k] = gse;
        }
      }
    }
    const LdsTab rows{row_a_s, row_se_s, (int)(r0 - rs)};
    process_block<T, ROWW, COLW>(w, st, g, par, rows, ColRegs{acol, scol}, p.F_inv);
  }
}

template <typename T, bool ROWW, bool COLW>
static int interior_grid() {
  // resident interior workgroups on the device (a multiple of 8), per device
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cache[dev] == 0) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void*>(cast_interior_kernel<T, ROWW, COLW>), 256, 0) !=
            hipSuccess ||
        per_cu < 1)
      per_cu = 1;
    cache[dev] = std::max(T6_XCDS, (num_cus() * per_cu) / T6_XCDS * T6_XCDS);
  }
  return cache[dev];
}

template <typename T, bool ROWW, bool COLW>
static void launch_cast_kernels(CastK k, const CastArgs& a, hipStream_t s) {
  const dim3 block(256);
  const int64_t ntiles = k.n_istrips * k.n_isteps;
  if (ntiles > 0) {
    const int64_t G = interior_grid<T, ROWW, COLW>();
    hipLaunchKernelGGL((cast_interior_kernel<T, ROWW, COLW>), dim3((unsigned)G), dim3(256), 0, s,
                       k);
  }
  // edge rectangles: (1) the partial last strip over all rows,
  // (2) the rows below the interior for the full strips
  auto edge = [&](int64_t rstart, int64_t rend, int64_t strip0, int64_t nstrips) {
    if (rend <= rstart || nstrips <= 0) return;
    const int64_t rows = rend - rstart;
    const int64_t target = (int64_t)num_cus() * 8;
    int64_t segs = std::max<int64_t>(1, (target + nstrips - 1) / nstrips);
    const int64_t steps = (rows + CAST_STEP_ROWS - 1) / CAST_STEP_ROWS;
    segs = std::min(segs, steps);
    const int64_t steps_per_wg =
        std::min<int64_t>((steps + segs - 1) / segs, CAST_MAX_ROWS_PER_WG / CAST_STEP_ROWS);
    k.rows_per_wg = steps_per_wg * CAST_STEP_ROWS;
    segs = (rows + k.rows_per_wg - 1) / k.rows_per_wg;
    k.rstart = rstart;
    k.rend = rend;
    k.seg0 = 0;
    k.strip0 = strip0;
    k.nstrips = nstrips;
    hipLaunchKernelGGL((cast_edge_kernel<T, ROWW, COLW>), dim3((unsigned)(segs * nstrips)), block,
                       0, s, k);
  };
  const int64_t strips = (a.K + CAST_STRIP_COLS - 1) / CAST_STRIP_COLS;
  edge(0, a.M, k.n_istrips, strips - k.n_istrips);
  edge(k.n_isteps * T6_ROWS, a.M, 0, k.n_istrips);
}

template <typename T>
static int launch_cast_t(const CastArgs& a, hipStream_t s) {
  CastK k;
  k.x = a.x;
  k.M = a.M;
  k.K = a.K;
  k.row_mode = a.row_mode;
  k.row_amax = a.row_amax;
  k.col_mode = a.col_mode;
  k.col_amax = a.col_amax;
  k.F = a.F;
  k.F_inv = a.F_inv;
  k.q_row = a.q_row;
  k.s_row = a.s_row;
  k.q_col = a.q_col;
  k.s_col = a.s_col;
  k.noop = a.noop;
  constexpr int V = 16 / sizeof(T);
  k.vec_load = ((a.K % V) == 0) && ((reinterpret_cast<uintptr_t>(a.x) & 15) == 0);
  k.row_store4 = (a.K % 8 == 0) && ((reinterpret_cast<uintptr_t>(a.q_row) & 3) == 0);
  k.col_store8 = (a.M % 16 == 0) && ((reinterpret_cast<uintptr_t>(a.q_col) & 7) == 0);
  // Interior (persistent, super-step scheduled) path: 16-byte aligned rows
  // and outputs aligned for their 16- and 4-byte stores (K % 256 == 0 for the
  // rowwise scales, M % 64 == 0 for the transposed copy), and every in-tile
  // offset within 31 bits.
  const int64_t lim = 0x7FFFFFFF;
  const bool fast = k.vec_load && (a.K % 256 == 0) && (a.M % T6_ROWS == 0) &&
                    (!a.q_row || (reinterpret_cast<uintptr_t>(a.q_row) & 15) == 0) &&
                    (!a.s_row || (reinterpret_cast<uintptr_t>(a.s_row) & 15) == 0) &&
                    (!a.q_col || (reinterpret_cast<uintptr_t>(a.q_col) & 15) == 0) &&
                    (!a.s_col || (reinterpret_cast<uintptr_t>(a.s_col) & 7) == 0) &&
                    (int64_t)16 * a.K * (int64_t)sizeof(T) < lim;
  k.n_istrips = fast ? a.K / T6_COLS : 0;
  k.n_isteps = fast ? a.M / T6_ROWS : 0;
  if (k.n_istrips == 0 || k.n_isteps == 0) k.n_istrips = k.n_isteps = 0;
  const bool rw = a.q_row != nullptr, cw = a.q_col != nullptr;
  if (rw && cw) launch_cast_kernels<T, true, true>(k, a, s);
  else if (rw) launch_cast_kernels<T, true, false>(k, a, s);
  else launch_cast_kernels<T, false, true>(k, a, s);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

int launch_cast(const CastArgs& a, hipStream_t s) {
  return a.in_dtype == 0 ? launch_cast_t<uint16_t>(a, s) : launch_cast_t<float>(a, s);
}

}  // namespace nvfp4

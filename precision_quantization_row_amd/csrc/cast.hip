// cast.hip -- the quantize-transpose pass of row-scaled NVFP4 (gfx950).
//
// One read of X produces both copies (TransformerEngine row-scaled backward
// PR summary: the columnwise / transposed output is emitted in the same kernel
// pass as the rowwise one, each direction with its own second-level amax).
//
// Geometry. A lane always works on a 16 x 8 register block of X (16 rows, 8
// consecutive columns), which gives both directions without moving data:
//   rowwise   -- a 16-element row block spans the lane pair (l, l^1); their
//                8-element maxima meet through one DPP swap. The pair splits
//                the 16 block-scale computations (even lane: even rows, odd
//                lane: odd rows) and DPP broadcasts hand each row's encode
//                factor to both lanes.
//   columnwise-- each of the lane's 8 columns has all 16 rows of a column
//                block in the lane itself: the block max is a register
//                reduction (packed u16 max for BF16), no data exchange.
// Loads are whole row segments (16 bytes per lane, consecutive lanes on
// consecutive columns), so X is never read column-strided.
//
// Two kernels share that block code. The interior kernel (persistent,
// 256 x 256 macro tiles, buffer addressing with scalar row offsets, outputs
// staged so that whole lines leave the workgroup) takes every tile of an
// aligned shape; the edge kernel takes the rest with per-element bounds
// checks.
#include "nvfp4_device.h"
#include "nvfp4_launch.h"

#include <algorithm>
#include <atomic>

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
  // interior kernel: macro tiles of 256 rows x 256 columns, n_istrips strips
  // by n_isteps macro rows; if half_last, the last macro row is 128 rows (its
  // first sub-step only)
  int64_t n_istrips, n_isteps, half_last;
  // strips an XCD's workgroups take side by side (tile order within the XCD)
  int64_t sgroup;
  // edge kernel: rows [rstart, rend) in segments of rows_per_wg (a multiple of
  // CAST_STEP_ROWS, <= CAST_MAX_ROWS_PER_WG); workgroup b takes segment
  // seg0 + b / nstrips of strip strip0 + b % nstrips
  int64_t rstart, rend, rows_per_wg;
  int64_t seg0, strip0, nstrips;
  // grouped tokens (grp_G > 0): x holds grp_T token rows; output row r reads
  // token row token_row(r) of x, or is a zero row (padding, past the groups)
  const int64_t* grp_rows;
  int64_t grp_G, grp_align, grp_T;
  // 2-D blocks: one scale per 16 x 16 tile, per-tensor amax row_amax[0]
  int blk2d;
  // four-over-six block scales (1x16 blocks; the checked kernel only)
  int four_six;
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
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xA0, 0xF, 0xF, true));
}
__device__ __forceinline__ float bcast_odd(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xF5, 0xF, 0xF, true));
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

// X is read once by this pass: non-temporal loads keep it from displacing the
// partially written scale lines that are still merging in L2.
template <typename T>
__device__ __forceinline__ void load_row_buf(__amdgpu_buffer_rsrc_t rx, uint32_t vo, uint32_t so,
                                             uint32_t (&out)[Blk<T>::NW]) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)vo, (int)so, 2 /* nt */);
  out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
  if constexpr (sizeof(T) == 4) {
    const u32x4 u = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)(vo + 16u), (int)so, 2 /* nt */);
    out[4] = u.x; out[5] = u.y; out[6] = u.z; out[7] = u.w;
  }
}

// ------------------------------------------------------------------ stores
// Eight bytes to any address as naturally aligned pieces (one 8-byte store
// when the address allows, else 2-4 stores of 4, 2 and 1 bytes). A lane's
// columns c + k have c % 8 == 0, so for one k the address alignment is the
// same on every lane and the branch is uniform.
__device__ __forceinline__ void store8_pieces(uint8_t* dst, uint32_t w0, uint32_t w1) {
  const uint64_t v = (uint64_t)w0 | ((uint64_t)w1 << 32);
  switch (reinterpret_cast<uintptr_t>(dst) & 7) {
    case 0:
      *reinterpret_cast<uint2*>(dst) = make_uint2(w0, w1);
      break;
    case 4:
      reinterpret_cast<uint32_t*>(dst)[0] = w0;
      reinterpret_cast<uint32_t*>(dst)[1] = w1;
      break;
    case 2:
    case 6:
      *reinterpret_cast<uint16_t*>(dst) = (uint16_t)v;
      *reinterpret_cast<uint32_t*>(dst + 2) = (uint32_t)(v >> 16);
      *reinterpret_cast<uint16_t*>(dst + 6) = (uint16_t)(v >> 48);
      break;
    case 1:
    case 5:
      dst[0] = (uint8_t)v;
      *reinterpret_cast<uint16_t*>(dst + 1) = (uint16_t)(v >> 8);
      *reinterpret_cast<uint32_t*>(dst + 3) = (uint32_t)(v >> 24);
      dst[7] = (uint8_t)(v >> 56);
      break;
    default:  // 3, 7
      dst[0] = (uint8_t)v;
      *reinterpret_cast<uint32_t*>(dst + 1) = (uint32_t)(v >> 8);
      *reinterpret_cast<uint16_t*>(dst + 5) = (uint16_t)(v >> 40);
      dst[7] = (uint8_t)(v >> 56);
      break;
  }
}

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
    } else if (rb0 + 16 <= re) {
      store8_pieces(dst, w0, w1);
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
struct NoMid {
  __device__ __forceinline__ void operator()() const {}
};

template <typename T, bool ROWW, bool COLW, class Store, class RowTab, class ColTab,
          class Mid = NoMid>
__device__ __forceinline__ void process_block(const uint32_t (&w)[16][Blk<T>::NW],
                                              const Store& st, int g, int par, const RowTab& row,
                                              const ColTab& col, float f_inv,
                                              const Mid& mid = Mid()) {
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

  mid();  // between the phases: the rows are no longer needed one by one

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

// ------------------------------------------------------- four-over-six
// Four-over-six block scaling (the torchao four-over-six PR descriptions name
// the quantizer, its MSE choice and its bound-256 second-level scale). Each
// block has two candidate scales, the block max mapped to the E2M1 maximum 6
// or to 4; both go through the same byte / D / encode steps, both candidates
// are dequantized as the decoder does it (y = RN(e2m1(code) * D)), and the one
// with the smaller squared error is kept, the max-6 one on a tie. The error is
// summed in binary64 in a fixed order -- elements 0..7 in order, elements
// 8..15 in order, then the two sums added -- so every lane that takes a
// block's decision takes the same one. Blocks cut at the matrix edge read
// zeros past it, whose squared error is exactly zero.
struct Cand {
  uint32_t byte;
  float enc, dec;
};

// One candidate: s32 = RN(RN(bamax / top) * S_enc), then the guarded chain
// (IEEE divisions, no range conditions).
__device__ __forceinline__ Cand cand_scale(float bamax, float top, float a, float s_enc,
                                           float f_inv) {
  const float s32 = fminf((bamax / top) * s_enc, kE4M3Max);
  const int pk = __builtin_amdgcn_cvt_pk_fp8_f32(s32, s32, 0, false);
  Cand c;
  c.byte = (uint32_t)pk & 0xFFu;
  const float sq = __builtin_amdgcn_cvt_f32_fp8(pk, 0);
  c.dec = (sq * a) * f_inv;
  c.enc = (c.dec == 0.0f) ? 0.0f : fminf(1.0f / c.dec, kFltMax);
  return c;
}

// Sum over 8 elements, in order, of (x_k - RN(e2m1(code_k) * d))^2 in
// binary64; code k is nibble k of word (decoded exactly by fp4x2_decode).
__device__ __forceinline__ double sq_error8(const float (&x)[8], uint32_t word, float d) {
  float v[8];
  const f32x2 p0 = fp4x2_decode<0>(word), p1 = fp4x2_decode<1>(word);
  const f32x2 p2 = fp4x2_decode<2>(word), p3 = fp4x2_decode<3>(word);
  v[0] = p0[0]; v[1] = p0[1]; v[2] = p1[0]; v[3] = p1[1];
  v[4] = p2[0]; v[5] = p2[1]; v[6] = p3[0]; v[7] = p3[1];
  double s = 0.0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const double e = (double)x[k] - (double)(v[k] * d);
    s = s + e * e;
  }
  return s;
}

__device__ __forceinline__ double dpp_swap1_f64(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = dpp_swap1((uint32_t)b), hi = dpp_swap1((uint32_t)(b >> 32));
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Both directions of one 64-row step with four-over-six block scales (the
// checked kernel's lane layout: lane pair (l, l ^ 1) holds a row block, the
// even lane its elements 0..7).
template <typename T, bool ROWW, bool COLW, class Store, class RowTab, class ColTab>
__device__ __forceinline__ void process_block_46(const uint32_t (&w)[16][Blk<T>::NW],
                                                 const Store& st, int g, int par,
                                                 const RowTab& row, const ColTab& col,
                                                 float f_inv) {
  uint32_t cm[8];  // magnitude bits of the lane's column maxima
#pragma unroll
  for (int k = 0; k < 8; ++k) cm[k] = 0u;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t h[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int i = 2 * j + e;
      uint32_t m = 0u;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const uint32_t av = __float_as_uint(elem<T>(w, i, k)) & kAbsF32;
        if constexpr (COLW) cm[k] = max(cm[k], av);
        m = max(m, av);
      }
      h[e] = m;
    }
    if constexpr (ROWW) {
      const uint32_t b0 = max(h[0], dpp_swap1(h[0]));
      const uint32_t b1 = max(h[1], dpp_swap1(h[1]));
      const int lr = 16 * g + 2 * j + par;
      const float a = row.a(lr), se = row.s(lr);
      const float bm = __uint_as_float(par ? b1 : b0);
      const Cand c6 = cand_scale(bm, kE2M1Max, a, se, f_inv);
      const Cand c4 = cand_scale(bm, 4.0f, a, se, f_inv);
      bool four[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        // the candidates of row 2j + e, from the lane that owns it
        const float e6 = e ? bcast_odd(c6.enc) : bcast_even(c6.enc);
        const float d6 = e ? bcast_odd(c6.dec) : bcast_even(c6.dec);
        const float e4 = e ? bcast_odd(c4.enc) : bcast_even(c4.enc);
        const float d4 = e ? bcast_odd(c4.dec) : bcast_even(c4.dec);
        float x[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) x[k] = elem<T>(w, 2 * j + e, k);
        const uint32_t w6 = e2m1_pack8(x[0] * e6, x[1] * e6, x[2] * e6, x[3] * e6, x[4] * e6,
                                       x[5] * e6, x[6] * e6, x[7] * e6);
        const uint32_t w4 = e2m1_pack8(x[0] * e4, x[1] * e4, x[2] * e4, x[3] * e4, x[4] * e4,
                                       x[5] * e4, x[6] * e4, x[7] * e4);
        const double p6 = sq_error8(x, w6, d6), p4 = sq_error8(x, w4, d4);
        const double q6 = dpp_swap1_f64(p6), q4 = dpp_swap1_f64(p4);
        const double s6 = par ? q6 + p6 : p6 + q6;  // elements 0..7 first
        const double s4 = par ? q4 + p4 : p4 + q4;
        four[e] = s4 < s6;
        st.row_codes(2 * j + e, four[e] ? w4 : w6);
      }
      st.row_scale(j, four[par] ? c4.byte : c6.byte);
    }
  }
  if constexpr (COLW) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t cb = cm[k];
      const Cand c6 = cand_scale(__uint_as_float(cb), kE2M1Max, col.a(k), col.s(k), f_inv);
      const Cand c4 = cand_scale(__uint_as_float(cb), 4.0f, col.a(k), col.s(k), f_inv);
      float lo[8], hi[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        lo[i] = elem<T>(w, i, k);
        hi[i] = elem<T>(w, 8 + i, k);
      }
      auto pack = [](const float (&v)[8], float f) {
        return e2m1_pack8(v[0] * f, v[1] * f, v[2] * f, v[3] * f, v[4] * f, v[5] * f, v[6] * f,
                          v[7] * f);
      };
      const uint32_t a6 = pack(lo, c6.enc), b6 = pack(hi, c6.enc);
      const uint32_t a4 = pack(lo, c4.enc), b4 = pack(hi, c4.enc);
      const double s6 = sq_error8(lo, a6, c6.dec) + sq_error8(hi, b6, c6.dec);
      const double s4 = sq_error8(lo, a4, c4.dec) + sq_error8(hi, b4, c4.dec);
      const bool four = s4 < s6;
      st.col(k, four ? a4 : a6, four ? b4 : b6, four ? c4.byte : c6.byte);
    }
  }
}

// Two E2M1 codes into byte `sel` (a constant after unrolling) of `old`.
__device__ __forceinline__ uint32_t cvt_fp4x2_sel(uint32_t old, float v0, float v1, int sel) {
  switch (sel & 3) {
    case 0: return NVFP4_CVT_FP4X2(old, v0, v1, 0);
    case 1: return NVFP4_CVT_FP4X2(old, v0, v1, 1);
    case 2: return NVFP4_CVT_FP4X2(old, v0, v1, 2);
    default: return NVFP4_CVT_FP4X2(old, v0, v1, 3);
  }
}

// Packed maximum of three dwords of two 16-bit magnitude patterns each. With
// F16, one v_pk_maximum3_f16 (the patterns compared as f16 numbers: the same
// order as integers for patterns below 0x7C00, an f16 infinity or NaN above);
// otherwise two integer v_pk_max_u16.
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
template <bool F16>
__device__ __forceinline__ uint32_t pk_max3_mag(uint32_t a, uint32_t b, uint32_t c) {
  if constexpr (F16) {
    const f16x2 x = __builtin_bit_cast(f16x2, a), y = __builtin_bit_cast(f16x2, b),
                z = __builtin_bit_cast(f16x2, c);
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_maximum(
                                            __builtin_elementwise_maximum(x, y), z));
  } else {
    return pk_max_u16(pk_max_u16(a, b), c);
  }
}

// Block maxima of a BF16 16 x 8 lane block: cm[d] = packed maxima over the 16
// rows of the lane's columns 2d, 2d + 1; rb[i] = packed maxima of row i over
// its even and its odd columns. F16 selects the three-input compare above.
template <bool F16, bool ROWW, bool COLW>
__device__ __forceinline__ void maxima_bf16(const uint32_t (&w)[16][4], uint32_t (&cm)[4],
                                            uint32_t (&rb)[16]) {
#pragma unroll
  for (int d = 0; d < 4; ++d) cm[d] = 0u;
#pragma unroll
  for (int i = 0; i < 16; i += 2) {
    uint32_t a[4], b[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      a[d] = w[i][d] & kAbsBf16x2;
      b[d] = w[i + 1][d] & kAbsBf16x2;
    }
    if constexpr (COLW) {
#pragma unroll
      for (int d = 0; d < 4; ++d) cm[d] = pk_max3_mag<F16>(cm[d], a[d], b[d]);
    }
    if constexpr (ROWW) {
      rb[i] = pk_max_u16(pk_max3_mag<F16>(a[0], a[1], a[2]), a[3]);
      rb[i + 1] = pk_max_u16(pk_max3_mag<F16>(b[0], b[1], b[2]), b[3]);
    }
  }
}

// The same two directions as process_block, in three batched phases, so that
// independent work sits side by side for the scheduler:
//   1. every block maximum of the 16 x 8 block (integer max on magnitudes);
//   2. all 16 block scales (8 row blocks shared with the lane pair, 8 column
//      blocks) -- 16 independent dependency chains;
//   3. every element converted to fp32 once, multiplied by its row and its
//      column encode factor, both products converted to E2M1.
// `mid` runs after phase 1 (the next tile's loads can be issued there).
template <typename T, bool ROWW, bool COLW, class Store, class RowTab, class ColTab, class Mid>
__device__ __forceinline__ void process_block_batched(const uint32_t (&w)[16][Blk<T>::NW],
                                                      const Store& st, int g, int par,
                                                      const RowTab& row, const ColTab& col,
                                                      float f_inv, const Mid& mid) {
  constexpr int NW = Blk<T>::NW;
  // ---- phase 1: maxima. BF16: cm[d] holds the packed column maxima of
  // dword d, rb[i] the packed maxima of row i's even and odd columns (folded
  // after the exchange with the lane pair). FP32: plain magnitude bits.
  uint32_t cm[NW];
  uint32_t rb[16];
  if constexpr (sizeof(T) == 2) {
    maxima_bf16<true, ROWW, COLW>(w, cm, rb);
    // The fast form compares BF16 magnitudes as f16 numbers, which orders
    // them like integers unless a pattern reads as an f16 infinity or NaN
    // (magnitudes >= 2^121). The column maxima cover every element (the row
    // maxima do when there is no column direction); if any of them reached
    // that range the lane redoes the maxima with integer compares.
    uint32_t m = 0u;
    if constexpr (COLW) {
      m = pk_max_u16(pk_max_u16(cm[0], cm[1]), pk_max_u16(cm[2], cm[3]));
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) m = pk_max_u16(m, rb[i]);
    }
    if (max(m & 0xFFFFu, m >> 16) >= 0x7C00u) maxima_bf16<false, ROWW, COLW>(w, cm, rb);
  } else {
#pragma unroll
    for (int d = 0; d < NW; ++d) cm[d] = 0u;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      uint32_t m = 0u;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const uint32_t av = w[i][k] & kAbsF32;
        if constexpr (COLW) cm[k] = max(cm[k], av);
        m = max(m, av);
      }
      rb[i] = m;
    }
  }
  mid();

  // ---- phase 2: scales. The lane's line amaxes and S_enc values are read
  // from their tables first, all 16 chains take the unguarded form, and one
  // range check over all of them (smallest block max, smallest and largest
  // D) decides; a lane outside either range (tiny blocks, extreme decode
  // scales) redoes all of its scales with the guarded form and stages its
  // scale bytes again.
  float renc[8];  // encode factor of this lane's row 2j + par
  float cenc[8];
  uint32_t bsel[8];
  float ta[8], ts[8], tca[8], tcs[8];
  if constexpr (ROWW) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      ta[j] = row.a(16 * g + 2 * j + par);
      ts[j] = row.s(16 * g + 2 * j + par);
    }
  }
  if constexpr (COLW) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      tca[k] = col.a(k);
      tcs[k] = col.s(k);
    }
  }
  auto col_bits = [&](int k) -> uint32_t {
    if constexpr (sizeof(T) == 2)
      return (k & 1) ? (cm[k >> 1] & 0xFFFF0000u) : (cm[k >> 1] << 16);
    else
      return cm[k];
  };
  uint32_t bmin = 0xFFFFFFFFu, dmin = 0xFFFFFFFFu, dmax = 0u, dsig = 0u;
  if constexpr (ROWW) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      // the lane sends its partner the maximum of the partner's row and takes
      // the partner's maximum of its own row: one swap per row pair
      const uint32_t mine = par ? rb[2 * j + 1] : rb[2 * j];
      const uint32_t other = par ? rb[2 * j] : rb[2 * j + 1];
      if constexpr (sizeof(T) == 2) {
        const uint32_t u = pk_max_u16(mine, dpp_swap1(other));
        bsel[j] = max(u & 0xFFFFu, u >> 16) << 16;
      } else {
        bsel[j] = max(mine, dpp_swap1(other));
      }
      uint32_t byte;
      const uint32_t db =
          block_scale_unchecked(__uint_as_float(bsel[j]), ta[j], ts[j], f_inv, &byte, &renc[j]);
      st.row_scale(j, byte);
      bmin = min(bmin, bsel[j]);
      dmin = min(dmin, db);
      dmax = max(dmax, db);
      dsig = max(dsig, db & kSigMask);
    }
  }
  if constexpr (COLW) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      uint32_t byte;
      const uint32_t db = block_scale_unchecked(__uint_as_float(col_bits(k)), tca[k], tcs[k], f_inv,
                                                &byte, &cenc[k]);
      st.col_scale(k, byte);
      bmin = min(bmin, col_bits(k));
      dmin = min(dmin, db);
      dmax = max(dmax, db);
      dsig = max(dsig, db & kSigMask);
    }
  }
  // the fast forms hold for bamax >= 2^-121 and D in [2^-126, 2^126) whose
  // significand is not all ones (recip_fast_ok for every block)
  const bool ok = (bmin >= kFastBamaxMin) & (dmin >= 0x00800000u) & (dmax < 0x7E800000u) &
                  (dsig != kSigMask);
  if (!ok) {
    // The block maxima pass through an empty asm statement so that the
    // compiler cannot share work between the two forms: sharing would keep
    // the fast form's intermediates alive past their last fast use.
    if constexpr (ROWW) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint32_t byte, bm = bsel[j];
        asm volatile("" : "+v"(bm));
        block_scale(__uint_as_float(bm), ta[j], ts[j], f_inv, &byte, &renc[j]);
        st.row_scale(j, byte);
      }
    }
    if constexpr (COLW) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        uint32_t byte, bm = col_bits(k);
        asm volatile("" : "+v"(bm));
        block_scale(__uint_as_float(bm), tca[k], tcs[k], f_inv, &byte, &cenc[k]);
        st.col_scale(k, byte);
      }
    }
  }

  // ---- phase 3: codes. Byte j & 3 of cc[k][j >> 2] holds rows 2j, 2j+1 of
  // column k; byte 0 starts from the first product's own bits (the other bytes
  // are written later), so the accumulators need no zeroing.
  uint32_t cc[8][2];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float xv[2][8];
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int k = 0; k < 8; ++k) xv[e][k] = elem<T>(w, 2 * j + e, k);
    if constexpr (ROWW) {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float r = e ? bcast_odd(renc[j]) : bcast_even(renc[j]);
        st.row_codes(2 * j + e, e2m1_pack8(xv[e][0] * r, xv[e][1] * r, xv[e][2] * r, xv[e][3] * r,
                                           xv[e][4] * r, xv[e][5] * r, xv[e][6] * r, xv[e][7] * r));
      }
    }
    if constexpr (COLW) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float p0 = xv[0][k] * cenc[k], p1 = xv[1][k] * cenc[k];
        cc[k][j >> 2] = cvt_fp4x2_sel((j & 3) ? cc[k][j >> 2] : __float_as_uint(p0), p0, p1, j);
      }
    }
  }
  if constexpr (COLW) {
#pragma unroll
    for (int k = 0; k < 8; ++k) st.col_codes(k, cc[k][0], cc[k][1]);
  }
}

// 2-D blocks: the lane pair (l, l ^ 1) holds one 16 x 16 tile (16 rows, 8
// columns each). The tile's max magnitude gives one scale (per-tensor amax a,
// S_enc s_enc) for all its 16 rows and 16 columns, so every element is
// multiplied once and both copies encode the same products: the rowwise codes
// pair neighbouring columns, the transposed codes neighbouring rows.
template <typename T, bool ROWW, bool COLW, class Store, class Mid>
__device__ __forceinline__ void process_block_2d(const uint32_t (&w)[16][Blk<T>::NW],
                                                 const Store& st, float a, float s_enc,
                                                 float f_inv, const Mid& mid) {
  constexpr int NW = Blk<T>::NW;
  uint32_t m = 0u;
  if constexpr (sizeof(T) == 2) {
    uint32_t cm[NW];
#pragma unroll
    for (int d = 0; d < NW; ++d) cm[d] = 0u;
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
      for (int d = 0; d < NW; ++d) cm[d] = pk_max_u16(cm[d], w[i][d] & kAbsBf16x2);
    const uint32_t t = pk_max_u16(pk_max_u16(cm[0], cm[1]), pk_max_u16(cm[2], cm[3]));
    m = max(t & 0xFFFFu, t >> 16) << 16;
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
      for (int k = 0; k < NW; ++k) m = max(m, w[i][k] & kAbsF32);
  }
  m = max(m, dpp_swap1(m));
  mid();
  uint32_t byte;
  float enc;
  if (!block_scale_fast(__uint_as_float(m), a, s_enc, f_inv, &byte, &enc))
    block_scale(__uint_as_float(m), a, s_enc, f_inv, &byte, &enc);
  if constexpr (ROWW) {
#pragma unroll
    for (int j = 0; j < 8; ++j) st.row_scale(j, byte);
  }
  uint32_t cc[8][2];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float pv[2][8];
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int k = 0; k < 8; ++k) pv[e][k] = elem<T>(w, 2 * j + e, k) * enc;
    if constexpr (ROWW) {
#pragma unroll
      for (int e = 0; e < 2; ++e)
        st.row_codes(2 * j + e, e2m1_pack8(pv[e][0], pv[e][1], pv[e][2], pv[e][3], pv[e][4],
                                           pv[e][5], pv[e][6], pv[e][7]));
    }
    if constexpr (COLW) {
#pragma unroll
      for (int k = 0; k < 8; ++k)
        cc[k][j >> 2] = cvt_fp4x2_sel((j & 3) ? cc[k][j >> 2] : __float_as_uint(pv[0][k]), pv[0][k],
                                      pv[1][k], j);
    }
  }
  if constexpr (COLW) {
#pragma unroll
    for (int k = 0; k < 8; ++k) st.col(k, cc[k][0], cc[k][1], byte);
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
// The lane's 8 columns, read from LDS (8 consecutive entries).
struct ColLds {
  const float* pa;
  const float* ps;
  __device__ __forceinline__ float a(int k) const { return pa[k]; }
  __device__ __forceinline__ float s(int k) const { return ps[k]; }
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
// Interior macro tiles are 256 rows x 256 columns, walked in two sub-steps of
// 128 rows. A workgroup is 4 waves; in a sub-step wave w holds rows
// rs + 32w .. +32 and lane (h = lane / 32, L = lane % 32) the 16 x 8 register
// block at rows rs + 32w + 16h .. +16, columns c0 + 8L .. +8. A load
// instruction reads 512 contiguous bytes of two rows (BF16).
//
// Why 256 x 256. On this GPU a store stream costs close to plain streaming
// only when whole 128-byte lines leave the workgroup at once; partial lines
// merge in the caches and their late write-back also slows whatever kernel
// runs next. With 256 columns a rowwise-code row segment is 128 bytes, and
// with 256 rows a transposed-code column segment is 128 bytes. Both are
// written with non-temporal stores: rowwise codes straight from registers
// (32 lanes x 4 bytes per row), transposed codes from LDS once the macro
// tile is complete (8 lanes per column). The scales (16 bytes per row and per
// column of the tile) take ordinary stores.
//
// Schedule. Workgroup b runs on XCD x = b % 8 as its j = b / 8-th of
// P = grid / 8 workgroups there. XCD x owns the S = ceil(strips / 8)
// consecutive strips x S .. x S + S - 1, taken in groups of G strips (the last
// group may hold fewer); a group's tiles are listed macro row by macro row,
// its strips side by side. The workgroup's u-th macro tile is number
// t = u P + j of the XCD's list, so the P workgroups of one round cover a block
// of G strips by P / G macro rows: rows and columns both leave their codes in
// runs of several 128-byte lines, and a row's rowwise scales (16 bytes per
// strip) and a column's transposed scales (16 bytes per macro tile) are
// written by one XCD, whose L2 merges them into lines.
constexpr int IT_COLS = 256;                 // strip width
constexpr int IT_SUB = 128;                  // rows per sub-step
constexpr int IT_MACRO = 2 * IT_SUB;         // rows per macro tile
constexpr int IT_XCDS = 8;

// Without the columnwise copy the transposed staging shrinks to a stub (the
// code that touches it is never reached), so rowwise-only launches fit more
// workgroups per CU.
template <bool COLW>
struct ITSmem {
  static constexpr int QCOLS = COLW ? IT_COLS : 1;
  // transposed codes of the macro tile, [buf][storage column][16 slots x 8 B].
  // Slot s holds rows 16s .. +16 of the column. Column c is stored at
  // c ^ ((c >> 3) & 1) and slot s at position s ^ ((c >> 3) & 15), so the 64
  // lanes of one store instruction spread over all 64 banks.
  uint8_t qc[2][QCOLS][128];
  // transposed scales, [buf][entry][16 blocks]; column 8L + k at entry 32k + L
  uint8_t sc[2][QCOLS][16];
  // rowwise scales of a sub-step, [buf][row][16 blocks]
  uint8_t sr[2][IT_SUB][16];
  // per-wave row amax / S_enc of the wave's 32 rows
  float ra[4][32], rs[4][32];
  // column amax / S_enc of the strip's 256 columns (modes 0 and 1); grouped
  // tokens use mode 2 and keep their group table here instead: gtok[g] and
  // gpad[g] are the ends of group g in token rows and in padded rows
  union { float ca[IT_COLS]; uint32_t gtok[IT_COLS]; };
  union { float cs[IT_COLS]; uint32_t gpad[IT_COLS]; };
  // row-group mode: the group amax / S_enc of each wave half's 16-row block,
  // repeated for the lane's 8 columns
  float ga[4][2][8], gs[4][2][8];
};

struct StoreIT {
  __amdgpu_buffer_rsrc_t qr;  // rowwise codes of the wave's 32 rows
  uint32_t vo_qr, qrs;
  uint8_t* sr;
  uint8_t* qc;
  uint8_t* sc;
  int wv, h, L, par, slot;
  __device__ __forceinline__ void row_codes(int i, uint32_t word) const {
    __builtin_amdgcn_raw_buffer_store_b32(word, qr, (int)vo_qr, (int)(i * qrs), 2 /* nt */);
  }
  __device__ __forceinline__ void row_scale(int j, uint32_t byte) const {
    sr[(32 * wv + 16 * h + 2 * j + par) * 16 + (L >> 1)] = (uint8_t)byte;
  }
  __device__ __forceinline__ void col_codes(int k, uint32_t w0, uint32_t w1) const {
    const int c = 8 * L + k;
    const int pos = slot ^ (L & 15);
    *reinterpret_cast<uint2*>(qc + (c ^ (L & 1)) * 128 + 8 * pos) = make_uint2(w0, w1);
  }
  // column 8L + k is stored at entry 32k + L, so the lanes of one write land
  // in different banks
  __device__ __forceinline__ void col_scale(int k, uint32_t byte) const {
    sc[(32 * k + L) * 16 + slot] = (uint8_t)byte;
  }
  __device__ __forceinline__ void col(int k, uint32_t w0, uint32_t w1, uint32_t byte) const {
    col_codes(k, w0, w1);
    col_scale(k, byte);
  }
};

// Grouped tokens in the interior kernel. The group table is built once per
// workgroup in 32-bit form: inclusive prefix sums of the group sizes in token
// rows (gtok) and rounded up to the alignment in padded rows (gpad), both
// saturating at 2^31 - 1 (the host sends only T, M < 2^31 here, so a
// saturated end lies past every row the kernel touches); entries from G on
// hold 0xFFFFFFFF in gpad. All 256 threads.
template <class SM>
__device__ __forceinline__ void build_group_table32(SM& sm, const int64_t* rows, int G,
                                                    int64_t align) {
  constexpr uint32_t CL = 0x7FFFFFFFu;
  const int t = threadIdx.x;
  const int64_t n = t < G ? min(max(rows[t], (int64_t)0), (int64_t)CL) : 0;
  sm.gtok[t] = (uint32_t)n;
  sm.gpad[t] = (uint32_t)min((n + align - 1) / align * align, (int64_t)CL);
  __syncthreads();
  for (int off = 1; off < IT_COLS; off <<= 1) {
    uint32_t a = 0u, b = 0u;
    if (t >= off) {
      a = sm.gtok[t - off];
      b = sm.gpad[t - off];
    }
    __syncthreads();
    if (t >= off) {
      sm.gtok[t] = min(sm.gtok[t] + a, CL);
      sm.gpad[t] = min(sm.gpad[t] + b, CL);
    }
    __syncthreads();
  }
  if (t >= G) sm.gpad[t] = 0xFFFFFFFFu;
  __syncthreads();
}

// Where a wave's 32 padded rows pr0 .. pr0 + 31 come from (pr0 a multiple of
// 16; the alignment is one too, so each 16-row half lies in one group or past
// the last). Half h is n[h] consecutive token rows, then zero rows. The two
// halves lie within 32 token rows of `base`: half 0 at base, half 1 at
// base + d1 (0 <= d1 <= 16: when both halves hold tokens, half 0 is 16 rows of
// its group or that group's last rows, and the tokens of half 1 follow).
// lim = token rows from base that the buffer may read (at most 32, never past
// T). Every value is wave-uniform; all 64 lanes must be active.
struct WaveRows {
  int64_t base;
  uint32_t lim, d1, n0, n1;
};

template <class SM>
__device__ __forceinline__ WaveRows grouped_wave_rows(const SM& sm, int G, uint32_t T,
                                                      int lane, uint32_t pr0) {
  // group of a padded row = the number of groups that end at or before it
  const u32x4 e = *reinterpret_cast<const u32x4*>(&sm.gpad[4 * lane]);
  const uint32_t pr1 = pr0 + 16u;
  const uint32_t g0 = __builtin_popcountll(__builtin_amdgcn_ballot_w64(e.x <= pr0)) +
                      __builtin_popcountll(__builtin_amdgcn_ballot_w64(e.y <= pr0)) +
                      __builtin_popcountll(__builtin_amdgcn_ballot_w64(e.z <= pr0)) +
                      __builtin_popcountll(__builtin_amdgcn_ballot_w64(e.w <= pr0));
  const uint32_t g1 = __builtin_popcountll(__builtin_amdgcn_ballot_w64(e.x <= pr1)) +
                      __builtin_popcountll(__builtin_amdgcn_ballot_w64(e.y <= pr1)) +
                      __builtin_popcountll(__builtin_amdgcn_ballot_w64(e.z <= pr1)) +
                      __builtin_popcountll(__builtin_amdgcn_ballot_w64(e.w <= pr1));
  auto half = [&](uint32_t g, uint32_t pr, uint32_t& src, uint32_t& n) {
    src = 0u;
    n = 0u;
    if (g >= (uint32_t)G) return;  // past the last group: zero rows
    const uint32_t sp = g ? __builtin_amdgcn_readfirstlane(sm.gpad[g - 1]) : 0u;
    const uint32_t st = g ? __builtin_amdgcn_readfirstlane(sm.gtok[g - 1]) : 0u;
    const uint32_t et = __builtin_amdgcn_readfirstlane(sm.gtok[g]);
    src = st + (pr - sp);
    n = src < et ? min(et - src, 16u) : 0u;
    n = src < T ? min(n, T - src) : 0u;
  };
  uint32_t s0, n0, s1, n1;
  half(g0, pr0, s0, n0);
  half(g1, pr1, s1, n1);
  WaveRows w;
  w.base = n0 ? s0 : (n1 ? s1 : 0u);
  w.d1 = (n0 && n1) ? s1 - s0 : 0u;
  w.n0 = n0;
  w.n1 = n1;
  w.lim = (uint32_t)min((int64_t)32, max((int64_t)T - w.base, (int64_t)0));
  return w;
}

// The whole aligned dwords of bytes [lo, hi) of a 128-byte column segment,
// to the global address A of any alignment. This lane (t of the column's 8
// consecutive lanes) holds the segment's dwords S[4t .. 4t + 3] and prev =
// S[4t - 1] (from lane t - 1). Output dword m lies at E + 4m, E = A - A % 4,
// and holds segment bytes 4m - A % 4 .. +3, built from S[m - 1] and S[m] with
// a byte funnel shift; lane 7 also builds the dword past S[31]. Only dwords
// whose four bytes all lie in [lo, hi) are written here (an aligned, whole
// 16-byte piece as one non-temporal store, as in the aligned flush);
// store_segment_ends writes the at most 3 + 3 bytes at the two ends.
__device__ __forceinline__ void store_segment_dwords(uint8_t* A, const u32x4& q, uint32_t prev,
                                                     int t, int lo, int hi) {
  const uint32_t ra = (uint32_t)(reinterpret_cast<uintptr_t>(A) & 3);
  if (16 * t + 16 - (int)ra + (t == 7 ? 4 : 0) <= lo || 16 * t - (int)ra >= hi) return;
  if ((reinterpret_cast<uintptr_t>(A + 16 * t) & 15) == 0 && 16 * t >= lo && 16 * t + 16 <= hi) {
    __builtin_nontemporal_store(q, reinterpret_cast<u32x4*>(A + 16 * t));
    return;
  }
  uint8_t* E = A - ra;
  const uint32_t sv[5] = {prev, q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    if (i == 4 && t != 7) break;
    const int m = 4 * t + i;
    const int b0 = 4 * m - (int)ra;
    if (b0 >= lo && b0 + 4 <= hi) {
      const uint32_t cur = i < 4 ? sv[i + 1] : 0u;
      const uint32_t val = ra ? __builtin_amdgcn_alignbyte(cur, sv[i], 4u - ra) : cur;
      *reinterpret_cast<uint32_t*>(E + 4 * m) = val;
    }
  }
}

// The bytes of [lo, hi) that store_segment_dwords leaves: those before the
// first aligned address and from the last aligned address on (all of them
// when no whole aligned dword fits). seg(b) reads segment byte b.
template <class Seg>
__device__ __forceinline__ void store_segment_ends(uint8_t* A, int lo, int hi, const Seg& seg) {
  const int f = lo + (int)((4u - (uint32_t)(reinterpret_cast<uintptr_t>(A + lo) & 3)) & 3u);
  const int l = hi - (int)(reinterpret_cast<uintptr_t>(A + hi) & 3);
  if (f >= l) {
    for (int b = lo; b < hi; ++b) A[b] = seg(b);
  } else {
    for (int b = lo; b < f; ++b) A[b] = seg(b);
    for (int b = l; b < hi; ++b) A[b] = seg(b);
  }
}

// Bytes [lo, hi) (0 <= lo < hi <= 16) of 16 bytes in LDS to the global
// address dst + lo .. of any alignment: one 16-byte store when aligned and
// whole, four dwords when dword-aligned and whole, else byte by byte (on
// this GPU the plain byte stores ran faster than dwords built with funnel
// shifts, whose partial end dwords diverge).
__device__ __forceinline__ void store_bytes_any(uint8_t* dst, const uint8_t* src, int lo, int hi) {
  if (((reinterpret_cast<uintptr_t>(dst) & 15) == 0) && lo == 0 && hi == 16) {
    *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
    return;
  }
  if (((reinterpret_cast<uintptr_t>(dst) & 3) == 0) && lo == 0 && hi == 16) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(src);
    uint32_t* d = reinterpret_cast<uint32_t*>(dst);
    d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
    return;
  }
  for (int b = lo; b < hi; ++b) dst[b] = src[b];
}

// VAR: 0 = 1x16 blocks, 1 = grouped tokens (1x16), 2 = 2-D 16 x 16 blocks,
// 3 = four-over-six 1x16 blocks (one direction per launch).
// GEN (1x16 blocks only): any M and any K % 16 == 0 with 16-byte rows, in
// one launch. The last strip and the last macro row may be partial: a lane
// whose columns lie past K loads nothing (an offset past its buffer's range
// reads as zeros) and stores nothing, rows past M read as zeros and are not
// stored, the zero elements of a cut block change neither its maximum nor
// its codes, and only the output bytes of existing rows and columns are
// written. Output rows may have any alignment (odd M gives transposed rows of
// an odd number of bytes): the transposed flush builds aligned dwords with
// byte funnel shifts. Macro tiles are spread evenly over the XCDs (a
// contiguous run of the strip-major tile list each), so a matrix with few
// strips still uses every XCD.
template <typename T, bool ROWW, bool COLW, int VAR, bool SPLIT = false, bool GEN = false>
__global__ void __launch_bounds__(256, sizeof(T) == 2 ? 2 : 1) cast_interior_kernel(const CastK p) {
  static_assert(!GEN || VAR == 0, "general shapes take the 1x16 block code");
  if (p.noop != nullptr && *p.noop == 1.0f) return;
  constexpr bool GRP = VAR == 1, B2D = VAR == 2;
  constexpr int NW = Blk<T>::NW;
  __shared__ __attribute__((aligned(16))) ITSmem<COLW> sm;
  const T* __restrict__ x = static_cast<const T*>(p.x);
  const int tid = threadIdx.x;
  // The wave index is uniform across a wave; reading it into a scalar register
  // keeps every buffer descriptor derived from it scalar (no per-lane loop
  // around the buffer loads and stores).
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int h = lane >> 5, L = lane & 31, par = lane & 1;
  const int64_t K = p.K;

  const int64_t per = gridDim.x / IT_XCDS;
  const int64_t xcd = blockIdx.x % IT_XCDS, jw = blockIdx.x / IT_XCDS;
  const int64_t nstrips = p.n_istrips, nmr = p.n_isteps;  // strips, macro rows
  const int64_t spx = (nstrips + IT_XCDS - 1) / IT_XCDS;  // strips per XCD
  // GEN: this XCD's run [t_lo, t_lo + ntiles_x) of the strip-major tile list
  const int64_t t_all = nstrips * nmr;
  const int64_t t_lo = GEN ? xcd * t_all / IT_XCDS : 0;
  const int64_t ntiles_x = GEN ? (xcd + 1) * t_all / IT_XCDS - t_lo : nmr * spx;  // macro tiles per XCD
  const int64_t n_v = 2 * ((ntiles_x + per - 1) / per);  // sub-steps scheduled

  const uint32_t rowbytes = (uint32_t)(K * (int64_t)sizeof(T));
  const int64_t qrs = (K + 1) / 2, srs = (K + 15) / 16;
  const int64_t qcs = (p.M + 1) / 2, scs = (p.M + 15) / 16;
  // 2-D blocks: the per-tensor amax and its S_enc
  float a2d = 0.0f, s2d = 1.0f;
  if constexpr (B2D) {
    a2d = ROWW ? p.row_amax[0] : p.col_amax[0];
    s2d = global_encode_scale(a2d, p.F);
  }

  // The last round of macro tiles: when it holds at most half as many tiles
  // as the XCD has workgroups, its tiles are split into their two 128-row
  // halves, one per workgroup, each flushed on its own (64 B of transposed
  // codes and 8 scale bytes per column), so that twice as many workgroups
  // share the round.
  const int64_t rounds = (ntiles_x + per - 1) / per;
  const int64_t last_n = ntiles_x - (rounds - 1) * per;  // tiles in the last round
  // (compiled in only where the host expects it: the extra schedule logic
  // costs the plain variant registers)
  const bool split_last = SPLIT && rounds > 0 && 2 * last_n <= per;

  // sub-step v: macro tile origin (m0, c0), which 128-row half of it (sub)
  // and whether that half is flushed on its own (solo: a split half, or the
  // 128-row last macro row); false when outside the interior (uniform per
  // workgroup)
  // (32-bit index arithmetic: the host sends only grids whose tile counts fit)
  auto tile_of = [&](int64_t v, int64_t& m0, int64_t& c0, int& sub, bool& solo) -> bool {
    uint32_t t;
    if (split_last && (v >> 1) == rounds - 1) {
      if ((v & 1) || jw >= 2 * last_n) return false;
      t = (uint32_t)(rounds - 1) * (uint32_t)per + (uint32_t)(jw >> 1);
      sub = (int)(jw & 1);
      solo = true;
    } else {
      t = (uint32_t)(v >> 1) * (uint32_t)per + (uint32_t)jw;
      sub = (int)(v & 1);
      solo = false;
    }
    uint32_t r;
    int64_t strip;
    if constexpr (GEN) {
      // the XCD's run of the strip-major list: strip by strip, macro row by
      // macro row
      const uint32_t gi = (uint32_t)t_lo + t;
      strip = gi / (uint32_t)nmr;
      r = gi - (uint32_t)strip * (uint32_t)nmr;
    } else {
      // strip groups of sg strips (the XCD's last group may hold fewer), each
      // walked macro row by macro row with its strips side by side
      const uint32_t sg = (uint32_t)p.sgroup, gsz = sg * (uint32_t)nmr;
      const uint32_t g = t / gsz, rem = t - g * gsz;
      const uint32_t sgl = min(sg, (uint32_t)spx - min(g * sg, (uint32_t)spx));
      r = sgl ? rem / sgl : (uint32_t)nmr;
      const uint32_t qs = rem - r * sgl;
      strip = xcd * spx + g * sg + qs;
    }
    m0 = (int64_t)r * IT_MACRO;
    c0 = strip * IT_COLS;
    const bool last_half = p.half_last && r == (uint32_t)nmr - 1;  // a 128-row macro row
    solo = solo || last_half;
    return t < (uint64_t)ntiles_x && strip < nstrips && !(last_half && sub == 1);
  };
  auto next_sub = [&](int64_t v, int64_t& m0, int64_t& c0, int& sub, bool& solo) -> int64_t {
    while (v < n_v && !tile_of(v, m0, c0, sub, solo)) ++v;
    return v;
  };
  const uint32_t vo_lane = (uint32_t)h * 16u * rowbytes + (uint32_t)(8 * L * sizeof(T));
  // GEN: a lane whose 8 columns lie past K takes an offset beyond every
  // buffer range (reads zeros, stores nothing); K % 16 == 0, so a lane's
  // columns are all inside or all past
  auto lane_vo = [&](int64_t c0) -> uint32_t {
    if constexpr (GEN) return (c0 + 8 * L < K) ? vo_lane : 0x80000000u;
    else return vo_lane;
  };
  // rows of the wave that exist (GEN: the last macro row may be cut)
  auto wave_nr = [&](int64_t rs) -> int64_t {
    if constexpr (GEN) return min(max(p.M - (rs + 32 * wv), (int64_t)0), (int64_t)32);
    else return 32;
  };
  auto wave_rows = [&](int64_t rs, int64_t c0) {
    return make_rsrc(x + (rs + 32 * wv) * K + c0, wave_nr(rs) * K * (int64_t)sizeof(T));
  };
  // grouped tokens: the rows of a sub-step come through a WaveRows map; a
  // lane's row i past its half's n rows gets an offset beyond the buffer's
  // range, which reads as zero
  if constexpr (GRP) build_group_table32(sm, p.grp_rows, (int)p.grp_G, p.grp_align);
  const uint32_t grp_T = (uint32_t)p.grp_T;
  auto grp_map = [&](int64_t rs) { return grouped_wave_rows(sm, (int)p.grp_G, grp_T, lane, (uint32_t)(rs + 32 * wv)); };
  auto grp_rsrc = [&](const WaveRows& m, int64_t c0) {
    return make_rsrc(x + m.base * K + c0, (int64_t)m.lim * K * (int64_t)sizeof(T));
  };
  auto grp_vo = [&](const WaveRows& m) {
    return (h ? m.d1 * rowbytes : 0u) + (uint32_t)(8 * L * sizeof(T));
  };
  auto grp_load = [&](const __amdgpu_buffer_rsrc_t& r, uint32_t v, uint32_t n, int i,
                      uint32_t (&out)[NW]) {
    load_row_buf<T>(r, (uint32_t)i < n ? v : 0x80000000u, (uint32_t)i * rowbytes, out);
  };
  // The first PF rows of each half of the wave's next sub-step are loaded while
  // the current one's block scales and codes are computed (BF16: 32 registers;
  // FP32 has none to spare). Loading all 16 rows ahead needs 32 more registers
  // than the 1x16 code has at 2 waves per SIMD and ends up slower; the 2-D
  // code, which cannot start before all 16 rows are in, has them to spare.
  // (the general variant keeps a few more values live per sub-step and
  // prefetches 4 rows, which keeps it within 256 registers)
  constexpr int PF = sizeof(T) == 2 ? (B2D ? 16 : (GEN ? 4 : 8)) : 0;
  uint32_t pf[PF > 0 ? PF : 1][NW];
  auto prefetch = [&](int64_t rs, int64_t c0, WaveRows m) {
    if constexpr (PF > 0) {
      if constexpr (GRP) {
        const __amdgpu_buffer_rsrc_t rn = grp_rsrc(m, c0);
        const uint32_t gv = grp_vo(m), gn = h ? m.n1 : m.n0;
#pragma unroll
        for (int i = 0; i < PF; ++i) grp_load(rn, gv, gn, i, pf[i]);
      } else {
        // the loads leave ahead of the other wave's arithmetic on the SIMD
        // (not for four-over-six, which is bound by that arithmetic)
        const __amdgpu_buffer_rsrc_t rn = wave_rows(rs, c0);
        const uint32_t vo = lane_vo(c0);
        if constexpr (VAR != 3) __builtin_amdgcn_s_setprio(2);
#pragma unroll
        for (int i = 0; i < PF; ++i) load_row_buf<T>(rn, vo, (uint32_t)i * rowbytes, pf[i]);
        if constexpr (VAR != 3) __builtin_amdgcn_s_setprio(0);
      }
    }
  };

  int sbuf = 0, mbuf = 0;
  int64_t m0 = 0, c0 = 0, c0_tab = -1;
  int cur_sub = 0;
  bool cur_solo = false;
  int64_t v = next_sub(0, m0, c0, cur_sub, cur_solo);
  WaveRows gm{0, 0u, 0u, 0u, 0u};  // grouped: the current sub-step's rows
  if constexpr (GRP) {
    if (v < n_v) gm = grp_map(m0 + cur_sub * IT_SUB);
  }
  if (v < n_v) prefetch(m0 + cur_sub * IT_SUB, c0, gm);
  while (v < n_v) {
    const int sub = cur_sub;
    const int64_t rs = m0 + sub * IT_SUB;
    // column amax / S_enc: the strip's table in LDS (modes 0 and 1, filled
    // when the strip changes), or the group amax of the lane's 16-row block
    // (mode 2)
    ColLds ctab{&sm.ca[8 * L], &sm.cs[8 * L]};
    if constexpr (COLW && !B2D) {
      if (GRP || p.col_mode == 2) {
        if (L < 8) {
          const int64_t gr = rs + 32 * wv + 16 * h;
          const float a = (!GEN || gr < p.M) ? p.col_amax[gr] : 0.0f;
          sm.ga[wv][h][L] = a;
          sm.gs[wv][h][L] = global_encode_scale(a, p.F);
        }
        __builtin_amdgcn_wave_barrier();
        ctab = ColLds{&sm.ga[wv][h][0], &sm.gs[wv][h][0]};
      } else if (c0 != c0_tab) {
        const float a = p.col_mode == 0 ? p.col_amax[0]
                        : ((!GEN || c0 + tid < K) ? p.col_amax[c0 + tid] : 0.0f);
        __syncthreads();  // every wave is done with the previous strip's table
        sm.ca[tid] = a;
        sm.cs[tid] = global_encode_scale(a, p.F);
        __syncthreads();
        c0_tab = c0;
      }
    }
    // row amax / S_enc of the wave's 32 rows
    if constexpr (ROWW && !B2D) {
      if (lane < 32) {
        const int64_t rr = rs + 32 * wv + lane;
        const float a = (p.row_mode == 0) ? p.row_amax[0]
                        : ((!GEN || rr < p.M) ? p.row_amax[rr] : 0.0f);
        sm.ra[wv][lane] = a;
        sm.rs[wv][lane] = global_encode_scale(a, p.F);
      }
      __builtin_amdgcn_wave_barrier();
    }
    uint32_t w[16][NW];
    if constexpr (GRP) {
      const __amdgpu_buffer_rsrc_t rx = grp_rsrc(gm, c0);
      const uint32_t gv = grp_vo(gm), gn = h ? gm.n1 : gm.n0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (i < PF) {
#pragma unroll
          for (int d = 0; d < NW; ++d) w[i][d] = pf[i < PF ? i : 0][d];
        } else {
          grp_load(rx, gv, gn, i, w[i]);
        }
      }
    } else {
      const __amdgpu_buffer_rsrc_t rx = wave_rows(rs, c0);
      const uint32_t vo = lane_vo(c0);
      if constexpr (VAR != 3) __builtin_amdgcn_s_setprio(2);  // as in the prefetch
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (i < PF) {
#pragma unroll
          for (int d = 0; d < NW; ++d) w[i][d] = pf[i < PF ? i : 0][d];
        } else {
          load_row_buf<T>(rx, vo, (uint32_t)i * rowbytes, w[i]);
        }
      }
      if constexpr (VAR != 3) __builtin_amdgcn_s_setprio(0);
    }
    int64_t m0n = 0, c0n = 0;
    int subn = 0;
    bool solon = false;
    const int64_t vn = next_sub(v + 1, m0n, c0n, subn, solon);
    WaveRows gmn{0, 0u, 0u, 0u, 0u};
    if constexpr (GRP) {
      if (vn < n_v) gmn = grp_map(m0n + subn * IT_SUB);
    }

    StoreIT st;
    st.wv = wv;
    st.h = h;
    st.L = L;
    st.par = par;
    st.slot = 8 * sub + 2 * wv + h;
    st.qrs = (uint32_t)qrs;
    st.sr = &sm.sr[sbuf][0][0];
    st.qc = &sm.qc[mbuf][0][0];
    st.sc = &sm.sc[mbuf][0][0];
    if constexpr (ROWW) {
      st.qr = make_rsrc(p.q_row + (rs + 32 * wv) * qrs + c0 / 2, wave_nr(rs) * qrs);
      st.vo_qr = (!GEN || c0 + 8 * L < K) ? (uint32_t)h * 16u * (uint32_t)qrs + (uint32_t)(4 * L)
                                          : 0x80000000u;
    }
    auto mid = [&]() {
      if constexpr (GRP) {
        if (vn < n_v) prefetch(m0n + subn * IT_SUB, c0n, gmn);
      } else {
        if (vn < n_v) prefetch(m0n + subn * IT_SUB, c0n, WaveRows{0, 0u, 0u, 0u, 0u});
      }
    };
    if constexpr (B2D) {
      process_block_2d<T, ROWW, COLW>(w, st, a2d, s2d, p.F_inv, mid);
    } else if constexpr (VAR == 3) {
      mid();
      process_block_46<T, ROWW, COLW>(w, st, h, par, LdsTab{sm.ra[wv], sm.rs[wv], 0}, ctab,
                                      p.F_inv);
    } else {
      process_block_batched<T, ROWW, COLW>(w, st, h, par, LdsTab{sm.ra[wv], sm.rs[wv], 0}, ctab,
                                           p.F_inv, mid);
    }
    __syncthreads();  // the sub-step's staged outputs are complete
    // the flush's stores, too, go out ahead of the other workgroup's arithmetic
    if constexpr (VAR != 3) __builtin_amdgcn_s_setprio(1);

    if constexpr (ROWW) {  // 128 rows x 16 B
      if constexpr (GEN) {
        // the rows that exist, the strip's blocks that exist
        if (tid < IT_SUB && rs + tid < p.M)
          store_bytes_any(p.s_row + (rs + tid) * srs + c0 / 16, &sm.sr[sbuf][tid][0], 0,
                          (int)min((K - c0) / 16, (int64_t)16));
      } else {
        if (tid < IT_SUB)
          *reinterpret_cast<uint4*>(p.s_row + (rs + tid) * srs + c0 / 16) =
              *reinterpret_cast<const uint4*>(&sm.sr[sbuf][tid][0]);
      }
    }
    sbuf ^= 1;
    // a half flushed on its own (the last macro row of a matrix with
    // M % 256 = 128, or a split tile of the last round) writes 64 B of codes
    // and 8 scale bytes per column, those of its own 128 rows
    const bool half = cur_solo;
    if (GEN && COLW && (sub == 1 || half)) {
      // bytes [lo, hi) of each column's 128 B of codes (a half: its own 64 B;
      // cut at the column's last byte), to rows of any alignment
      const int lo = half ? 64 * sub : 0;
      const int hi = (int)min((int64_t)(half ? lo + 64 : 128), qcs - m0 / 2);
#pragma unroll
      for (int it = 0; it < IT_COLS * 8 / 256; ++it) {
        const int pidx = tid + 256 * it;
        const int c = pidx >> 3, t = pidx & 7;
        const int f = (c >> 3) & 15;
        u32x4 q = *reinterpret_cast<const u32x4*>(&sm.qc[mbuf][c ^ (f & 1)][16 * (t ^ (f >> 1))]);
        if (f & 1) q = (u32x4){q.z, q.w, q.x, q.y};
        const uint32_t prev = (uint32_t)__shfl_up((int)q.w, 1, 8);  // S[4t - 1] (t > 0)
        if (c0 + c < K && hi > lo)
          store_segment_dwords(p.q_col + (c0 + c) * qcs + m0 / 2, q, prev, t, lo, hi);
      }
      // the unaligned bytes at both ends of each column's segment: one
      // thread per column (byte b of column c sits in slot b / 8, stored at
      // slot position (b / 8) ^ f of storage column c ^ (f & 1))
      {
        const int c = tid, f = (c >> 3) & 15;
        const uint8_t* col = &sm.qc[mbuf][c ^ (f & 1)][0];
        if (c0 + c < K && hi > lo)
          store_segment_ends(p.q_col + (c0 + c) * qcs + m0 / 2, lo, hi, [&](int b) {
            return col[8 * ((b >> 3) ^ f) + (b & 7)];
          });
      }
      {
        const int c = 8 * (tid & 31) + (tid >> 5);
        const int slo = half ? 8 * sub : 0;
        const int shi = (int)min((int64_t)(half ? slo + 8 : 16), scs - m0 / 16);
        if (c0 + c < K && shi > slo)
          store_bytes_any(p.s_col + (c0 + c) * scs + m0 / 16, &sm.sc[mbuf][tid][0], slo, shi);
      }
      mbuf ^= 1;
    } else if (COLW && (sub == 1 || half)) {
      // 256 columns x 128 B of transposed codes: 8 lanes per column, whole
      // lines, slots restored to row order
#pragma unroll
      for (int it = 0; it < IT_COLS * 8 / 256; ++it) {
        const int pidx = tid + 256 * it;
        const int c = pidx >> 3, t = pidx & 7;
        if (half && (t >> 2) != sub) continue;
        const int f = (c >> 3) & 15;
        u32x4 q = *reinterpret_cast<const u32x4*>(&sm.qc[mbuf][c ^ (f & 1)][16 * (t ^ (f >> 1))]);
        if (f & 1) q = (u32x4){q.z, q.w, q.x, q.y};
        __builtin_nontemporal_store(q, reinterpret_cast<u32x4*>(p.q_col + (c0 + c) * qcs + m0 / 2 + 16 * t));
      }
      // 256 columns x 16 B of transposed scales (entry tid holds column
      // 8 (tid % 32) + tid / 32)
      {
        const u32x4 q = *reinterpret_cast<const u32x4*>(&sm.sc[mbuf][tid][0]);
        const int c = 8 * (tid & 31) + (tid >> 5);
        uint8_t* dst = p.s_col + (c0 + c) * scs + m0 / 16;
        if ((scs & 15) == 0 && !half) {
          *reinterpret_cast<u32x4*>(dst) = q;
        } else {
          uint32_t* d4 = reinterpret_cast<uint32_t*>(dst);
          if (!half || sub == 0) { d4[0] = q.x; d4[1] = q.y; }
          if (!half || sub == 1) { d4[2] = q.z; d4[3] = q.w; }
        }
      }
      mbuf ^= 1;
    }
    if constexpr (VAR != 3) __builtin_amdgcn_s_setprio(0);
    v = vn;
    m0 = m0n;
    c0 = c0n;
    cur_sub = subn;
    cur_solo = solon;
    if constexpr (GRP) gm = gmn;
  }
}

// ------------------------------------------------------------- edge kernel
// Tiles outside the interior: the partial last strip, the partial last
// 64-row step, or every tile of a shape the buffer path cannot take. One
// workgroup per segment of rows_per_wg rows of one strip, checked loads and
// stores. Launched over a rectangle: segment seg0 + b / nstrips of the row
// range [rstart, rend), strip strip0 + b % nstrips.
template <typename T, bool ROWW, bool COLW, bool B2D, bool FOS = false>
__global__ void __launch_bounds__(256) cast_edge_kernel(const CastK p) {
  static_assert(!(B2D && FOS), "one block rule at a time");
  if (p.noop != nullptr && *p.noop == 1.0f) return;
  constexpr int NW = Blk<T>::NW;
  __shared__ float row_a_s[CAST_MAX_ROWS_PER_WG];
  __shared__ float row_se_s[CAST_MAX_ROWS_PER_WG];
  __shared__ GroupTable gt;
  const T* __restrict__ x = static_cast<const T*>(p.x);
  const bool grouped = p.grp_G > 0;  // uniform
  if (grouped) build_group_table(gt, p.grp_rows, p.grp_G, p.grp_align);
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

  if constexpr (ROWW && !B2D) {
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
    for (int i = 0; i < 16; ++i) {
      if (grouped) {  // padding rows and rows past the groups read as zeros
        const int64_t rr = rb0 + i;
        const int64_t src = rr < re ? token_row(gt, (int)p.grp_G, rr) : -1;
        load_row_checked<T>(x, p.grp_T, K, src < 0 ? p.grp_T : src, c, vec, w[i]);
      } else {
        load_row_checked<T>(x, re, K, rb0 + i, c, vec, w[i]);
      }
    }
    st.rb0 = rb0;
    if constexpr (B2D) {
      const float a = ROWW ? p.row_amax[0] : p.col_amax[0];
      process_block_2d<T, ROWW, COLW>(w, st, a, global_encode_scale(a, p.F), p.F_inv, NoMid());
      continue;
    }
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
    if constexpr (FOS)
      process_block_46<T, ROWW, COLW>(w, st, g, par, rows, ColRegs{acol, scol}, p.F_inv);
    else
      process_block<T, ROWW, COLW>(w, st, g, par, rows, ColRegs{acol, scol}, p.F_inv);
  }
}

template <typename T, bool ROWW, bool COLW, int VAR, bool SPLIT = false, bool GEN = false>
static int interior_grid() {
  // resident interior workgroups on the device (a multiple of 8), per device
  // (host threads may fill an entry concurrently, with the same value)
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int g = cache[dev].load(std::memory_order_relaxed);
  if (g == 0) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu,
            reinterpret_cast<const void*>(cast_interior_kernel<T, ROWW, COLW, VAR, SPLIT, GEN>),
            256, 0) != hipSuccess ||
        per_cu < 1)
      per_cu = 1;
    g = std::max(IT_XCDS, (num_cus() * per_cu) / IT_XCDS * IT_XCDS);
    cache[dev].store(g, std::memory_order_relaxed);
  }
  return g;
}

// The launched grid: at most the resident workgroups, and no more than the
// work needs, two workgroups per macro tile of an XCD (each takes one 128-row
// half of a tile when the tiles fit one round), so that a small matrix does
// not dispatch hundreds of workgroups that find nothing to do. ntx: macro
// tiles per XCD. Stays a multiple of the XCD count.
static int64_t fit_grid(int64_t resident, int64_t ntx) {
  return std::min<int64_t>(resident, (int64_t)IT_XCDS * std::max<int64_t>(1, 2 * ntx));
}

// General shapes in one launch of the macro-tile kernel (1x16 blocks): every
// macro tile of the ceil(M / 256) x ceil(K / 256) grid, cut ones included.
template <typename T, bool ROWW, bool COLW>
static void launch_cast_general(const CastK& k, hipStream_t s) {
  const int64_t nt = k.n_istrips * k.n_isteps;
  const int64_t ntx = (nt + IT_XCDS - 1) / IT_XCDS;
  const int64_t G0 = fit_grid(interior_grid<T, ROWW, COLW, 0, false, true>(), ntx);
  const int64_t per = G0 / IT_XCDS;
  const int64_t rounds = (ntx + per - 1) / per;
  const bool split = per > 0 && rounds > 0 && 2 * (ntx - (rounds - 1) * per) <= per;
  if (split) {
    const int64_t G = fit_grid(interior_grid<T, ROWW, COLW, 0, true, true>(), ntx);
    hipLaunchKernelGGL((cast_interior_kernel<T, ROWW, COLW, 0, true, true>), dim3((unsigned)G),
                       dim3(256), 0, s, k);
  } else {
    hipLaunchKernelGGL((cast_interior_kernel<T, ROWW, COLW, 0, false, true>), dim3((unsigned)G0),
                       dim3(256), 0, s, k);
  }
}

template <typename T, bool ROWW, bool COLW>
static void launch_cast_kernels(CastK k, const CastArgs& a, hipStream_t s) {
  const dim3 block(256);
  const int64_t ntiles = k.n_istrips * k.n_isteps;
  if (ntiles > 0) {
    // all resident workgroups (a partly idle last round costs less than
    // fewer waves per CU), unless the tiles need fewer. Whether the last round
    // splits its tiles into halves (at most half as many tiles as an XCD has
    // workgroups) picks the kernel variant that carries that schedule.
    const int64_t ntx = k.n_isteps * ((k.n_istrips + IT_XCDS - 1) / IT_XCDS);
    auto split = [&](int64_t G) {
      const int64_t per = G / IT_XCDS;
      const int64_t rounds = (ntx + per - 1) / per;
      return per > 0 && rounds > 0 && 2 * (ntx - (rounds - 1) * per) <= per;
    };
    if (k.grp_G > 0) {
      if (split(fit_grid(interior_grid<T, ROWW, COLW, 1>(), ntx))) {
        const int64_t G = fit_grid(interior_grid<T, ROWW, COLW, 1, true>(), ntx);
        hipLaunchKernelGGL((cast_interior_kernel<T, ROWW, COLW, 1, true>), dim3((unsigned)G),
                           dim3(256), 0, s, k);
      } else {
        const int64_t G = fit_grid(interior_grid<T, ROWW, COLW, 1>(), ntx);
        hipLaunchKernelGGL((cast_interior_kernel<T, ROWW, COLW, 1>), dim3((unsigned)G), dim3(256),
                           0, s, k);
      }
    } else if (k.blk2d) {
      if (split(fit_grid(interior_grid<T, ROWW, COLW, 2>(), ntx))) {
        const int64_t G = fit_grid(interior_grid<T, ROWW, COLW, 2, true>(), ntx);
        hipLaunchKernelGGL((cast_interior_kernel<T, ROWW, COLW, 2, true>), dim3((unsigned)G),
                           dim3(256), 0, s, k);
      } else {
        const int64_t G = fit_grid(interior_grid<T, ROWW, COLW, 2>(), ntx);
        hipLaunchKernelGGL((cast_interior_kernel<T, ROWW, COLW, 2>), dim3((unsigned)G), dim3(256),
                           0, s, k);
      }
    } else if (k.four_six) {
      if constexpr (!(ROWW && COLW)) {
        if (split(fit_grid(interior_grid<T, ROWW, COLW, 3>(), ntx))) {
          const int64_t G = fit_grid(interior_grid<T, ROWW, COLW, 3, true>(), ntx);
          hipLaunchKernelGGL((cast_interior_kernel<T, ROWW, COLW, 3, true>), dim3((unsigned)G),
                             dim3(256), 0, s, k);
        } else {
          const int64_t G = fit_grid(interior_grid<T, ROWW, COLW, 3>(), ntx);
          hipLaunchKernelGGL((cast_interior_kernel<T, ROWW, COLW, 3>), dim3((unsigned)G),
                             dim3(256), 0, s, k);
        }
      }
    } else if (split(fit_grid(interior_grid<T, ROWW, COLW, 0>(), ntx))) {
      const int64_t G = fit_grid(interior_grid<T, ROWW, COLW, 0, true>(), ntx);
      hipLaunchKernelGGL((cast_interior_kernel<T, ROWW, COLW, 0, true>), dim3((unsigned)G),
                         dim3(256), 0, s, k);
    } else {
      const int64_t G = fit_grid(interior_grid<T, ROWW, COLW, 0>(), ntx);
      hipLaunchKernelGGL((cast_interior_kernel<T, ROWW, COLW, 0>), dim3((unsigned)G), dim3(256), 0,
                         s, k);
    }
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
    if (k.blk2d)
      hipLaunchKernelGGL((cast_edge_kernel<T, ROWW, COLW, true>), dim3((unsigned)(segs * nstrips)),
                         block, 0, s, k);
    else if (k.four_six) {
      // one direction per launch (both directions' candidates in one kernel
      // exceed the register file)
      if constexpr (!(ROWW && COLW))
        hipLaunchKernelGGL((cast_edge_kernel<T, ROWW, COLW, false, true>),
                           dim3((unsigned)(segs * nstrips)), block, 0, s, k);
    } else
      hipLaunchKernelGGL((cast_edge_kernel<T, ROWW, COLW, false>), dim3((unsigned)(segs * nstrips)),
                         block, 0, s, k);
  };
  const int64_t strips = (a.K + CAST_STRIP_COLS - 1) / CAST_STRIP_COLS;
  if (ntiles > 0)  // the interior spans every column: the rows below it remain
    edge(k.n_isteps * IT_MACRO - (k.half_last ? IT_SUB : 0), a.M, 0, strips);
  else
    edge(0, a.M, 0, strips);
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
  k.grp_rows = a.grp_rows;
  k.grp_G = a.grp_G;
  k.grp_align = a.grp_align;
  k.grp_T = a.grp_T;
  k.blk2d = a.blk2d;
  k.four_six = a.four_six;
  constexpr int V = 16 / sizeof(T);
  k.vec_load = ((a.K % V) == 0) && ((reinterpret_cast<uintptr_t>(a.x) & 15) == 0);
  k.row_store4 = (a.K % 8 == 0) && ((reinterpret_cast<uintptr_t>(a.q_row) & 3) == 0);
  k.col_store8 = (a.M % 16 == 0) && ((reinterpret_cast<uintptr_t>(a.q_col) & 7) == 0);
  // Interior (persistent macro-tile) path: 16-byte aligned rows, K % 256 == 0
  // (whole strips; 16-byte rowwise-scale stores), M % 64 == 0 (16-byte
  // transposed-code stores, at least 4-byte transposed-scale stores), outputs
  // aligned for those stores, and every in-tile offset within 31 bits. Rows
  // below the last whole macro tile go to the edge kernel.
  const int64_t lim = 0x7FFFFFFF;
  const int64_t scs = (a.M + 15) / 16;
  const uintptr_t sc_align = (scs % 16 == 0) ? 15 : 3;
  // Grouped tokens (always row mode LINE, column mode ROWGROUP) take the
  // interior path too when token rows and padded rows index in 31 bits (a
  // masked row's offset, 2^31 + 15 rows, then stays within 32 bits).
  const bool grp_ok = a.grp_G == 0 || (a.grp_G <= IT_COLS && a.row_mode == 1 && a.col_mode == 2 &&
                                       a.grp_T < lim && a.M < lim);
  const bool fast = grp_ok && k.vec_load && (a.K % IT_COLS == 0) && (a.M % 64 == 0) &&
                    (!a.q_row || (reinterpret_cast<uintptr_t>(a.q_row) & 3) == 0) &&
                    (!a.s_row || (reinterpret_cast<uintptr_t>(a.s_row) & 15) == 0) &&
                    (!a.q_col || (reinterpret_cast<uintptr_t>(a.q_col) & 15) == 0) &&
                    (!a.s_col || (reinterpret_cast<uintptr_t>(a.s_col) & sc_align) == 0) &&
                    (int64_t)32 * a.K * (int64_t)sizeof(T) < lim;
  k.n_istrips = fast ? a.K / IT_COLS : 0;
  k.n_isteps = fast ? a.M / IT_MACRO : 0;
  k.half_last = fast && (a.M % IT_MACRO) >= IT_SUB;  // one more, 128-row macro row
  k.n_isteps += k.half_last;
  // Up to sixteen strips side by side: in one round of an XCD's 64
  // workgroups the macro tiles form a block of several strips by several macro
  // rows, so each row's codes and each column's transposed codes leave in runs
  // of several 128-byte lines. On 8192 x 28672 (14 strips per XCD), same box:
  // 1 strip 227.0 us per step and 146.4 us per cast, 8 strips 225.7 / 143.7,
  // all 14 strips 226.0 / 140.9.
  k.sgroup = 16;
  // the kernel indexes macro tiles with 32-bit arithmetic: tiles per XCD and
  // sub-steps per workgroup stay far below 2^31
  if (k.n_isteps * ((k.n_istrips + IT_XCDS - 1) / IT_XCDS) >= ((int64_t)1 << 30))
    k.n_istrips = k.n_isteps = 0;
  if (k.n_istrips == 0 || k.n_isteps == 0) k.n_istrips = k.n_isteps = k.half_last = 0;
  const bool rw = a.q_row != nullptr, cw = a.q_col != nullptr;
  // Shapes the plain macro-tile path covers alone keep it; every other shape
  // with 16-byte rows, K % 16 == 0 and plain 1x16 blocks takes the general
  // variant in one launch (no edge launches).
  const bool alone = k.n_istrips > 0 && a.M % IT_SUB == 0;
  const bool general = !alone && a.grp_G == 0 && !a.blk2d && !a.four_six && k.vec_load &&
                       a.K % 16 == 0 && (int64_t)32 * a.K * (int64_t)sizeof(T) < lim &&
                       (!a.q_row || (reinterpret_cast<uintptr_t>(a.q_row) & 3) == 0);
  if (general) {
    CastK g = k;
    g.n_istrips = (a.K + IT_COLS - 1) / IT_COLS;
    g.n_isteps = (a.M + IT_MACRO - 1) / IT_MACRO;
    const int64_t tail = a.M % IT_MACRO;
    g.half_last = tail != 0 && tail <= IT_SUB;  // the last macro row has one sub-step
    if (g.n_isteps * g.n_istrips < ((int64_t)1 << 30)) {
      if (rw && cw) launch_cast_general<T, true, true>(g, s);
      else if (rw) launch_cast_general<T, true, false>(g, s);
      else launch_cast_general<T, false, true>(g, s);
      return hipGetLastError() == hipSuccess ? 0 : -3;
    }
  }
  if (rw && cw && a.four_six) {
    launch_cast_kernels<T, true, false>(k, a, s);
    launch_cast_kernels<T, false, true>(k, a, s);
  } else if (rw && cw) launch_cast_kernels<T, true, true>(k, a, s);
  else if (rw) launch_cast_kernels<T, true, false>(k, a, s);
  else launch_cast_kernels<T, false, true>(k, a, s);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

int launch_cast(const CastArgs& a, hipStream_t s) {
  return a.in_dtype == 0 ? launch_cast_t<uint16_t>(a, s) : launch_cast_t<float>(a, s);
}

}  // namespace nvfp4

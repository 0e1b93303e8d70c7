// nvfp4_device.h -- device-side building blocks of the NVFP4 kernels (gfx950).
//
// Every floating-point step is a single IEEE binary32 operation rounded to
// nearest-even with subnormals kept: the library is compiled without fast-math
// and with -ffp-contract=off, HIP's '/' is the correctly rounded division, and
// fp32 denormals are not flushed on gfx950 by default.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

constexpr float kFltMax = 3.402823466e38f;
constexpr float kE4M3Max = 448.0f;
constexpr float kE2M1Max = 6.0f;

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- bit helpers
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  u16x2 x = __builtin_bit_cast(u16x2, a), y = __builtin_bit_cast(u16x2, b);
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(x, y));
}
// A dword holding two BF16 values: element 0 in the low half.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Magnitude bit patterns compare like the magnitudes (finite, non-NaN input).
constexpr uint32_t kAbsBf16x2 = 0x7FFF7FFFu;
constexpr uint32_t kAbsF32 = 0x7FFFFFFFu;

// Swap with the neighbouring lane (lane ^ 1) through DPP quad_perm [1,0,3,2].
__device__ __forceinline__ uint32_t dpp_swap1(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
}
__device__ __forceinline__ float dpp_swap1(float v) {
  return __uint_as_float(dpp_swap1(__float_as_uint(v)));
}
// Max over the 16 lanes of a DPP row (lanes 16r .. 16r+15); every lane of the
// row gets the result. quad xor 1, quad xor 2, half-row mirror, row mirror.
__device__ __forceinline__ uint32_t row16_max(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false));
  return v;
}

// ------------------------------------------------------------ scale pipeline
// Second-level encode scale of a line: a == 0 -> 1, else min(RN(F / a), FLT_MAX).
__device__ __forceinline__ float global_encode_scale(float a, float F) {
  if (a == 0.0f) return 1.0f;
  return fminf(F / a, kFltMax);
}

// RN(x / 6) for x >= 0. For x >= 2^-125 the product with RN(1/6) is within
// an ulp of x/6, its residual fma(-q, 6, x) is exact, and one correction step
// gives the correctly rounded quotient (checked exhaustively on gfx950 against
// the IEEE division for every finite x >= 2^-125); smaller x take the IEEE
// division.
__device__ __forceinline__ float div6_rn(float x) {
  constexpr float kR6 = 0.16666667163372039794921875f;  // RN(1/6)
  if (x >= 0x1p-125f) {
    const float q = x * kR6;
    return __builtin_fmaf(__builtin_fmaf(-q, kE2M1Max, x), kR6, q);
  }
  return x / kE2M1Max;
}

// Significand field of a binary32 pattern that is all ones: d = (2 - 2^-23) 2^k.
constexpr uint32_t kSigMask = 0x007FFFFFu;

// min(RN(1 / d), FLT_MAX) for d > 0. For d in [2^-126, 2^126) the hardware
// reciprocal r is within an ulp of 1/d, and one Newton step
// fma(fma(-d, r, 1), r, r) gives RN(1/d) from either neighbour of 1/d except
// at one significand: for d = (2 - 2^-23) 2^k, 1/d lies 2^-48 relative above
// the midpoint between 2^-k-1 and its successor, and from r = 2^-k-1 the
// step computes exactly that midpoint, which rounds to even (the wrong side).
// Those d, and d outside the range, take the IEEE division, so the result
// never depends on which neighbour the hardware returns (the exception and
// the exactness elsewhere are shown by exact rational arithmetic over every
// significand, from both neighbours).
__device__ __forceinline__ float recip_newton(float d) {
  const float r = __builtin_amdgcn_rcpf(d);
  return __builtin_fmaf(__builtin_fmaf(-d, r, 1.0f), r, r);
}
__device__ __forceinline__ float recip_rn(float d) {
  if (d >= 0x1p-126f && d < 0x1p126f && (__float_as_uint(d) & kSigMask) != kSigMask)
    return recip_newton(d);
  return fminf(1.0f / d, kFltMax);
}

// The fast reciprocal form holds for this decode-scale bit pattern: D in
// [2^-126, 2^126) and a significand that is not all ones.
__device__ __forceinline__ bool recip_fast_ok(uint32_t db) {
  return ((db - 0x00800000u) < 0x7E000000u) & ((db & kSigMask) != kSigMask);
}

// One block: from its max magnitude, the line amax a, the line's S_enc and
// F_inv, produce the stored E4M3 byte and the element encode factor:
//   s32  = RN(RN(bamax / 6) * S_enc), clamped to 448 (also maps +inf to 448)
//   byte = E4M3 round-to-nearest-even of s32 (v_cvt_pk_fp8_f32: OCP E4M3FN,
//          equal to the RNE definition for every s32 in [0, 448], checked
//          exhaustively on gfx950), sq = its exact value
//   D    = RN(RN(sq * a) * F_inv)
//   enc  = D == 0 ? 0 : min(RN(1 / D), FLT_MAX)
__device__ __forceinline__ void block_scale(float bamax, float a, float s_enc, float f_inv,
                                            uint32_t* byte, float* enc) {
  const float s32 = fminf(div6_rn(bamax) * s_enc, kE4M3Max);
  const int pk = __builtin_amdgcn_cvt_pk_fp8_f32(s32, s32, 0, false);
  *byte = (uint32_t)pk & 0xFFu;
  const float sq = __builtin_amdgcn_cvt_f32_fp8(pk, 0);
  const float d = (sq * a) * f_inv;
  *enc = (d == 0.0f) ? 0.0f : recip_rn(d);
}

// The unguarded scale chain itself: *byte (low byte) and *enc as block_scale
// gives them whenever bamax >= 2^-121 and recip_fast_ok(D) holds; returns D's
// bit pattern so that callers can check those conditions for many blocks at
// once.
// RN(bamax / 6) is fma(bamax, H, RN(bamax * L)) with H = RN(1/6) and
// L = RN(1/6 - H): bamax / 6 is never closer to a rounding midpoint than a
// sixth of an ulp, far more than this two-term product's error, and the
// result equals the IEEE quotient for every finite bamax >= 2^-121 (checked
// exhaustively, binary32 arithmetic emulated exactly). The converter keeps
// the upper half of its first operand's register, so it starts from s32's
// own bits (no zeroing move); only the low byte is used.
constexpr uint32_t kFastBamaxMin = 0x03000000u;  // bit pattern of 2^-121
__device__ __forceinline__ float div6_two_term(float x) {
  constexpr float kR6 = 0.16666667163372039794921875f;  // RN(1/6)
  constexpr float kR6lo = -0x1.555556p-28f;              // RN(1/6 - RN(1/6))
  return __builtin_fmaf(x, kR6, x * kR6lo);
}
__device__ __forceinline__ uint32_t block_scale_unchecked(float bamax, float a, float s_enc,
                                                          float f_inv, uint32_t* byte, float* enc) {
  const float s32 = fminf(div6_two_term(bamax) * s_enc, kE4M3Max);
  const int pk = __builtin_amdgcn_cvt_pk_fp8_f32(s32, s32, __float_as_int(s32), false);
  *byte = (uint32_t)pk;
  const float sq = __builtin_amdgcn_cvt_f32_fp8(pk, 0);
  const float d = (sq * a) * f_inv;
  *enc = recip_newton(d);
  return __float_as_uint(d);
}

// block_scale without its range guards: the same results whenever
// bamax >= 2^-121 (the two-term quotient above) and recip_fast_ok(D) (then
// D != 0 too), which it reports. *byte is the converter's packed result: its
// low byte is the scale byte. Callers redo the lanes where it returns false
// with block_scale.
__device__ __forceinline__ bool block_scale_fast(float bamax, float a, float s_enc, float f_inv,
                                                 uint32_t* byte, float* enc) {
  const uint32_t db = block_scale_unchecked(bamax, a, s_enc, f_inv, byte, enc);
  const uint32_t bb = __float_as_uint(bamax);
  return (bb >= kFastBamaxMin) & recip_fast_ok(db);
}

// block_scale that also returns the block's decode scale D (the factor the
// dequantize multiplies each code value by).
__device__ __forceinline__ void block_scale_dec(float bamax, float a, float s_enc, float f_inv,
                                                uint32_t* byte, float* enc, float* dec) {
  const float s32 = fminf(div6_rn(bamax) * s_enc, kE4M3Max);
  const int pk = __builtin_amdgcn_cvt_pk_fp8_f32(s32, s32, 0, false);
  *byte = (uint32_t)pk & 0xFFu;
  const float sq = __builtin_amdgcn_cvt_f32_fp8(pk, 0);
  const float d = (sq * a) * f_inv;
  *dec = d;
  *enc = (d == 0.0f) ? 0.0f : recip_rn(d);
}

// --------------------------------------------------------------- E2M1 encode
// v_cvt_scalef32_pk_fp4_f32 with scale 1.0 converts two fp32 values to E2M1
// with round-to-nearest-even, saturation at 6 and the sign bit kept (-0 and
// negatives rounding to 0 give 0x8); this equals the definition for every
// non-NaN fp32 input (checked exhaustively on gfx950). The first value lands
// in the low nibble of byte SEL of the result, the second in the high nibble;
// the other bytes of `old` pass through.
#define NVFP4_CVT_FP4X2(old, v0, v1, SEL) \
  __builtin_amdgcn_cvt_scalef32_pk_fp4_f32((old), (v0), (v1), 1.0f, (SEL))

// Eight elements -> one dword of eight nibbles (element k in nibble k). All
// four bytes are written, so the first convert may start from any value: it
// takes v0's own bits, a register that dies there (no zeroing move).
__device__ __forceinline__ uint32_t e2m1_pack8(float v0, float v1, float v2, float v3, float v4,
                                               float v5, float v6, float v7) {
  uint32_t w = NVFP4_CVT_FP4X2(__float_as_uint(v0), v0, v1, 0);
  w = NVFP4_CVT_FP4X2(w, v2, v3, 1);
  w = NVFP4_CVT_FP4X2(w, v4, v5, 2);
  w = NVFP4_CVT_FP4X2(w, v6, v7, 3);
  return w;
}

// ------------------------------------------------------------ decoding
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two E2M1 codes (byte SEL of w, low nibble first) -> two floats, exact:
// v_cvt_scalef32_pk_f32_fp4 with scale 1.0 equals the E2M1 table for every
// byte and select (checked exhaustively on gfx950).
template <int SEL>
__device__ __forceinline__ f32x2 fp4x2_decode(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
}

// Two floats -> two BF16 (element 0 in the low half), round to nearest even:
// v_cvt_pk_bf16_f32 equals the RNE definition for every non-NaN fp32
// (checked exhaustively on gfx950).
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// One float -> BF16 bits, round to nearest even, in integer arithmetic (the
// carry into bit 16 is the rounding; ties keep an even bit 16). Non-NaN input.
__device__ __forceinline__ uint32_t bf16_rne(float y) {
  const uint32_t b = __float_as_uint(y);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// E4M3 byte -> float, exact. Low 7 bits: exponent field e, mantissa m;
// e == 0: m * 2^-9, else (1 + m/8) * 2^(e-7) = fp32 pattern (byte + (120<<3)) << 20.
__device__ __forceinline__ float e4m3_value(uint32_t byte) {
  const uint32_t mag = byte & 0x7Fu;
  const float v = mag < 8u ? (float)mag * 0x1p-9f : __uint_as_float((mag + (120u << 3)) << 20);
  return (byte & 0x80u) ? -v : v;
}

// E2M1 code -> float, exact: magnitude field e = (c >> 1) & 3, mantissa m = c & 1;
// e == 0: 0.5 m; else fp32 pattern ((e + 126) << 23) | (m << 22). Bit 3 = sign.
__device__ __forceinline__ float e2m1_value(uint32_t c) {
  const uint32_t e = (c >> 1) & 3u, m = c & 1u;
  const uint32_t mag = e == 0u ? (m ? 0x3F000000u : 0u) : (((e + 126u) << 23) | (m << 22));
  return __uint_as_float(mag | ((c & 8u) << 28));
}

// -------------------------------------------------------- grouped tokens
// Ragged token groups laid out padded (grouped-GEMM PR description: groups
// zero-padded to an alignment before quantization): group g holds rows[g]
// consecutive token rows starting at tok0[g] and occupies the padded rows
// [pad0[g], pad0[g + 1]), its size rounded up to `align`. Both prefix sums
// live in LDS; every workgroup of 256 threads builds them itself (G <= 256).
constexpr int GRP_MAX = 256;

struct GroupTable {
  int64_t tok0[GRP_MAX + 1];
  int64_t pad0[GRP_MAX + 1];
};

// Inclusive scan of the sizes (negative sizes count as 0); all 256 threads.
__device__ __forceinline__ void build_group_table(GroupTable& gt, const int64_t* rows, int64_t G,
                                                  int64_t align) {
  const int t = threadIdx.x;
  const int64_t n = (t < G) ? max(rows[t], (int64_t)0) : 0;
  gt.tok0[t + 1] = n;
  gt.pad0[t + 1] = (n + align - 1) / align * align;
  if (t == 0) gt.tok0[0] = gt.pad0[0] = 0;
  __syncthreads();
  for (int off = 1; off < GRP_MAX; off <<= 1) {
    int64_t a = 0, b = 0;
    if (t >= off) {
      a = gt.tok0[t + 1 - off];
      b = gt.pad0[t + 1 - off];
    }
    __syncthreads();
    if (t >= off) {
      gt.tok0[t + 1] += a;
      gt.pad0[t + 1] += b;
    }
    __syncthreads();
  }
}

// The group holding v, for starts[0] <= v < starts[G]: the last g with
// starts[g] <= v (empty groups share their start with the next group).
__device__ __forceinline__ int group_of(const int64_t* starts, int G, int64_t v) {
  int lo = 0, hi = G;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (starts[mid] <= v) lo = mid;
    else hi = mid;
  }
  return lo;
}

// Token row behind padded row pr, or -1 for a padding row (or a row past the
// last group).
__device__ __forceinline__ int64_t token_row(const GroupTable& gt, int G, int64_t pr) {
  if (pr < 0 || pr >= gt.pad0[G]) return -1;
  const int g = group_of(gt.pad0, G, pr);
  const int64_t r = pr - gt.pad0[g];
  return r < gt.tok0[g + 1] - gt.tok0[g] ? gt.tok0[g] + r : -1;
}

// The same prefix sums held in the registers of one wave, 32-bit: lane l
// keeps the inclusive ends of groups 4l .. 4l + 3 in token rows (tok) and in
// padded rows (pad), saturating at 2^31 - 1; groups from G on end at
// 0xFFFFFFFF. Built by every lane of a wave with no LDS and no barrier
// (G <= 256). For rows below 2^31 - 1 the saturated ends lie past every row
// looked up, so the map below is exact there.
struct LaneEnds {
  uint32_t tok[4], pad[4];
};

__device__ __forceinline__ LaneEnds lane_group_ends(const int64_t* rows, int G, int64_t align,
                                                    int lane) {
  constexpr uint32_t CL = 0x7FFFFFFFu;
  LaneEnds e;
  uint32_t st = 0u, sp = 0u;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int g = 4 * lane + k;
    const int64_t n = g < G ? min(max(rows[g], (int64_t)0), (int64_t)CL) : 0;
    st = min(st + (uint32_t)n, CL);
    sp = min(sp + (uint32_t)min((n + align - 1) / align * align, (int64_t)CL), CL);
    e.tok[k] = st;
    e.pad[k] = sp;
  }
  // inclusive scan of the lane totals, then shift to an exclusive offset
  uint32_t it = st, ip = sp;
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t ot = (uint32_t)__shfl_up((int)it, off), op = (uint32_t)__shfl_up((int)ip, off);
    if (lane >= off) {
      it = min(it + ot, CL);
      ip = min(ip + op, CL);
    }
  }
  uint32_t xt = (uint32_t)__shfl_up((int)it, 1), xp = (uint32_t)__shfl_up((int)ip, 1);
  if (lane == 0) xt = xp = 0u;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const bool live = 4 * lane + k < G;
    e.tok[k] = live ? min(e.tok[k] + xt, CL) : 0xFFFFFFFFu;
    e.pad[k] = live ? min(e.pad[k] + xp, CL) : 0xFFFFFFFFu;
  }
  return e;
}

// Number of groups whose end (in `ends`) is at or before v: for a row v below
// the last end, the index of the group holding it. v is wave-uniform; all 64
// lanes active.
__device__ __forceinline__ uint32_t groups_ending_by(const uint32_t (&ends)[4], uint32_t v) {
  return __builtin_popcountll(__builtin_amdgcn_ballot_w64(ends[0] <= v)) +
         __builtin_popcountll(__builtin_amdgcn_ballot_w64(ends[1] <= v)) +
         __builtin_popcountll(__builtin_amdgcn_ballot_w64(ends[2] <= v)) +
         __builtin_popcountll(__builtin_amdgcn_ballot_w64(ends[3] <= v));
}

// End of group g (wave-uniform, 0 <= g < 256) from the lane that holds it.
__device__ __forceinline__ uint32_t group_end_at(const uint32_t (&ends)[4], uint32_t g) {
  const uint32_t k = g & 3u;
  const uint32_t v = k == 0u ? ends[0] : (k == 1u ? ends[1] : (k == 2u ? ends[2] : ends[3]));
  return (uint32_t)__shfl((int)v, (int)(g >> 2));
}

}  // namespace nvfp4

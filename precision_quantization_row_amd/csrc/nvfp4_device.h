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

// E4M3 (OCP E4M3FN) round-to-nearest-even of s in [0, 448]. Returns the byte
// and its exact value in *decoded.
//  s <  2^-6: the subnormal grid m * 2^-9, m = RNE(s * 2^9) in 0..8 (8 is the
//             smallest normal, byte 0x08, so the carry is seamless)
//  s >= 2^-6: keep 3 mantissa bits of the fp32 pattern with RNE; a carry into
//             the exponent is the correct next binade; the exponent is rebiased
//             from 127 to 7 by subtracting 120 << 3.
__device__ __forceinline__ uint32_t e4m3_rne(float s, float* decoded) {
  if (s < 0x1p-6f) {
    const float m = rintf(s * 512.0f);
    *decoded = m * 0x1p-9f;
    return (uint32_t)m;
  }
  const uint32_t b = __float_as_uint(s);
  const uint32_t r = (b + 0x7FFFFu + ((b >> 20) & 1u)) & 0xFFF00000u;
  *decoded = __uint_as_float(r);
  return (r >> 20) - (120u << 3);
}

// One block: from its max magnitude, the line amax a, the line's S_enc and
// F_inv, produce the stored E4M3 byte and the element encode factor.
__device__ __forceinline__ void block_scale(float bamax, float a, float s_enc, float f_inv,
                                            uint32_t* byte, float* enc) {
  float s32 = (bamax / kE2M1Max) * s_enc;
  s32 = fminf(s32, kE4M3Max);  // also maps +inf to 448
  float sq;
  *byte = e4m3_rne(s32, &sq);
  const float d = (sq * a) * f_inv;
  *enc = (d == 0.0f) ? 0.0f : fminf(1.0f / d, kFltMax);
}

// --------------------------------------------------------------- E2M1 encode
// Round-to-nearest-even onto {0, .5, 1, 1.5, 2, 3, 4, 6}, saturating at 6,
// sign bit (bit 3) copied from v (so -0 and negatives rounding to 0 give 0x8).
//  |v| < 1: code = RNE(2|v|) in 0..2 (0.25 -> 0, 0.75 -> 2: ties to even)
//  |v| >= 1: keep 1 mantissa bit of the fp32 pattern with RNE; exponent
//            rebias 127 -> 1 is a subtraction of 126 << 1; clamp to 7.
__device__ __forceinline__ uint32_t e2m1_rne(float v) {
  const uint32_t bits = __float_as_uint(v);
  const uint32_t sign = (bits >> 28) & 8u;
  const uint32_t mb = bits & kAbsF32;
  const float m = __uint_as_float(mb);
  uint32_t code;
  if (m < 1.0f) {
    code = (uint32_t)rintf(m * 2.0f);
  } else {
    const uint32_t t = (mb + 0x1FFFFFu + ((mb >> 22) & 1u)) >> 22;
    code = min(t - 252u, 7u);
  }
  return sign | code;
}

// Four elements -> four nibbles in the low 16 bits (element 0 lowest).
__device__ __forceinline__ uint32_t e2m1_pack4(float v0, float v1, float v2, float v3) {
  return e2m1_rne(v0) | (e2m1_rne(v1) << 4) | (e2m1_rne(v2) << 8) | (e2m1_rne(v3) << 12);
}

}  // namespace nvfp4

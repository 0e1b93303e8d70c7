// dequant.hip -- NVFP4 dequantize (gfx950).
//
// The inverse of one packed copy (torchao backward-overrides PR description:
// the decode follows TransformerEngine's dequantize kernel, (scale * amax) *
// factor_inv with a correctly rounded FP32 reciprocal, per-tensor and
// row-scaled, BF16 or FP32 output):
//   D   = RN(RN(e4m3(byte) * a) * F_inv)
//   y_k = RN(e2m1(code_k) * D), BF16 output = RNE(y_k)
// Two kernels: a vector kernel for lines of whole blocks with aligned rows
// (the common case, below), and a general kernel, one thread per 1x16 block
// with per-element bounds, for every other shape or alignment.
// Scale bytes are E4M3FN magnitudes as the quantizer writes them (0x00-0x7E);
// bytes with the sign bit decode to negative scales; 0x7F and 0xFF (the
// format's NaN encodings) are outside the contract.
#include "nvfp4_device.h"
#include "nvfp4_launch.h"

#include <algorithm>

namespace nvfp4 {

template <bool OUT_BF16>
__global__ void __launch_bounds__(256) dequant_kernel(const DequantArgs p, int64_t nb, int vec) {
  if (p.noop != nullptr && *p.noop == 1.0f) return;
  const int64_t R = p.R, C = p.C;
  const int64_t qrs = (C + 1) / 2;
  const int64_t total = R * nb;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total; t += stride) {
    const int64_t r = t / nb, b = t - (t / nb) * nb;
    const float a = p.amax_mode == 0 ? p.amax[0] : (p.amax_mode == 1 ? p.amax[r] : p.amax[16 * b]);
    const float d = (e4m3_value(p.sc[r * nb + b]) * a) * p.F_inv;
    const int64_t c0 = 16 * b;
    const bool full = vec && (c0 + 16 <= C);
    uint32_t w0 = 0u, w1 = 0u;
    const uint8_t* qp = p.q + r * qrs + c0 / 2;
    if (full) {
      const uint2 v = *reinterpret_cast<const uint2*>(qp);
      w0 = v.x;
      w1 = v.y;
    } else {
      for (int k = 0; k < 8; ++k)
        if (c0 + 2 * k < C) {
          const uint32_t byte = qp[k];
          if (k < 4) w0 |= byte << (8 * k);
          else w1 |= byte << (8 * (k - 4));
        }
    }
    float y[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const uint32_t code = ((k < 8 ? w0 : w1) >> (4 * (k & 7))) & 0xFu;
      y[k] = e2m1_value(code) * d;
    }
    if constexpr (OUT_BF16) {
      uint16_t* out = static_cast<uint16_t*>(p.y) + r * C + c0;
      if (full) {
        uint32_t o[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) o[k] = bf16_rne(y[2 * k]) | (bf16_rne(y[2 * k + 1]) << 16);
        reinterpret_cast<uint4*>(out)[0] = make_uint4(o[0], o[1], o[2], o[3]);
        reinterpret_cast<uint4*>(out)[1] = make_uint4(o[4], o[5], o[6], o[7]);
      } else {
        for (int k = 0; k < 16; ++k)
          if (c0 + k < C) out[k] = (uint16_t)bf16_rne(y[k]);
      }
    } else {
      float* out = static_cast<float*>(p.y) + r * C + c0;
      if (full) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
          reinterpret_cast<float4*>(out)[k] = make_float4(y[4 * k], y[4 * k + 1], y[4 * k + 2], y[4 * k + 3]);
      } else {
        for (int k = 0; k < 16; ++k)
          if (c0 + k < C) out[k] = y[k];
      }
    }
  }
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Vector path: C % 16 == 0, code rows 4-byte aligned, output rows 16-byte
// aligned. A lane decodes EPL consecutive elements of one line (8 for BF16
// output: 4 code bytes in, 16 B out; 4 for FP32 output: 2 code bytes in, 16 B
// out), so each store instruction of a wave writes 1 KB of one line. A line is
// walked in chunks of 256 * EPL elements, one chunk per workgroup iteration;
// the output is written once and never re-read here, so it takes
// non-temporal stores. The scale byte is decoded with v_cvt_f32_fp8 (E4M3FN:
// exact for every byte except 0x7F / 0xFF, the format's NaN encodings).
template <bool OUT_BF16>
__global__ void __launch_bounds__(256) dequant_vec_kernel(const DequantArgs p, int64_t nchunk) {
  if (p.noop != nullptr && *p.noop == 1.0f) return;
  constexpr int EPL = OUT_BF16 ? 8 : 4;
  const int64_t C = p.C, qrs = C / 2, nb = C / 16;
  const int64_t total = p.R * nchunk;
  for (int64_t tile = blockIdx.x; tile < total; tile += gridDim.x) {
    const int64_t r = tile / nchunk;
    const int64_t c = (tile - r * nchunk) * (256 * EPL) + (int64_t)threadIdx.x * EPL;
    if (c >= C) continue;  // C % 16 == 0: a lane's EPL elements are all inside the line
    const int64_t b = c >> 4;
    const float a = p.amax_mode == 0 ? p.amax[0] : (p.amax_mode == 1 ? p.amax[r] : p.amax[16 * b]);
    const float d = (__builtin_amdgcn_cvt_f32_fp8((int)p.sc[r * nb + b], 0) * a) * p.F_inv;
    const uint8_t* qp = p.q + r * qrs + c / 2;
    if constexpr (OUT_BF16) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(qp);
      const f32x2 v0 = fp4x2_decode<0>(w), v1 = fp4x2_decode<1>(w);
      const f32x2 v2 = fp4x2_decode<2>(w), v3 = fp4x2_decode<3>(w);
      const u32x4 o = {bf16x2_rne(v0.x * d, v0.y * d), bf16x2_rne(v1.x * d, v1.y * d),
                       bf16x2_rne(v2.x * d, v2.y * d), bf16x2_rne(v3.x * d, v3.y * d)};
      __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(static_cast<uint16_t*>(p.y) + r * C + c));
    } else {
      const uint32_t w = *reinterpret_cast<const uint16_t*>(qp);
      const f32x2 v0 = fp4x2_decode<0>(w), v1 = fp4x2_decode<1>(w);
      const u32x4 o = {__float_as_uint(v0.x * d), __float_as_uint(v0.y * d),
                       __float_as_uint(v1.x * d), __float_as_uint(v1.y * d)};
      __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(static_cast<float*>(p.y) + r * C + c));
    }
  }
}

int launch_dequant(const DequantArgs& a, hipStream_t s) {
  const int64_t nb = (a.C + 15) / 16;
  const int64_t total = a.R * nb;
  const int vec = (a.C % 16 == 0) && ((reinterpret_cast<uintptr_t>(a.q) & 3) == 0) &&
                  ((reinterpret_cast<uintptr_t>(a.y) & 15) == 0);
  if (vec) {
    const int epl = a.out_dtype == 0 ? 8 : 4;
    const int64_t nchunk = (a.C + 256 * epl - 1) / (256 * epl);
    const int64_t blocks =
        std::max<int64_t>(1, std::min<int64_t>(a.R * nchunk, (int64_t)num_cus() * 8));
    if (a.out_dtype == 0)
      hipLaunchKernelGGL((dequant_vec_kernel<true>), dim3((unsigned)blocks), dim3(256), 0, s, a, nchunk);
    else
      hipLaunchKernelGGL((dequant_vec_kernel<false>), dim3((unsigned)blocks), dim3(256), 0, s, a, nchunk);
    return hipGetLastError() == hipSuccess ? 0 : -3;
  }
  // general path: one thread per block, any alignment and any C
  const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>((total + 255) / 256, (int64_t)num_cus() * 16));
  if (a.out_dtype == 0)
    hipLaunchKernelGGL((dequant_kernel<true>), dim3((unsigned)blocks), dim3(256), 0, s, a, nb, 0);
  else
    hipLaunchKernelGGL((dequant_kernel<false>), dim3((unsigned)blocks), dim3(256), 0, s, a, nb, 0);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // namespace nvfp4

// nvfp4_identities.hip -- TEST PROBES for the device building blocks in
// precision_quantization_row_amd/csrc/nvfp4_device.h.
//
// Each probe runs one of those functions (the same inline code the kernels
// use) over a run of inputs and writes the raw results; the tests compare
// them with the CPU oracle's definitions over the functions' whole input
// ranges. Nothing here is part of the library.
//
// Runs of binary32 bit patterns: element i of a run starting at `start`
// holds the pattern start + i (the caller keeps start + n <= 2^32).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4_device.h"

using namespace nvfp4;

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ int64_t gtid() { return (int64_t)blockIdx.x * blockDim.x + threadIdx.x; }
__device__ __forceinline__ int64_t gstride() { return (int64_t)gridDim.x * blockDim.x; }

// E2M1 encode with scale 1 (e2m1_pack8): 8 patterns -> one dword of nibbles.
__global__ void fp4_encode_kernel(uint32_t start, int64_t n8, uint32_t* out) {
  for (int64_t t = gtid(); t < n8; t += gstride()) {
    const uint32_t b = start + (uint32_t)(8 * t);
    out[t] = e2m1_pack8(__uint_as_float(b), __uint_as_float(b + 1u), __uint_as_float(b + 2u),
                        __uint_as_float(b + 3u), __uint_as_float(b + 4u), __uint_as_float(b + 5u),
                        __uint_as_float(b + 6u), __uint_as_float(b + 7u));
  }
}

// E4M3 encode of a non-negative scale: the converter in both operand forms
// the scale chains use (a zero third operand, and the scale's own bits).
__global__ void fp8_encode_kernel(uint32_t start, int64_t n, uint8_t* out_zero, uint8_t* out_self) {
  for (int64_t t = gtid(); t < n; t += gstride()) {
    const float s = __uint_as_float(start + (uint32_t)t);
    out_zero[t] = (uint8_t)__builtin_amdgcn_cvt_pk_fp8_f32(s, s, 0, false);
    out_self[t] = (uint8_t)__builtin_amdgcn_cvt_pk_fp8_f32(s, s, __float_as_int(s), false);
  }
}

// Decodes over every byte / code: E4M3 by the converter (byte 0 of a word
// whose upper bytes hold 4 different fill patterns) and by e4m3_value; E2M1
// by fp4x2_decode at each of the four selects (the other bytes filled) and
// by e2m1_value. One workgroup of 256 threads.
__global__ void decode_kernel(float* fp8_hw /*[4][256]*/, float* fp8_sw /*[256]*/,
                              float* fp4_hw /*[4][256][2]*/, float* fp4_sw /*[16]*/) {
  const uint32_t b = threadIdx.x;
  const uint32_t fill[4] = {0x000000u, 0xFFFFFFu, 0x5A3C96u, 0x7F7F7Fu};
#pragma unroll
  for (int f = 0; f < 4; ++f)
    fp8_hw[f * 256 + b] = __builtin_amdgcn_cvt_f32_fp8((int)((fill[f] << 8) | b), 0);
  fp8_sw[b] = e4m3_value(b);
  const uint32_t other = 0xA5A5A5A5u;
  f32x2 v;
  v = fp4x2_decode<0>((other & ~0xFFu) | b);
  fp4_hw[(0 * 256 + b) * 2] = v.x, fp4_hw[(0 * 256 + b) * 2 + 1] = v.y;
  v = fp4x2_decode<1>((other & ~0xFF00u) | (b << 8));
  fp4_hw[(1 * 256 + b) * 2] = v.x, fp4_hw[(1 * 256 + b) * 2 + 1] = v.y;
  v = fp4x2_decode<2>((other & ~0xFF0000u) | (b << 16));
  fp4_hw[(2 * 256 + b) * 2] = v.x, fp4_hw[(2 * 256 + b) * 2 + 1] = v.y;
  v = fp4x2_decode<3>((other & ~0xFF000000u) | (b << 24));
  fp4_hw[(3 * 256 + b) * 2] = v.x, fp4_hw[(3 * 256 + b) * 2 + 1] = v.y;
  if (b < 16) fp4_sw[b] = e2m1_value(b);
}

// FP32 -> BF16 round to nearest even: bf16x2_rne on pattern pairs (hardware
// converter) and bf16_rne on each pattern (integer form).
__global__ void bf16_kernel(uint32_t start, int64_t n2, uint32_t* out_hw, uint16_t* out_sw) {
  for (int64_t t = gtid(); t < n2; t += gstride()) {
    const uint32_t b = start + (uint32_t)(2 * t);
    const float x0 = __uint_as_float(b), x1 = __uint_as_float(b + 1u);
    out_hw[t] = bf16x2_rne(x0, x1);
    out_sw[2 * t] = (uint16_t)bf16_rne(x0);
    out_sw[2 * t + 1] = (uint16_t)bf16_rne(x1);
  }
}

// Reciprocal of a decode scale: the guarded recip_rn and the bare Newton
// form recip_newton.
__global__ void recip_kernel(uint32_t start, int64_t n, float* out_rn, float* out_newton) {
  for (int64_t t = gtid(); t < n; t += gstride()) {
    const float d = __uint_as_float(start + (uint32_t)t);
    out_rn[t] = recip_rn(d);
    out_newton[t] = recip_newton(d);
  }
}

// x / 6: the guarded div6_rn and the bare two-term product div6_two_term.
__global__ void div6_kernel(uint32_t start, int64_t n, float* out_rn, float* out_tt) {
  for (int64_t t = gtid(); t < n; t += gstride()) {
    const float x = __uint_as_float(start + (uint32_t)t);
    out_rn[t] = div6_rn(x);
    out_tt[t] = div6_two_term(x);
  }
}

// The scaled FP4 converter with an arbitrary scale operand: element i is
// converted with scale s[i] (the pair's second value is 0); byte i receives
// the pair's code byte (element i in the low nibble).
__global__ void fp4_scaled_kernel(const float* x, const float* s, int64_t n, uint8_t* out) {
  for (int64_t t = gtid(); t < n; t += gstride()) {
    const uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, x[t], 0.0f, s[t], 0);
    out[t] = (uint8_t)(w & 0xFFu);
  }
}

unsigned grid_for(int64_t n) {
  const int64_t g = (n + kThreads - 1) / kThreads;
  return (unsigned)(g < 1 ? 1 : (g > 65536 ? 65536 : g));
}

int done() { return hipGetLastError() == hipSuccess ? 0 : -3; }

bool run_ok(uint32_t start, int64_t n, int64_t unit) {
  return n > 0 && n % unit == 0 && (uint64_t)start + (uint64_t)n <= (1ull << 32) &&
         start % unit == 0;
}

}  // namespace

extern "C" {

// Each entry point checks its run (n > 0, a multiple of the unit it packs,
// start + n <= 2^32) and returns -1 if it does not hold, else 0 or -3 after
// enqueuing one kernel on `stream`. Output sizes (device memory):
//   probe_fp4_encode  out [n / 2] bytes (two nibbles per byte, pattern order)
//   probe_fp8_encode  out_zero [n], out_self [n] bytes
//   probe_decode      fp8_hw [1024], fp8_sw [256], fp4_hw [2048], fp4_sw [16] floats
//   probe_bf16        out_hw [n / 2] dwords, out_sw [n] halfwords
//   probe_recip       out_rn [n], out_newton [n] floats
//   probe_div6        out_rn [n], out_tt [n] floats
//   probe_fp4_scaled  x [n], s [n] floats in; out [n] bytes
int probe_fp4_encode(uint32_t start, int64_t n, void* out, void* stream) {
  if (!run_ok(start, n, 8) || out == nullptr) return -1;
  hipLaunchKernelGGL(fp4_encode_kernel, dim3(grid_for(n / 8)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), start, n / 8, static_cast<uint32_t*>(out));
  return done();
}

int probe_fp8_encode(uint32_t start, int64_t n, void* out_zero, void* out_self, void* stream) {
  if (!run_ok(start, n, 1) || out_zero == nullptr || out_self == nullptr) return -1;
  hipLaunchKernelGGL(fp8_encode_kernel, dim3(grid_for(n)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), start, n, static_cast<uint8_t*>(out_zero),
                     static_cast<uint8_t*>(out_self));
  return done();
}

int probe_decode(void* fp8_hw, void* fp8_sw, void* fp4_hw, void* fp4_sw, void* stream) {
  if (!fp8_hw || !fp8_sw || !fp4_hw || !fp4_sw) return -1;
  hipLaunchKernelGGL(decode_kernel, dim3(1), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<float*>(fp8_hw), static_cast<float*>(fp8_sw),
                     static_cast<float*>(fp4_hw), static_cast<float*>(fp4_sw));
  return done();
}

int probe_bf16(uint32_t start, int64_t n, void* out_hw, void* out_sw, void* stream) {
  if (!run_ok(start, n, 2) || out_hw == nullptr || out_sw == nullptr) return -1;
  hipLaunchKernelGGL(bf16_kernel, dim3(grid_for(n / 2)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), start, n / 2,
                     static_cast<uint32_t*>(out_hw), static_cast<uint16_t*>(out_sw));
  return done();
}

int probe_recip(uint32_t start, int64_t n, void* out_rn, void* out_newton, void* stream) {
  if (!run_ok(start, n, 1) || out_rn == nullptr || out_newton == nullptr) return -1;
  hipLaunchKernelGGL(recip_kernel, dim3(grid_for(n)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), start, n, static_cast<float*>(out_rn),
                     static_cast<float*>(out_newton));
  return done();
}

int probe_div6(uint32_t start, int64_t n, void* out_rn, void* out_tt, void* stream) {
  if (!run_ok(start, n, 1) || out_rn == nullptr || out_tt == nullptr) return -1;
  hipLaunchKernelGGL(div6_kernel, dim3(grid_for(n)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), start, n, static_cast<float*>(out_rn),
                     static_cast<float*>(out_tt));
  return done();
}

int probe_fp4_scaled(const void* x, const void* s, int64_t n, void* out, void* stream) {
  if (x == nullptr || s == nullptr || out == nullptr || n <= 0) return -1;
  hipLaunchKernelGGL(fp4_scaled_kernel, dim3(grid_for(n)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const float*>(x),
                     static_cast<const float*>(s), n, static_cast<uint8_t*>(out));
  return done();
}

}  // extern "C"

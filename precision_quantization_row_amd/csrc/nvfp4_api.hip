// nvfp4_api.hip -- the C ABI declared in include/nvfp4.h.
//
// Validation happens before anything is enqueued; the host never reads device
// memory (noop, amax and group offsets stay on the device), so every call is
// asynchronous on the caller's stream. The library owns no device memory.
#include <atomic>
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include "nvfp4.h"
#include "nvfp4_launch.h"

namespace nvfp4 {

int num_cus() {
  // per-device cache; calls from several host threads may fill an entry
  // concurrently (with the same value), hence the atomics
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

static bool fused_env_enabled() {
  const char* v = getenv("NVFP4_FUSED_AMAX");
  return !(v != nullptr && strcmp(v, "0") == 0);
}

static bool valid_bound(float b) { return isfinite(b) && b > 0.0f && b <= 448.0f; }

}  // namespace nvfp4

using namespace nvfp4;

extern "C" {

const char* nvfp4_status_string(int status) {
  switch (status) {
    case NVFP4_OK: return "ok";
    case NVFP4_ERR_ARG: return "invalid argument";
    case NVFP4_ERR_UNSUPPORTED: return "unsupported request";
    case NVFP4_ERR_HIP: return "HIP launch failure";
    default: return "unknown status";
  }
}

int nvfp4_amax_path(int in_dtype, int64_t M, int64_t K, int want_row, int want_col, unsigned flags) {
  if (!want_row && !want_col) return 0;
  // rows of whole 16-byte vectors: K % 8 == 0 (BF16), K % 4 == 0 (FP32)
  const int64_t v = in_dtype == NVFP4_BF16 ? 8 : 4;
  const bool fused = want_row && want_col && (in_dtype == NVFP4_BF16 || in_dtype == NVFP4_FP32) &&
                     M > 0 && K > 0 && K % v == 0 && !(flags & NVFP4_FLAG_FORCE_TWO_KERNEL) &&
                     fused_env_enabled();
  return fused ? 1 : 2;
}

int nvfp4_amax_rowcol(const void* x, int in_dtype, int64_t M, int64_t K, float* row_amax,
                      float* col_amax, float* tensor_amax, const float* noop, unsigned flags,
                      void* stream) {
  if (x == nullptr || M < 1 || K < 1) return NVFP4_ERR_ARG;
  if (in_dtype != NVFP4_BF16 && in_dtype != NVFP4_FP32) return NVFP4_ERR_ARG;
  if (!row_amax && !col_amax && !tensor_amax) return NVFP4_ERR_ARG;
  if (flags & ~(unsigned)NVFP4_FLAG_FORCE_TWO_KERNEL) return NVFP4_ERR_ARG;
  if (M > (int64_t)1 << 40 || K > (int64_t)1 << 40) return NVFP4_ERR_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int rc = launch_amax_init(row_amax, M, col_amax, K, tensor_amax, noop, s);
  if (rc) return NVFP4_ERR_HIP;
  int path = nvfp4_amax_path(in_dtype, M, K, row_amax != nullptr, col_amax != nullptr, flags);
  // the fused pass reads 16-byte vectors: an X that is not 16-byte aligned
  // (a view with a storage offset) takes the two-kernel path, which checks
  // alignment itself
  if (path == 1 && (reinterpret_cast<uintptr_t>(x) & 15) != 0) path = 2;
  if (path == 1)
    rc = launch_fused_amax(x, in_dtype, M, K, row_amax, col_amax, noop, s);
  else if (path == 2)
    rc = launch_row_col_amax(x, in_dtype, M, K, row_amax, col_amax, noop, s);
  if (rc) return NVFP4_ERR_HIP;
  if (tensor_amax) {
    rc = launch_tensor_amax(x, in_dtype, M * K, tensor_amax, noop, s);
    if (rc) return NVFP4_ERR_HIP;
  }
  return NVFP4_OK;
}

int nvfp4_group_amax_expand(float* row_amax, int64_t M, const int64_t* group_end, int64_t G,
                            int32_t* status, const float* noop, void* stream) {
  if (row_amax == nullptr || group_end == nullptr || M < 1 || G < 1 || G > 65535) return NVFP4_ERR_ARG;
  return launch_group_expand(row_amax, M, group_end, G, status, noop,
                             static_cast<hipStream_t>(stream))
             ? NVFP4_ERR_HIP
             : NVFP4_OK;
}

int nvfp4_check_group_end(const int64_t* group_end, int64_t G, int64_t M) {
  if (group_end == nullptr || M < 1 || G < 1 || G > 65535) return NVFP4_ERR_ARG;
  int64_t b = 0;
  for (int64_t g = 0; g < G; ++g) {
    const int64_t e = group_end[g];
    if (e < 0 || e > M || e < b || (e != M && e % 16 != 0)) return NVFP4_ERR_ARG;
    b = e;
  }
  return NVFP4_OK;
}

static int quantize_impl(const void* x, int in_dtype, int64_t M, int64_t K, int row_mode,
                         const float* row_amax, int col_mode, const float* col_amax, float bound,
                         uint8_t* q_row, uint8_t* s_row, uint8_t* q_col, uint8_t* s_col,
                         const float* noop, void* stream, int four_six) {
  if (x == nullptr || M < 1 || K < 1) return NVFP4_ERR_ARG;
  if (M > (int64_t)1 << 40 || K > (int64_t)1 << 40) return NVFP4_ERR_ARG;
  if (in_dtype != NVFP4_BF16 && in_dtype != NVFP4_FP32) return NVFP4_ERR_ARG;
  if (!valid_bound(bound)) return NVFP4_ERR_ARG;
  const bool rw = q_row != nullptr || s_row != nullptr;
  const bool cw = q_col != nullptr || s_col != nullptr;
  if (!rw && !cw) return NVFP4_ERR_ARG;
  if (rw) {
    if (!q_row || !s_row || !row_amax) return NVFP4_ERR_ARG;
    if (row_mode != NVFP4_AMAX_TENSOR && row_mode != NVFP4_AMAX_LINE) return NVFP4_ERR_ARG;
  }
  if (cw) {
    if (!q_col || !s_col || !col_amax) return NVFP4_ERR_ARG;
    if (col_mode != NVFP4_AMAX_TENSOR && col_mode != NVFP4_AMAX_LINE &&
        col_mode != NVFP4_AMAX_ROWGROUP)
      return NVFP4_ERR_ARG;
  }
  CastArgs a;
  a.x = x;
  a.in_dtype = in_dtype;
  a.M = M;
  a.K = K;
  a.row_mode = row_mode;
  a.row_amax = row_amax;
  a.col_mode = col_mode;
  a.col_amax = col_amax;
  a.F = bound * 6.0f;
  a.F_inv = 1.0f / a.F;
  a.q_row = rw ? q_row : nullptr;
  a.s_row = rw ? s_row : nullptr;
  a.q_col = cw ? q_col : nullptr;
  a.s_col = cw ? s_col : nullptr;
  a.noop = noop;
  a.four_six = four_six;
  return launch_cast(a, static_cast<hipStream_t>(stream)) ? NVFP4_ERR_HIP : NVFP4_OK;
}

int nvfp4_quantize_transpose(const void* x, int in_dtype, int64_t M, int64_t K, int row_mode,
                             const float* row_amax, int col_mode, const float* col_amax,
                             float bound, uint8_t* q_row, uint8_t* s_row, uint8_t* q_col,
                             uint8_t* s_col, const float* noop, void* stream) {
  return quantize_impl(x, in_dtype, M, K, row_mode, row_amax, col_mode, col_amax, bound, q_row,
                       s_row, q_col, s_col, noop, stream, 0);
}

int nvfp4_quantize_rowcol(const void* x, int in_dtype, int64_t M, int64_t K, float bound,
                          float* row_amax, float* col_amax, uint8_t* q_row, uint8_t* s_row,
                          uint8_t* q_col, uint8_t* s_col, const float* noop, void* stream) {
  if (x == nullptr || M < 1 || K < 1 || row_amax == nullptr || col_amax == nullptr)
    return NVFP4_ERR_ARG;
  if (M > (int64_t)1 << 40 || K > (int64_t)1 << 40) return NVFP4_ERR_ARG;
  if (in_dtype != NVFP4_BF16 && in_dtype != NVFP4_FP32) return NVFP4_ERR_ARG;
  if (!valid_bound(bound)) return NVFP4_ERR_ARG;
  if (!q_row || !s_row || !q_col || !s_col) return NVFP4_ERR_ARG;
  const int rc = nvfp4_amax_rowcol(x, in_dtype, M, K, row_amax, col_amax, nullptr, noop, 0, stream);
  if (rc != NVFP4_OK) return rc;
  return quantize_impl(x, in_dtype, M, K, NVFP4_AMAX_LINE, row_amax, NVFP4_AMAX_LINE, col_amax,
                       bound, q_row, s_row, q_col, s_col, noop, stream, 0);
}

int nvfp4_quantize_4over6(const void* x, int in_dtype, int64_t M, int64_t K, int row_mode,
                          const float* row_amax, int col_mode, const float* col_amax, float bound,
                          uint8_t* q_row, uint8_t* s_row, uint8_t* q_col, uint8_t* s_col,
                          const float* noop, void* stream) {
  return quantize_impl(x, in_dtype, M, K, row_mode, row_amax, col_mode, col_amax, bound, q_row,
                       s_row, q_col, s_col, noop, stream, 1);
}

int nvfp4_quantize_2d(const void* x, int in_dtype, int64_t M, int64_t K, const float* tensor_amax,
                      float bound, uint8_t* q_row, uint8_t* s_row, uint8_t* q_col, uint8_t* s_col,
                      const float* noop, void* stream) {
  if (x == nullptr || tensor_amax == nullptr || M < 1 || K < 1) return NVFP4_ERR_ARG;
  if (M > (int64_t)1 << 40 || K > (int64_t)1 << 40) return NVFP4_ERR_ARG;
  if (in_dtype != NVFP4_BF16 && in_dtype != NVFP4_FP32) return NVFP4_ERR_ARG;
  if (!valid_bound(bound)) return NVFP4_ERR_ARG;
  const bool rw = q_row != nullptr || s_row != nullptr;
  const bool cw = q_col != nullptr || s_col != nullptr;
  if (!rw && !cw) return NVFP4_ERR_ARG;
  if (rw && (!q_row || !s_row)) return NVFP4_ERR_ARG;
  if (cw && (!q_col || !s_col)) return NVFP4_ERR_ARG;
  CastArgs a;
  a.x = x;
  a.in_dtype = in_dtype;
  a.M = M;
  a.K = K;
  a.row_mode = NVFP4_AMAX_TENSOR;
  a.row_amax = tensor_amax;
  a.col_mode = NVFP4_AMAX_TENSOR;
  a.col_amax = tensor_amax;
  a.F = bound * 6.0f;
  a.F_inv = 1.0f / a.F;
  a.q_row = rw ? q_row : nullptr;
  a.s_row = rw ? s_row : nullptr;
  a.q_col = cw ? q_col : nullptr;
  a.s_col = cw ? s_col : nullptr;
  a.noop = noop;
  a.blk2d = 1;
  return launch_cast(a, static_cast<hipStream_t>(stream)) ? NVFP4_ERR_HIP : NVFP4_OK;
}

int nvfp4_quantize_grouped(const void* x, int in_dtype, int64_t T, int64_t K,
                           const int64_t* group_rows, int64_t G, int64_t align, int64_t M_out,
                           float bound, float* row_amax, uint8_t* q_row, uint8_t* s_row,
                           uint8_t* q_col, uint8_t* s_col, const float* noop, void* stream) {
  if (x == nullptr || group_rows == nullptr || row_amax == nullptr) return NVFP4_ERR_ARG;
  if (T < 1 || K < 1 || M_out < 1) return NVFP4_ERR_ARG;
  if (T > (int64_t)1 << 40 || K > (int64_t)1 << 40 || M_out > (int64_t)1 << 40) return NVFP4_ERR_ARG;
  if (T >= (int64_t)0x7FFFFFFF || M_out >= (int64_t)0x7FFFFFFF) return NVFP4_ERR_UNSUPPORTED;
  if (in_dtype != NVFP4_BF16 && in_dtype != NVFP4_FP32) return NVFP4_ERR_ARG;
  if (G < 1) return NVFP4_ERR_ARG;
  if (G > NVFP4_GROUPS_MAX) return NVFP4_ERR_UNSUPPORTED;
  if (align < 16 || align > 4096 || align % 16 != 0) return NVFP4_ERR_ARG;
  if (!valid_bound(bound)) return NVFP4_ERR_ARG;
  const bool rw = q_row != nullptr || s_row != nullptr;
  const bool cw = q_col != nullptr || s_col != nullptr;
  if (!rw && !cw) return NVFP4_ERR_ARG;
  if (rw && (!q_row || !s_row)) return NVFP4_ERR_ARG;
  if (cw && (!q_col || !s_col)) return NVFP4_ERR_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (launch_grouped_amax(x, in_dtype, T, K, group_rows, G, align, M_out, row_amax, noop, s))
    return NVFP4_ERR_HIP;
  CastArgs a;
  a.x = x;
  a.in_dtype = in_dtype;
  a.M = M_out;
  a.K = K;
  a.row_mode = NVFP4_AMAX_LINE;
  a.row_amax = row_amax;
  a.col_mode = NVFP4_AMAX_ROWGROUP;
  a.col_amax = row_amax;
  a.F = bound * 6.0f;
  a.F_inv = 1.0f / a.F;
  a.q_row = rw ? q_row : nullptr;
  a.s_row = rw ? s_row : nullptr;
  a.q_col = cw ? q_col : nullptr;
  a.s_col = cw ? s_col : nullptr;
  a.noop = noop;
  a.grp_rows = group_rows;
  a.grp_G = G;
  a.grp_align = align;
  a.grp_T = T;
  return launch_cast(a, s) ? NVFP4_ERR_HIP : NVFP4_OK;
}

int nvfp4_quantize_dequantize(const void* x, int in_dtype, int64_t M, int64_t K, int row_mode,
                              const float* row_amax, float bound, uint8_t* q_row, uint8_t* s_row,
                              void* y, int out_dtype, const float* noop, void* stream) {
  if (x == nullptr || row_amax == nullptr || y == nullptr || M < 1 || K < 1) return NVFP4_ERR_ARG;
  if (M > (int64_t)1 << 40 || K > (int64_t)1 << 40) return NVFP4_ERR_ARG;
  if (in_dtype != NVFP4_BF16 && in_dtype != NVFP4_FP32) return NVFP4_ERR_ARG;
  if (out_dtype != NVFP4_BF16 && out_dtype != NVFP4_FP32) return NVFP4_ERR_ARG;
  if (row_mode != NVFP4_AMAX_TENSOR && row_mode != NVFP4_AMAX_LINE) return NVFP4_ERR_ARG;
  if (!valid_bound(bound)) return NVFP4_ERR_ARG;
  if ((q_row == nullptr) != (s_row == nullptr)) return NVFP4_ERR_ARG;
  QdqArgs a;
  a.x = x;
  a.in_dtype = in_dtype;
  a.M = M;
  a.K = K;
  a.amax_mode = row_mode;
  a.amax = row_amax;
  a.F = bound * 6.0f;
  a.F_inv = 1.0f / a.F;
  a.q = q_row;
  a.sc = s_row;
  a.y = y;
  a.out_dtype = out_dtype;
  a.noop = noop;
  return launch_qdq(a, static_cast<hipStream_t>(stream)) ? NVFP4_ERR_HIP : NVFP4_OK;
}

int nvfp4_dequantize(const uint8_t* q, const uint8_t* sc, int64_t R, int64_t C, int amax_mode,
                     const float* amax, float bound, void* y, int out_dtype, const float* noop,
                     void* stream) {
  if (q == nullptr || sc == nullptr || amax == nullptr || y == nullptr) return NVFP4_ERR_ARG;
  if (R < 1 || C < 1 || R > (int64_t)1 << 40 || C > (int64_t)1 << 40) return NVFP4_ERR_ARG;
  if (amax_mode != NVFP4_AMAX_TENSOR && amax_mode != NVFP4_AMAX_LINE &&
      amax_mode != NVFP4_AMAX_ROWGROUP)
    return NVFP4_ERR_ARG;
  if (out_dtype != NVFP4_BF16 && out_dtype != NVFP4_FP32) return NVFP4_ERR_ARG;
  if (!valid_bound(bound)) return NVFP4_ERR_ARG;
  DequantArgs a;
  a.q = q;
  a.sc = sc;
  a.R = R;
  a.C = C;
  a.amax_mode = amax_mode;
  a.amax = amax;
  a.F_inv = 1.0f / (bound * 6.0f);
  a.y = y;
  a.out_dtype = out_dtype;
  a.noop = noop;
  return launch_dequant(a, static_cast<hipStream_t>(stream)) ? NVFP4_ERR_HIP : NVFP4_OK;
}

}  // extern "C"

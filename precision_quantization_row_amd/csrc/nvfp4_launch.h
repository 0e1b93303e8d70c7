// nvfp4_launch.h -- host-side launchers shared by the C ABI (nvfp4_api.hip).
// Each returns 0 on success or -3 (NVFP4_ERR_HIP) when the launch failed.
// Arguments are validated by the caller before any of these run.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

// Compute units of the current device (cached per device).
int num_cus();

int launch_amax_init(float* ra, int64_t M, float* ca, int64_t K, float* ta, const float* noop,
                     hipStream_t s);
int launch_fused_amax(const void* x, int in_dtype, int64_t M, int64_t K, float* ra, float* ca,
                      const float* noop, hipStream_t s);
int launch_row_col_amax(const void* x, int in_dtype, int64_t M, int64_t K, float* ra, float* ca,
                        const float* noop, hipStream_t s);
int launch_tensor_amax(const void* x, int in_dtype, int64_t n, float* ta, const float* noop,
                       hipStream_t s);
int launch_group_expand(float* ra, int64_t M, const int64_t* group_end, int64_t G,
                        int32_t* status, const float* noop, hipStream_t s);
// grouped tokens: the group amax of each token group over the group's padded
// rows, 0 past the last group; every row of ra [M_out] is written
int launch_grouped_amax(const void* x, int in_dtype, int64_t T, int64_t K, const int64_t* grows,
                        int64_t G, int64_t align, int64_t M_out, float* ra, const float* noop,
                        hipStream_t s);

struct CastArgs {
  const void* x;
  int in_dtype;  // 0 BF16, 1 FP32
  int64_t M, K;
  int row_mode;
  const float* row_amax;
  int col_mode;
  const float* col_amax;
  float F, F_inv;
  uint8_t *q_row, *s_row, *q_col, *s_col;
  const float* noop;
  // grouped tokens (grp_G > 0): x holds grp_T token rows; output row r is
  // token row token_row(r) or a zero row (padding)
  const int64_t* grp_rows = nullptr;
  int64_t grp_G = 0, grp_align = 16, grp_T = 0;
  // 2-D 16 x 16 blocks (row and column mode TENSOR, one amax)
  int blk2d = 0;
  // four-over-six block scales (1x16 blocks)
  int four_six = 0;
};
int launch_cast(const CastArgs& a, hipStream_t s);

struct DequantArgs {
  const uint8_t* q;
  const uint8_t* sc;
  int64_t R, C;
  int amax_mode;
  const float* amax;
  float F_inv;
  void* y;
  int out_dtype;  // 0 BF16, 1 FP32
  const float* noop;
};
int launch_dequant(const DequantArgs& a, hipStream_t s);

// rowwise quantize and the dequantize of that copy in one pass
struct QdqArgs {
  const void* x;
  int in_dtype;    // 0 BF16, 1 FP32
  int64_t M, K;
  int amax_mode;   // 0 TENSOR, 1 LINE
  const float* amax;
  float F, F_inv;
  uint8_t *q, *sc;  // both or neither
  void* y;
  int out_dtype;   // 0 BF16, 1 FP32
  const float* noop;
};
int launch_qdq(const QdqArgs& a, hipStream_t s);

}  // namespace nvfp4

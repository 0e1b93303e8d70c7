/*
 * nvfp4_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, scalar CPU statement of row-scaled NVFP4 quantize-transpose
 * and its inverse. Only the tests, the smoke check and the CPU-baseline leg of
 * the bench may load this library. The product path (the HIP library) never
 * links, calls or includes anything from here, and this file includes nothing
 * from the product.
 *
 * Sources (the pages):
 *  [P1] TransformerEngine PR "NVFP4: enable row-scaled transpose quantization
 *       for backward" -- summary, sequence diagram, description.
 *  [P2] TransformerEngine PR "row-scaled nvfp4 path: fuse row/col amax into a
 *       single TMA-tiled kernel" -- commit message, flowchart, host-wrapper
 *       review, description.
 *  [P3] torchao PR "Add NVFP4 four-over-six grouped GEMM for MoE training" --
 *       description (group amax expansion, bound-aware scales, padding).
 *  [P4] torchao PR "Add backward overrides and 1x16 weights to NVFP4
 *       four-over-six" -- description (the dequantize expression).
 *
 * Precision: every floating-point step is one IEEE-754 binary32 operation
 * rounded to nearest-even, because [P4] fixes the decode as FP32 with a
 * correctly rounded FP32 reciprocal, and the amax is an FP32 max ([P2]
 * description). Build with -O2 -fno-fast-math -ffp-contract=off on x86-64
 * (SSE arithmetic, no FTZ/DAZ), so subnormals are kept.
 *
 * Where the pages leave a step open, the reading used is written next to it.
 * No blocking, fusion or reordering: each line, then each block of 16, then
 * each element, in the order the definition states. The only parallelism is
 * an OpenMP loop over independent lines, which cannot change any bit.
 *
 * Inputs are finite (NaN and +-inf are outside the contract; asserted).
 */
#include <assert.h>
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_MODE_TENSOR 0   /* one amax for every line: a[0]                  */
#define ORC_MODE_LINE 1     /* one amax per line: a[line]                     */
#define ORC_MODE_ROWGROUP 2 /* block b of a line uses a[16*b] (a group amax  */
                            /* already expanded along the line's positions)   */

/* ---------------------------------------------------------------------------
 * E2M1 (the 4-bit element format named in [P1] review snippets: FP4 e2m1).
 * Magnitude grid for the 3 magnitude bits, in code order. Bit 3 is the sign.
 * ------------------------------------------------------------------------- */
static const double E2M1_GRID[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

float orc_e2m1_value(int code) {
  double m = E2M1_GRID[code & 7];
  return (float)((code & 8) ? -m : m);
}

/* Nearest grid point to v, ties to the even code, values at or past 6
 * saturate to 6 (the nearest finite point), sign bit = sign bit of v (so -0
 * and small negatives that round to zero give code 8). Reading: round-to-
 * nearest-even with saturation; the pages never state a rounding rule.
 *
 * Distances are taken in double. For 0.25 <= |v| < 6 (where ties can happen)
 * v has no bit below 2^-25 and no bit above 2^2, so every difference is exact
 * in 53 bits; for |v| < 0.25 the distance to 0 is |v| itself and every other
 * distance exceeds 0.25. |v| >= 6 is decided before any distance is taken
 * (for huge |v| the rounded distances to 4 and 6 would compare equal). */
uint8_t orc_e2m1_encode(float v) {
  assert(!isnan(v));
  int neg = signbit(v) ? 1 : 0;
  int best = 0;
  if (fabsf(v) >= 6.0f) {
    best = 7;
  } else {
    double m = fabs((double)v);
    double best_d = fabs(m - E2M1_GRID[0]);
    for (int k = 1; k < 8; ++k) {
      double d = fabs(m - E2M1_GRID[k]);
      if (d < best_d || (d == best_d && (k & 1) == 0)) {
        best = k;
        best_d = d;
      }
    }
  }
  return (uint8_t)((neg << 3) | best);
}

/* ---------------------------------------------------------------------------
 * E4M3 (the scale format named in [P1] review snippets: "FP8 e4m3 (or raw
 * uint8 byte)"). Reading: the OCP E4M3FN encoding -- 4 exponent bits, bias 7,
 * 3 mantissa bits, no infinity, 0x7F/0xFF NaN, largest finite 448. Scales are
 * non-negative, so only bytes 0x00..0x7E occur.
 * ------------------------------------------------------------------------- */
float orc_e4m3_value(int byte) {
  int e = (byte >> 3) & 0xF;
  int m = byte & 7;
  double v = (e == 0) ? ldexp((double)m, -9)              /* m/8 * 2^-6 */
                      : ldexp(1.0 + (double)m / 8.0, e - 7);
  return (float)((byte & 0x80) ? -v : v);
}

/* The 127 finite non-negative E4M3 values by byte, filled from
 * orc_e4m3_value once when the library is loaded (so the search below does
 * not recompute them for every input). */
static double E4M3_VALUES[0x7F];
__attribute__((constructor)) static void fill_e4m3_values(void) {
  for (int b = 0; b <= 0x7E; ++b) E4M3_VALUES[b] = (double)orc_e4m3_value(b);
}

/* Nearest of the 127 finite non-negative E4M3 values, ties to the even byte,
 * saturating at 448. s must be >= 0 (scales are magnitudes). s >= 448 is
 * decided first. Below it, for s >= 2^-21 the difference to any value (bits
 * 2^8 .. 2^-9) spans at most 53 bits and is exact in double; for s < 2^-21
 * the distance to 0 is s itself and every other distance is near 2^-9. */
uint8_t orc_e4m3_encode(float s) {
  assert(!isnan(s) && s >= 0.0f);
  if (s >= 448.0f) return 0x7E;
  int best = 0;
  double best_d = INFINITY;
  for (int b = 0; b <= 0x7E; ++b) {
    double d = fabs((double)s - E4M3_VALUES[b]);
    if (d < best_d || (d == best_d && (b & 1) == 0)) {
      best = b;
      best_d = d;
    }
  }
  return (uint8_t)best;
}

/* ---------------------------------------------------------------------------
 * Second-level ("global") encode scale of a line.
 * [P3] description: the second-level scale is "bound-aware" (bound 448 or
 * 256); [P4] description: decode is (scale * amax) * factor_inv with
 * factor_inv a correctly rounded FP32 reciprocal. Reading: factor =
 * RN(bound * 6) (6 = largest E2M1 magnitude), factor_inv = RN(1 / factor),
 * S_enc = RN(factor / a), clamped to FLT_MAX; a == 0 gives 1.0 (every output
 * of such a line is zero whatever S_enc is).
 * ------------------------------------------------------------------------- */
float orc_factor(float bound) { return bound * 6.0f; }
float orc_factor_inv(float bound) { return 1.0f / orc_factor(bound); }

float orc_global_encode_scale(float a, float bound) {
  if (a == 0.0f) return 1.0f;
  float s = orc_factor(bound) / a;
  if (s > FLT_MAX) s = FLT_MAX;
  return s;
}

/* ---------------------------------------------------------------------------
 * One 1x16 block ([P4] description: "1x16" blocks; [P1] summary: the
 * ROW_SCALED path overrides the per-line encode scale of each block).
 *   bamax = max |x_k| over the block's elements (a partial last block uses only
 *           the elements that exist -- reading, the pages are silent on tails)
 *   s32   = RN( RN(bamax / 6) * S_enc )          -- block decode scale in
 *                                                   globally encoded units
 *   byte  = E4M3( min(s32, 448) )                -- stored scale
 *   D     = RN( RN(e4m3(byte) * a) * factor_inv ) -- [P4] decode expression
 *   enc   = D == 0 ? 0 : min(RN(1 / D), FLT_MAX)  -- reading: zero scale => 0
 *   code  = E2M1( RN(x_k * enc) )
 * Op order of s32 / enc is a reading; D is the pages' decode expression, so
 * quantize and dequantize share one FP32 decode scale per block.
 * ------------------------------------------------------------------------- */
/* The scale byte and the encode factor of a block whose max magnitude is
 * bamax, under second-level amax a (the steps s32 .. enc above). */
static float block_scale_to(float bamax, float top, float a, float bound, uint8_t *scale_byte) {
  const float s_enc = orc_global_encode_scale(a, bound);
  const float f_inv = orc_factor_inv(bound);
  float s32 = (bamax / top) * s_enc;
  if (s32 > 448.0f) s32 = 448.0f;
  uint8_t b = orc_e4m3_encode(s32);
  float sq = orc_e4m3_value(b);
  float d = (sq * a) * f_inv;
  float enc = 0.0f;
  if (d != 0.0f) {
    enc = 1.0f / d;
    if (enc > FLT_MAX) enc = FLT_MAX;
  }
  *scale_byte = b;
  return enc;
}

static float block_scale(float bamax, float a, float bound, uint8_t *scale_byte) {
  return block_scale_to(bamax, 6.0f, a, bound, scale_byte);
}

/* The FP32 decode scale of a stored byte (the [P4] expression). */
static float decode_scale(uint8_t byte, float a, float bound) {
  return (orc_e4m3_value(byte) * a) * orc_factor_inv(bound);
}

static void quantize_block(const float *x, int64_t stride, int n, float a,
                           float bound, uint8_t *codes, uint8_t *scale_byte) {
  float bamax = 0.0f;
  for (int k = 0; k < n; ++k) {
    float v = x[(int64_t)k * stride];
    assert(isfinite(v));
    float m = fabsf(v);
    if (m > bamax) bamax = m;
  }
  const float enc = block_scale(bamax, a, bound, scale_byte);
  for (int k = 0; k < n; ++k) codes[k] = orc_e2m1_encode(x[(int64_t)k * stride] * enc);
}

/* ---------------------------------------------------------------------------
 * Four-over-six block scaling ([P3] and [P4] descriptions: the recipe's
 * "four-over-six" quantizer with an MSE choice and the bound-256 second-level
 * scale; the pages name the method and define nothing more). Reading: a block
 * has two candidate scales, the standard one (block max mapped to the largest
 * E2M1 magnitude, 6) and one that maps the block max to 4:
 *   s32 = RN( RN(bamax / 6) * S_enc )   or   RN( RN(bamax / 4) * S_enc ),
 * each through the same byte / D / enc / code steps as above. Each candidate
 * is dequantized as the decoder does it, y_k = RN(e2m1(code_k) * D), and the
 * one with the smaller squared error is kept (the standard one on a tie).
 * The error is taken in binary64: d_k = (double)x_k - (double)y_k, the
 * rounded square d_k * d_k, the squares of elements 0..7 summed in order, of
 * elements 8..15 summed in order, then the two sums added (a short last block
 * uses the elements it has, split the same way). The kept byte decodes
 * through the same expression, so the dequantizer needs no flag.
 * ------------------------------------------------------------------------- */
static double block_sq_error(const float *x, int64_t stride, int n, const uint8_t *codes,
                             float d) {
  double lo = 0.0, hi = 0.0;
  for (int k = 0; k < n; ++k) {
    const float y = orc_e2m1_value(codes[k]) * d;
    const double e = (double)x[(int64_t)k * stride] - (double)y;
    const double e2 = e * e;
    if (k < 8)
      lo = lo + e2;
    else
      hi = hi + e2;
  }
  return lo + hi;
}

static void quantize_block_46(const float *x, int64_t stride, int n, float a, float bound,
                              uint8_t *codes, uint8_t *scale_byte) {
  float bamax = 0.0f;
  for (int k = 0; k < n; ++k) {
    float v = x[(int64_t)k * stride];
    assert(isfinite(v));
    float m = fabsf(v);
    if (m > bamax) bamax = m;
  }
  uint8_t b6, b4, c6[16], c4[16];
  const float enc6 = block_scale_to(bamax, 6.0f, a, bound, &b6);
  const float enc4 = block_scale_to(bamax, 4.0f, a, bound, &b4);
  for (int k = 0; k < n; ++k) {
    c6[k] = orc_e2m1_encode(x[(int64_t)k * stride] * enc6);
    c4[k] = orc_e2m1_encode(x[(int64_t)k * stride] * enc4);
  }
  const double e6 = block_sq_error(x, stride, n, c6, decode_scale(b6, a, bound));
  const double e4 = block_sq_error(x, stride, n, c4, decode_scale(b4, a, bound));
  const int four = e4 < e6;
  *scale_byte = four ? b4 : b6;
  memcpy(codes, four ? c4 : c6, (size_t)n);
}

/* Quantize one line of n elements (element k at x[k*stride]).
 * block_amax[b] is the second-level amax block b uses.
 * Output: ceil(n/2) packed code bytes -- element 2t in the low nibble, 2t+1
 * in the high nibble, a missing last high nibble is 0 (reading; [P3] only says
 * the two nibble lanes exist) -- and ceil(n/16) scale bytes. */
static void quantize_line_impl(const float *x, int64_t n, int64_t stride,
                               const float *block_amax, float bound, int four_six,
                               uint8_t *q, uint8_t *s) {
  const int64_t nblk = (n + 15) / 16;
  memset(q, 0, (size_t)((n + 1) / 2));
  for (int64_t b = 0; b < nblk; ++b) {
    int cnt = (int)((n - 16 * b) < 16 ? (n - 16 * b) : 16);
    uint8_t codes[16];
    if (four_six)
      quantize_block_46(x + 16 * b * stride, stride, cnt, block_amax[b], bound, codes, &s[b]);
    else
      quantize_block(x + 16 * b * stride, stride, cnt, block_amax[b], bound, codes, &s[b]);
    for (int k = 0; k < cnt; ++k) {
      int64_t e = 16 * b + k;
      if (e & 1)
        q[e >> 1] |= (uint8_t)(codes[k] << 4);
      else
        q[e >> 1] |= codes[k];
    }
  }
}

void orc_quantize_line(const float *x, int64_t n, int64_t stride,
                       const float *block_amax, float bound, uint8_t *q,
                       uint8_t *s) {
  quantize_line_impl(x, n, stride, block_amax, bound, 0, q, s);
}

void orc_quantize_line_46(const float *x, int64_t n, int64_t stride,
                          const float *block_amax, float bound, uint8_t *q,
                          uint8_t *s) {
  quantize_line_impl(x, n, stride, block_amax, bound, 1, q, s);
}

/* The second-level amax of block b of a line, by mode. */
static float block_amax_of(int mode, const float *amax, int64_t line, int64_t b) {
  switch (mode) {
    case ORC_MODE_TENSOR: return amax[0];
    case ORC_MODE_LINE: return amax[line];
    default: return amax[16 * b];
  }
}

/* Rowwise copy: line i = row i of X [M][K] (K-contiguous) -> q [M][ceil(K/2)],
 * s [M][ceil(K/16)]. ([P1] sequence diagram: rowwise FP4 feeds fprop.) */
static void quantize_rows_impl(const float *X, int64_t M, int64_t K, int mode,
                               const float *amax, float bound, int four_six, uint8_t *q,
                               uint8_t *s) {
  const int64_t qb = (K + 1) / 2, sb = (K + 15) / 16;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t i = 0; i < M; ++i) {
    float *ba = (float *)malloc((size_t)sb * sizeof(float));
    assert(ba);
    for (int64_t b = 0; b < sb; ++b) ba[b] = block_amax_of(mode, amax, i, b);
    quantize_line_impl(X + i * K, K, 1, ba, bound, four_six, q + i * qb, s + i * sb);
    free(ba);
  }
}

void orc_quantize_rowwise(const float *X, int64_t M, int64_t K, int mode,
                          const float *amax, float bound, uint8_t *q, uint8_t *s) {
  quantize_rows_impl(X, M, K, mode, amax, bound, 0, q, s);
}

void orc_quantize_rowwise_46(const float *X, int64_t M, int64_t K, int mode,
                             const float *amax, float bound, uint8_t *q, uint8_t *s) {
  quantize_rows_impl(X, M, K, mode, amax, bound, 1, q, s);
}

/* Columnwise (transposed) copy: line j = column j of X -> q [K][ceil(M/2)],
 * s [K][ceil(M/16)]. ([P1] summary: the columnwise output is the transpose,
 * consumed by wgrad; its per-column amax has K entries.) */
static void quantize_cols_impl(const float *X, int64_t M, int64_t K, int mode,
                               const float *amax, float bound, int four_six, uint8_t *q,
                               uint8_t *s) {
  const int64_t qb = (M + 1) / 2, sb = (M + 15) / 16;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t j = 0; j < K; ++j) {
    float *ba = (float *)malloc((size_t)sb * sizeof(float));
    assert(ba);
    for (int64_t b = 0; b < sb; ++b) ba[b] = block_amax_of(mode, amax, j, b);
    quantize_line_impl(X + j, M, K, ba, bound, four_six, q + j * qb, s + j * sb);
    free(ba);
  }
}

void orc_quantize_colwise(const float *X, int64_t M, int64_t K, int mode,
                          const float *amax, float bound, uint8_t *q, uint8_t *s) {
  quantize_cols_impl(X, M, K, mode, amax, bound, 0, q, s);
}

void orc_quantize_colwise_46(const float *X, int64_t M, int64_t K, int mode,
                             const float *amax, float bound, uint8_t *q, uint8_t *s) {
  quantize_cols_impl(X, M, K, mode, amax, bound, 1, q, s);
}

/* ---------------------------------------------------------------------------
 * 2-D blocks ([P4] description: the 1x16 weight option mirrors TE's switch
 * that turns 2-D quantization off, so TE's default weight blocks are 2-D; the
 * pages name the option and define nothing more). Reading: a block is a 16 x 16
 * tile of X (rows 16I .., columns 16J .., cut at the matrix edge), its max
 * magnitude gives one scale through the same steps as a 1x16 block, under one
 * per-tensor amax a, and every element of the tile is encoded with that
 * scale. Both copies keep the 1x16 layouts: row r holds the scale of tile
 * (r/16, J) at s_row[r][J], column c the scale of tile (I, c/16) at
 * s_col[c][I], so a tile's byte appears on each of its 16 rows and 16
 * columns, and q_col is the exact transpose of q_row.
 * ------------------------------------------------------------------------- */
void orc_quantize_2d(const float *X, int64_t M, int64_t K, float a, float bound,
                     uint8_t *q_row, uint8_t *s_row, uint8_t *q_col, uint8_t *s_col) {
  const int64_t qrb = (K + 1) / 2, srb = (K + 15) / 16;
  const int64_t qcb = (M + 1) / 2, scb = (M + 15) / 16;
  memset(q_row, 0, (size_t)(M * qrb));
  memset(q_col, 0, (size_t)(K * qcb));
  for (int64_t ti = 0; ti < scb; ++ti) {
    for (int64_t tj = 0; tj < srb; ++tj) {
      const int64_t r0 = 16 * ti, r1 = r0 + 16 < M ? r0 + 16 : M;
      const int64_t c0 = 16 * tj, c1 = c0 + 16 < K ? c0 + 16 : K;
      float tamax = 0.0f;
      for (int64_t r = r0; r < r1; ++r)
        for (int64_t c = c0; c < c1; ++c) {
          assert(isfinite(X[r * K + c]));
          float m = fabsf(X[r * K + c]);
          if (m > tamax) tamax = m;
        }
      uint8_t b;
      const float enc = block_scale(tamax, a, bound, &b);
      for (int64_t r = r0; r < r1; ++r) s_row[r * srb + tj] = b;
      for (int64_t c = c0; c < c1; ++c) s_col[c * scb + ti] = b;
      for (int64_t r = r0; r < r1; ++r)
        for (int64_t c = c0; c < c1; ++c) {
          const uint8_t code = orc_e2m1_encode(X[r * K + c] * enc);
          q_row[r * qrb + c / 2] |= (uint8_t)((c & 1) ? code << 4 : code);
          q_col[c * qcb + r / 2] |= (uint8_t)((r & 1) ? code << 4 : code);
        }
    }
  }
}

/* ---------------------------------------------------------------------------
 * Dequantize ([P4] description: four_over_six_dequantize follows the TE
 * kernel, (scale * amax) * factor_inv, FP32, per-tensor and row-scaled):
 *   y_k = RN( e2m1(code_k) * RN( RN(e4m3(byte) * a) * factor_inv ) )
 * q [R][ceil(C/2)], s [R][ceil(C/16)] -> y [R][C] FP32. A BF16 output is the
 * round-to-nearest-even of this FP32 value (done by the caller).
 * ------------------------------------------------------------------------- */
void orc_dequantize(const uint8_t *q, const uint8_t *s, int64_t R, int64_t C,
                    int mode, const float *amax, float bound, float *y) {
  const int64_t qb = (C + 1) / 2, sb = (C + 15) / 16;
  const float f_inv = orc_factor_inv(bound);
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t r = 0; r < R; ++r) {
    for (int64_t c = 0; c < C; ++c) {
      int64_t b = c / 16;
      float a = block_amax_of(mode, amax, r, b);
      float d = (orc_e4m3_value(s[r * sb + b]) * a) * f_inv;
      uint8_t byte = q[r * qb + c / 2];
      int code = (c & 1) ? (byte >> 4) : (byte & 0xF);
      y[r * C + c] = orc_e2m1_value(code) * d;
    }
  }
}

/* ---------------------------------------------------------------------------
 * amax ([P1] sequence diagram: rowwise amax has M entries, columnwise amax K;
 * [P2] description: an exact max reduction, so every evaluation order gives
 * the same bits).
 * ------------------------------------------------------------------------- */
void orc_amax_rows(const float *X, int64_t M, int64_t K, float *ra) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < M; ++i) {
    float m = 0.0f;
    for (int64_t j = 0; j < K; ++j) {
      float v = fabsf(X[i * K + j]);
      if (v > m) m = v;
    }
    ra[i] = m;
  }
}

void orc_amax_cols(const float *X, int64_t M, int64_t K, float *ca) {
  for (int64_t j = 0; j < K; ++j) ca[j] = 0.0f;
  for (int64_t i = 0; i < M; ++i)
    for (int64_t j = 0; j < K; ++j) {
      float v = fabsf(X[i * K + j]);
      if (v > ca[j]) ca[j] = v;
    }
}

float orc_amax_tensor(const float *X, int64_t n) {
  float m = 0.0f;
  for (int64_t i = 0; i < n; ++i) {
    float v = fabsf(X[i]);
    if (v > m) m = v;
  }
  return m;
}

/* [P3] description: per-tensor grouped activations use per-group global
 * scales; the group amaxes are expanded to a per-row amax vector. Group g
 * holds rows [group_end[g-1], group_end[g]) (group_end[-1] = 0); every row of
 * a group gets the max of the group's row amaxes. */
void orc_group_amax_expand(const float *ra, const int64_t *group_end, int64_t G,
                           float *out) {
  int64_t start = 0;
  for (int64_t g = 0; g < G; ++g) {
    float m = 0.0f;
    for (int64_t i = start; i < group_end[g]; ++i)
      if (ra[i] > m) m = ra[i];
    for (int64_t i = start; i < group_end[g]; ++i) out[i] = m;
    start = group_end[g];
  }
}

/* ---------------------------------------------------------------------------
 * BF16 output of the dequantize ([P4] description: BF16 or FP32 output of the
 * FP32 decode). Reading: the BF16 value nearest to the FP32 value, ties to the
 * even bit pattern (round to nearest even), and past the largest finite BF16
 * the rounding of an unbounded exponent, i.e. to infinity at or beyond the
 * midpoint 2^128 - 2^119. The candidates are x with its low 16 bits cleared
 * (the BF16 value next to x toward zero) and the next BF16 value away from
 * zero; every distance below is exact in double (24-bit values within a
 * factor of two of each other, or 2^128 against a value of exponent 127).
 * NaN is outside the contract (a quiet NaN pattern is returned).
 * ------------------------------------------------------------------------- */
uint16_t orc_bf16_round(float x) {
  uint32_t b;
  memcpy(&b, &x, sizeof b);
  if (isnan(x)) return (uint16_t)((b >> 16) | 0x0040u);
  if (isinf(x)) return (uint16_t)(b >> 16);
  const uint32_t lo = b & 0xFFFF0000u;
  float flo;
  memcpy(&flo, &lo, sizeof flo);
  const double m_lo = fabs((double)flo);
  /* magnitude one BF16 step up; from the largest finite BF16 that is 2^128 */
  const uint32_t hi_mag = (lo & 0x7FFFFFFFu) + 0x00010000u;
  double m_hi;
  if (hi_mag >= 0x7F800000u) {
    m_hi = ldexp(1.0, 128);
  } else {
    float fhi;
    memcpy(&fhi, &hi_mag, sizeof fhi);
    m_hi = (double)fhi;
  }
  const double m = fabs((double)x);
  const double d_lo = m - m_lo, d_hi = m_hi - m;
  const uint16_t p_lo = (uint16_t)(lo >> 16);
  if (d_lo < d_hi) return p_lo;
  if (d_lo > d_hi) return (uint16_t)(p_lo + 1u);
  return (p_lo & 1u) ? (uint16_t)(p_lo + 1u) : p_lo;
}

void orc_bf16_round_array(const float *v, int64_t n, uint16_t *out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_round(v[i]);
}

/* Forms over a run of binary32 bit patterns start, start + 1, ...
 * (start + n <= 2^32), for exhaustive checks of hardware converters and
 * arithmetic shortcuts against the definitions above. Patterns outside a
 * function's domain get a marker the caller masks out: 0xFF for the element
 * encoders (NaN input; negative input for E4M3), the pattern itself for the
 * divisions (negative or NaN input). */
static float bits_to_float(uint32_t u) {
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

void orc_e2m1_encode_bits(uint32_t start, int64_t n, uint8_t *out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    const float v = bits_to_float(start + (uint32_t)i);
    out[i] = isnan(v) ? 0xFF : orc_e2m1_encode(v);
  }
}

void orc_e4m3_encode_bits(uint32_t start, int64_t n, uint8_t *out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    const float v = bits_to_float(start + (uint32_t)i);
    out[i] = (isnan(v) || v < 0.0f || signbit(v)) ? 0xFF : orc_e4m3_encode(v);
  }
}

void orc_bf16_round_bits(uint32_t start, int64_t n, uint16_t *out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_round(bits_to_float(start + (uint32_t)i));
}

/* The block-scale divisions of the definition: RN(x / 6) (step s32 with the
 * standard top 6) and the encode factor min(RN(1 / D), FLT_MAX) for D > 0. */
void orc_div6_bits(uint32_t start, int64_t n, float *out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    const uint32_t u = start + (uint32_t)i;
    const float x = bits_to_float(u);
    out[i] = (isnan(x) || signbit(x)) ? x : x / 6.0f;
  }
}

void orc_recip_bits(uint32_t start, int64_t n, float *out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    const uint32_t u = start + (uint32_t)i;
    const float d = bits_to_float(u);
    if (isnan(d) || signbit(d) || d == 0.0f) {
      out[i] = d;
    } else {
      float r = 1.0f / d;
      if (r > FLT_MAX) r = FLT_MAX;
      out[i] = r;
    }
  }
}

/* Array forms of the element converters, for exhaustive checks. */
void orc_e2m1_encode_array(const float *v, int64_t n, uint8_t *out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e2m1_encode(v[i]);
}

void orc_e4m3_encode_array(const float *v, int64_t n, uint8_t *out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_encode(v[i]);
}

/* Threads the OpenMP loops above use (reported next to oracle timings). */
#ifdef _OPENMP
#include <omp.h>
int orc_max_threads(void) { return omp_get_max_threads(); }
void orc_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
#else
int orc_max_threads(void) { return 1; }
void orc_set_threads(int n) { (void)n; }
#endif

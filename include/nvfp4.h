/*
 * nvfp4.h -- C ABI of libnvfp4.so: row-scaled NVFP4 quantize-transpose on
 * AMD Instinct MI355X (gfx950).
 *
 * What is computed (sources: TransformerEngine PR "NVFP4: enable row-scaled
 * transpose quantization for backward" -- summary and sequence diagram;
 * TransformerEngine PR "row-scaled nvfp4 path: fuse row/col amax into a
 * single TMA-tiled kernel" -- commit message, flowchart, host-wrapper review,
 * description; torchao PR "Add NVFP4 four-over-six grouped GEMM for MoE
 * training" -- description; torchao PR "Add backward overrides and 1x16
 * weights to NVFP4 four-over-six" -- description):
 *
 *   X is an M x K row-major matrix (BF16 or FP32). A "line" is a row of X
 *   (rowwise copy, length K) or a column of X (columnwise / transposed copy,
 *   length M). Each line is cut into 1x16 blocks (the last one may be short).
 *   a      = the line's second-level amax (per tensor, per line, or per group)
 *   S_enc  = a == 0 ? 1 : min(RN(F / a), FLT_MAX),  F = RN(bound * 6)
 *   bamax  = max |x| over the block
 *   byte   = E4M3_RNE(min(RN(RN(bamax / 6) * S_enc), 448))   (stored scale)
 *   D      = RN(RN(e4m3(byte) * a) * F_inv),       F_inv = RN(1 / F)
 *   enc    = D == 0 ? 0 : min(RN(1 / D), FLT_MAX)
 *   code   = E2M1_RNE_SATFINITE(RN(x * enc)), sign bit kept (so -0 -> 0x8)
 *   dequantize: y = RN(e2m1(code) * D)   (BF16 output: RNE of the FP32 y)
 * Every step is one IEEE binary32 operation rounded to nearest even, with
 * subnormals kept. The decode D is the pages' (scale * amax) * factor_inv;
 * the remaining op order, the zero-scale rule and the rounding rules are
 * readings of pages that leave them open.
 *
 * Layouts (all packed, no pitch, no GEMM swizzle):
 *   rowwise codes   q_row [M][ceil(K/2)]  element 2t in the low nibble
 *   rowwise scales  s_row [M][ceil(K/16)] E4M3 bytes
 *   colwise codes   q_col [K][ceil(M/2)]  (the transpose: column j of X)
 *   colwise scales  s_col [K][ceil(M/16)]
 *   A missing last high nibble (odd line length) is written as 0.
 *
 * Conventions for every entry point:
 *   - Pointers are device memory of the current HIP device, owned by the
 *     caller. The library allocates nothing and keeps no device state, so
 *     calls on different streams never share scratch.
 *   - `stream` is a hipStream_t (NULL = the null stream). Calls only enqueue
 *     work; nothing synchronizes and the host never reads device data.
 *   - `noop` is NULL or a device pointer to one float. If *noop == 1.0f when
 *     the kernels run, the call has no observable effect on any buffer
 *     (amax buffers included); any other value runs normally.
 *   - Arguments are validated before anything is enqueued; a rejected call
 *     returns NVFP4_ERR_ARG / NVFP4_ERR_UNSUPPORTED and changes nothing.
 *     A failed launch returns NVFP4_ERR_HIP.
 *   - Inputs must be finite; NaN / +-inf are outside the contract. The
 *     second-level amax must stay below FLT_MAX / 448 so that scale * amax
 *     is finite.
 */
#ifndef NVFP4_H_
#define NVFP4_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NVFP4_OK = 0,
  NVFP4_ERR_ARG = -1,         /* bad pointer, size, enum or bound           */
  NVFP4_ERR_UNSUPPORTED = -2, /* valid request this build cannot serve      */
  NVFP4_ERR_HIP = -3          /* the HIP runtime reported a launch failure  */
} nvfp4_status;

typedef enum { NVFP4_BF16 = 0, NVFP4_FP32 = 1 } nvfp4_dtype;

typedef enum {
  NVFP4_AMAX_TENSOR = 0,  /* amax[0] for every line (per-tensor NVFP4)       */
  NVFP4_AMAX_LINE = 1,    /* amax[line]: row-scaled ([M] rows / [K] columns) */
  NVFP4_AMAX_ROWGROUP = 2 /* transposed copy of grouped tokens: block b of a
                             column uses amax[16*b], an [M] per-row vector of
                             group amaxes (groups must start on 16-row
                             boundaries for this to equal per-group calls)   */
} nvfp4_amax_mode;

enum { NVFP4_FLAG_FORCE_TWO_KERNEL = 1u }; /* skip the fused amax kernel */

/* Which amax kernels nvfp4_amax_rowcol runs for these arguments.
 * Returns 1 for the fused row+column pass, 2 for the separate row / column
 * kernels, 0 when neither vector is requested. Host-only; enqueues nothing.
 * The fused pass runs when both row and column vectors are requested, X's
 * rows are whole 16-byte vectors (K % 8 == 0 for BF16, K % 4 == 0 for
 * FP32), the flag is clear and the environment variable NVFP4_FUSED_AMAX is
 * not "0" (the kill switch of the fused-amax PR description; its gate, BF16
 * with 128-aligned dimensions, is what its TMA tiles need, and this pass
 * has no such need). nvfp4_amax_rowcol also sends an X that is not 16-byte
 * aligned to the separate kernels. Both paths give identical bits (exact
 * max). */
int nvfp4_amax_path(int in_dtype, int64_t M, int64_t K, int want_row, int want_col,
                    unsigned flags);

/* Per-row, per-column and/or per-tensor amax of X (the pre-pass of the
 * two-pass design: fused-amax PR commit message and description; sequence
 * diagram of the row-scaled backward PR).
 *   x           [M][K] BF16 or FP32, 16-byte aligned for the vector paths
 *   row_amax    [M] float or NULL:  row_amax[i] = max_j |x_ij|
 *   col_amax    [K] float or NULL:  col_amax[j] = max_i |x_ij|
 *   tensor_amax [1] float or NULL:  max over all of X
 * At least one output must be non-NULL. Outputs are overwritten (a noop-aware
 * kernel zeroes them on the device, then the reductions publish with atomic
 * max), never accumulated across calls. M, K >= 1. */
int nvfp4_amax_rowcol(const void* x, int in_dtype, int64_t M, int64_t K, float* row_amax,
                      float* col_amax, float* tensor_amax, const float* noop, unsigned flags,
                      void* stream);

/* Group amax expansion for grouped (MoE) tokens (grouped-GEMM PR
 * description: per-group global scales, the group amaxes expanded to a
 * per-row amax vector). In place on row_amax [M]: group g holds rows
 * [group_end[g-1], group_end[g]) with group_end[-1] = 0, and every row of a
 * group receives the max of the group's entries. group_end is a device int64
 * array [G], non-decreasing, last entry <= M; entries are clamped to [0, M]
 * on the device, so a bad array cannot cause an out-of-bounds access. Rows
 * past group_end[G-1] are left unchanged. G >= 1, G <= 65535.
 *   status  device int32 [1] or NULL. Non-NULL: the ends are validated on
 *           the device first (the rules of nvfp4_check_group_end) and
 *           *status receives 0 when they hold, else 1 + the first group
 *           that breaks one; then row_amax is expanded only when *status is
 *           0 and left unchanged otherwise (rejected without a host read).
 *           NULL: no validation; misaligned groups still expand, but mode
 *           ROWGROUP blocks that straddle two groups then mix their amaxes.
 * The group ends stay on the device, so nothing synchronizes. */
int nvfp4_group_amax_expand(float* row_amax, int64_t M, const int64_t* group_end, int64_t G,
                            int32_t* status, const float* noop, void* stream);

/* Host-side validation of group ends the caller holds in host memory
 * (row-scaled backward PR review, on the grouped GEMM's scale checks: a clear
 * error rather than silently wrong results):
 * returns NVFP4_OK when every entry lies in [0, M], the entries are
 * non-decreasing and every entry other than M is a multiple of 16, so that
 * no 1x16 block of the transposed copy straddles a group boundary in mode
 * ROWGROUP; NVFP4_ERR_ARG otherwise (also for G < 1, G > 65535, M < 1 or a
 * NULL pointer). Reads group_end [G] on the host; enqueues nothing. */
int nvfp4_check_group_end(const int64_t* group_end, int64_t G, int64_t M);

/* Quantize X into the rowwise copy, the columnwise (transposed) copy, or
 * both, in one pass over X (row-scaled backward PR summary: the columnwise
 * output is emitted in the same kernel pass with its own per-column amax).
 *   row_mode / row_amax: TENSOR ([1]) or LINE ([M]); used if q_row != NULL
 *   col_mode / col_amax: TENSOR ([1]), LINE ([K]) or ROWGROUP ([M]); used if
 *                        q_col != NULL
 *   bound: the E4M3 scale bound, finite, 0 < bound <= 448 (448 and 256 are
 *          the tested values: grouped-GEMM PR, "bound-aware")
 *   q_row [M][ceil(K/2)] and s_row [M][ceil(K/16)] (both or neither)
 *   q_col [K][ceil(M/2)] and s_col [K][ceil(M/16)] (both or neither)
 * At least one copy must be requested. Every byte of the requested outputs
 * is written (unless noop). */
int nvfp4_quantize_transpose(const void* x, int in_dtype, int64_t M, int64_t K, int row_mode,
                             const float* row_amax, int col_mode, const float* col_amax,
                             float bound, uint8_t* q_row, uint8_t* s_row, uint8_t* q_col,
                             uint8_t* s_col, const float* noop, void* stream);

/* The whole row-scaled quantize in one call: per-row and per-column amax of
 * X, then both copies with mode LINE in both directions (row-scaled backward
 * PR, sequence diagram: the amax pass, then the cast that writes both
 * copies; fused-amax PR, "Performance": the full quantize is what it times).
 * Enqueues exactly what nvfp4_amax_rowcol(x, ..., row_amax, col_amax, NULL,
 * noop, 0, stream) followed by nvfp4_quantize_transpose(x, ..., LINE,
 * row_amax, LINE, col_amax, bound, q_row, s_row, q_col, s_col, noop, stream)
 * would, so the results are theirs byte for byte.
 *   row_amax [M], col_amax [K]: written (the amax vectors)
 *   q_row, s_row, q_col, s_col: as nvfp4_quantize_transpose, all four required
 * Validation, noop and errors as those two calls; every argument is checked
 * before anything is enqueued. */
int nvfp4_quantize_rowcol(const void* x, int in_dtype, int64_t M, int64_t K, float bound,
                          float* row_amax, float* col_amax, uint8_t* q_row, uint8_t* s_row,
                          uint8_t* q_col, uint8_t* s_col, const float* noop, void* stream);

/* Four-over-six block scales (four-over-six grouped-GEMM and backward-
 * overrides PR descriptions: the quantizer is named there together with its
 * MSE choice and its bound-256 second-level scale; nothing more is defined,
 * so this is a reading). Arguments, layouts, modes, validation and noop are
 * those of nvfp4_quantize_transpose. Each 1x16 block gets one of two scales:
 * the standard one (block max mapped to the E2M1 maximum 6) or the one that
 * maps the block max to 4, whichever dequantizes the block with the smaller
 * squared error (summed in binary64: elements 0..7 in order, elements 8..15
 * in order, then the two sums; the max-6 scale on a tie). The chosen byte is
 * an ordinary E4M3 block scale, so nvfp4_dequantize decodes the result
 * unchanged. Bound 256 keeps the max-4 scale of a block that holds the line
 * amax below 448 (6/4 * 256 = 384). Both copies requested: one launch per
 * copy (X is read once for each); it computes both candidates per block. */
int nvfp4_quantize_4over6(const void* x, int in_dtype, int64_t M, int64_t K, int row_mode,
                          const float* row_amax, int col_mode, const float* col_amax, float bound,
                          uint8_t* q_row, uint8_t* s_row, uint8_t* q_col, uint8_t* s_col,
                          const float* noop, void* stream);

/* 2-D 16 x 16 blocks (backward-overrides PR description: its 1x16 weight
 * option mirrors TE's switch that turns 2-D weight quantization off, so 2-D
 * blocks are TE's default for weights; the pages define nothing more). One
 * scale per 16 x 16 tile of X, from the tile's max magnitude through the
 * same steps as a 1x16 block, under the per-tensor amax tensor_amax[0]
 * (device float, e.g. from nvfp4_amax_rowcol). Tiles at the matrix edge use
 * the elements that exist. The outputs keep the 1x16 layouts of
 * nvfp4_quantize_transpose: each tile's scale byte is written on its 16 rows
 * (s_row) and its 16 columns (s_col), and q_col is the exact transpose of
 * q_row, so nvfp4_dequantize in mode TENSOR decodes either copy.
 *   q_row [M][ceil(K/2)] and s_row [M][ceil(K/16)] (both or neither)
 *   q_col [K][ceil(M/2)] and s_col [K][ceil(M/16)] (both or neither)
 * At least one copy must be requested. */
int nvfp4_quantize_2d(const void* x, int in_dtype, int64_t M, int64_t K, const float* tensor_amax,
                      float bound, uint8_t* q_row, uint8_t* s_row, uint8_t* q_col, uint8_t* s_col,
                      const float* noop, void* stream);

/* Grouped tokens, padded on the way in, in one call (grouped-GEMM PR
 * description: ragged token groups zero-padded to an alignment before
 * quantization, per-group global scales from each group's amax expanded to
 * its rows, so that the call equals quantizing each group on its own;
 * padded rows quantize to zero codes). The group sizes stay on the device
 * and no pointer lists are involved, so the call has a fixed shape for a
 * captured graph.
 *   x          [T][K] BF16 or FP32: the G groups back to back (group g holds
 *              group_rows[g] rows); token rows past the groups are ignored,
 *              and group rows past T read as zero rows
 *   group_rows [G] device int64, entries >= 0 (negative entries count as
 *              0); 1 <= G <= NVFP4_GROUPS_MAX
 *   align      a multiple of 16 in [16, 4096] (128 in the pages' recipe)
 *   M_out      rows of the padded layout the outputs hold. Group g occupies
 *              rows [P_g, P_{g+1}), P_0 = 0, P_{g+1} = P_g + group_rows[g]
 *              rounded up to align; rows past P_G are zero rows. Rows that
 *              do not fit in M_out are dropped (and take no part in their
 *              group's amax), so size M_out for the worst case
 *              (T + G * (align - 1), rounded up to align).
 *   row_amax   [M_out] float, written: the group amax on every row of a
 *              group, 0 past P_G
 *   q_row [M_out][ceil(K/2)], s_row [M_out][ceil(K/16)] (both or neither)
 *   q_col [K][ceil(M_out/2)], s_col [K][ceil(M_out/16)] (both or neither):
 *              rowwise codes with the per-row amax, transposed codes with
 *              the group amax of each 16-row block (as mode ROWGROUP)
 * At least one copy must be requested. T and M_out must be below 2^31 - 1
 * (NVFP4_ERR_UNSUPPORTED otherwise). */
#define NVFP4_GROUPS_MAX 256
int nvfp4_quantize_grouped(const void* x, int in_dtype, int64_t T, int64_t K,
                           const int64_t* group_rows, int64_t G, int64_t align, int64_t M_out,
                           float bound, float* row_amax, uint8_t* q_row, uint8_t* s_row,
                           uint8_t* q_col, uint8_t* s_col, const float* noop, void* stream);

/* Dequantize one packed copy (backward-overrides PR description: the inverse
 * (scale * amax) * factor_inv with a correctly rounded FP32 reciprocal,
 * per-tensor and row-scaled, BF16 or FP32 output).
 *   q [R][ceil(C/2)], sc [R][ceil(C/16)]: a rowwise copy (R = M, C = K) or a
 *       columnwise copy (R = K, C = M)
 *   amax_mode / amax: TENSOR ([1]), LINE ([R]) or ROWGROUP ([C])
 *   y [R][C] of out_dtype (NVFP4_BF16 or NVFP4_FP32).
 * Scale bytes are E4M3FN values as nvfp4_quantize_transpose writes them
 * (0x00-0x7E); a byte with the sign bit set decodes to the negative scale.
 * 0x7F and 0xFF are the format's NaN encodings and are outside the contract
 * (the output for their blocks is unspecified). */
int nvfp4_dequantize(const uint8_t* q, const uint8_t* sc, int64_t R, int64_t C, int amax_mode,
                     const float* amax, float bound, void* y, int out_dtype, const float* noop,
                     void* stream);

/* Rowwise quantize and the dequantize of that copy in one pass over X
 * (backward-overrides PR description: the "dequantized" policy keeps the
 * rowwise fprop codes and scales and runs the backward GEMMs in BF16 on their
 * dequantization). Equal to nvfp4_quantize_transpose (rowwise copy only)
 * followed by nvfp4_dequantize of that copy, with X read once.
 *   row_mode / row_amax: TENSOR ([1]) or LINE ([M])
 *   q_row [M][ceil(K/2)], s_row [M][ceil(K/16)]: both or neither (NULL:
 *          only the dequantized operand is written)
 *   y [M][K], out_dtype BF16 (round to nearest even of the FP32 value) or
 *          FP32 */
int nvfp4_quantize_dequantize(const void* x, int in_dtype, int64_t M, int64_t K, int row_mode,
                              const float* row_amax, float bound, uint8_t* q_row, uint8_t* s_row,
                              void* y, int out_dtype, const float* noop, void* stream);

/* Human-readable name of a status code (static storage). */
const char* nvfp4_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H_ */

/*
 * dsa_row_topk.h -- C ABI of the cooperative per-row top-k for very long rows
 * and very large k on MI355X (gfx950).
 *
 * The report on vllm PR #56628 (key source) names persistent_topk and
 * cooperative_topk as consumers of the masked decode logits that bound their
 * scan by the same per-row ends as the mask; vllm PR #57459 (Summary) states
 * that the row top-k takes those bounds.  This is that row top-k when a row
 * is far longer than one workgroup scans quickly (a million columns and
 * beyond) or k is large:
 *   per row r: s = starts[r / starts_repeat] (starts NULL: 0),
 *   e' = min(ends[r / ends_repeat], width), L = max(0, e' - s) (s < 0: empty);
 *   out[r, 0:min(k, L)) = the min(k, L) columns of [s, e') with the largest
 *   values (float order, -0 below +0), ties to the lower column, ascending
 *   absolute column ids; out[r, min(k, L):k) = -1.
 * It equals dsa_topk(DSA_TOPK_TOKENS) with block_ids NULL and k_tokens = k.
 *
 * Layout: logits fp32 device view [rows, width], element (r, c) at
 * logits[r * row_stride + c * col_stride]; starts/ends int32 device arrays;
 * out int32 device [rows, k], contiguous, fully written.  Every fp32 value is
 * ranked by the order-preserving key (u >= 2^31 ? ~u : u | 2^31 on its bits):
 * infinities rank as values, a NaN ranks by its bit pattern.
 *
 * The context owns a workspace of (66816 + 12 + P (269 + 2 seg)) words per
 * row, P pieces per row fixed at init from the shape and the device's CU
 * count and seg (list entries per piece) about 4 k / P + 256 (it does not grow
 * with the row length).  dsa_row_topk enqueues five launches on `stream`
 * (three digit passes, the placement of every piece's output, the emit); the
 * second pass also lists each piece's keys from the first digit's bin up when
 * they fit, and the later launches then work on those lists instead of
 * reading the row again.  It allocates nothing, never synchronizes and can be
 * captured in a HIP graph.  Calls on one context must be ordered on one
 * stream.  Returns
 * DSA_OK or a negative dsa_status (see dsa_select.h); the message is
 * dsa_row_topk_last_error().
 */
#ifndef DSA_ROW_TOPK_H
#define DSA_ROW_TOPK_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "dsa_select.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct dsa_topk_shape {
  int32_t rows;          /* >= 0 */
  int32_t k;             /* >= 1 (may exceed the width) */
  int64_t width;         /* >= 0, < 2^31 */
  int64_t row_stride;    /* >= 1 */
  int64_t col_stride;    /* >= 1 */
  int32_t starts_repeat; /* >= 1 */
  int32_t ends_repeat;   /* >= 1 */
} dsa_topk_shape;

typedef struct dsa_topk_ctx dsa_topk_ctx;

/* Validates the shape, fixes the pieces per row and allocates and zeroes the
 * workspace on `device` (not while capturing). */
int dsa_row_topk_init(const dsa_topk_shape* shape, int device, dsa_topk_ctx** out);

/* Frees the workspace (after the device finished using it). */
int dsa_row_topk_destroy(dsa_topk_ctx* ctx);

/* Pieces per row chosen at init (> 0), or a negative dsa_status. */
int dsa_row_topk_pieces(const dsa_topk_ctx* ctx);

/* The pieces per row and workspace size dsa_row_topk_init would choose for
 * `shape` on a device with `cus` compute units, computed on the host without
 * touching any device (same validation).  Either output may be NULL.
 * Returns DSA_OK or a negative dsa_status. */
int dsa_row_topk_plan(const dsa_topk_shape* shape, int cus, int32_t* pieces,
                      int64_t* workspace_bytes);

int dsa_row_topk(dsa_topk_ctx* ctx, const float* logits, const int32_t* starts,
                 const int32_t* ends, int32_t* out, hipStream_t stream);

const char* dsa_row_topk_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* DSA_ROW_TOPK_H */

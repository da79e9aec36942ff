/*
 * dsa_indexer.h -- C ABI of the fused FP8 indexer-logits producer plus
 * selection on MI355X (gfx950).
 *
 * What it computes follows the page on vllm PR #48726, "Fused DSA indexer
 * Top-k kernel (LiteTopk)" (Motivation; "LiteTopK: fused indexer scoring and
 * TopK"): the prefill indexer scores every query/key pair with an FP8
 * multi-query product and selects per query row, and the fused form never
 * stores the [queries, keys] score matrix.  The score (the page names it, the
 * formula is the DSA indexer's):
 *     logit[t, c] = kscale[c] * sum_h w[t, h] * max(0, q[t, h] . k[c])
 * and on each row's live range [s, e') the selection chain of dsa_select.h
 * ("DSA candidate-block kernels walk each row's live context", vllm PR
 * #57459, Summary): block scores over block_size-wide blocks counted from s
 * with the block holding e'-1 pinned to +inf, the top-k_blocks blocks (ties
 * to the lower id), then the top-k_tokens keys of the row with every column
 * of a dropped block ranked as -inf (ties to the lower column).
 *
 * Layout (device memory, caller-owned):
 *   q       uint8 [queries, heads, head_dim]  OCP FP8 E4M3 codes
 *   k       uint8 [keys, head_dim]            OCP FP8 E4M3 codes
 *   w       float [queries, heads]
 *   kscale  float [keys], or NULL (all 1)
 *   starts  int32, or NULL (all 0): row t reads starts[t / starts_repeat]
 *   ends    int32: row t reads ends[t / ends_repeat]; e' = min(end, keys)
 *   block_ids  int32 [queries, k_blocks]  ids relative to s, ascending, -1 pads
 *   token_ids  int32 [queries, k_tokens]  key positions, ascending, -1 pads
 *   logits_out float [queries, keys], or NULL: when given, each row's logits
 *              over [s, e') are stored there (a testing aid; nothing else of
 *              the buffer is written)
 * q and k must be 16-byte aligned.  E4M3 NaN codes (0x7F, 0xFF) are outside
 * the input contract.  Arithmetic: the FP8 products are summed by the matrix
 * cores in fp32, the per-head terms w * max(0, .) and their sum in fp32, and
 * the key scale is applied last.
 *
 * Limits: head_dim 128; heads 16, 32 or 64; block_size 1, 2, 4, 8 or 16;
 * k_blocks <= 512; when k_blocks * block_size > k_tokens, k_tokens <= 512.
 * Beyond them DSA_ERR_UNSUPPORTED.  The call is asynchronous on `stream`,
 * allocates nothing, keeps no state between calls and can be captured in a
 * HIP graph; its per-row candidate buffer lives in on-chip memory, so the
 * workspace does not grow with the number of keys.  Returns DSA_OK or a
 * negative dsa_status (message: dsa_indexer_last_error()).
 */
#ifndef DSA_INDEXER_H
#define DSA_INDEXER_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "dsa_select.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct dsa_indexer_shape {
  int32_t queries;        /* >= 0 */
  int32_t heads;          /* 16, 32 or 64 */
  int32_t head_dim;       /* 128 */
  int32_t block_size;     /* 1, 2, 4, 8 or 16 */
  int32_t k_blocks;       /* 1..512 */
  int32_t k_tokens;       /* >= 1 */
  int64_t keys;           /* >= 0, < 2^31 */
  int32_t starts_repeat;  /* >= 1 */
  int32_t ends_repeat;    /* >= 1 */
} dsa_indexer_shape;

int dsa_indexer_select(const dsa_indexer_shape* shape, int device, const uint8_t* q,
                       const uint8_t* k, const float* w, const float* kscale,
                       const int32_t* starts, const int32_t* ends, int32_t* block_ids,
                       int32_t* token_ids, float* logits_out, hipStream_t stream);

/* Text of the last dsa_indexer_select error on the calling thread ("" if none). */
const char* dsa_indexer_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* DSA_INDEXER_H */

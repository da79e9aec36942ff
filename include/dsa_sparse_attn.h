/*
 * dsa_sparse_attn.h -- C ABI of the sparse attention over each query row's
 * selected tokens on MI355X (gfx950).
 *
 * The page on vllm PR #57273 ("Qwen4Exp QSA: sm_90 tuning table", Purpose)
 * describes the consumer of the 2048 selected tokens per query: grouped-query
 * attention over those tokens alone, read from a paged bf16 K/V cache, split
 * over several programs and merged, with a fused output gate; the page on
 * vllm PR #48726 ("LiteDSA: grouped masked sparse attention") requires each
 * query to attend exactly its own selected set and reports the log-sum-exp.
 * Per query row r and query head h (kv head g = h / group):
 *   P(r)  = the row's token ids that are >= 0 (positions of sequence
 *           n = r / rows_per_seq), each mapped to a cache slot:
 *           slot = page_table[n * pages_per_seq + pos / page_size] * page_size
 *                  + pos % page_size   (page_table NULL: slot = pos);
 *   s_j   = sm_scale * dot(q[r, h, :], K[slot_j, g, :]);
 *   lse   = ln sum_j exp(s_j);  o = sum_j exp(s_j - lse) * V[slot_j, g, :];
 *   out[r, h, :] = o * sigmoid(gate[r, h, :])   (gate NULL: o);
 *   lse[r, h] = lse.  An empty P(r) gives out = 0 and lse = -inf.
 * Ids whose page lies beyond the table, whose table entry is negative or
 * whose slot is not below num_slots are skipped and set status bit 0.
 *
 * Layout (all device pointers, caller-owned): q, gate, out bf16 [rows,
 * kv_heads * group, head_dim] contiguous; k_cache and v_cache bf16, element
 * (slot, g, d) at slot * slot_stride + g * head_stride + d (strides in
 * elements, multiples of 8, pointers 16-byte aligned); token_ids int32 [rows,
 * k_tokens] contiguous (the selection's output: ascending, -1 pads, though any
 * order works); page_table int32 [num_seqs, pages_per_seq] or NULL; lse fp32
 * [rows, kv_heads * group] or NULL.  Inputs are bf16 codes, computation is
 * fp32 with bf16 products on the matrix cores (the softmax weights are
 * rounded to bf16 before they multiply V), the output is rounded to bf16.
 *
 * Limits: head_dim 128 or 256; group >= 1 and kv_heads >= 1 with kv_heads *
 * group <= 2^20; page_size a power of two; num_slots < 2^31.  Union mode also
 * needs union_rows <= 16, union_rows * k_tokens <= 32768 and rows_per_seq %
 * union_rows == 0.
 *
 * Head tiles: one matrix product covers 16 (row, query head) pairs, so each
 * kv head's group of query heads is cut into T equal tiles, T the smallest
 * divisor of group with union_rows * group / T <= 16 (union_rows counts 1
 * outside union mode): T = 1 up to 16 heads per kv head, 8 for 128.  The
 * tiles of one kv head run side by side in one workgroup where they fit
 * (up to four tiles), so its K and V rows are read once from memory for all
 * of them.
 *
 * Union mode (shape.union_rows >= 2; the page on vllm PR #48726, "LiteDSA:
 * grouped masked sparse attention", packs neighbouring queries into one
 * matrix tile and runs one product over the union of their selected
 * positions, each query still attending exactly its own set): consecutive rows are taken in groups of
 * union_rows (all of one sequence, so union_rows divides rows_per_seq; the
 * last group may be shorter).  The group's ids are merged into one list of
 * distinct positions, each with a bit per row that selected it, and every
 * union token's K and V rows are read for all union_rows * group (row, head)
 * pairs at once, union_rows * group / T of them per matrix tile.  The result is the attention above with each row's ids taken as a
 * set: an id a row lists twice counts once (ids from the selection are
 * distinct, so the two modes then agree).  Union mode issues two launches
 * (the union, then the attention) and holds union_rows * k_tokens 8-byte
 * entries per group in the workspace.
 *
 * dsa_sparse_attn enqueues its launches on `stream`, allocates nothing, never
 * synchronizes and can be captured in a HIP graph.  When a row's tokens are
 * split over several workgroups (chunks > 1), each writes a partial
 * (maximum, sum, unnormalised output) to the context's workspace and the last
 * one to arrive merges them; the arrival counters reset themselves, so calls
 * on one context must be ordered on one stream.  Returns DSA_OK or a negative
 * dsa_status (see dsa_select.h); the message is dsa_sparse_attn_last_error().
 */
#ifndef DSA_SPARSE_ATTN_H
#define DSA_SPARSE_ATTN_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#include "dsa_select.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct dsa_attn_shape {
  int32_t rows;           /* query rows, >= 0 */
  int32_t kv_heads;       /* >= 1 */
  int32_t group;          /* query heads per kv head, >= 1 */
  int32_t head_dim;       /* 128 or 256 */
  int32_t k_tokens;       /* ids per row, >= 1 */
  int32_t rows_per_seq;   /* rows sharing one page-table row, >= 1 */
  int32_t page_size;      /* power of two, >= 1 (ignored without a table) */
  int32_t pages_per_seq;  /* page-table row length (ignored without a table) */
  int64_t num_slots;      /* cache slots, < 2^31 */
  int64_t k_slot_stride, k_head_stride;   /* elements */
  int64_t v_slot_stride, v_head_stride;   /* elements */
  int32_t chunks;         /* workgroups per (row or union group, workgroup's head tiles); 0 = chosen at init */
  int32_t union_rows;     /* 0 or 1: each row on its own; >= 2: union mode (see above) */
} dsa_attn_shape;

typedef struct dsa_attn_ctx dsa_attn_ctx;

/* Validates the shape, fixes the chunks per (row, kv head) from the shape
 * and the device's CU count, and allocates and zeroes the workspace on
 * `device` (not while capturing). */
int dsa_sparse_attn_init(const dsa_attn_shape* shape, int device, dsa_attn_ctx** out);

/* Frees the workspace (after the device finished using it). */
int dsa_sparse_attn_destroy(dsa_attn_ctx* ctx);

/* The launch plan of a shape on a device with `cus` compute units, computed
 * on the host without touching any device (the same validation and choices
 * as dsa_sparse_attn_init; for sizing ahead of time and for host-side tests).
 * Returns DSA_OK or a negative dsa_status. */
typedef struct dsa_attn_plan_info {
  int32_t head_tiles;       /* T: equal parts of each kv head's group (see Head tiles) */
  int32_t heads_per_tile;   /* group / T */
  int32_t tiles_per_group;  /* head tiles per workgroup: 1, 2 or 4 */
  int32_t chunks;           /* workgroups per (row or union group, workgroup's tiles) */
  int32_t grid_groups;      /* workgroups of the attention launch */
  int64_t workspace_bytes;
} dsa_attn_plan_info;
int dsa_sparse_attn_plan(const dsa_attn_shape* shape, int cus, dsa_attn_plan_info* info);

/* Chunks per (row, workgroup's head tiles), or per (union group, workgroup's
 * head tiles) in union mode, chosen at init (> 0), or a negative dsa_status. */
int dsa_sparse_attn_chunks(const dsa_attn_ctx* ctx);

int dsa_sparse_attn(dsa_attn_ctx* ctx, const uint16_t* q, const uint16_t* k_cache,
                    const uint16_t* v_cache, const int32_t* token_ids,
                    const int32_t* page_table, const uint16_t* gate, float sm_scale,
                    uint16_t* out, float* lse, hipStream_t stream);

/* The same attention over fp8 caches ([57273] names bf16 and fp8 K/V): k_cache
 * and v_cache hold OCP E4M3 codes (1 byte per element, same layout and strides
 * in elements, pointers 8-byte aligned) with one scale per tensor, K = e4m3(k)
 * * k_scale and V = e4m3(v) * v_scale.  The codes are converted to bf16
 * exactly on load; k_scale joins the score scale and v_scale the final
 * normalisation, both in fp32.  E4M3 NaN codes are outside the contract.
 * Same context as dsa_sparse_attn (a context may serve both). */
int dsa_sparse_attn_fp8(dsa_attn_ctx* ctx, const uint16_t* q, const uint8_t* k_cache,
                        const uint8_t* v_cache, float k_scale, float v_scale,
                        const int32_t* token_ids, const int32_t* page_table,
                        const uint16_t* gate, float sm_scale, uint16_t* out, float* lse,
                        hipStream_t stream);

/* Sticky status bits of the context (bit 0: some id was not addressable and
 * was skipped).  Synchronizes the device; not for use under capture. */
int dsa_sparse_attn_read_status(dsa_attn_ctx* ctx, uint32_t* status);

/* Clears the status word (synchronous). */
int dsa_sparse_attn_reset_status(dsa_attn_ctx* ctx);

const char* dsa_sparse_attn_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* DSA_SPARSE_ATTN_H */

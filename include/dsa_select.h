/*
 * dsa_select.h -- C ABI of the MI355X (gfx950) library for DeepSeek-style
 * sparse attention (DSA) decode-time candidate selection.
 *
 * What the operations compute is stated by the pages
 *   [P1] "DSA candidate-block kernels walk each row's live context"
 *        (vllm PR #57459), Summary;
 *   [P4] report on vllm PR #56628, "Stride the DSA decode candidate mask over
 *        the live context", sections on implementation and key source.
 *
 * Data model (all indices in elements):
 *   logits   fp32 view [rows, width]; element (r, c) lives at
 *            logits[r * row_stride + c * col_stride].  A col_stride of 2 is
 *            the "packed column" view of [P4]; the interleaved elements are
 *            never read or written.
 *   starts   int32, nullable (NULL: every row starts at 0).  Row r reads
 *            starts[r / starts_repeat].
 *   ends     int32, row r reads ends[r / ends_repeat].
 *   Per row: s = start, e' = min(end, width), L = max(0, e' - s),
 *   nlb = ceil(L / block_size) live blocks, counted from s: block b covers
 *   columns [s + b*B, min(s + (b+1)*B, e')).  A row with L == 0 or s < 0 is
 *   empty: its outputs are all -1 and nothing is written for it (s < 0 also
 *   raises the status word, see dsa_read_status).
 *   Order: the float order, with -0 below +0 (order-preserving uint32 key of
 *   the fp32 bits); equal values go to the lower index.  Values inside
 *   [s, e') are expected to be finite (no NaN, no +/-inf).
 *
 * Every entry point is asynchronous on the given stream, never allocates,
 * never synchronizes, launches a grid fixed by the shape given to
 * dsa_select_init (only loop trip counts depend on starts/ends), and can be
 * captured in a HIP graph.  Calls that share one context must be ordered on
 * one stream (a context's workspace is used by its fused calls).
 *
 * Return value: DSA_OK (0) or a negative dsa_status; no call throws.  The
 * message of the last failure on the calling thread is dsa_last_error().
 * rows == 0 or width == 0 makes every compute call a successful no-op.
 * All buffers are owned by the caller, except the context workspace, which
 * the library allocates at init and frees at destroy.
 */
#ifndef DSA_SELECT_H
#define DSA_SELECT_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dsa_status {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARG = -1,  /* null pointer, bad size or stride, bad mode */
  DSA_ERR_UNSUPPORTED = -2,  /* a size beyond the library's limits */
  DSA_ERR_CAPTURING = -3,    /* dsa_reset_workspace on a capturing stream */
  DSA_ERR_HIP = -4,          /* a HIP runtime call failed (message has it) */
  DSA_ERR_DESTROYED = -5     /* the context was destroyed */
} dsa_status;

enum { DSA_TOPK_BLOCKS = 0, DSA_TOPK_TOKENS = 1 };
enum {
  DSA_WRITE_MASK = 1u,    /* dsa_select_fused: write the mask into logits */
  DSA_TWO_LAUNCHES = 2u   /* dsa_select_fused: run long rows' second pass as a
                             second launch instead of waiting in the first */
};

typedef struct dsa_shape {
  int32_t rows;          /* >= 0 */
  int32_t block_size;    /* B >= 1 (candidate_block_size of [P1]) */
  int32_t k_blocks;      /* K_blk >= 1: blocks kept per row */
  int32_t k_tokens;      /* K_tok >= 1: tokens kept per row */
  int64_t width;         /* >= 0, < 2^31 (max_model_len) */
  int64_t row_stride;    /* >= 1; with rows > 1, >= (width-1)*col_stride+1 */
  int64_t col_stride;    /* >= 1 */
  int32_t starts_repeat; /* >= 1 */
  int32_t ends_repeat;   /* >= 1 */
} dsa_shape;

typedef struct dsa_ctx dsa_ctx;

/*
 * Launch geometry chosen at init (for benchmarks and tests).  Rows longer
 * than one workgroup's share are split either per row (P workgroups each) or,
 * when rows <= min(CUs / 2, 256), by a balanced split in which equal ranges of the
 * concatenated long rows go to the workgroups of each pass (then
 * programs_per_row is 0).
 */
typedef struct dsa_launch_info {
  int32_t programs_per_row;   /* P of the per-row split; 0 for the balanced split */
  int32_t threads_per_group;
  int32_t grid_groups;        /* workgroups of the fused launch (one-launch mode) */
  int32_t small_row_blocks;   /* rows with nlb <= this run in one workgroup */
  int64_t workspace_bytes;
  int32_t fused_launches;     /* kernel launches per dsa_select_fused call */
} dsa_launch_info;

/*
 * dsa_select_init -- [P1] Summary (the launch shape is derived from the
 * tensor shapes alone and stays fixed for graph replay while the work follows
 * each row's [start, end)); [P4] implementation (a fixed grid keeps graph
 * capture valid).  Validates the shape, chooses the launch geometry from the
 * shape and the device's CU count only, and allocates and zeroes the
 * workspace on `device` (so call it outside stream capture).  On success *out
 * owns the workspace until dsa_select_destroy.  Errors: DSA_ERR_INVALID_ARG
 * for a null pointer or a bad size, stride or repeat; DSA_ERR_UNSUPPORTED
 * for width >= 2^31 or k_blocks + k_tokens > 131072; DSA_ERR_HIP when the
 * allocation fails (nothing is then left allocated and *out is NULL).
 */
int dsa_select_init(const dsa_shape* shape, int device, dsa_ctx** out);

/* dsa_select_destroy -- free the workspace (after the device finished using it). */
int dsa_select_destroy(dsa_ctx* ctx);

int dsa_select_query(const dsa_ctx* ctx, dsa_launch_info* info);

/*
 * dsa_select_plan -- the launch geometry and workspace size that
 * dsa_select_init would choose for `shape` on a device with `cus` compute
 * units, computed on the host without touching any device (for sizing a
 * workspace ahead of time and for host-side tests).  The shape is validated
 * as dsa_select_init validates it.  Returns DSA_OK or a negative dsa_status.
 */
int dsa_select_plan(const dsa_shape* shape, int cus, dsa_launch_info* info);

/*
 * dsa_block_scores -- [P1] Summary (block scoring over the row's range, the
 * newest-block pin).  For every row and every live block b < nlb:
 *   scores[r * nblocks + b] = the block's live value with the largest key,
 *   and scores[r * nblocks + nlb - 1] = +inf (the block holding column e'-1).
 * nblocks = ceil(width / block_size); entries b >= nlb are NOT written (the
 * caller pre-fills them, e.g. with -inf, once).  scores is device fp32
 * [rows, nblocks], contiguous.
 */
int dsa_block_scores(dsa_ctx* ctx, const float* logits, const int32_t* starts,
                     const int32_t* ends, float* scores, hipStream_t stream);

/*
 * dsa_topk -- per-row top-k with ties to the lower index; output ascending,
 * padded with -1, into out [rows, K] (device int32, contiguous).
 *   mode DSA_TOPK_BLOCKS: src = scores [rows, nblocks] as written by
 *     dsa_block_scores; ranks scores[r, 0:nlb) and keeps K = k_blocks,
 *     min(K, nlb) ids relative to s ([P1]: the block top-k inside
 *     select_candidate_blocks).  block_ids must be NULL.
 *   mode DSA_TOPK_TOKENS: src = logits (the view above); ranks the row's
 *     columns [s, e') as masked by block_ids ([P1]: the row top-k bounds its
 *     scan by the same ends): a column keeps its value if its block is listed
 *     in block_ids[r] (int32 [rows, k_blocks], ascending ids in [0, nlb), -1
 *     pads), else it ranks as -inf.  block_ids NULL ranks the row as it is.
 *     Keeps K = k_tokens, min(K, L) absolute column ids.
 */
int dsa_topk(dsa_ctx* ctx, int mode, const float* src, const int32_t* starts,
             const int32_t* ends, const int32_t* block_ids, int32_t* out,
             hipStream_t stream);

/*
 * dsa_candidate_mask -- [P4] implementation and key source (strided mask over
 * the live range), [P1] Summary (no writes at or past end).  In place: every
 * column in [s, e') whose block is not listed in block_ids[r] (int32
 * [rows, k_blocks]; -1 and ids outside [0, nlb) are ignored) becomes -inf.
 * Nothing outside [s, e') is read or written.
 */
int dsa_candidate_mask(dsa_ctx* ctx, float* logits, const int32_t* starts,
                       const int32_t* ends, const int32_t* block_ids,
                       hipStream_t stream);

/*
 * dsa_select_fused -- [P1] Summary (select_candidate_blocks scores the blocks
 * of the row's range with the newest-block pin and feeds apply_candidate_mask;
 * the row top-k bounds its scan by the same ends); [P4] implementation and
 * key source (the mask strided over [start, end), flags from the candidate
 * blocks).  The whole chain in one pass over the live logits:
 * block scores (with the pin) -> top-k_blocks blocks -> mask -> top-k_tokens
 * tokens of the masked row.  Outputs equal those of dsa_block_scores,
 * dsa_topk(BLOCKS), dsa_candidate_mask, dsa_topk(TOKENS) run in that order:
 *   block_ids [rows, k_blocks] int32 (relative to s), token_ids [rows,
 *   k_tokens] int32 (absolute), scores (nullable) as dsa_block_scores.
 * flags & DSA_WRITE_MASK: write the mask into logits in place; otherwise
 * logits is only read.  flags & DSA_TWO_LAUNCHES: for rows too long for one
 * workgroup, launch the second pass separately instead of having its
 * workgroups wait (time-bounded) in the same launch; results are identical.
 * Uses the context workspace (calls on one context must not overlap).
 */
int dsa_select_fused(dsa_ctx* ctx, float* logits, const int32_t* starts,
                     const int32_t* ends, int32_t* block_ids, int32_t* token_ids,
                     float* scores, uint32_t flags, hipStream_t stream);

/*
 * dsa_select_fused_noalloc -- for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): dsa_select_fused for `shape` on `device` without a context.
 * Same arguments, outputs and flags as dsa_select_fused; the workspace is a
 * library-owned array of 256 MiB per device (held from the first call on that
 * device until the process ends), and the call allocates nothing.  A shape
 * whose workspace would exceed 256 MiB is rejected with DSA_ERR_UNSUPPORTED
 * before anything is launched (dsa_select_query on a context of the shape
 * reports its workspace_bytes).  Each call first clears, on `stream`, the
 * workspace words that must start at zero, then launches the fused kernel.
 * status: nullable device pointer to one uint32 that the caller zeroes; the
 * kernels OR into it the bits described under dsa_read_status (NULL: not
 * reported).  Every call on one device shares that device's array: calls
 * that overlap in time on one device (on different streams, or from several
 * threads) race and give undefined results; order them on one stream.
 */
int dsa_select_fused_noalloc(const dsa_shape* shape, int device, float* logits,
                             const int32_t* starts, const int32_t* ends,
                             int32_t* block_ids, int32_t* token_ids, float* scores,
                             uint32_t flags, uint32_t* status, hipStream_t stream);

/*
 * dsa_read_status -- copy the context's device status word to *out after
 * synchronizing the context's device.  Bit 0: a row had start < 0 (treated as
 * empty).  Bit 1: a second-pass wait gave up after its time limit (the row's
 * outputs are then incomplete).  Bit 2: a fused call found its workspace
 * inconsistent, which only a call cut short can leave behind.  0 means no
 * contract violation since init or the last reset.  The calls return before
 * the device runs, so this word is how a fused call reports a given-up wait:
 * after bit 1 or bit 2 the workspace may hold a partial row state, and the
 * caller must call dsa_reset_workspace before the next call on the context
 * (bit 0 alone needs no reset).
 */
int dsa_read_status(dsa_ctx* ctx, uint32_t* out);

/* dsa_reset_workspace -- re-zero the workspace and status word (not capturable). */
int dsa_reset_workspace(dsa_ctx* ctx, hipStream_t stream);

/* Text of the last error on the calling thread ("" if none). */
const char* dsa_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* DSA_SELECT_H */

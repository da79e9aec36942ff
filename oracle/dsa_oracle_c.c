/*
 * Second CPU oracle for DSA decode-time candidate selection, in plain C.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  The HIP library never
 * calls it and shares no code with it.
 *
 * It states the same chain as oracle/dsa_oracle.py, from the same passages
 * (vllm PR #57459 "DSA candidate-block kernels walk each row's live context",
 * Summary; report on vllm PR #56628 "Stride the DSA decode candidate mask over
 * the live context", implementation and key source), with one difference of
 * method: each top-k is found by threshold selection instead of a full sort.
 * The k-th largest key T is located by quickselect on a copy of the keys;
 * every key above T is kept, then the first (k - #above) keys equal to T in
 * index order.  That is the top-k with ties to the lower index by definition,
 * reached by an algorithm independent of both the full sort of the numpy
 * oracle and the radix select of the GPU kernels.
 *
 * Per row r (all in elements):
 *   s  = starts ? starts[r / starts_repeat] : 0,  e = ends[r / ends_repeat],
 *   e' = min(e, width), L = max(0, e' - s); s < 0 makes the row empty.
 *   Blocks of B columns are counted from s; nlb = ceil(L / B).
 *   score[b] = the live value of block b with the largest order key;
 *   score[nlb - 1] = +inf (the newest block is always kept).
 *   Kept blocks: top-min(K_blk, nlb) scores, ties to the lower block id.
 *   Mask: every live column of a block that is not kept becomes -inf.
 *   Tokens: top-min(K_tok, L) columns of the masked live span, ties to the
 *   lower column.
 * Outputs are ascending and padded with -1; block ids are relative to s,
 * token ids are absolute columns.
 *
 * Rows are split statically over the threads (thread t takes rows
 * t, t + n, t + 2n, ...).  The logits are read from `src`; the mask is
 * written into `dst` (which may be `src`), at the same element offsets.
 */
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define KEY_NEG_INF 0x007FFFFFu   /* order key of -inf */
#define KEY_POS_INF 0xFF800000u   /* order key of +inf */
#define BITS_NEG_INF 0xFF800000u  /* fp32 bits of -inf */

/* Order-preserving key of the fp32 bits: unsigned order of keys is the float
 * order, with -0 below +0. */
static uint32_t key_of_bits(uint32_t u) { return (u & 0x80000000u) ? ~u : (u | 0x80000000u); }
static uint32_t bits_of_key(uint32_t k) { return (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k; }

static uint32_t load_bits(const float* p) {
  uint32_t u;
  memcpy(&u, p, 4);
  return u;
}

/* The k-th largest value (k >= 1) of a[0..n): quickselect, a is reordered. */
static uint32_t kth_largest(uint32_t* a, int64_t n, int64_t k) {
  int64_t lo = 0, hi = n - 1, want = k - 1; /* index in descending order */
  while (lo < hi) {
    /* median of three as the pivot */
    const int64_t mid = lo + (hi - lo) / 2;
    uint32_t x = a[lo], y = a[mid], z = a[hi], piv;
    if ((x >= y && x <= z) || (x <= y && x >= z)) piv = x;
    else if ((y >= x && y <= z) || (y <= x && y >= z)) piv = y;
    else piv = z;
    /* three-way partition, descending: [lo, gt) > piv, [gt, i) == piv, (lt, hi] < piv */
    int64_t gt = lo, i = lo, lt = hi;
    while (i <= lt) {
      if (a[i] > piv) {
        uint32_t t = a[gt]; a[gt] = a[i]; a[i] = t;
        ++gt; ++i;
      } else if (a[i] < piv) {
        uint32_t t = a[lt]; a[lt] = a[i]; a[i] = t;
        --lt;
      } else {
        ++i;
      }
    }
    if (want < gt) hi = gt - 1;
    else if (want > lt) lo = lt + 1;
    else return piv;
  }
  return a[lo];
}

/* keep[i] = 1 for the top-min(k, n) of keys[0..n), ties to the lower index.
 * tmp holds n words of scratch.  Returns the number kept. */
static int64_t top_k_flags(const uint32_t* keys, int64_t n, int64_t k, uint8_t* keep,
                           uint32_t* tmp) {
  if (k > n) k = n;
  if (k <= 0) {
    memset(keep, 0, (size_t)n);
    return 0;
  }
  if (k == n) {
    memset(keep, 1, (size_t)n);
    return n;
  }
  memcpy(tmp, keys, (size_t)n * 4);
  const uint32_t T = kth_largest(tmp, n, k);
  int64_t above = 0;
  for (int64_t i = 0; i < n; ++i) above += keys[i] > T;
  int64_t ties = k - above; /* equal keys taken, lowest index first */
  for (int64_t i = 0; i < n; ++i) {
    if (keys[i] > T) keep[i] = 1;
    else if (keys[i] == T && ties > 0) { keep[i] = 1; --ties; }
    else keep[i] = 0;
  }
  return k;
}

typedef struct {
  const float* src;
  float* dst;
  int64_t rows, width, row_stride, col_stride;
  const int32_t *starts, *ends;
  int32_t starts_repeat, ends_repeat, B, k_blocks, k_tokens, write_mask;
  int32_t* block_ids;   /* [rows, k_blocks] */
  int32_t* token_ids;   /* [rows, k_tokens] */
  float* scores;        /* [rows, nblocks], nullable; only b < nlb written */
  int64_t nblocks;
  int32_t nthreads, repeat;
  int status;
} job_t;

typedef struct {
  job_t* job;
  int32_t t;
} arg_t;

static void one_row(const job_t* j, int64_t r, uint32_t* keys, uint32_t* bkey, uint32_t* tmp,
                    uint8_t* keep_b, uint8_t* keep_t) {
  int32_t* bout = j->block_ids + r * j->k_blocks;
  int32_t* tout = j->token_ids + r * j->k_tokens;
  for (int32_t i = 0; i < j->k_blocks; ++i) bout[i] = -1;
  for (int32_t i = 0; i < j->k_tokens; ++i) tout[i] = -1;
  const int64_t s = j->starts ? (int64_t)j->starts[r / j->starts_repeat] : 0;
  const int64_t e = (int64_t)j->ends[r / j->ends_repeat];
  const int64_t ec = e < j->width ? e : j->width;
  if (s < 0 || ec <= s) return;
  const int64_t L = ec - s, B = j->B;
  const int64_t nlb = (L + B - 1) / B;
  const float* row = j->src + r * j->row_stride;
  float* orow = j->dst + r * j->row_stride;
  for (int64_t c = 0; c < L; ++c) keys[c] = key_of_bits(load_bits(row + (s + c) * j->col_stride));
  /* block scores: max key per block, the newest pinned to +inf */
  for (int64_t b = 0; b < nlb; ++b) {
    uint32_t m = 0;
    const int64_t c1 = (b + 1) * B < L ? (b + 1) * B : L;
    for (int64_t c = b * B; c < c1; ++c) m = keys[c] > m ? keys[c] : m;
    bkey[b] = m;
  }
  bkey[nlb - 1] = KEY_POS_INF;
  if (j->scores) {
    float* sc = j->scores + r * j->nblocks;
    for (int64_t b = 0; b < nlb; ++b) {
      const uint32_t u = bits_of_key(bkey[b]);
      memcpy(&sc[b], &u, 4);
    }
  }
  /* block top-k */
  top_k_flags(bkey, nlb, j->k_blocks, keep_b, tmp);
  int64_t n = 0;
  for (int64_t b = 0; b < nlb; ++b)
    if (keep_b[b]) bout[n++] = (int32_t)b;
  /* mask: a column of a dropped block ranks (and is stored) as -inf */
  for (int64_t c = 0; c < L; ++c) {
    if (!keep_b[c / B]) {
      keys[c] = KEY_NEG_INF;
      if (j->write_mask) {
        const uint32_t u = BITS_NEG_INF;
        memcpy(orow + (s + c) * j->col_stride, &u, 4);
      }
    }
  }
  /* token top-k over the masked live span */
  top_k_flags(keys, L, j->k_tokens, keep_t, tmp);
  n = 0;
  for (int64_t c = 0; c < L; ++c)
    if (keep_t[c]) tout[n++] = (int32_t)(s + c);
}

static void* worker(void* p) {
  arg_t* a = (arg_t*)p;
  job_t* j = a->job;
  const int64_t cap = j->width > 0 ? j->width : 1;
  uint32_t* keys = (uint32_t*)malloc((size_t)cap * 4);
  uint32_t* bkey = (uint32_t*)malloc((size_t)cap * 4);
  uint32_t* tmp = (uint32_t*)malloc((size_t)cap * 4);
  uint8_t* kb = (uint8_t*)malloc((size_t)cap);
  uint8_t* kt = (uint8_t*)malloc((size_t)cap);
  if (!keys || !bkey || !tmp || !kb || !kt) {
    j->status = -1;
  } else {
    for (int32_t rep = 0; rep < j->repeat; ++rep)
      for (int64_t r = a->t; r < j->rows; r += j->nthreads) one_row(j, r, keys, bkey, tmp, kb, kt);
  }
  free(keys); free(bkey); free(tmp); free(kb); free(kt);
  return NULL;
}

/* Runs the chain on every row, `repeat` times over (for timing; the outputs
 * are the same each time when dst != src).  Returns 0, or -1 on a bad
 * argument or a failed allocation. */
int dsa_oracle_select(const float* src, float* dst, int64_t rows, int64_t width,
                      int64_t row_stride, int64_t col_stride, const int32_t* starts,
                      const int32_t* ends, int32_t starts_repeat, int32_t ends_repeat,
                      int32_t block_size, int32_t k_blocks, int32_t k_tokens, int32_t write_mask,
                      int32_t* block_ids, int32_t* token_ids, float* scores, int32_t nthreads,
                      int32_t repeat) {
  if (rows < 0 || width < 0 || block_size < 1 || k_blocks < 1 || k_tokens < 1 ||
      starts_repeat < 1 || ends_repeat < 1 || col_stride < 1 || nthreads < 1 || repeat < 0)
    return -1;
  if (rows == 0) return 0;
  if (!src || !dst || !ends || !block_ids || !token_ids) return -1;
  job_t j;
  memset(&j, 0, sizeof(j));
  j.src = src; j.dst = dst; j.rows = rows; j.width = width;
  j.row_stride = row_stride; j.col_stride = col_stride;
  j.starts = starts; j.ends = ends; j.starts_repeat = starts_repeat; j.ends_repeat = ends_repeat;
  j.B = block_size; j.k_blocks = k_blocks; j.k_tokens = k_tokens; j.write_mask = write_mask;
  j.block_ids = block_ids; j.token_ids = token_ids; j.scores = scores;
  j.nblocks = width > 0 ? (width + block_size - 1) / block_size : 0;
  j.nthreads = nthreads; j.repeat = repeat;
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  arg_t* args = (arg_t*)malloc(sizeof(arg_t) * (size_t)nthreads);
  if (!th || !args) { free(th); free(args); return -1; }
  int started = 0;
  for (int32_t t = 0; t < nthreads; ++t) {
    args[t].job = &j;
    args[t].t = t;
    if (pthread_create(&th[t], NULL, worker, &args[t]) != 0) { j.status = -1; break; }
    ++started;
  }
  for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
  free(th); free(args);
  return j.status;
}

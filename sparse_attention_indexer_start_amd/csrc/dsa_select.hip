// C ABI of DSA decode-time candidate selection on MI355X: context set-up,
// argument checks and launches.  The kernels are in dsa_kernels.hpp.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <type_traits>

#include "dsa_kernels.hpp"

namespace dsa {

// Block top-k over given scores (no block-size dependence).
__global__ __launch_bounds__(NT) void k_topk_blocks(Params p) {
  __shared__ Smem sm;
  const int r = blockIdx.x;
  const Row rb = row_bounds(p, r);
  int32_t* out = p.block_ids + (int64_t)r * p.k_blocks;
  if (rb.L == 0) {
    for (int i = threadIdx.x; i < p.k_blocks; i += NT) out[i] = -1;
    return;
  }
  const float* src = p.in_scores + (int64_t)r * p.nblocks;
  const int nlb = rb.nlb, Kp = min(p.k_blocks, nlb);
  auto getk = [&](int i) { return f2key(src[i]); };
  uint32_t T = 0, q = 0xFFFFFFFFu;
  if (nlb > Kp) wg_radix_select<NT>(nlb, (uint32_t)Kp, getk, sm, T, q);
  wg_select_compact<NT>(nlb, T, q, getk,
      [&](int i, uint32_t rank, bool kept, uint64_t, int) { if (kept) out[rank] = i; }, sm);
  for (int i = Kp + threadIdx.x; i < p.k_blocks; i += NT) out[i] = -1;
}

// Zeroes n32 words at p (vector stores; n32 a multiple of 4, p 16-byte aligned).
__global__ __launch_bounds__(256) void k_zero_words(uint32_t* p, int64_t n32) {
  uint4* q = reinterpret_cast<uint4*>(p);
  const int64_t n4 = n32 / 4;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256)
    q[i] = make_uint4(0u, 0u, 0u, 0u);
}

}  // namespace dsa

// Workspace of dsa_select_fused_noalloc: one copy per device, held until the
// process ends.  In host code this name is only a handle; its device address
// comes from hipGetSymbolAddress, once per device.
static constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)256 << 20;
static __device__ __align__(256) uint32_t scratch[NOALLOC_SCRATCH_BYTES / 4];

// ===========================================================================
// Host side: the C ABI.
// ===========================================================================
using namespace dsa;

struct dsa_ctx {
  dsa_shape sh;
  int device;
  int cus;
  int32_t nblocks, P, G, small_blocks;
  int32_t balanced, NQ, cnt_stride;
  int64_t dblk_cap, tkey_cap;
  void* ws;
  size_t ws_bytes;
  uint32_t *ws_key, *ws_list, *ws_flat, *ws_hist, *ws_cnt, *ws_row, *ws_sel, *ws_dblk, *ws_tkey,
      *ws_tcol, *ws_cand, *ws_ccnt, *status;
  int32_t pregather;
  uint32_t magic;
};

namespace {

constexpr uint32_t CTX_MAGIC = 0x44534131u;
thread_local std::string g_err;

// Per-device state of the allocation-free entry point.
constexpr int NOALLOC_MAX_DEVICES = 64;
struct NoallocDevice {
  bool ready;
  int cus;
  uint32_t* ptr;   // this device's copy of `scratch`
};
NoallocDevice g_noalloc[NOALLOC_MAX_DEVICES];
std::mutex g_noalloc_mutex;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Runs f with ctx->device current, restoring the caller's device afterwards.
template <class F>
int on_device(int device, F&& f) {
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (cur != device && (e = hipSetDevice(device)) != hipSuccess) return hip_fail(e, "hipSetDevice");
  const int rc = f();
  if (cur != device) (void)hipSetDevice(cur);
  return rc;
}

// Launches kernel `k` for block size B: the specialised code for the sizes
// with one, the generic code (any B) otherwise.
void launch_bs(int B, Kernel k, unsigned grid, const Params& p, hipStream_t stream) {
  switch (B) {
    case 1: launch<1>(k, grid, p, stream); break;
    case 2: launch<2>(k, grid, p, stream); break;
    case 4: launch<4>(k, grid, p, stream); break;
    case 8: launch<8>(k, grid, p, stream); break;
    case 16: launch<16>(k, grid, p, stream); break;
    case 32: launch<32>(k, grid, p, stream); break;
    case 64: launch<64>(k, grid, p, stream); break;
    default: launch<0>(k, grid, p, stream); break;
  }
}

Params base_params(const dsa_ctx* c) {
  Params p;
  std::memset(&p, 0, sizeof(p));
  p.width = c->sh.width;
  p.row_stride = c->sh.row_stride;
  p.col_stride = c->sh.col_stride;
  p.rows = c->sh.rows;
  p.B = c->sh.block_size;
  p.k_blocks = c->sh.k_blocks;
  p.k_tokens = c->sh.k_tokens;
  p.starts_repeat = c->sh.starts_repeat;
  p.ends_repeat = c->sh.ends_repeat;
  p.nblocks = c->nblocks;
  p.P = c->P;
  p.G = c->G;
  p.balanced = c->balanced;
  p.NQ = c->NQ;
  p.cnt_stride = c->cnt_stride;
  p.small_blocks = c->small_blocks;
  p.ws_key = c->ws_key;
  p.ws_list = reinterpret_cast<uint64_t*>(c->ws_list);
  p.ws_flat = c->ws_flat;
  p.ws_hist = c->ws_hist;
  p.ws_cnt = c->ws_cnt;
  p.ws_row = c->ws_row;
  p.ws_sel = c->ws_sel;
  p.ws_dblk = c->ws_dblk;
  p.ws_tkey = c->ws_tkey;
  p.ws_tcol = c->ws_tcol;
  p.ws_cand = reinterpret_cast<uint64_t*>(c->ws_cand);
  p.ws_ccnt = c->ws_ccnt;
  p.pregather = c->pregather;
  p.dblk_cap = c->dblk_cap;
  p.tkey_cap = c->tkey_cap;
  p.status = c->status;
  return p;
}

int check_ctx(const dsa_ctx* c) {
  if (c == nullptr) return fail(DSA_ERR_INVALID_ARG, "null context");
  if (c->magic != CTX_MAGIC) return fail(DSA_ERR_DESTROYED, "context was destroyed");
  return DSA_OK;
}

bool empty_shape(const dsa_ctx* c) { return c->sh.rows == 0 || c->sh.width == 0; }

// Whether some row of this shape can be split over its P workgroups (the
// device-side rule of Params::one_group, taken at the widest row).
bool may_split(const dsa_ctx* c) {
  return c->nblocks > c->small_blocks ||
         (c->sh.width > SMALL_COLS && (c->P > 1 || c->balanced));
}

// Workgroups of the one-launch fused call.
int fused_grid(const dsa_ctx* c) {
  if (!may_split(c)) return c->G;
  if (c->balanced) return 2 * c->sh.rows + 2 * (c->NQ + c->sh.rows - 1);
  return 2 * c->G + c->sh.rows;
}

int launch_check(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, what);
  return DSA_OK;
}

int validate_shape(const dsa_shape* s, int device) {
  if (s == nullptr) return fail(DSA_ERR_INVALID_ARG, "shape is null");
  if (s->rows < 0 || s->width < 0) return fail(DSA_ERR_INVALID_ARG, "rows and width must be >= 0");
  if (s->width >= (int64_t)1 << 31) return fail(DSA_ERR_UNSUPPORTED, "width must be < 2^31");
  if (s->block_size < 1) return fail(DSA_ERR_INVALID_ARG, "block_size must be >= 1");
  if (s->k_blocks < 1 || s->k_tokens < 1) return fail(DSA_ERR_INVALID_ARG, "k_blocks and k_tokens must be >= 1");
  if (s->col_stride < 1 || s->row_stride < 1) return fail(DSA_ERR_INVALID_ARG, "strides must be >= 1");
  if (s->starts_repeat < 1 || s->ends_repeat < 1) return fail(DSA_ERR_INVALID_ARG, "repeats must be >= 1");
  if (s->rows > 1 && s->width > 0 && s->row_stride < (s->width - 1) * s->col_stride + 1)
    return fail(DSA_ERR_INVALID_ARG, "row_stride %lld overlaps rows of width %lld at col_stride %lld",
                (long long)s->row_stride, (long long)s->width, (long long)s->col_stride);
  if ((int64_t)s->k_blocks + s->k_tokens > BITMAP_BITS)
    return fail(DSA_ERR_UNSUPPORTED, "k_blocks + k_tokens must be <= %d", BITMAP_BITS);
  if (device < 0) return fail(DSA_ERR_INVALID_ARG, "device must be >= 0");
  return DSA_OK;
}

// Workspace slots, in layout order.  The first three are the words that must
// be zero when a call starts (the status word, the row states and the digit
// histograms); the others are written before they are read.
enum Slot { S_STATUS, S_ROW, S_HIST, S_KEY, S_LIST, S_FLAT, S_CNT, S_SEL, S_DBLK, S_TKEY,
            S_TCOL, S_CAND, S_CCNT, N_SLOTS };
constexpr int N_ZERO_SLOTS = 3;

int64_t slot_words(int64_t w) { return (w + 63) / 64 * 64; }

// Launch geometry and workspace sizes of a shape on a device with `cus` CUs
// (no device call); words[i] = the size of slot i in 32-bit words.
int plan_ctx(const dsa_shape* s, int device, int cus, dsa_ctx* c, int64_t* words) {
  std::memset(c, 0, sizeof(*c));
  c->sh = *s;
  c->device = device;
  c->magic = CTX_MAGIC;
  c->cus = cus;
  const int64_t nb = s->width > 0 ? (s->width + s->block_size - 1) / s->block_size : 0;
  c->nblocks = (int32_t)nb;
  c->small_blocks = LIST_CAP;
  // Workgroups per row: about two per CU in all (one resident round at two
  // workgroups per CU), no more than one per 256 blocks of the buffer, and
  // at most NT.
  const int64_t target = (int64_t)cus * 2;
  int64_t P = s->rows > 0 ? (target + s->rows - 1) / s->rows : 1;
  const int64_t pmax = std::max<int64_t>(1, (nb + 255) / 256);
  P = std::max<int64_t>(1, std::min<int64_t>({P, pmax, (int64_t)NT}));
  c->P = (int32_t)P;
  const int64_t G = P * s->rows;
  if (G > (int64_t)1 << 30) return fail(DSA_ERR_UNSUPPORTED, "too many rows");
  c->G = (int32_t)G;
  // Balanced split of long rows when one workgroup can scan every row's
  // bounds and the rows are few: rows <= CUs / 2 (and <= 256).  With more rows
  // the owners and final workgroups leave too few workers, and the per-row
  // split is faster (208 rows of up to 65,536 strided columns: 48.9 us
  // against 51.6; a 96-row decode batch keeps the balanced kernel, whose
  // short-row path also emits the token ids in closed form: 9.6 us against
  // 10.4).  A pass has at most NQ + rows - 1 non-empty pieces
  // (one per worker plus one per row boundary inside a worker's range);
  // with the rows' owners that is one resident round at two workgroups per
  // CU when NQ = 2 * CUs - rows + 1, less a reserve of slots for the rows'
  // final workgroups, which run while the pass-2 pieces still store -inf.
  // (Without it a 32-row decode batch of 1M-wide rows took 83 us instead of
  // 62; a 208-row batch on the balanced split ran fastest with 64, against
  // 32, 48, 80, 96, 128 or every row.)
  const int64_t reserve = std::min<int64_t>(s->rows, 64);
  c->NQ = (int32_t)std::max<int64_t>(
      1, std::min<int64_t>((int64_t)cus * 2 - s->rows + 1 - reserve, NT));
  c->balanced = (s->rows >= 1 && s->rows <= cus / 2 && s->rows <= 256) ? 1 : 0;
  c->cnt_stride = std::max(c->P, c->NQ);
  const int64_t F = (s->k_tokens + s->block_size - 1) / s->block_size;
  // Token domain of a row: at most nlow + Kp <= 2*K_blk + F blocks (also
  // with repeated ids given to the standalone token top-k).
  c->dblk_cap = 2 * (int64_t)s->k_blocks + F + 1;
  c->tkey_cap = c->dblk_cap * s->block_size;
  for (int i = 0; i < N_SLOTS; ++i) words[i] = 0;
  if (empty_shape(c)) return DSA_OK;
  const bool long_rows = may_split(c);
  const int64_t R = s->rows;
  const int64_t n_key = long_rows ? R * nb : 0;
  const int64_t n_cnt = long_rows ? R * c->cnt_stride : 0;
  // Token candidates are gathered in pass 2 when the kept blocks hold more
  // columns than the token top-k keeps (otherwise the closed form applies).
  c->pregather = ((int64_t)s->k_blocks * s->block_size > s->k_tokens &&
                  (s->block_size == 4 || s->block_size == 8 || s->block_size == 16)) ? 1 : 0;
  const int64_t n_cand = long_rows && c->pregather ? 2 * R * nb : 0;
  words[S_STATUS] = 64;
  words[S_ROW] = R * ROW_STATE;
  words[S_HIST] = long_rows ? R * HIST_WORDS : 0;
  words[S_KEY] = n_key;
  words[S_LIST] = 2 * n_key;
  words[S_FLAT] = n_key;
  words[S_CNT] = n_cnt;
  words[S_SEL] = R * s->k_blocks;
  words[S_DBLK] = R * c->dblk_cap;
  words[S_TKEY] = R * c->tkey_cap;
  words[S_TCOL] = R * c->tkey_cap;
  words[S_CAND] = 2 * n_cand;
  words[S_CCNT] = n_cnt;
  int64_t total = 0;
  for (int i = 0; i < N_SLOTS; ++i) total += slot_words(words[i]);
  c->ws_bytes = (size_t)total * 4;
  return DSA_OK;
}

// Points the context's slots into the workspace at `base` (256-byte aligned).
void assign_slots(dsa_ctx* c, uint32_t* base, const int64_t* words) {
  uint32_t** slots[N_SLOTS] = {&c->status, &c->ws_row, &c->ws_hist, &c->ws_key, &c->ws_list,
                               &c->ws_flat, &c->ws_cnt, &c->ws_sel, &c->ws_dblk, &c->ws_tkey,
                               &c->ws_tcol, &c->ws_cand, &c->ws_ccnt};
  int64_t pos = 0;
  for (int i = 0; i < N_SLOTS; ++i) {
    *slots[i] = words[i] ? base + pos : nullptr;
    pos += slot_words(words[i]);
  }
}

// Words at the start of the workspace that must be zero when a call starts.
int64_t zero_words(const int64_t* words) {
  int64_t n = 0;
  for (int i = 0; i < N_ZERO_SLOTS; ++i) n += slot_words(words[i]);
  return n;
}

// The fused launch(es) of one call on a planned context.
int launch_fused(const dsa_ctx* c, float* logits, const int32_t* starts, const int32_t* ends,
                 int32_t* block_ids, int32_t* token_ids, float* scores, uint32_t flags,
                 hipStream_t stream) {
  Params p = base_params(c);
  p.logits = logits;
  p.starts = starts;
  p.ends = ends;
  p.block_ids = block_ids;
  p.token_ids = token_ids;
  p.scores = scores;
  p.flags = flags & DSA_WRITE_MASK;
  // Long rows need the second pass: in the same launch (its workgroups wait
  // for their row's first pass) or, on request, in a second launch.
  const bool long_rows = may_split(c);
  const bool two = long_rows && (flags & DSA_TWO_LAUNCHES);
  p.balanced = long_rows && c->balanced;
  // First launch: short rows and pass 1; pass 2 in the same launch or a
  // second one.
  const int npc = c->NQ + c->sh.rows - 1;
  const int first = p.balanced ? c->sh.rows + npc : c->G;
  const int second = p.balanced ? npc + c->sh.rows : c->G + c->sh.rows;
  const int grid = fused_grid(c);
  int r2 = DSA_OK;
  const Kernel kern = p.balanced ? Kernel::FusedBalanced : Kernel::Fused;
  p.phase_base = 0;
  launch_bs(p.B, kern, (unsigned)(two ? first : grid), p, stream);
  if ((r2 = launch_check("k_fused launch")) != DSA_OK) return r2;
  if (two) {
    p.phase_base = first;
    launch_bs(p.B, kern, (unsigned)second, p, stream);
    r2 = launch_check("k_fused (second pass) launch");
  }
  return r2;
}

}  // namespace

extern "C" {

const char* dsa_last_error(void) { return g_err.c_str(); }

int dsa_select_init(const dsa_shape* s, int device, dsa_ctx** out) {
  if (out == nullptr) return fail(DSA_ERR_INVALID_ARG, "out is null");
  *out = nullptr;
  int rc = validate_shape(s, device);
  if (rc != DSA_OK) return rc;
  dsa_ctx* c = new (std::nothrow) dsa_ctx;
  if (!c) return fail(DSA_ERR_HIP, "host allocation failed");
  rc = on_device(device, [&]() -> int {
    int cus = 0;
    hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute(CU count)");
    int64_t words[N_SLOTS];
    const int r = plan_ctx(s, device, cus, c, words);
    if (r != DSA_OK || empty_shape(c)) return r;
    e = hipMalloc(&c->ws, c->ws_bytes);
    if (e != hipSuccess) return hip_fail(e, "hipMalloc(workspace)");
    e = hipMemset(c->ws, 0, c->ws_bytes);
    if (e != hipSuccess) return hip_fail(e, "hipMemset(workspace)");
    e = hipDeviceSynchronize();
    if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize");
    assign_slots(c, static_cast<uint32_t*>(c->ws), words);
    return DSA_OK;
  });
  if (rc != DSA_OK) {
    if (c->ws) (void)hipFree(c->ws);
    delete c;
    return rc;
  }
  *out = c;
  return DSA_OK;
}

int dsa_select_destroy(dsa_ctx* c) {
  int rc = check_ctx(c);
  if (rc != DSA_OK) return rc;
  c->magic = 0;
  if (c->ws) {
    rc = on_device(c->device, [&]() -> int {
      hipError_t e = hipFree(c->ws);
      return e == hipSuccess ? DSA_OK : hip_fail(e, "hipFree(workspace)");
    });
  }
  delete c;
  return rc;
}

namespace {
void fill_info(const dsa_ctx* c, dsa_launch_info* info) {
  const bool split = may_split(c) && c->balanced;
  info->programs_per_row = split ? 0 : c->P;
  info->threads_per_group = NT;
  info->grid_groups = fused_grid(c);
  info->small_row_blocks = c->small_blocks;
  info->workspace_bytes = (int64_t)c->ws_bytes;
  info->fused_launches = 1;
}
}  // namespace

int dsa_select_query(const dsa_ctx* c, dsa_launch_info* info) {
  int rc = check_ctx(c);
  if (rc != DSA_OK) return rc;
  if (!info) return fail(DSA_ERR_INVALID_ARG, "info is null");
  fill_info(c, info);
  return DSA_OK;
}

int dsa_select_plan(const dsa_shape* s, int cus, dsa_launch_info* info) {
  if (!info) return fail(DSA_ERR_INVALID_ARG, "info is null");
  if (cus < 1) return fail(DSA_ERR_INVALID_ARG, "cus must be >= 1 (got %d)", cus);
  int rc = validate_shape(s, 0);
  if (rc != DSA_OK) return rc;
  dsa_ctx c;
  int64_t words[N_SLOTS];
  rc = plan_ctx(s, 0, cus, &c, words);
  if (rc != DSA_OK) return rc;
  fill_info(&c, info);
  return DSA_OK;
}

int dsa_block_scores(dsa_ctx* c, const float* logits, const int32_t* starts, const int32_t* ends,
                     float* scores, hipStream_t stream) {
  int rc = check_ctx(c);
  if (rc != DSA_OK) return rc;
  if (empty_shape(c)) return DSA_OK;
  if (!logits || !ends || !scores) return fail(DSA_ERR_INVALID_ARG, "logits, ends and scores must be non-null");
  return on_device(c->device, [&]() -> int {
    Params p = base_params(c);
    p.logits = const_cast<float*>(logits);
    p.starts = starts;
    p.ends = ends;
    p.scores = scores;
    launch_bs(p.B, Kernel::Scores, (unsigned)c->G, p, stream);
    return launch_check("k_scores launch");
  });
}

int dsa_topk(dsa_ctx* c, int mode, const float* src, const int32_t* starts, const int32_t* ends,
             const int32_t* block_ids, int32_t* out, hipStream_t stream) {
  int rc = check_ctx(c);
  if (rc != DSA_OK) return rc;
  if (mode != DSA_TOPK_BLOCKS && mode != DSA_TOPK_TOKENS) return fail(DSA_ERR_INVALID_ARG, "bad mode %d", mode);
  if (mode == DSA_TOPK_BLOCKS && block_ids) return fail(DSA_ERR_INVALID_ARG, "block_ids must be null in BLOCKS mode");
  if (empty_shape(c)) return DSA_OK;
  if (!src || !ends || !out) return fail(DSA_ERR_INVALID_ARG, "src, ends and out must be non-null");
  return on_device(c->device, [&]() -> int {
    Params p = base_params(c);
    p.starts = starts;
    p.ends = ends;
    if (mode == DSA_TOPK_BLOCKS) {
      p.in_scores = src;
      p.block_ids = out;
      hipLaunchKernelGGL(k_topk_blocks, dim3(c->sh.rows), dim3(NT), 0, stream, p);
      return launch_check("k_topk_blocks launch");
    }
    p.logits = const_cast<float*>(src);
    p.in_ids = block_ids;
    p.token_ids = out;
    launch_bs(p.B, Kernel::TopkTokens, (unsigned)c->sh.rows, p, stream);
    return launch_check("k_topk_tokens launch");
  });
}

int dsa_candidate_mask(dsa_ctx* c, float* logits, const int32_t* starts, const int32_t* ends,
                       const int32_t* block_ids, hipStream_t stream) {
  int rc = check_ctx(c);
  if (rc != DSA_OK) return rc;
  if (empty_shape(c)) return DSA_OK;
  if (!logits || !ends || !block_ids) return fail(DSA_ERR_INVALID_ARG, "logits, ends and block_ids must be non-null");
  return on_device(c->device, [&]() -> int {
    Params p = base_params(c);
    p.logits = logits;
    p.starts = starts;
    p.ends = ends;
    p.in_ids = block_ids;
    launch_bs(p.B, Kernel::Mask, (unsigned)c->G, p, stream);
    return launch_check("k_mask launch");
  });
}

int dsa_select_fused(dsa_ctx* c, float* logits, const int32_t* starts, const int32_t* ends,
                     int32_t* block_ids, int32_t* token_ids, float* scores, uint32_t flags,
                     hipStream_t stream) {
  int rc = check_ctx(c);
  if (rc != DSA_OK) return rc;
  if (flags & ~(uint32_t)(DSA_WRITE_MASK | DSA_TWO_LAUNCHES))
    return fail(DSA_ERR_INVALID_ARG, "unknown flags %#x", flags);
  if (empty_shape(c)) return DSA_OK;
  if (!logits || !ends || !block_ids || !token_ids)
    return fail(DSA_ERR_INVALID_ARG, "logits, ends, block_ids and token_ids must be non-null");
  return on_device(c->device, [&]() -> int {
    return launch_fused(c, logits, starts, ends, block_ids, token_ids, scores, flags, stream);
  });
}

int dsa_select_fused_noalloc(const dsa_shape* s, int device, float* logits,
                             const int32_t* starts, const int32_t* ends, int32_t* block_ids,
                             int32_t* token_ids, float* scores, uint32_t flags,
                             uint32_t* status, hipStream_t stream) {
  int rc = validate_shape(s, device);
  if (rc != DSA_OK) return rc;
  if (flags & ~(uint32_t)(DSA_WRITE_MASK | DSA_TWO_LAUNCHES))
    return fail(DSA_ERR_INVALID_ARG, "unknown flags %#x", flags);
  if (s->rows == 0 || s->width == 0) return DSA_OK;
  if (!logits || !ends || !block_ids || !token_ids)
    return fail(DSA_ERR_INVALID_ARG, "logits, ends, block_ids and token_ids must be non-null");
  if (device >= NOALLOC_MAX_DEVICES)
    return fail(DSA_ERR_UNSUPPORTED, "device %d: at most %d devices", device, NOALLOC_MAX_DEVICES);
  return on_device(device, [&]() -> int {
    NoallocDevice& nd = g_noalloc[device];
    {
      std::lock_guard<std::mutex> lock(g_noalloc_mutex);
      if (!nd.ready) {
        // Once per device, with the device current: the device address of
        // this device's copy of the scratch array, and the CU count.
        void* ptr = nullptr;
        hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        int cus = 0;
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
        if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute(CU count)");
        nd.ptr = static_cast<uint32_t*>(ptr);
        nd.cus = cus;
        nd.ready = true;
      }
    }
    dsa_ctx c;
    int64_t words[N_SLOTS];
    int r = plan_ctx(s, device, nd.cus, &c, words);
    if (r != DSA_OK) return r;
    if (c.ws_bytes > NOALLOC_SCRATCH_BYTES)
      return fail(DSA_ERR_UNSUPPORTED,
                  "this shape needs %lld bytes of workspace; the allocation-free entry point "
                  "holds %lld (use dsa_select_init and dsa_select_fused)",
                  (long long)c.ws_bytes, (long long)NOALLOC_SCRATCH_BYTES);
    assign_slots(&c, nd.ptr, words);
    if (status) c.status = status;
    // The scratch keeps the previous call's contents (of any shape): the words
    // that must start at zero are cleared by a kernel on the call's stream.
    const int64_t nz = zero_words(words);
    const unsigned zb = (unsigned)std::min<int64_t>((nz / 4 + 255) / 256, 1024);
    hipLaunchKernelGGL(k_zero_words, dim3(zb), dim3(256), 0, stream, nd.ptr, nz);
    if ((r = launch_check("k_zero_words launch")) != DSA_OK) return r;
    return launch_fused(&c, logits, starts, ends, block_ids, token_ids, scores, flags, stream);
  });
}

int dsa_read_status(dsa_ctx* c, uint32_t* out) {
  int rc = check_ctx(c);
  if (rc != DSA_OK) return rc;
  if (!out) return fail(DSA_ERR_INVALID_ARG, "out is null");
  *out = 0;
  if (!c->status) return DSA_OK;
  return on_device(c->device, [&]() -> int {
    hipError_t e = hipDeviceSynchronize();
    if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize");
    e = hipMemcpy(out, c->status, sizeof(uint32_t), hipMemcpyDeviceToHost);
    return e == hipSuccess ? DSA_OK : hip_fail(e, "hipMemcpy(status)");
  });
}

int dsa_reset_workspace(dsa_ctx* c, hipStream_t stream) {
  int rc = check_ctx(c);
  if (rc != DSA_OK) return rc;
  if (!c->ws) return DSA_OK;
  return on_device(c->device, [&]() -> int {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(stream, &cs);
    if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
    if (cs != hipStreamCaptureStatusNone) return fail(DSA_ERR_CAPTURING, "reset on a capturing stream");
    e = hipMemsetAsync(c->ws, 0, c->ws_bytes, stream);
    return e == hipSuccess ? DSA_OK : hip_fail(e, "hipMemsetAsync(workspace)");
  });
}

}  // extern "C"

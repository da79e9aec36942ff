// Cooperative per-row top-k over very long rows (MI355X, gfx950).
//
// The report on vllm PR #56628 (key source) names the row top-k consumers of
// the masked decode logits, persistent_topk and cooperative_topk, which bound
// their scan by the same per-row ends as the mask; vllm PR #57459 (Summary)
// states that the row top-k takes those bounds.  This is that operation for
// rows far longer than one workgroup can scan: per row, the K best columns of
// [s, e') (e' = min(end, width)) by value, ties to the lower column, output
// ascending and padded with -1.
//
// Each row is cut into P pieces (P fixed by the shape and the CU count; the
// pieces follow the row's own live length), and every step is a launch of its
// own on the caller's stream, so no workgroup ever waits on another:
//   hist  (rows x P)  a 12-, 12- then 8-bit digit histogram of the pieces'
//                     keys (only keys matching the digits found so far),
//                     merged into the row's histogram with atomics;
//   find  (rows)      the digit holding the K-th key, from the row's
//                     histogram; after the third digit (or once a whole bin is
//                     taken) the row's rule (T, q) is fixed: keep key > T, and
//                     the first q keys equal to T in column order;
//   count (rows x P)  each piece's keys above T and equal to T;
//   scan  (rows)      each piece's output offset and its share of the ties;
//   emit  (rows x P)  each piece's kept columns, in column order.
// Passes whose digit is already settled return at once.  The workspace (one
// histogram, a few state words and two counts per piece, per row) does not
// depend on the row length.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>

#include "dsa_device.hpp"
#include "dsa_row_topk.h"

namespace dsa {
namespace rt {

constexpr int NT = 256;
constexpr int FNT = 512;          // the find step (a 4096-bin search needs 8 bins per thread)
constexpr int MIN_PIECE = 4096;   // columns per piece at least (when the row has them)
constexpr int STATE = 8;          // [0] prefix [1] krem [2] done [3] T [4] q [5] Kt

struct Args {
  const float* logits;
  const int32_t* starts;
  const int32_t* ends;
  int32_t* out;
  int64_t width, row_stride, col_stride;
  int32_t rows, k, starts_repeat, ends_repeat, P, pass;
  uint32_t* hist;    // [rows][4096]
  uint32_t* state;   // [rows][STATE]
  uint32_t* cnt;     // [rows][P][2]  keys above T, keys equal to T
  uint32_t* off;     // [rows][P][2]  output offset, ties taken
};

struct Live {
  int64_t s, L;
};

DSA_DEV Live live_range(const Args& a, int r) {
  const int32_t* ep = a.ends + r / a.ends_repeat;
  const int32_t* sp = a.starts ? a.starts + r / a.starts_repeat : ep;
  const int32_t sv = *sp, ev = *ep;
  const int64_t s = a.starts ? (int64_t)sv : 0;
  const int64_t e = (int64_t)ev < a.width ? (int64_t)ev : a.width;
  Live lv;
  lv.s = s;
  lv.L = (s < 0 || e <= s) ? 0 : e - s;
  return lv;
}

// Columns [c0, c1) of the live range that piece j of P covers.
DSA_DEV void piece_range(int64_t L, int P, int j, int64_t& c0, int64_t& c1) {
  const int64_t C = (L + P - 1) / P;
  c0 = min(L, (int64_t)j * C);
  c1 = min(L, c0 + C);
}

// Visits the keys of columns [c0, c1) of a row: f(column, key), four
// columns per thread per round, loads issued together.
template <class F>
DSA_DEV void for_keys(const Args& a, const float* rowp, int64_t c0, int64_t c1, F f) {
  const int64_t cs = a.col_stride;
  constexpr int U = 4;
  for (int64_t b = c0 + (int64_t)threadIdx.x; b < c1; b += (int64_t)NT * U) {
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = b + (int64_t)u * NT;
      v[u] = rowp[(c < c1 ? c : c0) * cs];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = b + (int64_t)u * NT;
      if (c < c1) f(c, f2key(v[u]));
    }
  }
}

__global__ __launch_bounds__(NT) void k_rt_hist(Args a) {
  __shared__ uint32_t h[HIST_WORDS];
  const int r = (int)(blockIdx.x / (unsigned)a.P), j = (int)(blockIdx.x % (unsigned)a.P);
  const Live lv = live_range(a, r);
  if (lv.L == 0) return;
  const uint32_t* st = a.state + (int64_t)r * STATE;
  uint32_t prefix = 0;
  if (a.pass > 0) {
    if (st[2]) return;                    // the rule is already fixed
    prefix = st[0];
  }
  for (int i = threadIdx.x; i < HIST_WORDS; i += NT) h[i] = 0;
  __syncthreads();
  int64_t c0, c1;
  piece_range(lv.L, a.P, j, c0, c1);
  const float* rowp = a.logits + (int64_t)r * a.row_stride + lv.s * a.col_stride;
  if (a.pass == 0) {
    for_keys(a, rowp, c0, c1, [&](int64_t, uint32_t k) { atomicAdd(&h[k >> 20], 1u); });
  } else if (a.pass == 1) {
    const uint32_t p = prefix >> 20;
    for_keys(a, rowp, c0, c1, [&](int64_t, uint32_t k) {
      if ((k >> 20) == p) atomicAdd(&h[(k >> 8) & 0xFFFu], 1u);
    });
  } else {
    const uint32_t p = prefix >> 8;
    for_keys(a, rowp, c0, c1, [&](int64_t, uint32_t k) {
      if ((k >> 8) == p) atomicAdd(&h[k & 0xFFu], 1u);
    });
  }
  __syncthreads();
  uint32_t* gh = a.hist + (int64_t)r * HIST_WORDS;
  for (int i = threadIdx.x; i < HIST_WORDS; i += NT)
    if (h[i]) atomicAdd(&gh[i], h[i]);
}

__global__ __launch_bounds__(FNT) void k_rt_find(Args a) {
  __shared__ Smem sm;
  const int r = (int)blockIdx.x;
  const Live lv = live_range(a, r);
  uint32_t* st = a.state + (int64_t)r * STATE;
  uint32_t* gh = a.hist + (int64_t)r * HIST_WORDS;
  const int64_t Kt = min((int64_t)a.k, lv.L);
  uint32_t prefix, krem, done;
  if (a.pass == 0) {
    prefix = 0;
    krem = (uint32_t)Kt;
    done = 0;
  } else {
    prefix = st[0];
    krem = st[1];
    done = st[2];
  }
  if (lv.L == 0 || done) {
    if (a.pass == 0 && threadIdx.x == 0) {   // an empty row keeps nothing
      st[2] = 1; st[3] = 0xFFFFFFFFu; st[4] = 0; st[5] = 0;
    }
    return;
  }
  const int nb = a.pass == 2 ? 256 : HIST_WORDS;
  const int shift = a.pass == 0 ? 20 : (a.pass == 1 ? 8 : 0);
  uint32_t T = 0, q = 0;
  if (a.pass == 0 && Kt == lv.L) {
    // every column is kept
    done = 1;
    T = 0;
    q = 0xFFFFFFFFu;
  } else {
    for (int i = threadIdx.x; i < nb; i += FNT) sm.hist[i] = gh[i];
    __syncthreads();
    uint32_t d, above, in_bin;
    find_bin<FNT>(sm.hist, nb, krem, sm, d, above, in_bin);
    prefix |= d << shift;
    krem -= above;
    if (a.pass == 2) {
      done = 1;
      T = prefix;
      q = krem;
    } else if (in_bin == krem) {
      // the whole bin is kept: every key from the bin's lowest value up
      done = 1;
      if (prefix == 0) {
        T = 0;
        q = 0xFFFFFFFFu;
      } else {
        T = prefix - 1;
        q = 0;
      }
    }
  }
  // clear the row's histogram for the next pass (and the next call)
  for (int i = threadIdx.x; i < HIST_WORDS; i += FNT) gh[i] = 0;
  if (threadIdx.x == 0) {
    st[0] = prefix;
    st[1] = krem;
    st[2] = done;
    st[3] = T;
    st[4] = q;
    st[5] = (uint32_t)Kt;
  }
}

__global__ __launch_bounds__(NT) void k_rt_count(Args a) {
  __shared__ uint32_t wv[64];
  const int r = (int)(blockIdx.x / (unsigned)a.P), j = (int)(blockIdx.x % (unsigned)a.P);
  const Live lv = live_range(a, r);
  uint32_t* cp = a.cnt + ((int64_t)r * a.P + j) * 2;
  if (lv.L == 0) return;
  const uint32_t* st = a.state + (int64_t)r * STATE;
  const uint32_t T = st[3];
  int64_t c0, c1;
  piece_range(lv.L, a.P, j, c0, c1);
  const float* rowp = a.logits + (int64_t)r * a.row_stride + lv.s * a.col_stride;
  uint32_t gt = 0, eq = 0;
  for_keys(a, rowp, c0, c1, [&](int64_t, uint32_t k) {
    gt += k > T;
    eq += k == T;
  });
  uint32_t tg, te;
  (void)wg_excl_scan<NT>(gt, wv, tg);
  (void)wg_excl_scan<NT>(eq, wv, te);
  if (threadIdx.x == 0) {
    cp[0] = tg;
    cp[1] = te;
  }
}

__global__ __launch_bounds__(NT) void k_rt_scan(Args a) {
  __shared__ uint32_t wv[64];
  const int r = (int)blockIdx.x;
  const Live lv = live_range(a, r);
  const uint32_t* st = a.state + (int64_t)r * STATE;
  int32_t* outp = a.out + (int64_t)r * a.k;
  const int64_t Kt = lv.L == 0 ? 0 : min((int64_t)a.k, lv.L);
  for (int64_t i = Kt + threadIdx.x; i < a.k; i += NT) outp[i] = -1;
  if (lv.L == 0) return;
  const uint32_t q = st[4];
  uint32_t base_gt = 0, base_eq = 0;
  for (int j0 = 0; j0 < a.P; j0 += NT) {
    const int j = j0 + (int)threadIdx.x;
    const uint32_t* cp = a.cnt + ((int64_t)r * a.P + (j < a.P ? j : 0)) * 2;
    const uint32_t gt = j < a.P ? cp[0] : 0u, eq = j < a.P ? cp[1] : 0u;
    uint32_t tg, te;
    const uint32_t xg = wg_excl_scan<NT>(gt, wv, tg) + base_gt;
    const uint32_t xe = wg_excl_scan<NT>(eq, wv, te) + base_eq;
    if (j < a.P) {
      // ties before this piece: xe; this piece takes the ones still allowed
      const uint32_t before = min(xe, q);
      const uint32_t take = min(eq, q - before);
      uint32_t* op = a.off + ((int64_t)r * a.P + j) * 2;
      op[0] = xg + before;
      op[1] = take;
    }
    base_gt += tg;
    base_eq += te;
  }
}

__global__ __launch_bounds__(NT) void k_rt_emit(Args a) {
  __shared__ uint32_t wv[64];
  const int r = (int)(blockIdx.x / (unsigned)a.P), j = (int)(blockIdx.x % (unsigned)a.P);
  const Live lv = live_range(a, r);
  if (lv.L == 0) return;
  const uint32_t* st = a.state + (int64_t)r * STATE;
  const uint32_t T = st[3];
  const uint32_t kt = st[5];   // kept columns of the row (bounds every store below)
  const uint32_t* op = a.off + ((int64_t)r * a.P + j) * 2;
  uint32_t pos = op[0];
  const uint32_t take = op[1];
  int64_t c0, c1;
  piece_range(lv.L, a.P, j, c0, c1);
  const float* rowp = a.logits + (int64_t)r * a.row_stride + lv.s * a.col_stride;
  int32_t* outp = a.out + (int64_t)r * a.k;
  const int64_t cs = a.col_stride;
  const int32_t s32 = (int32_t)lv.s;
  uint32_t ties = 0;   // ties of this piece before the current round
  // Rounds of NT * 4 columns; thread t takes 4 consecutive columns, so the
  // workgroup's exclusive scans give every kept column its place in order.
  constexpr int U = 4;
  for (int64_t b = c0; b < c1; b += (int64_t)NT * U) {
    const int64_t cb = b + (int64_t)threadIdx.x * U;
    uint32_t k[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = cb + u;
      const float v = rowp[(c < c1 ? c : c0) * cs];
      k[u] = c < c1 ? f2key(v) : 0u;
    }
    uint32_t ne = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) ne += (cb + u < c1) && k[u] == T;
    uint32_t te;
    uint32_t xe = wg_excl_scan<NT>(ne, wv, te) + ties;
    bool kept[U];
    uint32_t nk = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool v = cb + u < c1;
      const bool eq = v && k[u] == T;
      kept[u] = (v && k[u] > T) || (eq && xe < take);
      xe += eq;
      nk += kept[u];
    }
    uint32_t tk;
    uint32_t xk = wg_excl_scan<NT>(nk, wv, tk) + pos;
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (kept[u]) {
        if (xk < kt) outp[xk] = s32 + (int32_t)(cb + u);
        ++xk;
      }
    ties += te;
    pos += tk;
  }
}

}  // namespace rt
}  // namespace dsa

// ===========================================================================
// Host side
// ===========================================================================
using namespace dsa::rt;

struct dsa_topk_ctx {
  dsa_topk_shape sh;
  int device;
  int P;
  void* ws;
  size_t ws_bytes;
  uint32_t *hist, *state, *cnt, *off;
  uint32_t magic;
};

namespace {

constexpr uint32_t RT_MAGIC = 0x44535254u;
thread_local std::string g_rt_err;

int rt_fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_rt_err = buf;
  return code;
}

int rt_hip(hipError_t e, const char* what) {
  return rt_fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

struct DeviceScope {
  int prev = -1;
  bool switched = false;
  hipError_t e = hipSuccess;
  explicit DeviceScope(int device) {
    e = hipGetDevice(&prev);
    if (e == hipSuccess && prev != device) {
      e = hipSetDevice(device);
      switched = e == hipSuccess;
    }
  }
  ~DeviceScope() {
    if (switched) (void)hipSetDevice(prev);
  }
};

}  // namespace

extern "C" {

const char* dsa_row_topk_last_error(void) { return g_rt_err.c_str(); }

int dsa_row_topk_init(const dsa_topk_shape* s, int device, dsa_topk_ctx** out) {
  if (!out) return rt_fail(DSA_ERR_INVALID_ARG, "out is null");
  *out = nullptr;
  if (!s) return rt_fail(DSA_ERR_INVALID_ARG, "shape is null");
  if (s->rows < 0 || s->width < 0) return rt_fail(DSA_ERR_INVALID_ARG, "rows and width must be >= 0");
  if (s->width >= ((int64_t)1 << 31)) return rt_fail(DSA_ERR_UNSUPPORTED, "width must be < 2^31");
  if (s->k < 1) return rt_fail(DSA_ERR_INVALID_ARG, "k must be >= 1");
  if (s->col_stride < 1 || s->row_stride < 1) return rt_fail(DSA_ERR_INVALID_ARG, "strides must be >= 1");
  if (s->starts_repeat < 1 || s->ends_repeat < 1) return rt_fail(DSA_ERR_INVALID_ARG, "repeats must be >= 1");
  if (s->rows > 1 && s->width > 0 && s->row_stride < (s->width - 1) * s->col_stride + 1)
    return rt_fail(DSA_ERR_INVALID_ARG, "row_stride overlaps rows");
  if (device < 0) return rt_fail(DSA_ERR_INVALID_ARG, "device must be >= 0");
  DeviceScope ds(device);
  if (ds.e != hipSuccess) return rt_hip(ds.e, "hipSetDevice");
  int cus = 0;
  hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
  if (e != hipSuccess) return rt_hip(e, "hipDeviceGetAttribute(CU count)");
  dsa_topk_ctx* c = new (std::nothrow) dsa_topk_ctx;
  if (!c) return rt_fail(DSA_ERR_HIP, "host allocation failed");
  std::memset(c, 0, sizeof(*c));
  c->sh = *s;
  c->device = device;
  c->magic = RT_MAGIC;
  // Pieces per row: about eight workgroups per CU over all rows, each piece
  // at least MIN_PIECE columns of the widest row, at most 4096.
  const int64_t R = std::max<int64_t>(1, s->rows);
  int64_t P = (8 * (int64_t)cus + R - 1) / R;
  P = std::min<int64_t>(P, std::max<int64_t>(1, (s->width + MIN_PIECE - 1) / MIN_PIECE));
  P = std::max<int64_t>(1, std::min<int64_t>(P, 4096));
  if (P * R > ((int64_t)1 << 31) - 1) { delete c; return rt_fail(DSA_ERR_UNSUPPORTED, "too many rows"); }
  c->P = (int)P;
  if (s->rows > 0 && s->width > 0) {
    const int64_t words = R * dsa::HIST_WORDS + R * STATE + 2 * R * P + 2 * R * P;
    c->ws_bytes = (size_t)words * 4;
    e = hipMalloc(&c->ws, c->ws_bytes);
    if (e != hipSuccess) { delete c; return rt_hip(e, "hipMalloc(workspace)"); }
    e = hipMemset(c->ws, 0, c->ws_bytes);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) { (void)hipFree(c->ws); delete c; return rt_hip(e, "hipMemset(workspace)"); }
    uint32_t* base = static_cast<uint32_t*>(c->ws);
    c->hist = base;
    c->state = c->hist + R * dsa::HIST_WORDS;
    c->cnt = c->state + R * STATE;
    c->off = c->cnt + 2 * R * P;
  }
  *out = c;
  return DSA_OK;
}

int dsa_row_topk_destroy(dsa_topk_ctx* c) {
  if (!c || c->magic != RT_MAGIC) return rt_fail(DSA_ERR_INVALID_ARG, "bad context");
  c->magic = 0;
  int rc = DSA_OK;
  if (c->ws) {
    DeviceScope ds(c->device);
    const hipError_t e = hipFree(c->ws);
    if (e != hipSuccess) rc = rt_hip(e, "hipFree(workspace)");
  }
  delete c;
  return rc;
}

int dsa_row_topk_pieces(const dsa_topk_ctx* c) {
  if (!c || c->magic != RT_MAGIC) return rt_fail(DSA_ERR_INVALID_ARG, "bad context");
  return c->P;
}

int dsa_row_topk(dsa_topk_ctx* c, const float* logits, const int32_t* starts,
                 const int32_t* ends, int32_t* out, hipStream_t stream) {
  if (!c || c->magic != RT_MAGIC) return rt_fail(DSA_ERR_INVALID_ARG, "bad context");
  if (c->sh.rows == 0 || c->sh.width == 0) return DSA_OK;
  if (!logits || !ends || !out) return rt_fail(DSA_ERR_INVALID_ARG, "logits, ends and out must be non-null");
  DeviceScope ds(c->device);
  if (ds.e != hipSuccess) return rt_hip(ds.e, "hipSetDevice");
  Args a;
  std::memset(&a, 0, sizeof(a));
  a.logits = logits; a.starts = starts; a.ends = ends; a.out = out;
  a.width = c->sh.width; a.row_stride = c->sh.row_stride; a.col_stride = c->sh.col_stride;
  a.rows = c->sh.rows; a.k = c->sh.k; a.starts_repeat = c->sh.starts_repeat;
  a.ends_repeat = c->sh.ends_repeat; a.P = c->P;
  a.hist = c->hist; a.state = c->state; a.cnt = c->cnt; a.off = c->off;
  const unsigned pieces = (unsigned)((int64_t)c->sh.rows * c->P), rows = (unsigned)c->sh.rows;
  for (int pass = 0; pass < 3; ++pass) {
    a.pass = pass;
    hipLaunchKernelGGL(k_rt_hist, dim3(pieces), dim3(NT), 0, stream, a);
    hipLaunchKernelGGL(k_rt_find, dim3(rows), dim3(FNT), 0, stream, a);
  }
  hipLaunchKernelGGL(k_rt_count, dim3(pieces), dim3(NT), 0, stream, a);
  hipLaunchKernelGGL(k_rt_scan, dim3(rows), dim3(NT), 0, stream, a);
  hipLaunchKernelGGL(k_rt_emit, dim3(pieces), dim3(NT), 0, stream, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return rt_hip(e, "row top-k launch");
  return DSA_OK;
}

}  // extern "C"

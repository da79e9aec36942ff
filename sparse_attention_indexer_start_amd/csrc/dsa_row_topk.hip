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
// own on the caller's stream:
//   hist  (rows x P, three launches)  a 12-, 12- then 8-bit digit histogram
//         of the pieces' keys (only keys matching the digits found so far),
//         merged into the row's histogram of that digit with atomics.  Each
//         piece of the next launch finds the previous digit itself from that
//         histogram (all find the same one), so no piece waits for another.
//         The third launch also keeps each piece's suffix counts over the
//         last digit.  A row whose K-th key's bin is taken whole is settled
//         early: keep every key from that bin up;
//   count (rows x P)  places every piece's output: from the suffix counts
//         after three digits (no read of the row), or, for a row settled
//         early, from each piece's keys above and equal to T, the last piece
//         to arrive placing the pieces;
//   emit  (rows x P)  each piece's kept columns, in column order, and the -1
//         padding.
// The rule is: keep key > T, and the first q keys equal to T in column
// order.  When every key from the first digit's bin up fits the row's lists,
// the second launch also appends those keys with their columns to each
// piece's list in column order; the third launch, the count of a row settled
// early and the emit then iterate the lists instead of reading the row
// (list mode; a piece whose list part overflows sends the row back to
// reading it).  Each digit's histogram is cleared by a later launch that no
// longer reads it, so consecutive calls and graph replays need no clearing
// launch.  The workspace (the histograms, a few state words, per-piece
// counts, suffix counts and lists, per row) does not depend on the row
// length.
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

constexpr int NT = 512;
constexpr int MIN_PIECE = 8192;   // columns per piece at least (when the row has them)
constexpr int SFX = 257;          // per-piece suffix counts of the last digit, and the sentinel
// The first and second digits' histograms have H0_REPS copies each: piece j adds to copy
// j % H0_REPS (512 pieces adding to the same hundred-odd bins of one copy serialise on their
// atomics).  Each copy also has 64 bucket counts (bins 64b .. 64b + 63), so a reader finds the
// bucket, then the bin, summing the copies of 64 counts at each step instead of reading every
// bin.
constexpr int H0_REPS = 8;
constexpr int H0_BUCKETS = 64;
constexpr int HCOPY = H0_REPS * HIST_WORDS;        // one digit's copies of the bins
constexpr int BCOPY = H0_REPS * H0_BUCKETS;        // one digit's copies of the bucket counts
// A row's histograms: the first and the second digit's copies, the last digit's histogram,
// then the first and the second digit's bucket counts.
constexpr int ROW_HIST = 2 * HCOPY + 256 + 2 * BCOPY;
// State words of a row.  [0] prefix [1] krem after the first digit, [2] mode,
// [3] T [4] q [5] Kt, [6] list mode chosen, [7] arrival ticket of the count
// pass, [8] prefix [9] krem after the second digit, [11] some piece's list
// overflowed.  A pass reads only words that earlier
// launches wrote: the pieces of one launch start at different times, so a
// word one piece writes must not be one another piece of the launch reads
// (the one exception, the mode set to "settled early", is a value every
// piece of that launch reaches on its own).
constexpr int STATE = 12;
// A piece's list is LW parts, one per wave of the listing pass, in column order.
constexpr int LW = NT / 64;
// Row modes: selection running; empty; every column kept; settled before the
// third digit (the count pass places the pieces).
constexpr uint32_t M_RUN = 0, M_EMPTY = 1, M_ALL = 2, M_COUNT = 3;

struct Args {
  const float* logits;
  const int32_t* starts;
  const int32_t* ends;
  int32_t* out;
  int64_t width, row_stride, col_stride;
  int32_t rows, k, starts_repeat, ends_repeat, P, pass, seg;
  uint32_t* hist;    // [rows][ROW_HIST]  first, second and last digit histograms
  uint32_t* state;   // [rows][STATE]
  uint32_t* cnt;     // [rows][P][2]  keys above T, keys equal to T
  uint32_t* off;     // [rows][P][2]  output offset, ties taken
  uint32_t* sfx;     // [rows][P][SFX]  third pass: keys above each last digit
  int2* list;        // [rows][P][seg]  list mode: (column, key) of the first digit's bin and up
  uint32_t* lcnt;    // [rows][P]  entries of each piece's list
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

// Columns [c0, c1) of the live range that piece j of P covers (pieces are a
// multiple of 4 columns long, so a 16-byte aligned row keeps them aligned).
DSA_DEV void piece_range(int64_t L, int P, int j, int64_t& c0, int64_t& c1) {
  const int64_t C = ((L + P - 1) / P + 3) & ~(int64_t)3;
  c0 = min(L, (int64_t)j * C);
  c1 = min(L, c0 + C);
}

// Whether columns from c0 on can be read as aligned float4 vectors.
DSA_DEV bool vec_cols(const Args& a, const float* rowp, int64_t c0) {
  return a.col_stride == 1 && (reinterpret_cast<uintptr_t>(rowp + c0) & 15u) == 0;
}

// Visits the keys of columns [c0, c1) of a row: f(column, key).  Contiguous
// aligned rows are read as float4 vectors, four per thread in flight (the
// last partial vector column by column); other rows column by column, four
// loads per thread in flight.
template <class F>
DSA_DEV void for_keys(const Args& a, const float* rowp, int64_t c0, int64_t c1, F f) {
  const int64_t cs = a.col_stride;
  constexpr int U = 4;
  if (vec_cols(a, rowp, c0)) {
    const int64_t n4 = (c1 - c0) >> 2;
    const float4* vp = reinterpret_cast<const float4*>(rowp + c0);
    for (int64_t b = threadIdx.x; b < n4; b += (int64_t)NT * U) {
      float4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t i = b + (int64_t)u * NT;
        v[u] = vp[i < n4 ? i : 0];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t i = b + (int64_t)u * NT;
        if (i < n4) {
          const int64_t c = c0 + 4 * i;
          f(c, f2key(v[u].x));
          f(c + 1, f2key(v[u].y));
          f(c + 2, f2key(v[u].z));
          f(c + 3, f2key(v[u].w));
        }
      }
    }
    for (int64_t c = c0 + 4 * n4 + threadIdx.x; c < c1; c += NT) f(c, f2key(rowp[c]));
    return;
  }
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

// Visits a piece's list entries (list mode): f(column, key), any order.
// Entry i of a piece's list (its LW parts in order, pre[] their running
// counts) and where it is stored.
DSA_DEV int64_t list_slot(const uint32_t* pre, uint32_t capw, uint32_t i) {
  int w = 0;
#pragma unroll
  for (int x = 1; x < LW; ++x) w += i >= pre[x];
  return (int64_t)w * capw + (i - pre[w]);
}

// Running counts of a piece's LW list parts (pre[LW] = the whole list).
DSA_DEV void list_parts(const Args& a, int64_t pj, uint32_t* pre) {
  uint32_t n[LW];
#pragma unroll
  for (int w = 0; w < LW; ++w) n[w] = a.lcnt[pj * LW + w];
  pre[0] = 0;
#pragma unroll
  for (int w = 0; w < LW; ++w) pre[w + 1] = pre[w] + n[w];
}

template <class F>
DSA_DEV void for_list(const Args& a, int r, int j, F f) {
  const int64_t pj = (int64_t)r * a.P + j;
  const uint32_t capw = (uint32_t)(a.seg / LW);
  uint32_t pre[LW + 1];
  list_parts(a, pj, pre);
  const int2* seg = a.list + pj * a.seg;
  for (uint32_t i = threadIdx.x; i < pre[LW]; i += NT) {
    const int2 e = seg[list_slot(pre, capw, i)];
    f((int64_t)e.x, (uint32_t)e.y);
  }
}

// Whether the row runs on its pieces' lists: chosen by the second pass and
// no piece's list overflowed.
DSA_DEV bool list_mode(const uint32_t* st) { return st[6] != 0u && st[11] == 0u; }

// Keys of 16 consecutive columns cb .. cb + 15 of [c0, c1) (0 past c1).
DSA_DEV void load16(const Args& a, const float* rowp, bool vec, int64_t c0, int64_t c1, int64_t cb,
                    uint32_t* k) {
  constexpr int U = 16;
  if (vec && cb + U <= c1) {
    const float4* vp = reinterpret_cast<const float4*>(rowp + cb);
    float4 v[U / 4];
#pragma unroll
    for (int u = 0; u < U / 4; ++u) v[u] = vp[u];
#pragma unroll
    for (int u = 0; u < U / 4; ++u) {
      k[4 * u] = f2key(v[u].x);
      k[4 * u + 1] = f2key(v[u].y);
      k[4 * u + 2] = f2key(v[u].z);
      k[4 * u + 3] = f2key(v[u].w);
    }
  } else {
    const int64_t cs = a.col_stride;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = cb + u;
      const float v = rowp[(c < c1 ? c : c0) * cs];
      k[u] = c < c1 ? f2key(v) : 0u;
    }
  }
}

// Block-wide exclusive scan of one value per thread (NT threads); also the
// total.  wv needs NT / 64 words; two barriers.
DSA_DEV uint32_t block_excl_scan(uint32_t x, uint32_t* wv, uint32_t& total) {
  constexpr int NW = NT / 64;
  const uint32_t inc = wave_incl_scan(x);
  __syncthreads();
  if ((threadIdx.x & 63) == 63) wv[threadIdx.x >> 6] = inc;
  __syncthreads();
  uint32_t off = 0, tot = 0;
  const int w = (int)(threadIdx.x >> 6);
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const uint32_t v = wv[i];
    off += i < w ? v : 0u;
    tot += v;
  }
  total = tot;
  return off + inc - x;
}

// The digit d of bins h[0, nb) (nb <= 8 * NT) holding the krem-th largest
// key: count(bins > d) < krem <= count(bins >= d).  Also that count above d
// and h[d].  Each thread sums up to eight consecutive bins.
DSA_DEV void find_digit(const uint32_t* h, int nb, uint32_t krem, uint32_t* wv, uint32_t* misc,
                        uint32_t& d, uint32_t& above, uint32_t& in_bin) {
  const int per = nb >= NT ? nb / NT : 1;
  const int lo = (int)threadIdx.x * per;
  uint32_t v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (i < per && lo + i < nb) ? h[lo + i] : 0u;
  uint32_t c = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) c += v[i];
  if (threadIdx.x == 0) { misc[0] = 0; misc[1] = 0; misc[2] = 0; }
  uint32_t total;
  const uint32_t excl = block_excl_scan(c, wv, total);
  const uint32_t sfx = total - excl - c;   // keys in the bins above this thread's
  if (sfx < krem && krem <= sfx + c) {
    uint32_t acc = sfx;
    bool found = false;
#pragma unroll
    for (int i = 7; i >= 0; --i) {
      if (!found && i < per) {
        if (acc + v[i] >= krem) {
          misc[0] = (uint32_t)(lo + i);
          misc[1] = acc;
          misc[2] = v[i];
          found = true;
        } else {
          acc += v[i];
        }
      }
    }
  }
  __syncthreads();
  d = misc[0];
  above = misc[1];
  in_bin = misc[2];
}

// Wave 0: of 64 counts (lane l holds count l; higher l = larger keys), the
// one holding the krem-th largest key, the count above it, and its count.
DSA_DEV void wave_pick(uint32_t v, uint32_t krem, int& pick, uint32_t& above, uint32_t& in_bin) {
  const int l = (int)(threadIdx.x & 63);
  const uint32_t vr = __shfl(v, 63 - l);            // lane l: count 63 - l
  const uint32_t inc = wave_incl_scan(vr);         // counts 63 - l .. 63
  const bool hit = inc - vr < krem && krem <= inc;
  const uint64_t b = __ballot(hit);
  const int lh = b ? (int)__builtin_ctzll(b) : 63;
  pick = 63 - lh;
  above = __shfl(inc - vr, lh);
  in_bin = __shfl(vr, lh);
}

// find_digit for a histogram kept as H0_REPS copies of the bins and of the
// bucket counts: the bucket from the bucket counts, then the bin from that
// bucket's 64 bins, both on wave 0.
DSA_DEV void find_digit_copies(const uint32_t* h0, const uint32_t* buckets, uint32_t krem,
                           uint32_t* misc, uint32_t& d, uint32_t& above, uint32_t& in_bin) {
  if (threadIdx.x < 64) {
    const int l = (int)threadIdx.x;
    uint32_t c[H0_REPS];
#pragma unroll
    for (int x = 0; x < H0_REPS; ++x) c[x] = buckets[x * H0_BUCKETS + l];
    uint32_t v = 0;
#pragma unroll
    for (int x = 0; x < H0_REPS; ++x) v += c[x];
    int bk;
    uint32_t ab, ib;
    wave_pick(v, krem, bk, ab, ib);
    const int bin = bk * 64 + l;
#pragma unroll
    for (int x = 0; x < H0_REPS; ++x) c[x] = h0[x * HIST_WORDS + bin];
    v = 0;
#pragma unroll
    for (int x = 0; x < H0_REPS; ++x) v += c[x];
    int bn;
    uint32_t a2, i2;
    wave_pick(v, krem - ab, bn, a2, i2);
    if (l == 0) {
      misc[0] = (uint32_t)(bk * 64 + bn);
      misc[1] = ab + a2;
      misc[2] = i2;
    }
  }
  __syncthreads();
  d = misc[0];
  above = misc[1];
  in_bin = misc[2];
}

// Output offsets of the row's P pieces from their counts (keys above T and
// equal to T), each piece taking its share of the q ties in column order.
template <class Counts>
DSA_DEV void place_pieces(const Args& a, int r, uint32_t q, uint32_t* wv, Counts counts) {
  uint32_t base_gt = 0, base_eq = 0;
  for (int j0 = 0; j0 < a.P; j0 += NT) {
    const int j = j0 + (int)threadIdx.x;
    uint32_t gt = 0, eq = 0;
    if (j < a.P) counts(j, gt, eq);
    uint32_t tg, te;
    const uint32_t xg = block_excl_scan(gt, wv, tg) + base_gt;
    const uint32_t xe = block_excl_scan(eq, wv, te) + base_eq;
    if (j < a.P) {
      const uint32_t before = min(xe, q);
      uint32_t* op = a.off + ((int64_t)r * a.P + j) * 2;
      op[0] = xg + before;
      op[1] = min(eq, q - before);
    }
    base_gt += tg;
    base_eq += te;
  }
}

// Last of the row's P pieces to arrive (each wave's stores and atomics
// drained first).  The last one resets the ticket.
DSA_DEV bool last_piece(uint32_t* ticket, int P, uint32_t* misc) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t n = atomicAdd(ticket, 1u);
    misc[3] = n == (uint32_t)(P - 1);
    if (misc[3]) st_shared(ticket, 0u);
  }
  __syncthreads();
  return misc[3] != 0;
}

// Words [0, n) of a row's buffer that piece j of P clears.
DSA_DEV void clear_slice(uint32_t* buf, int n, int P, int j) {
  const int per = (n + P - 1) / P;
  const int b0 = min(n, j * per), b1 = min(n, b0 + per);
  for (int i = b0 + (int)threadIdx.x; i < b1; i += NT) buf[i] = 0u;
}

__global__ __launch_bounds__(NT) void k_rt_hist(Args a) {
  __shared__ uint32_t h[HIST_WORDS];
  __shared__ uint32_t wv[NT / 64];
  __shared__ uint32_t misc[8];
  const int r = (int)(blockIdx.x / (unsigned)a.P), j = (int)(blockIdx.x % (unsigned)a.P);
  const Live lv = live_range(a, r);
  uint32_t* st = a.state + (int64_t)r * STATE;
  uint32_t* h0 = a.hist + (int64_t)r * ROW_HIST;    // H0_REPS copies
  uint32_t* h1 = h0 + HCOPY;                         // H0_REPS copies
  uint32_t* h2 = h1 + HCOPY;
  uint32_t* b0 = h2 + 256;                           // bucket counts of h0, h1
  uint32_t* b1 = b0 + BCOPY;
  const int64_t Kt = min((int64_t)a.k, lv.L);
  uint32_t prefix = 0, krem = (uint32_t)Kt;
  bool listing = false;   // second pass: also list the first digit's bin and up
  if (a.pass == 0) {
    clear_slice(h2, 256, a.P, j);          // the last call's third digit
    const uint32_t mode = lv.L == 0 ? M_EMPTY : (Kt == lv.L ? M_ALL : M_RUN);
    if (j == 0 && threadIdx.x == 0) {
      st[0] = 0; st[1] = (uint32_t)Kt; st[2] = mode; st[5] = (uint32_t)Kt;
      st[6] = 0; st[11] = 0;
    }
    if (mode != M_RUN) return;
  } else {
    if (a.pass == 2) {                     // no longer read
      clear_slice(h0, HCOPY, a.P, j);
      clear_slice(b0, BCOPY, a.P, j);
    }
    if (st[2] != M_RUN) return;
    if (a.pass == 2) {
      prefix = st[0];
      krem = st[1];
    }
    uint32_t* out_pk = a.pass == 1 ? &st[0] : &st[8];
    // The previous digit, from the previous pass's histogram (every piece
    // finds the same one).
    uint32_t d, above, in_bin;
    if (a.pass == 1) find_digit_copies(h0, b0, krem, misc, d, above, in_bin);
    else find_digit_copies(h1, b1, krem, misc, d, above, in_bin);
    prefix |= d << (a.pass == 1 ? 20 : 8);
    krem -= above;
    if (in_bin == krem) {
      // the whole bin is kept: every key from the bin's lowest value up
      if (j == 0 && threadIdx.x == 0) {
        st[2] = M_COUNT;
        st[3] = prefix == 0 ? 0u : prefix - 1;
        st[4] = prefix == 0 ? 0xFFFFFFFFu : 0u;
      }
      return;
    }
    if (j == 0 && threadIdx.x == 0) {
      out_pk[0] = prefix;
      out_pk[1] = krem;
    }
    if (a.pass == 1) {
      // List mode when every key from the first digit's bin up fits the
      // pieces' lists (every piece reaches the same choice).
      listing = (uint64_t)above + in_bin <= (uint64_t)a.P * (uint64_t)a.seg;
      if (j == 0 && threadIdx.x == 0) st[6] = listing ? 1u : 0u;
    }
  }
  for (int i = threadIdx.x; i < HIST_WORDS; i += NT) h[i] = 0;
  __syncthreads();
  int64_t c0, c1;
  piece_range(lv.L, a.P, j, c0, c1);
  const float* rowp = a.logits + (int64_t)r * a.row_stride + lv.s * a.col_stride;
  uint32_t above = 0;   // third pass: keys above the 24-bit prefix
  if (a.pass == 0) {
    for_keys(a, rowp, c0, c1, [&](int64_t, uint32_t k) { atomicAdd(&h[k >> 20], 1u); });
  } else if (a.pass == 1 && !listing) {
    const uint32_t p = prefix >> 20;
    for_keys(a, rowp, c0, c1, [&](int64_t, uint32_t k) {
      if ((k >> 20) == p) atomicAdd(&h[(k >> 8) & 0xFFFu], 1u);
    });
  } else if (a.pass == 1) {
    // The same histogram, and every key of the first digit's bin and up with
    // its column appended to a list in column order.  Wave w streams the w-th
    // contiguous eighth of the piece (lane-contiguous float4 loads, four in
    // flight per lane) into its own part of the piece's list; a wave-wide
    // prefix count places the entries of a round, and only rounds holding
    // some entry pay for it.
    const uint32_t p = prefix >> 20;
    const int w = (int)(threadIdx.x >> 6), l = (int)(threadIdx.x & 63);
    const uint32_t capw = (uint32_t)(a.seg / LW);
    int2* segw = a.list + ((int64_t)r * a.P + j) * a.seg + (int64_t)w * capw;
    const int64_t Cw = (((c1 - c0) + LW - 1) / LW + 3) & ~(int64_t)3;
    const int64_t w0 = min(c1, c0 + (int64_t)w * Cw), w1 = min(c1, w0 + Cw);
    uint32_t run = 0;
    // keys kk[0..n) of consecutive columns col0 .. col0 + n - 1 held by each lane
    auto take = [&](const uint32_t* kk, int n, bool valid, int64_t col0) {
      uint32_t q = 0;
      for (int i = 0; i < n; ++i) {
        const bool in = valid && (kk[i] >> 20) >= p;
        if (valid && (kk[i] >> 20) == p) atomicAdd(&h[(kk[i] >> 8) & 0xFFFu], 1u);
        q += in;
      }
      if (__ballot(q != 0) == 0) return;                 // wave-uniform
      const uint32_t inc = wave_incl_scan(q);
      uint32_t x = run + inc - q;
      for (int i = 0; i < n; ++i)
        if (valid && (kk[i] >> 20) >= p) {
          if (x < capw) segw[x] = make_int2((int32_t)(col0 + i), (int32_t)kk[i]);
          ++x;
        }
      run += __shfl(inc, 63);
    };
    if (vec_cols(a, rowp, c0)) {
      const int64_t n4 = (w1 - w0) >> 2;
      const float4* vp = reinterpret_cast<const float4*>(rowp + w0);
      constexpr int U = 4;
      for (int64_t b = 0; b < n4; b += 64 * U) {
        float4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t i = b + u * 64 + l;
          v[u] = vp[i < n4 ? i : 0];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t i = b + u * 64 + l;
          const uint32_t kk[4] = {f2key(v[u].x), f2key(v[u].y), f2key(v[u].z), f2key(v[u].w)};
          take(kk, 4, i < n4, w0 + 4 * i);
        }
      }
      if (w1 - w0 - 4 * n4 > 0) {                       // the last partial vector
        const int64_t ct = w0 + 4 * n4 + l;
        const uint32_t kt1 = f2key(rowp[ct < w1 ? ct : w0]);
        take(&kt1, 1, ct < w1, ct);
      }
    } else {
      const int64_t cs = a.col_stride;
      for (int64_t b = w0; b < w1; b += 64) {
        const int64_t c = b + l;
        const uint32_t kk = f2key(rowp[(c < w1 ? c : w0) * cs]);
        take(&kk, 1, c < w1, c);
      }
    }
    if (l == 0) {
      a.lcnt[((int64_t)r * a.P + j) * LW + w] = min(run, capw);
      if (run > capw) atomicOr(&st[11], 1u);   // the row falls back to reading the row
    }
  } else {
    const uint32_t p = prefix >> 8;
    auto f = [&](int64_t, uint32_t k) {
      if ((k >> 8) == p) atomicAdd(&h[k & 0xFFu], 1u);
      above += (k >> 8) > p;
    };
    if (list_mode(st)) for_list(a, r, j, f);
    else for_keys(a, rowp, c0, c1, f);
  }
  uint32_t tot_above = 0;
  if (a.pass == 2) (void)block_excl_scan(above, wv, tot_above);
  __syncthreads();
  const int nb = a.pass == 2 ? 256 : HIST_WORDS;
  if (a.pass < 2) {
    // copy j % H0_REPS: the bins (consecutive lanes on consecutive bins, so
    // one wave's atomics cover four cache lines), then the bucket counts:
    // thread t sums bins 8t .. 8t + 7 (all of bucket t / 8) and the 8 lanes
    // of a bucket add its count
    static_assert(HIST_WORDS == 8 * NT && NT / 8 == H0_BUCKETS, "bins and buckets per thread");
    uint32_t* gh = (a.pass == 0 ? h0 : h1) + (int64_t)(j % H0_REPS) * HIST_WORDS;
    uint32_t* gb = (a.pass == 0 ? b0 : b1) + (j % H0_REPS) * H0_BUCKETS;
    for (int i = threadIdx.x; i < HIST_WORDS; i += NT)
      if (h[i]) atomicAdd(&gh[i], h[i]);
    uint32_t bs = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) bs += h[8 * (int)threadIdx.x + i];
    bs += __shfl_xor(bs, 1);
    bs += __shfl_xor(bs, 2);
    bs += __shfl_xor(bs, 4);
    if ((threadIdx.x & 7) == 0 && bs) atomicAdd(&gb[threadIdx.x >> 3], bs);
  } else {
    for (int i = threadIdx.x; i < nb; i += NT)
      if (h[i]) atomicAdd(&h2[i], h[i]);
  }
  if (a.pass == 2) {
    // Suffix counts: S[b] = keys above the prefix + keys of last digits >= b.
    uint32_t* sp = a.sfx + ((int64_t)r * a.P + j) * SFX;
    const uint32_t x = threadIdx.x < 256 ? h[255 - threadIdx.x] : 0u;
    uint32_t t2;
    const uint32_t ex = block_excl_scan(x, wv, t2);   // over digits 255, 254, ...
    if (threadIdx.x < 256) sp[255 - threadIdx.x] = tot_above + ex + x;
    if (threadIdx.x == 0) sp[256] = tot_above;
  }
}

// Places every piece's output.  Rows that ran three digits: the last digit
// from the third histogram, and this piece's place from every piece's suffix
// counts (keys above T in the pieces before it, then its share of the q ties
// in column order); no read of the row.  Rows settled before the third
// digit: each piece's keys above and equal to T, the last piece to arrive
// placing the pieces.
__global__ __launch_bounds__(NT) void k_rt_count(Args a) {
  __shared__ uint32_t wv[NT / 64];
  __shared__ uint32_t misc[8];
  const int r = (int)(blockIdx.x / (unsigned)a.P), j = (int)(blockIdx.x % (unsigned)a.P);
  const Live lv = live_range(a, r);
  if (lv.L == 0) return;
  uint32_t* st = a.state + (int64_t)r * STATE;
  if (st[2] == M_RUN) {
    const uint32_t* h2 = a.hist + (int64_t)r * ROW_HIST + 2 * HCOPY;
    uint32_t d, above, in_bin;
    find_digit(h2, 256, st[9], wv, misc, d, above, in_bin);
    const uint32_t q = st[9] - above;
    const uint32_t* sf = a.sfx + (int64_t)r * a.P * SFX;
    uint32_t gt = 0, eq = 0;
    for (int i = threadIdx.x; i < j; i += NT) {
      const uint32_t g1 = sf[(int64_t)i * SFX + d + 1];
      gt += g1;
      eq += sf[(int64_t)i * SFX + d] - g1;
    }
    uint32_t xg, xe;
    (void)block_excl_scan(gt, wv, xg);
    (void)block_excl_scan(eq, wv, xe);
    if (threadIdx.x == 0) {
      const uint32_t* me = sf + (int64_t)j * SFX;
      const uint32_t before = min(xe, q);
      uint32_t* op = a.off + ((int64_t)r * a.P + j) * 2;
      op[0] = xg + before;
      op[1] = min(me[d] - me[d + 1], q - before);
      if (j == 0) st[3] = st[8] | d;
    }
    return;
  }
  if (st[2] != M_COUNT) return;
  const uint32_t T = st[3], q = st[4];
  int64_t c0, c1;
  piece_range(lv.L, a.P, j, c0, c1);
  const float* rowp = a.logits + (int64_t)r * a.row_stride + lv.s * a.col_stride;
  uint32_t gt = 0, eq = 0;
  auto f = [&](int64_t, uint32_t k) {
    gt += k > T;
    eq += k == T;
  };
  if (list_mode(st)) for_list(a, r, j, f);   // every key >= T is listed
  else for_keys(a, rowp, c0, c1, f);
  uint32_t tg, te;
  (void)block_excl_scan(gt, wv, tg);
  (void)block_excl_scan(eq, wv, te);
  uint32_t* cp = a.cnt + ((int64_t)r * a.P + j) * 2;
  if (threadIdx.x == 0) {
    st_shared(&cp[0], tg);
    st_shared(&cp[1], te);
  }
  if (!last_piece(&st[7], a.P, misc)) return;
  place_pieces(a, r, q, wv, [&](int jj, uint32_t& g, uint32_t& e) {
    const uint32_t* c = a.cnt + ((int64_t)r * a.P + jj) * 2;
    g = ld_shared(&c[0]);
    e = ld_shared(&c[1]);
  });
}

__global__ __launch_bounds__(NT) void k_rt_emit(Args a) {
  __shared__ uint32_t wv[NT / 64];
  const int r = (int)(blockIdx.x / (unsigned)a.P), j = (int)(blockIdx.x % (unsigned)a.P);
  // Every word this piece needs besides its list entries is loaded at once
  // (the bounds, the row's state, this piece's place and list part counts),
  // so that they cost one memory round trip instead of a chain of them.
  const uint32_t* st = a.state + (int64_t)r * STATE;
  const int64_t pj = (int64_t)r * a.P + j;
  const uint32_t st2 = st[2], st3 = st[3], st5 = st[5], st6 = st[6], st11 = st[11];
  const uint32_t off0 = a.off[pj * 2], off1 = a.off[pj * 2 + 1];
  uint32_t pre[LW + 1];
  list_parts(a, pj, pre);
  const Live lv = live_range(a, r);
  int32_t* outp = a.out + (int64_t)r * a.k;
  const int64_t Kt = min((int64_t)a.k, lv.L);
  {
    // -1 over [Kt, k), split over the row's pieces
    const int64_t n = a.k - Kt, per = (n + a.P - 1) / a.P;
    const int64_t p0 = Kt + min(n, (int64_t)j * per), p1 = Kt + min(n, ((int64_t)j + 1) * per);
    for (int64_t i = p0 + threadIdx.x; i < p1; i += NT) outp[i] = -1;
  }
  uint32_t* h1 = a.hist + (int64_t)r * ROW_HIST + HCOPY;
  clear_slice(h1, HCOPY, a.P, j);             // read by the third pass only
  clear_slice(h1 + HCOPY + 256 + BCOPY, BCOPY, a.P, j);   // and its bucket counts
  if (lv.L == 0) return;
  const uint32_t mode = st2;
  const uint32_t kt = st5;     // kept columns of the row (bounds every store below)
  int64_t c0, c1;
  piece_range(lv.L, a.P, j, c0, c1);
  uint32_t T, pos, take;
  if (mode == M_ALL) {
    T = 0;                     // every column kept, in order
    pos = (uint32_t)c0;
    take = 0xFFFFFFFFu;
  } else {                     // placed by the count pass
    T = st3;
    pos = off0;
    take = off1;
  }
  const float* rowp = a.logits + (int64_t)r * a.row_stride + lv.s * a.col_stride;
  const int32_t s32 = (int32_t)lv.s;
  uint32_t ties = 0;   // ties of this piece before the current round
  // Rounds of NT * 16 columns (or list entries); thread t takes 16 consecutive
  // ones, so the workgroup's exclusive scans give every kept column its place
  // in order.
  constexpr int U = 16;
  auto round = [&](const uint32_t* k, const int64_t* col, const bool* valid) {
    uint32_t ne = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) ne += valid[u] && k[u] == T;
    uint32_t te;
    uint32_t xe = block_excl_scan(ne, wv, te) + ties;
    bool kept[U];
    uint32_t nk = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool eq = valid[u] && k[u] == T;
      kept[u] = (valid[u] && k[u] > T) || (eq && xe < take);
      xe += eq;
      nk += kept[u];
    }
    uint32_t tk;
    uint32_t xk = block_excl_scan(nk, wv, tk) + pos;
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (kept[u]) {
        if (xk < kt) outp[xk] = s32 + (int32_t)col[u];
        ++xk;
      }
    ties += te;
    pos += tk;
  };
  if (mode != M_ALL && st6 != 0u && st11 == 0u) {
    // list mode: the piece's list holds every key >= T of the piece, in
    // column order, as LW consecutive parts
    const uint32_t capw = (uint32_t)(a.seg / LW);
    const uint32_t n = pre[LW];
    const int2* seg = a.list + pj * a.seg;
    for (uint32_t b = 0; b < n; b += (uint32_t)NT * U) {
      const uint32_t ib = b + threadIdx.x * U;
      uint32_t k[U];
      int64_t col[U];
      bool valid[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t i = ib + u;
        valid[u] = i < n;
        const int2 e = seg[valid[u] ? list_slot(pre, capw, i) : 0];
        k[u] = (uint32_t)e.y;
        col[u] = e.x;
      }
      round(k, col, valid);
    }
    return;
  }
  const bool vec = vec_cols(a, rowp, c0);
  for (int64_t b = c0; b < c1; b += (int64_t)NT * U) {
    const int64_t cb = b + (int64_t)threadIdx.x * U;
    uint32_t k[U];
    int64_t col[U];
    bool valid[U];
    load16(a, rowp, vec, c0, c1, cb, k);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      col[u] = cb + u;
      valid[u] = cb + u < c1;
    }
    round(k, col, valid);
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
  int P, seg;
  void* ws;
  size_t ws_bytes;
  uint32_t *hist, *state, *cnt, *off, *sfx, *lcnt;
  int2* list;
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

}  // extern "C"

namespace {

// Validates a shape and plans it for a device with `cus` CUs into c: pieces
// per row, list entries per piece and the workspace size.  No device call.
int rt_plan(const dsa_topk_shape* s, int cus, dsa_topk_ctx* c) {
  if (!s) return rt_fail(DSA_ERR_INVALID_ARG, "shape is null");
  if (s->rows < 0 || s->width < 0) return rt_fail(DSA_ERR_INVALID_ARG, "rows and width must be >= 0");
  if (s->width >= ((int64_t)1 << 31)) return rt_fail(DSA_ERR_UNSUPPORTED, "width must be < 2^31");
  if (s->k < 1) return rt_fail(DSA_ERR_INVALID_ARG, "k must be >= 1");
  if (s->col_stride < 1 || s->row_stride < 1) return rt_fail(DSA_ERR_INVALID_ARG, "strides must be >= 1");
  if (s->starts_repeat < 1 || s->ends_repeat < 1) return rt_fail(DSA_ERR_INVALID_ARG, "repeats must be >= 1");
  if (s->rows > 1 && s->width > 0 && s->row_stride < (s->width - 1) * s->col_stride + 1)
    return rt_fail(DSA_ERR_INVALID_ARG, "row_stride overlaps rows");
  if (cus < 1) return rt_fail(DSA_ERR_INVALID_ARG, "cus must be >= 1");
  std::memset(c, 0, sizeof(*c));
  c->sh = *s;
  // Pieces per row: about two workgroups per CU over all rows (each piece's
  // histogram is merged into its row's with atomics, so fewer, longer pieces
  // contend less), each piece at least MIN_PIECE columns of the widest row,
  // at most 4096.
  const int64_t R = std::max<int64_t>(1, s->rows);
  int64_t P = (2 * (int64_t)cus + R - 1) / R;
  P = std::min<int64_t>(P, std::max<int64_t>(1, (s->width + MIN_PIECE - 1) / MIN_PIECE));
  P = std::max<int64_t>(1, std::min<int64_t>(P, 4096));
  if (P * R > ((int64_t)1 << 31) - 1) return rt_fail(DSA_ERR_UNSUPPORTED, "too many rows");
  c->P = (int)P;
  // List entries per piece: four times a piece's share of K plus 256 (the
  // first digit's bin usually holds far fewer keys than K), at most a piece.
  const int64_t cmax = ((s->width + P - 1) / P + 3) & ~(int64_t)3;
  int64_t seg = std::max<int64_t>(1, std::min<int64_t>(cmax, 4 * ((s->k + P - 1) / P) + 256));
  seg = (seg + LW - 1) / LW * LW + LW;   // LW equal parts (each wave of the listing pass)
  c->seg = (int)seg;
  if (s->rows > 0 && s->width > 0) {
    // [lists][histograms][state][counts][offsets][suffix counts][list counts]
    const int64_t words = 2 * R * P * seg + R * ROW_HIST + R * STATE + 2 * R * P + 2 * R * P +
                          R * P * SFX + R * P * LW;
    c->ws_bytes = (size_t)words * 4;
  }
  return DSA_OK;
}

}  // namespace

extern "C" {

int dsa_row_topk_plan(const dsa_topk_shape* s, int cus, int32_t* pieces, int64_t* workspace_bytes) {
  dsa_topk_ctx c;
  const int rc = rt_plan(s, cus, &c);
  if (rc != DSA_OK) return rc;
  if (pieces) *pieces = c.P;
  if (workspace_bytes) *workspace_bytes = (int64_t)c.ws_bytes;
  return DSA_OK;
}

int dsa_row_topk_init(const dsa_topk_shape* s, int device, dsa_topk_ctx** out) {
  if (!out) return rt_fail(DSA_ERR_INVALID_ARG, "out is null");
  *out = nullptr;
  {
    dsa_topk_ctx check;   // the shape is validated before any device call
    const int rc = rt_plan(s, 1, &check);
    if (rc != DSA_OK) return rc;
  }
  if (device < 0) return rt_fail(DSA_ERR_INVALID_ARG, "device must be >= 0");
  DeviceScope ds(device);
  if (ds.e != hipSuccess) return rt_hip(ds.e, "hipSetDevice");
  int cus = 0;
  hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
  if (e != hipSuccess) return rt_hip(e, "hipDeviceGetAttribute(CU count)");
  dsa_topk_ctx* c = new (std::nothrow) dsa_topk_ctx;
  if (!c) return rt_fail(DSA_ERR_HIP, "host allocation failed");
  const int rc = rt_plan(s, cus, c);
  if (rc != DSA_OK) { delete c; return rc; }
  c->device = device;
  c->magic = RT_MAGIC;
  const int64_t R = std::max<int64_t>(1, s->rows), P = c->P, seg = c->seg;
  if (s->rows > 0 && s->width > 0) {
    e = hipMalloc(&c->ws, c->ws_bytes);
    if (e != hipSuccess) { delete c; return rt_hip(e, "hipMalloc(workspace)"); }
    e = hipMemset(c->ws, 0, c->ws_bytes);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) { (void)hipFree(c->ws); delete c; return rt_hip(e, "hipMemset(workspace)"); }
    c->list = static_cast<int2*>(c->ws);
    uint32_t* base = reinterpret_cast<uint32_t*>(c->list + R * P * seg);
    c->hist = base;
    c->state = c->hist + R * ROW_HIST;
    c->cnt = c->state + R * STATE;
    c->off = c->cnt + 2 * R * P;
    c->sfx = c->off + 2 * R * P;
    c->lcnt = c->sfx + R * P * SFX;
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
  a.hist = c->hist; a.state = c->state; a.cnt = c->cnt; a.off = c->off; a.sfx = c->sfx;
  a.list = c->list; a.lcnt = c->lcnt; a.seg = c->seg;
  const unsigned pieces = (unsigned)((int64_t)c->sh.rows * c->P);
  for (int pass = 0; pass < 3; ++pass) {
    a.pass = pass;
    hipLaunchKernelGGL(k_rt_hist, dim3(pieces), dim3(NT), 0, stream, a);
  }
  hipLaunchKernelGGL(k_rt_count, dim3(pieces), dim3(NT), 0, stream, a);
  hipLaunchKernelGGL(k_rt_emit, dim3(pieces), dim3(NT), 0, stream, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return rt_hip(e, "row top-k launch");
  return DSA_OK;
}

}  // extern "C"

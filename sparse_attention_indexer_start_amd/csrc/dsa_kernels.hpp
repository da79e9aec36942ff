// Kernels of DSA decode-time candidate selection on MI355X (gfx950).
//
// Per row r of an fp32 logits view with live range [s, e') (e' = min(end,
// width), L = e' - s), the chain is (vllm PR #57459 Summary; report on vllm PR
// #56628, implementation and key source):
//   block scores   max-key value of each B-wide block counted from s, with the
//                  block holding e'-1 pinned to +inf;
//   block top-k    the K_blk best blocks (ties to the lower id);
//   mask           -inf over every live column of a dropped block, nothing
//                  written at or past e' or before s;
//   token top-k    the K_tok best columns of the masked row over [s, e').
//
// Launch shape: P workgroups per row (P from the shape and CU count only),
// ordered part-major so that the first workgroup of every row is dispatched
// first.  Trip counts follow each row's live range, so the grid is fixed and
// the calls replay under HIP graphs.
//
// A row with at most LIST_CAP live blocks is handled end to end by its first
// workgroup from LDS.  A longer row is split over its P workgroups in two
// passes of one launch: pass 1 scores a chunk of blocks into the workspace,
// adds a 12-bit key-digit histogram and takes the row's pass-1 ticket.
// Pass-2 workgroups (grid indices above every pass-1 workgroup) wait until
// every ticket is in, find the digit that holds the K_blk-th score from the
// histogram, mask each block below the digit and list the others; the row's
// final workgroup settles the exact selection among the listed blocks, masks
// the rejected ones and runs the token top-k.  A pass-2 or final workgroup
// waits only for workgroups with lower grid indices, which never wait on
// higher ones, and its wait is time-bounded.
//
// This header holds the kernel templates; each block-size specialisation is
// compiled in a translation unit of its own (dsa_bs_unit.hip) and reached
// from the host through dsa::launch<BS>.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "dsa_device.hpp"
#include "dsa_select.h"

namespace dsa {

constexpr int NT = 512;        // threads per workgroup (8 waves)
constexpr int UNROLL = 4;      // float4 loads in flight per lane in the score pass
// ... and in a long row's pass 1, which streams the whole row (measured: 8 in
// flight there is 1 us faster on 1M-wide rows; the one-workgroup path of short
// rows is faster with 4).
constexpr int UNROLL_LONG = 8;
// Row state words: [0] pass-1 ticket, [1] pass-2 ticket, [3] ready word (written
// by the pass-2 pieces for the final step: ready_word(d, keys above d's bin)),
// [4] low flag, [6] lists-gathered flag.  Each row's state has a 128-byte line of its
// own: workgroups poll these words.
constexpr int ROW_STATE = 32;
// The ready word: d + 1 in bits 0..12, the count of keys above d's bin from
// bit 13 (it is below K_blk <= 2^17).  One word, so a workgroup that sees the
// flag has both values, with no ordering between separate stores to rely on.
DSA_DEV uint32_t ready_word(uint32_t d, uint32_t above) { return (d + 1u) | (above << 13); }
DSA_DEV uint32_t ready_digit(uint32_t w) { return (w & 0x1FFFu) - 1u; }
DSA_DEV uint32_t ready_above(uint32_t w) { return w >> 13; }
constexpr int UNROLL_STRIDED = 8;   // scalar loads in flight per lane: 4 * this
// One workgroup reads at most a few tens of GB/s, so a row longer than this is
// split over its P workgroups even when its block keys would fit in LDS.
constexpr int SMALL_COLS = 16384;
constexpr uint32_t KEPT_FLAG = 0x80000000u;
constexpr uint64_t WAIT_LIMIT_TICKS = 200000000ull;   // 2 s of the 100 MHz clock
// A pass-2 piece holds its -inf stores until the row's final workgroup has
// read the row's lists (loads issued under a store stream take ~15x longer);
// this wait orders work only, so it is short and gives up silently.
constexpr uint64_t HOLD_LIMIT_TICKS = 2000ull;         // 20 us

struct Params {
  float* logits;
  const int32_t* starts;
  const int32_t* ends;
  const int32_t* in_ids;      // block ids given to mask / token top-k
  const float* in_scores;     // scores given to block top-k
  int32_t* block_ids;
  int32_t* token_ids;
  float* scores;
  int64_t width, row_stride, col_stride;
  int32_t rows, B, k_blocks, k_tokens, starts_repeat, ends_repeat;
  int32_t nblocks, P, G, small_blocks, phase_base;
  // Balanced split (rows <= NT): workgroups [0, rows) own the short rows,
  // then NQ pass-1 and NQ pass-2 workgroups share the long rows' blocks.
  int32_t balanced, NQ, cnt_stride;

  // A row is handled by one workgroup when its keys fit in LDS and it is short
  // (or the shape gives each row a single workgroup anyway).
  __device__ __forceinline__ bool one_group(int32_t nlb, int32_t L) const {
    return nlb <= small_blocks && (L <= SMALL_COLS || (P == 1 && !balanced));
  }
  uint32_t flags;
  uint32_t* ws_key;    // [rows][nblocks]  block keys of long rows
  uint64_t* ws_list;   // [rows][nblocks]  listed blocks per piece: (id, key) pairs
  uint32_t* ws_flat;   // [rows][nblocks]  listed blocks, gathered (overflow)
  uint32_t* ws_hist;   // [rows][HIST_WORDS]
  uint32_t* ws_cnt;    // [rows][max(P, NQ)]  list length per piece
  uint32_t* ws_row;    // [rows][ROW_STATE]
  uint32_t* ws_sel;    // [rows][k_blocks]   (overflow)
  uint32_t* ws_dblk;   // [rows][dblk_cap]   (overflow)
  uint32_t* ws_tkey;   // [rows][tkey_cap]   (overflow)
  uint32_t* ws_tcol;   // [rows][tkey_cap]   (overflow)
  uint64_t* ws_cand;   // [rows][2 * nblocks]  token candidates: (column, key) pairs
  uint32_t* ws_ccnt;   // [rows][max(P, NQ)]  candidates per piece (~0u: overflow)
  int64_t dblk_cap, tkey_cap;
  int32_t pregather;   // K_blk * B > K_tok and B in {4, 8, 16}
  uint32_t* status;
};

struct Row {
  int64_t s;
  int32_t L, nlb;
  bool bad;
};

DSA_DEV Row row_bounds(const Params& p, int r) {
  Row rb;
  // Both loads are issued before either value is used (without starts the
  // first one re-reads the end and is discarded), so one round trip serves.
  const int32_t* ep = p.ends + r / p.ends_repeat;
  const int32_t* sp = p.starts ? p.starts + r / p.starts_repeat : ep;
  const int32_t sv = *sp;
  const int32_t ev = *ep;
  const int64_t s = p.starts ? (int64_t)sv : 0;
  const int64_t e = (int64_t)ev;
  const int64_t ec = e < p.width ? e : p.width;
  rb.bad = s < 0;
  const int64_t L = (s < 0 || ec <= s) ? 0 : ec - s;
  rb.s = s < 0 ? 0 : s;
  rb.L = (int32_t)L;
  rb.nlb = (int32_t)((L + p.B - 1) / p.B);
  return rb;
}

DSA_DEV float* row_ptr(const Params& p, int r, const Row& rb) {
  return p.logits + (int64_t)r * p.row_stride + rb.s * p.col_stride;
}

DSA_DEV bool vec_ok(const Params& p, const float* rowp) {
  return p.col_stride == 1 && ((reinterpret_cast<uintptr_t>(rowp) & 15u) == 0);
}

// Grid index -> (row, part), part-major: every row's part 0 comes first.
DSA_DEV void part_of(const Params& p, int g, int& r, int& part) {
  part = g / p.rows;
  r = g - part * p.rows;
}

DSA_DEV void chunk_of(const Row& rb, int P, int part, int& b0, int& b1) {
  const int cb = (rb.nlb + P - 1) / P;
  b0 = min(rb.nlb, part * cb);
  b1 = min(rb.nlb, b0 + cb);
}

// ---------------------------------------------------------------------------
// Balanced split.  The long rows' blocks are concatenated in row order
// (sm.pfx[r] = blocks of long rows before r, sm.pfx[rows] = total T) and
// worker w of a pass takes [w * C, (w + 1) * C) of them, C = ceil(T / NQ)
// (sm.pfx[rows + 1]), so every worker streams the same number of blocks
// whatever the row lengths.  The part of a row inside one worker's range is a
// piece.
// ---------------------------------------------------------------------------
DSA_DEV uint64_t worker_lo(const Smem& sm, int rows, int w) {
  const uint64_t T = sm.pfx[rows], C = sm.pfx[rows + 1];
  const uint64_t lo = (uint64_t)w * C;
  return lo < T ? lo : T;
}
// The worker whose range holds concatenated block x < T: floor(x / C), from a
// double quotient corrected by one step either way (x < 2^53).
DSA_DEV int worker_of(const Smem& sm, int rows, uint64_t x) {
  const uint64_t C = sm.pfx[rows + 1];
  uint64_t q = (uint64_t)((double)x / (double)C);
  if (q * C > x) --q;
  else if ((q + 1) * C <= x) ++q;
  return (int)q;
}

// Pieces of long row r and the first block of piece j (row-relative).
DSA_DEV int piece_count(const Params& p, const Smem& sm, const Row& rb, int r) {
  if (!p.balanced) return p.P;
  return worker_of(sm, p.rows, sm.pfx[r + 1] - 1) - worker_of(sm, p.rows, sm.pfx[r]) + 1;
}
DSA_DEV int piece_start(const Params& p, const Smem& sm, const Row& rb, int r, int j) {
  if (!p.balanced) return min(rb.nlb, j * ((rb.nlb + p.P - 1) / p.P));
  if (j == 0) return 0;
  const int w = worker_of(sm, p.rows, sm.pfx[r]) + j;
  return (int)(worker_lo(sm, p.rows, w) - sm.pfx[r]);
}

template <int BS>
DSA_DEV int div_b(int64_t x, int B) {
  if constexpr (BS > 0) return (int)(x / BS);
  else return (int)(x / B);
}

// Max key over columns [c, c + n) of a block (n <= B), loads issued together.
template <int BS>
DSA_DEV uint32_t block_max_key(const float* rowp, int64_t cs, bool vec, int64_t c, int n) {
  uint32_t m = 0;
  if constexpr (BS >= 4) {
    if (vec && n == BS) {
      f4v v[BS / 4];
#pragma unroll
      for (int j = 0; j < BS / 4; ++j) v[j] = *reinterpret_cast<const f4v*>(rowp + c + 4 * j);
#pragma unroll
      for (int j = 0; j < BS / 4; ++j)
        m = max(m, max(max(f2key(v[j].x), f2key(v[j].y)), max(f2key(v[j].z), f2key(v[j].w))));
      return m;
    }
  }
  for (int j = 0; j < n; ++j) m = max(m, f2key(rowp[(c + j) * cs]));
  return m;
}

// ---------------------------------------------------------------------------
// Block scores of blocks [b0, b1): emit(b, key) once per block.
// ---------------------------------------------------------------------------
// `low` is set when some live value of the range ranks at or below -inf.
// On a contiguous range with B >= 4, mid() runs once, in every thread, after
// the first round's loads are issued and before any is used (work that can
// overlap their latency; it may hold a barrier).
struct NoMid {
  DSA_DEV void operator()() const {}
};
template <int BS, int UNR = UNROLL, class Emit, class Mid = NoMid>
DSA_DEV void score_blocks(const float* rowp, int64_t cs, int B, int L, int b0, int b1,
                          int nlb, bool vec, Emit emit, bool& low, Mid mid = Mid()) {
  if constexpr (BS >= 4) {
    constexpr int G = BS / 4;          // lanes per block, 4 columns per lane
    const int64_t cbeg = (int64_t)b0 * BS;
    const int64_t cend = min((int64_t)b1 * BS, (int64_t)L);
    const int64_t t4 = (int64_t)threadIdx.x * 4;
    const bool leader = (threadIdx.x % G) == 0;
    if (!vec) {
      if constexpr (BS == 16) {
        // Strided or unaligned: one column per lane per slot, so the lanes of
        // a load instruction read consecutive columns (each touched line is
        // requested once, not once per column of a lane's group); a block is
        // 16 consecutive lanes.  (For B of 4 and 8 this form makes the
        // compiler give the kernel a scratch frame, so they keep the form
        // below.)
        constexpr int US = 2 * UNROLL_STRIDED;
        const bool lead = (threadIdx.x % BS) == 0;
        for (int64_t c0 = cbeg; c0 < cend; c0 += (int64_t)NT * US) {
          float v[US];
#pragma unroll
          for (int u = 0; u < US; ++u) {
            const int64_t col = c0 + (int64_t)u * NT + threadIdx.x;
            v[u] = col < cend ? rowp[col * cs] : __uint_as_float(0xFFFFFFFFu);
          }
#pragma unroll
          for (int u = 0; u < US; ++u) {
            const int64_t col = c0 + (int64_t)u * NT + threadIdx.x;
            const uint32_t kk = f2key(v[u]);
            low |= col < cend && kk <= KEY_NEG_INF;
            const uint32_t m = group_max<BS>(kk);
            if (lead && col < cend) {
              const int b = (int)(col / BS);
              emit(b, b == nlb - 1 ? KEY_POS_INF : m);
            }
          }
        }
        return;
      }
      // Strided or unaligned, other B: scalar loads, UNROLL_STRIDED groups of 4
      // in flight.
      const int64_t sstep = (int64_t)NT * 4 * UNROLL_STRIDED;
      for (int64_t c0 = cbeg; c0 < cend; c0 += sstep) {
        float v[UNROLL_STRIDED][4];
#pragma unroll
        for (int u = 0; u < UNROLL_STRIDED; ++u) {
          const int64_t col = c0 + (int64_t)u * NT * 4 + t4;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            v[u][j] = (col + j < cend) ? rowp[(col + j) * cs] : __uint_as_float(0xFFFFFFFFu);
        }
#pragma unroll
        for (int u = 0; u < UNROLL_STRIDED; ++u) {
          const int64_t col = c0 + (int64_t)u * NT * 4 + t4;
          uint32_t m = 0;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t kk = f2key(v[u][j]);
            m = max(m, kk);
            low |= (col + j < cend) && kk <= KEY_NEG_INF;
          }
          m = group_max<G>(m);
          if (leader && col < cend) {
            const int b = (int)(col / BS);
            emit(b, b == nlb - 1 ? KEY_POS_INF : m);
          }
        }
      }
      return;
    }
    const int64_t step = (int64_t)NT * 4 * UNR;
    for (int64_t c0 = cbeg; c0 < cend; c0 += step) {
      uint32_t k[UNR];
      if (vec) {
        // Whole vectors first, so that all UNR loads are in flight together;
        // the one partial vector at the end of the range is filled afterwards.
        const float z = __uint_as_float(0xFFFFFFFFu);    // key 0: below every float
        f4v v[UNR];
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
          const int64_t col = c0 + (int64_t)u * NT * 4 + t4;
          v[u] = col + 4 <= cend ? *reinterpret_cast<const f4v*>(rowp + col) : f4v{z, z, z, z};
        }
        // The partial vector's scalars go into registers of their own, so
        // their loads are in flight together with the vector loads.
        int tu = -1;
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
          const int64_t col = c0 + (int64_t)u * NT * 4 + t4;
          if (col < cend && col + 4 > cend) tu = u;
        }
        float t0 = z, t1 = z, t2 = z;
        if (tu >= 0) {
          const int64_t col = c0 + (int64_t)tu * NT * 4 + t4;
          t0 = rowp[col];
          if (col + 1 < cend) t1 = rowp[col + 1];
          if (col + 2 < cend) t2 = rowp[col + 2];
        }
#pragma unroll
        for (int u = 0; u < UNR; ++u)
          if (u == tu) v[u] = f4v{t0, t1, t2, z};
        if (c0 == cbeg) mid();
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
          const int64_t col = c0 + (int64_t)u * NT * 4 + t4;
          k[u] = max(max(f2key(v[u].x), f2key(v[u].y)), max(f2key(v[u].z), f2key(v[u].w)));
#pragma unroll
          for (int j = 0; j < 4; ++j)
            low |= (col + j < cend) && f2key(v[u][j]) <= KEY_NEG_INF;
        }
      } else {
        float v[UNR][4];
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
          const int64_t col = c0 + (int64_t)u * NT * 4 + t4;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            v[u][j] = (col + j < cend) ? rowp[(col + j) * cs] : __uint_as_float(0xFFFFFFFFu);
        }
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
          const int64_t col = c0 + (int64_t)u * NT * 4 + t4;
          k[u] = max(max(f2key(v[u][0]), f2key(v[u][1])), max(f2key(v[u][2]), f2key(v[u][3])));
#pragma unroll
          for (int j = 0; j < 4; ++j)
            low |= (col + j < cend) && f2key(v[u][j]) <= KEY_NEG_INF;
        }
      }
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const uint32_t m = group_max<G>(k[u]);
        const int64_t col = c0 + (int64_t)u * NT * 4 + t4;
        if (leader && col < cend) {
          const int b = (int)(col / BS);
          emit(b, b == nlb - 1 ? KEY_POS_INF : m);
        }
      }
    }
  } else if constexpr (BS == 1 || BS == 2) {
    const int64_t cbeg = (int64_t)b0 * BS;
    const int64_t cend = min((int64_t)b1 * BS, (int64_t)L);
    for (int64_t c0 = cbeg + (int64_t)threadIdx.x * 4; c0 < cend; c0 += (int64_t)NT * 4 * UNR) {
      uint32_t k[UNR][4];
#pragma unroll
      for (int u = 0; u < UNR; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t col = c0 + (int64_t)u * NT * 4 + j;
          k[u][j] = col < cend ? f2key(rowp[col * cs]) : 0u;
          low |= col < cend && k[u][j] <= KEY_NEG_INF;
        }
#pragma unroll
      for (int u = 0; u < UNR; ++u)
#pragma unroll
        for (int j = 0; j < 4; j += BS) {
          const int64_t col = c0 + (int64_t)u * NT * 4 + j;
          if (col < cend) {
            uint32_t m = k[u][j];
            if constexpr (BS == 2) m = max(m, k[u][j + 1]);
            const int b = (int)(col / BS);
            emit(b, b == nlb - 1 ? KEY_POS_INF : m);
          }
        }
    }
  } else {
    // Any block size: one lane per block.
    for (int b = b0 + (int)threadIdx.x; b < b1; b += NT) {
      const int64_t c0 = (int64_t)b * B;
      const int n = (int)min((int64_t)B, (int64_t)L - c0);
      const uint32_t m = block_max_key<0>(rowp, cs, false, c0, n);
      uint32_t mn = 0xFFFFFFFFu;
      for (int j = 0; j < n; ++j) mn = min(mn, f2key(rowp[(c0 + j) * cs]));
      low |= mn <= KEY_NEG_INF;
      emit(b, b == nlb - 1 ? KEY_POS_INF : m);
    }
  }
}

// ---------------------------------------------------------------------------
// -inf over the live columns of blocks b in [b0, b1) with masked(b).
// ---------------------------------------------------------------------------
template <int BS, class IsMasked>
DSA_DEV void mask_blocks(float* rowp, int64_t cs, int B, int L, int b0, int b1, bool vec,
                         IsMasked masked) {
  const int64_t cbeg = (int64_t)b0 * B;
  const int64_t cend = min((int64_t)b1 * B, (int64_t)L);
  if constexpr (BS >= 4) {
    if (vec) {
      for (int64_t col = cbeg + (int64_t)threadIdx.x * 4; col < cend; col += (int64_t)NT * 4) {
        if (!masked((int)(col / BS))) continue;
        if (col + 4 <= cend) {
          store_ninf4(rowp + col);
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (col + j < cend) store_ninf(rowp + col + j);
        }
      }
      return;
    }
    // Strided or unaligned: one column per lane, so each store instruction
    // covers consecutive columns (each touched line once, not once per
    // column of a lane's group).
    for (int64_t col = cbeg + (int64_t)threadIdx.x; col < cend; col += NT)
      if (masked((int)(col / BS))) store_ninf(rowp + col * cs);
  } else {
    for (int64_t col = cbeg + (int64_t)threadIdx.x; col < cend; col += NT)
      if (masked(div_b<BS>(col, B))) store_ninf(rowp + col * cs);
  }
}

// -inf over the live columns of block b, by one lane (vector stores when the
// block is whole and aligned).
template <int BS>
DSA_DEV void mask_block_lane(float* rowp, int64_t cs, int B, int L, bool vec, int64_t b) {
  const int64_t c0 = b * B;
  const int n = (int)min((int64_t)B, (int64_t)L - c0);
  if constexpr (BS >= 4) {
    if (vec && n == BS) {
#pragma unroll
      for (int t = 0; t < BS / 4; ++t) store_ninf4(rowp + c0 + 4 * t);
      return;
    }
  }
  for (int e = 0; e < n; ++e) store_ninf(rowp + (c0 + e) * cs);
}

// -inf over one whole block (called by one lane).
DSA_DEV void mask_one_block(float* rowp, int64_t cs, int B, int L, uint32_t b) {
  const int64_t c0 = (int64_t)b * B;
  const int64_t c1 = min(c0 + B, (int64_t)L);
  for (int64_t c = c0; c < c1; ++c) store_ninf(rowp + c * cs);
}

DSA_DEV void write_empty_row(const Params& p, int r) {
  if (p.block_ids)
    for (int i = threadIdx.x; i < p.k_blocks; i += NT) p.block_ids[(int64_t)r * p.k_blocks + i] = -1;
  if (p.token_ids)
    for (int i = threadIdx.x; i < p.k_tokens; i += NT) p.token_ids[(int64_t)r * p.k_tokens + i] = -1;
}

// Visit the live columns of kept blocks sel[j0..j1) in column order:
// visit(column, key).  Loads of GB blocks are issued together.
template <int BS, class Visit>
DSA_DEV void gather_kept(const float* rowp, int64_t cs, int B, int L, bool vec,
                         const uint32_t* sel, int j0, int j1, Visit visit) {
  if constexpr (BS >= 4) {
    constexpr int GB = (BS / 4) >= 8 ? 1 : 8 / (BS / 4);
    for (int j = j0; j < j1; j += GB) {
      uint32_t kk[GB][BS];
      int64_t c0s[GB];
      bool full[GB];
#pragma unroll
      for (int g = 0; g < GB; ++g) {
        c0s[g] = -1;
        full[g] = false;
        if (j + g < j1) {
          c0s[g] = (int64_t)sel[j + g] * BS;
          full[g] = vec && c0s[g] + BS <= L;
        }
      }
      // Whole blocks by vector loads; strided, unaligned or partial (newest)
      // blocks by scalar loads into registers of their own.  All loads are
      // issued before any value is used.
      f4v v[GB][BS / 4];
      float sv[GB][BS];
#pragma unroll
      for (int g = 0; g < GB; ++g)
#pragma unroll
        for (int t = 0; t < BS / 4; ++t)
          v[g][t] = full[g] ? *reinterpret_cast<const f4v*>(rowp + c0s[g] + 4 * t) : f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int g = 0; g < GB; ++g) {
        const int n = (c0s[g] >= 0 && !full[g]) ? (int)min((int64_t)BS, (int64_t)L - c0s[g]) : 0;
#pragma unroll
        for (int e = 0; e < BS; ++e) sv[g][e] = e < n ? rowp[(c0s[g] + e) * cs] : 0.f;
      }
#pragma unroll
      for (int g = 0; g < GB; ++g)
#pragma unroll
        for (int t = 0; t < BS / 4; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            kk[g][4 * t + e] = full[g] ? f2key(v[g][t][e]) : f2key(sv[g][4 * t + e]);
#pragma unroll
      for (int g = 0; g < GB; ++g) {
        if (c0s[g] < 0) continue;
        const int n = (int)min((int64_t)BS, (int64_t)L - c0s[g]);
#pragma unroll
        for (int e = 0; e < BS; ++e)
          if (e < n) visit(c0s[g] + e, kk[g][e]);
      }
    }
  } else {
    for (int j = j0; j < j1; ++j) {
      const int64_t c0 = (int64_t)sel[j] * B;
      const int n = (int)min((int64_t)B, (int64_t)L - c0);
      for (int e = 0; e < n; ++e) visit(c0 + e, f2key(rowp[(c0 + e) * cs]));
    }
  }
}

// ---------------------------------------------------------------------------
// Token top-k of one row (one workgroup).
//   sel     ascending kept block ids (Kp of them); nullptr: rank the row as is.
//   tlo     a key no larger than the largest value of any kept block other
//           than the newest (0 when unknown).
// When the kept blocks hold at least Kt columns at or above some bound beta
// (beta = tlo if enough columns reach it, else the smallest finite key), every
// one of the Kt best columns reaches beta, so only kept columns >= beta are
// ranked.  Otherwise the ranked domain is every kept block plus the
// F = ceil(Kt/B) lowest non-kept blocks in block order: a non-kept column ranks
// as -inf and no -inf column beyond the first Kt of them can enter the top Kt.
// Either way the result equals ranking the whole masked row.
// ---------------------------------------------------------------------------
template <int BS>
DSA_DEV void token_stage(const Params& p, int r, const Row& rb, const float* rowp,
                         const uint32_t* sel, int Kp, uint32_t tlo, bool canonical,
                         bool no_low, Smem& sm, const uint32_t* nonkept = nullptr,
                         int n_nonkept = 0) {
  const int L = rb.L, nlb = rb.nlb, B = p.B;
  const int64_t cs = p.col_stride;
  const bool vec = vec_ok(p, rowp);
  const int Kt = min(p.k_tokens, L);
  int32_t* tout = p.token_ids + (int64_t)r * p.k_tokens;
  if (L <= p.k_tokens) {
    for (int i = threadIdx.x; i < p.k_tokens; i += NT) tout[i] = i < L ? (int32_t)(rb.s + i) : -1;
    return;
  }
  if (sel == nullptr) {
    auto getk = [&](int i) { return f2key(rowp[(int64_t)i * cs]); };
    uint32_t T, q;
    wg_radix_select<NT>(L, (uint32_t)Kt, getk, sm, T, q);
    wg_select_compact<NT>(L, T, q, getk,
        [&](int i, uint32_t rank, bool kept, uint64_t, int) {
          if (kept) tout[rank] = (int32_t)(rb.s + i);
        }, sm);
    for (int i = Kt + threadIdx.x; i < p.k_tokens; i += NT) tout[i] = -1;
    return;
  }

  // Kept columns: every kept block is whole except the newest (the row's last).
  const bool newest_kept = canonical && Kp > 0 && sel[Kp - 1] == (uint32_t)(nlb - 1);
  const int64_t C = newest_kept ? (int64_t)(Kp - 1) * B + (L - (int64_t)(nlb - 1) * B) : -1;
  if (C >= 0 && C <= Kt) {
    // ---- closed form: all kept columns, then the lowest non-kept columns ----
    // Valid when every kept column ranks above -inf (checked here): then the
    // Kt best columns are the C kept ones and the first q = Kt - C of the
    // non-kept (-inf) columns in column order.
    // (no_low: the scores pass saw no live value at or below -inf.)
    uint32_t tf = (uint32_t)C;
    if (!no_low) {
      const int bpt = (Kp + NT - 1) / NT;
      const int j0 = min(Kp, (int)threadIdx.x * bpt), j1 = min(Kp, j0 + bpt);
      uint32_t cf = 0;
      gather_kept<BS>(rowp, cs, B, L, vec, sel, j0, j1, [&](int64_t, uint32_t k) { cf += k > KEY_NEG_INF; });
      (void)wg_excl_scan<NT>(cf, sm.wv, tf);
    }
    if ((int64_t)tf == C) {
      const int q = Kt - (int)C;
      for (int idx = threadIdx.x; idx < Kt; idx += NT) {
        int64_t col;
        int rank;
        if (idx < (int)C) {
          const int j = div_b<BS>(idx, B);
          const int e = idx - j * B;
          const int64_t b = sel[j];
          col = b * B + e;
          rank = idx + (int)min((int64_t)q, (b - j) * B);
        } else {
          const int f = idx - (int)C;
          const int i = div_b<BS>(f, B);
          const int e = f - i * B;
          // the i-th non-kept block, from the list when it holds it; else the
          // number of kept blocks below it is the first j with sel[j] - j > i
          // (sel[j] - j counts non-kept blocks below sel[j])
          int64_t bnk;
          if (i < n_nonkept) {
            bnk = nonkept[i];
          } else {
            int lo = 0, hi = Kp;
            while (lo < hi) {
              const int mid = (lo + hi) >> 1;
              if ((int64_t)sel[mid] - mid > i) hi = mid;
              else lo = mid + 1;
            }
            bnk = i + lo;
          }
          col = bnk * B + e;
          rank = f + (int)(bnk - i) * B;
        }
        tout[rank] = (int32_t)(rb.s + col);
      }
      for (int i = Kt + threadIdx.x; i < p.k_tokens; i += NT) tout[i] = -1;
      return;
    }
  }

  if ((int64_t)Kp * B >= Kt) {
    // ---- pre-filtered kept columns (thread-contiguous kept blocks) ----
    const int bpt = (Kp + NT - 1) / NT;
    const int j0 = min(Kp, (int)threadIdx.x * bpt), j1 = min(Kp, j0 + bpt);
    uint32_t ca = 0, cf = 0;
    gather_kept<BS>(rowp, cs, B, L, vec, sel, j0, j1, [&](int64_t, uint32_t k) {
      ca += k >= tlo;
      cf += k > KEY_NEG_INF;
    });
    uint32_t ta, tf;
    const uint32_t oa = wg_excl_scan<NT>(ca, sm.wv, ta);
    const uint32_t of = wg_excl_scan<NT>(cf, sm.wv, tf);
    const bool use_a = tlo > KEY_NEG_INF && ta >= (uint32_t)Kt;
    if (use_a || tf >= (uint32_t)Kt) {
      const uint32_t bound = use_a ? tlo : KEY_NEG_INF + 1u;
      const uint32_t m = use_a ? ta : tf;
      uint32_t off = use_a ? oa : of;
      const bool lds = m <= (uint32_t)TK_CAP;
      uint32_t* fkey = lds ? sm.tkey : p.ws_tkey + (int64_t)r * p.tkey_cap;
      uint32_t* fcol = lds ? sm.kid : p.ws_tcol + (int64_t)r * p.tkey_cap;
      gather_kept<BS>(rowp, cs, B, L, vec, sel, j0, j1, [&](int64_t c, uint32_t k) {
        if (k >= bound) {
          fkey[off] = k;
          fcol[off] = (uint32_t)c;
          ++off;
        }
      });
      __syncthreads();
      uint32_t T = 0, q = 0xFFFFFFFFu;
      auto getk = [&](int i) { return fkey[i]; };
      if ((int)m > Kt) wg_radix_select<NT>((int)m, (uint32_t)Kt, getk, sm, T, q);
      wg_select_compact<NT>((int)m, T, q, getk,
          [&](int i, uint32_t rank, bool kept, uint64_t, int) {
            if (kept) tout[rank] = (int32_t)(rb.s + fcol[i]);
          }, sm);
      for (int i = Kt + threadIdx.x; i < p.k_tokens; i += NT) tout[i] = -1;
      return;
    }
  }

  // ---- kept blocks plus the lowest F non-kept blocks ----
  const int F = (Kt + B - 1) / B;
  const int nlow = min(nlb, Kp + F);
  uint32_t* lowbits = sm.hist;
  for (int j = threadIdx.x; j < (nlow + 31) / 32; j += NT) lowbits[j] = 0;
  __syncthreads();
  for (int j = threadIdx.x; j < Kp; j += NT) {
    const uint32_t b = sel[j];
    if (b < (uint32_t)nlow) atomicOr(&lowbits[b >> 5], 1u << (b & 31));
  }
  __syncthreads();
  const bool db_lds = (nlow + Kp) <= DB_CAP;
  uint32_t* dblk = db_lds ? sm.kid : p.ws_dblk + (int64_t)r * p.dblk_cap;
  auto lowkey = [&](int b) -> uint32_t { return ((lowbits[b >> 5] >> (b & 31)) & 1u) ? 2u : 1u; };
  const uint32_t n1 = wg_select_compact<NT>(nlow, 1u, (uint32_t)F, lowkey,
      [&](int b, uint32_t rank, bool kept, uint64_t, int) {
        if (kept) dblk[rank] = (uint32_t)b | (lowkey(b) == 2u ? KEPT_FLAG : 0u);
      }, sm);
  const uint32_t n2 = wg_compact<NT>(Kp, [&](int j) { return sel[j] >= (uint32_t)nlow; },
      [&](int j, uint32_t rank) { dblk[n1 + rank] = sel[j] | KEPT_FLAG; }, sm);
  __syncthreads();
  const int nd = (int)(n1 + n2);
  const int last = (int)(dblk[nd - 1] & ~KEPT_FLAG);
  const int nc = (nd - 1) * B + min(B, L - last * B);
  uint32_t* tkey = nc <= TK_CAP ? sm.tkey : p.ws_tkey + (int64_t)r * p.tkey_cap;
  constexpr int U = 8;
  uint32_t cgt = 0, cge = 0;
  for (int i0 = threadIdx.x; i0 < nc; i0 += NT * U) {
    uint32_t k[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * NT;
      k[u] = KEY_NEG_INF;
      if (i < nc) {
        const int d = div_b<BS>(i, B);
        const uint32_t e = dblk[d];
        const int64_t c = (int64_t)(e & ~KEPT_FLAG) * B + (i - d * B);
        if ((e & KEPT_FLAG) && c < L) k[u] = f2key(rowp[c * cs]);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (i0 + u * NT < nc) {
        tkey[i0 + u * NT] = k[u];
        cgt += k[u] > KEY_NEG_INF;
        cge += k[u] >= KEY_NEG_INF;
      }
    }
  }
  uint32_t tgt, tge;
  (void)wg_excl_scan<NT>(cgt, sm.wv, tgt);
  (void)wg_excl_scan<NT>(cge, sm.wv, tge);
  uint32_t T = 0, q = 0xFFFFFFFFu;
  auto getk = [&](int i) { return tkey[i]; };
  if (tgt <= (uint32_t)Kt && (uint32_t)Kt <= tge) {
    // All columns above -inf, then the lowest-index -inf columns.
    T = KEY_NEG_INF;
    q = (uint32_t)Kt - tgt;
  } else if (nc > Kt) {
    wg_radix_select<NT>(nc, (uint32_t)Kt, getk, sm, T, q);
  }
  wg_select_compact<NT>(nc, T, q, getk,
      [&](int i, uint32_t rank, bool kept, uint64_t, int) {
        if (kept) {
          const int d = div_b<BS>(i, B);
          tout[rank] = (int32_t)(rb.s + (int64_t)(dblk[d] & ~KEPT_FLAG) * B + (i - d * B));
        }
      }, sm);
  for (int i = Kt + threadIdx.x; i < p.k_tokens; i += NT) tout[i] = -1;
}

// -inf over the blocks of a short row marked in sm.bits.
template <int BS>
DSA_DEV void mask_dropped_short(float* rowp, int64_t cs, int B, int L, int nlb, bool vec,
                                Smem& sm) {
  mask_blocks<BS>(rowp, cs, B, L, 0, nlb, vec,
                  [&](int b) { return ((sm.bits[b >> 5] >> (b & 31)) & 1u) != 0u; });
}

// ---------------------------------------------------------------------------
// A row with nlb <= LIST_CAP: the whole chain in one workgroup, keys in LDS.
// ---------------------------------------------------------------------------
// FUSE_TOK: the token top-k in closed form inside the block emit pass (see
// below).  It costs registers, so it is compiled into the balanced-split
// kernel (decode batches) only; without it the short-row path of the
// per-row-split kernel stays free of scratch.
template <int BS, bool FUSE_TOK>
DSA_DEV void small_row(const Params& p, int r, const Row& rb, Smem& sm) {
  float* rowp = row_ptr(p, r, rb);
  const bool vec = vec_ok(p, rowp);
  const int nlb = rb.nlb, L = rb.L, B = p.B;
  const int Kp = min(p.k_blocks, nlb);
  int32_t* bout = p.block_ids + (int64_t)r * p.k_blocks;
  uint32_t* sel = Kp <= SEL_CAP ? sm.sel : p.ws_sel + (int64_t)r * p.k_blocks;
  const bool need_keys = nlb > p.k_blocks || p.scores != nullptr;
  uint32_t T = 0, q = 0xFFFFFFFFu;
  bool no_low = false, do_mask = false, mask_late = false;
  int n_nonkept = 0;
  if (!need_keys) {
    // Every live block is kept; the result follows from the bounds.
    for (int i = threadIdx.x; i < p.k_blocks; i += NT) bout[i] = i < nlb ? i : -1;
    for (int i = threadIdx.x; i < nlb; i += NT) sel[i] = (uint32_t)i;
  } else {
    float* sc = p.scores ? p.scores + (int64_t)r * p.nblocks : nullptr;
    uint32_t* keys = sm.keys();
    bool low = false;
    // When a select follows, each key's top digit is counted as it is scored
    // (the select's first histogram), and the barrier after the scores
    // completes it.  The histogram is cleared first, behind a barrier of its
    // own: a lane's count may land before another wave's clear otherwise.
    const bool do_select = nlb > Kp;
    // On a contiguous row (B >= 4) the clear runs while the row's first loads
    // are in flight: score_blocks calls it after issuing them, and its barrier
    // waits for the LDS stores only.
    const bool clear_mid = BS >= 4 && vec;
    if (do_select && !clear_mid) {
      for (int j = threadIdx.x; j < HIST_WORDS; j += NT) sm.hist[j] = 0;
      if (!vec)
        for (int j = threadIdx.x; j < (nlb + 31) / 32; j += NT) sm.bits[j] = 0;
      __syncthreads();
    }
    auto clear_hist = [&]() {
      if (do_select && clear_mid) {
        static_assert(HIST_WORDS == 8 * NT, "two 16-byte stores per thread");
        uint4* h4 = reinterpret_cast<uint4*>(sm.hist);   // the first member of Smem
        h4[threadIdx.x] = make_uint4(0, 0, 0, 0);
        h4[threadIdx.x + NT] = make_uint4(0, 0, 0, 0);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
      }
    };
    score_blocks<BS>(rowp, p.col_stride, B, L, 0, nlb, nlb, vec, [&](int b, uint32_t k) {
      keys[b] = k;
      if (sc) sc[b] = key2f(k);
      if (do_select) atomicAdd(&sm.hist[k >> 20], 1u);
    }, low, clear_hist);
    no_low = __syncthreads_or(low) == 0;
    auto getk = [&](int i) { return keys[i]; };
    if (do_select) wg_radix_select<NT>(nlb, (uint32_t)Kp, getk, sm, T, q, true, true);
    // The token top-k in closed form, written by this same pass, when every
    // kept column ranks above -inf (no live value at or below -inf), the
    // newest block is kept (its +inf key is above T) and the kept columns
    // C = (Kp - 1) * B + (the newest block's columns) are at most Kt: the
    // tokens are then the C kept columns plus the first Kt - C columns of the
    // dropped blocks in column order.  In ascending order, kept block i with
    // kept-rank j (all earlier kept blocks whole) starts at position
    // j * B + min(Kt - C, (i - j) * B), and a dropped column c taken by the
    // fill sits at position c - s (every block before it is taken whole).
    const int Kt = min(p.k_tokens, L);
    const int64_t C = (int64_t)(Kp - 1) * B + (L - (int64_t)(nlb - 1) * B);
    const bool fuse_tok = FUSE_TOK && no_low && T < KEY_POS_INF && L > p.k_tokens && C <= Kt;
    const int64_t qt = (int64_t)Kt - C;
    int32_t* tout = p.token_ids + (int64_t)r * p.k_tokens;
    const int32_t s32 = (int32_t)rb.s;
    // One ordered pass: kept ids out, the lowest non-kept ids listed (for the
    // token fill), and each non-kept block masked.  On a contiguous row the
    // lane that owns a block stores it with 16-byte stores as it goes.  On a
    // strided row that would write one word into each of 64 lines per store
    // instruction (and every partial-line write costs a read-modify-write),
    // so the block is marked in a bitmap instead and the -inf stores run
    // column by column across the workgroup at the end (the token stage reads
    // kept columns only).
    do_mask = (p.flags & DSA_WRITE_MASK) && nlb > Kp;
    mask_late = do_mask && !vec;
    uint32_t* nonkept = sm.tkey;
    wg_rule_emit<NT>(nlb, T, q, getk, [&](int i, uint32_t rank, bool kept) {
      const int n = (int)min((int64_t)B, (int64_t)L - (int64_t)i * B);
      if (kept) {
        if (rank < (uint32_t)Kp) {   // (always, for an exact histogram)
          bout[rank] = i;
          if (!fuse_tok) sel[rank] = (uint32_t)i;
          else {
            const int64_t pos = (int64_t)rank * B + min(qt, ((int64_t)i - rank) * B);
            if constexpr (BS > 0) {
#pragma unroll
              for (int e = 0; e < BS; ++e)
                if (e < n) tout[pos + e] = s32 + i * BS + e;
            } else {
              for (int e = 0; e < n; ++e) tout[pos + e] = s32 + i * B + e;
            }
          }
        }
      } else {
        const uint32_t nk = (uint32_t)i - rank;
        if (!fuse_tok) {
          if (nk < (uint32_t)TK_CAP) nonkept[nk] = (uint32_t)i;
        } else if ((int64_t)nk * B < qt) {
          const int m = (int)min((int64_t)n, qt - (int64_t)nk * B);
          for (int e = 0; e < m; ++e) tout[(int64_t)i * B + e] = s32 + i * B + e;
        }
        if (mask_late) atomicOr(&sm.bits[i >> 5], 1u << (i & 31));
        else if (do_mask) mask_block_lane<BS>(rowp, p.col_stride, B, L, vec, i);
      }
    }, sm);
    n_nonkept = min(nlb - Kp, TK_CAP);
    for (int i = Kp + threadIdx.x; i < p.k_blocks; i += NT) bout[i] = -1;
    if (fuse_tok) {
      for (int i = Kt + threadIdx.x; i < p.k_tokens; i += NT) tout[i] = -1;
      if (mask_late) {
        __syncthreads();
        mask_dropped_short<BS>(rowp, p.col_stride, B, L, nlb, vec, sm);
      }
      return;
    }
  }
  __syncthreads();
  token_stage<BS>(p, r, rb, rowp, sel, Kp, T, true, no_low, sm, sm.tkey, n_nonkept);
  if (mask_late) {
    __syncthreads();
    mask_dropped_short<BS>(rowp, p.col_stride, B, L, nlb, vec, sm);
  }
}

// Workgroup-wide ticket on a workspace counter: true in the last of `total`
// arrivals.  Each wave first drains its own stores and atomics.
DSA_DEV bool arrive_last(uint32_t* ticket, uint32_t total, Smem& sm) {
  vm_drain();
  __syncthreads();
  if (threadIdx.x == 0) sm.misc[2] = atomicAdd(ticket, 1u);
  __syncthreads();
  return sm.misc[2] == total - 1;
}

// ---------------------------------------------------------------------------
// Pass 1 of a long row: scores of one chunk, digit histogram, and in the last
// workgroup of the row the digit of the K_blk-th score.
// ---------------------------------------------------------------------------
template <int BS>
DSA_DEV void long_pass1(const Params& p, int r, int b0, int b1, int npieces, const Row& rb,
                        Smem& sm) {
  float* rowp = row_ptr(p, r, rb);
  const bool vec = vec_ok(p, rowp);
  for (int j = threadIdx.x; j < HIST_WORDS; j += NT) sm.hist[j] = 0;
  __syncthreads();
  uint32_t* wk = p.ws_key + (int64_t)r * p.nblocks;
  float* sc = p.scores ? p.scores + (int64_t)r * p.nblocks : nullptr;
  bool low = false;
  constexpr int UNR = BS >= 4 ? UNROLL_LONG : UNROLL;   // (B of 1, 2: registers)
  score_blocks<BS, UNR>(rowp, p.col_stride, p.B, rb.L, b0, b1, rb.nlb, vec, [&](int b, uint32_t k) {
    st_shared(&wk[b], k);
    if (sc) sc[b] = key2f(k);
    atomicAdd(&sm.hist[k >> 20], 1u);
  }, low);
  uint32_t* st = p.ws_row + (int64_t)r * ROW_STATE;
  if (__syncthreads_or(low) && threadIdx.x == 0) atomicOr(&st[4], 1u);
  uint32_t* gh = p.ws_hist + (int64_t)r * HIST_WORDS;
  for (int j = threadIdx.x; j < HIST_WORDS; j += NT) {
    const uint32_t c = sm.hist[j];
    if (c) atomicAdd(&gh[j], c);
  }
  // The row's lists-read flag is cleared before the ticket (pass 2 holds its
  // -inf stores until the final workgroup sets it); once all npieces tickets
  // are in, the pass-2 pieces find the digit from the histogram themselves.
  if (threadIdx.x == 0) st_shared(&st[6], 0u);
  (void)arrive_last(&st[0], 0u, sm);
  (void)npieces;
}

// map[i] = the piece holding entry i of the pieces' concatenated lists, for
// i < n <= 8 * NT (offs: exclusive offsets of the P <= NT pieces): each
// non-empty piece marks its first entry, then a running maximum carries the
// marks forward.  Three barriers.
DSA_DEV void build_piece_map(uint32_t* map, const uint32_t* offs, int P, uint32_t n, Smem& sm) {
  const int t = (int)threadIdx.x;
  uint32_t* mp = map + 8 * t;
  const bool mine = 8u * (uint32_t)t < n;
  if (mine) {
    *reinterpret_cast<uint4*>(mp) = make_uint4(0u, 0u, 0u, 0u);
    *reinterpret_cast<uint4*>(mp + 4) = make_uint4(0u, 0u, 0u, 0u);
  }
  __syncthreads();
  if (t < P) {
    const uint32_t o = offs[t], next = t + 1 < P ? offs[t + 1] : n;
    if (next > o) map[o] = (uint32_t)t;
  }
  __syncthreads();
  uint32_t v[8];
  uint32_t run = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = 0;
  if (mine) {
    const uint4 a = *reinterpret_cast<const uint4*>(mp);
    const uint4 b = *reinterpret_cast<const uint4*>(mp + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      run = max(run, v[e]);
      v[e] = run;
    }
  }
  // The carry from earlier threads: running maximum of the thread maxima.
  const uint32_t inc = wave_incl_max(run);
  if (lane() == 63) sm.wv[wave()] = inc;
  __syncthreads();
  uint32_t carry = 0;
  for (int x = 0; x < wave(); ++x) carry = max(carry, sm.wv[x]);
  const uint32_t prev = (uint32_t)__shfl_up((int)inc, 1, 64);
  if (lane() != 0) carry = max(carry, prev);
  if (mine) {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = max(v[e], carry);
    *reinterpret_cast<uint4*>(mp) = make_uint4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<uint4*>(mp + 4) = make_uint4(v[4], v[5], v[6], v[7]);
  }
  __syncthreads();
}

// Largest j < P with offs[j] <= i (offs nondecreasing, offs[0] = 0).
DSA_DEV int piece_of(const uint32_t* offs, int P, uint32_t i) {
  int lo = 0, hi = P - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (offs[mid] <= i) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// ---------------------------------------------------------------------------
// Last workgroup of pass 2: exact selection among the listed blocks, masks of
// the rejected ones, outputs, token top-k.  General form: the list is
// gathered from the per-piece lists and the token top-k reads the kept
// blocks' values back from the logits.
// ---------------------------------------------------------------------------
template <int BS>
DSA_DEV void final_row_general(const Params& p, int r, const Row& rb, Smem& sm) {
  float* rowp = row_ptr(p, r, rb);
  const bool vec = vec_ok(p, rowp);
  const int nlb = rb.nlb, B = p.B;
  const int P = piece_count(p, sm, rb, r);   // <= NT
  const int64_t cs = p.col_stride;
  const uint32_t* wk = p.ws_key + (int64_t)r * p.nblocks;
  const uint64_t* wl = p.ws_list + (int64_t)r * p.nblocks;
  const uint32_t* st = p.ws_row + (int64_t)r * ROW_STATE;
  const int t = (int)threadIdx.x;
  const bool jt = t < P;
  // One round trip: the row's digit, the keys above it, the piece counts.
  const uint32_t rw = ld_shared(&st[3]);
  const uint32_t digit = ready_digit(rw), above = ready_above(rw);
  const uint32_t c_raw = ld_shared(&p.ws_cnt[(int64_t)r * p.cnt_stride + (jt ? t : 0)]);
  const uint32_t c = jt ? c_raw : 0u;
  // Exclusive prefix of the per-piece list lengths; piece j's list starts at
  // its first block (sm.hist[2 * NT + j]).
  uint32_t n_list;
  const uint32_t off = wg_excl_scan<NT>(c, sm.wv, n_list);
  if (jt) {
    sm.hist[t] = off;
    sm.hist[2 * NT + t] = (uint32_t)piece_start(p, sm, rb, r, t);
  }
  __syncthreads();
  int Kp = min(p.k_blocks, nlb);
  if ((int)n_list < Kp) {
    // Only after a call was cut short (stale workspace): keep the list.
    if (t == 0) atomicOr(p.status, 4u);
    Kp = (int)n_list;
  }
  int32_t* bout = p.block_ids + (int64_t)r * p.k_blocks;
  uint32_t* sel = Kp <= SEL_CAP ? sm.sel : p.ws_sel + (int64_t)r * p.k_blocks;
  const bool write_mask = (p.flags & DSA_WRITE_MASK) != 0;
  uint32_t T = 0, q = 0xFFFFFFFFu;
  constexpr int U = 8;
  if (n_list <= (uint32_t)LIST_CAP) {
    // The list and its keys in LDS: loads issued unconditionally (clamped
    // index), stores guarded.
    uint32_t* lids = sm.ids();
    uint32_t* lkeys = sm.keys();
    uint32_t* pmap = sm.tkey;
    build_piece_map(pmap, sm.hist, P, n_list, sm);
    for (int i0 = t; i0 < (int)n_list; i0 += NT * U) {
      uint32_t src[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t i = (uint32_t)min(i0 + u * NT, (int)n_list - 1);
        const uint32_t j = pmap[i];
        src[u] = sm.hist[2 * NT + j] + (i - sm.hist[j]);
      }
      uint64_t v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = ld_shared64(&wl[src[u]]);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = i0 + u * NT;
        if (i < (int)n_list) {
          lids[i] = (uint32_t)v[u];
          lkeys[i] = (uint32_t)(v[u] >> 32);
        }
      }
    }
    __syncthreads();
    if (t == 0) st_shared(const_cast<uint32_t*>(&st[6]), 1u);   // lists read: -inf may go
    auto getk = [&](int i) { return lkeys[i]; };
    if ((int)n_list > Kp) wg_radix_select_low<NT>((int)n_list, digit, (uint32_t)Kp - above, getk, sm, T, q);
    wg_rule_emit<NT>((int)n_list, T, q, getk, [&](int i, uint32_t rank, bool kept) {
      const uint32_t b = lids[i];
      if (kept) {
        if (rank < (uint32_t)Kp) {
          bout[rank] = (int32_t)b;
          sel[rank] = b;
        }
      } else if (write_mask) {
        mask_block_lane<BS>(rowp, cs, B, rb.L, vec, b);
      }
    }, sm);
  } else {
    // Longer lists: gathered into the workspace, keys read through it.
    uint32_t* lid = p.ws_flat + (int64_t)r * p.nblocks;
    for (int i0 = t; i0 < (int)n_list; i0 += NT * U) {
      uint32_t v[U], src[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t i = (uint32_t)min(i0 + u * NT, (int)n_list - 1);
        const int j = piece_of(sm.hist, P, i);
        src[u] = sm.hist[2 * NT + j] + (i - sm.hist[j]);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = (uint32_t)ld_shared64(&wl[src[u]]);
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (i0 + u * NT < (int)n_list) st_shared(&lid[i0 + u * NT], v[u]);
    }
    vm_drain();
    __syncthreads();
    auto getk = [&](int i) { return ld_shared(&wk[ld_shared(&lid[i])]); };
    if ((int)n_list > Kp) wg_radix_select<NT>((int)n_list, (uint32_t)Kp, getk, sm, T, q);
    wg_select_compact<NT>((int)n_list, T, q, getk,
        [&](int i, uint32_t rank, bool kept, uint64_t, int) {
          const uint32_t b = ld_shared(&lid[i]);
          if (kept) {
            if (rank < (uint32_t)Kp) {
              bout[rank] = (int32_t)b;
              sel[rank] = b;
            }
          } else if (write_mask) {
            mask_one_block(rowp, cs, B, rb.L, b);
          }
        }, sm);
  }
  for (int i = Kp + t; i < p.k_blocks; i += NT) bout[i] = -1;
  __syncthreads();
  const bool no_low = ld_shared(&st[4]) == 0u;
  token_stage<BS>(p, r, rb, rowp, sel, Kp, T, true, no_low, sm);
}


// Last workgroup of pass 2, with the token candidates gathered by pass 2.
// The listed blocks (every block whose key's top digit reaches the digit d of
// the K_blk-th score) come with their keys, so the block top-k only resolves
// the ties inside d's bin.  When at least K_tok values of the kept blocks
// reach beta = d << 20 (each kept block other than the newest has its maximum
// there), the K_tok best columns of the masked row are among the candidates
// (values >= beta of listed blocks) that lie in kept blocks: they are ranked
// there.  Otherwise, and whenever the lists do not fit, the general form runs.
template <int BS>
DSA_DEV void final_row(const Params& p, int r, const Row& rb, Smem& sm) {
  constexpr bool PG_OK = BS >= 4 && BS <= 16;
  if constexpr (!PG_OK) {
    final_row_general<BS>(p, r, rb, sm);
  } else {
    if (!p.pregather) return final_row_general<BS>(p, r, rb, sm);
    const int nlb = rb.nlb, P = piece_count(p, sm, rb, r);
    const int Kp = min(p.k_blocks, nlb), Kt = min(p.k_tokens, rb.L);
    uint32_t* st = p.ws_row + (int64_t)r * ROW_STATE;
    const int t = (int)threadIdx.x;
    // The row's digit and the keys above it, loaded with the piece counts.
    const uint32_t rw = ld_shared(&st[3]);
    const uint32_t digit = ready_digit(rw), above = ready_above(rw);
    const uint32_t beta = digit << 20;
    float* rowp = row_ptr(p, r, rb);
    const bool vec = vec_ok(p, rowp);
    uint32_t* lkeys = sm.keys();
    uint32_t* lids = sm.ids();
    uint32_t* tk = sm.tkey;
    const uint64_t* wl = p.ws_list + (int64_t)r * p.nblocks;
    const int64_t creg = (int64_t)r * 2 * p.nblocks;
    constexpr int U = 8;
    uint32_t n_list, n_cand;
    uint32_t ccol[U];   // candidate t + u * NT: its column (its key goes to tk)
    auto is_fast = [&](bool ovf) {
      return !ovf && beta > KEY_NEG_INF && rb.L > p.k_tokens && n_list >= (uint32_t)Kp &&
             n_list <= (uint32_t)LIST_CAP && n_cand <= (uint32_t)TK_CAP && nlb <= BITMAP_BITS &&
             Kp <= SEL_CAP;
    };
    // Candidate slot u of this thread is candidate cbase + u * cst when
    // u * cst < crem.
    uint32_t cbase = (uint32_t)t, cst = (uint32_t)NT, crem = 0u;
    bool gathered = false;
    if (P <= 64) {
      // Every wave holds the piece table in its lanes (lane j: piece j) and
      // scans it itself, without a barrier.  When every piece's list and
      // candidates fit 8 entries per thread of an equal share of the
      // workgroup (NT / P threads per piece), each thread copies
      // entries of its own piece only, so no search maps entries to pieces,
      // and the lists and candidates come in one round trip.
      const int l = lane();
      const int jl = l < P ? l : 0;
      const uint32_t c_raw = ld_shared(&p.ws_cnt[(int64_t)r * p.cnt_stride + jl]);
      const uint32_t cc_raw = ld_shared(&p.ws_ccnt[(int64_t)r * p.cnt_stride + jl]);
      const uint32_t ps = (uint32_t)piece_start(p, sm, rb, r, jl);
      const bool ovf = ballot(l < P && cc_raw == 0xFFFFFFFFu) != 0;
      const uint32_t c = l < P ? c_raw : 0u;
      const uint32_t cc = (l < P && !ovf) ? cc_raw : 0u;
      const uint32_t cinc = wave_incl_scan(c), ccinc = wave_incl_scan(cc);
      n_list = (uint32_t)__builtin_amdgcn_readlane((int)cinc, 63);
      n_cand = (uint32_t)__builtin_amdgcn_readlane((int)ccinc, 63);
      if (!is_fast(ovf)) return final_row_general<BS>(p, r, rb, sm);
      const uint32_t tpp = (uint32_t)(NT / P);   // threads per piece
      const uint32_t cmax = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_max(max(c, cc)), 63);
      if (cmax <= (uint32_t)U * tpp) {
        const uint32_t off = cinc - c, coff = ccinc - cc;
        const int j = (int)((uint32_t)t / tpp);
        const uint32_t ti = (uint32_t)t - (uint32_t)j * tpp;
        const bool live = j < P;
        const int js = live ? j : 0;
        const uint32_t cj = (uint32_t)__shfl((int)c, js, 64);
        const uint32_t ccj = (uint32_t)__shfl((int)cc, js, 64);
        const uint32_t oj = (uint32_t)__shfl((int)off, js, 64);
        const uint32_t coj = (uint32_t)__shfl((int)coff, js, 64);
        const uint32_t pj = (uint32_t)__shfl((int)ps, js, 64);
        // Clamped indices: every load is issued, only the stores are guarded.
        const uint32_t cl = cj ? cj - 1u : 0u, ccl = ccj ? ccj - 1u : 0u;
        uint64_t vl[U], vc[U];
#pragma unroll
        for (int u = 0; u < U; ++u) vl[u] = ld_shared64(&wl[pj + min(ti + u * tpp, cl)]);
        if (n_cand != 0u) {
#pragma unroll
          for (int u = 0; u < U; ++u)
            vc[u] = ld_shared64(&p.ws_cand[creg + 2 * (int64_t)pj + min(ti + u * tpp, ccl)]);
        } else {
#pragma unroll
          for (int u = 0; u < U; ++u) vc[u] = 0u;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const uint32_t i = ti + u * tpp;
          if (live && i < cj) {
            lids[oj + i] = (uint32_t)vl[u];
            lkeys[oj + i] = (uint32_t)(vl[u] >> 32);
          }
          ccol[u] = (uint32_t)vc[u];
          if (live && i < ccj) tk[coj + i] = (uint32_t)(vc[u] >> 32);
        }
        cbase = coj + ti;
        cst = tpp;
        crem = (live && ccj > ti) ? ccj - ti : 0u;
        gathered = true;
      }
    }
    if (!gathered) {
      const bool jt = t < P;
      const int tc0 = jt ? t : 0;
      const uint32_t c_raw = ld_shared(&p.ws_cnt[(int64_t)r * p.cnt_stride + tc0]);
      const uint32_t cc_raw = ld_shared(&p.ws_ccnt[(int64_t)r * p.cnt_stride + tc0]);
      const uint32_t c = jt ? c_raw : 0u, cc = jt ? cc_raw : 0u;
      const bool ovf = __syncthreads_or(cc == 0xFFFFFFFFu) != 0;
      const uint32_t off = wg_excl_scan<NT>(c, sm.wv, n_list);
      const uint32_t coff = wg_excl_scan<NT>(ovf ? 0u : cc, sm.wv, n_cand);
      if (!is_fast(ovf)) return final_row_general<BS>(p, r, rb, sm);

      // Piece tables (kept until the candidates are gathered; the selects
      // below clear sm.hist): candidate offsets, first blocks, list offsets.
      uint32_t* coffs = sm.sel;
      uint32_t* pstart = sm.sel + NT;
      uint32_t* loffs = sm.sel + 2 * NT;
      if (jt) {
        coffs[t] = coff;
        pstart[t] = (uint32_t)piece_start(p, sm, rb, r, t);
        loffs[t] = off;
      }
      __syncthreads();
      // Gather the list (ids and keys) and the candidate keys in piece order.
      // Loads are issued unconditionally (clamped index) so that a batch is in
      // flight together; only the stores are guarded.
      // Entry -> piece maps (in sm.hist, free until the block select) instead
      // of a search per entry: a search loop between loads would also make the
      // compiler wait for every load issued before it.
      uint32_t* pmap = sm.hist;
      build_piece_map(pmap, loffs, P, n_list, sm);
      for (int i0 = t; i0 < (int)n_list; i0 += NT * U) {
        uint32_t src[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const uint32_t i = (uint32_t)min(i0 + u * NT, (int)n_list - 1);
          const uint32_t j = pmap[i];
          src[u] = pstart[j] + (i - loffs[j]);
        }
        uint64_t v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = ld_shared64(&wl[src[u]]);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int i = i0 + u * NT;
          if (i < (int)n_list) {
            lids[i] = (uint32_t)v[u];
            lkeys[i] = (uint32_t)(v[u] >> 32);
          }
        }
      }
      // Candidate keys to LDS; their columns stay in registers until the list
      // space is free again (n_cand <= TK_CAP = U * NT: one batch).
      __syncthreads();
      build_piece_map(pmap, coffs, P, n_cand, sm);
      {
        uint32_t a[U];
        int64_t src[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const uint32_t i = (uint32_t)min(t + u * NT, max((int)n_cand - 1, 0));
          const uint32_t j = n_cand ? pmap[i] : 0u;
          src[u] = creg + 2 * (int64_t)pstart[j] + (i - coffs[j]);
        }
        const bool any = n_cand != 0;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const uint64_t v = any ? ld_shared64(&p.ws_cand[src[u]]) : 0u;
          ccol[u] = (uint32_t)v;
          a[u] = (uint32_t)(v >> 32);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (t + u * NT < (int)n_cand) tk[t + u * NT] = a[u];
      }
      crem = n_cand > (uint32_t)t ? n_cand - (uint32_t)t : 0u;
    }
    __syncthreads();
    if (t == 0) st_shared(&st[6], 1u);   // the row's lists are read: -inf may go

    // Block top-k: the keys above d's bin are kept; the ties inside it are
    // resolved on the lower 20 bits.  Leaves sm.hist zero.
    uint32_t T = 0, q = 0xFFFFFFFFu;
    auto getk = [&](int i) { return lkeys[i]; };
    if ((int)n_list > Kp) {
      wg_radix_select_low<NT>((int)n_list, digit, (uint32_t)Kp - above, getk, sm, T, q);
    } else {
      for (int j = t; j < HIST_WORDS; j += NT) sm.hist[j] = 0;
      __syncthreads();
    }
    const bool wm = (p.flags & DSA_WRITE_MASK) != 0;
    int32_t* bout = p.block_ids + (int64_t)r * p.k_blocks;
    wg_rule_emit<NT>((int)n_list, T, q, getk, [&](int i, uint32_t rank, bool kept) {
      const uint32_t b = lids[i];
      if (kept) {
        if (rank < (uint32_t)Kp) bout[rank] = (int32_t)b;
        atomicOr(&sm.hist[b >> 5], 1u << (b & 31));    // kept-block bitmap
      } else if (wm) {
        mask_block_lane<BS>(rowp, p.col_stride, BS, rb.L, vec, b);
      }
    }, sm);
    for (int i = Kp + t; i < p.k_blocks; i += NT) bout[i] = -1;
    __syncthreads();

    // Candidate columns; a candidate outside the kept blocks ranks nowhere.
    uint32_t* tc = sm.keys();
    uint32_t nk = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (u * cst < crem) {
        const uint32_t i = cbase + u * cst;
        const uint32_t b = ccol[u] / BS;
        tc[i] = ccol[u];
        if ((sm.hist[b >> 5] >> (b & 31)) & 1u) ++nk;
        else tk[i] = 0u;
      }
    }
    uint32_t n_keep;
    (void)wg_excl_scan<NT>(nk, sm.wv, n_keep);
    if ((int)n_keep < Kt) {
      // Fewer kept values reach beta than tokens wanted: rank the kept
      // blocks' columns from the logits.
      for (int j = t; j < Kp; j += NT) sm.sel[j] = ld_shared(reinterpret_cast<const uint32_t*>(bout + j));
      __syncthreads();
      const bool no_low = ld_shared(&st[4]) == 0u;
      token_stage<BS>(p, r, rb, rowp, sm.sel, Kp, T, true, no_low, sm);
      return;
    }
    uint32_t T2 = 0, q2 = 0xFFFFFFFFu;
    auto gk = [&](int i) { return tk[i]; };
    if ((int)n_cand > Kt) wg_radix_select<NT>((int)n_cand, (uint32_t)Kt, gk, sm, T2, q2);
    int32_t* tout = p.token_ids + (int64_t)r * p.k_tokens;
    wg_rule_emit<NT>((int)n_cand, T2, q2, gk, [&](int i, uint32_t rank, bool kept) {
      if (kept) tout[rank] = (int32_t)(rb.s + tc[i]);
    }, sm);
    for (int i = Kt + t; i < p.k_tokens; i += NT) tout[i] = -1;
  }
}

// Thread 0 waits (time-bounded) until a row-state word reaches `target`; the
// value it saw is left in sm.misc[4].  Returns false if the wait gave up
// (status bit 1).
DSA_DEV bool wait_at_least(const Params& p, const uint32_t* word, uint32_t target, Smem& sm) {
  if (threadIdx.x == 0) {
    uint32_t ok = 1;
    uint32_t v = ld_shared(word);
    if (v < target) {
      const uint64_t t0 = wall_clock64();
      while ((v = ld_shared(word)) < target) {
        __builtin_amdgcn_s_sleep(8);
        if (wall_clock64() - t0 > WAIT_LIMIT_TICKS) {
          atomicOr(p.status, 2u);
          ok = 0;
          break;
        }
      }
    }
    sm.misc[3] = ok;
    sm.misc[4] = v;
  }
  __syncthreads();
  return sm.misc[3] != 0u;
}

// Thread 0 waits at most HOLD_LIMIT_TICKS for a flag; no error if it does not
// come.
DSA_DEV void hold_for(const uint32_t* flag) {
  if (threadIdx.x == 0 && ld_shared(flag) == 0u) {
    const uint64_t t0 = wall_clock64();
    while (ld_shared(flag) == 0u && wall_clock64() - t0 < HOLD_LIMIT_TICKS) __builtin_amdgcn_s_sleep(8);
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Pass 2 of a long row, one piece: first the list of the piece's blocks whose
// top digit reaches the row's digit (and their token candidates), published
// with a count on the row's pass-2 ticket; then -inf over every other block of
// the piece.  The row's final workgroup starts as soon as all lists are in.
// ---------------------------------------------------------------------------
template <int BS>
DSA_DEV void long_pass2(const Params& p, int r, int b0, int b1, int part, int npieces,
                        const Row& rb, Smem& sm) {
  uint32_t* st = p.ws_row + (int64_t)r * ROW_STATE;
  if (!wait_at_least(p, &st[0], (uint32_t)npieces, sm)) return;
  // Every pass-1 ticket is in, so the row's histogram is complete: find the
  // digit d of the K_blk-th block key (every piece does, with the same
  // result) and publish it with the count above d's bin for the final step.
  uint32_t* gh = p.ws_hist + (int64_t)r * HIST_WORDS;
  {
    constexpr int PER = HIST_WORDS / NT;
    uint32_t h[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) h[u] = ld_shared(&gh[threadIdx.x + u * NT]);
#pragma unroll
    for (int u = 0; u < PER; ++u) sm.hist[threadIdx.x + u * NT] = h[u];
    __syncthreads();
  }
  uint32_t digit, above, in_bin;
  find_bin<NT>(sm.hist, HIST_WORDS, (uint32_t)min(p.k_blocks, rb.nlb), sm, digit, above, in_bin);
  if (threadIdx.x == 0) st_shared(&st[3], ready_word(digit, above));
  float* rowp = row_ptr(p, r, rb);
  const bool vec = vec_ok(p, rowp);
  const uint32_t* wk = p.ws_key + (int64_t)r * p.nblocks;
  uint64_t* wl = p.ws_list + (int64_t)r * p.nblocks;
  // Token candidates: every live value of a listed block whose key reaches
  // the lower edge beta of the digit's bin, in column order, into this
  // piece's region of 2 entries per block.
  constexpr bool PG_OK = BS >= 4 && BS <= 16;
  const uint32_t beta = digit << 20;
  const bool pg = PG_OK && p.pregather && beta > KEY_NEG_INF;
  const int64_t creg = (int64_t)r * 2 * p.nblocks + 2 * (int64_t)b0;
  const uint32_t ccap = 2u * (uint32_t)(b1 - b0);
  uint32_t* keys = sm.keys();
  uint32_t* lids = sm.ids();
  // Listed flags of the whole piece, kept for the masking phase when they fit.
  const bool keep_bits = b1 - b0 <= BITMAP_BITS;
  uint32_t* lbits = sm.hist;
  uint32_t cnt = 0, ccnt = 0;
  bool cover = false;
  // Listing, one sub-chunk of CHUNK_CAP blocks at a time: keys in registers
  // (block s0 + threadIdx.x + u * NT), listed flags by ballot, ordered
  // compaction from per-(batch, wave) counts.  The next sub-chunk's keys are
  // loaded while the current one is compacted.  Listed ids also go to LDS
  // (all sub-chunks, in block order) for the candidate pass below.
  constexpr int U = CHUNK_CAP / NT;
  constexpr int NW = NT / 64;
  const int w = wave(), l = lane();
  uint32_t k[U];
  {
    const int n = min(b1 - b0, CHUNK_CAP);
#pragma unroll
    for (int u = 0; u < U; ++u) k[u] = ld_shared(&wk[b0 + min((int)threadIdx.x + u * NT, n - 1)]);
  }
  for (int s0 = b0; s0 < b1; s0 += CHUNK_CAP) {
    const int n = min(b1 - s0, CHUNK_CAP);
    uint64_t m[U];
#pragma unroll
    for (int u = 0; u < U; ++u) m[u] = ballot((int)threadIdx.x + u * NT < n && (k[u] >> 20) >= digit);
    uint32_t kn[U];
    const int s1 = s0 + CHUNK_CAP;
    if (s1 < b1) {
      const int n1 = min(b1 - s1, CHUNK_CAP);
#pragma unroll
      for (int u = 0; u < U; ++u) kn[u] = ld_shared(&wk[s1 + min((int)threadIdx.x + u * NT, n1 - 1)]);
    }
    if (l == 0) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        sm.wv[u * NW + w] = popc(m[u]);
        if (keep_bits) {
          const int wi = ((s0 - b0) >> 5) + ((u * NT + w * 64) >> 5);
          lbits[wi] = (uint32_t)m[u];
          lbits[wi + 1] = (uint32_t)(m[u] >> 32);
        }
      }
    }
    __syncthreads();
    const uint32_t cj = l < U * NW ? sm.wv[l] : 0u;
    const uint32_t cinc = wave_incl_scan(cj);
    const uint32_t nl = (uint32_t)__builtin_amdgcn_readlane((int)cinc, 63);
    const uint32_t cx = cinc - cj;
    const uint32_t base = cnt;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t pb = (uint32_t)__builtin_amdgcn_ds_bpermute((u * NW + w) << 2, (int)cx);
      if ((m[u] >> l) & 1u) {
        const uint32_t rank = base + pb + mbcnt(m[u]);
        const uint32_t b = (uint32_t)(s0 + (int)threadIdx.x + u * NT);
        st_shared64(&wl[b0 + rank], pair(b, k[u]));
        if (rank < (uint32_t)LIST_CAP) lids[rank] = b;
      }
    }
    cnt += nl;
    __syncthreads();
    if (s1 < b1) {
#pragma unroll
      for (int u = 0; u < U; ++u) k[u] = kn[u];
    }
  }
  if constexpr (PG_OK) {
    if (pg && cnt > (uint32_t)LIST_CAP) cover = true;   // the ids did not all fit LDS
    if (pg && !cover) {
      // One listed block per thread per round: its values (loads issued
      // together), the count at or above beta, then ordered stores.
      for (int j0 = 0; j0 < (int)cnt; j0 += NT) {
        const int j = j0 + (int)threadIdx.x;
        uint32_t kk[BS];
        int64_t c0 = 0;
        int nv = 0;
        if (j < (int)cnt) {
          c0 = (int64_t)lids[j] * BS;
          nv = (int)min((int64_t)BS, (int64_t)rb.L - c0);
          if (vec && nv == BS) {
            f4v v[BS / 4];
#pragma unroll
            for (int t = 0; t < BS / 4; ++t) v[t] = *reinterpret_cast<const f4v*>(rowp + c0 + 4 * t);
#pragma unroll
            for (int t = 0; t < BS / 4; ++t) {
              kk[4 * t] = f2key(v[t].x);
              kk[4 * t + 1] = f2key(v[t].y);
              kk[4 * t + 2] = f2key(v[t].z);
              kk[4 * t + 3] = f2key(v[t].w);
            }
          } else {
#pragma unroll
            for (int e = 0; e < BS; ++e) kk[e] = e < nv ? f2key(rowp[(c0 + e) * p.col_stride]) : 0u;
          }
        }
        uint32_t c = 0;
#pragma unroll
        for (int e = 0; e < BS; ++e) c += (e < nv && kk[e] >= beta) ? 1u : 0u;
        uint32_t tot;
        uint32_t o = wg_excl_scan<NT>(c, sm.wv, tot);
        if (ccnt + tot > ccap) {
          cover = true;
          break;
        }
#pragma unroll
        for (int e = 0; e < BS; ++e) {
          if (e < nv && kk[e] >= beta) {
            st_shared64(&p.ws_cand[creg + ccnt + o], pair((uint32_t)(c0 + e), kk[e]));
            ++o;
          }
        }
        ccnt += tot;
      }
      __syncthreads();
    }
  }
  if (threadIdx.x == 0) {
    st_shared(&p.ws_cnt[(int64_t)r * p.cnt_stride + part], cnt);
    st_shared(&p.ws_ccnt[(int64_t)r * p.cnt_stride + part], (pg && !cover) ? ccnt : 0xFFFFFFFFu);
  }
  if (arrive_last(&st[1], (uint32_t)npieces, sm)) {
    // The last piece of the row: every piece has read the histogram, so its
    // non-zero bins and the pass-1 ticket are cleared for the next call.
    constexpr int PER = HIST_WORDS / NT;
    uint32_t h[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) h[u] = ld_shared(&gh[threadIdx.x + u * NT]);
#pragma unroll
    for (int u = 0; u < PER; ++u)
      if (h[u]) st_shared(&gh[threadIdx.x + u * NT], 0u);
    if (threadIdx.x == 0) st_shared(&st[0], 0u);
  }
  if (!(p.flags & DSA_WRITE_MASK)) return;
  // (The balanced split keeps slots free for the final workgroups, which
  // are therefore resident; in the per-row split they may not be.)
  if (p.balanced) hold_for(&st[6]);
  if (keep_bits) {
    mask_blocks<BS>(rowp, p.col_stride, p.B, rb.L, b0, b1, vec, [&](int b) {
      const int i = b - b0;
      return ((lbits[i >> 5] >> (i & 31)) & 1u) == 0u;
    });
    return;
  }
  for (int s0 = b0; s0 < b1; s0 += CHUNK_CAP) {
    const int n = min(b1 - s0, CHUNK_CAP);
    for (int i = threadIdx.x; i < n; i += NT) keys[i] = ld_shared(&wk[s0 + i]);
    __syncthreads();
    mask_blocks<BS>(rowp, p.col_stride, p.B, rb.L, s0, s0 + n, vec,
                    [&](int b) { return (keys[b - s0] >> 20) < digit; });
    __syncthreads();
  }
}

// The final workgroup of a long row: waits until every pass-2 piece of the row
// has published its list, then settles the row and resets its state.
template <int BS>
DSA_DEV void final_wg(const Params& p, int r, const Row& rb, int npieces, Smem& sm) {
  // The final workgroup is the row's critical path and shares its CU with
  // pass-2 pieces issuing -inf stores: with the candidate gather (the
  // shorter final), its waves issue first.  (Measured: 1 us less per call on
  // 1M-wide long rows; without the gather, slightly slower, so not there.)
  if (p.pregather) __builtin_amdgcn_s_setprio(2);
  uint32_t* st = p.ws_row + (int64_t)r * ROW_STATE;
  if (!wait_at_least(p, &st[1], (uint32_t)npieces, sm)) return;
  final_row<BS>(p, r, rb, sm);
  if (threadIdx.x == 0) {
    st_shared(&st[6], 1u);
    st_shared(&st[1], 0u);
    st_shared(&st[3], 0u);
    st_shared(&st[4], 0u);
  }
}

// ---------------------------------------------------------------------------
// The fused kernel.  Grid index g + phase_base < G: pass 1 (and the whole of
// a short row); otherwise pass 2.
// ---------------------------------------------------------------------------
template <int BS, bool FUSE_TOK>
DSA_DEV void own_short_row(const Params& p, int r, const Row& rb, Smem& sm) {
  if (rb.bad && threadIdx.x == 0) atomicOr(p.status, 1u);
  if (rb.L == 0) {
    write_empty_row(p, r);
    return;
  }
  small_row<BS, FUSE_TOK>(p, r, rb, sm);
}

// sm.pfx[0..rows]: blocks of long rows before each row; sm.row_s / row_L:
// each row's start and live length (rows <= 256).
DSA_DEV void build_plan(const Params& p, Smem& sm) {
  const int t = (int)threadIdx.x;
  uint32_t v = 0;
  if (t < p.rows) {
    const Row rb = row_bounds(p, t);
    if (rb.L > 0 && !p.one_group(rb.nlb, rb.L)) v = (uint32_t)rb.nlb;
    sm.row_s[t] = (uint32_t)rb.s;
    sm.row_L[t] = (uint32_t)rb.L;
  }
  uint32_t total;
  const uint32_t x = wg_excl_scan<NT>(v, sm.wv, total);
  if (t < p.rows) sm.pfx[t] = x;
  if (t == 0) {
    sm.pfx[p.rows] = total;
    sm.pfx[p.rows + 1] = ((uint64_t)total + (uint64_t)p.NQ - 1) / (uint64_t)p.NQ;
  }
  __syncthreads();
}

// Bounds of a long row from the plan (no second load of starts and ends).
DSA_DEV Row plan_row(const Params& p, const Smem& sm, int r) {
  Row rb;
  rb.s = sm.row_s[r];
  rb.L = (int32_t)sm.row_L[r];
  rb.nlb = (int32_t)(((int64_t)rb.L + p.B - 1) / p.B);
  rb.bad = false;
  return rb;
}

// Start of piece k of the balanced split, k in [0, NQ + rows - 1]: the pieces
// are cut at every worker boundary min(w * C, T), w = 1..NQ-1, and at every
// row boundary pfx[r], r = 1..rows-1 (empty pieces where two coincide or a
// row is short).  Piece k starts at element k - 1 of the merged boundary list
// (merge-path search; on ties worker boundaries come first), piece 0 at 0 and
// the last piece ends at T.
DSA_DEV uint64_t piece_bound(const Params& p, const Smem& sm, int k) {
  const uint64_t T = sm.pfx[p.rows];
  const int nA = p.NQ - 1, nB = p.rows - 1;
  if (k <= 0) return 0;
  if (k > nA + nB) return T;
  const int m = k - 1;
  auto A = [&](int i) { return worker_lo(sm, p.rows, i + 1); };
  auto Bv = [&](int j) { return sm.pfx[j + 1]; };
  int lo = max(0, m + 1 - nB), hi = min(m + 1, nA);
  while (lo < hi) {
    const int i = (lo + hi) >> 1;
    if (A(i) <= Bv(m - i)) lo = i + 1;
    else hi = i;
  }
  const int i = lo, j = m + 1 - lo;
  const uint64_t a = i > 0 ? A(i - 1) : 0, b = j > 0 ? Bv(j - 1) : 0;
  return a > b ? a : b;
}

// One piece of one pass of the balanced split (one workgroup per piece).
template <int BS>
DSA_DEV void balanced_piece(const Params& p, int k, bool pass2, Smem& sm) {
  build_plan(p, sm);
  const uint64_t T = sm.pfx[p.rows];
  if (T == 0) return;
  const uint64_t s0 = piece_bound(p, sm, k), s1 = piece_bound(p, sm, k + 1);
  if (s0 >= s1) return;
  int r;
  {
    int a = 0, b = p.rows - 1;   // largest r with pfx[r] <= s0: the long row holding s0
    while (a < b) {
      const int m = (a + b + 1) >> 1;
      if (sm.pfx[m] <= s0) a = m;
      else b = m - 1;
    }
    r = a;
  }
  const Row rb = plan_row(p, sm, r);
  const uint64_t rs = sm.pfx[r], re = sm.pfx[r + 1];
  const int w0 = worker_of(sm, p.rows, rs);
  const int np = worker_of(sm, p.rows, re - 1) - w0 + 1;
  const int part = worker_of(sm, p.rows, s0) - w0;
  const int b0 = (int)(s0 - rs), b1 = (int)(s1 - rs);
  if (!pass2) long_pass1<BS>(p, r, b0, b1, np, rb, sm);
  else long_pass2<BS>(p, r, b0, b1, part, np, rb, sm);
}

// ---------------------------------------------------------------------------
// The fused kernels.
// k_fused (per-row split): grid index g + phase_base < G is pass 1 of part
// g / rows of row g % rows (and the whole of a short row), [G, 2G) pass 2,
// then one final workgroup per row.
// k_fused_bal (balanced split): [0, rows) own the short rows, then one
// workgroup per pass-1 piece, one per pass-2 piece (NQ + rows - 1 each), then
// one final workgroup per row.  Every wait is on lower grid indices only.
// ---------------------------------------------------------------------------
template <int BS>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(4))) void k_fused(Params p) {
  __shared__ Smem sm;
  int g = (int)blockIdx.x + p.phase_base;
  if (g >= 2 * p.G) {                 // final workgroups, one per row
    const int r = g - 2 * p.G;
    const Row rb = row_bounds(p, r);
    if (p.one_group(rb.nlb, rb.L) || rb.L == 0) return;
    final_wg<BS>(p, r, rb, p.P, sm);
    return;
  }
  const bool pass2 = g >= p.G;
  if (pass2) g -= p.G;
  int r, part;
  part_of(p, g, r, part);
  const Row rb = row_bounds(p, r);
  if (p.one_group(rb.nlb, rb.L) || rb.L == 0) {
    if (pass2 || part != 0) return;
    own_short_row<BS, false>(p, r, rb, sm);
    return;
  }
  int b0, b1;
  chunk_of(rb, p.P, part, b0, b1);
  if (!pass2) long_pass1<BS>(p, r, b0, b1, p.P, rb, sm);
  else long_pass2<BS>(p, r, b0, b1, part, p.P, rb, sm);
}

template <int BS>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(4))) void k_fused_bal(Params p) {
  __shared__ Smem sm;
  int g = (int)blockIdx.x + p.phase_base;
  if (g < p.rows) {
    const Row rb = row_bounds(p, g);
    if (p.one_group(rb.nlb, rb.L) || rb.L == 0) own_short_row<BS, true>(p, g, rb, sm);
    return;
  }
  g -= p.rows;
  const int npc = p.NQ + p.rows - 1;   // pieces per pass
  if (g >= 2 * npc) {                  // final workgroups, one per row
    const int r = g - 2 * npc;
    build_plan(p, sm);
    if (sm.pfx[r + 1] == sm.pfx[r]) return;   // not a long row
    const Row rb = plan_row(p, sm, r);
    final_wg<BS>(p, r, rb, piece_count(p, sm, rb, r), sm);
    return;
  }
  const bool pass2 = g >= npc;
  balanced_piece<BS>(p, pass2 ? g - npc : g, pass2, sm);
}

// ---------------------------------------------------------------------------
// Standalone steps.
// ---------------------------------------------------------------------------
template <int BS>
__global__ __launch_bounds__(NT) void k_scores(Params p) {
  int r, part;
  part_of(p, (int)blockIdx.x, r, part);
  const Row rb = row_bounds(p, r);
  if (rb.L == 0) return;
  const float* rowp = row_ptr(p, r, rb);
  int b0, b1;
  chunk_of(rb, p.P, part, b0, b1);
  float* sc = p.scores + (int64_t)r * p.nblocks;
  bool low = false;
  score_blocks<BS>(rowp, p.col_stride, p.B, rb.L, b0, b1, rb.nlb, vec_ok(p, rowp),
                   [&](int b, uint32_t k) { sc[b] = key2f(k); }, low);
}

template <int BS>
__global__ __launch_bounds__(NT) void k_mask(Params p) {
  __shared__ uint32_t bits[HIST_WORDS];
  int r, part;
  part_of(p, (int)blockIdx.x, r, part);
  const Row rb = row_bounds(p, r);
  if (rb.L == 0) return;
  float* rowp = row_ptr(p, r, rb);
  const bool vec = vec_ok(p, rowp);
  int b0, b1;
  chunk_of(rb, p.P, part, b0, b1);
  const int32_t* ids = p.in_ids + (int64_t)r * p.k_blocks;
  for (int s0 = b0; s0 < b1; s0 += BITMAP_BITS) {
    const int s1 = min(b1, s0 + BITMAP_BITS);
    for (int j = threadIdx.x; j < (s1 - s0 + 31) / 32; j += NT) bits[j] = 0;
    __syncthreads();
    for (int j = threadIdx.x; j < p.k_blocks; j += NT) {
      const int b = ids[j];
      if (b >= s0 && b < s1) atomicOr(&bits[(b - s0) >> 5], 1u << ((b - s0) & 31));
    }
    __syncthreads();
    mask_blocks<BS>(rowp, p.col_stride, p.B, rb.L, s0, s1, vec, [&](int b) {
      return ((bits[(b - s0) >> 5] >> ((b - s0) & 31)) & 1u) == 0u;
    });
    __syncthreads();
  }
}

template <int BS>
__global__ __launch_bounds__(NT) void k_topk_tokens(Params p) {
  __shared__ Smem sm;
  const int r = blockIdx.x;
  const Row rb = row_bounds(p, r);
  if (rb.L == 0) {
    for (int i = threadIdx.x; i < p.k_tokens; i += NT) p.token_ids[(int64_t)r * p.k_tokens + i] = -1;
    return;
  }
  const float* rowp = row_ptr(p, r, rb);
  if (p.in_ids == nullptr) {
    token_stage<BS>(p, r, rb, rowp, nullptr, 0, 0u, false, false, sm);
    return;
  }
  const int32_t* ids = p.in_ids + (int64_t)r * p.k_blocks;
  uint32_t* sel = p.k_blocks <= SEL_CAP ? sm.sel : p.ws_sel + (int64_t)r * p.k_blocks;
  const int nlb = rb.nlb;
  const uint32_t kp = wg_compact<NT>(p.k_blocks, [&](int j) { return ids[j] >= 0 && ids[j] < nlb; },
                                     [&](int j, uint32_t rank) { sel[rank] = (uint32_t)ids[j]; }, sm);
  __syncthreads();
  token_stage<BS>(p, r, rb, rowp, sel, (int)kp, 0u, false, false, sm);
}


// The kernels a block-size unit launches.
enum class Kernel { Fused, FusedBalanced, Scores, Mask, TopkTokens };

// Launches kernel `k` for block size BS (0: any other size) on `grid`
// workgroups of NT threads.  Defined in dsa_bs_unit.hip, one
// specialisation per translation unit.
template <int BS>
void launch(Kernel k, unsigned grid, const Params& p, hipStream_t stream);
#define DSA_DECLARE_LAUNCH(bs) \
  template <> void launch<bs>(Kernel, unsigned, const Params&, hipStream_t);
DSA_DECLARE_LAUNCH(0)
DSA_DECLARE_LAUNCH(1)
DSA_DECLARE_LAUNCH(2)
DSA_DECLARE_LAUNCH(4)
DSA_DECLARE_LAUNCH(8)
DSA_DECLARE_LAUNCH(16)
DSA_DECLARE_LAUNCH(32)
DSA_DECLARE_LAUNCH(64)
#undef DSA_DECLARE_LAUNCH

}  // namespace dsa

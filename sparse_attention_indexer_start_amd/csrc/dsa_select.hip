// HIP kernels and C ABI for DSA decode-time candidate selection on MI355X.
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
// Launch shape: a grid of rows x P workgroups (P from the shape and CU count
// only), remapped so that a row's workgroups share one XCD.  Trip counts follow
// each row's live range, so the grid is fixed and the calls replay under HIP
// graphs.  A row with at most KEY_CAP live blocks is handled end to end by one
// workgroup from LDS; a longer row is split: pass 1 scores chunks of blocks
// into the workspace and a 12-bit key-digit histogram; the last workgroup of
// the row finds the digit holding the K_blk-th score; pass 2 masks every block
// below that digit and lists the rest, and the last workgroup of pass 2 settles
// the exact selection among the listed blocks, masks the rejected ones and runs
// the token top-k.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <type_traits>

#include "dsa_device.hpp"
#include "dsa_select.h"

namespace dsa {

constexpr int NT = 512;        // threads per workgroup (8 waves)
constexpr int UNROLL = 4;      // float4 loads in flight per lane in the score pass
constexpr int ROW_STATE = 4;   // ticket1, ticket2, digit, spare
constexpr uint32_t KEPT_FLAG = 0x80000000u;

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
  int32_t nblocks, P, G, small_blocks;
  uint32_t flags;
  uint32_t* ws_key;    // [rows][nblocks]
  uint32_t* ws_list;   // [rows][nblocks]
  uint32_t* ws_flat;   // [rows][nblocks]
  uint32_t* ws_hist;   // [rows][HIST_WORDS]
  uint32_t* ws_cnt;    // [rows][P]
  uint32_t* ws_row;    // [rows][ROW_STATE]
  uint32_t* ws_sel;    // [rows][k_blocks]
  uint32_t* ws_dblk;   // [rows][dblk_cap]
  uint32_t* ws_tkey;   // [rows][tkey_cap]
  int64_t dblk_cap, tkey_cap;
  uint32_t* status;
};

struct Row {
  int64_t s;
  int32_t L, nlb;
  bool bad;
};

DSA_DEV Row row_bounds(const Params& p, int r) {
  Row rb;
  const int64_t s = p.starts ? (int64_t)p.starts[r / p.starts_repeat] : 0;
  const int64_t e = (int64_t)p.ends[r / p.ends_repeat];
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

// Grid index -> (row, part).  gridDim.x is a multiple of 8; hardware places
// workgroup g on XCD g % 8, so consecutive logical groups (one row) share an
// XCD and its L2.
DSA_DEV bool map_group(const Params& p, int& r, int& part) {
  const int g = blockIdx.x;
  const int per = gridDim.x >> 3;
  const int logical = (g & 7) * per + (g >> 3);
  if (logical >= p.G) return false;
  r = logical / p.P;
  part = logical - r * p.P;
  return true;
}

DSA_DEV void chunk_of(const Row& rb, int P, int part, int& b0, int& b1) {
  const int cb = (rb.nlb + P - 1) / P;
  b0 = min(rb.nlb, part * cb);
  b1 = min(rb.nlb, b0 + cb);
}

template <int BS>
DSA_DEV int div_b(int64_t x, int B) {
  if constexpr (BS > 0) return (int)(x / BS);
  else return (int)(x / B);
}

// ---------------------------------------------------------------------------
// Block scores of blocks [b0, b1): emit(b, key) once per block.
// ---------------------------------------------------------------------------
template <int BS, class Emit>
DSA_DEV void score_blocks(const float* rowp, int64_t cs, int B, int L, int b0, int b1,
                          int nlb, bool vec, Emit emit) {
  if constexpr (BS >= 4) {
    constexpr int G = BS / 4;          // lanes per block, 4 columns per lane
    const int64_t cbeg = (int64_t)b0 * BS;
    const int64_t cend = min((int64_t)b1 * BS, (int64_t)L);
    const int64_t t4 = (int64_t)threadIdx.x * 4;
    const int64_t step = (int64_t)NT * 4 * UNROLL;
    const bool leader = (threadIdx.x % G) == 0;
    int64_t c0 = cbeg;
    for (; c0 + step <= cend; c0 += step) {
      uint32_t k[UNROLL];
      if (vec) {
        float4 v[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
          v[u] = *reinterpret_cast<const float4*>(rowp + c0 + (int64_t)u * NT * 4 + t4);
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
          k[u] = max(max(f2key(v[u].x), f2key(v[u].y)), max(f2key(v[u].z), f2key(v[u].w)));
      } else {
        float v[UNROLL][4];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
#pragma unroll
          for (int j = 0; j < 4; ++j) v[u][j] = rowp[(c0 + (int64_t)u * NT * 4 + t4 + j) * cs];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
          k[u] = max(max(f2key(v[u][0]), f2key(v[u][1])), max(f2key(v[u][2]), f2key(v[u][3])));
      }
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const uint32_t m = group_max<G>(k[u]);
        if (leader) {
          const int b = (int)((c0 + (int64_t)u * NT * 4 + t4) / BS);
          emit(b, b == nlb - 1 ? KEY_POS_INF : m);
        }
      }
    }
    for (; c0 < cend; c0 += (int64_t)NT * 4) {
      const int64_t col = c0 + t4;
      uint32_t m = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (col + j < cend) m = max(m, f2key(rowp[(col + j) * cs]));
      m = group_max<G>(m);
      if (leader && col < cend) {
        const int b = (int)(col / BS);
        emit(b, b == nlb - 1 ? KEY_POS_INF : m);
      }
    }
  } else if constexpr (BS == 1 || BS == 2) {
    const int64_t cbeg = (int64_t)b0 * BS;
    const int64_t cend = min((int64_t)b1 * BS, (int64_t)L);
    for (int64_t col = cbeg + (int64_t)threadIdx.x * 4; col < cend; col += (int64_t)NT * 4) {
      uint32_t k[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) k[j] = (col + j < cend) ? f2key(rowp[(col + j) * cs]) : 0u;
#pragma unroll
      for (int j = 0; j < 4; j += BS) {
        if (col + j < cend) {
          uint32_t m = k[j];
          if constexpr (BS == 2) m = max(m, k[j + 1]);
          const int b = (int)((col + j) / BS);
          emit(b, b == nlb - 1 ? KEY_POS_INF : m);
        }
      }
    }
  } else {
    // Any block size: one lane per block.
    for (int b = b0 + (int)threadIdx.x; b < b1; b += NT) {
      const int64_t c0 = (int64_t)b * B;
      const int64_t c1 = min(c0 + B, (int64_t)L);
      uint32_t m = 0;
      for (int64_t c = c0; c < c1; ++c) m = max(m, f2key(rowp[c * cs]));
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
  const float ninf = __uint_as_float(NEG_INF_BITS);
  const int64_t cbeg = (int64_t)b0 * B;
  const int64_t cend = min((int64_t)b1 * B, (int64_t)L);
  if constexpr (BS >= 4) {
    for (int64_t col = cbeg + (int64_t)threadIdx.x * 4; col < cend; col += (int64_t)NT * 4) {
      if (!masked((int)(col / BS))) continue;
      if (vec && col + 4 <= cend) {
        *reinterpret_cast<float4*>(rowp + col) = make_float4(ninf, ninf, ninf, ninf);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (col + j < cend) rowp[(col + j) * cs] = ninf;
      }
    }
  } else {
    for (int64_t col = cbeg + (int64_t)threadIdx.x; col < cend; col += NT)
      if (masked(div_b<BS>(col, B))) rowp[col * cs] = ninf;
  }
}

// ---------------------------------------------------------------------------
// Token top-k of one row (one workgroup).  sel: ascending kept block ids (Kp of
// them); nullptr means the row is ranked as it stands.  The ranked domain is
// every kept block plus the F = ceil(Kt/B) lowest non-kept blocks, in block
// order: a non-kept column ranks as -inf, and no -inf column beyond the first
// Kt of them can enter the top Kt, so the result equals ranking the whole
// masked row.
// ---------------------------------------------------------------------------
template <int BS>
DSA_DEV void token_stage(const Params& p, int r, const Row& rb, const float* rowp,
                         const uint32_t* sel, int Kp, Smem& sm) {
  const int L = rb.L, nlb = rb.nlb, B = p.B;
  const int64_t cs = p.col_stride;
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
  // Part 1: blocks below nlow, kept ones and the first F others.
  auto lowkey = [&](int b) -> uint32_t { return ((lowbits[b >> 5] >> (b & 31)) & 1u) ? 2u : 1u; };
  const uint32_t n1 = wg_select_compact<NT>(nlow, 1u, (uint32_t)F, lowkey,
      [&](int b, uint32_t rank, bool kept, uint64_t, int) {
        if (kept) dblk[rank] = (uint32_t)b | (lowkey(b) == 2u ? KEPT_FLAG : 0u);
      }, sm);
  // Part 2: kept blocks at or above nlow, in order.
  const uint32_t n2 = wg_compact<NT>(Kp, [&](int j) { return sel[j] >= (uint32_t)nlow; },
      [&](int j, uint32_t rank) { dblk[n1 + rank] = sel[j] | KEPT_FLAG; }, sm);
  __syncthreads();
  const int nd = (int)(n1 + n2);
  const int last = (int)(dblk[nd - 1] & ~KEPT_FLAG);
  const int nc = (nd - 1) * B + min(B, L - last * B);
  uint32_t* tkey = nc <= TK_CAP ? sm.tkey : p.ws_tkey + (int64_t)r * p.tkey_cap;
  for (int i = threadIdx.x; i < nc; i += NT) {
    const int d = div_b<BS>(i, B);
    const uint32_t e = dblk[d];
    const int64_t c = (int64_t)(e & ~KEPT_FLAG) * B + (i - d * B);
    tkey[i] = ((e & KEPT_FLAG) && c < L) ? f2key(rowp[c * cs]) : KEY_NEG_INF;
  }
  __syncthreads();
  uint32_t T = 0, q = 0xFFFFFFFFu;
  auto getk = [&](int i) { return tkey[i]; };
  if (nc > Kt) wg_radix_select<NT>(nc, (uint32_t)Kt, getk, sm, T, q);
  wg_select_compact<NT>(nc, T, q, getk,
      [&](int i, uint32_t rank, bool kept, uint64_t, int) {
        if (kept) {
          const int d = div_b<BS>(i, B);
          tout[rank] = (int32_t)(rb.s + (int64_t)(dblk[d] & ~KEPT_FLAG) * B + (i - d * B));
        }
      }, sm);
  for (int i = Kt + threadIdx.x; i < p.k_tokens; i += NT) tout[i] = -1;
}

DSA_DEV void write_empty_row(const Params& p, int r) {
  if (p.block_ids)
    for (int i = threadIdx.x; i < p.k_blocks; i += NT) p.block_ids[(int64_t)r * p.k_blocks + i] = -1;
  if (p.token_ids)
    for (int i = threadIdx.x; i < p.k_tokens; i += NT) p.token_ids[(int64_t)r * p.k_tokens + i] = -1;
}

// ---------------------------------------------------------------------------
// A row with nlb <= KEY_CAP: the whole chain in one workgroup, keys in LDS.
// ---------------------------------------------------------------------------
template <int BS>
DSA_DEV void small_row(const Params& p, int r, const Row& rb, Smem& sm) {
  float* rowp = row_ptr(p, r, rb);
  const bool vec = vec_ok(p, rowp);
  const int nlb = rb.nlb, L = rb.L, B = p.B;
  const int Kp = min(p.k_blocks, nlb);
  int32_t* bout = p.block_ids + (int64_t)r * p.k_blocks;
  uint32_t* sel = Kp <= SEL_CAP ? sm.sel : p.ws_sel + (int64_t)r * p.k_blocks;
  const bool need_keys = nlb > p.k_blocks || p.scores != nullptr;
  if (!need_keys) {
    // Every live block is kept; the result follows from the bounds.
    for (int i = threadIdx.x; i < p.k_blocks; i += NT) bout[i] = i < nlb ? i : -1;
    for (int i = threadIdx.x; i < nlb; i += NT) sel[i] = (uint32_t)i;
  } else {
    float* sc = p.scores ? p.scores + (int64_t)r * p.nblocks : nullptr;
    score_blocks<BS>(rowp, p.col_stride, B, L, 0, nlb, nlb, vec, [&](int b, uint32_t k) {
      sm.keys()[b] = k;
      if (sc) sc[b] = key2f(k);
    });
    __syncthreads();
    uint32_t T = 0, q = 0xFFFFFFFFu;
    auto getk = [&](int i) { return sm.keys()[i]; };
    if (nlb > Kp) wg_radix_select<NT>(nlb, (uint32_t)Kp, getk, sm, T, q);
    wg_select_compact<NT>(nlb, T, q, getk,
        [&](int i, uint32_t rank, bool kept, uint64_t word, int base) {
          if (kept) {
            bout[rank] = i;
            sel[rank] = (uint32_t)i;
          }
          if (i == base) {
            sm.selbits[base >> 5] = (uint32_t)word;
            sm.selbits[(base >> 5) + 1] = (uint32_t)(word >> 32);
          }
        }, sm);
    for (int i = Kp + threadIdx.x; i < p.k_blocks; i += NT) bout[i] = -1;
    __syncthreads();
    if ((p.flags & DSA_WRITE_MASK) && nlb > Kp)
      mask_blocks<BS>(rowp, p.col_stride, B, L, 0, nlb, vec,
                      [&](int b) { return ((sm.selbits[b >> 5] >> (b & 31)) & 1u) == 0u; });
  }
  __syncthreads();
  token_stage<BS>(p, r, rb, rowp, sel, Kp, sm);
}

// Workgroup-wide ticket: returns true in the last of `total` arrivals.  Every
// thread fences its own global writes before the barrier; after a true return
// every thread has acquired the other workgroups' writes.
DSA_DEV bool arrive_last(uint32_t* ticket, uint32_t total, Smem& sm) {
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) sm.misc[2] = atomicAdd(ticket, 1u);
  __syncthreads();
  const bool last = sm.misc[2] == total - 1;
  if (last) __threadfence();
  return last;
}

// ---------------------------------------------------------------------------
// Fused pass 1: small rows end to end; long rows: chunk scores + histogram,
// and the last workgroup of the row finds the digit of the K_blk-th score.
// ---------------------------------------------------------------------------
template <int BS>
__global__ __launch_bounds__(NT) void k_fused_p1(Params p) {
  __shared__ Smem sm;
  int r, part;
  if (!map_group(p, r, part)) return;
  const Row rb = row_bounds(p, r);
  if (rb.nlb <= p.small_blocks) {
    if (part != 0) return;
    if (rb.bad && threadIdx.x == 0) atomicOr(p.status, 1u);
    if (rb.L == 0) {
      write_empty_row(p, r);
      return;
    }
    small_row<BS>(p, r, rb, sm);
    return;
  }
  float* rowp = row_ptr(p, r, rb);
  const bool vec = vec_ok(p, rowp);
  int b0, b1;
  chunk_of(rb, p.P, part, b0, b1);
  for (int j = threadIdx.x; j < HIST_WORDS; j += NT) sm.hist[j] = 0;
  __syncthreads();
  uint32_t* wk = p.ws_key + (int64_t)r * p.nblocks;
  float* sc = p.scores ? p.scores + (int64_t)r * p.nblocks : nullptr;
  score_blocks<BS>(rowp, p.col_stride, p.B, rb.L, b0, b1, rb.nlb, vec, [&](int b, uint32_t k) {
    wk[b] = k;
    if (sc) sc[b] = key2f(k);
    atomicAdd(&sm.hist[k >> 20], 1u);
  });
  __syncthreads();
  uint32_t* gh = p.ws_hist + (int64_t)r * HIST_WORDS;
  for (int j = threadIdx.x; j < HIST_WORDS; j += NT) {
    const uint32_t c = sm.hist[j];
    if (c) atomicAdd(&gh[j], c);
  }
  uint32_t* st = p.ws_row + (int64_t)r * ROW_STATE;
  if (!arrive_last(&st[0], (uint32_t)p.P, sm)) return;
  for (int j = threadIdx.x; j < HIST_WORDS; j += NT) {
    sm.hist[j] = gh[j];
    gh[j] = 0;                        // clean for the next call
  }
  __syncthreads();
  uint32_t d, above;
  find_bin<NT>(sm.hist, HIST_WORDS, (uint32_t)min(p.k_blocks, rb.nlb), sm, d, above);
  if (threadIdx.x == 0) {
    st[2] = d;
    st[0] = 0;                        // reset the ticket for the next call
  }
}

// ---------------------------------------------------------------------------
// Fused pass 2 (long rows): mask blocks below the digit, list the others; the
// last workgroup of the row finishes the row.
// ---------------------------------------------------------------------------
template <int BS>
DSA_DEV void final_row(const Params& p, int r, const Row& rb, Smem& sm) {
  float* rowp = row_ptr(p, r, rb);
  const int nlb = rb.nlb, B = p.B, P = p.P;
  const int64_t cs = p.col_stride;
  const int cb = (nlb + P - 1) / P;
  const uint32_t* cnt = p.ws_cnt + (int64_t)r * P;
  const uint32_t* wk = p.ws_key + (int64_t)r * p.nblocks;
  const uint32_t* wl = p.ws_list + (int64_t)r * p.nblocks;
  // Exclusive prefix of the per-chunk list lengths (P <= NT).
  const uint32_t c = (int)threadIdx.x < P ? cnt[threadIdx.x] : 0u;
  uint32_t n_list;
  const uint32_t off = wg_excl_scan<NT>(c, sm.wv, n_list);
  if ((int)threadIdx.x < P) sm.hist[threadIdx.x] = off;
  __syncthreads();
  const bool in_lds = n_list <= (uint32_t)KEY_CAP;
  uint32_t* lid = in_lds ? sm.ids() : p.ws_flat + (int64_t)r * p.nblocks;
  for (int t = 0; t < P; ++t) {
    const uint32_t ct = cnt[t], ot = sm.hist[t];
    const int b0 = min(nlb, t * cb);
    for (int j = threadIdx.x; j < (int)ct; j += NT) lid[ot + j] = wl[b0 + j];
  }
  __syncthreads();
  if (in_lds) {
    for (int i = threadIdx.x; i < (int)n_list; i += NT) sm.keys()[i] = wk[lid[i]];
    __syncthreads();
  }
  auto getk = [&](int i) { return in_lds ? sm.keys()[i] : wk[lid[i]]; };
  int Kp = min(p.k_blocks, nlb);
  if ((int)n_list < Kp) {
    // Only after a call was cut short (stale workspace): keep the list.
    if (threadIdx.x == 0) atomicOr(p.status, 4u);
    Kp = (int)n_list;
  }
  uint32_t T = 0, q = 0xFFFFFFFFu;
  if ((int)n_list > Kp) wg_radix_select<NT>((int)n_list, (uint32_t)Kp, getk, sm, T, q);
  int32_t* bout = p.block_ids + (int64_t)r * p.k_blocks;
  uint32_t* sel = Kp <= SEL_CAP ? sm.sel : p.ws_sel + (int64_t)r * p.k_blocks;
  const bool write_mask = (p.flags & DSA_WRITE_MASK) != 0;
  const float ninf = __uint_as_float(NEG_INF_BITS);
  wg_select_compact<NT>((int)n_list, T, q, getk,
      [&](int i, uint32_t rank, bool kept, uint64_t, int) {
        const uint32_t b = lid[i];
        if (kept) {
          bout[rank] = (int32_t)b;
          sel[rank] = b;
        } else if (write_mask) {
          const int64_t c0 = (int64_t)b * B;
          const int64_t c1 = min(c0 + B, (int64_t)rb.L);
          for (int64_t col = c0; col < c1; ++col) rowp[col * cs] = ninf;
        }
      }, sm);
  for (int i = Kp + threadIdx.x; i < p.k_blocks; i += NT) bout[i] = -1;
  __syncthreads();
  token_stage<BS>(p, r, rb, rowp, sel, Kp, sm);
}

template <int BS>
__global__ __launch_bounds__(NT) void k_fused_p2(Params p) {
  __shared__ Smem sm;
  int r, part;
  if (!map_group(p, r, part)) return;
  const Row rb = row_bounds(p, r);
  if (rb.nlb <= p.small_blocks) return;
  float* rowp = row_ptr(p, r, rb);
  const bool vec = vec_ok(p, rowp);
  int b0, b1;
  chunk_of(rb, p.P, part, b0, b1);
  uint32_t* st = p.ws_row + (int64_t)r * ROW_STATE;
  const uint32_t digit = st[2];
  const uint32_t* wk = p.ws_key + (int64_t)r * p.nblocks;
  uint32_t* wl = p.ws_list + (int64_t)r * p.nblocks;
  const uint32_t n = wg_compact<NT>(b1 - b0, [&](int i) { return (wk[b0 + i] >> 20) >= digit; },
                                    [&](int i, uint32_t rank) { wl[b0 + rank] = (uint32_t)(b0 + i); }, sm);
  if (threadIdx.x == 0) p.ws_cnt[(int64_t)r * p.P + part] = n;
  if (p.flags & DSA_WRITE_MASK)
    mask_blocks<BS>(rowp, p.col_stride, p.B, rb.L, b0, b1, vec,
                    [&](int b) { return (wk[b] >> 20) < digit; });
  if (!arrive_last(&st[1], (uint32_t)p.P, sm)) return;
  final_row<BS>(p, r, rb, sm);
  if (threadIdx.x == 0) st[1] = 0;
}

// ---------------------------------------------------------------------------
// Standalone steps.
// ---------------------------------------------------------------------------
template <int BS>
__global__ __launch_bounds__(NT) void k_scores(Params p) {
  int r, part;
  if (!map_group(p, r, part)) return;
  const Row rb = row_bounds(p, r);
  if (rb.L == 0) return;
  const float* rowp = row_ptr(p, r, rb);
  int b0, b1;
  chunk_of(rb, p.P, part, b0, b1);
  float* sc = p.scores + (int64_t)r * p.nblocks;
  score_blocks<BS>(rowp, p.col_stride, p.B, rb.L, b0, b1, rb.nlb, vec_ok(p, rowp),
                   [&](int b, uint32_t k) { sc[b] = key2f(k); });
}

template <int BS>
__global__ __launch_bounds__(NT) void k_mask(Params p) {
  __shared__ uint32_t bits[HIST_WORDS];
  int r, part;
  if (!map_group(p, r, part)) return;
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
    token_stage<BS>(p, r, rb, rowp, nullptr, 0, sm);
    return;
  }
  const int32_t* ids = p.in_ids + (int64_t)r * p.k_blocks;
  uint32_t* sel = p.k_blocks <= SEL_CAP ? sm.sel : p.ws_sel + (int64_t)r * p.k_blocks;
  const int nlb = rb.nlb;
  const uint32_t kp = wg_compact<NT>(p.k_blocks, [&](int j) { return ids[j] >= 0 && ids[j] < nlb; },
                                     [&](int j, uint32_t rank) { sel[rank] = (uint32_t)ids[j]; }, sm);
  __syncthreads();
  token_stage<BS>(p, r, rb, rowp, sel, (int)kp, sm);
}

}  // namespace dsa

// ===========================================================================
// Host side: the C ABI.
// ===========================================================================
using namespace dsa;

struct dsa_ctx {
  dsa_shape sh;
  int device;
  int cus;
  int32_t nblocks, P, G, Gpad, small_blocks;
  int64_t dblk_cap, tkey_cap;
  void* ws;
  size_t ws_bytes;
  uint32_t *ws_key, *ws_list, *ws_flat, *ws_hist, *ws_cnt, *ws_row, *ws_sel, *ws_dblk, *ws_tkey,
      *status;
  uint32_t magic;
};

namespace {

constexpr uint32_t CTX_MAGIC = 0x44534131u;
thread_local std::string g_err;

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

template <class F>
void with_bs(int B, F&& f) {
  switch (B) {
    case 1: f(std::integral_constant<int, 1>{}); break;
    case 2: f(std::integral_constant<int, 2>{}); break;
    case 4: f(std::integral_constant<int, 4>{}); break;
    case 8: f(std::integral_constant<int, 8>{}); break;
    case 16: f(std::integral_constant<int, 16>{}); break;
    case 32: f(std::integral_constant<int, 32>{}); break;
    case 64: f(std::integral_constant<int, 64>{}); break;
    default: f(std::integral_constant<int, 0>{}); break;
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
  p.small_blocks = c->small_blocks;
  p.ws_key = c->ws_key;
  p.ws_list = c->ws_list;
  p.ws_flat = c->ws_flat;
  p.ws_hist = c->ws_hist;
  p.ws_cnt = c->ws_cnt;
  p.ws_row = c->ws_row;
  p.ws_sel = c->ws_sel;
  p.ws_dblk = c->ws_dblk;
  p.ws_tkey = c->ws_tkey;
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

int launch_check(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, what);
  return DSA_OK;
}

}  // namespace

extern "C" {

const char* dsa_last_error(void) { return g_err.c_str(); }

int dsa_select_init(const dsa_shape* s, int device, dsa_ctx** out) {
  if (out == nullptr) return fail(DSA_ERR_INVALID_ARG, "out is null");
  *out = nullptr;
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

  dsa_ctx* c = new (std::nothrow) dsa_ctx;
  if (!c) return fail(DSA_ERR_HIP, "host allocation failed");
  std::memset(c, 0, sizeof(*c));
  c->sh = *s;
  c->device = device;
  c->magic = CTX_MAGIC;
  const int64_t nb = s->width > 0 ? (s->width + s->block_size - 1) / s->block_size : 0;
  c->nblocks = (int32_t)nb;
  c->small_blocks = KEY_CAP;

  int rc = on_device(device, [&]() -> int {
    hipDeviceProp_t prop;
    hipError_t e = hipGetDeviceProperties(&prop, device);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
    c->cus = prop.multiProcessorCount;
    // Workgroups per row: enough groups to cover the CUs several times over,
    // no more than one per 256 blocks of the buffer, and at most NT.
    const int64_t target = (int64_t)c->cus * 8;
    int64_t P = s->rows > 0 ? (target + s->rows - 1) / s->rows : 1;
    const int64_t pmax = std::max<int64_t>(1, (nb + 255) / 256);
    P = std::max<int64_t>(1, std::min<int64_t>({P, pmax, (int64_t)NT}));
    c->P = (int32_t)P;
    const int64_t G = P * s->rows;
    if (G > (int64_t)1 << 30) return fail(DSA_ERR_UNSUPPORTED, "too many rows");
    c->G = (int32_t)G;
    c->Gpad = (int32_t)((G + 7) / 8 * 8);
    const int64_t F = (s->k_tokens + s->block_size - 1) / s->block_size;
    // Token domain of a row: at most nlow + Kp <= 2*K_blk + F blocks (also
    // with repeated ids given to the standalone token top-k).
    c->dblk_cap = 2 * (int64_t)s->k_blocks + F + 1;
    c->tkey_cap = c->dblk_cap * s->block_size;
    if (empty_shape(c)) return DSA_OK;
    const bool long_rows = nb > c->small_blocks;
    const int64_t R = s->rows;
    const int64_t n_key = long_rows ? R * nb : 0;
    const int64_t n_hist = long_rows ? R * HIST_WORDS : 0;
    const int64_t n_cnt = long_rows ? R * P : 0;
    const int64_t words[] = {n_key, n_key, n_key, n_hist, n_cnt, R * ROW_STATE,
                             R * s->k_blocks, R * c->dblk_cap, R * c->tkey_cap, 64};
    int64_t total = 0;
    for (int64_t w : words) total += (w + 63) / 64 * 64;
    c->ws_bytes = (size_t)total * 4;
    e = hipMalloc(&c->ws, c->ws_bytes);
    if (e != hipSuccess) return hip_fail(e, "hipMalloc(workspace)");
    e = hipMemset(c->ws, 0, c->ws_bytes);
    if (e != hipSuccess) return hip_fail(e, "hipMemset(workspace)");
    e = hipDeviceSynchronize();
    if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize");
    uint32_t* base = static_cast<uint32_t*>(c->ws);
    uint32_t** slots[] = {&c->ws_key, &c->ws_list, &c->ws_flat, &c->ws_hist, &c->ws_cnt,
                          &c->ws_row, &c->ws_sel, &c->ws_dblk, &c->ws_tkey, &c->status};
    int64_t pos = 0;
    for (int i = 0; i < 10; ++i) {
      *slots[i] = words[i] ? base + pos : nullptr;
      pos += (words[i] + 63) / 64 * 64;
    }
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

int dsa_select_query(const dsa_ctx* c, dsa_launch_info* info) {
  int rc = check_ctx(c);
  if (rc != DSA_OK) return rc;
  if (!info) return fail(DSA_ERR_INVALID_ARG, "info is null");
  info->programs_per_row = c->P;
  info->threads_per_group = NT;
  info->grid_groups = c->Gpad;
  info->small_row_blocks = c->small_blocks;
  info->workspace_bytes = (int64_t)c->ws_bytes;
  info->fused_launches = c->nblocks > c->small_blocks ? 2 : 1;
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
    with_bs(p.B, [&](auto bs) {
      hipLaunchKernelGGL((k_scores<decltype(bs)::value>), dim3(c->Gpad), dim3(NT), 0, stream, p);
    });
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
    with_bs(p.B, [&](auto bs) {
      hipLaunchKernelGGL((k_topk_tokens<decltype(bs)::value>), dim3(c->sh.rows), dim3(NT), 0, stream, p);
    });
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
    with_bs(p.B, [&](auto bs) {
      hipLaunchKernelGGL((k_mask<decltype(bs)::value>), dim3(c->Gpad), dim3(NT), 0, stream, p);
    });
    return launch_check("k_mask launch");
  });
}

int dsa_select_fused(dsa_ctx* c, float* logits, const int32_t* starts, const int32_t* ends,
                     int32_t* block_ids, int32_t* token_ids, float* scores, uint32_t flags,
                     hipStream_t stream) {
  int rc = check_ctx(c);
  if (rc != DSA_OK) return rc;
  if (flags & ~(uint32_t)DSA_WRITE_MASK) return fail(DSA_ERR_INVALID_ARG, "unknown flags %#x", flags);
  if (empty_shape(c)) return DSA_OK;
  if (!logits || !ends || !block_ids || !token_ids)
    return fail(DSA_ERR_INVALID_ARG, "logits, ends, block_ids and token_ids must be non-null");
  return on_device(c->device, [&]() -> int {
    Params p = base_params(c);
    p.logits = logits;
    p.starts = starts;
    p.ends = ends;
    p.block_ids = block_ids;
    p.token_ids = token_ids;
    p.scores = scores;
    p.flags = flags;
    const bool two = c->nblocks > c->small_blocks;
    int r2 = DSA_OK;
    with_bs(p.B, [&](auto bs) {
      constexpr int BS = decltype(bs)::value;
      hipLaunchKernelGGL((k_fused_p1<BS>), dim3(c->Gpad), dim3(NT), 0, stream, p);
      if ((r2 = launch_check("k_fused_p1 launch")) != DSA_OK) return;
      if (two) {
        hipLaunchKernelGGL((k_fused_p2<BS>), dim3(c->Gpad), dim3(NT), 0, stream, p);
        r2 = launch_check("k_fused_p2 launch");
      }
    });
    return r2;
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

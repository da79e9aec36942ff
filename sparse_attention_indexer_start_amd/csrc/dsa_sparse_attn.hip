// Sparse attention over each query row's selected tokens (MI355X, gfx950).
//
// The page on vllm PR #57273 ("Qwen4Exp QSA: sm_90 tuning table", Purpose)
// describes the consumer of the selection: grouped-query attention of each
// query over its 2048 selected tokens, read from a paged bf16 K/V cache,
// split over several programs and merged, with a fused output gate.  The page
// on vllm PR #48726 ("LiteDSA: grouped masked sparse attention") requires the
// attention to stay query-exact and reports the log-sum-exp beside the output.
//
// Work unit: one workgroup of four waves per (row, group of 1, 2 or 4 kv
// heads, chunk), a chunk being a run of 32-token steps of the row's id list;
// the waves of one kv head share the steps (with one kv head per workgroup,
// wave w takes steps w, w + 4, ...), so the waves of different heads read the
// same tokens at once.  Per step a wave gathers 32 tokens' K and V rows straight from
// the cache into registers, already in the layout of the matrix instructions
// (no LDS): S^T = K Q^T on v_mfma_f32_16x16x32_bf16 gives each lane one
// query head (lane % 16) and eight tokens, which is both the layout of the
// online softmax (one head per lane, a maximum over the four 16-lane groups)
// and the B operand of O^T = V^T P^T.  The V operand needs eight tokens of one
// dimension per lane; lanes load 16-byte pieces (eight dimensions of one
// token) and byte permutes regroup them.  The four waves merge through LDS;
// with one chunk the workgroup writes the gated bf16 output and the LSE, else
// it writes a partial (maximum, sum, unnormalised output) and the last
// workgroup of the (row, kv head) to arrive merges the partials.
//
// Union mode (the page on vllm PR #48726, "LiteDSA: grouped masked sparse
// attention": one product over the union of neighbouring queries'
// selections, each query still attending exactly its own set).  A first launch merges the ids of each
// group of union_rows consecutive rows into distinct positions, each with a
// bit per row that selected it (k_union), and the attention kernel then runs
// per (group, kv heads, chunk) with the group's (row, head) pairs as the 16
// rows of the matrix tile, reading every union token's K and V once.  Scores
// of tokens a row did not select are -inf before the online softmax, so each
// row's result is its own set's attention.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>

#include "dsa_sparse_attn.h"

#define SA_DEV __device__ __forceinline__

namespace dsa {
namespace sa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int WAVES = 4;
constexpr int NT = 64 * WAVES;
constexpr int STEP = 32;          // tokens per wave step
constexpr int GMAX = 16;          // query heads per kv head (one matrix tile)
constexpr float NEG_INF = -__builtin_huge_valf();

struct Args {
  const uint16_t* q;
  const void* kc;       // bf16 or E4M3 codes
  const void* vc;
  const int32_t* ids;
  const int32_t* table;
  const uint16_t* gate;
  uint16_t* out;
  float* lse;
  float* part_o;        // [pairs * chunks][G][D]
  float* part_ml;       // [pairs * chunks][G][2]
  uint32_t* tickets;    // [rows * hkv / hw]
  uint32_t* status;
  int64_t k_ss, k_hs, v_ss, v_hs, num_slots;
  // hkv and G count head tiles: the group's query heads are cut into tdiv
  // tiles of G heads (kv head k's tiles are k * tdiv .. k * tdiv + tdiv - 1),
  // so that each tile's (row, head) pairs fit one matrix tile.
  int32_t rows, hkv, G, K, rows_per_seq, page_shift, pps, chunks, spc;
  int32_t hw;           // head tiles per workgroup (1, 2 or 4; divides hkv)
  int32_t tdiv;         // head tiles per kv head
  float c2;             // sm_scale * log2(e) (times k_scale for fp8 caches)
  float vscale;         // v_scale for fp8 caches, else 1
  // union mode
  const int2* ent;      // [groups][cap]: (position, bit per row of the group)
  const int32_t* cnt;   // [groups]: union entries of each group
  int32_t U;            // rows per group (1 outside union mode)
  int32_t P;            // (row, head) pairs per tile: G, or U * G
  int32_t cap;          // entries per group, U * K
};

// --- union of a group's ids ------------------------------------------------
constexpr int UNT = 1024;          // threads of the union kernel
constexpr int UWIN = 262144;       // positions per window (a 32 KB presence bitmap)
constexpr int UCAP = 32768;        // largest U * K
constexpr int UIPT = UCAP / UNT;   // ids held per thread

struct UArgs {
  const int32_t* ids;
  int2* ent;
  int32_t* cnt;
  int32_t rows, K, U, cap;
};

SA_DEV uint4 ld16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Eight cache elements at an element offset, as the raw bits a load returns
// and as eight bf16 (E4M3 converts to bf16 exactly; the hardware conversion
// with a unit scale was checked on all 256 codes).
template <bool FP8>
struct KV;
template <>
struct KV<false> {
  typedef uint4 raw;
  static SA_DEV raw ld(const void* base, int64_t off) {
    return *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
  }
  static SA_DEV uint4 bf(raw r) { return r; }
  static SA_DEV raw zero() { return make_uint4(0, 0, 0, 0); }
};
template <>
struct KV<true> {
  typedef uint2 raw;
  static SA_DEV raw ld(const void* base, int64_t off) {
    return *reinterpret_cast<const uint2*>(static_cast<const uint8_t*>(base) + off);
  }
  template <bool HI>
  static SA_DEV uint32_t pk(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
  }
  static SA_DEV uint4 bf(raw r) {
    return make_uint4(pk<false>(r.x), pk<true>(r.x), pk<false>(r.y), pk<true>(r.y));
  }
  static SA_DEV raw zero() { return make_uint2(0, 0); }
};

// Cache slot of position `pos` of sequence `seq`; -1 for padding (pos < 0) and
// for positions that are not addressable (`bad` is then set).
SA_DEV int slot_of(const Args& a, int seq, int pos, bool& bad) {
  if (pos < 0) return -1;
  int64_t slot = pos;
  if (a.table) {
    const int page = pos >> a.page_shift;
    if (page >= a.pps) { bad = true; return -1; }
    const int phys = a.table[(int64_t)seq * a.pps + page];
    if (phys < 0) { bad = true; return -1; }
    slot = ((int64_t)phys << a.page_shift) | (pos & ((1 << a.page_shift) - 1));
  }
  if (slot >= a.num_slots) { bad = true; return -1; }
  return (int)slot;
}

// Block-wide sums and minima over the UNT threads of the union kernel.
SA_DEV int wave_incl_sum(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int x = __shfl_up(v, o);
    if (lane >= o) v += x;
  }
  return v;
}
SA_DEV int wave_min(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o));
  return v;
}

// One workgroup per group of U consecutive rows.  The group's U * K ids are
// placed window by window (UWIN positions each; windows holding no id are
// skipped): every id in the window sets its position's bit in a presence
// bitmap; a block-wide prefix count over the bitmap's words then gives each
// distinct position its union index (so a repeated id counts once), each id
// ORs its row's bit into that entry's 16-bit row mask, and the ids of each
// entry's lowest row write it out as (position, row mask) at its index.  The
// work per thread follows its own ids and bitmap words, not the density of
// the window.  The attention kernel maps positions to cache slots as it does
// for a row's own list.
__global__ void __launch_bounds__(UNT) k_union(UArgs a) {
  constexpr int NW = UWIN / 32;               // bitmap words
  constexpr int WPT = NW / UNT;               // words per thread
  __shared__ uint4 pres4[NW / 4];             // presence bits
  __shared__ int wpre[NW];                    // set bits in earlier words of the window
  __shared__ uint4 mask4[UCAP / 8];           // 16-bit row masks by union index
  __shared__ int wred[UNT / 64];
  __shared__ int wmin[UNT / 64];
  __shared__ int wmax[UNT / 64];
  uint32_t* pres = reinterpret_cast<uint32_t*>(pres4);
  uint32_t* maskw = reinterpret_cast<uint32_t*>(mask4);
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int gi = blockIdx.x;
  const int r0 = gi * a.U, nr = min(a.U, a.rows - r0);
  const int E = nr * a.K;
  const int32_t* ids = a.ids + (int64_t)r0 * a.K;
  // Thread t holds ids t + UNT * i; loads are clamped so that a batch of
  // them is in flight at once, and the value of an index past E is ignored.
  // Up to UNT * BATCH ids (every decode shape) stay in registers; more are
  // re-read from the cache at each pass.
  constexpr int BATCH = 8;
  const bool held = E <= UNT * BATCH;
  int hp[BATCH];
  uint32_t hb[BATCH];                           // bit of the id's row in the group
#pragma unroll
  for (int i = 0; i < BATCH; ++i) {
    const int e = min(t + UNT * i, E - 1);
    hp[i] = ids[e];
    hb[i] = 1u << (e / a.K);
  }
  // fn(position, row bit, valid) over this thread's ids; every lane of a
  // wave takes part in each call (valid is false past E), so that fn may
  // exchange values between lanes.
  auto each_id = [&](auto&& fn) {
    if (held) {
#pragma unroll
      for (int i = 0; i < BATCH; ++i) fn(hp[i], hb[i], t + UNT * i < E);
      return;
    }
#pragma unroll 1
    for (int i0 = 0; i0 < UIPT && 64 * wv + UNT * i0 < E; i0 += BATCH) {   // uniform per wave
      int p[BATCH];
#pragma unroll
      for (int i = 0; i < BATCH; ++i) p[i] = ids[min(t + UNT * (i0 + i), E - 1)];
#pragma unroll
      for (int i = 0; i < BATCH; ++i) {
        const int e = t + UNT * (i0 + i);
        fn(p[i], e < E ? 1u << (e / a.K) : 0u, e < E);
      }
    }
  };
  // lo, hi: the group's lowest and highest position
  int lo = INT32_MAX, hi = -1;
  each_id([&](int p, uint32_t, bool v) {
    if (v && p >= 0) {
      lo = min(lo, p);
      hi = max(hi, p);
    }
  });
  lo = wave_min(lo);
  hi = -wave_min(-hi);
  if (lane == 0) {
    wmin[wv] = lo;
    wmax[wv] = hi;
  }
  __syncthreads();
  lo = INT32_MAX;
#pragma unroll
  for (int k = 0; k < UNT / 64; ++k) {
    lo = min(lo, wmin[k]);
    hi = max(hi, wmax[k]);
  }
  int total = 0;
  int2* ent = a.ent + (int64_t)gi * a.cap;
  while (lo != INT32_MAX) {                     // uniform: every thread holds the same lo
    const int base = lo - lo % UWIN;
    const int64_t end = (int64_t)base + UWIN;
    // Only the bitmap's words up to the group's highest position are used
    // (cleared and scanned); the rest count as empty.
    const int nwc = (int)min((int64_t)NW, ((int64_t)hi - base) / 32 + 1);
    const int nq = (nwc + 3) / 4;               // 16-byte groups of words in use
    for (int k = t; k < nq; k += UNT) pres4[k] = make_uint4(0, 0, 0, 0);
    __syncthreads();                            // cleared
    int nxt = INT32_MAX;
    each_id([&](int p, uint32_t, bool v) {
      const bool in = v && p >= base && p < end;
      const int o = p - base;
      if (in) atomicOr(&pres[o >> 5], 1u << (o & 31));
      if (v && p >= end) nxt = min(nxt, p);
    });
    nxt = wave_min(nxt);
    if (lane == 0) wmin[wv] = nxt;
    __syncthreads();                            // bitmap complete
    // Thread t owns words WPT t .. WPT t + WPT - 1.
    uint32_t w[WPT];
    int c = 0;
#pragma unroll
    for (int k = 0; k < WPT / 4; ++k) {
      const int qk = t * (WPT / 4) + k;
      const uint4 x = qk < nq ? pres4[qk] : make_uint4(0, 0, 0, 0);
      w[4 * k] = x.x; w[4 * k + 1] = x.y; w[4 * k + 2] = x.z; w[4 * k + 3] = x.w;
    }
#pragma unroll
    for (int k = 0; k < WPT; ++k) c += __popc(w[k]);
    const int incl = wave_incl_sum(c, lane);
    if (lane == 63) wred[wv] = incl;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int k = 0; k < UNT / 64; ++k) {
      before += k < wv ? wred[k] : 0;
      all += wred[k];
    }
    {
      int run = before + incl - c;
#pragma unroll
      for (int k = 0; k < WPT; ++k) {
        wpre[WPT * t + k] = run;
        run += __popc(w[k]);
      }
    }
    // the row masks of this window's `all` entries (two per word)
    for (int k = t; k < (all + 7) / 8; k += UNT) mask4[k] = make_uint4(0, 0, 0, 0);
    __syncthreads();                            // union indices known, masks cleared
    each_id([&](int p, uint32_t rb, bool v) {
      if (v && p >= base && p < end) {
        const int o = p - base;
        const int u = wpre[o >> 5] + __popc(pres[o >> 5] & ((1u << (o & 31)) - 1u));
        atomicOr(&maskw[u >> 1], rb << (16 * (u & 1)));
      }
    });
    __syncthreads();                            // row masks complete
    // Each entry is written by the ids of its lowest row (the same value if
    // that row lists the position twice), so that every thread writes at
    // most its own ids' entries however dense the window.
    each_id([&](int p, uint32_t rb, bool v) {
      if (v && p >= base && p < end) {
        const int o = p - base;
        const int u = wpre[o >> 5] + __popc(pres[o >> 5] & ((1u << (o & 31)) - 1u));
        const uint32_t m = (maskw[u >> 1] >> (16 * (u & 1))) & 0xFFFFu;
        if ((m & (0u - m)) == rb) ent[total + u] = make_int2(p, (int)m);
      }
    });
    total += all;
    lo = INT32_MAX;
#pragma unroll
    for (int k = 0; k < UNT / 64; ++k) lo = min(lo, wmin[k]);
    __syncthreads();                            // masks, indices and wred read: clear after
  }
  if (t == 0) a.cnt[gi] = total;
}

// Agent-scope relaxed 64-bit accesses for words one workgroup writes and
// another reads: they compile to coherent loads and stores on gfx950, across
// the XCDs' separate L2 caches.
SA_DEV void st_coh64(float* p, float x, float y) {
  const uint64_t v = (uint64_t)__float_as_uint(x) | ((uint64_t)__float_as_uint(y) << 32);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
SA_DEV float2 ld_coh64(const float* p) {
  const uint64_t v = __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<float*>(p)),
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float((uint32_t)v), __uint_as_float((uint32_t)(v >> 32)));
}

SA_DEV uint32_t word_of(const uint4 x, int k) {
  return k == 0 ? x.x : k == 1 ? x.y : k == 2 ? x.z : x.w;
}

SA_DEV float bf2f(uint32_t b) { return __uint_as_float(b << 16); }

// Round to bf16, nearest even (inputs are finite or +-inf).
SA_DEV uint32_t f2bf(float f) {
  const __bf16 h = (__bf16)f;
  return (uint32_t)__builtin_bit_cast(unsigned short, h);
}

template <int D>
struct __align__(16) Smem {
  float o[WAVES][GMAX][D];
  float m[WAVES][GMAX];
  float l[WAVES][GMAX];
  uint32_t last;
};

// Normalise, gate and store four consecutive dimensions of one head.
SA_DEV void store_out(const Args& a, int row, int h, int d, float4 o, float L, float M, int D) {
  const float inv = L > 0.f ? a.vscale / L : 0.f;
  float v[4] = {o.x * inv, o.y * inv, o.z * inv, o.w * inv};
  const int hq = a.hkv * a.G;
  const int64_t base = ((int64_t)row * hq + h) * D + d;
  if (a.gate) {
    const uint2 g = *reinterpret_cast<const uint2*>(a.gate + base);
    const float gv[4] = {bf2f(g.x & 0xFFFFu), bf2f(g.x >> 16), bf2f(g.y & 0xFFFFu), bf2f(g.y >> 16)};
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = v[i] / (1.f + __expf(-gv[i]));
  }
  uint2 w;
  w.x = f2bf(v[0]) | (f2bf(v[1]) << 16);
  w.y = f2bf(v[2]) | (f2bf(v[3]) << 16);
  *reinterpret_cast<uint2*>(a.out + base) = w;
  if (d == 0 && a.lse)
    a.lse[(int64_t)row * hq + h] = L > 0.f ? (M + __log2f(L)) * 0.69314718055994531f : NEG_INF;
}

// Row and query head of pair h of a tile: the tile of (row or group `ru`,
// kv head g) holds heads g*G .. g*G + G - 1 of one row, or in union mode
// those heads of each of the group's rows in turn.
template <bool UN>
SA_DEV void pair_of(const Args& a, int ru, int g, int h, int& row, int& head) {
  if (UN) {
    const int r = h / a.G;
    row = ru * a.U + r;
    head = g * a.G + (h - r * a.G);
  } else {
    row = ru;
    head = g * a.G + h;
  }
}

template <int D, bool FP8, bool UN>
__global__ void __launch_bounds__(NT, 2) k_sparse_attn(Args a) {
  typedef KV<FP8> T;
  constexpr int KS = D / 32;      // 32-dimension steps of q.k
  constexpr int NC = D / 128;     // 128-dimension halves of V
  constexpr int OT = D / 16;      // 16-dimension output tiles
  __shared__ Smem<D> sm;

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int n = lane & 15, j = lane >> 4;
  // Workgroups are dealt to the eight XCDs in turn (block b to XCD b % 8).
  // XCD x takes the x-th contiguous eighth of the work units instead, so the
  // rows of one sequence (and their cache pages) share one XCD's L2 and
  // address-translation caches.
  int unit;
  {
    const int nb = gridDim.x, per = nb >> 3, rem = nb & 7;
    const int x = blockIdx.x & 7, k = blockIdx.x >> 3;
    unit = x * per + min(x, rem) + k;
  }
  // A workgroup covers hw kv heads of one row over one chunk: wave w works
  // on kv head gb*hw + w % hw, and the waves of one head share the chunk's
  // steps, so the waves of different heads read the same tokens' cache rows
  // (the same pages) at the same time.
  const int gblocks = a.hkv / a.hw, wph = WAVES / a.hw;
  const int wgp = unit / a.chunks, chunk = unit - wgp * a.chunks;
  // ru: the row, or in union mode the group of rows
  const int ru = wgp / gblocks, gb = wgp - ru * gblocks;
  const int g = gb * a.hw + w % a.hw, wi = w / a.hw;
  const int kvh = g / a.tdiv;     // the cache's kv head of head tile g
  const int seq = (UN ? ru * a.U : ru) / a.rows_per_seq;
  const int hq = a.hkv * a.G;
  // (row, head) pairs in the tile: G, or G per row of the group
  const int np = UN ? min(a.U, a.rows - ru * a.U) * a.G : a.G;

  // Query operand: lane (pair n, group j) holds q[row, head, 32s + 8j .. +8].
  uint4 qr[KS];
  {
    int qrow, qhead;
    pair_of<UN>(a, ru, g, min(n, np - 1), qrow, qhead);
    const uint16_t* qp = a.q + ((int64_t)qrow * hq + qhead) * D + 8 * j;
#pragma unroll
    for (int s = 0; s < KS; ++s) qr[s] = n < np ? ld16(qp + 32 * s) : make_uint4(0, 0, 0, 0);
  }
  f32x4 oacc[OT];
#pragma unroll
  for (int t = 0; t < OT; ++t) oacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = NEG_INF, l_run = 0.f;
  bool bad = false;

  // Steps of this chunk.  In union mode the list is the group's union, whose
  // length is known only now; the chunks split it evenly.
  int nlist = a.K, spc = a.spc;
  if (UN) {
    nlist = a.cnt[ru];
    const int st = (nlist + STEP - 1) / STEP;
    spc = (st + a.chunks - 1) / a.chunks;
  }
  const int steps = (nlist + STEP - 1) / STEP;
  const int st0 = chunk * spc, st1 = min(steps, st0 + spc);
  const int32_t* idrow = a.ids + (int64_t)ru * a.K;
  const int2* erow = a.ent + (int64_t)ru * a.cap;

  // Token of step st for this lane: its position (-1 past the chunk or the
  // list), and in union mode its (position, row bits) entry.
  auto pos_of = [&](int st) -> int {
    const int tix = st * STEP + (lane & 31);
    return (st < st1 && tix < nlist) ? idrow[tix] : -1;
  };
  auto ent_of = [&](int st) -> int2 {
    const int tix = st * STEP + (lane & 31);
    return (st < st1 && tix < nlist) ? erow[tix] : make_int2(-1, 0);
  };
  // The next step's id is loaded while this step's K/V loads are in flight,
  // so a step waits for two memory round trips (page table, K/V) instead of
  // three.
  int pos = -1;
  int2 en = make_int2(-1, 0);
  if constexpr (UN) en = ent_of(st0 + wi);
  else pos = pos_of(st0 + wi);
  for (int st = st0 + wi; st < st1; st += wph) {
    int slot;
    uint32_t rbits = 0;
    if constexpr (UN) {
      slot = slot_of(a, seq, en.x, bad);
      rbits = (uint32_t)en.y;
      en = ent_of(st + wph);
    } else {
      slot = slot_of(a, seq, pos, bad);
      pos = pos_of(st + wph);
    }
    if (__ballot(slot >= 0) == 0) continue;        // nothing to attend in this step
    // Union mode: bit t of `mine` says whether this lane's row (pair n) lists
    // token t of the step (lanes t and 32 + t hold the same token).
    uint32_t mine = ~0u;
    if (UN) {
#pragma unroll
      for (int r = 0; r < GMAX; ++r) {
        if (r * a.G < np) {
          const uint32_t b = (uint32_t)__ballot((rbits >> r) & 1u);
          if (n / a.G == r) mine = b;
        }
      }
    }
    // Slots of this lane's tokens: K rows n and 16 + n; V and score tokens
    // 4j + e and 16 + 4j + e (e < 4).
    const int sk0 = __shfl(slot, n), sk1 = __shfl(slot, 16 + n);
    int sv[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sv[e] = __shfl(slot, 4 * j + e);
      sv[4 + e] = __shfl(slot, 16 + 4 * j + e);
    }
    typename T::raw ka[KS], kb[KS];
    {
      const int64_t o0 = (int64_t)max(sk0, 0) * a.k_ss + (int64_t)kvh * a.k_hs + 8 * j;
      const int64_t o1 = (int64_t)max(sk1, 0) * a.k_ss + (int64_t)kvh * a.k_hs + 8 * j;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        ka[s] = sk0 >= 0 ? T::ld(a.kc, o0 + 32 * s) : T::zero();
        kb[s] = sk1 >= 0 ? T::ld(a.kc, o1 + 32 * s) : T::zero();
      }
    }
    typename T::raw vr[8][NC];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int64_t ov = (int64_t)max(sv[e], 0) * a.v_ss + (int64_t)kvh * a.v_hs + 8 * n;
#pragma unroll
      for (int c = 0; c < NC; ++c) vr[e][c] = sv[e] >= 0 ? T::ld(a.vc, ov + 128 * c) : T::zero();
    }
    // Scores S^T[token][head]: lane (n, j) receives tokens 4j + r and 16 + 4j + r.
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, T::bf(ka[s])),
                                                   __builtin_bit_cast(bf16x8, qr[s]), s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, T::bf(kb[s])),
                                                   __builtin_bit_cast(bf16x8, qr[s]), s1, 0, 0, 0);
    }
    float sc[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool m0 = sv[r] >= 0 && ((mine >> (4 * j + r)) & 1u);
      const bool m1 = sv[4 + r] >= 0 && ((mine >> (16 + 4 * j + r)) & 1u);
      sc[r] = m0 ? s0[r] * a.c2 : NEG_INF;
      sc[4 + r] = m1 ? s1[r] * a.c2 : NEG_INF;
    }
    float tmax = sc[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) tmax = fmaxf(tmax, sc[e]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = m_new == NEG_INF ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    float p[8], psum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[e] = __builtin_amdgcn_exp2f(sc[e] - m_use);
      psum += p[e];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (__ballot(alpha != 1.f)) {
#pragma unroll
      for (int t = 0; t < OT; ++t) oacc[t] *= alpha;
    }
    uint4 pw;
    pw.x = f2bf(p[0]) | (f2bf(p[1]) << 16);
    pw.y = f2bf(p[2]) | (f2bf(p[3]) << 16);
    pw.z = f2bf(p[4]) | (f2bf(p[5]) << 16);
    pw.w = f2bf(p[6]) | (f2bf(p[7]) << 16);
    const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
    uint4 vq[8][NC];
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int c = 0; c < NC; ++c) vq[e][c] = T::bf(vr[e][c]);
    // O^T[dim][head] += V^T P^T.  Tile (c, i) holds dimensions 128c + 8m + i
    // (m = row of the tile); its A operand on lane (m = n, j) is the eight
    // tokens' values of dimension 128c + 8n + i, regrouped from vq.
#pragma unroll
    for (int c = 0; c < NC; ++c) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        // bf16 of dimension i: low half of word i/2 (i even) or high half (i odd)
        const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
        uint4 av;
        av.x = __builtin_amdgcn_perm(word_of(vq[1][c], i >> 1), word_of(vq[0][c], i >> 1), sel);
        av.y = __builtin_amdgcn_perm(word_of(vq[3][c], i >> 1), word_of(vq[2][c], i >> 1), sel);
        av.z = __builtin_amdgcn_perm(word_of(vq[5][c], i >> 1), word_of(vq[4][c], i >> 1), sel);
        av.w = __builtin_amdgcn_perm(word_of(vq[7][c], i >> 1), word_of(vq[6][c], i >> 1), sel);
        oacc[c * 8 + i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, av), pb, oacc[c * 8 + i], 0, 0, 0);
      }
    }
  }
  if (__ballot(bad) && lane == 0) atomicOr(a.status, 1u);

  // Merge the four waves through LDS.  Lane (n, j) holds, for tile (c, i) and
  // element r, head n and dimension 128c + 8(4j + r) + i.
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (n < np) {
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float* dst = &sm.o[w][n][128 * c + 32 * j + 8 * r];
        *reinterpret_cast<float4*>(dst) =
            make_float4(oacc[c * 8 + 0][r], oacc[c * 8 + 1][r], oacc[c * 8 + 2][r], oacc[c * 8 + 3][r]);
        *reinterpret_cast<float4*>(dst + 4) =
            make_float4(oacc[c * 8 + 4][r], oacc[c * 8 + 5][r], oacc[c * 8 + 6][r], oacc[c * 8 + 7][r]);
      }
    if (j == 0) {
      sm.m[w][n] = m_run;
      sm.l[w][n] = l_run;
    }
  }
  __syncthreads();

  constexpr int D4 = D / 4;
  const int n4 = np * D4;
  for (int e = threadIdx.x; e < a.hw * n4; e += NT) {
    const int gl = e / n4, e2 = e - gl * n4;
    const int h = e2 / D4, d = (e2 - h * D4) * 4;
    const int gh = gb * a.hw + gl;
    int orow, ohead;
    pair_of<UN>(a, ru, gh, h, orow, ohead);
    float M = NEG_INF;
    for (int v = gl; v < WAVES; v += a.hw) M = fmaxf(M, sm.m[v][h]);
    float L = 0.f;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int v = gl; v < WAVES; v += a.hw) {
      const float f = sm.m[v][h] == NEG_INF ? 0.f : __builtin_amdgcn_exp2f(sm.m[v][h] - M);
      L += sm.l[v][h] * f;
      const float4 x = *reinterpret_cast<const float4*>(&sm.o[v][h][d]);
      o.x += x.x * f; o.y += x.y * f; o.z += x.z * f; o.w += x.w * f;
    }
    if (a.chunks == 1) {
      store_out(a, orow, ohead, d, o, L, M, D);
    } else {
      const int64_t pu = ((int64_t)ru * a.hkv + gh) * a.chunks + chunk;
      float* po = a.part_o + (pu * a.P + h) * D + d;
      st_coh64(po, o.x, o.y);
      st_coh64(po + 2, o.z, o.w);
      if (d == 0) st_coh64(a.part_ml + (pu * a.P + h) * 2, M, L);
    }
  }
  if (a.chunks == 1) return;

  // Last of the (row, kv head)'s chunks to arrive merges the partials.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) sm.last = atomicAdd(&a.tickets[wgp], 1u) == (uint32_t)(a.chunks - 1);
  __syncthreads();
  if (!sm.last) return;
  // Stage every chunk's (maximum, sum) of the workgroup's hw * np pairs in
  // LDS (the wave partials' space, no longer needed), turn each pair's
  // maxima into the chunks' weights there, then sum the partial outputs.
  const int npp = a.hw * np;
  float2* cw = reinterpret_cast<float2*>(&sm.o[0][0][0]);   // [npp][chunks]
  float* pM = &sm.m[0][0];                                    // [npp]
  float* pL = &sm.l[0][0];
  auto unit_of = [&](int pr, int ch, int& h) -> int64_t {
    const int gl = pr / np;
    h = pr - gl * np;
    return ((int64_t)ru * a.hkv + gb * a.hw + gl) * a.chunks + ch;
  };
  for (int e = threadIdx.x; e < npp * a.chunks; e += NT) {
    const int pr = e / a.chunks, ch = e - pr * a.chunks;
    int h;
    const int64_t u = unit_of(pr, ch, h);
    cw[e] = ld_coh64(a.part_ml + (u * a.P + h) * 2);
  }
  __syncthreads();
  for (int pr = threadIdx.x; pr < npp; pr += NT) {
    float2* c = cw + (int64_t)pr * a.chunks;
    float M = NEG_INF;
    for (int ch = 0; ch < a.chunks; ++ch) M = fmaxf(M, c[ch].x);
    float L = 0.f;
    for (int ch = 0; ch < a.chunks; ++ch) {
      const float f = c[ch].x == NEG_INF ? 0.f : __builtin_amdgcn_exp2f(c[ch].x - M);
      L += c[ch].y * f;
      c[ch].x = f;
    }
    pM[pr] = M;
    pL[pr] = L;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < a.hw * n4; e += NT) {
    const int pr = e / D4, d = (e - pr * D4) * 4;
    int h;
    const int64_t u0 = unit_of(pr, 0, h);
    int orow, ohead;
    pair_of<UN>(a, ru, gb * a.hw + pr / np, h, orow, ohead);
    const float2* c = cw + (int64_t)pr * a.chunks;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    int ch = 0;
    for (; ch + 4 <= a.chunks; ch += 4) {
      float2 x[4][2];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float* po = a.part_o + ((u0 + ch + k) * a.P + h) * D + d;
        x[k][0] = ld_coh64(po);
        x[k][1] = ld_coh64(po + 2);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float f = c[ch + k].x;
        o.x += x[k][0].x * f; o.y += x[k][0].y * f; o.z += x[k][1].x * f; o.w += x[k][1].y * f;
      }
    }
    for (; ch < a.chunks; ++ch) {
      const float* po = a.part_o + ((u0 + ch) * a.P + h) * D + d;
      const float2 x0 = ld_coh64(po), x1 = ld_coh64(po + 2);
      const float f = c[ch].x;
      o.x += x0.x * f; o.y += x0.y * f; o.z += x1.x * f; o.w += x1.y * f;
    }
    store_out(a, orow, ohead, d, o, pL[pr], pM[pr], D);
  }
  if (threadIdx.x == 0)
    __hip_atomic_store(&a.tickets[wgp], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace sa
}  // namespace dsa

// ===========================================================================
// Host side
// ===========================================================================
using namespace dsa::sa;

struct dsa_attn_ctx {
  dsa_attn_shape sh;
  int device;
  int chunks, spc, hw;
  int T, hkv, G;        // head tiles per kv head, head tiles in all, query heads per tile
  int U, nru, cap;      // rows per union group (1 outside union mode), groups or rows, U * K
  void* ws;
  size_t ws_bytes, head_bytes;   // workspace, and its part before the union entries
  float *part_o, *part_ml;
  uint32_t *tickets, *status;
  int2* ent;            // union mode: [nru][cap]
  int32_t* cnt;         // union mode: [nru]
  uint32_t magic;
};

namespace {

constexpr uint32_t SA_MAGIC = 0x44534154u;
thread_local std::string g_sa_err;

int sa_fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_sa_err = buf;
  return code;
}

int sa_hip(hipError_t e, const char* what) {
  return sa_fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
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

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

extern "C" {

const char* dsa_sparse_attn_last_error(void) { return g_sa_err.c_str(); }

}  // extern "C"

namespace {

// Validates a shape (everything but the device) and plans its launch on a
// device with `cus` CUs into c: head tiles, tiles per workgroup, chunks and
// the workspace size.  No device call.
int attn_plan(const dsa_attn_shape* s, int cus, dsa_attn_ctx* c) {
  if (!s) return sa_fail(DSA_ERR_INVALID_ARG, "shape is null");
  if (s->rows < 0) return sa_fail(DSA_ERR_INVALID_ARG, "rows must be >= 0");
  if (s->kv_heads < 1) return sa_fail(DSA_ERR_INVALID_ARG, "kv_heads must be >= 1");
  if (s->group < 1) return sa_fail(DSA_ERR_INVALID_ARG, "group must be >= 1 (got %d)", s->group);
  if ((int64_t)s->kv_heads * s->group > (1 << 20))
    return sa_fail(DSA_ERR_UNSUPPORTED, "kv_heads * group must be <= 2^20");
  if (s->head_dim != 128 && s->head_dim != 256)
    return sa_fail(DSA_ERR_UNSUPPORTED, "head_dim must be 128 or 256 (got %d)", s->head_dim);
  if (s->k_tokens < 1) return sa_fail(DSA_ERR_INVALID_ARG, "k_tokens must be >= 1");
  if (s->rows_per_seq < 1) return sa_fail(DSA_ERR_INVALID_ARG, "rows_per_seq must be >= 1");
  if (s->page_size < 1 || (s->page_size & (s->page_size - 1)) || s->page_size > (1 << 24))
    return sa_fail(DSA_ERR_INVALID_ARG, "page_size must be a power of two in [1, 2^24]");
  if (s->pages_per_seq < 0) return sa_fail(DSA_ERR_INVALID_ARG, "pages_per_seq must be >= 0");
  if (s->num_slots < 0 || s->num_slots >= ((int64_t)1 << 31))
    return sa_fail(DSA_ERR_UNSUPPORTED, "num_slots must be in [0, 2^31)");
  const int64_t D = s->head_dim;
  if (s->k_slot_stride % 8 || s->k_head_stride % 8 || s->v_slot_stride % 8 || s->v_head_stride % 8)
    return sa_fail(DSA_ERR_INVALID_ARG, "cache strides must be multiples of 8 elements");
  if (s->k_head_stride < D || s->v_head_stride < D ||
      s->k_slot_stride < (s->kv_heads - 1) * s->k_head_stride + D ||
      s->v_slot_stride < (s->kv_heads - 1) * s->v_head_stride + D)
    return sa_fail(DSA_ERR_INVALID_ARG, "cache strides overlap heads or slots");
  if (s->chunks < 0) return sa_fail(DSA_ERR_INVALID_ARG, "chunks must be >= 0");
  if (s->union_rows < 0) return sa_fail(DSA_ERR_INVALID_ARG, "union_rows must be >= 0");
  if (cus < 1) return sa_fail(DSA_ERR_INVALID_ARG, "cus must be >= 1");
  const int U = std::max(1, s->union_rows);
  if (U > 1) {
    if (U > GMAX)
      return sa_fail(DSA_ERR_UNSUPPORTED, "union_rows must be <= %d (one bit per row; got %d)", GMAX,
                     U);
    if ((int64_t)U * s->k_tokens > UCAP)
      return sa_fail(DSA_ERR_UNSUPPORTED, "union_rows * k_tokens must be <= %d", UCAP);
    if (s->rows_per_seq % U)
      return sa_fail(DSA_ERR_INVALID_ARG, "union_rows must divide rows_per_seq (a group lies in "
                     "one sequence)");
  }
  // Head tiles: the fewest equal parts of the group whose (row, head) pairs,
  // union_rows rows of them in union mode, fit one 16-row matrix tile.
  int T = 1;
  while (s->group % T || (int64_t)U * (s->group / T) > GMAX) ++T;
  const int64_t hkv = (int64_t)s->kv_heads * T;
  const int64_t pairs = (int64_t)s->rows * hkv;
  if (pairs > ((int64_t)1 << 30)) return sa_fail(DSA_ERR_UNSUPPORTED, "too many rows or heads");
  // Head tiles per workgroup (the tiles of one kv head are neighbours, so a
  // workgroup's waves read the same cache rows), and chunks per (row or union
  // group, group of head tiles): enough workgroups for two per CU, each chunk
  // at least one step per wave of one row's list (a union holds between
  // k_tokens and U * k_tokens tokens; more chunks would multiply the partials
  // the last workgroup merges, U * G pairs of them per chunk and tile).
  const int G = s->group / T;
  const int hw = hkv % 4 == 0 ? 4 : hkv % 2 == 0 ? 2 : 1;
  const int64_t nru = U > 1 ? (s->rows + U - 1) / U : s->rows;
  const int64_t wgp = nru * (hkv / hw);
  const int64_t steps = (s->k_tokens + STEP - 1) / STEP;
  const int64_t maxc = std::max<int64_t>(1, steps / (WAVES / hw));
  int64_t ch = s->chunks > 0 ? s->chunks
                             : (2 * (int64_t)cus + std::max<int64_t>(wgp, 1) - 1) / std::max<int64_t>(wgp, 1);
  ch = std::max<int64_t>(1, std::min<int64_t>(ch, s->chunks > 0 ? steps : maxc));
  // the merge stages hw * U * group (maximum, sum) pairs per chunk in the
  // waves' LDS partial space
  ch = std::min<int64_t>(ch, (int64_t)WAVES * GMAX * D * 4 / (8 * hw * U * G));
  const int64_t spc = (steps + ch - 1) / ch;
  ch = (steps + spc - 1) / spc;
  if (wgp * ch > ((int64_t)1 << 31) - 1) return sa_fail(DSA_ERR_UNSUPPORTED, "grid too large");
  std::memset(c, 0, sizeof(*c));
  c->sh = *s;
  c->chunks = (int)ch;
  c->spc = (int)spc;
  c->hw = hw;
  c->T = T;
  c->hkv = (int)hkv;
  c->G = G;
  c->U = U;
  c->nru = (int)nru;
  c->cap = U * s->k_tokens;
  // [partial outputs][partial (max, sum)][tickets][status] then, in union
  // mode, [entries][counts]
  const int64_t P = (int64_t)U * G;
  const int64_t units = ch > 1 ? nru * hkv * ch : 0;
  const int64_t floats = units * P * (D + 2);
  const int64_t nticket = nru * hkv;
  c->head_bytes = ((size_t)floats * 4 + (size_t)(nticket + 1) * 4 + 255) & ~(size_t)255;
  const size_t ent_bytes = U > 1 ? (size_t)nru * c->cap * 8 + (size_t)nru * 4 : 0;
  c->ws_bytes = c->head_bytes + ent_bytes + 256;
  return DSA_OK;
}

}  // namespace

extern "C" {

int dsa_sparse_attn_plan(const dsa_attn_shape* s, int cus, dsa_attn_plan_info* info) {
  if (!info) return sa_fail(DSA_ERR_INVALID_ARG, "info is null");
  dsa_attn_ctx c;
  const int rc = attn_plan(s, cus, &c);
  if (rc != DSA_OK) return rc;
  info->head_tiles = c.T;
  info->heads_per_tile = c.G;
  info->tiles_per_group = c.hw;
  info->chunks = c.chunks;
  info->grid_groups = (int32_t)((int64_t)c.nru * (c.hkv / c.hw) * c.chunks);
  info->workspace_bytes = (int64_t)c.ws_bytes;
  return DSA_OK;
}

int dsa_sparse_attn_init(const dsa_attn_shape* s, int device, dsa_attn_ctx** out) {
  if (!out) return sa_fail(DSA_ERR_INVALID_ARG, "out is null");
  *out = nullptr;
  {
    dsa_attn_ctx check;   // the shape is validated before any device call
    const int rc = attn_plan(s, 1, &check);
    if (rc != DSA_OK) return rc;
  }
  if (device < 0) return sa_fail(DSA_ERR_INVALID_ARG, "device must be >= 0");
  DeviceScope ds(device);
  if (ds.e != hipSuccess) return sa_hip(ds.e, "hipSetDevice");
  int cus = 0;
  hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
  if (e != hipSuccess) return sa_hip(e, "hipDeviceGetAttribute(CU count)");
  dsa_attn_ctx* c = new (std::nothrow) dsa_attn_ctx;
  if (!c) return sa_fail(DSA_ERR_HIP, "host allocation failed");
  const int rc = attn_plan(s, cus, c);
  if (rc != DSA_OK) { delete c; return rc; }
  c->device = device;
  c->magic = SA_MAGIC;
  const size_t head_bytes = c->head_bytes;
  const int64_t D = s->head_dim, P = (int64_t)c->U * c->G;
  const int64_t units = c->chunks > 1 ? (int64_t)c->nru * c->hkv * c->chunks : 0;
  const int64_t nticket = (int64_t)c->nru * c->hkv;
  const int U = c->U;
  const int64_t nru = c->nru;
  e = hipMalloc(&c->ws, c->ws_bytes);
  if (e != hipSuccess) { delete c; return sa_hip(e, "hipMalloc(workspace)"); }
  e = hipMemset(c->ws, 0, c->ws_bytes);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) { (void)hipFree(c->ws); delete c; return sa_hip(e, "hipMemset(workspace)"); }
  float* f = static_cast<float*>(c->ws);
  c->part_o = f;
  c->part_ml = f + units * P * D;
  c->tickets = reinterpret_cast<uint32_t*>(c->part_ml + units * P * 2);
  c->status = c->tickets + nticket;
  if (U > 1) {
    c->ent = reinterpret_cast<int2*>(static_cast<char*>(c->ws) + head_bytes);
    c->cnt = reinterpret_cast<int32_t*>(c->ent + (int64_t)nru * c->cap);
  }
  *out = c;
  return DSA_OK;
}

int dsa_sparse_attn_destroy(dsa_attn_ctx* c) {
  if (!c || c->magic != SA_MAGIC) return sa_fail(DSA_ERR_INVALID_ARG, "bad context");
  c->magic = 0;
  int rc = DSA_OK;
  if (c->ws) {
    DeviceScope ds(c->device);
    const hipError_t e = hipFree(c->ws);
    if (e != hipSuccess) rc = sa_hip(e, "hipFree(workspace)");
  }
  delete c;
  return rc;
}

int dsa_sparse_attn_chunks(const dsa_attn_ctx* c) {
  if (!c || c->magic != SA_MAGIC) return sa_fail(DSA_ERR_INVALID_ARG, "bad context");
  return c->chunks;
}

}  // extern "C"

namespace {

int sa_launch(dsa_attn_ctx* c, const uint16_t* q, const void* k_cache, const void* v_cache,
              bool fp8, float k_scale, float v_scale, const int32_t* token_ids,
              const int32_t* page_table, const uint16_t* gate, float sm_scale, uint16_t* out,
              float* lse, hipStream_t stream) {
  if (!c || c->magic != SA_MAGIC) return sa_fail(DSA_ERR_INVALID_ARG, "bad context");
  const dsa_attn_shape& s = c->sh;
  if (s.rows == 0) return DSA_OK;
  if (!q || !k_cache || !v_cache || !token_ids || !out)
    return sa_fail(DSA_ERR_INVALID_ARG, "q, k_cache, v_cache, token_ids and out must be non-null");
  const uintptr_t cache_align = fp8 ? 7u : 15u;
  if (!aligned16(q) || ((uintptr_t)k_cache & cache_align) || ((uintptr_t)v_cache & cache_align) ||
      ((uintptr_t)out & 7u) || (gate && ((uintptr_t)gate & 7u)))
    return sa_fail(DSA_ERR_INVALID_ARG, "q must be 16-byte aligned, the caches 16-byte (bf16) or "
                   "8-byte (fp8) aligned, out and gate 8-byte aligned");
  if (fp8 && (!std::isfinite(k_scale) || !std::isfinite(v_scale)))
    return sa_fail(DSA_ERR_INVALID_ARG, "k_scale and v_scale must be finite");
  if (page_table && s.pages_per_seq < 1)
    return sa_fail(DSA_ERR_INVALID_ARG, "a page table needs pages_per_seq >= 1");
  if (!std::isfinite(sm_scale)) return sa_fail(DSA_ERR_INVALID_ARG, "sm_scale must be finite");
  DeviceScope ds(c->device);
  if (ds.e != hipSuccess) return sa_hip(ds.e, "hipSetDevice");
  Args a;
  std::memset(&a, 0, sizeof(a));
  a.q = q; a.kc = k_cache; a.vc = v_cache; a.ids = token_ids; a.table = page_table;
  a.gate = gate; a.out = out; a.lse = lse;
  a.part_o = c->part_o; a.part_ml = c->part_ml; a.tickets = c->tickets; a.status = c->status;
  a.k_ss = s.k_slot_stride; a.k_hs = s.k_head_stride;
  a.v_ss = s.v_slot_stride; a.v_hs = s.v_head_stride; a.num_slots = s.num_slots;
  a.rows = s.rows; a.hkv = c->hkv; a.G = c->G; a.tdiv = c->T; a.K = s.k_tokens;
  a.rows_per_seq = s.rows_per_seq;
  int shift = 0;
  while ((1 << shift) < s.page_size) ++shift;
  a.page_shift = shift;
  a.pps = s.pages_per_seq;
  a.chunks = c->chunks; a.spc = c->spc; a.hw = c->hw;
  a.c2 = sm_scale * 1.4426950408889634f * (fp8 ? k_scale : 1.0f);
  a.vscale = fp8 ? v_scale : 1.0f;
  a.U = c->U;
  a.P = c->U * c->G;
  a.cap = c->cap;
  a.ent = c->ent;
  a.cnt = c->cnt;
  const bool un = c->U > 1;
  if (un) {
    UArgs u;
    std::memset(&u, 0, sizeof(u));
    u.ids = token_ids; u.ent = c->ent; u.cnt = c->cnt;
    u.rows = s.rows; u.K = s.k_tokens; u.U = c->U; u.cap = c->cap;
    hipLaunchKernelGGL(k_union, dim3((unsigned)c->nru), dim3(UNT), 0, stream, u);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return sa_hip(e, "launch k_union");
  }
  const unsigned grid = (unsigned)((int64_t)c->nru * (c->hkv / c->hw) * c->chunks);
#define SA_GO(DD, F8, UN_) \
  hipLaunchKernelGGL((k_sparse_attn<DD, F8, UN_>), dim3(grid), dim3(NT), 0, stream, a)
  if (s.head_dim == 256) {
    if (fp8) { if (un) SA_GO(256, true, true); else SA_GO(256, true, false); }
    else { if (un) SA_GO(256, false, true); else SA_GO(256, false, false); }
  } else {
    if (fp8) { if (un) SA_GO(128, true, true); else SA_GO(128, true, false); }
    else { if (un) SA_GO(128, false, true); else SA_GO(128, false, false); }
  }
#undef SA_GO
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return sa_hip(e, "launch k_sparse_attn");
  return DSA_OK;
}

}  // namespace

extern "C" {

int dsa_sparse_attn(dsa_attn_ctx* c, const uint16_t* q, const uint16_t* k_cache,
                    const uint16_t* v_cache, const int32_t* token_ids,
                    const int32_t* page_table, const uint16_t* gate, float sm_scale,
                    uint16_t* out, float* lse, hipStream_t stream) {
  return sa_launch(c, q, k_cache, v_cache, false, 1.0f, 1.0f, token_ids, page_table, gate,
                   sm_scale, out, lse, stream);
}

int dsa_sparse_attn_fp8(dsa_attn_ctx* c, const uint16_t* q, const uint8_t* k_cache,
                        const uint8_t* v_cache, float k_scale, float v_scale,
                        const int32_t* token_ids, const int32_t* page_table,
                        const uint16_t* gate, float sm_scale, uint16_t* out, float* lse,
                        hipStream_t stream) {
  return sa_launch(c, q, k_cache, v_cache, true, k_scale, v_scale, token_ids, page_table, gate,
                   sm_scale, out, lse, stream);
}

int dsa_sparse_attn_read_status(dsa_attn_ctx* c, uint32_t* status) {
  if (!c || c->magic != SA_MAGIC || !status) return sa_fail(DSA_ERR_INVALID_ARG, "bad context or status");
  DeviceScope ds(c->device);
  if (ds.e != hipSuccess) return sa_hip(ds.e, "hipSetDevice");
  hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpy(status, c->status, 4, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return sa_hip(e, "read status");
  return DSA_OK;
}

int dsa_sparse_attn_reset_status(dsa_attn_ctx* c) {
  if (!c || c->magic != SA_MAGIC) return sa_fail(DSA_ERR_INVALID_ARG, "bad context");
  DeviceScope ds(c->device);
  if (ds.e != hipSuccess) return sa_hip(ds.e, "hipSetDevice");
  hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemset(c->status, 0, 4);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) return sa_hip(e, "reset status");
  return DSA_OK;
}

}  // extern "C"

// Device building blocks for DSA candidate selection on gfx950 (CDNA4).
//
// Everything here works on 64-lane wavefronts: ballots are 64-bit, lane ranks
// come from v_mbcnt, and the segmented block maximum uses DPP row permutes.
// Values are never rounded: fp32 logits are mapped to order-preserving uint32
// keys and only compared, so every reduction order gives identical bits.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#define DSA_DEV __device__ __forceinline__

namespace dsa {

// ---------------------------------------------------------------------------
// Order key: unsigned order of the key == float order (-0 below +0).
// ---------------------------------------------------------------------------
constexpr uint32_t KEY_POS_INF = 0xFF800000u;   // key of +inf
constexpr uint32_t KEY_NEG_INF = 0x007FFFFFu;   // key of -inf
constexpr uint32_t NEG_INF_BITS = 0xFF800000u;  // fp32 bits of -inf

DSA_DEV uint32_t f2key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
DSA_DEV float key2f(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// ---------------------------------------------------------------------------
// Workspace words shared between workgroups of one launch.  Agent-scope
// relaxed atomics compile to coherent (sc1) loads and stores on gfx950, so no
// L2 write-back or invalidate is needed; vm_drain() waits until this wave's
// stores and atomics have completed before a ticket is taken.
// ---------------------------------------------------------------------------
DSA_DEV uint32_t ld_shared(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
DSA_DEV void st_shared(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
DSA_DEV uint64_t ld_shared64(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
DSA_DEV void st_shared64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
DSA_DEV uint64_t pair(uint32_t lo, uint32_t hi) { return (uint64_t)lo | ((uint64_t)hi << 32); }
DSA_DEV void vm_drain() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

typedef float f4v __attribute__((ext_vector_type(4)));
DSA_DEV void store_ninf4(float* p) {   // 16-byte aligned, streaming
  const f4v v = {__uint_as_float(NEG_INF_BITS), __uint_as_float(NEG_INF_BITS),
                 __uint_as_float(NEG_INF_BITS), __uint_as_float(NEG_INF_BITS)};
  __builtin_nontemporal_store(v, reinterpret_cast<f4v*>(p));
}
DSA_DEV void store_ninf(float* p) { __builtin_nontemporal_store(__uint_as_float(NEG_INF_BITS), p); }

// ---------------------------------------------------------------------------
// Wavefront helpers (wave64)
// ---------------------------------------------------------------------------
DSA_DEV int lane() { return threadIdx.x & 63; }
DSA_DEV int wave() { return threadIdx.x >> 6; }
DSA_DEV uint64_t ballot(bool p) { return __ballot(p); }
DSA_DEV uint32_t popc(uint64_t m) { return (uint32_t)__popcll(m); }
// Number of set bits of m in lanes below the calling lane.
DSA_DEV uint32_t mbcnt(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Max over aligned groups of G consecutive lanes (G in 1,2,4,8,16), every lane
// of a group gets the group maximum.  DPP: quad_perm [1,0,3,2], quad_perm
// [2,3,0,1], row_half_mirror, row_mirror.  The whole wave must be active.
template <int G>
DSA_DEV uint32_t group_max(uint32_t x) {
  if constexpr (G >= 2)
    x = max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false));
  if constexpr (G >= 4)
    x = max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false));
  if constexpr (G >= 8)
    x = max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x141, 0xF, 0xF, false));
  if constexpr (G >= 16)
    x = max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x140, 0xF, 0xF, false));
  return x;
}

// Inclusive prefix sum over the 64 lanes: row_shr 1/2/4/8 within each row of
// 16 lanes, then row_bcast 15 and 31 carry row totals into the rows above.
DSA_DEV uint32_t wave_incl_scan(uint32_t x) {
  x += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0u, x, 0x142, 0xA, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0u, x, 0x143, 0xC, 0xF, false);
  return x;
}

// Inclusive running maximum over the 64 lanes (same DPP pattern as the sum).
DSA_DEV uint32_t wave_incl_max(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0u, x, 0x111, 0xF, 0xF, true));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0u, x, 0x112, 0xF, 0xF, true));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0u, x, 0x114, 0xF, 0xF, true));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0u, x, 0x118, 0xF, 0xF, true));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0u, x, 0x142, 0xA, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0u, x, 0x143, 0xC, 0xF, false));
  return x;
}

// ---------------------------------------------------------------------------
// Shared memory of one workgroup (about 73 KB: two workgroups per CU).
// ---------------------------------------------------------------------------
constexpr int HIST_WORDS = 4096;       // 12-bit digit histogram, or a 131072-bit bitmap
constexpr int LIST_CAP = 4096;         // block keys / listed blocks / token columns
constexpr int SEL_CAP = 2048;          // kept block ids
constexpr int TK_CAP = 4096;           // token keys
constexpr int DB_CAP = 2 * LIST_CAP;   // token-domain blocks (aliases kid)
constexpr int BITMAP_BITS = HIST_WORDS * 32;
constexpr int CHUNK_CAP = LIST_CAP;    // blocks per sub-chunk in the mask pass

struct __align__(16) Smem {
  uint32_t hist[HIST_WORDS];
  uint32_t kid[2 * LIST_CAP];   // [0, LIST_CAP): keys, [LIST_CAP, 2*LIST_CAP): ids
  uint32_t sel[SEL_CAP];
  uint32_t tkey[TK_CAP];
  uint32_t bits[CHUNK_CAP / 32];  // a short row's dropped-block bitmap
  uint32_t wv[64];
  uint32_t misc[16];
  uint64_t pfx[514];            // long-row block prefix over rows, then the chunk
  uint32_t row_s[256];          // balanced split: each row's start and live length
  uint32_t row_L[256];
  DSA_DEV uint32_t* keys() { return kid; }
  DSA_DEV uint32_t* ids() { return kid + LIST_CAP; }
};

// Exclusive scan of one value per thread over the workgroup; also the total.
// The caller must pass a barrier before wv is written again.
template <int NT>
DSA_DEV uint32_t wg_excl_scan_once(uint32_t x, uint32_t* wv, uint32_t& total) {
  constexpr int NW = NT / 64;
  const uint32_t inc = wave_incl_scan(x);
  if (lane() == 63) wv[wave()] = inc;
  __syncthreads();
  uint32_t off = 0, tot = 0;
  const int w = wave();
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const uint32_t v = wv[i];
    off += (i < w) ? v : 0u;
    tot += v;
  }
  total = tot;
  return off + inc - x;
}

template <int NT>
DSA_DEV uint32_t wg_excl_scan(uint32_t x, uint32_t* wv, uint32_t& total) {
  const uint32_t r = wg_excl_scan_once<NT>(x, wv, total);
  __syncthreads();
  return r;
}

// hist[0..nb) (nb a power of two, 256 <= nb <= 8 * NT): find d with
// count(bins > d) < krem <= count(bins >= d); also count(bins > d) and hist[d].
// Each thread holds its bins in registers; two barriers in all.
template <int NT>
DSA_DEV void find_bin(const uint32_t* hist, int nb, uint32_t krem, Smem& sm,
                      uint32_t& d, uint32_t& above, uint32_t& in_bin) {
  const int per = nb >= NT ? nb / NT : 1;
  const int lo = (int)threadIdx.x * per;
  uint32_t h[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) h[j] = (j < per && lo + j < nb) ? hist[lo + j] : 0u;
  uint32_t c = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) c += h[j];
  if (threadIdx.x == 0) {   // defined result even if the counts fall short; written
    sm.misc[0] = 0;          // before the scan's barrier, so the finder's write wins
    sm.misc[1] = 0;
    sm.misc[5] = 0;
  }
  uint32_t total;
  const uint32_t excl = wg_excl_scan_once<NT>(c, sm.wv, total);
  const uint32_t sfx = total - (excl + c);   // count in bins above this thread's bins
  if (sfx < krem && krem <= sfx + c) {
    uint32_t acc = sfx, dd = (uint32_t)lo, hh = 0;
    bool done = false;
#pragma unroll
    for (int j = 7; j >= 0; --j) {
      if (!done && j < per) {
        if (acc + h[j] >= krem) {
          dd = (uint32_t)(lo + j);
          hh = h[j];
          done = true;
        } else {
          acc += h[j];
        }
      }
    }
    sm.misc[0] = dd;
    sm.misc[1] = acc;
    sm.misc[5] = hh;
  }
  __syncthreads();
  d = sm.misc[0];
  above = sm.misc[1];
  in_bin = sm.misc[5];
}

// hist[0..NB) (NB a power of two, 256 <= NB <= 8 * NT): find d with
// count(bins > d) < krem <= count(bins >= d), count(bins > d) and hist[d],
// and leave hist[0..NB) zero.  Bins are read with 16-byte LDS loads; two
// barriers.
template <int NT, int NB>
DSA_DEV void find_bin_zero(uint32_t* hist, uint32_t krem, Smem& sm, uint32_t& d,
                           uint32_t& above, uint32_t& in_bin) {
  constexpr int PER = NB >= NT ? NB / NT : 1;
  constexpr int ACT = NB / PER;              // threads holding bins
  static_assert(PER == 1 || PER == 2 || PER % 4 == 0, "bins per thread");
  const int t = (int)threadIdx.x;
  uint32_t h[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) h[j] = 0u;
  if (t < ACT) {
    uint32_t* hp = hist + t * PER;
    if constexpr (PER % 4 == 0) {
#pragma unroll
      for (int j = 0; j < PER; j += 4) {
        const uint4 v = *reinterpret_cast<const uint4*>(hp + j);
        h[j] = v.x; h[j + 1] = v.y; h[j + 2] = v.z; h[j + 3] = v.w;
      }
#pragma unroll
      for (int j = 0; j < PER; j += 4) *reinterpret_cast<uint4*>(hp + j) = make_uint4(0u, 0u, 0u, 0u);
    } else {
#pragma unroll
      for (int j = 0; j < PER; ++j) h[j] = hp[j];
#pragma unroll
      for (int j = 0; j < PER; ++j) hp[j] = 0u;
    }
  }
  uint32_t c = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) c += h[j];
  if (t == 0) {   // defined result even if the counts fall short; written
    sm.misc[0] = 0;   // before the scan's barrier, so the finder's write wins
    sm.misc[1] = 0;
    sm.misc[5] = 0;
  }
  uint32_t total;
  const uint32_t excl = wg_excl_scan_once<NT>(c, sm.wv, total);
  const uint32_t sfx = total - (excl + c);   // count in bins above this thread's
  if (sfx < krem && krem <= sfx + c) {
    uint32_t acc = sfx, dd = 0, ab = 0, hb = 0;
    bool found = false;
#pragma unroll
    for (int j = PER - 1; j >= 0; --j) {
      const bool hit = !found && acc + h[j] >= krem;
      dd = hit ? (uint32_t)j : dd;
      ab = hit ? acc : ab;
      hb = hit ? h[j] : hb;
      found = found || hit;
      acc += h[j];
    }
    sm.misc[0] = (uint32_t)(t * PER) + dd;
    sm.misc[1] = ab;
    sm.misc[5] = hb;
  }
  __syncthreads();
  d = sm.misc[0];
  above = sm.misc[1];
  in_bin = sm.misc[5];
}

// The bin starting at key `lo` (and everything above it) is kept whole.
DSA_DEV void keep_from(uint32_t lo, uint32_t& T, uint32_t& q) {
  if (lo == 0) {
    T = 0;
    q = 0xFFFFFFFFu;
  } else {
    T = lo - 1;
    q = 0;
  }
}

// Radix passes 2 and 3 (bits 19..8, then 7..0) of the top-K rule below, among
// the keys whose top 12 bits equal those of `prefix`, krem of which are still
// to be taken.  The 4096-word histogram must be zero on entry and is zero on
// return.
template <int NT, class ForKeys>
DSA_DEV void radix_low_passes(ForKeys for_keys, uint32_t prefix, uint32_t krem, Smem& sm,
                              uint32_t& T, uint32_t& q) {
  uint32_t d, above, in_bin;
  const uint32_t p20 = prefix >> 20;
  for_keys([&](uint32_t k) {
    if ((k >> 20) == p20) atomicAdd(&sm.hist[(k >> 8) & 0xFFFu], 1u);
  });
  __syncthreads();
  find_bin_zero<NT, 4096>(sm.hist, krem, sm, d, above, in_bin);
  prefix |= d << 8;
  krem -= above;
  if (in_bin == krem) return keep_from(prefix, T, q);
  const uint32_t p8 = prefix >> 8;
  for_keys([&](uint32_t k) {
    if ((k >> 8) == p8) atomicAdd(&sm.hist[k & 0xFFu], 1u);
  });
  __syncthreads();
  find_bin_zero<NT, 256>(sm.hist, krem, sm, d, above, in_bin);
  T = prefix | d;
  q = krem - above;
}

// Radix passes of the top-K rule below over keys visited by
// for_keys(f) (f(key) once per element).  Digits of 12, 12 and 8 bits over
// the 4096-word histogram, which must be zero on entry and is zero on return.
// top_counted: the caller has already counted every key's top digit into the
// histogram (and passed a barrier since).
template <int NT, class ForKeys>
DSA_DEV void radix_passes(ForKeys for_keys, uint32_t K, Smem& sm, uint32_t& T, uint32_t& q,
                          bool top_counted = false) {
  uint32_t d, above, in_bin;
  if (!top_counted) {
    for_keys([&](uint32_t k) { atomicAdd(&sm.hist[k >> 20], 1u); });
    __syncthreads();
  }
  find_bin_zero<NT, 4096>(sm.hist, K, sm, d, above, in_bin);
  const uint32_t krem = K - above;
  if (in_bin == krem) return keep_from(d << 20, T, q);
  radix_low_passes<NT>(for_keys, d << 20, krem, sm, T, q);
}

template <int NT, int U, class GetKey>
DSA_DEV void radix_select_regs(int n, uint32_t K, GetKey getk, Smem& sm, uint32_t& T,
                               uint32_t& q, bool top_counted = false) {
  uint32_t k[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int i = (int)threadIdx.x + u * NT;
    k[u] = i < n ? getk(i) : 0u;
  }
  radix_passes<NT>([&](auto f) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      if ((int)threadIdx.x + u * NT < n) f(k[u]);
  }, K, sm, T, q, top_counted);
}

// The (T, q) rule for the top K of getk(0..n), n <= 8 * NT, when the top
// 12-bit digit of the K-th key is known to be d20 and `above` keys have a
// larger top digit (so krem = K - above are taken from digit d20).
template <int NT, class GetKey>
DSA_DEV void wg_radix_select_low(int n, uint32_t d20, uint32_t krem, GetKey getk, Smem& sm,
                                 uint32_t& T, uint32_t& q) {
  for (int j = threadIdx.x; j < HIST_WORDS; j += NT) sm.hist[j] = 0;
  __syncthreads();
  auto run = [&](auto u_tag) {
    constexpr int U = decltype(u_tag)::value;
    uint32_t k[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = (int)threadIdx.x + u * NT;
      k[u] = i < n ? getk(i) : 0u;
    }
    radix_low_passes<NT>([&](auto f) {
#pragma unroll
      for (int u = 0; u < U; ++u)
        if ((int)threadIdx.x + u * NT < n) f(k[u]);
    }, d20 << 20, krem, sm, T, q);
  };
  if (n <= NT) run(std::integral_constant<int, 1>{});
  else if (n <= 2 * NT) run(std::integral_constant<int, 2>{});
  else if (n <= 4 * NT) run(std::integral_constant<int, 4>{});
  else run(std::integral_constant<int, 8>{});
}

// Top-K selection rule over getk(0..n), 1 <= K <= n: element i is kept iff
// key > T, or key == T and it is among the first q such elements in index
// order.  MSB-first radix select (digits of 12, 12 and 8 bits) with LDS
// histograms; it stops early once the digit bin holding the K-th key is kept
// whole.  Up to 8 * NT keys are held in registers across the passes; longer
// inputs are re-read each pass, U loads at a time per thread.
// hist_zero: the caller guarantees sm.hist[0..4096) is zero.  On return it is.
// top_counted: instead, the caller has counted every key's top 12-bit digit
// into sm.hist (and passed a barrier since).
template <int NT, int U = 8, class GetKey>
DSA_DEV void wg_radix_select(int n, uint32_t K, GetKey getk, Smem& sm, uint32_t& T,
                             uint32_t& q, bool hist_zero = false, bool top_counted = false) {
  if (!hist_zero && !top_counted) {
    for (int j = threadIdx.x; j < HIST_WORDS; j += NT) sm.hist[j] = 0;
    __syncthreads();
  }
  if (n <= NT) return radix_select_regs<NT, 1>(n, K, getk, sm, T, q, top_counted);
  if (n <= 2 * NT) return radix_select_regs<NT, 2>(n, K, getk, sm, T, q, top_counted);
  if (n <= 4 * NT) return radix_select_regs<NT, 4>(n, K, getk, sm, T, q, top_counted);
  if (n <= 8 * NT) return radix_select_regs<NT, 8>(n, K, getk, sm, T, q, top_counted);
  radix_passes<NT>([&](auto f) {
    for (int i0 = threadIdx.x; i0 < n; i0 += NT * U) {
      uint32_t k[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = i0 + u * NT;
        k[u] = i < n ? getk(i) : 0u;
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (i0 + u * NT < n) f(k[u]);
    }
  }, K, sm, T, q, top_counted);
}

// Ordered application of the (T, q) rule to [0, n), n <= 8 * NT, keys held in
// registers (element i = threadIdx.x + u * NT): emit(i, rank, kept) for every
// i, rank = kept elements before i.  Returns the kept count.  One barrier; the
// caller must pass a barrier before sm.wv is written again.
template <int NT, int U, class GetKey, class Emit>
DSA_DEV uint32_t rule_emit_regs(int n, uint32_t T, uint32_t q, GetKey getk, Emit emit,
                                Smem& sm) {
  constexpr int NW = NT / 64;
  static_assert(U * NW <= 64, "one lane per (batch, wave) pair");
  const int w = wave(), l = lane();
  uint64_t mg[U], me[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int i = (int)threadIdx.x + u * NT;
    const bool v = i < n;
    const uint32_t k = v ? getk(i) : 0u;
    mg[u] = ballot(v && k > T);
    me[u] = ballot(v && k == T);
  }
  if (l == 0) {
#pragma unroll
    for (int u = 0; u < U; ++u) sm.wv[u * NW + w] = popc(mg[u]) | (popc(me[u]) << 16);
  }
  __syncthreads();
  // Lane j of every wave holds pair j = (batch, wave) in index order.
  const uint32_t cj = l < U * NW ? sm.wv[l] : 0u;
  const uint32_t gj = cj & 0xFFFFu, ej = cj >> 16;
  const uint32_t eqx = wave_incl_scan(ej) - ej;
  const uint32_t take = q > eqx ? min(ej, q - eqx) : 0u;
  const uint32_t kj = gj + take;
  const uint32_t kinc = wave_incl_scan(kj);
  const uint32_t kx = kinc - kj;
  const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)kinc, 63);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int pair = u * NW + w;
    const uint32_t base = (uint32_t)__builtin_amdgcn_ds_bpermute(pair << 2, (int)kx);
    const uint32_t eqb = (uint32_t)__builtin_amdgcn_ds_bpermute(pair << 2, (int)eqx);
    const int i = (int)threadIdx.x + u * NT;
    const bool gt = (mg[u] >> l) & 1u;
    const bool eq = (me[u] >> l) & 1u;
    const bool kept = gt || (eq && eqb + mbcnt(me[u]) < q);
    const uint64_t km = ballot(kept);
    if (i < n) emit(i, base + mbcnt(km), kept);
  }
  return total;
}

// The (T, q) rule applied in index order over getk(0..n) for n <= 8 * NT;
// see rule_emit_regs.
template <int NT, class GetKey, class Emit>
DSA_DEV uint32_t wg_rule_emit(int n, uint32_t T, uint32_t q, GetKey getk, Emit emit, Smem& sm) {
  if (n <= NT) return rule_emit_regs<NT, 1>(n, T, q, getk, emit, sm);
  if (n <= 2 * NT) return rule_emit_regs<NT, 2>(n, T, q, getk, emit, sm);
  if (n <= 4 * NT) return rule_emit_regs<NT, 4>(n, T, q, getk, emit, sm);
  return rule_emit_regs<NT, 8>(n, T, q, getk, emit, sm);
}

// Ordered pass over [0, n) applying the (T, q) rule above.  emit(i, rank,
// kept, word, base) is called for every i, with rank = kept elements before
// i and word = the 64-bit kept mask of [base, base + 64).  Returns the kept
// count.  Each wave walks one contiguous segment, four 64-groups at a time.
template <int NT, class GetKey, class Emit>
DSA_DEV uint32_t wg_select_compact(int n, uint32_t T, uint32_t q, GetKey getk,
                                   Emit emit, Smem& sm) {
  constexpr int NW = NT / 64;
  constexpr int G = 4;
  const int w = wave(), l = lane();
  const int seg = (((n + NW - 1) / NW) + 63) & ~63;
  const int lo = min(n, w * seg), hi = min(n, lo + seg);
  uint32_t cgt = 0, ceq = 0;
  for (int b0 = lo; b0 < hi; b0 += 64 * G) {
    uint32_t k[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int i = b0 + 64 * g + l;
      k[g] = i < hi ? getk(i) : 0u;
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const bool v = b0 + 64 * g + l < hi;
      cgt += popc(ballot(v && k[g] > T));
      ceq += popc(ballot(v && k[g] == T));
    }
  }
  if (l == 0) {
    sm.wv[w] = cgt;
    sm.wv[NW + w] = ceq;
  }
  __syncthreads();
  uint32_t selb = 0, eqb = 0, my_sel = 0, my_eq = 0;
#pragma unroll
  for (int x = 0; x < NW; ++x) {
    if (x == w) {
      my_sel = selb;
      my_eq = eqb;
    }
    const uint32_t g = sm.wv[x], e = sm.wv[NW + x];
    const uint32_t take = q > eqb ? min(e, q - eqb) : 0u;
    selb += g + take;
    eqb += e;
  }
  __syncthreads();
  for (int b0 = lo; b0 < hi; b0 += 64 * G) {
    uint32_t k[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int i = b0 + 64 * g + l;
      k[g] = i < hi ? getk(i) : 0u;
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int base = b0 + 64 * g;
      if (base >= hi) break;
      const int i = base + l;
      const bool v = i < hi;
      const bool gt = v && k[g] > T;
      const bool eq = v && k[g] == T;
      const uint64_t meq = ballot(eq);
      const bool kept = gt || (eq && (my_eq + mbcnt(meq)) < q);
      const uint64_t mk = ballot(kept);
      if (v) emit(i, my_sel + mbcnt(mk), kept, mk, base);
      my_sel += popc(mk);
      my_eq += popc(meq);
    }
  }
  return selb;
}

// Ordered compaction of [0, n) by a predicate: emit(i, rank) for pred(i).
template <int NT, class Pred, class Emit>
DSA_DEV uint32_t wg_compact(int n, Pred pred, Emit emit, Smem& sm) {
  constexpr int NW = NT / 64;
  const int w = wave(), l = lane();
  const int seg = (((n + NW - 1) / NW) + 63) & ~63;
  const int lo = min(n, w * seg), hi = min(n, lo + seg);
  uint32_t c = 0;
  for (int base = lo; base < hi; base += 64) {
    const int i = base + l;
    c += popc(ballot(i < hi && pred(i)));
  }
  if (l == 0) sm.wv[w] = c;
  __syncthreads();
  uint32_t off = 0, tot = 0;
#pragma unroll
  for (int x = 0; x < NW; ++x) {
    const uint32_t v = sm.wv[x];
    off += (x < w) ? v : 0u;
    tot += v;
  }
  __syncthreads();
  for (int base = lo; base < hi; base += 64) {
    const int i = base + l;
    const bool p = i < hi && pred(i);
    const uint64_t m = ballot(p);
    if (p) emit(i, off + mbcnt(m));
    off += popc(m);
  }
  return tot;
}

}  // namespace dsa

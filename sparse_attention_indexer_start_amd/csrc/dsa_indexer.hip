// Fused FP8 indexer logits plus selection on MI355X (gfx950): the logits of
// each query row are produced tile by tile with FP8 matrix-core
// instructions and consumed at once by the row's selection chain, so the
// [queries, keys] logits matrix is never stored.
//
// The page on vllm PR #48726 ("Fused DSA indexer Top-k kernel (LiteTopk)",
// "LiteTopK: fused indexer scoring and TopK") describes the prefill indexer as
// an FP8 multi-query score per query/key pair followed by a per-row top-k, and
// LiteTopK as computing that top-k without the score matrix, with a candidate
// workspace bounded independently of the sequence length.  The score taken
// here is the DSA indexer's:
//   logit[t, c] = kscale[c] * sum_h w[t, h] * max(0, q[t, h] . k[c])
// with OCP E4M3 q and k.  On it each row runs the decode path's chain (vllm
// PR #57459, Summary): block scores over the row's live range [s, e') with
// the newest block pinned to +inf, the top-K_blk blocks, and the top-K_tok
// tokens of the row masked to the kept blocks.
//
// One wavefront owns one query row:
//   * its 64 x 128 FP8 query block stays in registers as the A operand of
//     v_mfma_scale_f32_16x16x128_f8f6f4 (one instruction per 16 heads);
//   * 16 keys at a time (2 KB, one contiguous span) are the B operand; lane l
//     carries key l % 16 and bytes [32 * (l / 16), +32) of it, the same
//     byte slice its A operand holds of its head, so each instruction sums
//     all 128 dimensions;
//   * the 16 x 16 result holds, in lane l, key l % 16 and heads
//     4 * (l / 16) + i; each lane applies ReLU and the head weights to its
//     heads, and two cross-lane adds finish the sum over heads;
//   * block maxima of B consecutive keys come from a DPP maximum across lanes;
//   * a per-wave LDS buffer keeps the row's candidate blocks: a block enters
//     only above the running threshold, and when the buffer is full an exact
//     radix select keeps the K_blk best (ties to the lower id) and raises the
//     threshold to the K_blk-th key.  A later block with a key equal to the
//     threshold loses its tie to the kept ones, which all have lower ids.
// Tokens: when the kept blocks hold at most K_tok columns the token ids
// follow from the kept block ids (all kept columns, then the lowest-index
// dropped columns, which rank as -inf in the masked row); otherwise the kept
// blocks' logits are computed again, gathered 16 columns at a time, and the
// same streaming select keeps the K_tok best.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "dsa_device.hpp"
#include "dsa_indexer.h"

namespace dsa {
namespace idx {

constexpr int WAVES = 4;            // query rows per workgroup
// Two forms of the per-row machinery.  The narrow one (768 candidate entries
// per wave, keys staged 64 at a time: 51 KB of LDS and at most 168 VGPRs)
// fits three workgroups per CU, and the extra waves hide the matrix and LDS
// latencies between the epilogues' vector instructions; the wide one (1024
// entries, 128 keys per stage, two workgroups per CU) keeps K up to 512.
template <bool WIDE>
struct Form {
  static constexpr int CAP = WIDE ? 1024 : 768;   // candidate entries per wave
  static constexpr int KMAX = CAP / 2;            // largest K the streaming select keeps
  static constexpr int STAGE = WIDE ? 128 : 64;   // keys staged in LDS per step (shared mode)
  static constexpr int MIN_WG = WIDE ? 2 : 3;     // workgroups per CU the registers allow
};
constexpr int D = 128;              // head dimension (bytes per FP8 key)

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

struct Args {
  const uint8_t* q;       // [Q, H, D]
  const uint8_t* k;       // [S, D]
  const float* w;         // [Q, H]
  const float* kscale;    // [S] or null
  const int32_t* starts;  // or null
  const int32_t* ends;
  int32_t* block_ids;     // [Q, K_blk]
  int32_t* token_ids;     // [Q, K_tok]
  float* logits_out;      // [Q, S] or null
  int64_t S;
  int32_t Q, H, B, k_blocks, k_tokens, starts_repeat, ends_repeat;
};

template <int CAP>
struct WaveLds {
  uint32_t key[CAP];
  uint32_t id[CAP];
  uint32_t hist[256];
  uint32_t sel[CAP / 2];
};

// Completes this wave's LDS operations and keeps the compiler from moving
// LDS accesses across this point (lanes read what other lanes wrote).
DSA_DEV void wave_lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
}

// Exact top-K over the n (<= CAP) entries of the wave's buffer, in buffer
// order: afterwards the buffer holds exactly min(K, n) entries in their
// original order.  Returns the key of the K-th best (the new threshold), or
// 0 when n <= K.
template <int CAP>
DSA_DEV uint32_t wave_keep_top(WaveLds<CAP>& s, int n, int K) {
  const int l = lane();
  if (n <= K) return 0u;
  constexpr int PER = CAP / 64;
  uint32_t kk[PER], ii[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int j = u * 64 + l;
    kk[u] = j < n ? s.key[j] : 0u;
    ii[u] = j < n ? s.id[j] : 0u;
  }
  // MSB-first radix select with 8-bit digits: T = the K-th largest key,
  // q = how many entries equal to T are kept (the first ones in order).
  uint32_t prefix = 0, krem = (uint32_t)K;
#pragma unroll 1
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    const uint32_t hi_mask = pass == 0 ? 0u : (0xFFFFFFFFu << (shift + 8));
#pragma unroll
    for (int j = 0; j < 4; ++j) s.hist[4 * l + j] = 0u;
    wave_lds_sync();
#pragma unroll
    for (int u = 0; u < PER; ++u)
      if (u * 64 + l < n && (kk[u] & hi_mask) == prefix)
        atomicAdd(&s.hist[(kk[u] >> shift) & 0xFFu], 1u);
    wave_lds_sync();
    // lane l holds bins 4l..4l+3; count above a lane's bins from the top
    uint32_t h[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) h[j] = s.hist[4 * l + j];
    const uint32_t c = h[0] + h[1] + h[2] + h[3];
    const uint32_t incl = wave_incl_scan(c);
    const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
    const uint32_t sfx = total - incl;               // keys in bins of higher lanes
    uint32_t dd = 0, ab = 0;
    bool hit = false;
    if (sfx < krem && krem <= sfx + c) {
      uint32_t acc = sfx;
#pragma unroll
      for (int j = 3; j >= 0; --j) {
        if (!hit && acc + h[j] >= krem) {
          dd = (uint32_t)(4 * l + j);
          ab = acc;
          hit = true;
        } else if (!hit) {
          acc += h[j];
        }
      }
    }
    const uint64_t m = ballot(hit);
    const int src = m ? (int)__builtin_ctzll(m) : 0;   // one lane finds the bin
    dd = (uint32_t)__builtin_amdgcn_readlane((int)dd, src);
    ab = (uint32_t)__builtin_amdgcn_readlane((int)ab, src);
    prefix |= dd << shift;
    krem -= ab;
  }
  const uint32_t T = prefix, q = krem;
  // Ordered compaction in place (every entry is in registers already).
  uint32_t base = 0, eq_before = 0;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const bool v = u * 64 + l < n;
    const bool gt = v && kk[u] > T;
    const bool eq = v && kk[u] == T;
    const uint64_t me = ballot(eq);
    const bool kept = gt || (eq && eq_before + mbcnt(me) < q);
    const uint64_t mk = ballot(kept);
    if (kept) {
      const uint32_t r = base + mbcnt(mk);
      s.key[r] = kk[u];
      s.id[r] = ii[u];
    }
    base += popc(mk);
    eq_before += popc(me);
  }
  wave_lds_sync();
  return T;
}

// Offers one (key, id) per lane (where `valid`); entries above the running
// threshold `thr` are appended in lane order.  A full buffer is first cut to
// its K best, which raises the threshold.
template <int CAP>
DSA_DEV void wave_offer(WaveLds<CAP>& s, int& n, uint32_t& thr, int K, bool valid, uint32_t key,
                        uint32_t id) {
  uint64_t m = ballot(valid && key > thr);
  if (m == 0) return;
  if (n + (int)popc(m) > CAP) {          // (at most 32 offers at a time)
    thr = wave_keep_top(s, n, K);
    n = K;
    m = ballot(valid && key > thr);
    if (m == 0) return;
  }
  if ((m >> lane()) & 1u) {
    const int r = n + (int)mbcnt(m);
    s.key[r] = key;
    s.id[r] = id;
  }
  n += (int)popc(m);
}

// 32 bytes of FP8 key `col` for this lane's slice.
DSA_DEV v8i load_key_slice(const uint8_t* k, int64_t col) {
  const int4* p = reinterpret_cast<const int4*>(k + col * D + (lane() >> 4) * 32);
  const int4 a = p[0], b = p[1];
  v8i r;
  r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w;
  r[4] = b.x; r[5] = b.y; r[6] = b.z; r[7] = b.w;
  return r;
}

// x summed over the four lanes l % 16 + 16 j (every lane gets the sum):
// v_permlane32_swap exchanges the two 32-lane halves of a register and
// v_permlane16_swap the two 16-lane rows of each half, without LDS.
DSA_DEV float sum_over_lane_groups(float x) {
  const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __uint_as_float(h[0]) + __uint_as_float(h[1]);   // x(l) + x(l ^ 32)
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);            // y(l) + y(l ^ 16)
}

// Logit of key `col` (the same value in the four lanes l % 16 == col slot).
template <int HG>
DSA_DEV float logit_of(const v8i (&qa)[HG], const float (&wr)[HG][4], v8i kb) {
  float part = 0.f;
#pragma unroll
  for (int g = 0; g < HG; ++g) {
    v4f acc = {0.f, 0.f, 0.f, 0.f};
    // E8M0 scales of 127 (2^0): the plain FP8 product.
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[g], kb, acc, 0, 0, 0, 127, 0, 127);
#pragma unroll
    for (int i = 0; i < 4; ++i)   // ReLU as one signed-integer max of the bits
      part += wr[g][i] * __int_as_float(max(__float_as_int(acc[i]), 0));
  }
  return sum_over_lane_groups(part);
}

// 2 * HG matrix-core instructions for a pair of 16-key halves: acc[h][g]
// = heads 16g.. of this lane's slot times half h's keys.
template <int HG>
DSA_DEV void mfma_pair(const v8i (&qa)[HG], v8i ka, v8i kb, v4f (&acc)[2][HG]) {
  const v4f z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int g = 0; g < HG; ++g) {
    acc[0][g] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[g], ka, z, 0, 0, 0, 127, 0, 127);
    acc[1][g] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[g], kb, z, 0, 0, 0, 127, 0, 127);
  }
}

// The head sums of a pair: lanes 0-15 get the first half's key l % 16,
// lanes 16-31 the second half's (lanes 32-63 the same again).
template <int HG>
DSA_DEV float epilogue_pair(const float (&wr)[HG][4], const v4f (&acc)[2][HG]) {
  float pa = 0.f, pb = 0.f;
#pragma unroll
  for (int g = 0; g < HG; ++g)
#pragma unroll
    for (int i = 0; i < 4; ++i) {   // ReLU as one signed-integer max of the bits
      pa += wr[g][i] * __int_as_float(max(__float_as_int(acc[0][g][i]), 0));
      pb += wr[g][i] * __int_as_float(max(__float_as_int(acc[1][g][i]), 0));
    }
  pa = sum_over_lane_groups(pa);
  pb = sum_over_lane_groups(pb);
  return (lane() & 16) ? pb : pa;
}

// The B operand of half h (keys 16h..16h+15 of a staged 32-key tile) for
// this lane: key 16h + l % 16, bytes [32 * (l / 16), +32).  Tile rows are
// 128 bytes; their 16-byte chunks are stored XOR-swizzled by the row's low
// three bits, so the 16 rows read by one instruction spread over the banks.
DSA_DEV v8i lds_key_slice(const uint8_t* tile, int h) {
  const int r = 16 * h + (lane() & 15);
  const int j0 = 2 * (lane() >> 4);
  const int4 x = *reinterpret_cast<const int4*>(tile + r * D + 16 * (j0 ^ (r & 7)));
  const int4 y = *reinterpret_cast<const int4*>(tile + r * D + 16 * ((j0 + 1) ^ (r & 7)));
  v8i v;
  v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
  v[4] = y.x; v[5] = y.y; v[6] = y.z; v[7] = y.w;
  return v;
}

template <int HG, int BS, bool WIDE>
__global__ __launch_bounds__(64 * WAVES, Form<WIDE>::MIN_WG) void k_indexer_select(Args a) {
  constexpr int CAP = Form<WIDE>::CAP;
  constexpr int STAGE = Form<WIDE>::STAGE;
  __shared__ WaveLds<CAP> lds[WAVES];
  __shared__ __align__(16) uint8_t ktile[2][STAGE * D];   // staged keys, double buffered
  __shared__ int64_t row_s[WAVES], row_e[WAVES];
  const int w = wave(), l = lane();
  WaveLds<CAP>& s = lds[w];
  const int t = (int)blockIdx.x * WAVES + w;
  // Row bounds (both loads issued before either is used); rows past the
  // last query are empty.
  int64_t s0 = 0, e0 = 0;
  if (t < a.Q) {
    const int32_t* ep = a.ends + t / a.ends_repeat;
    const int32_t* sp = a.starts ? a.starts + t / a.starts_repeat : ep;
    const int32_t sv = *sp, ev = *ep;
    s0 = a.starts ? (int64_t)sv : 0;
    e0 = (int64_t)ev < a.S ? (int64_t)ev : a.S;
  }
  const int64_t L64 = (s0 < 0 || e0 <= s0) ? 0 : e0 - s0;
  const int L = (int)L64;
  if (l == 0) {
    row_s[w] = L ? s0 : -1;
    row_e[w] = L ? e0 : -1;
  }
  __syncthreads();
  // The workgroup stages each key tile once for all its rows when every
  // non-empty row starts at the same offset modulo 16 (then every row's
  // blocks line up with the 16-key halves of the tiles).
  int64_t base = -1, top = -1;
  int live_rows = 0;
  for (int x = 0; x < WAVES; ++x) {
    if (row_s[x] < 0) continue;
    ++live_rows;
    base = base < 0 ? row_s[x] : min(base, row_s[x]);
    top = max(top, row_e[x]);
  }
  bool shared_mode = live_rows >= 2;
  for (int x = 0; x < WAVES; ++x)
    if (row_s[x] >= 0 && ((row_s[x] - base) & 15) != 0) shared_mode = false;
  const int64_t s_ = s0;
  const int nlb = (L + BS - 1) / BS;
  const int Kb = min(a.k_blocks, nlb);
  // This lane's query slices (A operands) and head weights.
  v8i qa[HG];
  float wr[HG][4];
  if (L > 0) {
    const uint8_t* qrow = a.q + (int64_t)t * a.H * D;
#pragma unroll
    for (int g = 0; g < HG; ++g) {
      const int4* p = reinterpret_cast<const int4*>(qrow + (16 * g + (l & 15)) * D + (l >> 4) * 32);
      const int4 x = p[0], y = p[1];
      qa[g][0] = x.x; qa[g][1] = x.y; qa[g][2] = x.z; qa[g][3] = x.w;
      qa[g][4] = y.x; qa[g][5] = y.y; qa[g][6] = y.z; qa[g][7] = y.w;
#pragma unroll
      for (int i = 0; i < 4; ++i) wr[g][i] = a.w[(int64_t)t * a.H + 16 * g + 4 * (l >> 4) + i];
    }
  }
  const uint8_t* krow = a.k + s_ * D;
  float* lout = (a.logits_out && L > 0) ? a.logits_out + (int64_t)t * a.S + s_ : nullptr;
  const int c16 = l & 15;
  const int lo32 = l & 31;

  // ---- block pass: logits tile by tile, block maxima, streaming top-K_blk ----
  // Two 16-key halves per step.  After the head sums every lane group holds
  // its key's logit, so lanes 0-15 take the first half's and lanes 16-31 the
  // second's: one block maximum and one offer serve 32 keys.
  int n = 0;
  uint32_t thr = 0u;
  // One step's 32 logits (lanes 0-31, key k0 + lane, row-relative column
  // col) go to the block maxima and the candidate buffer.
  // ks: the key scale of this lane's key (1 without scales).
  auto consume = [&](float lg, int col, float ks) {
    const bool valid = l < 32 && col >= 0 && col < L;
    lg *= ks;
    if (lout && valid) lout[col] = lg;
    uint32_t key = valid ? f2key(lg) : 0u;
    key = group_max<BS>(key);
    const int b = col >= 0 ? col / BS : -1;
    const bool head = valid && (col % BS) == 0;
    if (b == nlb - 1) key = KEY_POS_INF;
    wave_offer(s, n, thr, Kb, head, key, (uint32_t)b);
  };
  if (shared_mode) {
    // Each thread stages PER_T of the 16-byte chunks of a STAGE-key step
    // (8 per key); the next step's chunks are loaded into registers while
    // this step's halves are computed from LDS.
    const int tid = (int)threadIdx.x;
    constexpr int PER_T = STAGE * D / 16 / (64 * WAVES);
    static_assert(PER_T * 32 == STAGE, "32 key rows per staged chunk round");
    // chunk u of this thread: key row (tid >> 3) + 32 u, chunk tid & 7
    const int tr = tid >> 3, tj = tid & 7;
    const int soff0 = tr * D + 16 * (tj ^ (tr & 7));     // (row + 32 u) & 7 == row & 7
    static_assert(PER_T == 2 || PER_T == 4, "two or four staged chunks per thread");
    int4 nxt0, nxt1, nxt2, nxt3;                         // nxt2, nxt3: four per thread
#define DSA_IDX_FETCH(k0)                                                                   \
    do {                                                                                    \
      const uint8_t* src_ = a.k + 16 * tj;                                                  \
      nxt0 = *reinterpret_cast<const int4*>(src_ + min((k0) + tr, top - 1) * D);            \
      nxt1 = *reinterpret_cast<const int4*>(src_ + min((k0) + tr + 32, top - 1) * D);       \
      if constexpr (PER_T == 4) {                                                           \
        nxt2 = *reinterpret_cast<const int4*>(src_ + min((k0) + tr + 64, top - 1) * D);     \
        nxt3 = *reinterpret_cast<const int4*>(src_ + min((k0) + tr + 96, top - 1) * D);     \
      }                                                                                     \
    } while (0)
#define DSA_IDX_STAGE(buf)                                                                  \
    do {                                                                                    \
      *reinterpret_cast<int4*>((buf) + soff0) = nxt0;                                       \
      *reinterpret_cast<int4*>((buf) + soff0 + 32 * D) = nxt1;                              \
      if constexpr (PER_T == 4) {                                                           \
        *reinterpret_cast<int4*>((buf) + soff0 + 64 * D) = nxt2;                            \
        *reinterpret_cast<int4*>((buf) + soff0 + 96 * D) = nxt3;                            \
      }                                                                                     \
    } while (0)
    // key scales of this lane's keys in a step (k0 + 32 m + l % 32), one
    // step ahead like the keys
    float ksc[STAGE / 32], ksn[STAGE / 32];
#pragma unroll
    for (int m = 0; m < STAGE / 32; ++m) {
      ksc[m] = a.kscale ? a.kscale[min(base + 32 * m + lo32, top - 1)] : 1.f;
      ksn[m] = 1.f;
    }
    DSA_IDX_FETCH(base);
    DSA_IDX_STAGE(ktile[0]);
    __syncthreads();
    int cur = 0;
    for (int64_t k0 = base; k0 < top; k0 += STAGE) {
      const bool more = k0 + STAGE < top;
      if (more) {
        DSA_IDX_FETCH(k0 + STAGE);
        if (a.kscale) {
#pragma unroll
          for (int m = 0; m < STAGE / 32; ++m)
            ksn[m] = a.kscale[min(k0 + STAGE + 32 * m + lo32, top - 1)];
        }
      }
      if (L > 0 && k0 + STAGE > s_ && k0 < e0) {
        const uint8_t* tile = ktile[cur];
        // Software pipeline over the step's pairs: the next pair's matrix
        // instructions are issued between the current pair's epilogue
        // instructions, so the matrix core and the vector ALU overlap within
        // the wave.
        v4f acc[2][2][HG];
        mfma_pair<HG>(qa, lds_key_slice(tile, 0), lds_key_slice(tile, 1), acc[0]);
#pragma unroll
        for (int m = 0; m < STAGE / 32; ++m) {
          if (m + 1 < STAGE / 32)
            mfma_pair<HG>(qa, lds_key_slice(tile, 2 * m + 2), lds_key_slice(tile, 2 * m + 3),
                          acc[(m + 1) & 1]);
          const float lg = epilogue_pair<HG>(wr, acc[m & 1]);
          if (m + 1 < STAGE / 32) {
#pragma unroll
            for (int x = 0; x < 2 * HG; ++x) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one matrix instruction
              __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // then four vector ALU
            }
          }
          consume(lg, (int)(k0 + 32 * m - s_) + lo32, ksc[m]);
        }
      }
      if (more) DSA_IDX_STAGE(ktile[cur ^ 1]);
#pragma unroll
      for (int m = 0; m < STAGE / 32; ++m) ksc[m] = ksn[m];
      __syncthreads();
      cur ^= 1;
    }
#undef DSA_IDX_FETCH
#undef DSA_IDX_STAGE
  } else if (L > 0) {
    // Each wave streams its own keys; a step's loads are issued one half ahead.
    v8i kx = load_key_slice(krow, min(c16, L - 1));
    for (int c0 = 0; c0 < L; c0 += 32) {
      const v8i ky = load_key_slice(krow, min(c0 + 16 + c16, L - 1));
      const float lga = logit_of<HG>(qa, wr, kx);
      if (c0 + 32 < L) kx = load_key_slice(krow, min(c0 + 32 + c16, L - 1));
      const float lgb = logit_of<HG>(qa, wr, ky);
      const int col = c0 + lo32;
      consume((l & 16) ? lgb : lga, col, a.kscale ? a.kscale[s_ + min(col, L - 1)] : 1.f);
    }
  }
  int32_t* bout = a.block_ids + (int64_t)t * a.k_blocks;
  int32_t* tout = a.token_ids + (int64_t)t * a.k_tokens;
  if (t >= a.Q) return;
  if (L == 0) {
    for (int i = l; i < a.k_blocks; i += 64) bout[i] = -1;
    for (int i = l; i < a.k_tokens; i += 64) tout[i] = -1;
    return;
  }
  const float* ksr = a.kscale ? a.kscale + s_ : nullptr;
  wave_lds_sync();
  (void)wave_keep_top(s, n, Kb);
  n = min(n, Kb);
  wave_lds_sync();
  // kept block ids, ascending
  for (int i = l; i < a.k_blocks; i += 64) bout[i] = i < n ? (int32_t)s.id[i] : -1;
  for (int i = l; i < n; i += 64) s.sel[i] = s.id[i];
  wave_lds_sync();

  // ---- token stage ----
  const int Kt = min(a.k_tokens, L);
  const int64_t C = (int64_t)(n - 1) * BS + (L - (int64_t)(nlb - 1) * BS);
  const int32_t s32 = (int32_t)s_;
  if (C <= Kt) {
    // all kept columns, then the first Kt - C dropped columns in column order
    const int64_t qt = Kt - C;
    for (int r = l; r < n; r += 64) {
      const int bb = (int)s.sel[r];
      const int cnt = min(BS, L - bb * BS);
      const int64_t pos = (int64_t)r * BS + min(qt, ((int64_t)bb - r) * BS);
      for (int e = 0; e < cnt; ++e) tout[pos + e] = s32 + bb * BS + e;
    }
    for (int f = l; f < qt; f += 64) {
      // the (f / BS)-th dropped block: i + (kept blocks below it)
      const int i = f / BS;
      int lo = 0, hi = n;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if ((int)s.sel[mid] - mid > i) hi = mid;
        else lo = mid + 1;
      }
      const int bnk = i + lo;
      const int col = bnk * BS + (f - i * BS);
      tout[col] = s32 + col;      // every block before it is taken whole
    }
    for (int i = Kt + l; i < a.k_tokens; i += 64) tout[i] = -1;
    return;
  }
  // Kept columns' logits again, 16 gathered columns at a time (kept column j
  // is column sel[j / BS] * BS + j % BS; only the newest block is partial).
  n = 0;
  thr = 0u;
  for (int j0 = 0; j0 < C; j0 += 16) {
    const int j = j0 + c16;
    const bool valid = j < C;
    const int jj = valid ? j : (int)C - 1;
    const int col = (int)s.sel[jj / BS] * BS + jj % BS;
    const v8i kbj = load_key_slice(krow, col);
    const float ksj = ksr ? ksr[col] : 1.f;
    const float lg = logit_of<HG>(qa, wr, kbj) * ksj;
    wave_offer(s, n, thr, Kt, valid && l < 16, f2key(lg), (uint32_t)col);
  }
  wave_lds_sync();
  (void)wave_keep_top(s, n, Kt);
  n = min(n, Kt);
  wave_lds_sync();
  for (int i = l; i < a.k_tokens; i += 64) tout[i] = i < n ? s32 + (int32_t)s.id[i] : -1;
}

}  // namespace idx
}  // namespace dsa

// ===========================================================================
// Host side
// ===========================================================================
namespace {

thread_local std::string g_idx_err;

int idx_fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_idx_err = buf;
  return code;
}

template <int HG, bool WIDE>
int launch_hg(int B, unsigned grid, const dsa::idx::Args& a, hipStream_t st) {
  using namespace dsa::idx;
  const dim3 g(grid), t(64 * WAVES);
  switch (B) {
    case 1: hipLaunchKernelGGL((k_indexer_select<HG, 1, WIDE>), g, t, 0, st, a); break;
    case 2: hipLaunchKernelGGL((k_indexer_select<HG, 2, WIDE>), g, t, 0, st, a); break;
    case 4: hipLaunchKernelGGL((k_indexer_select<HG, 4, WIDE>), g, t, 0, st, a); break;
    case 8: hipLaunchKernelGGL((k_indexer_select<HG, 8, WIDE>), g, t, 0, st, a); break;
    default: hipLaunchKernelGGL((k_indexer_select<HG, 16, WIDE>), g, t, 0, st, a); break;
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return idx_fail(DSA_ERR_HIP, "k_indexer_select launch: %s", hipGetErrorString(e));
  return DSA_OK;
}

}  // namespace

extern "C" {

const char* dsa_indexer_last_error(void) { return g_idx_err.c_str(); }

int dsa_indexer_select(const dsa_indexer_shape* sh, int device, const uint8_t* q,
                       const uint8_t* k, const float* w, const float* kscale,
                       const int32_t* starts, const int32_t* ends, int32_t* block_ids,
                       int32_t* token_ids, float* logits_out, hipStream_t stream) {
  using namespace dsa::idx;
  if (!sh) return idx_fail(DSA_ERR_INVALID_ARG, "shape is null");
  if (sh->queries < 0 || sh->keys < 0) return idx_fail(DSA_ERR_INVALID_ARG, "queries and keys must be >= 0");
  if (sh->keys >= ((int64_t)1 << 31)) return idx_fail(DSA_ERR_UNSUPPORTED, "keys must be < 2^31");
  if (sh->head_dim != D) return idx_fail(DSA_ERR_UNSUPPORTED, "head_dim must be %d", D);
  if (sh->heads != 16 && sh->heads != 32 && sh->heads != 64)
    return idx_fail(DSA_ERR_UNSUPPORTED, "heads must be 16, 32 or 64");
  const int B = sh->block_size;
  if (B != 1 && B != 2 && B != 4 && B != 8 && B != 16)
    return idx_fail(DSA_ERR_UNSUPPORTED, "block_size must be 1, 2, 4, 8 or 16");
  if (sh->k_blocks < 1 || sh->k_tokens < 1)
    return idx_fail(DSA_ERR_INVALID_ARG, "k_blocks and k_tokens must be >= 1");
  constexpr int KMAX = Form<true>::KMAX;
  if (sh->k_blocks > KMAX) return idx_fail(DSA_ERR_UNSUPPORTED, "k_blocks must be <= %d", KMAX);
  const bool recompute = (int64_t)sh->k_blocks * B > sh->k_tokens;   // tokens selected again
  if (recompute && sh->k_tokens > KMAX)
    return idx_fail(DSA_ERR_UNSUPPORTED,
                    "k_tokens must be <= %d when k_blocks * block_size exceeds it", KMAX);
  // the narrow form when its buffer holds every K the call keeps
  constexpr int KN = Form<false>::KMAX;
  const bool wide = sh->k_blocks > KN || (recompute && sh->k_tokens > KN);
  if (sh->starts_repeat < 1 || sh->ends_repeat < 1)
    return idx_fail(DSA_ERR_INVALID_ARG, "repeats must be >= 1");
  if (device < 0) return idx_fail(DSA_ERR_INVALID_ARG, "device must be >= 0");
  if (sh->queries == 0) return DSA_OK;
  if (!q || !k || !w || !ends || !block_ids || !token_ids)
    return idx_fail(DSA_ERR_INVALID_ARG, "q, k, w, ends, block_ids and token_ids must be non-null");
  if (((uintptr_t)q | (uintptr_t)k) & 15u)
    return idx_fail(DSA_ERR_INVALID_ARG, "q and k must be 16-byte aligned");
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return idx_fail(DSA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (cur != device && (e = hipSetDevice(device)) != hipSuccess)
    return idx_fail(DSA_ERR_HIP, "hipSetDevice: %s", hipGetErrorString(e));
  Args a;
  std::memset(&a, 0, sizeof(a));
  a.q = q; a.k = k; a.w = w; a.kscale = kscale; a.starts = starts; a.ends = ends;
  a.block_ids = block_ids; a.token_ids = token_ids; a.logits_out = logits_out;
  a.S = sh->keys; a.Q = sh->queries; a.H = sh->heads; a.B = B;
  a.k_blocks = sh->k_blocks; a.k_tokens = sh->k_tokens;
  a.starts_repeat = sh->starts_repeat; a.ends_repeat = sh->ends_repeat;
  const unsigned grid = (unsigned)((sh->queries + WAVES - 1) / WAVES);
  int rc;
  if (sh->heads == 16)
    rc = wide ? launch_hg<1, true>(B, grid, a, stream) : launch_hg<1, false>(B, grid, a, stream);
  else if (sh->heads == 32)
    rc = wide ? launch_hg<2, true>(B, grid, a, stream) : launch_hg<2, false>(B, grid, a, stream);
  else
    rc = wide ? launch_hg<4, true>(B, grid, a, stream) : launch_hg<4, false>(B, grid, a, stream);
  if (cur != device) (void)hipSetDevice(cur);
  return rc;
}

}  // extern "C"

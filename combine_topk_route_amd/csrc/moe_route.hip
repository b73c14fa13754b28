// MI355X (gfx950, CDNA4) kernels for MoE top-k routing, dispatch and combine,
// behind the C ABI declared in include/moe_route.h.
//
// The operations follow "Efficient and portable mixture-of-experts
// communication" (sections "Introduction", "Dispatch", "Combine") and
// "Enabling trillion-parameter models on AWS EFA" (sections "Send and Receive
// Buffers", "Dispatch and Combine"); the router is the Mixtral special case of
// "Lower latency and higher throughput with multi-node DeepSeek deployment",
// section "MoE Router".  The pages' kernels target NVSHMEM / EFA on H100 and
// H200; here everything is one GPU, and the kernels are shaped for wave64,
// DPP/ballot cross-lane operations, LDS and HBM3E:
//
//   route_topk_kernel    batches above 2048 tokens: 16, 32 or 64 lanes per
//                        token (the fewest that still fill the chip), each
//                        lane holding consecutive experts; every lane caches
//                        its 4 best order-preserving 32-bit keys, so each of
//                        the k selection rounds is one DPP maximum over the
//                        cache heads of the token's lanes.  The weights are
//                        the winners' softmax probabilities renormalised
//                        over the k winners, formed from their k numerators
//                        alone (the E-term denominator cancels).  It also
//                        runs group-limited routing where every group is
//                        1-16 whole lanes.  Inside moe_route_dispatch
//                        (E >= 128) the routing kernels also count each pair
//                        into the send histogram with an atomic add, in
//                        place of send_hist_kernel.  Below 128 experts,
//                        route_topk_lds_count_kernel counts each 16-token
//                        tile in LDS and adds the tile's bins instead.
//   route_wave_kernel    one wave per token (small batches, and group-limited
//                        routing the lane-group kernel cannot hold): k rounds
//                        of a wave-wide maximum of the keys, the lowest
//                        expert index holding it found by ballot.
//   send_hist_kernel     per-block expert histogram; each wave groups equal
//                        experts with ballots so the hot expert costs one LDS
//                        update per wave, not 64.
//   send_rank_kernel     stable slot of every pair: rank among equal experts
//                        inside a wave (mbcnt), exclusive prefix across waves
//                        (LDS), and across blocks from the histogram matrix,
//                        which every block scans for itself.  Small inputs run
//                        histogram, scan and slots in one block of 8 or 16
//                        waves.
//   send_recv_kernel     small batches (T*k <= 2048, k <= 8): block 0 runs the
//                        single-block send while the other blocks copy rows,
//                        each finding its token's k rows from topk_idx with
//                        ballot counts (lower experts, earlier equal ones).
//   route_send_kernel    small batches up to T*k = 4096: routing (one wave per
//                        token) and the single-block send in one launch; the
//                        last block to finish routing, found with a
//                        device-scope arrival counter, runs the send.
//   dispatch_recv_kernel one block per (token, two 1 KiB column slices); each
//                        wave copies both slices to one of the token's k
//                        rows: two cached 16-byte loads per lane (the block's
//                        waves share them), both issued before the
//                        non-temporal 16-byte stores.
//   dispatch_recv_fp8_kernel
//                        the same scatter with block-scaled fp8 payloads:
//                        each 16-lane DPP row holds one 128-element block, so
//                        its amax is an in-row DPP maximum; the block's waves
//                        quantise 8 slices into LDS once, then each wave
//                        streams one destination row's codes and scales.
//   send_recv_fp8_kernel small batches, as send_recv_kernel with the fp8
//                        receive: block 0 sends, the other blocks quantise a
//                        4096-element unit of a token's row into LDS while
//                        they count its rows, then store it to each of them.
//   combine_kernel       one wave per (token, 1 KiB column slice): k
//                        non-temporal 16-byte row loads in flight, fp32 fma
//                        chain in j order, one bf16 RNE (v_cvt_pk_bf16_f32).
//                        The token's rows and weights come through the scalar
//                        cache into SGPRs.  k = 1, 2, 4, 8 run
//                        combine_small_k_kernel, which loads them all before
//                        issuing its row loads back to back; for k < 8 a wave
//                        covers several slices so that 16 row loads are in
//                        flight.  Above 256 MiB of combine bytes the output
//                        rows are stored with the sc1 cache policy.
//
// There is no dense contraction here, so no MFMA: the row kernels are bound by
// HBM bandwidth and the routing / send kernels by latency.

#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

#include <atomic>
#include <mutex>
#include <tuple>
#include <utility>

#include "moe_route.h"

namespace {

constexpr int kWave = 64;
constexpr int kMaxE = 1024;
constexpr int kMaxK = 32;
constexpr int kMaxGroups = 64;  // one lane per group in the group selection
constexpr int64_t kMaxPairs = (int64_t(1) << 31) - 1;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// wave helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u));
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

// DPP controls (gfx9): quad permutes, row mirrors and the row broadcasts.
constexpr int kDppQuad1032 = 0xB1;     // quad_perm:[1,0,3,2]
constexpr int kDppQuad2301 = 0x4E;     // quad_perm:[2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowBcast15 = 0x142;  // lane 15 of each row -> next row
constexpr int kDppRowBcast31 = 0x143;  // lane 31 -> rows 2 and 3
constexpr int kDppRowShr1 = 0x111;     // row_shr:1 (lane i of a row reads lane i-1)
constexpr int kDppRowShr2 = 0x112;
constexpr int kDppRowShr4 = 0x114;
constexpr int kDppRowShr8 = 0x118;

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp(uint32_t old, uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(old), static_cast<int>(v),
                                                           CTRL, ROW_MASK, 0xF, false));
}

__device__ __forceinline__ uint32_t readlane(uint32_t v, int lane) {
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), lane));
}

// Wave-wide reductions over all 64 lanes (all must be active).  The four
// in-row steps leave every lane of a 16-lane row with the row's result; the
// two broadcasts fold rows into lane 63, which is read into a scalar.  The
// `old` operand of each DPP move is the operation's identity (lanes a row
// mask leaves out then contribute nothing), which lets the compiler fuse the
// move into the arithmetic: one v_max_u32_dpp per step.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#define MOE_STEP(CTRL, RM) v = max(v, dpp<CTRL, RM>(0u, v))
  MOE_STEP(kDppQuad1032, 0xF);
  MOE_STEP(kDppQuad2301, 0xF);
  MOE_STEP(kDppRowHalfMirror, 0xF);
  MOE_STEP(kDppRowMirror, 0xF);
  MOE_STEP(kDppRowBcast15, 0xA);
  MOE_STEP(kDppRowBcast31, 0xC);
#undef MOE_STEP
  return readlane(v, kWave - 1);
}

// Inclusive prefix sum over the 64 lanes (all active): four shifts inside
// each 16-lane row, then each row's running total carried into the rows
// above it by the two row broadcasts.  Lanes a shift or a row mask leaves
// out take the identity 0.
__device__ __forceinline__ int32_t wave_incl_scan(int32_t v) {
  uint32_t u = static_cast<uint32_t>(v);
#define MOE_STEP(CTRL, RM) u += dpp<CTRL, RM>(0u, u)
  MOE_STEP(kDppRowShr1, 0xF);
  MOE_STEP(kDppRowShr2, 0xF);
  MOE_STEP(kDppRowShr4, 0xF);
  MOE_STEP(kDppRowShr8, 0xF);
  MOE_STEP(kDppRowBcast15, 0xA);
  MOE_STEP(kDppRowBcast31, 0xC);
#undef MOE_STEP
  return static_cast<int32_t>(u);
}

// Lanes of the wave whose `valid` lane holds the same expert id `e`
// (all lanes of the wave must be active).  One ballot per bit of the id.
__device__ __forceinline__ uint64_t same_expert_lanes(int e, bool valid, int nbits) {
  uint64_t m = ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t v = ballot(bit);
    m &= bit ? v : ~v;
  }
  return m;
}

// In-place exclusive scan of data[0, n) in LDS (n <= 1024); returns the total.
// Every thread of the block must call it.  tmp: >= 17 ints of LDS.
__device__ int32_t block_excl_scan(int32_t* data, int n, int32_t* tmp) {
  const int nthreads = blockDim.x;
  const int nwaves = nthreads / kWave;
  const int lane = lane_id();
  const int wid = threadIdx.x / kWave;
  const int per = (n + nthreads - 1) / nthreads;
  const int beg = threadIdx.x * per;
  int32_t s = 0;
  for (int i = 0; i < per; ++i)
    if (beg + i < n) s += data[beg + i];
  const int32_t incl = wave_incl_scan(s);
  if (lane == kWave - 1) tmp[wid] = incl;
  __syncthreads();
  if (wid == 0) {
    const int32_t ws = lane < nwaves ? tmp[lane] : 0;
    const int32_t wi = wave_incl_scan(ws);
    if (lane < nwaves) tmp[lane] = wi - ws;
    if (lane == nwaves - 1) tmp[16] = wi;
  }
  __syncthreads();
  int32_t run = tmp[wid] + incl - s;
  for (int i = 0; i < per; ++i) {
    if (beg + i < n) {
      const int32_t v = data[beg + i];
      data[beg + i] = run;
      run += v;
    }
  }
  const int32_t total = tmp[16];
  __syncthreads();
  return total;
}

// ---------------------------------------------------------------------------
// route: softmax + top-k, one wave per token
// ---------------------------------------------------------------------------

// Monotone map of a float onto uint32 (larger float -> larger key), with -0.0
// folded into +0.0 so that the two compare equal.  Every finite float maps
// above 0x007FFFFF, so 0 can mark "not a candidate".
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  u = (u == 0x80000000u) ? 0u : u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inverse of order_key on its image (a folded -0.0 comes back as +0.0).
__device__ __forceinline__ float key_value(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// s_waitcnt operand that waits for every vector memory operation of the wave
// (vmcnt 0) and leaves the export and LDS/scalar counters unconstrained:
// vmcnt bits [3:0] and [15:14] = 0, expcnt [6:4] = 7, lgkmcnt [11:8] = 15.
constexpr int kWaitVmcnt0 = 0x0F70;

constexpr int kRouteWavesPerBlock = 4;
constexpr int kRouteThreads = kRouteWavesPerBlock * kWave;
constexpr int64_t kRouteWaveMaxTokens = 2048;  // up to here plain routing uses one wave per token
constexpr int64_t kRouteMaxBlocks = int64_t(1) << 20;  // beyond this, waves loop over token tiles
// Fewest experts for which moe_route_dispatch's routing kernel counts the send
// histogram itself: with fewer, its per-pair atomics pile onto too few
// addresses (E = 8: each takes a few hundred).
constexpr int kRouteCountMinE = 128;

// Softmax numerator exp(a - m).  The difference is split into its fp32
// rounding d and the exact remainder r (TwoSum), and exp(d + r) is taken as
// exp(d) * (1 + r): the subtraction then adds no error of its own.  A
// difference beyond the fp32 range (finite logits more than FLT_MAX apart)
// is held at -FLT_MAX: exp gives 0 and r stays finite, where -inf would make
// r, and the whole softmax, NaN.
__device__ __forceinline__ float shifted_exp(float a, float m) {
  const float b = -m;
  const float d = fmaxf(a + b, -__FLT_MAX__);
  const float bb = d - a;
  const float r = (a - (d - bb)) + (b - bb);
  const float ed = expf(d);
  return __builtin_fmaf(ed, r, ed);
}

// Maximum over the G lanes that share one token (G = 16, 32 or 64; a group
// starts at a multiple of G).  Every lane of the group gets the result.
template <int G>
__device__ __forceinline__ uint32_t group_max_u32(uint32_t v) {
  v = max(v, dpp<kDppQuad1032, 0xF>(0u, v));
  v = max(v, dpp<kDppQuad2301, 0xF>(0u, v));
  v = max(v, dpp<kDppRowHalfMirror, 0xF>(0u, v));
  v = max(v, dpp<kDppRowMirror, 0xF>(0u, v));
  if constexpr (G == 32) {
    v = max(v, dpp<kDppRowBcast15, 0xA>(0u, v));
    const uint32_t lo = readlane(v, 31), hi = readlane(v, kWave - 1);
    v = lane_id() < 32 ? lo : hi;
  } else if constexpr (G == 64) {
    v = max(v, dpp<kDppRowBcast15, 0xA>(0u, v));
    v = max(v, dpp<kDppRowBcast31, 0xC>(0u, v));
    v = readlane(v, kWave - 1);
  }
  return v;
}

// Error-free sum of two floats: s + e == a + b exactly (TwoSum; the result
// does not depend on the operand order).
__device__ __forceinline__ void two_sum(float a, float b, float& s, float& e) {
  s = a + b;
  const float bb = s - a;
  e = (a - (s - bb)) + (b - bb);
}

// (s, c) <- the compensated sum over the token's G lanes of (s, c): every
// step adds the partner's sum exactly (TwoSum) and carries the rounding
// error in c.  Every lane of the group gets bit-identical results: the
// in-row steps are butterflies and TwoSum is exact in either operand order,
// and the cross-row result is read from one lane.  Lanes that a row mask
// leaves out add (0, 0), which changes nothing.
template <int G>
__device__ __forceinline__ void group_sum_compensated(float& s, float& c) {
#define MOE_STEP(CTRL, RM)                                                     \
  {                                                                            \
    const float os = __uint_as_float(dpp<CTRL, RM>(0u, __float_as_uint(s)));   \
    const float oc = __uint_as_float(dpp<CTRL, RM>(0u, __float_as_uint(c)));   \
    float e;                                                                   \
    two_sum(s, os, s, e);                                                      \
    c = (c + oc) + e;                                                          \
  }
  MOE_STEP(kDppQuad1032, 0xF);
  MOE_STEP(kDppQuad2301, 0xF);
  MOE_STEP(kDppRowHalfMirror, 0xF);
  MOE_STEP(kDppRowMirror, 0xF);
  if constexpr (G == 32) {
    MOE_STEP(kDppRowBcast15, 0xA);
    const bool lo = lane_id() < 32;
    const uint32_t s_lo = readlane(__float_as_uint(s), 31), s_hi = readlane(__float_as_uint(s), 63);
    const uint32_t c_lo = readlane(__float_as_uint(c), 31), c_hi = readlane(__float_as_uint(c), 63);
    s = __uint_as_float(lo ? s_lo : s_hi);
    c = __uint_as_float(lo ? c_lo : c_hi);
  } else if constexpr (G == 64) {
    MOE_STEP(kDppRowBcast15, 0xA);
    MOE_STEP(kDppRowBcast31, 0xC);
    s = __uint_as_float(readlane(__float_as_uint(s), kWave - 1));
    c = __uint_as_float(readlane(__float_as_uint(c), kWave - 1));
  }
#undef MOE_STEP
}

// The G bits of wave mask m that belong to token slot q (lanes q*G ..).
template <int G>
__device__ __forceinline__ uint64_t token_bits(uint64_t m, int q) {
  if constexpr (G == kWave)
    return m;
  else
    return (m >> (q * G)) & ((uint64_t(1) << G) - 1);
}

// Insert (kv, i) into a lane's cache of its C best candidates, kept in the
// selection order: larger key first, and among equal keys the lower item
// (= lower expert).  Items are pushed in ascending order with strict
// comparisons, so the lower item stays ahead on ties.
template <int C>
__device__ __forceinline__ void cache_push(uint32_t kv, int i, uint32_t (&h)[C], int (&hi)[C]) {
  bool gt[C];
#pragma unroll
  for (int c = 0; c < C; ++c) gt[c] = kv > h[c];
#pragma unroll
  for (int c = C - 1; c > 0; --c) {
    h[c] = gt[c - 1] ? h[c - 1] : (gt[c] ? kv : h[c]);
    hi[c] = gt[c - 1] ? hi[c - 1] : (gt[c] ? i : hi[c]);
  }
  h[0] = gt[0] ? kv : h[0];
  hi[0] = gt[0] ? i : hi[0];
}

// Plain top-k routing.  G lanes per token, 64 / G tokens per wave; lane g of
// a token holds the IPL consecutive experts g*IPL .. g*IPL + IPL - 1, so a
// lower lane always holds lower experts.  Each lane caches its C best
// candidates in selection order; a selection round is then one group maximum
// over the cache heads, and the lowest lane holding that maximum owns the
// winner (the lowest expert index on ties).  The owner pops its head.  A lane
// whose cache runs empty while it still holds candidates rescans its items
// for the best C after the popped one; with C = 4 that needs a lane to hold
// four of a token's winners (about 1 % of tokens at E = 256, k = 8).
// VEC: 16-byte logit loads (IPL % 4 == 0, E % 4 == 0, 16-byte aligned rows).
// COUNT: the owner of winner j also adds the pair p = t*k + j to the send
// histogram matrix, row p / chunk (chunk >= 64 > j, so a token's pairs span at
// most two rows); the matrix must hold zeros beforehand.
// GROUPED: group-limited routing (as in route_wave_kernel) where every group
// is 2^lg whole lanes (E / n_group == 2^lg * IPL, lg <= 4): a group's score
// is its lanes' largest key, folded over those lanes by DPP; topk_group
// rounds of a group maximum keep the best groups (ties to the lower group),
// and the lanes of the other groups drop their keys before the k rounds.
// The calling wave routes tokens t_wave .. t_wave + 64/G - 1 (t_wave < T).
// LDS (with COUNT): hist_mat is the calling block's LDS tile of matrix rows
// row_first, row_first + 1, ...; the counts go there instead.
template <int G, int IPL, bool VEC, bool COUNT, bool GROUPED, bool LDS = false>
__device__ __forceinline__ void route_topk_tile(const float* __restrict__ logits, int64_t T,
                                                int E, int k, int topk_group, int lg,
                                                int32_t* __restrict__ topk_idx,
                                                float* __restrict__ topk_w,
                                                int32_t* __restrict__ hist_mat, uint32_t chunk,
                                                int64_t t_wave, uint32_t row_first = 0u) {
  constexpr int TPW = kWave / G;         // tokens per wave
  constexpr int C = IPL < 4 ? IPL : 4;   // cached candidates per lane
  const int lane = lane_id();
  const int q = lane / G;  // token slot inside the wave
  const int g = lane % G;  // lane inside the token's group
  const int64_t t = t_wave + q;
  const int64_t t_ld = t < T ? t : T - 1;  // lanes past T repeat the last token and store nothing
  const int e0 = g * IPL;
  const float* row = logits + t_ld * E + e0;
  int32_t* idx_out = topk_idx + t_ld * k;
  uint32_t row0 = 0u, rem0 = 0u;  // histogram row and offset in it of the pair t*k
  if constexpr (COUNT) {
    const uint32_t p0 = uint32_t(t_ld * k);
    row0 = p0 / chunk;
    rem0 = p0 - row0 * chunk;
  }

  float lv[IPL];
  if constexpr (VEC) {
#pragma unroll
    for (int v = 0; v < IPL / 4; ++v) {
      float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
      if (e0 + 4 * v < E) f = *reinterpret_cast<const float4*>(row + 4 * v);
      lv[4 * v] = f.x;
      lv[4 * v + 1] = f.y;
      lv[4 * v + 2] = f.z;
      lv[4 * v + 3] = f.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < IPL; ++i) lv[i] = e0 + i < E ? row[i] : 0.f;
  }

  // Order keys (0 marks "no expert"); the maximum logit is the maximum key.
  uint32_t key[IPL];
#pragma unroll
  for (int i = 0; i < IPL; ++i) key[i] = e0 + i < E ? order_key(lv[i]) : 0u;

  if constexpr (GROUPED) {
    // Every lane of group g >> lg ends up with the group's score; lanes past
    // E form groups of their own with score 0, which no round picks (a real
    // group's score is a nonzero key, and topk_group <= n_group).
    uint32_t score = 0u;
#pragma unroll
    for (int i = 0; i < IPL; ++i) score = max(score, key[i]);
    if (lg >= 1) score = max(score, dpp<kDppQuad1032, 0xF>(0u, score));
    if (lg >= 2) score = max(score, dpp<kDppQuad2301, 0xF>(0u, score));
    if (lg >= 3) score = max(score, dpp<kDppRowHalfMirror, 0xF>(0u, score));
    if (lg >= 4) score = max(score, dpp<kDppRowMirror, 0xF>(0u, score));
    const int my_group = g >> lg;
    bool kept = false;
    for (int r = 0; r < topk_group; ++r) {
      const uint32_t best = group_max_u32<G>(score);
      // the lowest lane with the best score lies in the lowest such group
      const int pick = int(__builtin_ctzll(token_bits<G>(ballot(score == best), q))) >> lg;
      if (my_group == pick) {
        kept = true;
        score = 0u;
      }
    }
    if (!kept) {
#pragma unroll
      for (int i = 0; i < IPL; ++i) key[i] = 0u;
    }
  }

  uint32_t h[C];
  int hi[C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    h[c] = 0u;
    hi[c] = 0;
  }
#pragma unroll
  for (int i = 0; i < IPL; ++i) cache_push<C>(key[i], i, h, hi);
  int rem = E - e0 < IPL ? (E - e0 > 0 ? E - e0 : 0) : IPL;  // candidates not yet taken

  uint32_t my_key = 0u;  // lane g < k: key of winner j = g
  uint32_t top = 0u;     // the first winner's key: the token's largest logit
  for (int j = 0; j < k; ++j) {
    const uint32_t best = group_max_u32<G>(h[0]);
    top = max(top, best);  // winners come in descending order: the first one
    const bool hit = h[0] == best;
    const uint64_t hits = ballot(hit);
    bool owner = hit;
    if (__popcll(hits) > TPW) {
      // Some token has equal heads in several lanes: its lowest lane wins.
      owner = hit && (token_bits<G>(hits, q) & ((uint64_t(1) << g) - 1)) == 0;
    }
    if (g == j) my_key = best;
    const uint32_t kp = h[0];
    const int ip = hi[0];
    if (owner) {
      if (t < T) {
        idx_out[j] = e0 + ip;  // the owner reports winner j
        if constexpr (COUNT) {
          const uint32_t row = row0 + (rem0 + uint32_t(j) >= chunk ? 1u : 0u);
          if constexpr (LDS)
            atomicAdd(hist_mat + (row - row_first) * uint32_t(E) + e0 + ip, 1);
          else
            __hip_atomic_fetch_add(hist_mat + size_t(row) * E + e0 + ip, 1, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      --rem;
#pragma unroll
      for (int c = 0; c + 1 < C; ++c) {
        h[c] = h[c + 1];
        hi[c] = hi[c + 1];
      }
      h[C - 1] = 0u;
    }
    const bool refill = owner && h[0] == 0u && rem > 0 && j + 1 < k;
    if (ballot(refill) != 0) {
      if (refill) {
        // The best C among the items after the popped one (kp, ip) in the
        // selection order: smaller key, or equal key and higher item.
#pragma unroll
        for (int c = 0; c < C; ++c) h[c] = 0u;
#pragma unroll
        for (int i = 0; i < IPL; ++i) {
          const uint32_t kv = key[i];
          const bool after = kv < kp || (kv == kp && i > ip);
          cache_push<C>(after ? kv : 0u, i, h, hi);
        }
      }
    }
  }

  // Lane g < k of each token: numerator of winner g against the largest
  // logit; the winners' total by a compensated sum over the group; winner
  // g's share of it.  That share is its softmax probability renormalised
  // over the k winners: the softmax denominator cancels, so it is never
  // formed.
  float z = 0.f;
  if (g < k) z = shifted_exp(key_value(my_key), key_value(top));
  float zsum = z, zcomp = 0.f;
  group_sum_compensated<G>(zsum, zcomp);
  if (g < k && t < T) topk_w[t * k + g] = z / (zsum + zcomp);
}

// Waves take tiles of 64/G tokens in grid-stride order, so the grid stays
// within the launch's 32-bit work-item count at any T.  No block barrier
// follows the loop: a wave past T just leaves.
template <int G, int IPL, bool VEC, bool COUNT, bool GROUPED>
__global__ __launch_bounds__(kRouteThreads) void route_topk_kernel(
    const float* __restrict__ logits, int64_t T, int E, int k, int topk_group, int lg,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, int32_t* __restrict__ hist_mat,
    uint32_t chunk) {
  constexpr int TPW = kWave / G;  // tokens per wave
  const int64_t stride = int64_t(gridDim.x) * kRouteWavesPerBlock * TPW;
  for (int64_t t_wave = (int64_t(blockIdx.x) * kRouteWavesPerBlock + threadIdx.x / kWave) * TPW;
       t_wave < T; t_wave += stride)
    route_topk_tile<G, IPL, VEC, COUNT, GROUPED>(logits, T, E, k, topk_group, lg, topk_idx,
                                                 topk_w, hist_mat, chunk, t_wave);
}

// Counting routing for few experts (E < kRouteCountMinE), where one global
// atomic per pair would pile onto too few addresses: each block routes tiles
// of TPB tokens (one wave tile each) and counts the tile's pairs in LDS, one
// bin per (matrix row, expert), then adds its nonzero bins to the matrix.
// A tile's TPB * k <= 16 * 32 pairs span at most kRows rows (chunk >= 64).
// The tile loop's bounds are the same for every wave of the block, so all of
// them reach each barrier; a wave whose tile starts past T only counts in.
template <int G, int IPL, bool VEC>
__global__ __launch_bounds__(kRouteThreads) void route_topk_lds_count_kernel(
    const float* __restrict__ logits, int64_t T, int E, int k, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, int32_t* __restrict__ hist_mat, uint32_t chunk) {
  constexpr int TPB = kRouteWavesPerBlock * (kWave / G);  // tokens per block tile
  constexpr int kRows = (TPB * kMaxK + 63) / 64 + 1;
  __shared__ int32_t bins[kRows * kRouteCountMinE];
  const int wid = threadIdx.x / kWave;
  const int64_t stride = int64_t(gridDim.x) * TPB;
  for (int64_t t_block = int64_t(blockIdx.x) * TPB; t_block < T; t_block += stride) {
    const int64_t t_end = t_block + TPB < T ? t_block + TPB : T;
    const uint32_t row_first = uint32_t(t_block * k / chunk);
    const int n = int(uint32_t((t_end * k - 1) / chunk) - row_first + 1) * E;
    for (int i = threadIdx.x; i < n; i += kRouteThreads) bins[i] = 0;
    __syncthreads();
    const int64_t t_wave = t_block + int64_t(wid) * (kWave / G);
    if (t_wave < T)
      route_topk_tile<G, IPL, VEC, true, false, true>(logits, T, E, k, 1, 0, topk_idx, topk_w,
                                                      bins, chunk, t_wave, row_first);
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += kRouteThreads) {
      const int32_t c = bins[i];
      if (c != 0)
        __hip_atomic_fetch_add(hist_mat + size_t(row_first) * E + i, c, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();  // the next tile clears the bins
  }
}

// One wave per token; IPL logits per lane (expert e = lane + 64 * i).  The
// shortest dependent chain per token, so small batches use it for plain
// routing too.  GROUPED: group-limited routing; experts form n_group
// contiguous groups, a group's score is its largest logit, and only the
// topk_group best groups (ties to the lower group) take part in the top-k.
// Routing of token t by the calling wave (all 64 lanes active).
// COUNT: as in route_topk_kernel, lane j < k adds pair t*k + j to the
// zero-initialised send histogram matrix.
template <int IPL, bool GROUPED, bool COUNT>
__device__ __forceinline__ void route_wave_token(const float* __restrict__ logits, int64_t t, int E,
                                                 int k, int n_group, int topk_group,
                                                 int32_t* __restrict__ topk_idx,
                                                 float* __restrict__ topk_w,
                                                 int32_t* __restrict__ hist_mat, uint32_t chunk) {
  const int lane = lane_id();
  const float* row = logits + t * E;

  uint32_t key[IPL];  // order keys; 0 marks "no expert"
#pragma unroll
  for (int i = 0; i < IPL; ++i) {
    const int e = lane + i * kWave;
    key[i] = e < E ? order_key(row[e]) : 0u;
  }

  if (GROUPED) {
    const int gs = E / n_group;
    int grp[IPL];
#pragma unroll
    for (int i = 0; i < IPL; ++i) grp[i] = (lane + i * kWave) / gs;
    // Lane g ends up holding the key of group g's largest logit.
    uint32_t gv = 0u;
    for (int g = 0; g < n_group; ++g) {
      uint32_t local = 0u;
#pragma unroll
      for (int i = 0; i < IPL; ++i) local = grp[i] == g ? max(local, key[i]) : local;
      const uint32_t gk = wave_max_u32(local);
      if (lane == g) gv = gk;
    }
    uint64_t kept = 0;
    for (int r = 0; r < topk_group; ++r) {
      const uint32_t best = wave_max_u32(gv);
      const int g = __builtin_ctzll(ballot(gv == best));  // lowest group with that score
      kept |= uint64_t(1) << g;
      if (lane == g) gv = 0u;
    }
#pragma unroll
    for (int i = 0; i < IPL; ++i)
      if (lane + i * kWave >= E || !((kept >> grp[i]) & 1)) key[i] = 0u;  // grp < 64 here
  }

  // k rounds: the largest remaining key, then the lowest expert index that
  // holds it (the first item slot with a match and, inside it, the lowest
  // lane).  Selected keys are zeroed.  Lane j keeps winner j.
  int my_e = 0;
  uint32_t my_key = 0u;
  uint32_t top = 0u;  // the first winner's key: the largest logit (its group is kept)
  for (int j = 0; j < k; ++j) {
    uint32_t best = 0u;
#pragma unroll
    for (int i = 0; i < IPL; ++i) best = max(best, key[i]);
    best = wave_max_u32(best);
    top = max(top, best);  // winners come in descending order: the first one
    int item = 0;
    uint64_t hit = 0;
#pragma unroll
    for (int i = IPL - 1; i >= 0; --i) {
      const uint64_t h = ballot(key[i] == best);
      if (h != 0) {
        item = i;
        hit = h;
      }
    }
    const int owner = __builtin_ctzll(hit);
#pragma unroll
    for (int i = 0; i < IPL; ++i)
      if (i == item && lane == owner) key[i] = 0u;
    if (lane == j) {
      my_e = item * kWave + owner;
      my_key = best;
    }
  }
  // Winner j's numerator against the largest logit, on lane j; their total
  // in winner order.  Fast2Sum: the winners come in descending order, so
  // zsum >= zj >= 0 and the rounding error of zsum + zj is exactly
  // zj - (ns - zsum).  Winner j's share of the total is its softmax
  // probability renormalised over the k winners: the softmax denominator
  // cancels, so it is never formed.
  const float my_z = lane < k ? shifted_exp(key_value(my_key), key_value(top)) : 0.f;
  float zsum = 0.f, zcomp = 0.f;
  for (int j = 0; j < k; ++j) {
    const float zj = __uint_as_float(readlane(__float_as_uint(my_z), j));
    const float ns = zsum + zj;
    zcomp += zj - (ns - zsum);
    zsum = ns;
  }
  if (lane < k) {
    topk_idx[t * k + lane] = my_e;
    topk_w[t * k + lane] = my_z / (zsum + zcomp);
    if constexpr (COUNT) {
      const uint32_t pr = uint32_t(t * k + lane);
      __hip_atomic_fetch_add(hist_mat + size_t(pr / chunk) * E + my_e, 1, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

template <int IPL, bool GROUPED, bool COUNT>
__global__ __launch_bounds__(kRouteThreads) void route_wave_kernel(
    const float* __restrict__ logits, int64_t T, int E, int k, int n_group, int topk_group,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, int32_t* __restrict__ hist_mat,
    uint32_t chunk) {
  // Grid-stride over tokens, as in route_topk_kernel; no block barrier follows.
  const int64_t stride = int64_t(gridDim.x) * kRouteWavesPerBlock;
  for (int64_t t = int64_t(blockIdx.x) * kRouteWavesPerBlock + threadIdx.x / kWave; t < T;
       t += stride)
    route_wave_token<IPL, GROUPED, COUNT>(logits, t, E, k, n_group, topk_group, topk_idx, topk_w,
                                          hist_mat, chunk);
}

// ---------------------------------------------------------------------------
// dispatch send: histogram, scan, stable slots
// ---------------------------------------------------------------------------

constexpr int kSendThreads = 512;
constexpr int kSendWaves = kSendThreads / kWave;
constexpr int kSendItems = 4;  // pair indices each lane loads before processing them
constexpr int64_t kSendFusedMaxPairs = 4096;
// Above one 8-wave step (2048 pairs) the single block would park slots in
// memory for a second step; a 16-wave block keeps them in registers (its
// per-wave counts take 16 * E ints of LDS, hence the limit on E).
constexpr int kSendWideThreads = 1024;
constexpr int kSendWideMaxE = 512;
// Multi-block send: about kSendChunkTarget pairs per block, kSendRankItems
// per lane (8 waves), at most kSendMatrixInts counts in the [block][expert]
// histogram matrix.
constexpr int64_t kSendChunkTarget = 1024;
constexpr int kSendRankItems = 2;
constexpr int kSendMaxBlocks = 64;
constexpr int kSendMatrixInts = 16384;

struct SendPlan {
  bool fused;
  int threads;    // of the single fused block: kSendThreads or kSendWideThreads
  int nb;         // blocks of the histogram and rank kernels
  int64_t chunk;  // pairs per block
  size_t ws_bytes;
};

SendPlan plan_send(int64_t P, int E) {
  SendPlan p{};
  if (P <= kSendFusedMaxPairs) {
    const bool one_step = P <= int64_t(kSendWaves) * kWave * kSendItems;
    p.fused = true;
    p.threads = !one_step && E <= kSendWideMaxE ? kSendWideThreads : kSendThreads;
    p.nb = 1;
    p.chunk = P > 0 ? P : 1;
    p.ws_bytes = 0;
    return p;
  }
  int64_t nb = (P + kSendChunkTarget - 1) / kSendChunkTarget;
  int64_t nb_max = kSendMatrixInts / E;
  if (nb_max > kSendMaxBlocks) nb_max = kSendMaxBlocks;
  if (nb > nb_max) nb = nb_max;
  if (nb < 1) nb = 1;
  int64_t chunk = (P + nb - 1) / nb;
  chunk = (chunk + kWave - 1) / kWave * kWave;
  nb = (P + chunk - 1) / chunk;
  p.fused = false;
  p.nb = int(nb);
  p.chunk = chunk;
  p.ws_bytes = (size_t(nb) * size_t(E) * sizeof(int32_t) + 255) / 256 * 256;
  return p;
}

// The pairs [a, b) this wave handles inside chunk `bid`.
__device__ __forceinline__ void wave_range(int64_t P, int64_t chunk, int bid, int64_t& a,
                                           int64_t& b) {
  const int nwaves = blockDim.x / kWave;
  const int wid = threadIdx.x / kWave;
  const int64_t c0 = int64_t(bid) * chunk;
  const int64_t c1 = c0 + chunk < P ? c0 + chunk : P;
  int64_t per = (c1 - c0 + nwaves - 1) / nwaves;
  per = (per + kWave - 1) / kWave * kWave;
  a = c0 + wid * per;
  b = a + per < c1 ? a + per : c1;
}

__global__ __launch_bounds__(kSendThreads) void send_hist_kernel(const int32_t* __restrict__ idx,
                                                                 int64_t P, int E, int nbits,
                                                                 int64_t chunk,
                                                                 int32_t* __restrict__ ws_cnt) {
  extern __shared__ int32_t hist[];  // [E]
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  int64_t a, b;
  wave_range(P, chunk, blockIdx.x, a, b);
  for (int64_t s0 = a; s0 < b; s0 += kWave * kSendRankItems) {
    int ev[kSendRankItems];
#pragma unroll
    for (int u = 0; u < kSendRankItems; ++u) {
      const int64_t p = s0 + u * kWave + lane_id();
      ev[u] = p < b ? idx[p] : -1;
    }
#pragma unroll
    for (int u = 0; u < kSendRankItems; ++u) {
      if (s0 + u * kWave >= b) continue;  // wave-uniform: past the wave's range
      const int e = ev[u];
      const bool valid = uint32_t(e) < uint32_t(E);
      const uint64_t peers = same_expert_lanes(e, valid, nbits);
      if (valid && lanes_below(peers) == 0) atomicAdd(&hist[e], int32_t(__popcll(peers)));
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) ws_cnt[int64_t(blockIdx.x) * E + e] = hist[e];
}

// Stable slot of every pair.  Pass 1: inside each wave, lanes with the same
// expert are ranked by lane order (mbcnt over the matching-lane mask) on top
// of the wave's running count kept in LDS; the wave-local slot is parked in
// pair_row.  The expert offsets and this block's first slot in each expert
// come from the per-block histogram matrix (multi-block) or from the wave
// counts themselves (FUSED, one block).  Pass 2 adds the exclusive prefix
// over waves and the block base, and writes row_token.
// The rank step of block `bid` (0 for FUSED), run by a block of THREADS
// threads; sm: its dynamic LDS.  arrivals (multi-block only; nullptr: keep
// the matrix): each block counts in once its column sums of the histogram
// matrix are in LDS, and the last one clears the matrix and the counter for
// the next call.
template <bool FUSED, int THREADS, int ITEMS>
__device__ __forceinline__ void send_rank_block(
    int bid, int32_t* sm, const int32_t* __restrict__ idx, int64_t P, int E, int k, int nbits,
    int64_t chunk, int nb, int32_t* __restrict__ ws_cnt, uint32_t* __restrict__ arrivals, int L,
    int R, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ rank_offsets, int32_t* __restrict__ pair_row,
    int32_t* __restrict__ row_token) {
  // LDS: [W][E] per-wave counts | [E] base | [17] scan temporaries | [2][THREADS]
  // partial column sums (multi-block)
  constexpr int nwaves = THREADS / kWave;  // launched with THREADS threads (at most 16 waves)
  const int wid = threadIdx.x / kWave;
  int32_t* hist = sm;
  int32_t* base = sm + nwaves * E;
  int32_t* scan_tmp = base + E;
  int32_t* part = scan_tmp + 17;
  int64_t a, b;
  wave_range(P, chunk, bid, a, b);
  // The first step's expert indices are requested before the matrix loads
  // below, so the two memory round trips overlap.
  int ev0[ITEMS];
#pragma unroll
  for (int u = 0; u < ITEMS; ++u) {
    const int64_t p = a + u * kWave + lane_id();
    ev0[u] = p < b ? idx[p] : -1;
  }
  for (int i = threadIdx.x; i < nwaves * E; i += blockDim.x) hist[i] = 0;
  // Multi-block: each expert's total and this block's prefix (the blocks
  // before it), summed straight from the [block][expert] histogram matrix
  // (L2-resident) with one batch of independent loads per thread.  Up to
  // THREADS experts, G threads share a column, each summing every G-th row,
  // and their partial sums meet in LDS; above that (E <= 2 * THREADS) each
  // thread sums two columns.
  int32_t pre[2] = {0, 0};
  const bool shared_cols = E <= THREADS;
  if (!FUSED) {
    constexpr int kBatch = 32;
    const int G = shared_cols ? min(THREADS / E, nb) : 1;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int e = shared_cols ? int(threadIdx.x) % E : int(threadIdx.x) + q * THREADS;
      const int g = shared_cols ? int(threadIdx.x) / E : 0;
      if ((shared_cols && q > 0) || e >= E || g >= G) continue;
      int32_t tot = 0, before = 0;
      for (int r0 = g; r0 < nb; r0 += G * kBatch) {
        int32_t v[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int r = r0 + u * G;
          v[u] = r < nb ? ws_cnt[r * E + e] : 0;
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          tot += v[u];
          before += r0 + u * G < bid ? v[u] : 0;
        }
      }
      if (shared_cols) {
        part[threadIdx.x] = tot;
        part[THREADS + threadIdx.x] = before;
      } else {
        base[e] = tot;
        pre[q] = before;
      }
    }
  }
  __syncthreads();
  // Every thread's matrix loads have returned (their sums are in LDS), so
  // the block may count in; the result is first needed after pass 1.
  __shared__ int32_t clear_mat;
  uint32_t arrived_before = 0u;
  if (!FUSED && arrivals != nullptr && threadIdx.x == 0)
    arrived_before =
        __hip_atomic_fetch_add(arrivals, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (!FUSED && shared_cols && int(threadIdx.x) < E) {
    const int G = min(THREADS / E, nb);
    int32_t tot = 0, before = 0;
    for (int g = 0; g < G; ++g) {
      tot += part[g * E + threadIdx.x];
      before += part[THREADS + g * E + threadIdx.x];
    }
    base[threadIdx.x] = tot;
    pre[0] = before;
  }

  int32_t* my_hist = hist + wid * E;
  // A wave whose range fits in one step keeps experts and local slots in
  // registers for pass 2; longer ranges park the local slot in pair_row.
  const bool one_step = b - a <= int64_t(kWave) * ITEMS;
  int keep_e[ITEMS];
  int32_t keep_slot[ITEMS];
  for (int64_t s0 = a; s0 < b; s0 += kWave * ITEMS) {
    int ev[ITEMS];
#pragma unroll
    for (int u = 0; u < ITEMS; ++u) {
      const int64_t p = s0 + u * kWave + lane_id();
      ev[u] = s0 == a ? ev0[u] : (p < b ? idx[p] : -1);
    }
#pragma unroll
    for (int u = 0; u < ITEMS; ++u) {
      const int64_t p = s0 + u * kWave + lane_id();
      keep_e[u] = -1;
      keep_slot[u] = -1;
      if (s0 + u * kWave >= b) continue;  // wave-uniform: past the wave's range
      const int e = ev[u];
      const bool valid = uint32_t(e) < uint32_t(E);
      const uint64_t peers = same_expert_lanes(e, valid, nbits);
      int32_t slot = -1;  // -1: expert index out of range, the pair is dropped
      if (valid) {
        const uint32_t below = lanes_below(peers);
        const int32_t cur = my_hist[e];
        slot = cur + int32_t(below);
        if (below == 0) my_hist[e] = cur + int32_t(__popcll(peers));
      }
      keep_e[u] = e;
      keep_slot[u] = slot;
      if (!one_step && p < b) pair_row[p] = slot;
    }
  }
  if (!FUSED && threadIdx.x == 0)
    clear_mat = arrivals != nullptr && arrived_before == uint32_t(nb - 1);
  __syncthreads();

  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int32_t c[nwaves];
#pragma unroll
    for (int w = 0; w < nwaves; ++w) c[w] = hist[w * E + e];
    int32_t run = 0;
#pragma unroll
    for (int w = 0; w < nwaves; ++w) {
      hist[w * E + e] = run;
      run += c[w];
    }
    if (FUSED) base[e] = run;
  }
  __syncthreads();
  // base[e]: total pairs of expert e -> exclusive offsets.
  const int32_t total = block_excl_scan(base, E, scan_tmp);
  if (FUSED || bid == 0) {
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
      offsets[e] = base[e];
      counts[e] = (e + 1 < E ? base[e + 1] : total) - base[e];
    }
    if (threadIdx.x == 0) offsets[E] = total;
    if (rank_offsets != nullptr) {
      for (int r = threadIdx.x; r < R; r += blockDim.x) rank_offsets[r] = base[r * L];
      if (threadIdx.x == 0) rank_offsets[R] = total;
    }
  }
  __syncthreads();
  if (!FUSED) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int e = threadIdx.x + q * THREADS;
      if (e < E) base[e] += pre[q];
    }
    __syncthreads();
  }

  for (int64_t s0 = a; s0 < b; s0 += kWave * ITEMS) {
    if (!one_step) {
#pragma unroll
      for (int u = 0; u < ITEMS; ++u) {
        const int64_t p = s0 + u * kWave + lane_id();
        keep_e[u] = p < b ? idx[p] : -1;
        keep_slot[u] = p < b ? pair_row[p] : -1;
      }
    }
#pragma unroll
    for (int u = 0; u < ITEMS; ++u) {
      const int64_t p = s0 + u * kWave + lane_id();
      if (p < b) {
        const int e = keep_e[u];
        int32_t r = -1;
        if (uint32_t(e) < uint32_t(E)) {
          r = base[e] + my_hist[e] + keep_slot[u];
          // Always below P with a clean histogram matrix; a matrix left
          // dirty (a workspace not zeroed as documented) drops the pair
          // instead of storing out of bounds.
          if (uint64_t(uint32_t(r)) < uint64_t(P))
            row_token[r] = int32_t(p) / k;
          else
            r = -1;
        }
        pair_row[p] = r;
      }
    }
  }
  if (!FUSED && clear_mat) {  // every block has read the matrix: zero it for the next call
    for (int i = threadIdx.x; i < nb * E; i += THREADS) ws_cnt[i] = 0;
    if (threadIdx.x == 0) __hip_atomic_store(arrivals, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <bool FUSED, int THREADS, int ITEMS>
__global__ __launch_bounds__(THREADS) void send_rank_kernel(
    const int32_t* __restrict__ idx, int64_t P, int E, int k, int nbits, int64_t chunk, int nb,
    int32_t* __restrict__ ws_cnt, uint32_t* __restrict__ arrivals, int L, int R,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ rank_offsets, int32_t* __restrict__ pair_row,
    int32_t* __restrict__ row_token) {
  extern __shared__ int32_t sm[];
  send_rank_block<FUSED, THREADS, ITEMS>(blockIdx.x, sm, idx, P, E, k, nbits, chunk, nb, ws_cnt,
                                         arrivals, L, R, counts, offsets, rank_offsets, pair_row,
                                         row_token);
}

// ---------------------------------------------------------------------------
// route + send in one launch for small batches
// ---------------------------------------------------------------------------

// Every block routes THREADS / 64 tokens, one wave each, then counts itself
// in on `arrivals` after a device-scope fence.  The block that arrives last
// sees every token's routing and runs the single-block send; it then resets
// the counter for the next call on the stream.  No block ever waits for
// another, so the grid drains whatever the residency.
template <int IPL, int THREADS, bool GROUPED>
__global__ __launch_bounds__(THREADS) void route_send_kernel(
    const float* __restrict__ logits, int64_t T, int E, int k, int n_group, int topk_group,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, uint32_t* __restrict__ arrivals,
    int nbits, int L, int R, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ rank_offsets, int32_t* __restrict__ pair_row,
    int32_t* __restrict__ row_token) {
  extern __shared__ int32_t sm[];
  __shared__ int32_t is_last;
  const int64_t t = int64_t(blockIdx.x) * (THREADS / kWave) + threadIdx.x / kWave;
  if (t < T)
    route_wave_token<IPL, GROUPED, false>(logits, t, E, k, n_group, topk_group, topk_idx, topk_w,
                                          nullptr, 1u);
  // Release the block's routing at device scope before it counts in.  Each
  // wave waits until its own stores have reached the L2 (vmcnt 0); after the
  // barrier, thread 0's agent-scope release writes the L2 back, which then
  // covers every wave's stores.  The last block to arrive acquires, so it
  // sees every block's routing.  (One write-back per block: a release in
  // every wave cost 1.5 us at DSv3 decode, and a full fence would write the
  // L2 back once more.)
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const uint32_t before =
        __hip_atomic_fetch_add(arrivals, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    is_last = before == gridDim.x - 1;
    if (is_last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
  if (!is_last) return;  // the whole block leaves
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  const int64_t P = T * k;
  send_rank_block<true, THREADS, kSendItems>(0, sm, topk_idx, P, E, k, nbits, P, 1, nullptr,
                                             nullptr, L, R, counts, offsets, rank_offsets,
                                             pair_row, row_token);
  if (threadIdx.x == 0)  // every block has counted in: ready for the next call on the stream
    __hip_atomic_store(arrivals, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// dispatch recv and combine: one block per (token, 1 KiB slice of the row)
// ---------------------------------------------------------------------------

constexpr int kSlice = 64;             // 16-byte chunks per slice: one per lane
constexpr int kMaxRowThreads = 1024;
constexpr int64_t kMaxRowBlocks = int64_t(1) << 21;  // beyond this, blocks loop

// Slices of a row one recv wave copies per unit: it issues all their loads
// before its stores, so each block keeps kRecvSlices KiB of x in flight.
// Two slices hide the latency of x when it comes from HBM (a cold cache) at
// no cost when it is cache-resident and the routing spreads over the
// experts; four are slower either way.  The measurement variants of the
// other counts are built from this same source with MOE_RECV_SLICES.
#ifndef MOE_RECV_SLICES
#define MOE_RECV_SLICES 2
#endif
constexpr int kRecvSlices = MOE_RECV_SLICES;
static_assert(kRecvSlices >= 1 && kRecvSlices <= 8, "slices per recv wave");

// The recv kernel's stores: global stores with the non-temporal hint.  A
// buffer written once and read by a later kernel gains nothing from being
// kept in the L2 or the Infinity Cache, and write-back stores there cost
// more than they save when x is cache-resident.  For measurement,
// MOE_RECV_STORE = 0..31 builds the kernel with buffer stores carrying that
// cache-policy word instead (sc0 = 1, nt = 2, sc1 = 16); such a build takes
// buffers of at most 4 GiB.
#ifndef MOE_RECV_STORE
#define MOE_RECV_STORE -1
#endif
constexpr int kRecvStore = MOE_RECV_STORE;
static_assert(kRecvStore >= -1 && kRecvStore <= 31, "recv store form");

// Store v as 16-byte chunk i of buf (nbytes: the buffer's size in bytes,
// used only by the measurement forms).
__device__ __forceinline__ void recv_store(const u32x4 v, u32x4* __restrict__ buf, int64_t i,
                                           uint32_t nbytes) {
  if constexpr (kRecvStore < 0) {
    __builtin_nontemporal_store(v, &buf[i]);
  } else {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(buf, 0, nbytes, 0x00020000);
    __builtin_amdgcn_raw_buffer_store_b128(v, rs, uint32_t(i) * 16u, 0, kRecvStore);
  }
}

struct RecvPlan {
  int groups;  // waves per block; wave g writes destinations g*per .. g*per+per-1
  int per;
  int nsb;     // units (kRecvSlices slices each) per row
  int64_t units;
  unsigned nblocks;
};

RecvPlan plan_recv(int64_t T, int C, int k) {
  RecvPlan p{};
  p.groups = k < kMaxRowThreads / kSlice ? k : kMaxRowThreads / kSlice;
  p.per = (k + p.groups - 1) / p.groups;
  const int ncs = (C + kSlice - 1) / kSlice;
  p.nsb = (ncs + kRecvSlices - 1) / kRecvSlices;
  p.units = T * p.nsb;
  p.nblocks = unsigned(p.units < kMaxRowBlocks ? p.units : kMaxRowBlocks);
  return p;
}

// Destinations per recv wave: k <= 32 over at most 16 waves.
constexpr int kRecvMaxPer = kMaxK / (kMaxRowThreads / kSlice);

template <int U>
__global__ __launch_bounds__(kMaxRowThreads) void dispatch_recv_kernel(
    const u32x4* __restrict__ x, const int32_t* __restrict__ pair_row, int64_t T, int C, int k,
    int per, int nsb, int64_t units, u32x4* __restrict__ buf, int64_t capacity) {
  const int g = __builtin_amdgcn_readfirstlane(threadIdx.x / kSlice);
  const uint32_t nbytes = kRecvStore < 0 ? 0u : uint32_t(capacity * C * 16);
  for (int64_t unit = blockIdx.x; unit < units; unit += gridDim.x) {
    const int64_t t = unit / nsb;
    const int c0 = int(unit - t * nsb) * (U * kSlice) + lane_id();
    // Cached loads: the block's waves read the same slices.  Every v[u] is
    // assigned in every unit, so no value lives across units and nothing
    // makes the second load wait for the first.
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + u * kSlice;
      v[u] = c < C ? x[t * C + c] : u32x4{0u, 0u, 0u, 0u};
    }
    // The wave's destination rows (uniform: scalar loads), loaded without a
    // branch (the index is clamped into the token's k entries, and unused
    // ones are dropped afterwards) so that they are in flight together with
    // the row loads.
    int32_t r[kRecvMaxPer];
#pragma unroll
    for (int jj = 0; jj < kRecvMaxPer; ++jj) {
      const int j = g * per + jj;
      const int32_t v_r = pair_row[t * k + (j < k ? j : k - 1)];
      r[jj] = jj < per && j < k ? v_r : -1;
    }
#pragma unroll
    for (int jj = 0; jj < kRecvMaxPer; ++jj) {
      if (uint64_t(int64_t(r[jj])) < uint64_t(capacity)) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = c0 + u * kSlice;
          if (c < C) recv_store(v[u], buf, int64_t(r[jj]) * C + c, nbytes);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// send and recv in one launch for small batches
// ---------------------------------------------------------------------------

constexpr int64_t kSendRecvMaxPairs = int64_t(kSendWaves) * kWave * kSendItems;  // one 8-wave step
constexpr int kSendRecvMaxK = kSendWaves;  // one wave per destination row
constexpr int kSendRecvSlices = 8;         // 1 KiB slices of a row per copy unit

// The row of pair (t, j) with expert e is the number of pairs with a lower
// expert (e's offset) plus the number of earlier pairs with expert e (its
// slot in the stable order).  A block that needs the rows of one token's
// k <= 8 pairs before the send has written them counts both over topk_idx
// with ballots, so the counts are wave-uniform and need no reduction inside
// a wave.  Each wave counts its share of the pairs into part[wid]; after a
// block barrier, token_rows_finish sums the waves' counts into rows[j]
// (-1 for an invalid expert, which the send drops).
__device__ __forceinline__ void token_rows_count(const int32_t* __restrict__ idx, int64_t P,
                                                 int64_t pt, int k, int wid, int lane,
                                                 uint32_t (*part)[2 * kSendRecvMaxK]) {
  int ej[kSendRecvMaxK];
#pragma unroll
  for (int j = 0; j < kSendRecvMaxK; ++j) ej[j] = j < k ? idx[pt + j] : -1;
  uint32_t lt[kSendRecvMaxK], eq[kSendRecvMaxK];
#pragma unroll
  for (int j = 0; j < kSendRecvMaxK; ++j) lt[j] = eq[j] = 0u;
  for (int64_t p0 = int64_t(wid) * kWave; p0 < P; p0 += kSendThreads) {  // wave-uniform bounds
    const int64_t p = p0 + lane;
    const bool in = p < P;
    const int v = in ? idx[p] : -1;
#pragma unroll
    for (int j = 0; j < kSendRecvMaxK; ++j) {
      if (j < k) {
        lt[j] += __popcll(ballot(in && uint32_t(v) < uint32_t(ej[j])));
        eq[j] += __popcll(ballot(in && v == ej[j] && p < pt + j));
      }
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int j = 0; j < kSendRecvMaxK; ++j) {
      part[wid][j] = lt[j];
      part[wid][kSendRecvMaxK + j] = eq[j];
    }
  }
}

__device__ __forceinline__ void token_rows_finish(const int32_t* __restrict__ idx, int64_t pt,
                                                  int E, int k,
                                                  const uint32_t (*part)[2 * kSendRecvMaxK],
                                                  int32_t* rows) {
  if (int(threadIdx.x) < k) {
    const int j = threadIdx.x;
    const int e = idx[pt + j];
    uint32_t r = 0u;
#pragma unroll
    for (int w = 0; w < kSendWaves; ++w) r += part[w][j] + part[w][kSendRecvMaxK + j];
    rows[j] = uint32_t(e) < uint32_t(E) ? int32_t(r) : -1;
  }
}

// Block 0 runs the single-block send.  Every other block copies up to 8
// slices of one token's row to the token's k rows, which it finds itself
// (token_rows_count / token_rows_finish), so the copies never wait for the
// send, which runs beside them.  Wave w copies to destination w (k <= 8).
__global__ __launch_bounds__(kSendThreads) void send_recv_kernel(
    const int32_t* __restrict__ idx, int64_t T, int E, int k, int nbits, int L, int R,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ rank_offsets, int32_t* __restrict__ pair_row,
    int32_t* __restrict__ row_token, const u32x4* __restrict__ x, int C, int nparts,
    int64_t units, u32x4* __restrict__ buf, int64_t capacity) {
  extern __shared__ int32_t sm[];
  const int64_t P = T * k;
  if (blockIdx.x == 0) {
    send_rank_block<true, kSendThreads, kSendItems>(0, sm, idx, P, E, k, nbits, P, 1, nullptr,
                                                    nullptr, L, R, counts, offsets, rank_offsets,
                                                    pair_row, row_token);
    return;
  }
  __shared__ uint32_t part[kSendWaves][2 * kSendRecvMaxK];  // per-wave counts
  __shared__ int32_t rows[kSendRecvMaxK];
  const int lane = lane_id();
  const int wid = threadIdx.x / kWave;
  for (int64_t unit = blockIdx.x - 1; unit < units; unit += gridDim.x - 1) {
    const int64_t t = unit / nparts;
    const int sp = int(unit - t * nparts);
    const int64_t pt = t * k;  // flat index of the token's first pair
    // The token's slices do not depend on the routing: their loads go out
    // first and arrive while the block counts its rows.
    u32x4 v[kSendRecvSlices];
#pragma unroll
    for (int s = 0; s < kSendRecvSlices; ++s) {
      const int c = (sp * kSendRecvSlices + s) * kSlice + lane;
      v[s] = wid < k && c < C ? x[t * C + c] : u32x4{0u, 0u, 0u, 0u};
    }
    token_rows_count(idx, P, pt, k, wid, lane, part);
    __syncthreads();
    token_rows_finish(idx, pt, E, k, part, rows);
    __syncthreads();
    if (wid < k) {
      const int32_t r = rows[wid];
      if (uint64_t(int64_t(r)) < uint64_t(capacity)) {
#pragma unroll
        for (int s = 0; s < kSendRecvSlices; ++s) {
          const int c = (sp * kSendRecvSlices + s) * kSlice + lane;
          if (c < C) __builtin_nontemporal_store(v[s], &buf[int64_t(r) * C + c]);
        }
      }
    }
    __syncthreads();  // part and rows are reused by the next unit
  }
}

// ---------------------------------------------------------------------------
// fp8 dispatch recv: block-scaled OCP E4M3 payloads
// ---------------------------------------------------------------------------

constexpr int kQuantBlock = 128;         // elements per scale
constexpr float kE4M3Max = 448.0f;       // largest finite E4M3 value
constexpr int kFp8Waves = 8;             // slices quantised per block
constexpr int kFp8SliceElems = kSlice * 8;
constexpr int kFp8BlockElems = kFp8Waves * kFp8SliceElems;  // 4096 elements per block

// Nearest E4M3 (4 exponent bits, bias 7, 3 mantissa bits, no infinities)
// code of a finite fp32, ties to the even code, saturating at +-448.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  uint32_t code;
  if (a >= 0x43E00000u) {         // |v| >= 448: saturate (NaN stays NaN)
    code = a > 0x7F800000u ? 0x7Fu : 0x7Eu;
  } else if (a >= 0x3C800000u) {  // |v| >= 2^-6: normal; round the mantissa at bit 20
    code = ((a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20) - (120u << 3);
  } else {                        // subnormal E4M3: multiples of 2^-9 (scaling is exact)
    code = uint32_t(__builtin_rintf(__uint_as_float(a) * 512.0f));
  }
  return sign | code;
}

// Maximum over the 16 lanes of each DPP row (every lane gets its row's value).
__device__ __forceinline__ uint32_t row16_max_u32(uint32_t v) {
  v = max(v, dpp<kDppQuad1032, 0xF>(0u, v));
  v = max(v, dpp<kDppQuad2301, 0xF>(0u, v));
  v = max(v, dpp<kDppRowHalfMirror, 0xF>(0u, v));
  v = max(v, dpp<kDppRowMirror, 0xF>(0u, v));
  return v;
}

// Wave w of a unit quantises slice w of the unit's 4096 elements (512
// elements, one 16-byte bf16 chunk per lane: 4 scale blocks of 16 lanes)
// into the unit's LDS tiles: codes at element offset 512 w, scales at 4 w.
// Dead chunks (past the row) come in as zeros and are never stored.
__device__ __forceinline__ void quantise_slice(const u32x4 v, int w, int lane,
                                               u32x4* __restrict__ q_lds,
                                               float* __restrict__ s_lds) {
  float f[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    f[2 * q] = __uint_as_float(v[q] << 16);
    f[2 * q + 1] = __uint_as_float(v[q] & 0xFFFF0000u);
  }
  uint32_t amax_bits = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax_bits = max(amax_bits, __float_as_uint(f[i]) & 0x7FFFFFFFu);
  amax_bits = row16_max_u32(amax_bits);
  const float amax = __uint_as_float(amax_bits);
  const float scale = amax > 0.f ? amax / kE4M3Max : 1.0f;
  uint32_t lo = 0u, hi = 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) lo |= e4m3_code(f[i] / scale) << (8 * i);
#pragma unroll
  for (int i = 0; i < 4; ++i) hi |= e4m3_code(f[4 + i] / scale) << (8 * i);
  reinterpret_cast<uint2*>(q_lds)[w * kWave + lane] = make_uint2(lo, hi);
  if ((lane & 15) == 0) s_lds[w * 4 + lane / 16] = scale;
}

// One wave stores a unit's codes and scales (from the LDS tiles) to
// destination row r: elements [e0, e0 + 4096) of the row, cut at H.
__device__ __forceinline__ void store_fp8_unit(const u32x4* __restrict__ q_lds,
                                               const float* __restrict__ s_lds, int32_t r,
                                               int e0, int H, int lane,
                                               uint8_t* __restrict__ buf_q,
                                               float* __restrict__ buf_s) {
  const int nbytes = H - e0 < kFp8BlockElems ? H - e0 : kFp8BlockElems;
  const int nunits = nbytes / 16;
  const int ns = nbytes / kQuantBlock;
  u32x4* dq = reinterpret_cast<u32x4*>(buf_q + int64_t(r) * H + e0);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int unit16 = u * kWave + lane;
    if (unit16 < nunits) __builtin_nontemporal_store(q_lds[unit16], &dq[unit16]);
  }
  if (lane < ns) buf_s[int64_t(r) * (H / kQuantBlock) + e0 / kQuantBlock + lane] = s_lds[lane];
}

__global__ __launch_bounds__(kFp8Waves* kWave) void dispatch_recv_fp8_kernel(
    const u32x4* __restrict__ x, const int32_t* __restrict__ pair_row, int64_t T, int C, int H,
    int k, int nsb, int64_t units, uint8_t* __restrict__ buf_q, float* __restrict__ buf_s,
    int64_t capacity) {
  __shared__ u32x4 q_lds[kFp8BlockElems / 16];         // 4 KiB of codes
  __shared__ float s_lds[kFp8BlockElems / kQuantBlock];  // 32 scales
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = lane_id();
  for (int64_t unit = blockIdx.x; unit < units; unit += gridDim.x) {
    const int64_t t = unit / nsb;
    const int sb = int(unit - t * nsb);
    // Phase 1: wave w quantises slice sb*8 + w (whole 16-lane scale blocks
    // are live or not, since H % 128 == 0).
    const int c = (sb * kFp8Waves + w) * kSlice + lane;  // 16-byte chunk of the bf16 row
    const u32x4 v = c < C ? x[t * C + c] : u32x4{0u, 0u, 0u, 0u};
    quantise_slice(v, w, lane, q_lds, s_lds);
    __syncthreads();
    // Phase 2: wave w writes the unit to destinations w, w + 8, ... of token t.
    for (int j = w; j < k; j += kFp8Waves) {
      const int32_t r = pair_row[t * k + j];
      if (uint64_t(int64_t(r)) < uint64_t(capacity))
        store_fp8_unit(q_lds, s_lds, r, sb * kFp8BlockElems, H, lane, buf_q, buf_s);
    }
    __syncthreads();  // the LDS tiles are reused by the next unit
  }
}

// Send + fp8 recv in one launch for small batches, as send_recv_kernel: block
// 0 runs the single-block send; every other block quantises one 4096-element
// unit of a token's row (wave w: slice w) while it counts the token's rows,
// then wave w stores the unit to destination w (k <= 8).
static_assert(kFp8Waves == kSendWaves, "one quantising wave per send wave");
__global__ __launch_bounds__(kSendThreads) void send_recv_fp8_kernel(
    const int32_t* __restrict__ idx, int64_t T, int E, int k, int nbits, int L, int R,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ rank_offsets, int32_t* __restrict__ pair_row,
    int32_t* __restrict__ row_token, const u32x4* __restrict__ x, int C, int H, int nsb,
    int64_t units, uint8_t* __restrict__ buf_q, float* __restrict__ buf_s, int64_t capacity) {
  extern __shared__ int32_t sm[];
  const int64_t P = T * k;
  if (blockIdx.x == 0) {
    send_rank_block<true, kSendThreads, kSendItems>(0, sm, idx, P, E, k, nbits, P, 1, nullptr,
                                                    nullptr, L, R, counts, offsets, rank_offsets,
                                                    pair_row, row_token);
    return;
  }
  __shared__ uint32_t part[kSendWaves][2 * kSendRecvMaxK];
  __shared__ int32_t rows[kSendRecvMaxK];
  __shared__ u32x4 q_lds[kFp8BlockElems / 16];
  __shared__ float s_lds[kFp8BlockElems / kQuantBlock];
  const int lane = lane_id();
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  for (int64_t unit = blockIdx.x - 1; unit < units; unit += gridDim.x - 1) {
    const int64_t t = unit / nsb;
    const int sb = int(unit - t * nsb);
    const int64_t pt = t * k;
    const int c = (sb * kFp8Waves + wid) * kSlice + lane;
    const u32x4 v = c < C ? x[t * C + c] : u32x4{0u, 0u, 0u, 0u};  // in flight while counting
    token_rows_count(idx, P, pt, k, wid, lane, part);
    quantise_slice(v, wid, lane, q_lds, s_lds);
    __syncthreads();
    token_rows_finish(idx, pt, E, k, part, rows);
    __syncthreads();
    if (wid < k) {
      const int32_t r = rows[wid];
      if (uint64_t(int64_t(r)) < uint64_t(capacity))
        store_fp8_unit(q_lds, s_lds, r, sb * kFp8BlockElems, H, lane, buf_q, buf_s);
    }
    __syncthreads();  // part, rows and the LDS tiles are reused by the next unit
  }
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 f = {lo, hi};
  const bf16x2 h = __builtin_convertvector(f, bf16x2);  // round-to-nearest-even
  return __builtin_bit_cast(uint32_t, h);
}

// Store o as 16-byte chunk c of row t of out (C chunks per row).  SC1: with
// the device-scope cache policy (sc1) instead of the default write-back.
// When combine streams its expert rows from HBM, its output writes cost far
// more than their own bytes under write-back, and sc1 makes the kernel 3-4 %
// faster; when everything fits in the Infinity Cache, write-back keeps the
// output there and sc1 is 5-9 % slower.  moe_combine picks by size.  A buffer
// store addresses 4 GiB, so the resource covers one row (at most 2 MiB); t
// is wave-uniform, so the resource stays in SGPRs.
constexpr int kCpolSc1 = 16;
template <bool SC1>
__device__ __forceinline__ void store_out_row(const u32x4 o, u32x4* __restrict__ out, int64_t t,
                                              int C, int c) {
  if constexpr (SC1) {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(out + t * C, 0, uint32_t(C) * 16u, 0x00020000);
    __builtin_amdgcn_raw_buffer_store_b128(o, rs, uint32_t(c) * 16u, 0, kCpolSc1);
  } else {
    out[t * C + c] = o;
  }
}

// Combine's bytes above which its output rows are stored with sc1: the
// 256 MiB Infinity Cache.  For measurement, MOE_COMBINE_SC1_MIN_BYTES = 0
// builds sc1 at every size and INT64_MAX write-back at every size.
#ifndef MOE_COMBINE_SC1_MIN_BYTES
#define MOE_COMBINE_SC1_MIN_BYTES (int64_t(256) << 20)
#endif
constexpr int64_t kCombineSc1MinBytes = MOE_COMBINE_SC1_MIN_BYTES;

constexpr int kCombineGroup = 8;  // expert rows loaded before their fma

template <bool SC1>
__global__ __launch_bounds__(kSlice) void combine_kernel(
    const u32x4* __restrict__ y, const int32_t* __restrict__ pair_row,
    const float* __restrict__ topk_w, int64_t T, int C, int k, int ncs, int64_t units,
    int64_t capacity, u32x4* __restrict__ out) {
  for (int64_t unit = blockIdx.x; unit < units; unit += gridDim.x) {
    const int64_t t = unit / ncs;
    const int c = int(unit - t * ncs) * kSlice + lane_id();
    if (c >= C) continue;
    const int32_t* prt = pair_row + t * k;  // uniform: scalar loads into SGPRs
    const float* wt = topk_w + t * k;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    for (int j0 = 0; j0 < k; j0 += kCombineGroup) {
      u32x4 v[kCombineGroup];
#pragma unroll
      for (int g = 0; g < kCombineGroup; ++g) {
        v[g] = u32x4{0u, 0u, 0u, 0u};
        if (j0 + g < k) {
          const int32_t r = prt[j0 + g];
          if (uint64_t(int64_t(r)) < uint64_t(capacity))
            v[g] = __builtin_nontemporal_load(&y[int64_t(r) * C + c]);
        }
      }
#pragma unroll
      for (int g = 0; g < kCombineGroup; ++g) {
        if (j0 + g < k) {
          const int32_t r = prt[j0 + g];
          if (uint64_t(int64_t(r)) < uint64_t(capacity)) {
            const float wj = wt[j0 + g];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const uint32_t word = v[g][q];
              acc[2 * q] = __builtin_fmaf(wj, __uint_as_float(word << 16), acc[2 * q]);
              acc[2 * q + 1] =
                  __builtin_fmaf(wj, __uint_as_float(word & 0xFFFF0000u), acc[2 * q + 1]);
            }
          }
        }
      }
    }
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
    store_out_row<SC1>(o, out, t, C, c);
  }
}

// Fixed k (1, 2, 4, 8): the token's k rows and weights are loaded first
// (wave-uniform, scalar), then all U * K row loads go out back to back.  For
// k < 8 one wave covers U slices of a token, so that 16 row loads are in
// flight per lane; otherwise a k = 2 wave would move only 3 KiB and the
// launch, not the memory system, would set the pace.  k = 8 takes one slice
// (U = 1, 8 loads in flight).
template <int K, int U, bool SC1>
__global__ __launch_bounds__(kSlice) void combine_small_k_kernel(
    const u32x4* __restrict__ y, const int32_t* __restrict__ pair_row,
    const float* __restrict__ topk_w, int64_t T, int C, int nsb, int64_t units, int64_t capacity,
    u32x4* __restrict__ out) {
  for (int64_t unit = blockIdx.x; unit < units; unit += gridDim.x) {
    const int64_t t = unit / nsb;
    const int sb = int(unit - t * nsb);
    int32_t r[K];
    float wj[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
      r[j] = pair_row[t * K + j];
      wj[j] = topk_w[t * K + j];
    }
    u32x4 v[U][K];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = (sb * U + u) * kSlice + lane_id();
#pragma unroll
      for (int j = 0; j < K; ++j)
        v[u][j] = (c < C && uint64_t(int64_t(r[j])) < uint64_t(capacity))
                      ? __builtin_nontemporal_load(&y[int64_t(r[j]) * C + c])
                      : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = (sb * U + u) * kSlice + lane_id();
      if (c >= C) continue;
      float acc[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = 0.f;
#pragma unroll
      for (int j = 0; j < K; ++j) {
        if (uint64_t(int64_t(r[j])) >= uint64_t(capacity)) continue;  // skipped term
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t word = v[u][j][q];
          acc[2 * q] = __builtin_fmaf(wj[j], __uint_as_float(word << 16), acc[2 * q]);
          acc[2 * q + 1] = __builtin_fmaf(wj[j], __uint_as_float(word & 0xFFFF0000u), acc[2 * q + 1]);
        }
      }
      u32x4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
      store_out_row<SC1>(o, out, t, C, c);
    }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

template <typename Tuple, size_t... I>
void arg_ptrs(Tuple& t, void** argv, std::index_sequence<I...>) {
  ((argv[I] = static_cast<void*>(&std::get<I>(t))), ...);
}

template <typename... KArgs, typename... Args>
int launch(void (*kern)(KArgs...), dim3 grid, dim3 block, size_t lds, hipStream_t st,
           Args... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel arity");
  // The dispatch packet holds the grid as 32-bit work-item counts; every
  // plan caps its grid well below that, and this keeps it so.
  if (uint64_t(grid.x) * block.x > 0xFFFFFFFFull) return MOE_ERR_INVALID_ARG;
  std::tuple<KArgs...> packed(static_cast<KArgs>(args)...);
  void* argv[sizeof...(KArgs)];
  arg_ptrs(packed, argv, std::index_sequence_for<KArgs...>{});
  const hipError_t e =
      hipLaunchKernel(reinterpret_cast<const void*>(kern), grid, block, argv, lds, st);
  return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_route_shape(int64_t T, int32_t E, int32_t k) {
  if (T < 0 || E < 1 || E > kMaxE || k < 1 || k > kMaxK || k > E) return MOE_ERR_INVALID_ARG;
  if (T > kMaxPairs / k) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

// Lanes per token (G) and experts per lane (IPL) of the lane-group routing
// kernel (batches above kRouteWaveMaxTokens).  The fewest lanes per token do
// the least work (wave-wide steps are shared by more tokens), but a lane's
// dependent chain grows with its IPL experts: up to 128 experts 16 lanes per
// token; above that the fewest lanes that still give the chip at least 4096
// waves (16 per CU).  At least 32 lanes for k > 16 (lane g < k of a token
// reports winner g), and IPL <= 24.
struct RoutePlan {
  int G;
  int IPL;
};

int route_gmin(int E, int k) {
  int gmin = E <= 384 ? 16 : (E <= 768 ? 32 : 64);
  if (k > 16 && gmin < 32) gmin = 32;
  return gmin;
}

int route_ipl(int E, int G) {  // the smallest instantiated items per lane that cover E
  const int need = (E + G - 1) / G;
  const int sizes[] = {1, 2, 4, 8, 16, 24};
  for (int v : sizes)
    if (v >= need) return v;
  return 24;
}

RoutePlan plan_route(int64_t T, int E, int k) {
  RoutePlan p{};
  p.G = route_gmin(E, k);
  if (E > 128)
    while (p.G < kWave && T * p.G / kWave < 4096) p.G *= 2;
  p.IPL = route_ipl(E, p.G);
  return p;
}

// Group-limited routing in the lane-group kernel needs every group to be
// 2^lg whole lanes (lg <= 4) and 16-byte logit loads.  Of the lanes per
// token allowed for (E, k), the plain plan's choice is tried first, then the
// others, nearest first.  False: no plan fits; the wave kernel routes.
bool plan_route_grouped(int64_t T, int E, int k, int n_group, const float* logits, RoutePlan& p,
                        int& lg) {
  if (E % 4 != 0 || !aligned(logits, 16)) return false;
  const int gs = E / n_group;
  const RoutePlan base = plan_route(T, E, k);
  const int tries[3] = {base.G, base.G == 32 ? 16 : 32, base.G == 64 ? 16 : 64};
  for (int G : tries) {
    if (G < route_gmin(E, k)) continue;
    const int ipl = route_ipl(E, G);
    if (ipl % 4 != 0 || ipl * G < E || gs % ipl != 0) continue;
    const int lanes = gs / ipl;
    if (lanes > 16 || (lanes & (lanes - 1)) != 0) continue;
    p.G = G;
    p.IPL = ipl;
    lg = __builtin_ctz(unsigned(lanes));
    return true;
  }
  return false;
}

// hist_mat: nullptr, or the zero-initialised [blocks][E] send histogram
// matrix with `chunk` pairs per row, which the routing kernels then fill.
int enqueue_route(const float* logits, int64_t T, int32_t E, int32_t k, int32_t n_group,
                  int32_t topk_group, int32_t* topk_idx, float* topk_w, hipStream_t s,
                  int32_t* hist_mat = nullptr, int64_t chunk = 1) {
  const dim3 block(kRouteThreads);
  const bool grouped = topk_group < n_group;  // keeping every group is plain top-k
  const bool count = hist_mat != nullptr;
  const uint32_t ch = uint32_t(chunk);
  RoutePlan gp{};
  int lg = 0;
  if (grouped && T > kRouteWaveMaxTokens &&
      plan_route_grouped(T, E, k, n_group, logits, gp, lg)) {
    const int64_t tokens_per_block = int64_t(kRouteWavesPerBlock) * (kWave / gp.G);
    const int64_t nb = (T + tokens_per_block - 1) / tokens_per_block;
    const dim3 grid(unsigned(nb < kRouteMaxBlocks ? nb : kRouteMaxBlocks));
#define MOE_GROUTE(G_, IPL_)                                                                    \
  if (gp.G == G_ && gp.IPL == IPL_)                                                             \
    return count ? launch(route_topk_kernel<G_, IPL_, true, true, true>, grid, block, 0, s,     \
                          logits, T, E, k, topk_group, lg, topk_idx, topk_w, hist_mat, ch)      \
                 : launch(route_topk_kernel<G_, IPL_, true, false, true>, grid, block, 0, s,    \
                          logits, T, E, k, topk_group, lg, topk_idx, topk_w, hist_mat, ch);
    MOE_GROUTE(16, 4);
    MOE_GROUTE(16, 8);
    MOE_GROUTE(16, 16);
    MOE_GROUTE(16, 24);
    MOE_GROUTE(32, 4);
    MOE_GROUTE(32, 8);
    MOE_GROUTE(32, 16);
    MOE_GROUTE(32, 24);
    MOE_GROUTE(64, 4);
    MOE_GROUTE(64, 8);
    MOE_GROUTE(64, 16);
#undef MOE_GROUTE
  }
  if (grouped || T <= kRouteWaveMaxTokens) {
    const int64_t nb = (T + kRouteWavesPerBlock - 1) / kRouteWavesPerBlock;
    const dim3 grid(unsigned(nb < kRouteMaxBlocks ? nb : kRouteMaxBlocks));
    const int ipl = (E + kWave - 1) / kWave;
    const int ng = grouped ? n_group : 1, tg = grouped ? topk_group : 1;
#define MOE_ROUTE_GC(IPL_, GR_)                                                              \
  return count ? launch(route_wave_kernel<IPL_, GR_, true>, grid, block, 0, s, logits, T, E, k, \
                        ng, tg, topk_idx, topk_w, hist_mat, ch)                                \
               : launch(route_wave_kernel<IPL_, GR_, false>, grid, block, 0, s, logits, T, E, \
                        k, ng, tg, topk_idx, topk_w, hist_mat, ch)
#define MOE_ROUTE(IPL_)            \
  {                                \
    if (grouped) MOE_ROUTE_GC(IPL_, true); \
    MOE_ROUTE_GC(IPL_, false);     \
  }
    if (ipl <= 1) MOE_ROUTE(1);
    if (ipl <= 2) MOE_ROUTE(2);
    if (ipl <= 4) MOE_ROUTE(4);
    if (ipl <= 8) MOE_ROUTE(8);
    MOE_ROUTE(16);
#undef MOE_ROUTE
#undef MOE_ROUTE_GC
  }
  const RoutePlan p = plan_route(T, E, k);
  const int64_t tokens_per_block = int64_t(kRouteWavesPerBlock) * (kWave / p.G);
  const int64_t nb = (T + tokens_per_block - 1) / tokens_per_block;
  const dim3 grid(unsigned(nb < kRouteMaxBlocks ? nb : kRouteMaxBlocks));
  const bool vec = p.IPL % 4 == 0 && E % 4 == 0 && aligned(logits, 16);
#define MOE_ROUTE_VC(G_, IPL_, VEC_)                                                          \
  return count ? launch(route_topk_kernel<G_, IPL_, VEC_, true, false>, grid, block, 0, s,     \
                        logits, T, E, k, 1, 0, topk_idx, topk_w, hist_mat, ch)                \
               : launch(route_topk_kernel<G_, IPL_, VEC_, false, false>, grid, block, 0, s,    \
                        logits, T, E, k, 1, 0, topk_idx, topk_w, hist_mat, ch)
#define MOE_ROUTE(G_, IPL_)                      \
  if (p.G == G_ && p.IPL == IPL_) {              \
    if (vec) MOE_ROUTE_VC(G_, IPL_, (IPL_ % 4 == 0)); \
    MOE_ROUTE_VC(G_, IPL_, false);               \
  }
  MOE_ROUTE(16, 1);
  MOE_ROUTE(16, 2);
  MOE_ROUTE(16, 4);
  MOE_ROUTE(16, 8);
  MOE_ROUTE(16, 16);
  MOE_ROUTE(16, 24);
  MOE_ROUTE(32, 1);
  MOE_ROUTE(32, 2);
  MOE_ROUTE(32, 4);
  MOE_ROUTE(32, 8);
  MOE_ROUTE(32, 16);
  MOE_ROUTE(32, 24);
  MOE_ROUTE(64, 1);
  MOE_ROUTE(64, 2);
  MOE_ROUTE(64, 4);
  MOE_ROUTE(64, 8);
  MOE_ROUTE(64, 16);
#undef MOE_ROUTE
#undef MOE_ROUTE_VC
  return MOE_ERR_INVALID_ARG;  // unreachable: plan_route covers every E <= 1024, k <= 32
}

// Plain routing that also counts the send histogram matrix in LDS first
// (route_topk_lds_count_kernel): for E < kRouteCountMinE with 16 lanes per
// token, at any T (below 2049 tokens it takes the place of the one wave per
// token kernel, and is faster than that kernel plus send_hist_kernel).
// False: the plan does not fit, and the caller counts with send_hist_kernel.
bool route_lds_count_fits(int64_t T, int32_t E, int32_t k) {
  return E < kRouteCountMinE && plan_route(T, E, k).G == 16;
}

int enqueue_route_lds_count(const float* logits, int64_t T, int32_t E, int32_t k,
                            int32_t* topk_idx, float* topk_w, int32_t* hist_mat, int64_t chunk,
                            hipStream_t s) {
  const RoutePlan p = plan_route(T, E, k);
  constexpr int TPB = kRouteWavesPerBlock * (kWave / 16);
  const int64_t nb = (T + TPB - 1) / TPB;
  const dim3 grid(unsigned(nb < kRouteMaxBlocks ? nb : kRouteMaxBlocks));
  const dim3 block(kRouteThreads);
  const bool vec = p.IPL % 4 == 0 && E % 4 == 0 && aligned(logits, 16);
  const uint32_t ch = uint32_t(chunk);
#define MOE_LDS_ROUTE(IPL_)                                                                  \
  if (p.IPL == IPL_)                                                                         \
    return vec ? launch(route_topk_lds_count_kernel<16, IPL_, (IPL_ % 4 == 0)>, grid, block, \
                        0, s, logits, T, E, k, topk_idx, topk_w, hist_mat, ch)               \
               : launch(route_topk_lds_count_kernel<16, IPL_, false>, grid, block, 0, s,     \
                        logits, T, E, k, topk_idx, topk_w, hist_mat, ch);
  MOE_LDS_ROUTE(1);
  MOE_LDS_ROUTE(2);
  MOE_LDS_ROUTE(4);
  MOE_LDS_ROUTE(8);
#undef MOE_LDS_ROUTE
  return MOE_ERR_INVALID_ARG;  // unreachable: E < 128 gives IPL <= 8 at 16 lanes per token
}

int check_groups(int32_t E, int32_t k, int32_t n_group, int32_t topk_group) {
  if (n_group < 1 || n_group > kMaxGroups || E % n_group != 0) return MOE_ERR_INVALID_ARG;
  if (topk_group < 1 || topk_group > n_group || int64_t(topk_group) * (E / n_group) < k)
    return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

int check_rows(int64_t T, int32_t H, int32_t k, int64_t capacity, const void* rows_in,
               const void* rows_out) {
  if (T < 0 || k < 1 || k > kMaxK || T > kMaxPairs / k) return MOE_ERR_INVALID_ARG;
  if (H < 8 || H > (1 << 20)) return MOE_ERR_INVALID_ARG;
  if (H % 8 != 0) return MOE_ERR_ALIGNMENT;
  if (capacity < T * k) return MOE_ERR_CAPACITY;
  if (T == 0) return MOE_OK;
  if (rows_in == nullptr || rows_out == nullptr) return MOE_ERR_INVALID_ARG;
  if (!aligned(rows_in, 16) || !aligned(rows_out, 16)) return MOE_ERR_ALIGNMENT;
  return MOE_OK;
}

int nbits_for(int E) {
  int n = 0;
  while ((1 << n) < E) ++n;
  return n;
}

int check_send(const int32_t* topk_idx, int64_t T, int32_t E, int32_t k, int32_t R,
               const int32_t* counts, const int32_t* offsets, const int32_t* pair_row,
               const int32_t* row_token, const int32_t* rank_offsets, const void* workspace,
               size_t workspace_bytes) {
  int st = check_route_shape(T, E, k);
  if (st != MOE_OK) return st;
  if (R < 1 || R > E || E % R != 0) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!topk_idx || !counts || !offsets || !pair_row || !row_token) return MOE_ERR_INVALID_ARG;
  const void* ints[] = {topk_idx, counts, offsets, pair_row, row_token, rank_offsets};
  for (const void* p : ints)
    if (!aligned(p, 4)) return MOE_ERR_ALIGNMENT;
  const SendPlan plan = plan_send(T * k, E);
  if (plan.ws_bytes > 0) {
    if (workspace == nullptr || workspace_bytes < plan.ws_bytes) return MOE_ERR_WORKSPACE;
    if (!aligned(workspace, 4)) return MOE_ERR_ALIGNMENT;
  }
  return MOE_OK;
}

// The histogram kernel of the multi-block send: fills the [blocks][E] matrix.
int enqueue_send_hist(const int32_t* topk_idx, int64_t T, int32_t E, int32_t k, int32_t* mat,
                      hipStream_t st) {
  const SendPlan plan = plan_send(T * k, E);
  return launch(send_hist_kernel, dim3(plan.nb), dim3(kSendThreads), size_t(E) * 4, st, topk_idx,
                T * k, E, nbits_for(E), plan.chunk, mat);
}

// The rank kernel of the multi-block send, given the filled [blocks][E]
// histogram matrix.
// histogram matrix, which it zeroes afterwards when `arrivals` is given.
int enqueue_send_ranks(const int32_t* topk_idx, int64_t T, int32_t E, int32_t k, int32_t R,
                       int32_t* counts, int32_t* offsets, int32_t* pair_row, int32_t* row_token,
                       int32_t* rank_offsets, int32_t* mat, uint32_t* arrivals, hipStream_t st) {
  const int64_t P = T * k;
  const SendPlan plan = plan_send(P, E);
  const size_t lds = (size_t(kSendWaves) * E + E + 17 + 2 * kSendThreads) * sizeof(int32_t);
  return launch(send_rank_kernel<false, kSendThreads, kSendRankItems>, dim3(plan.nb),
                dim3(kSendThreads), lds, st, topk_idx, P, E, k, nbits_for(E), plan.chunk, plan.nb,
                mat, arrivals, E / R, R, counts, offsets, rank_offsets, pair_row, row_token);
}

int enqueue_send(const int32_t* topk_idx, int64_t T, int32_t E, int32_t k, int32_t R,
                 int32_t* counts, int32_t* offsets, int32_t* pair_row, int32_t* row_token,
                 int32_t* rank_offsets, void* workspace, hipStream_t st) {
  const int64_t P = T * k;
  const SendPlan plan = plan_send(P, E);
  const int nbits = nbits_for(E);
  const int L = E / R;
  if (plan.fused) {
    const size_t lds = (size_t(plan.threads / kWave) * E + E + 17) * sizeof(int32_t);
    int32_t* none = nullptr;
    uint32_t* no_arrivals = nullptr;
    if (plan.threads == kSendWideThreads)
      return launch(send_rank_kernel<true, kSendWideThreads, kSendItems>, dim3(1),
                    dim3(kSendWideThreads), lds, st, topk_idx, P, E, k, nbits, plan.chunk, 1, none,
                    no_arrivals, L, R, counts, offsets, rank_offsets, pair_row, row_token);
    return launch(send_rank_kernel<true, kSendThreads, kSendItems>, dim3(1), dim3(kSendThreads),
                  lds, st, topk_idx, P, E, k, nbits, plan.chunk, 1, none, no_arrivals, L, R,
                  counts, offsets, rank_offsets, pair_row, row_token);
  }
  int32_t* ws = static_cast<int32_t*>(workspace);
  const int rc = enqueue_send_hist(topk_idx, T, E, k, ws, st);
  if (rc != MOE_OK) return rc;
  return enqueue_send_ranks(topk_idx, T, E, k, R, counts, offsets, pair_row, row_token,
                            rank_offsets, ws, nullptr, st);
}

int enqueue_recv(const void* x, const int32_t* pair_row, int64_t T, int32_t H, int32_t k,
                 void* buf, int64_t capacity, hipStream_t st) {
  const int C = H / 8;
  const RecvPlan p = plan_recv(T, C, k);
  if (kRecvStore >= 0 && uint64_t(capacity) * uint64_t(C) * 16u > 0xFFFFFFFFull)
    return MOE_ERR_INVALID_ARG;  // a measurement build: buffer stores address 4 GiB
  return launch(dispatch_recv_kernel<kRecvSlices>, dim3(p.nblocks), dim3(p.groups * kSlice), 0,
                st, static_cast<const u32x4*>(x), pair_row, T, C, k, p.per, p.nsb, p.units,
                static_cast<u32x4*>(buf), capacity);
}

// Send + recv in one launch: T*k <= 2048 (the 8-wave single-block send in one
// step) and k <= 8.
bool send_recv_fusable(int64_t T, int32_t k) {
  return T * k <= kSendRecvMaxPairs && k <= kSendRecvMaxK;
}

int enqueue_send_recv(const int32_t* topk_idx, const void* x, int64_t T, int32_t E, int32_t k,
                      int32_t H, int32_t R, int32_t* counts, int32_t* offsets, int32_t* pair_row,
                      int32_t* row_token, int32_t* rank_offsets, void* buf, int64_t capacity,
                      hipStream_t st) {
  const int C = H / 8;
  const int ncs = (C + kSlice - 1) / kSlice;
  const int nparts = (ncs + kSendRecvSlices - 1) / kSendRecvSlices;
  const int64_t units = T * nparts;
  const int64_t copy_blocks = units < kMaxRowBlocks ? units : kMaxRowBlocks;
  const size_t lds = (size_t(kSendWaves) * E + E + 17) * sizeof(int32_t);
  return launch(send_recv_kernel, dim3(unsigned(1 + copy_blocks)), dim3(kSendThreads), lds, st,
                topk_idx, T, E, k, nbits_for(E), E / R, R, counts, offsets, rank_offsets, pair_row,
                row_token, static_cast<const u32x4*>(x), C, nparts, units,
                static_cast<u32x4*>(buf), capacity);
}

int check_fp8_rows(int64_t T, int32_t H, int32_t k, int64_t capacity, const void* x,
                   const void* buf_q, const void* buf_s) {
  const int st = check_rows(T, H, k, capacity, x, buf_q);
  if (st != MOE_OK) return st;
  if (H % kQuantBlock != 0) return MOE_ERR_ALIGNMENT;
  if (T == 0) return MOE_OK;
  if (buf_s == nullptr) return MOE_ERR_INVALID_ARG;
  if (!aligned(buf_s, 4)) return MOE_ERR_ALIGNMENT;
  return MOE_OK;
}

int enqueue_recv_fp8(const void* x, const int32_t* pair_row, int64_t T, int32_t H, int32_t k,
                     void* buf_q, float* buf_s, int64_t capacity, hipStream_t st) {
  const int C = H / 8;
  const int nsb = (H + kFp8BlockElems - 1) / kFp8BlockElems;
  const int64_t units = T * nsb;
  const unsigned nblocks = unsigned(units < kMaxRowBlocks ? units : kMaxRowBlocks);
  return launch(dispatch_recv_fp8_kernel, dim3(nblocks), dim3(kFp8Waves * kWave), 0, st,
                static_cast<const u32x4*>(x), pair_row, T, C, H, k, nsb, units,
                static_cast<uint8_t*>(buf_q), buf_s, capacity);
}

int enqueue_send_recv_fp8(const int32_t* topk_idx, const void* x, int64_t T, int32_t E,
                          int32_t k, int32_t H, int32_t R, int32_t* counts, int32_t* offsets,
                          int32_t* pair_row, int32_t* row_token, int32_t* rank_offsets,
                          void* buf_q, float* buf_s, int64_t capacity, hipStream_t st) {
  const int nsb = (H + kFp8BlockElems - 1) / kFp8BlockElems;
  const int64_t units = T * nsb;
  const int64_t copy_blocks = units < kMaxRowBlocks ? units : kMaxRowBlocks;
  const size_t lds = (size_t(kSendWaves) * E + E + 17) * sizeof(int32_t);
  return launch(send_recv_fp8_kernel, dim3(unsigned(1 + copy_blocks)), dim3(kSendThreads), lds,
                st, topk_idx, T, E, k, nbits_for(E), E / R, R, counts, offsets, rank_offsets,
                pair_row, row_token, static_cast<const u32x4*>(x), H / 8, H, nsb, units,
                static_cast<uint8_t*>(buf_q), buf_s, capacity);
}

// Workspace of moe_route_dispatch: a block of arrival counters (word 0: the
// fused route + send launch; word 1: the rank kernel, whose last block
// zeroes the histogram matrix), then the send workspace.  All of it holds
// zeros between calls.
constexpr size_t kArrivalBytes = 256;

bool route_send_fusable(int64_t T, int32_t E, int32_t k) {
  return T <= kRouteWaveMaxTokens && plan_send(T * k, E).fused;
}

int enqueue_route_send(const float* logits, int64_t T, int32_t E, int32_t k, int32_t n_group,
                       int32_t topk_group, int32_t R, int32_t* topk_idx, float* topk_w,
                       uint32_t* arrivals, int32_t* counts, int32_t* offsets, int32_t* pair_row,
                       int32_t* row_token, int32_t* rank_offsets, hipStream_t st) {
  const bool grouped = topk_group < n_group;  // keeping every group is plain top-k
  const SendPlan plan = plan_send(T * k, E);
  const int waves = plan.threads / kWave;
  const size_t lds = (size_t(waves) * E + E + 17) * sizeof(int32_t);
  const dim3 grid(unsigned((T + waves - 1) / waves));
  const int ipl = (E + kWave - 1) / kWave;
  const int nbits = nbits_for(E);
  const int L = E / R;
#define MOE_FUSED(IPL_, THR_)                                                                 \
  return grouped ? launch(route_send_kernel<IPL_, THR_, true>, grid, dim3(THR_), lds, st,     \
                          logits, T, E, k, n_group, topk_group, topk_idx, topk_w, arrivals,   \
                          nbits, L, R, counts, offsets, rank_offsets, pair_row, row_token)    \
                 : launch(route_send_kernel<IPL_, THR_, false>, grid, dim3(THR_), lds, st,    \
                          logits, T, E, k, 1, 1, topk_idx, topk_w, arrivals, nbits, L, R,     \
                          counts, offsets, rank_offsets, pair_row, row_token)
#define MOE_FUSED_IPL(THR_)        \
  if (ipl <= 1) MOE_FUSED(1, THR_); \
  if (ipl <= 2) MOE_FUSED(2, THR_); \
  if (ipl <= 4) MOE_FUSED(4, THR_); \
  if (ipl <= 8) MOE_FUSED(8, THR_); \
  MOE_FUSED(16, THR_)
  if (plan.threads == kSendWideThreads) {
    MOE_FUSED_IPL(kSendWideThreads);
  }
  MOE_FUSED_IPL(kSendThreads);
#undef MOE_FUSED_IPL
#undef MOE_FUSED
}

// Argument checks of the route + send part of the one-call entry points
// (routing shape and groups, routing outputs, send outputs and workspace).
int check_route_and_send(const float* logits, int64_t T, int32_t E, int32_t k, int32_t n_group,
                         int32_t topk_group, int32_t R, const int32_t* topk_idx,
                         const float* topk_w, const int32_t* counts, const int32_t* offsets,
                         const int32_t* pair_row, const int32_t* row_token,
                         const int32_t* rank_offsets, const void* workspace,
                         size_t workspace_bytes) {
  int st = check_route_shape(T, E, k);
  if (st != MOE_OK) return st;
  st = check_groups(E, k, n_group, topk_group);
  if (st != MOE_OK) return st;
  if (T > 0 && (!logits || !topk_idx || !topk_w)) return MOE_ERR_INVALID_ARG;
  if (T > 0 && (!aligned(logits, 4) || !aligned(topk_idx, 4) || !aligned(topk_w, 4)))
    return MOE_ERR_ALIGNMENT;
  const size_t send_ws = workspace_bytes > kArrivalBytes ? workspace_bytes - kArrivalBytes : 0;
  const char* ws = static_cast<const char*>(workspace);
  return check_send(topk_idx, T, E, k, R, counts, offsets, pair_row, row_token, rank_offsets,
                    ws ? ws + kArrivalBytes : nullptr, send_ws);
}

// Route + send of the one-call entry points, on the caller's zeroed workspace
// (arrival counters, then the histogram matrix).  Small batches route and
// send in one launch; otherwise the multi-block send reads the histogram
// matrix, which the routing kernel fills itself when E is large enough (its
// atomics then spread over enough addresses) and the histogram kernel
// otherwise; the rank kernel's last block zeroes it again.
int enqueue_route_and_send(const float* logits, int64_t T, int32_t E, int32_t k, int32_t n_group,
                           int32_t topk_group, int32_t R, int32_t* topk_idx, float* topk_w,
                           int32_t* counts, int32_t* offsets, int32_t* pair_row,
                           int32_t* row_token, int32_t* rank_offsets, void* workspace,
                           hipStream_t s) {
  if (route_send_fusable(T, E, k))
    return enqueue_route_send(logits, T, E, k, n_group, topk_group, R, topk_idx, topk_w,
                              static_cast<uint32_t*>(workspace), counts, offsets, pair_row,
                              row_token, rank_offsets, s);
  const SendPlan plan = plan_send(T * k, E);
  int st;
  if (plan.fused) {  // single-block send: no histogram matrix
    st = enqueue_route(logits, T, E, k, n_group, topk_group, topk_idx, topk_w, s);
    if (st != MOE_OK) return st;
    return enqueue_send(topk_idx, T, E, k, R, counts, offsets, pair_row, row_token, rank_offsets,
                        nullptr, s);
  }
  int32_t* mat = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + kArrivalBytes);
  uint32_t* rank_arrivals = static_cast<uint32_t*>(workspace) + 1;
  const bool count = E >= kRouteCountMinE;
  if (!count && topk_group >= n_group && route_lds_count_fits(T, E, k)) {
    st = enqueue_route_lds_count(logits, T, E, k, topk_idx, topk_w, mat, plan.chunk, s);
  } else {
    st = enqueue_route(logits, T, E, k, n_group, topk_group, topk_idx, topk_w, s,
                       count ? mat : nullptr, plan.chunk);
    if (st == MOE_OK && !count) st = enqueue_send_hist(topk_idx, T, E, k, mat, s);
  }
  if (st != MOE_OK) return st;
  return enqueue_send_ranks(topk_idx, T, E, k, R, counts, offsets, pair_row, row_token,
                            rank_offsets, mat, rank_arrivals, s);
}

// ---------------------------------------------------------------------------
// scratch of moe_dispatch_noalloc: the send histogram matrix in device memory
// the library owns, for callers that cannot allocate
// ---------------------------------------------------------------------------

constexpr size_t kScratchBytes = size_t(kSendMatrixInts) * sizeof(int32_t);  // 64 KiB
constexpr int kMaxDevices = 64;

}  // namespace

// One copy per device, held until the process ends.  In host code the name
// stands for a host-side shadow, not a device address: kernels receive the
// address hipGetSymbolAddress returns for the device, never `scratch` itself.
static __device__ __align__(256) int32_t scratch[kSendMatrixInts];

namespace {

std::atomic<void*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the device that owns `st`, looked up once
// per device with that device current (each device holds its own copy at
// its own address).
int scratch_address(hipStream_t st, void** addr) {
  int dev = -1;
  const hipError_t e0 = st == nullptr ? hipGetDevice(&dev) : hipStreamGetDevice(st, &dev);
  if (e0 != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_INVALID_ARG;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      int cur = -1;
      if (hipGetDevice(&cur) != hipSuccess) return MOE_ERR_HIP;
      if (cur != dev && hipSetDevice(dev) != hipSuccess) return MOE_ERR_HIP;
      const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (cur != dev && hipSetDevice(cur) != hipSuccess) return MOE_ERR_HIP;
      if (e != hipSuccess || p == nullptr) return MOE_ERR_HIP;
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *addr = p;
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_strerror(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument (null pointer, size or limit out of range)";
    case MOE_ERR_ALIGNMENT: return "alignment (H % 8 != 0 or a row pointer not 16-byte aligned)";
    case MOE_ERR_CAPACITY: return "capacity below T*k (tokens are never dropped)";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP kernel launch failed";
    default: return "unknown status";
  }
}

int moe_route_topk(const float* logits, int64_t T, int32_t E, int32_t k, int32_t* topk_idx,
                   float* topk_w, void* stream) {
  return moe_route_topk_grouped(logits, T, E, k, 1, 1, topk_idx, topk_w, stream);
}

int moe_route_topk_grouped(const float* logits, int64_t T, int32_t E, int32_t k, int32_t n_group,
                           int32_t topk_group, int32_t* topk_idx, float* topk_w, void* stream) {
  int st = check_route_shape(T, E, k);
  if (st != MOE_OK) return st;
  st = check_groups(E, k, n_group, topk_group);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_idx || !topk_w) return MOE_ERR_INVALID_ARG;
  if (!aligned(logits, 4) || !aligned(topk_idx, 4) || !aligned(topk_w, 4)) return MOE_ERR_ALIGNMENT;
  return enqueue_route(logits, T, E, k, n_group, topk_group, topk_idx, topk_w,
                       static_cast<hipStream_t>(stream));
}

size_t moe_dispatch_workspace_bytes(int64_t T, int32_t E, int32_t k) {
  if (check_route_shape(T, E, k) != MOE_OK) return 0;
  return plan_send(T * k, E).ws_bytes;
}

int moe_dispatch_send(const int32_t* topk_idx, int64_t T, int32_t E, int32_t k,
                      int32_t num_vranks, int32_t* expert_counts, int32_t* expert_offsets,
                      int32_t* pair_row, int32_t* row_token, int32_t* rank_offsets,
                      void* workspace, size_t workspace_bytes, void* stream) {
  const int st = check_send(topk_idx, T, E, k, num_vranks, expert_counts, expert_offsets, pair_row,
                            row_token, rank_offsets, workspace, workspace_bytes);
  if (st != MOE_OK || T == 0) return st;
  return enqueue_send(topk_idx, T, E, k, num_vranks, expert_counts, expert_offsets, pair_row,
                      row_token, rank_offsets, workspace, static_cast<hipStream_t>(stream));
}

int moe_dispatch_recv(const void* x, const int32_t* pair_row, int64_t T, int32_t H, int32_t k,
                      void* buf, int64_t capacity, void* stream) {
  const int st = check_rows(T, H, k, capacity, x, buf);
  if (st != MOE_OK || T == 0) return st;
  if (pair_row == nullptr) return MOE_ERR_INVALID_ARG;
  if (!aligned(pair_row, 4)) return MOE_ERR_ALIGNMENT;
  return enqueue_recv(x, pair_row, T, H, k, buf, capacity, static_cast<hipStream_t>(stream));
}

int moe_dispatch(const int32_t* topk_idx, const void* x, int64_t T, int32_t E, int32_t k,
                 int32_t H, int32_t num_vranks, int32_t* expert_counts, int32_t* expert_offsets,
                 int32_t* pair_row, int32_t* row_token, int32_t* rank_offsets, void* buf,
                 int64_t capacity, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_send(topk_idx, T, E, k, num_vranks, expert_counts, expert_offsets, pair_row,
                      row_token, rank_offsets, workspace, workspace_bytes);
  if (st != MOE_OK) return st;
  st = check_rows(T, H, k, capacity, x, buf);
  if (st != MOE_OK || T == 0) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (send_recv_fusable(T, k))
    return enqueue_send_recv(topk_idx, x, T, E, k, H, num_vranks, expert_counts, expert_offsets,
                             pair_row, row_token, rank_offsets, buf, capacity, s);
  st = enqueue_send(topk_idx, T, E, k, num_vranks, expert_counts, expert_offsets, pair_row,
                    row_token, rank_offsets, workspace, s);
  if (st != MOE_OK) return st;
  return enqueue_recv(x, pair_row, T, H, k, buf, capacity, s);
}

int moe_dispatch_noalloc(const int32_t* topk_idx, const void* x, int64_t T, int32_t E,
                         int32_t k, int32_t H, int32_t num_vranks, int32_t* expert_counts,
                         int32_t* expert_offsets, int32_t* pair_row, int32_t* row_token,
                         int32_t* rank_offsets, void* buf, int64_t capacity, void* stream) {
  // Every argument is checked before the device's scratch is looked up; the
  // workspace check of the send half is the one failure expected here.
  int st = check_send(topk_idx, T, E, k, num_vranks, expert_counts, expert_offsets, pair_row,
                      row_token, rank_offsets, nullptr, 0);
  if (st != MOE_OK && st != MOE_ERR_WORKSPACE) return st;
  st = check_rows(T, H, k, capacity, x, buf);
  if (st != MOE_OK || T == 0) return st;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  const size_t need = plan_send(T * k, E).ws_bytes;
  if (need > kScratchBytes) return MOE_ERR_WORKSPACE;  // never above 64 KiB by the send plan
  if (need > 0) {
    const int rc = scratch_address(static_cast<hipStream_t>(stream), &ws);
    if (rc != MOE_OK) return rc;
    ws_bytes = kScratchBytes;
  }
  return moe_dispatch(topk_idx, x, T, E, k, H, num_vranks, expert_counts, expert_offsets, pair_row,
                      row_token, rank_offsets, buf, capacity, ws, ws_bytes, stream);
}

size_t moe_route_dispatch_workspace_bytes(int64_t T, int32_t E, int32_t k) {
  if (check_route_shape(T, E, k) != MOE_OK) return 0;
  return kArrivalBytes + plan_send(T * k, E).ws_bytes;
}

int moe_route_dispatch(const float* logits, const void* x, int64_t T, int32_t E, int32_t k,
                       int32_t n_group, int32_t topk_group, int32_t H, int32_t num_vranks,
                       int32_t* topk_idx, float* topk_w, int32_t* expert_counts,
                       int32_t* expert_offsets, int32_t* pair_row, int32_t* row_token,
                       int32_t* rank_offsets, void* buf, int64_t capacity, void* workspace,
                       size_t workspace_bytes, void* stream) {
  int st = check_route_and_send(logits, T, E, k, n_group, topk_group, num_vranks, topk_idx,
                                topk_w, expert_counts, expert_offsets, pair_row, row_token,
                                rank_offsets, workspace, workspace_bytes);
  if (st != MOE_OK) return st;
  st = check_rows(T, H, k, capacity, x, buf);
  if (st != MOE_OK || T == 0) return st;
  if (workspace == nullptr || workspace_bytes < kArrivalBytes) return MOE_ERR_WORKSPACE;
  if (!aligned(workspace, 4)) return MOE_ERR_ALIGNMENT;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (send_recv_fusable(T, k)) {  // route, then send and recv in one launch
    st = enqueue_route(logits, T, E, k, n_group, topk_group, topk_idx, topk_w, s);
    if (st != MOE_OK) return st;
    return enqueue_send_recv(topk_idx, x, T, E, k, H, num_vranks, expert_counts, expert_offsets,
                             pair_row, row_token, rank_offsets, buf, capacity, s);
  }
  st = enqueue_route_and_send(logits, T, E, k, n_group, topk_group, num_vranks, topk_idx, topk_w,
                              expert_counts, expert_offsets, pair_row, row_token, rank_offsets,
                              workspace, s);
  if (st != MOE_OK) return st;
  return enqueue_recv(x, pair_row, T, H, k, buf, capacity, s);
}

int moe_route_dispatch_fp8(const float* logits, const void* x, int64_t T, int32_t E, int32_t k,
                           int32_t n_group, int32_t topk_group, int32_t H, int32_t num_vranks,
                           int32_t* topk_idx, float* topk_w, int32_t* expert_counts,
                           int32_t* expert_offsets, int32_t* pair_row, int32_t* row_token,
                           int32_t* rank_offsets, void* buf_q, float* buf_scale,
                           int64_t capacity, void* workspace, size_t workspace_bytes,
                           void* stream) {
  int st = check_route_and_send(logits, T, E, k, n_group, topk_group, num_vranks, topk_idx,
                                topk_w, expert_counts, expert_offsets, pair_row, row_token,
                                rank_offsets, workspace, workspace_bytes);
  if (st != MOE_OK) return st;
  st = check_fp8_rows(T, H, k, capacity, x, buf_q, buf_scale);
  if (st != MOE_OK || T == 0) return st;
  if (workspace == nullptr || workspace_bytes < kArrivalBytes) return MOE_ERR_WORKSPACE;
  if (!aligned(workspace, 4)) return MOE_ERR_ALIGNMENT;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (send_recv_fusable(T, k)) {  // route, then send and fp8 recv in one launch
    st = enqueue_route(logits, T, E, k, n_group, topk_group, topk_idx, topk_w, s);
    if (st != MOE_OK) return st;
    return enqueue_send_recv_fp8(topk_idx, x, T, E, k, H, num_vranks, expert_counts,
                                 expert_offsets, pair_row, row_token, rank_offsets, buf_q,
                                 buf_scale, capacity, s);
  }
  st = enqueue_route_and_send(logits, T, E, k, n_group, topk_group, num_vranks, topk_idx, topk_w,
                              expert_counts, expert_offsets, pair_row, row_token, rank_offsets,
                              workspace, s);
  if (st != MOE_OK) return st;
  return enqueue_recv_fp8(x, pair_row, T, H, k, buf_q, buf_scale, capacity, s);
}

int moe_dispatch_recv_fp8(const void* x, const int32_t* pair_row, int64_t T, int32_t H, int32_t k,
                          void* buf_q, float* buf_scale, int64_t capacity, void* stream) {
  const int st = check_fp8_rows(T, H, k, capacity, x, buf_q, buf_scale);
  if (st != MOE_OK || T == 0) return st;
  if (pair_row == nullptr) return MOE_ERR_INVALID_ARG;
  if (!aligned(pair_row, 4)) return MOE_ERR_ALIGNMENT;
  return enqueue_recv_fp8(x, pair_row, T, H, k, buf_q, buf_scale, capacity,
                          static_cast<hipStream_t>(stream));
}

int moe_dispatch_fp8(const int32_t* topk_idx, const void* x, int64_t T, int32_t E, int32_t k,
                     int32_t H, int32_t num_vranks, int32_t* expert_counts,
                     int32_t* expert_offsets, int32_t* pair_row, int32_t* row_token,
                     int32_t* rank_offsets, void* buf_q, float* buf_scale, int64_t capacity,
                     void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_send(topk_idx, T, E, k, num_vranks, expert_counts, expert_offsets, pair_row,
                      row_token, rank_offsets, workspace, workspace_bytes);
  if (st != MOE_OK) return st;
  st = check_fp8_rows(T, H, k, capacity, x, buf_q, buf_scale);
  if (st != MOE_OK || T == 0) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (send_recv_fusable(T, k))
    return enqueue_send_recv_fp8(topk_idx, x, T, E, k, H, num_vranks, expert_counts,
                                 expert_offsets, pair_row, row_token, rank_offsets, buf_q,
                                 buf_scale, capacity, s);
  st = enqueue_send(topk_idx, T, E, k, num_vranks, expert_counts, expert_offsets, pair_row,
                    row_token, rank_offsets, workspace, s);
  if (st != MOE_OK) return st;
  return enqueue_recv_fp8(x, pair_row, T, H, k, buf_q, buf_scale, capacity, s);
}

int moe_combine(const void* y, const int32_t* pair_row, const float* topk_w, int64_t T, int32_t H,
                int32_t k, int64_t capacity, void* out, void* stream) {
  const int st = check_rows(T, H, k, capacity, y, out);
  if (st != MOE_OK || T == 0) return st;
  if (pair_row == nullptr || topk_w == nullptr) return MOE_ERR_INVALID_ARG;
  if (!aligned(pair_row, 4) || !aligned(topk_w, 4)) return MOE_ERR_ALIGNMENT;
  const int C = H / 8;
  const int ncs = (C + kSlice - 1) / kSlice;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const u32x4* yv = static_cast<const u32x4*>(y);
  u32x4* ov = static_cast<u32x4*>(out);
  auto small = [&](auto kern, int u) {
    const int nsb = (ncs + u - 1) / u;
    const int64_t units = T * nsb;
    const unsigned nblocks = unsigned(units < kMaxRowBlocks ? units : kMaxRowBlocks);
    return launch(kern, dim3(nblocks), dim3(kSlice), 0, s, yv, pair_row, topk_w, T, C, nsb, units,
                  capacity, ov);
  };
  const bool sc1 = 2 * T * H * (int64_t(k) + 1) > kCombineSc1MinBytes;
#define MOE_SMALL(K_, U_) \
  return sc1 ? small(combine_small_k_kernel<K_, U_, true>, U_) \
             : small(combine_small_k_kernel<K_, U_, false>, U_)
  if (k == 1) MOE_SMALL(1, 16);
  if (k == 2) MOE_SMALL(2, 8);
  if (k == 4) MOE_SMALL(4, 4);
  if (k == 8) MOE_SMALL(8, 1);
#undef MOE_SMALL
  const int64_t units = T * ncs;
  const unsigned nblocks = unsigned(units < kMaxRowBlocks ? units : kMaxRowBlocks);
  return sc1 ? launch(combine_kernel<true>, dim3(nblocks), dim3(kSlice), 0, s, yv, pair_row,
                      topk_w, T, C, k, ncs, units, capacity, ov)
             : launch(combine_kernel<false>, dim3(nblocks), dim3(kSlice), 0, s, yv, pair_row,
                      topk_w, T, C, k, ncs, units, capacity, ov);
}

}  // extern "C"

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
// LDS and HBM3E:
//
//   route_topk_kernel    one wave per token: fp32 softmax over E logits held
//                        in registers, k rounds of a wave-wide arg-max on a
//                        64-bit (logit, -index) key.
//   send_hist_kernel     per-block expert histogram; each wave groups equal
//   send_scan_kernel     experts with ballots so the hot expert costs one LDS
//   send_rank_kernel     update per wave, not 64.  One block scans the
//                        [block][expert] counts; the rank kernel gives each
//                        pair a stable slot (ballot + mbcnt inside a wave,
//                        LDS prefix across waves, scanned base across blocks).
//                        Small inputs run all three steps in one block.
//   dispatch_recv_kernel each token row is read from HBM once with 16-byte
//                        loads and written to its k rows with 16-byte
//                        non-temporal stores.
//   combine_kernel       per token: k independent 16-byte row loads in
//                        flight, fp32 fma chain in j order, one bf16 RNE
//                        (v_cvt_pk_bf16_f32), 16-byte stores.  Row indices and
//                        weights of a token tile are staged in LDS.
//
// There is no dense contraction here, so no MFMA: the row kernels are bound by
// HBM bandwidth and the routing / send kernels by latency.

#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

#include <tuple>
#include <utility>

#include "moe_route.h"

namespace {

constexpr int kWave = 64;
constexpr int kMaxE = 1024;
constexpr int kMaxK = 32;
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

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

__device__ __forceinline__ int32_t wave_incl_scan(int32_t v) {
  const int lane = lane_id();
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int32_t o = __shfl_up(v, off);
    if (lane >= off) v += o;
  }
  return v;
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
// Every thread of the block must call it.  scratch: >= 17 ints of LDS.
__device__ int32_t block_excl_scan(int32_t* data, int n, int32_t* scratch) {
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
  if (lane == kWave - 1) scratch[wid] = incl;
  __syncthreads();
  if (wid == 0) {
    const int32_t ws = lane < nwaves ? scratch[lane] : 0;
    const int32_t wi = wave_incl_scan(ws);
    if (lane < nwaves) scratch[lane] = wi - ws;
    if (lane == nwaves - 1) scratch[16] = wi;
  }
  __syncthreads();
  int32_t run = scratch[wid] + incl - s;
  for (int i = 0; i < per; ++i) {
    if (beg + i < n) {
      const int32_t v = data[beg + i];
      data[beg + i] = run;
      run += v;
    }
  }
  const int32_t total = scratch[16];
  __syncthreads();
  return total;
}

// ---------------------------------------------------------------------------
// route: softmax + top-k, one wave per token
// ---------------------------------------------------------------------------

// Monotone map of a float onto uint32 (larger float -> larger key), with -0.0
// folded into +0.0 so that the two compare equal.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  u = (u == 0x80000000u) ? 0u : u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kRouteWavesPerBlock = 4;

template <int IPL>  // logits held per lane: ceil(E / 64) rounded up to a template size
__global__ __launch_bounds__(kRouteWavesPerBlock* kWave) void route_topk_kernel(
    const float* __restrict__ logits, int64_t T, int E, int k, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w) {
  const int lane = lane_id();
  const int64_t t = int64_t(blockIdx.x) * kRouteWavesPerBlock + threadIdx.x / kWave;
  if (t >= T) return;  // whole waves leave; no block barrier follows
  const float* row = logits + t * E;

  float lv[IPL];
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < IPL; ++i) {
    const int e = lane + i * kWave;
    lv[i] = e < E ? row[e] : -INFINITY;
    m = fmaxf(m, lv[i]);
  }
  m = wave_max(m);

  // Softmax numerators exp(l - m).  The difference is split into its fp32
  // rounding d and the exact remainder r (TwoSum), and exp(d + r) is taken as
  // exp(d) * (1 + r): the subtraction then adds no error of its own.
  float pv[IPL];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < IPL; ++i) {
    const int e = lane + i * kWave;
    float z = 0.f;
    if (e < E) {
      const float a = lv[i], b = -m;
      const float d = a + b;
      const float bb = d - a;
      const float r = (a - (d - bb)) + (b - bb);
      const float ed = expf(d);
      z = __builtin_fmaf(ed, r, ed);
    }
    pv[i] = z;
    s += z;
  }
  s = wave_sum(s);
#pragma unroll
  for (int i = 0; i < IPL; ++i) pv[i] = pv[i] / s;  // fp32 softmax probabilities

  // k rounds of a wave-wide arg-max over the untaken experts.  Key: order_key
  // of the logit in the high half, ~e in the low half, so equal logits pick
  // the lower expert index.  Every finite logit has a key above 0.
  uint32_t taken = 0;
  int my_e = 0;
  float my_p = 0.f;
  float psum = 0.f, pcomp = 0.f;  // compensated sum of the selected probabilities
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0;
    float bestp = 0.f;
#pragma unroll
    for (int i = 0; i < IPL; ++i) {
      const int e = lane + i * kWave;
      if (e < E && !((taken >> i) & 1u)) {
        const uint64_t key = (uint64_t(order_key(lv[i])) << 32) | uint32_t(~uint32_t(e));
        if (key > best) {
          best = key;
          bestp = pv[i];
        }
      }
    }
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) {
      const uint64_t ob = __shfl_xor(best, off);
      const float op = __shfl_xor(bestp, off);
      if (ob > best) {
        best = ob;
        bestp = op;
      }
    }
    const uint32_t es = ~uint32_t(best);  // the winning expert, same on every lane
    if (int(es & (kWave - 1)) == lane) taken |= 1u << (es / kWave);
    if (lane == j) {
      my_e = int(es);
      my_p = bestp;
    }
    const float ns = psum + bestp;  // TwoSum of the running sum
    const float bv = ns - psum;
    pcomp += (psum - (ns - bv)) + (bestp - bv);
    psum = ns;
  }
  const float total = psum + pcomp;
  if (lane < k) {
    topk_idx[t * k + lane] = my_e;
    topk_w[t * k + lane] = my_p / total;
  }
}

// ---------------------------------------------------------------------------
// dispatch send: histogram, scan, stable slots
// ---------------------------------------------------------------------------

constexpr int kSendThreads = 512;
constexpr int kSendWaves = kSendThreads / kWave;
constexpr int kScanThreads = 1024;
constexpr int64_t kSendFusedMaxPairs = 4096;
constexpr int64_t kSendChunkTarget = 2048;
constexpr int kScanLdsCounts = 12288;  // [block][expert] counts staged in the scan block's LDS

struct SendPlan {
  bool fused;
  int nb;         // blocks of the histogram and rank kernels
  int64_t chunk;  // pairs per block
  size_t ws_bytes;
};

SendPlan plan_send(int64_t P, int E) {
  SendPlan p{};
  if (P <= kSendFusedMaxPairs) {
    p.fused = true;
    p.nb = 1;
    p.chunk = P > 0 ? P : 1;
    p.ws_bytes = 0;
    return p;
  }
  int64_t nb = (P + kSendChunkTarget - 1) / kSendChunkTarget;
  int64_t nb_max = kScanLdsCounts / E;
  if (nb_max > 1024) nb_max = 1024;
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

// The pairs [a, b) this wave handles inside its block's chunk.
__device__ __forceinline__ void wave_range(int64_t P, int64_t chunk, int64_t& a, int64_t& b) {
  const int nwaves = blockDim.x / kWave;
  const int wid = threadIdx.x / kWave;
  const int64_t c0 = int64_t(blockIdx.x) * chunk;
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
  wave_range(P, chunk, a, b);
  for (int64_t base = a; base < b; base += kWave) {
    const int64_t p = base + lane_id();
    int e = p < b ? idx[p] : -1;
    const bool valid = uint32_t(e) < uint32_t(E);
    const uint64_t peers = same_expert_lanes(e, valid, nbits);
    if (valid && lanes_below(peers) == 0) atomicAdd(&hist[e], int32_t(__popcll(peers)));
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) ws_cnt[int64_t(blockIdx.x) * E + e] = hist[e];
}

// One block: for every expert, exclusive scan of the per-block counts (in
// place, giving each block's first slot inside the expert), then an exclusive
// scan over experts for the offsets, which is added to the per-block bases.
__global__ __launch_bounds__(kScanThreads) void send_scan_kernel(
    int32_t* __restrict__ ws, int nb, int E, int L, int R, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ rank_offsets) {
  extern __shared__ int32_t sm[];  // [nb*E] counts | [E] totals | [17] scan scratch
  int32_t* cnt = sm;
  int32_t* tot = sm + nb * E;
  int32_t* scratch = tot + E;
  for (int i = threadIdx.x; i < nb * E; i += blockDim.x) cnt[i] = ws[i];
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int32_t run = 0;
    for (int b = 0; b < nb; ++b) {
      const int32_t c = cnt[b * E + e];
      cnt[b * E + e] = run;
      run += c;
    }
    tot[e] = run;
    counts[e] = run;
  }
  __syncthreads();
  const int32_t total = block_excl_scan(tot, E, scratch);
  for (int e = threadIdx.x; e < E; e += blockDim.x) offsets[e] = tot[e];
  if (threadIdx.x == 0) offsets[E] = total;
  if (rank_offsets != nullptr) {
    for (int r = threadIdx.x; r < R; r += blockDim.x) rank_offsets[r] = tot[r * L];
    if (threadIdx.x == 0) rank_offsets[R] = total;
  }
  for (int i = threadIdx.x; i < nb * E; i += blockDim.x) ws[i] = cnt[i] + tot[i % E];
}

// Stable slot of every pair.  Pass 1: inside each wave, lanes with the same
// expert are ranked by lane order (mbcnt over the matching-lane mask) on top
// of the wave's running count kept in LDS; the wave-local slot is parked in
// pair_row.  Then an exclusive prefix over waves per expert, plus the block's
// base (multi-block) or the block-wide offsets (fused), completes the row.
template <bool FUSED>
__global__ __launch_bounds__(kSendThreads) void send_rank_kernel(
    const int32_t* __restrict__ idx, int64_t P, int E, int k, int nbits, int64_t chunk,
    const int32_t* __restrict__ ws_base, int L, int R, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ rank_offsets,
    int32_t* __restrict__ pair_row, int32_t* __restrict__ row_token) {
  extern __shared__ int32_t sm[];  // [W][E] per-wave counts | [E] base | [17] scratch
  const int nwaves = blockDim.x / kWave;
  const int wid = threadIdx.x / kWave;
  int32_t* hist = sm;
  int32_t* base = sm + nwaves * E;
  int32_t* scratch = base + E;
  for (int i = threadIdx.x; i < nwaves * E; i += blockDim.x) hist[i] = 0;
  __syncthreads();

  int64_t a, b;
  wave_range(P, chunk, a, b);
  int32_t* my_hist = hist + wid * E;
  for (int64_t s0 = a; s0 < b; s0 += kWave) {
    const int64_t p = s0 + lane_id();
    const int e = p < b ? idx[p] : -1;
    const bool valid = uint32_t(e) < uint32_t(E);
    const uint64_t peers = same_expert_lanes(e, valid, nbits);
    if (valid) {
      const uint32_t below = lanes_below(peers);
      const int32_t cur = my_hist[e];
      pair_row[p] = cur + int32_t(below);
      if (below == 0) my_hist[e] = cur + int32_t(__popcll(peers));
    } else if (p < b) {
      pair_row[p] = -1;  // expert index out of range: the pair is dropped
    }
  }
  __syncthreads();

  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int32_t run = 0;
    for (int w = 0; w < nwaves; ++w) {
      const int32_t c = hist[w * E + e];
      hist[w * E + e] = run;
      run += c;
    }
    if (FUSED) {
      base[e] = run;
      counts[e] = run;
    } else {
      base[e] = ws_base[int64_t(blockIdx.x) * E + e];
    }
  }
  __syncthreads();
  if (FUSED) {
    const int32_t total = block_excl_scan(base, E, scratch);
    for (int e = threadIdx.x; e < E; e += blockDim.x) offsets[e] = base[e];
    if (threadIdx.x == 0) offsets[E] = total;
    if (rank_offsets != nullptr) {
      for (int r = threadIdx.x; r < R; r += blockDim.x) rank_offsets[r] = base[r * L];
      if (threadIdx.x == 0) rank_offsets[R] = total;
    }
  }

  for (int64_t s0 = a; s0 < b; s0 += kWave) {
    const int64_t p = s0 + lane_id();
    if (p < b) {
      const int e = idx[p];
      if (uint32_t(e) < uint32_t(E)) {
        const int32_t r = base[e] + my_hist[e] + pair_row[p];
        pair_row[p] = r;
        row_token[r] = int32_t(p) / k;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dispatch recv and combine: token-tile row kernels
// ---------------------------------------------------------------------------

constexpr int kRowThreads = 256;
constexpr int kRecvUnroll = 4;     // 16-byte row chunks per thread in flight
constexpr int kCombineUnroll = 1;  // tokens' chunks per thread per step
constexpr int kCombineGroup = 8;   // expert rows loaded before their fma

struct RowPlan {
  int TT;       // tokens per tile
  int CW;       // 16-byte chunks per tile (a column slice of the row)
  int ncs;      // column slices per row
  int64_t nblocks;
  size_t lds;
};

RowPlan plan_rows(int64_t T, int C, int k, int unroll, bool with_w, int min_blocks) {
  RowPlan p{};
  const int target = kRowThreads * unroll;
  p.TT = C >= target ? 1 : target / C;
  p.CW = C;
  auto blocks = [&](int TT, int CW) {
    return ((T + TT - 1) / TT) * int64_t((C + CW - 1) / CW);
  };
  while (blocks(p.TT, p.CW) < min_blocks) {
    if (p.TT > 1) {
      p.TT = (p.TT + 1) / 2;
    } else if (p.CW > kWave) {
      p.CW = ((p.CW / 2) + kWave - 1) / kWave * kWave;
    } else {
      break;
    }
  }
  p.ncs = (C + p.CW - 1) / p.CW;
  p.nblocks = blocks(p.TT, p.CW);
  p.lds = size_t(p.TT) * k * (with_w ? 8 : 4);
  return p;
}

__device__ __forceinline__ void tile_coords(int64_t T, int C, int TT, int CW, int ncs, int64_t& t0,
                                            int& nt, int& c0, int& cw) {
  const int64_t tile = blockIdx.x / ncs;
  const int cs = int(blockIdx.x - tile * ncs);
  t0 = tile * TT;
  nt = int(T - t0 < TT ? T - t0 : TT);
  c0 = cs * CW;
  cw = C - c0 < CW ? C - c0 : CW;
}

__global__ __launch_bounds__(kRowThreads) void dispatch_recv_kernel(
    const u32x4* __restrict__ x, const int32_t* __restrict__ pair_row, int64_t T, int C, int k,
    int TT, int CW, int ncs, u32x4* __restrict__ buf, int64_t capacity) {
  extern __shared__ int32_t pr_s[];  // [TT][k]
  int64_t t0;
  int nt, c0, cw;
  tile_coords(T, C, TT, CW, ncs, t0, nt, c0, cw);
  for (int i = threadIdx.x; i < nt * k; i += blockDim.x) pr_s[i] = pair_row[t0 * k + i];
  __syncthreads();
  const int units = nt * cw;
  for (int ub = 0; ub < units; ub += kRowThreads * kRecvUnroll) {
    u32x4 v[kRecvUnroll];
    int tl[kRecvUnroll], c[kRecvUnroll];
#pragma unroll
    for (int u = 0; u < kRecvUnroll; ++u) {
      const int uu = ub + u * kRowThreads + threadIdx.x;
      tl[u] = nt == 1 ? 0 : uu / cw;
      c[u] = c0 + uu - tl[u] * cw;
      if (uu < units) v[u] = __builtin_nontemporal_load(&x[(t0 + tl[u]) * C + c[u]]);
    }
#pragma unroll
    for (int u = 0; u < kRecvUnroll; ++u) {
      const int uu = ub + u * kRowThreads + threadIdx.x;
      if (uu < units) {
        for (int j = 0; j < k; ++j) {
          const int32_t r = pr_s[tl[u] * k + j];
          if (uint64_t(int64_t(r)) < uint64_t(capacity))
            __builtin_nontemporal_store(v[u], &buf[int64_t(r) * C + c[u]]);
        }
      }
    }
  }
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 f = {lo, hi};
  const bf16x2 h = __builtin_convertvector(f, bf16x2);  // round-to-nearest-even
  return __builtin_bit_cast(uint32_t, h);
}

__global__ __launch_bounds__(kRowThreads) void combine_kernel(
    const u32x4* __restrict__ y, const int32_t* __restrict__ pair_row,
    const float* __restrict__ topk_w, int64_t T, int C, int k, int TT, int CW, int ncs,
    int64_t capacity, u32x4* __restrict__ out) {
  extern __shared__ int32_t sm[];  // [TT][k] rows | [TT][k] weights
  int32_t* pr_s = sm;
  int64_t t0;
  int nt, c0, cw;
  tile_coords(T, C, TT, CW, ncs, t0, nt, c0, cw);
  float* w_s = reinterpret_cast<float*>(sm + TT * k);
  for (int i = threadIdx.x; i < nt * k; i += blockDim.x) {
    pr_s[i] = pair_row[t0 * k + i];
    w_s[i] = topk_w[t0 * k + i];
  }
  __syncthreads();
  const int units = nt * cw;
  for (int ub = 0; ub < units; ub += kRowThreads * kCombineUnroll) {
#pragma unroll
    for (int u = 0; u < kCombineUnroll; ++u) {
      const int uu = ub + u * kRowThreads + threadIdx.x;
      if (uu >= units) continue;
      const int tl = nt == 1 ? 0 : uu / cw;
      const int c = c0 + uu - tl * cw;
      const int32_t* prt = pr_s + tl * k;
      const float* wt = w_s + tl * k;
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
            const float wj = wt[j0 + g];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const uint32_t word = v[g][q];
              acc[2 * q] = __builtin_fmaf(wj, __uint_as_float(word << 16), acc[2 * q]);
              acc[2 * q + 1] = __builtin_fmaf(wj, __uint_as_float(word & 0xFFFF0000u), acc[2 * q + 1]);
            }
          }
        }
      }
      u32x4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
      out[(t0 + tl) * C + c] = o;
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

int enqueue_send(const int32_t* topk_idx, int64_t T, int32_t E, int32_t k, int32_t R,
                 int32_t* counts, int32_t* offsets, int32_t* pair_row, int32_t* row_token,
                 int32_t* rank_offsets, void* workspace, hipStream_t st) {
  const int64_t P = T * k;
  const SendPlan plan = plan_send(P, E);
  const int nbits = nbits_for(E);
  const int L = E / R;
  if (plan.fused) {
    const size_t lds = (size_t(kSendWaves) * E + E + 17) * sizeof(int32_t);
    return launch(send_rank_kernel<true>, dim3(1), dim3(kSendThreads), lds, st, topk_idx, P, E,
                  k, nbits, plan.chunk, static_cast<const int32_t*>(nullptr), L, R, counts,
                  offsets, rank_offsets, pair_row, row_token);
  }
  int32_t* ws = static_cast<int32_t*>(workspace);
  int rc = launch(send_hist_kernel, dim3(plan.nb), dim3(kSendThreads), size_t(E) * 4, st,
                  topk_idx, P, E, nbits, plan.chunk, ws);
  if (rc != MOE_OK) return rc;
  const size_t scan_lds = (size_t(plan.nb) * E + E + 17) * sizeof(int32_t);
  rc = launch(send_scan_kernel, dim3(1), dim3(kScanThreads), scan_lds, st, ws, plan.nb, E, L, R,
              counts, offsets, rank_offsets);
  if (rc != MOE_OK) return rc;
  const size_t lds = (size_t(kSendWaves) * E + E + 17) * sizeof(int32_t);
  return launch(send_rank_kernel<false>, dim3(plan.nb), dim3(kSendThreads), lds, st, topk_idx, P,
                E, k, nbits, plan.chunk, static_cast<const int32_t*>(ws), L, R, counts, offsets,
                rank_offsets, pair_row, row_token);
}

int min_row_blocks() { return 1024; }

int enqueue_recv(const void* x, const int32_t* pair_row, int64_t T, int32_t H, int32_t k,
                 void* buf, int64_t capacity, hipStream_t st) {
  const int C = H / 8;
  const RowPlan p = plan_rows(T, C, k, kRecvUnroll, false, min_row_blocks());
  return launch(dispatch_recv_kernel, dim3(unsigned(p.nblocks)), dim3(kRowThreads), p.lds, st,
                static_cast<const u32x4*>(x), pair_row, T, C, k, p.TT, p.CW, p.ncs,
                static_cast<u32x4*>(buf), capacity);
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
  const int st = check_route_shape(T, E, k);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_idx || !topk_w) return MOE_ERR_INVALID_ARG;
  if (!aligned(logits, 4) || !aligned(topk_idx, 4) || !aligned(topk_w, 4)) return MOE_ERR_ALIGNMENT;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(unsigned((T + kRouteWavesPerBlock - 1) / kRouteWavesPerBlock));
  const dim3 block(kRouteWavesPerBlock * kWave);
  const int ipl = (E + kWave - 1) / kWave;
  if (ipl <= 1) return launch(route_topk_kernel<1>, grid, block, 0, s, logits, T, E, k, topk_idx, topk_w);
  if (ipl <= 2) return launch(route_topk_kernel<2>, grid, block, 0, s, logits, T, E, k, topk_idx, topk_w);
  if (ipl <= 4) return launch(route_topk_kernel<4>, grid, block, 0, s, logits, T, E, k, topk_idx, topk_w);
  if (ipl <= 8) return launch(route_topk_kernel<8>, grid, block, 0, s, logits, T, E, k, topk_idx, topk_w);
  return launch(route_topk_kernel<16>, grid, block, 0, s, logits, T, E, k, topk_idx, topk_w);
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
  st = enqueue_send(topk_idx, T, E, k, num_vranks, expert_counts, expert_offsets, pair_row,
                    row_token, rank_offsets, workspace, s);
  if (st != MOE_OK) return st;
  return enqueue_recv(x, pair_row, T, H, k, buf, capacity, s);
}

int moe_combine(const void* y, const int32_t* pair_row, const float* topk_w, int64_t T, int32_t H,
                int32_t k, int64_t capacity, void* out, void* stream) {
  const int st = check_rows(T, H, k, capacity, y, out);
  if (st != MOE_OK || T == 0) return st;
  if (pair_row == nullptr || topk_w == nullptr) return MOE_ERR_INVALID_ARG;
  if (!aligned(pair_row, 4) || !aligned(topk_w, 4)) return MOE_ERR_ALIGNMENT;
  const int C = H / 8;
  const RowPlan p = plan_rows(T, C, k, 4, true, min_row_blocks());
  return launch(combine_kernel, dim3(unsigned(p.nblocks)), dim3(kRowThreads), p.lds,
                static_cast<hipStream_t>(stream), static_cast<const u32x4*>(y), pair_row, topk_w,
                T, C, k, p.TT, p.CW, p.ncs, capacity, static_cast<u32x4*>(out));
}

}  // extern "C"

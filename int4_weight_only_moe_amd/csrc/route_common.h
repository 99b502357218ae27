// Top-k routing device functions shared by the routing kernels: ordered
// float keys, wave-wide reductions without LDS, and the one-wave top-k of a
// token ("The Throughput Lever: Quantifying the MoE GEMM and Mapping the Road
// to B300", section "The Result: Two Regimes": each token activates its top-k
// experts; softmax weights renormalised over the kept ones).
#pragma once

#include "device_common.h"

namespace moe {

// Order-preserving map of a finite fp32 value to uint32 (larger value ->
// larger key); -0.0 is first turned into +0.0 so that the two tie. Key 0 is
// never produced for finite inputs and marks "absent / already taken".
__device__ __forceinline__ uint32_t order_key(float v) {
  uint32_t u = __float_as_uint(v + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t key) {
  uint32_t u = (key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key;
  return __uint_as_float(u);
}

// Cross-lane exchanges without LDS: DPP inside rows of 16 lanes, then the
// gfx950 row swaps (permlane16/32_swap) across rows. After each step every
// lane holds the combination of itself and its partner, so after all six
// every lane holds the value of the whole wave.
template <int kCtrl>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return __builtin_amdgcn_update_dpp(0u, v, kCtrl, 0xf, 0xf, false);
}
constexpr int kQuadSwap1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

// (hi, lo) lexicographic max
__device__ __forceinline__ void max_pair(uint32_t& hi, uint32_t& lo, uint32_t ohi, uint32_t olo) {
  const bool take = (ohi > hi) || (ohi == hi && olo > lo);
  hi = take ? ohi : hi;
  lo = take ? olo : lo;
}

__device__ __forceinline__ void wave_max_pair(uint32_t& hi, uint32_t& lo) {
  max_pair(hi, lo, dpp<kQuadSwap1>(hi), dpp<kQuadSwap1>(lo));
  max_pair(hi, lo, dpp<kQuadSwap2>(hi), dpp<kQuadSwap2>(lo));
  max_pair(hi, lo, dpp<kRowHalfMirror>(hi), dpp<kRowHalfMirror>(lo));
  max_pair(hi, lo, dpp<kRowMirror>(hi), dpp<kRowMirror>(lo));
  {  // rows 0<->1, 2<->3: one of the two results is this lane's own value
    const auto h = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    const auto l = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    hi = h[0]; lo = l[0];
    max_pair(hi, lo, h[1], l[1]);
  }
  {  // halves 0-31 <-> 32-63
    const auto h = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    const auto l = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
    hi = h[0]; lo = l[0];
    max_pair(hi, lo, h[1], l[1]);
  }
}

__device__ __forceinline__ float wave_sum(float v) {
  v += __uint_as_float(dpp<kQuadSwap1>(__float_as_uint(v)));
  v += __uint_as_float(dpp<kQuadSwap2>(__float_as_uint(v)));
  v += __uint_as_float(dpp<kRowHalfMirror>(__float_as_uint(v)));
  v += __uint_as_float(dpp<kRowMirror>(__float_as_uint(v)));
  {
    const auto h = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(h[0]) + __uint_as_float(h[1]);
  }
  {
    const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(h[0]) + __uint_as_float(h[1]);
  }
  return v;
}

// One wave routes token t. Lane l holds logits l, l+64, ... (VPL of them).
// Candidates compare as (key << 32) | ~e, so equal logits prefer the lower e.
__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint32_t umin(uint32_t a, uint32_t b) { return a < b ? a : b; }

// Wave-wide max / min of a 32-bit value, every lane gets the result.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = umax(v, dpp<kQuadSwap1>(v));
  v = umax(v, dpp<kQuadSwap2>(v));
  v = umax(v, dpp<kRowHalfMirror>(v));
  v = umax(v, dpp<kRowMirror>(v));
  const auto h = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = umax(h[0], h[1]);
  const auto g = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return umax(g[0], g[1]);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = umin(v, dpp<kQuadSwap1>(v));
  v = umin(v, dpp<kQuadSwap2>(v));
  v = umin(v, dpp<kRowHalfMirror>(v));
  v = umin(v, dpp<kRowMirror>(v));
  const auto h = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = umin(h[0], h[1]);
  const auto g = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return umin(g[0], g[1]);
}

// One wave's routing state for a token: lane l holds the order keys of
// experts l, l+64, ... (VPL of them); 0 = absent or already taken. The VPL
// loads are unconditional (indices past E read expert E - 1, then drop it),
// so they go out together: as conditional loads each became a branch with a
// wait for every load in flight, VPL round trips one after another.
template <int VPL>
__device__ __forceinline__ void topk_load(const float* __restrict__ row, int E, float (&x)[VPL]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    const int e = v * 64 + lane;
    x[v] = row[e < E ? e : E - 1];
  }
}
template <int VPL>
__device__ __forceinline__ void topk_keys_of(const float (&x)[VPL], int E, uint32_t (&key)[VPL]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int v = 0; v < VPL; ++v) key[v] = (v * 64 + lane < E) ? order_key(x[v]) : 0u;
}
template <int VPL>
__device__ __forceinline__ void topk_keys(const float* __restrict__ row, int E, uint32_t (&key)[VPL]) {
  float x[VPL];
  topk_load<VPL>(row, E, x);
  topk_keys_of<VPL>(x, E, key);
}

// Takes the largest remaining key (equal keys: the lower expert index) and
// returns its expert, the same in every lane; its key becomes 0. Each lane
// offers its largest key (strict comparison: the lowest v, i.e. the lowest
// expert, among equal ones), the wave maximum picks the key (a few
// cross-lane steps), and a ballot finds the lanes offering it: between lanes
// the lower expert index wins.
template <int VPL>
__device__ __forceinline__ int topk_take(uint32_t (&key)[VPL], uint32_t& taken_key) {
  const int lane = threadIdx.x & 63;
  uint32_t lm = key[0];
  int lv = 0;
#pragma unroll
  for (int v = 1; v < VPL; ++v) {
    const bool gt = key[v] > lm;
    lm = gt ? key[v] : lm;
    lv = gt ? v : lv;
  }
  const uint32_t m = wave_max_u32(lm);
  const uint32_t le = (uint32_t)(lv * 64 + lane);
  unsigned long long hold = __ballot(lm == m);
  if (__builtin_popcountll(hold) > 1) {  // equal logits in several lanes
    const uint32_t emin = wave_min_u32(lm == m ? le : 0xFFFFFFFFu);
    hold = __ballot(lm == m && le == emin);
  }
  const int wl = __builtin_ctzll(hold);
  const int we = __builtin_amdgcn_readlane((int)le, wl);
#pragma unroll
  for (int v = 0; v < VPL; ++v) key[v] = (lane == wl && v == lv) ? 0u : key[v];
  taken_key = m;
  return we;
}

// Set bits of m in the lanes below this one.
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Routes token t with one wave: `rounds` takes (k for the full routing), and
// the expert of take number `slot` is returned. With out_ids non-null the
// routing is complete (rounds = k) and lanes < k write expert and weight of
// their slot: weights = softmax over the k kept logits. (Each wave that
// needs only slot s stops after s + 1 takes.)
// The keys may be passed in (topk_keys or topk_load + topk_keys_of of row t).
template <int VPL>
__device__ __forceinline__ int topk_route_keys(uint32_t (&key)[VPL], int t, int k, int rounds, int slot,
                                               int32_t* __restrict__ out_ids, float* __restrict__ out_w,
                                               int32_t* ids_copy = nullptr) {
  const int lane = threadIdx.x & 63;
  uint32_t my_key = 0;
  int my_e = 0, e_slot = 0;
  for (int r = 0; r < rounds; ++r) {
    uint32_t m;
    const int we = topk_take<VPL>(key, m);
    e_slot = (r == slot) ? we : e_slot;
    if (lane == r) {
      my_key = m;
      my_e = we;
    }
  }
  if (out_ids) {
    const float l0 = key_value(__builtin_amdgcn_readfirstlane(my_key));
    const float exv = (lane < k) ? expf(key_value(my_key) - l0) : 0.0f;
    const float sum = wave_sum(exv);
    if (lane < k) {
      out_ids[(int64_t)t * k + lane] = my_e;
      out_w[(int64_t)t * k + lane] = exv / sum;
      if (ids_copy) ids_copy[t * k + lane] = my_e;
    }
  }
  return e_slot;
}
template <int VPL>
__device__ __forceinline__ int topk_route(const float* __restrict__ logits, int t, int E, int k, int rounds,
                                          int slot, int32_t* __restrict__ out_ids, float* __restrict__ out_w,
                                          int32_t* ids_copy = nullptr) {
  uint32_t key[VPL];
  topk_keys<VPL>(logits + (int64_t)t * E, E, key);
  return topk_route_keys<VPL>(key, t, k, rounds, slot, out_ids, out_w, ids_copy);
}

// One wave routes token t completely: topk_ids / topk_w [t*k + j] for j < k.
template <int VPL>
__device__ __forceinline__ void topk_token(const float* __restrict__ logits, int t, int E, int k,
                                           int32_t* __restrict__ topk_ids, float* __restrict__ topk_w,
                                           int32_t* ids_copy = nullptr) {
  topk_route<VPL>(logits, t, E, k, k, 0, topk_ids, topk_w, ids_copy);
}

// ---------------------------------------------------------------------------
// Routing and grouping of a small batch inside one workgroup (M <= 16,
// M*k <= 256, E <= 1024). Waves 0..M-1 route one token each; a bitmap of the
// touched experts in LDS ranks them. Top-k experts are distinct within a
// token, so no expert gets more than M <= 16 rows: every touched expert is
// exactly one block of any block_m >= 16, the blocks are the touched experts
// in ascending order, and a block's rows are that expert's assignments in
// ascending f (the stable per-expert order of the grouping).
constexpr int kSmallMaxTokens = 16;
constexpr int kSmallMaxAssign = 256;
constexpr int kSmallMaxExperts = 1024;

struct SmallRoute {
  int32_t ids[kSmallMaxAssign];                   // topk ids, f = t*k + j
  float wts[kSmallMaxAssign];                     // topk weights
  uint32_t bits[kSmallMaxExperts / 32];           // touched experts
  int32_t before[kSmallMaxExperts / 32 + 1];      // touched experts in the words below
  int32_t blk_e[kSmallMaxAssign];                 // expert of block r (rank r)
  int32_t blk_rows[kSmallMaxAssign][kSmallMaxTokens];  // rows of block r, then M*k
};

// Touched experts below x.
__device__ __forceinline__ int small_rank(const SmallRoute& sh, int x) {
  const int w = x >> 5, b = x & 31;
  return sh.before[w] + __builtin_popcount(sh.bits[w] & ((1u << b) - 1u));
}

// Fills sh for the batch; returns the number of touched experts (= blocks).
// Every thread of the workgroup (kThreads, at least 64 * M) must call it:
// it contains barriers.
template <int VPL, int kThreads>
__device__ int small_route(SmallRoute& sh, const float* __restrict__ logits, int M, int E, int k) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int MK = M * k, nwords = (E + 31) / 32;
  if (tid < nwords) sh.bits[tid] = 0u;
  if (wave < M) topk_token<VPL>(logits, wave, E, k, sh.ids, sh.wts);
  __syncthreads();
  for (int f = tid; f < MK; f += kThreads) atomicOr(&sh.bits[sh.ids[f] >> 5], 1u << (sh.ids[f] & 31));
  __syncthreads();
  if (wave == 0) {  // exclusive prefix of the words' popcounts (nwords <= 32)
    const int c = lane < nwords ? __builtin_popcount(sh.bits[lane]) : 0;
    int incl = c;
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) {
      const int t = __shfl_up(incl, o, 64);
      if (lane >= o) incl += t;
    }
    if (lane < nwords) sh.before[lane] = incl - c;
    if (lane == nwords - 1) sh.before[nwords] = incl;
  }
  __syncthreads();
  // (the same value in every lane: readfirstlane keeps loop counts scalar)
  const int nd = __builtin_amdgcn_readfirstlane(sh.before[nwords]);
  for (int x = tid; x < E; x += kThreads)
    if ((sh.bits[x >> 5] >> (x & 31)) & 1u) sh.blk_e[small_rank(sh, x)] = x;
  __syncthreads();
  // rows of each block: one ballot per 64 assignments, positions by lane rank
  for (int b = wave; b < nd; b += kThreads / 64) {
    const int e = sh.blk_e[b];
    int base = 0;
    for (int f0 = 0; f0 < MK; f0 += 64) {
      const int f = f0 + lane;
      const bool hit = f < MK && sh.ids[f] == e;
      const uint64_t hm = __ballot(hit);
      if (hit) sh.blk_rows[b][base + lanes_below(hm)] = f;
      base += __builtin_popcountll(hm);
    }
    if (lane >= base && lane < kSmallMaxTokens) sh.blk_rows[b][lane] = MK;
  }
  __syncthreads();
  return nd;
}

// The routing and grouping outputs exactly as moe_route_align lays them out
// for block_m = bm >= 16 (any threads of one workgroup, no barrier):
// topk_ids / topk_weights [M*k], sorted_ids [nd*bm], block_expert [nd],
// offsets [E+1], npp [1].
template <int kThreads>
__device__ void small_route_write(const SmallRoute& sh, int nd, int M, int E, int k, int bm,
                                  int32_t* __restrict__ topk_ids, float* __restrict__ topk_w,
                                  int32_t* __restrict__ sorted_ids, int32_t* __restrict__ block_expert,
                                  int32_t* __restrict__ offsets, int32_t* __restrict__ npp) {
  const int tid = threadIdx.x, MK = M * k;
  for (int f = tid; f < MK; f += kThreads) {
    topk_ids[f] = sh.ids[f];
    topk_w[f] = sh.wts[f];
  }
  for (int i = tid; i < nd * bm; i += kThreads) {
    const int b = i / bm, p = i % bm;
    sorted_ids[i] = p < kSmallMaxTokens ? sh.blk_rows[b][p] : MK;
  }
  for (int b = tid; b < nd; b += kThreads) block_expert[b] = sh.blk_e[b];
  for (int x = tid; x <= E; x += kThreads) offsets[x] = bm * (x < E ? small_rank(sh, x) : nd);
  if (tid == 0) *npp = bm * nd;
}

}  // namespace moe

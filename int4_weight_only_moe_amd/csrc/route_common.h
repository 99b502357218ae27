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
template <int VPL>
__device__ void topk_token(const float* __restrict__ logits, int t, int E, int k,
                           int32_t* __restrict__ topk_ids, float* __restrict__ topk_w,
                           int32_t* ids_copy = nullptr) {
  const int lane = threadIdx.x & 63;
  // Candidates as (key << 32 | ~e): larger means larger logit, then smaller
  // expert; 0 means none. Each lane sorts its VPL candidates once; every
  // round takes the wave maximum of the lane heads and the winning lane (the
  // candidates are unique) drops its head.
  uint64_t c[VPL];
  const float* row = logits + (int64_t)t * E;
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    const int e = v * 64 + lane;
    c[v] = (e < E) ? (((uint64_t)order_key(row[e]) << 32) | (uint32_t)~(uint32_t)e) : 0ull;
  }
#pragma unroll
  for (int i = 1; i < VPL; ++i) {
#pragma unroll
    for (int j = i; j > 0; --j) {
      const uint64_t hi = c[j] > c[j - 1] ? c[j] : c[j - 1];
      const uint64_t lo = c[j] > c[j - 1] ? c[j - 1] : c[j];
      c[j - 1] = hi;
      c[j] = lo;
    }
  }
  uint64_t mine = 0;
  for (int r = 0; r < k; ++r) {
    uint32_t bhi = (uint32_t)(c[0] >> 32), blo = (uint32_t)c[0];
    wave_max_pair(bhi, blo);
    const uint64_t best = ((uint64_t)bhi << 32) | blo;
    const bool won = c[0] == best;
#pragma unroll
    for (int v = 0; v < VPL; ++v) c[v] = won ? (v + 1 < VPL ? c[v + 1] : 0ull) : c[v];
    if (lane == r) mine = best;
  }
  const uint32_t my_key = (uint32_t)(mine >> 32);
  const int my_e = (int)~(uint32_t)mine;
  const float l0 = key_value(__builtin_amdgcn_readfirstlane(my_key));
  const float ex = (lane < k) ? expf(key_value(my_key) - l0) : 0.0f;
  const float sum = wave_sum(ex);
  if (lane < k) {
    topk_ids[(int64_t)t * k + lane] = my_e;
    topk_w[(int64_t)t * k + lane] = ex / sum;
    if (ids_copy) ids_copy[t * k + lane] = my_e;
  }
}

}  // namespace moe

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

template <int VPL>
__device__ __forceinline__ void topk_token(const float* __restrict__ logits, int t, int E, int k,
                           int32_t* __restrict__ topk_ids, float* __restrict__ topk_w,
                           int32_t* ids_copy = nullptr) {
  const int lane = threadIdx.x & 63;
  // Lane l holds experts l, l+64, ...: keys (0 = none) sorted descending with
  // their expert index, equal keys keeping ascending expert order. Each round
  // takes the wave maximum of the lane heads (32-bit: a few cross-lane
  // steps); a ballot finds the lane holding it, ties between lanes go to the
  // smallest expert index; that lane drops its head.
  uint32_t key[VPL], ex[VPL];
  const float* row = logits + (int64_t)t * E;
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    const int e = v * 64 + lane;
    key[v] = (e < E) ? order_key(row[e]) : 0u;
    ex[v] = (uint32_t)e;
  }
#pragma unroll
  for (int i = 1; i < VPL; ++i) {
#pragma unroll
    for (int j = i; j > 0; --j) {
      const bool sw = key[j] > key[j - 1];  // strict: equal keys keep ascending e
      const uint32_t k0 = sw ? key[j] : key[j - 1], k1 = sw ? key[j - 1] : key[j];
      const uint32_t e0 = sw ? ex[j] : ex[j - 1], e1 = sw ? ex[j - 1] : ex[j];
      key[j - 1] = k0; key[j] = k1; ex[j - 1] = e0; ex[j] = e1;
    }
  }
  uint32_t my_key = 0, my_e = 0;
  for (int r = 0; r < k; ++r) {
    const uint32_t m = wave_max_u32(key[0]);
    unsigned long long hold = __ballot(key[0] == m);
    if (__builtin_popcountll(hold) > 1) {  // equal logits in several lanes
      const uint32_t emin = wave_min_u32(key[0] == m ? ex[0] : 0xFFFFFFFFu);
      hold = __ballot(key[0] == m && ex[0] == emin);
    }
    const int wl = __builtin_ctzll(hold);
    const uint32_t we = __builtin_amdgcn_readlane(ex[0], wl);
    if (lane == wl) {
#pragma unroll
      for (int v = 0; v + 1 < VPL; ++v) {
        key[v] = key[v + 1];
        ex[v] = ex[v + 1];
      }
      key[VPL - 1] = 0u;
    }
    if (lane == r) {
      my_key = m;
      my_e = we;
    }
  }
  const float l0 = key_value(__builtin_amdgcn_readfirstlane(my_key));
  const float exv = (lane < k) ? expf(key_value(my_key) - l0) : 0.0f;
  const float sum = wave_sum(exv);
  if (lane < k) {
    topk_ids[(int64_t)t * k + lane] = (int)my_e;
    topk_w[(int64_t)t * k + lane] = exv / sum;
    if (ids_copy) ids_copy[t * k + lane] = (int)my_e;
  }
}

}  // namespace moe

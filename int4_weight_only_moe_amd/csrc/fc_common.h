// Device pieces shared by the grouped-GEMM kernels: raw buffer loads (an
// offset past the end of the buffer reads zeros without touching memory), the
// per-lane view of one chunk of a tile pair, and the MFMA step of one chunk.
#pragma once

#include "internal.h"
#include "device_common.h"

namespace moe {
namespace MOE_FMT_NS {

constexpr uint32_t kNeg136Pair = 0xC308C308u;  // two bf16 -136.0
constexpr uint32_t kOutOfRange = 0x80000000u;  // buffer offset that reads zeros
constexpr int kChunkXBytes = kChunkK * 2;      // one row's bf16 slice of a chunk

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // dword3 0x00020000: 32-bit data format, raw (unswizzled) addressing
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// Cache policy of a load (the buffer instruction's cache bits; on gfx950 bit 1
// is "nt", non-temporal). The weights are a stream read once per call: with
// nt they do not push reused lines (activations) out of the caches, and a
// plain streaming read of 132 MB runs ~12% faster with it than without.
#ifndef MOE_WEIGHT_CACHE_POLICY
#define MOE_WEIGHT_CACHE_POLICY 2
#endif
constexpr int kPolicyDefault = 0;
constexpr int kPolicyWeights = MOE_WEIGHT_CACHE_POLICY;

template <int kPolicy = kPolicyDefault>
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kPolicy);
  return make_uint4(v.x, v.y, v.z, v.w);
}
template <int kPolicy = kPolicyDefault>
__device__ __forceinline__ uint2 bload8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, kPolicy);
  return make_uint2(v.x, v.y);
}

// -136 times the sum of the 32 bf16 values a quad of lanes holds (8 per
// lane: one quantisation group when lanes 4q..4q+3 hold the group's four
// 16-byte vectors). It is the accumulator input that turns the MFMA of x
// with (q + 136) into the MFMA of x with q. Every lane of the quad gets it;
// the four lanes must all be active.
__device__ __forceinline__ float group_corr_quad(uint4 v) {
  const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) sum += __uint_as_float(w4[i] << 16) + __uint_as_float(w4[i] & 0xFFFF0000u);
  sum += __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(sum), 0xB1, 0xf, 0xf, false));
  sum += __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(sum), 0x4E, 0xf, 0xf, false));
  return -136.0f * sum;
}

template <int kPolicy = kPolicyDefault>
__device__ __forceinline__ uint32_t bload4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, kPolicy);
}

// Format-dependent pieces of a group's product. A tile row's 4 group scales
// take kScaleRowBytes (fp16: 8, E8M0: 4) at kTileNibbleBytes + row * that.
constexpr uint32_t kScaleRowBytes = kTileScaleBytes / kTileRows;
template <int kPolicy = kPolicyDefault>
__device__ __forceinline__ uint2 load_scales(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (kFmt == kFmtMxfp4)
    return make_uint2(bload4<kPolicy>(r, off), 0u);
  else
    return bload8<kPolicy>(r, off);
}
// Scale of group j (0..3) from a row's loaded scales: the fp16 value, or the
// E8M0 byte placed in an fp32 exponent field (the form dequant_fp4 takes).
__device__ __forceinline__ float group_scale(uint2 sw, int j) {
  if constexpr (kFmt == kFmtMxfp4)
    return __uint_as_float(((sw.x >> (8 * j)) & 0xFFu) << 23);
  else
    return f16_bits_to_f32(((j < 2 ? sw.x : sw.y) >> (16 * (j & 1))) & 0xFFFFu);
}
// The B operand of one group (8 codes of one dword): INT4 as q + 136 (the
// scale is applied to the MFMA result), FP4 already scaled (exact).
__device__ __forceinline__ bf16x8_t dequant_group(uint32_t q, float scale) {
  if constexpr (kFmt == kFmtMxfp4)
    return dequant_fp4(q, scale);
  else
    return dequant_u4_plus128(q);
}
// The MFMA accumulator input of a group: INT4 needs -136 * sum(x); FP4 codes
// carry no offset.
__device__ __forceinline__ f32x4_t group_c(f32x4_t corr) {
  if constexpr (kFmt == kFmtMxfp4)
    return f32x4_t{0.f, 0.f, 0.f, 0.f};
  else
    return corr;
}
// A running sum plus one group's MFMA result t: scaled by the group scale
// (INT4) or as is (FP4: the scale is in the B operand).
__device__ __forceinline__ float group_add(float acc, float t, float g) {
  if constexpr (kFmt == kFmtMxfp4)
    return acc + t;
  else
    return __builtin_fmaf(t, g, acc);
}

struct WChunk {
  uint4 q0, q1;  // codes of the two tiles of a pair, 16 B per lane each
  uint2 s0, s1;  // the 4 group scales of row (lane % 16) of each tile (E8M0: in s.x)
};

// One chunk = 4 groups: per group, widen both tiles' codes, then per active
// sub-tile one MFMA for -136*sum(x) and one per tile, scaled into the sums.
template <int S>
__device__ __forceinline__ void mma_chunk(const WChunk& w, const uint4 (&xa)[S][4], const bool (&sact)[S],
                                          const bf16x8_t neg136, f32x4_t (&acc0)[S], f32x4_t (&acc1)[S]) {
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
  const uint32_t q0[4] = {w.q0.x, w.q0.y, w.q0.z, w.q0.w};
  const uint32_t q1[4] = {w.q1.x, w.q1.y, w.q1.z, w.q1.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float g0 = group_scale(w.s0, j);
    const float g1 = group_scale(w.s1, j);
    const bf16x8_t b0 = dequant_group(q0[j], g0);
    const bf16x8_t b1 = dequant_group(q1[j], g1);
#pragma unroll
    for (int s = 0; s < S; ++s) {
      if (s > 0 && !sact[s]) continue;  // sub-tile 0 always holds a row
      const bf16x8_t xv = as_bf16x8(xa[s][j]);
      if constexpr (kFmt == kFmtMxfp4) {  // scaled operand: accumulate in the MFMA
        acc0[s] = mfma16x16x32(xv, b0, acc0[s]);
        acc1[s] = mfma16x16x32(xv, b1, acc1[s]);
        continue;
      }
      const f32x4_t off = group_c(mfma16x16x32(xv, neg136, zero4));
      const f32x4_t t0 = mfma16x16x32(xv, b0, off);
      const f32x4_t t1 = mfma16x16x32(xv, b1, off);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc0[s][i] = group_add(acc0[s][i], t0[i], g0);
        acc1[s][i] = group_add(acc1[s][i], t1[i], g1);
      }
    }
  }
}

// Epilogue of a workgroup's tile pair for the rows frow of its block:
// FC1 stores act_f = bf16(SiLU(gate) * up); FC2 adds w_f * y_f into the fp32
// accumulator with atomics. Lane l holds D rows 4*(l/16)+i, column l % 16.
template <int S, bool kFc1>
__device__ __forceinline__ void fc_epilogue(const FcArgs& a, const int pair, const int (&frow)[S],
                                            const bool (&sact)[S], const f32x4_t (&acc0)[S],
                                            const f32x4_t (&acc1)[S], const int lane) {
  const int MK = a.M * a.k;
  // recomputed here rather than kept live across the main loop
  const int col = (int)__lane_id() & 15;
  if constexpr (kFc1) {
    const int I = a.I;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      if (!sact[s]) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int f = __shfl(frow[s], 4 * (lane >> 4) + i, 64);
        if (f < 0 || f >= MK) continue;
        const float g = acc0[s][i], u = acc1[s][i];
        const float v = g / (1.0f + __expf(-g)) * u;
        a.act_out[(int64_t)f * I + 16 * pair + col] = (uint16_t)f32_to_bf16_bits(v);
      }
    }
  } else {
    const int H = a.H;
    const int c0 = kPairRows * pair;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      if (!sact[s]) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int f = __shfl(frow[s], 4 * (lane >> 4) + i, 64);
        if (f < 0 || f >= MK) continue;
        const int t = f / a.k;
        const float w = a.topk_weights[f];
        float* dst = a.acc + (int64_t)t * H + c0;
        unsafeAtomicAdd(dst + col, w * acc0[s][i]);
        unsafeAtomicAdd(dst + 16 + col, w * acc1[s][i]);
      }
    }
  }
}


// The work of one workgroup: block rows frow (per sub-tile, this lane's row
// lane % 16; entries outside [0, M*k) are padding) of expert e times tile
// pair `pair`, K split over the KSPLIT waves, then the FC1 or FC2 epilogue.
template <int S, int KSPLIT, int P, int NCH, bool kFc1>
__device__ __forceinline__ void fc_block(const FcArgs& a, const int e, const int pair, const int (&frow)[S],
                                         const int wave, const int lane) {
  const int K = kFc1 ? a.H : a.I;
  const int N = kFc1 ? 2 * a.I : a.H;
  const int MK = a.M * a.k;
  const int nkc = K / kChunkK;
  const int kc0 = wave * nkc / KSPLIT;
  // chunks of this wave: NCH when the launcher knows it (then the chunk loop
  // is unrolled into straight-line code), else computed at run time
  const int n = NCH > 0 ? NCH : (wave + 1) * nkc / KSPLIT - kc0;

  // Activation rows: lane's A-operand row is (lane % 16) of each sub-tile.
  const int rows_total = kFc1 ? a.M : MK;
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.act_in, (uint32_t)rows_total * (uint32_t)K * 2u);
  uint32_t xoff[S];
  bool sact[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int f = frow[s];
    const bool valid = (f >= 0) && (f < MK);
    const uint32_t r = valid ? (uint32_t)(kFc1 ? f / a.k : f) : 0u;
    xoff[s] = valid ? (r * (uint32_t)K + 8u * (lane >> 4) + (uint32_t)kc0 * kChunkK) * 2u : kOutOfRange;
    sact[s] = __builtin_amdgcn_readfirstlane(f) < MK;  // lane 0 holds row 16*s
  }

  const uint8_t* wbase = a.wpacked + (int64_t)e * packed_bytes_per_expert(N, K) +
                         ((int64_t)pair * nkc + kc0) * kPairChunkBytes;
  const uint32_t oq0 = 16u * lane, oq1 = kTileBytes + 16u * lane;
  const uint32_t os0 = kTileNibbleBytes + kScaleRowBytes * (lane & 15);
  const uint32_t os1 = kTileBytes + kTileNibbleBytes + kScaleRowBytes * (lane & 15);

  // One buffer descriptor per chunk (scalar arithmetic), so the per-lane
  // offsets stay four constant registers; a chunk at or past n has no bytes
  // in range and reads zeros.
  auto load_w = [&](int c) {
    const __amdgpu_buffer_rsrc_t wr =
        make_rsrc(wbase + (int64_t)c * kPairChunkBytes, c < n ? (uint32_t)kPairChunkBytes : 0u);
    WChunk w;
    w.q0 = bload16<kPolicyWeights>(wr, oq0);
    w.q1 = bload16<kPolicyWeights>(wr, oq1);
    w.s0 = load_scales<kPolicyWeights>(wr, os0);
    w.s1 = load_scales<kPolicyWeights>(wr, os1);
    return w;
  };
  auto load_x = [&](uint4 (&xa)[S][4], int c) {
    const uint32_t cb = (uint32_t)c * kChunkXBytes;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const uint32_t o = (c < n) ? xoff[s] + cb : kOutOfRange;
#pragma unroll
      for (int j = 0; j < 4; ++j) xa[s][j] = bload16(xr, o + 64u * j);
    }
  };

  const bf16x8_t neg136 = as_bf16x8(make_uint4(kNeg136Pair, kNeg136Pair, kNeg136Pair, kNeg136Pair));
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
  f32x4_t acc0[S], acc1[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    acc0[s] = zero4;
    acc1[s] = zero4;
  }

  // Ring of P chunks in flight: chunk c is loaded P steps before it is used.
  WChunk wb[P];
  uint4 xb[P][S][4];
#pragma unroll
  for (int j = 0; j < P; ++j) {
    wb[j] = load_w(j);
    load_x(xb[j], j);
  }
  if constexpr (NCH > 0) {
    // Straight-line: the compiler's memory-wait placement is exact here,
    // while a loop back-edge makes it wait for every load in flight.
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      mma_chunk<S>(wb[c % P], xb[c % P], sact, neg136, acc0, acc1);
      if (c + P < NCH) {
        wb[c % P] = load_w(c + P);
        load_x(xb[c % P], c + P);
      }
      __builtin_amdgcn_sched_barrier(0);  // bound live ranges to one chunk
    }
  } else {
    for (int c = 0; c < n; c += P) {
#pragma unroll
      for (int j = 0; j < P; ++j) {
        if (c + j < n) mma_chunk<S>(wb[j], xb[j], sact, neg136, acc0, acc1);
        wb[j] = load_w(c + j + P);
        load_x(xb[j], c + j + P);
      }
    }
  }

  // Sum the K-split partials in LDS.
  if constexpr (KSPLIT > 1) {
    __shared__ f32x4_t red[KSPLIT - 1][S][2][64];
    if (wave > 0) {
#pragma unroll
      for (int s = 0; s < S; ++s) {
        red[wave - 1][s][0][lane] = acc0[s];
        red[wave - 1][s][1][lane] = acc1[s];
      }
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 0; w < KSPLIT - 1; ++w) {
#pragma unroll
      for (int s = 0; s < S; ++s) {
        acc0[s] += red[w][s][0][lane];
        acc1[s] += red[w][s][1][lane];
      }
    }
  }

  fc_epilogue<S, kFc1>(a, pair, frow, sact, acc0, acc1, lane);
}


}  // namespace MOE_FMT_NS
}  // namespace moe

// FC1 (gate/up + SiLU*mul) and FC2 (+ routing-weighted combine) of the
// weight-only INT4 MoE layer on the gfx950 bf16 matrix cores.
//
// "The Throughput Lever: Quantifying the MoE GEMM and Mapping the Road to
// B300", sections "Phase 3: The INT4 Marlin MoE Throughput Lever" and "The
// Result: Two Regimes": the layer is a grouped GEMM whose cost is streaming
// the INT4 weights of the experts the batch touches; the DDTree page ("From
// PCIe to NVLink: The DDTree Deployment Journey", part V, priority 2) asks
// for the INT4 dequantisation fused into the MoE GEMM. Here the nibbles are
// widened in registers and fed straight to v_mfma_f32_16x16x32_bf16.
//
// Work decomposition (one workgroup = one block of block_m rows of one
// expert x one pair of 16-row weight tiles):
//   * the KSPLIT waves of a workgroup split the K range; each streams its
//     share of the pair's tiles (one 16-byte load per lane per tile) and the
//     activation slices of the block's rows (they are reused from L2);
//   * both streams go through a ring of P chunks in registers, issued with
//     raw buffer loads: an offset past the end of the buffer returns zeros
//     without touching memory, so padding rows and the ring's overrun need
//     no branch and the compiler can wait for exactly the chunk it uses;
//   * one MFMA covers exactly one quantisation group (32 channels): the
//     weights enter as q + 136 (see dequant_u4_plus128), an extra MFMA with
//     a constant -136 operand supplies -136 * sum(x) as the accumulator input,
//     and the group scale is applied to the fp32 MFMA result (scale after
//     the product, so the weights are never rounded);
//   * partial sums of the waves meet in LDS; wave 0 runs the epilogue.
// FC1 epilogue: act_f = bf16(SiLU(gate) * up); gate and up of one output
// column land in the same lane because a pair is (gate tile r, up tile r).
// FC2 epilogue: acc[t] += w_f * y_f with fp32 atomics into a workspace
// accumulator that FC1 clears; a last small kernel rounds acc to bf16 once.
// (A "last arriving workgroup converts" scheme needs agent-scope fences, and
// on gfx950 each of those writes back and invalidates the L2.)
#include "internal.h"
#include "device_common.h"

namespace moe {
namespace {

constexpr uint32_t kNeg136Pair = 0xC308C308u;  // two bf16 -136.0
constexpr uint32_t kOutOfRange = 0x80000000u;  // buffer offset that reads zeros
constexpr int kChunkXBytes = kChunkK * 2;      // one row's bf16 slice of a chunk

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // dword3 0x00020000: 32-bit data format, raw (unswizzled) addressing
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 bload8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
  return make_uint2(v.x, v.y);
}

struct WChunk {
  uint4 q0, q1;  // nibbles of the two tiles of a pair, 16 B per lane each
  uint2 s0, s1;  // the 4 group scales of row (lane % 16) of each tile
};

// One chunk = 4 groups: per group, widen both tiles' codes, then per active
// sub-tile one MFMA for -136*sum(x) and one per tile, scaled into the sums.
template <int S>
__device__ __forceinline__ void mma_chunk(const WChunk& w, const uint4 (&xa)[S][4], const bool (&sact)[S],
                                          const bf16x8_t neg136, f32x4_t (&acc0)[S], f32x4_t (&acc1)[S]) {
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
  const uint32_t q0[4] = {w.q0.x, w.q0.y, w.q0.z, w.q0.w};
  const uint32_t q1[4] = {w.q1.x, w.q1.y, w.q1.z, w.q1.w};
  const uint32_t s0w[2] = {w.s0.x, w.s0.y};
  const uint32_t s1w[2] = {w.s1.x, w.s1.y};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const bf16x8_t b0 = dequant_u4_plus128(q0[j]);
    const bf16x8_t b1 = dequant_u4_plus128(q1[j]);
    const float g0 = f16_bits_to_f32((s0w[j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
    const float g1 = f16_bits_to_f32((s1w[j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
#pragma unroll
    for (int s = 0; s < S; ++s) {
      if (s > 0 && !sact[s]) continue;  // sub-tile 0 always holds a row
      const bf16x8_t xv = as_bf16x8(xa[s][j]);
      const f32x4_t off = mfma16x16x32(xv, neg136, zero4);
      const f32x4_t t0 = mfma16x16x32(xv, b0, off);
      const f32x4_t t1 = mfma16x16x32(xv, b1, off);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc0[s][i] = __builtin_fmaf(t0[i], g0, acc0[s][i]);
        acc1[s][i] = __builtin_fmaf(t1[i], g1, acc1[s][i]);
      }
    }
  }
}

template <int S, int KSPLIT, int P, int NCH, bool kFc1>
__global__ __launch_bounds__(64 * KSPLIT) __attribute__((amdgpu_waves_per_eu(S == 1 ? 4 : 1)))
void fc_kernel(FcArgs a) {
  constexpr int kThreads = 64 * KSPLIT;
  const int lane = threadIdx.x & 63;
  // wave index, blocks, experts and chunk ranges are wave-uniform: keep them
  // in scalar registers so the buffer descriptors built from them are too
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int K = kFc1 ? a.H : a.I;
  const int N = kFc1 ? 2 * a.I : a.H;
  const int npairs = N / kPairRows;
  const int MK = a.M * a.k;

  if constexpr (kFc1) {
    // Clear FC2's fp32 accumulator (the start of the workspace), spread over
    // every workgroup of the grid.
    uint4* z = reinterpret_cast<uint4*>(a.acc);
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < a.zero_words16; i += stride)
      z[i] = make_uint4(0, 0, 0, 0);
  }

  const int pair = blockIdx.x % npairs;
  const int blk = blockIdx.x / npairs;
  // The three loads a workgroup starts with do not depend on each other:
  // issue them together (the row ids of blocks past the end are never used).
  const int32_t* rows = a.sorted_ids + (int64_t)blk * 16 * S;
  int frow[S];
#pragma unroll
  for (int s = 0; s < S; ++s) frow[s] = rows[16 * s + (lane & 15)];
  const int npp = __builtin_amdgcn_readfirstlane(*a.npp);
  const int e = __builtin_amdgcn_readfirstlane(a.block_expert[blk]);
  if (blk * 16 * S >= npp) return;
  if (e < 0 || e >= a.E) return;

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
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(wbase, (uint32_t)n * kPairChunkBytes);
  const uint32_t oq0 = 16u * lane, oq1 = kTileBytes + 16u * lane;
  const uint32_t os0 = kTileNibbleBytes + 8u * (lane & 15), os1 = kTileBytes + kTileNibbleBytes + 8u * (lane & 15);

  auto load_w = [&](int c) {
    const uint32_t base = (uint32_t)c * kPairChunkBytes;  // past n: reads zeros
    WChunk w;
    w.q0 = bload16(wr, base + oq0);
    w.q1 = bload16(wr, base + oq1);
    w.s0 = bload8(wr, base + os0);
    w.s1 = bload8(wr, base + os1);
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

  const int col = lane & 15;
  if constexpr (kFc1) {
    const int I = a.I;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      if (!sact[s]) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int f = rows[16 * s + 4 * (lane >> 4) + i];
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
        const int f = rows[16 * s + 4 * (lane >> 4) + i];
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

// out = bf16(acc), 8 values per thread.
__global__ __launch_bounds__(256) void finalize_kernel(const float* __restrict__ acc, uint16_t* __restrict__ out,
                                                       int64_t n8) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const float4 a = reinterpret_cast<const float4*>(acc)[2 * i];
  const float4 b = reinterpret_cast<const float4*>(acc)[2 * i + 1];
  uint4 o;
  o.x = f32_to_bf16_bits(a.x) | (f32_to_bf16_bits(a.y) << 16);
  o.y = f32_to_bf16_bits(a.z) | (f32_to_bf16_bits(a.w) << 16);
  o.z = f32_to_bf16_bits(b.x) | (f32_to_bf16_bits(b.y) << 16);
  o.w = f32_to_bf16_bits(b.z) | (f32_to_bf16_bits(b.w) << 16);
  reinterpret_cast<uint4*>(out)[i] = o;
}

// Chunks per wave the unrolled variants are built for: the 384-expert
// layer (hidden 7168 = 56 chunks, intermediate 2048 = 16 chunks) split over
// KSPLIT waves. Other shapes take the run-time loop.
template <int S, int KSPLIT, int P, bool kFc1>
void launch(const FcArgs& a, unsigned grid, hipStream_t stream) {
  const int nkc = (kFc1 ? a.H : a.I) / kChunkK;
  constexpr int kNchFc1 = 56 / KSPLIT, kNchFc2 = 16 / KSPLIT;
  constexpr int kNch = kFc1 ? kNchFc1 : kNchFc2;
  if (nkc == kNch * KSPLIT && kNch >= P)
    fc_kernel<S, KSPLIT, P, kNch, kFc1><<<grid, 64 * KSPLIT, 0, stream>>>(a);
  else
    fc_kernel<S, KSPLIT, P, 0, kFc1><<<grid, 64 * KSPLIT, 0, stream>>>(a);
}

template <bool kFc1>
hipError_t launch_fc(const FcArgs& a, hipStream_t stream) {
  const int N = kFc1 ? 2 * a.I : a.H;
  const int64_t nblk = a.cap / a.block_m;
  const int64_t grid = nblk * (N / kPairRows);
  if (grid <= 0 || grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  switch (a.block_m) {
    case 16: launch<1, 4, 3, kFc1>(a, (unsigned)grid, stream); break;
    case 32: launch<2, 4, 2, kFc1>(a, (unsigned)grid, stream); break;
    case 64: launch<4, 4, 2, kFc1>(a, (unsigned)grid, stream); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || kFc1) return err;
  const int64_t n8 = (int64_t)a.M * a.H / 8;
  finalize_kernel<<<(unsigned)((n8 + 255) / 256), 256, 0, stream>>>(a.acc, a.out, n8);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fc1(const FcArgs& a, hipStream_t stream) { return launch_fc<true>(a, stream); }
hipError_t launch_fc2(const FcArgs& a, hipStream_t stream) { return launch_fc<false>(a, stream); }

}  // namespace moe

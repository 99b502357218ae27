// FC1 (gate/up + SiLU*mul) and FC2 (+ routing-weighted combine) of the
// weight-only INT4 MoE layer on the gfx950 bf16 matrix cores.
//
// "The Throughput Lever: Quantifying the MoE GEMM and Mapping the Road to
// B300", sections "Phase 3: The INT4 Marlin MoE Throughput Lever" and "The
// Result: Two Regimes": the layer is a grouped GEMM whose cost is streaming
// the INT4 weights of the experts the batch touches; in the words of the
// DDTree page ("From PCIe to NVLink", part V, priority 2) the INT4 dequant is
// fused into the MoE GEMM. Here the nibbles are widened in registers and fed
// straight to v_mfma_f32_16x16x32_bf16.
//
// Work decomposition (one workgroup = one block of block_m rows of one
// expert x one pair of 16-row weight tiles):
//   * the KSPLIT waves of a workgroup split the K range; each streams its
//     share of the pair's tiles (one 16-byte load per lane per tile) and
//     loads the activation rows it needs directly (they are reused from L2);
//   * one MFMA covers exactly one quantisation group (32 channels): the
//     weights enter as q + 136 (see dequant_u4_plus128), an extra MFMA with
//     a constant -136 operand supplies -136 * sum(x) as the accumulator input,
//     and the group scale is applied to the fp32 MFMA result (scale after
//     the product, so the weights are never rounded);
//   * partial sums of the waves meet in LDS; wave 0 runs the epilogue.
// FC1 epilogue: act_f = bf16(SiLU(gate) * up), gate and up of one output
// column land in the same lane because a pair is (gate tile r, up tile r).
// FC2 epilogue: out_acc[t] += w_f * y_f with fp32 atomics; the workgroup
// that adds the k-th contribution of a [token, 32-column] tile rounds that
// tile to bf16 into the output (per-tile arrival counters, cleared by FC1).
#include "internal.h"
#include "device_common.h"

namespace moe {
namespace {

constexpr int kKSplit = 4;
constexpr int kThreads = 64 * kKSplit;
constexpr uint32_t kNeg136Pair = 0xC308C308u;  // two bf16 -136.0

template <int BM, bool kFc1>
__global__ __launch_bounds__(kThreads) void fc_kernel(FcArgs a) {
  constexpr int S = BM / 16;  // 16-row sub-tiles per block
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int K = kFc1 ? a.H : a.I;
  const int N = kFc1 ? 2 * a.I : a.H;
  const int npairs = N / kPairRows;
  const int MK = a.M * a.k;

  if constexpr (kFc1) {
    // Clear FC2's fp32 accumulator and arrival counters (contiguous at the
    // start of the workspace), spread over every workgroup of the grid.
    const int64_t n16 = a.zero_words16;
    uint4* z = reinterpret_cast<uint4*>(a.acc);
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += stride)
      z[i] = make_uint4(0, 0, 0, 0);
  }

  const int pair = blockIdx.x % npairs;
  const int blk = blockIdx.x / npairs;
  const int npp = *a.npp;
  if (blk * BM >= npp) return;
  const int e = a.block_expert[blk];
  if (e < 0 || e >= a.E) return;
  const int32_t* rows = a.sorted_ids + (int64_t)blk * BM;

  // Activation row of this lane in each sub-tile (A operand row = lane % 16).
  const uint16_t* rowp[S];
  bool rvalid[S];
  bool sact[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int f = rows[16 * s + (lane & 15)];
    rvalid[s] = (f >= 0) && (f < MK);
    const int64_t r = rvalid[s] ? (kFc1 ? f / a.k : f) : 0;
    rowp[s] = a.act_in + r * K + 8 * (lane >> 4);
    sact[s] = __builtin_amdgcn_readfirstlane(f) < MK;  // lane 0 holds row 16*s
  }

  const int nkc = K / kChunkK;
  const int kc0 = wave * nkc / kKSplit;
  const int kc1 = (wave + 1) * nkc / kKSplit;
  const uint8_t* wbase = a.wpacked + (int64_t)e * packed_bytes_per_expert(N, K) +
                         (int64_t)pair * nkc * kPairChunkBytes;

  const uint4 neg136v = make_uint4(kNeg136Pair, kNeg136Pair, kNeg136Pair, kNeg136Pair);
  const bf16x8_t neg136 = as_bf16x8(neg136v);
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
  f32x4_t acc0[S], acc1[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    acc0[s] = zero4;
    acc1[s] = zero4;
  }

  for (int kc = kc0; kc < kc1; ++kc) {
    const uint8_t* ch = wbase + (int64_t)kc * kPairChunkBytes;
    const uint4 wq0 = *reinterpret_cast<const uint4*>(ch + 16 * lane);
    const uint4 wq1 = *reinterpret_cast<const uint4*>(ch + kTileBytes + 16 * lane);
    const uint2 sc0 = *reinterpret_cast<const uint2*>(ch + kTileNibbleBytes + 8 * (lane & 15));
    const uint2 sc1 = *reinterpret_cast<const uint2*>(ch + kTileBytes + kTileNibbleBytes + 8 * (lane & 15));
    uint4 xa[S][4];
#pragma unroll
    for (int s = 0; s < S; ++s) {
      if (!sact[s]) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        xa[s][j] = rvalid[s] ? *reinterpret_cast<const uint4*>(rowp[s] + kc * kChunkK + 32 * j)
                             : make_uint4(0, 0, 0, 0);
      }
    }
    const uint32_t q0[4] = {wq0.x, wq0.y, wq0.z, wq0.w};
    const uint32_t q1[4] = {wq1.x, wq1.y, wq1.z, wq1.w};
    const uint32_t s0w[2] = {sc0.x, sc0.y};
    const uint32_t s1w[2] = {sc1.x, sc1.y};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x8_t b0 = dequant_u4_plus128(q0[j]);
      const bf16x8_t b1 = dequant_u4_plus128(q1[j]);
      const float g0 = f16_bits_to_f32((s0w[j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
      const float g1 = f16_bits_to_f32((s1w[j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
#pragma unroll
      for (int s = 0; s < S; ++s) {
        if (!sact[s]) continue;
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

  // Sum the K-split partials in LDS.
  __shared__ f32x4_t red[kKSplit - 1][S][2][64];
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
  for (int w = 0; w < kKSplit - 1; ++w) {
#pragma unroll
    for (int s = 0; s < S; ++s) {
      acc0[s] += red[w][s][0][lane];
      acc1[s] += red[w][s][1][lane];
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
    const int nst = H / kPairRows;
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
    __threadfence();
    // Arrival counters: one lane per row adds 1; the k-th arrival converts.
#pragma unroll
    for (int s = 0; s < S; ++s) {
      if (!sact[s]) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int f = rows[16 * s + 4 * (lane >> 4) + i];
        const bool valid = f >= 0 && f < MK;
        const int t = valid ? f / a.k : 0;
        int last = 0;
        if (valid && col == 0) {
          const uint32_t old = __hip_atomic_fetch_add(a.counters + (int64_t)t * nst + pair, 1u,
                                                      __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
          last = (old == (uint32_t)(a.k - 1)) ? 1 : 0;
        }
        last = __shfl(last, lane & ~15, 64);
        if (last) {
          __threadfence();
          const float* src = a.acc + (int64_t)t * H + c0 + 2 * col;
          const float v0 = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          const float v1 = __hip_atomic_load(src + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          const uint32_t packed = f32_to_bf16_bits(v0) | (f32_to_bf16_bits(v1) << 16);
          *reinterpret_cast<uint32_t*>(a.out + (int64_t)t * H + c0 + 2 * col) = packed;
        }
      }
    }
  }
}

template <bool kFc1>
hipError_t launch_fc(const FcArgs& a, hipStream_t stream) {
  const int N = kFc1 ? 2 * a.I : a.H;
  const int64_t nblk = a.cap / a.block_m;
  const int64_t grid = nblk * (N / kPairRows);
  if (grid <= 0 || grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  switch (a.block_m) {
    case 16: fc_kernel<16, kFc1><<<(unsigned)grid, kThreads, 0, stream>>>(a); break;
    case 32: fc_kernel<32, kFc1><<<(unsigned)grid, kThreads, 0, stream>>>(a); break;
    case 64: fc_kernel<64, kFc1><<<(unsigned)grid, kThreads, 0, stream>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fc1(const FcArgs& a, hipStream_t stream) { return launch_fc<true>(a, stream); }
hipError_t launch_fc2(const FcArgs& a, hipStream_t stream) { return launch_fc<false>(a, stream); }

}  // namespace moe

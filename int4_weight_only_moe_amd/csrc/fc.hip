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
#include "fc_common.h"

namespace moe {
namespace {

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

  fc_block<S, KSPLIT, P, NCH, kFc1>(a, e, pair, frow, wave, lane);
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
  if constexpr (S == 1 && kNch >= P) {  // unrolled code only fits registers for one sub-tile
    if (nkc == kNch * KSPLIT) {
      fc_kernel<S, KSPLIT, P, kNch, kFc1><<<grid, 64 * KSPLIT, 0, stream>>>(a);
      return;
    }
  }
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

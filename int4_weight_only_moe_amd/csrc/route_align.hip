// Top-k routing and per-expert grouping of the M*k (token, slot) assignments.
//
// Routing follows "The Throughput Lever: Quantifying the MoE GEMM and
// Mapping the Road to B300", section "The Result: Two Regimes" (each token
// activates its top-k experts): the k largest logits, ties to the lower
// expert index, weights = softmax over the kept logits.
// Grouping feeds the grouped GEMM of section "Phase 3: The INT4 Marlin MoE
// Throughput Lever": a per-expert histogram, a prefix sum of the counts padded
// to the tile size, a stable permutation of the assignments and the padding.
//
// Three launch shapes produce identical integers:
//   M <= 16:    one workgroup does the top-k (one wave per token) and ranks
//               the touched experts (small_route: one block per expert);
//   otherwise:  a top-k kernel with one wave per token over many
//               workgroups, then a grouping kernel: one workgroup, or from
//               4096 assignments on a grid of workgroups, one per segment of
//               the assignments.
#include "internal.h"
#include "device_common.h"
#include "route_common.h"

namespace moe {
namespace {

constexpr int kAlignThreads = 1024;
constexpr int kAlignWaves = kAlignThreads / 64;
constexpr int kMaxExperts = 1024;
constexpr int kIdsPerLane = 8;  // expert ids a lane loads at once in the grouping passes
constexpr int kTopkWavesPerBlock = 4;
// the grid grouping kernel from this many assignments on
#ifndef MOE_ALIGN_GRID_MIN_IDS
#define MOE_ALIGN_GRID_MIN_IDS 4096
#endif
constexpr int kAlignGridMinIds = MOE_ALIGN_GRID_MIN_IDS;
constexpr int kAlignGridSegIds = 2048;
constexpr int kAlignGridMaxBlocks = 256;
constexpr int kHistIdsPerLane = 16;  // ids a thread loads at once for the grid kernel's histograms
constexpr int kWaveIdRegs = 4;       // a wave's range held in registers up to 256 ids

template <int VPL>
__global__ __launch_bounds__(64 * kTopkWavesPerBlock) void topk_kernel(
    const float* __restrict__ logits, int M, int E, int k, int32_t* __restrict__ topk_ids,
    float* __restrict__ topk_w) {
  const int t = blockIdx.x * kTopkWavesPerBlock + (threadIdx.x >> 6);
  if (t >= M) return;
  topk_token<VPL>(logits, t, E, k, topk_ids, topk_w);
}

// Grouping by one workgroup of kAlignThreads threads.
//   counts     histogram of the expert ids (LDS atomics: order-free);
//   offsets    exclusive scan of the counts rounded up to block_m;
//   placement  each wave takes a contiguous range of f in ascending order;
//              a lane's rank among equal experts of its 64-lane step is the
//              number of lower lanes holding its expert (a ballot per bit of
//              the expert id), and earlier waves and steps add their counts,
//              so each expert's list is in ascending f without any
//              order-dependent atomic.
struct AlignShared {
  int cnt[kMaxExperts];
  int off[kMaxExperts + 1];
  int wave_tot[kAlignWaves];
  int wcnt[kAlignWaves][kMaxExperts];
};

// Lanes of the wave whose key equals this lane's, for keys below 2^nbits:
// one ballot per key bit, each lane keeping the lanes that agree with it on
// that bit, starting from the lanes in `live`. Wave-uniform control flow only.
__device__ __forceinline__ uint64_t equal_key_lanes(int key, int nbits, uint64_t live) {
  uint64_t m = live;
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (key >> b) & 1;
    const uint64_t bal = __ballot(bit);
    m &= bit ? bal : ~bal;
  }
  return m;
}

__device__ __forceinline__ void align_body(AlignShared& sh, const int32_t* __restrict__ ids, int MK, int E,
                           int block_m, int32_t* __restrict__ sorted_ids,
                           int32_t* __restrict__ block_expert, int32_t* __restrict__ offsets,
                           int32_t* __restrict__ npp_out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < E) {
    sh.cnt[tid] = 0;
    if (MK > 64) {
#pragma unroll
      for (int w = 0; w < kAlignWaves; ++w) sh.wcnt[w][tid] = 0;
    }
  }
  __syncthreads();
  // Wave w owns the contiguous assignment range [f0, f1) (placement below
  // keeps ascending f inside it). The ids are read kIdsPerLane per lane at a
  // time, all loads in flight before the first use; the pass counts both the
  // expert totals and the wave's own per-expert counts.
  const int seg = ((MK + kAlignWaves - 1) / kAlignWaves + 63) / 64 * 64;
  const int f0 = wave * seg, f1 = (f0 + seg < MK) ? f0 + seg : MK;
  if (MK > 64) {
    for (int fb = f0; fb < f1; fb += 64 * kIdsPerLane) {
      int ev[kIdsPerLane];
#pragma unroll
      for (int i = 0; i < kIdsPerLane; ++i) {
        const int f = fb + 64 * i + lane;
        ev[i] = f < f1 ? ids[f] : -1;
      }
#pragma unroll
      for (int i = 0; i < kIdsPerLane; ++i) {
        if (ev[i] >= 0 && ev[i] < E) {
          atomicAdd(&sh.cnt[ev[i]], 1);
          atomicAdd(&sh.wcnt[wave][ev[i]], 1);
        }
      }
    }
  } else if (tid < MK) {
    const int e = ids[tid];
    if (e >= 0 && e < E) atomicAdd(&sh.cnt[e], 1);
  }
  __syncthreads();

  // exclusive scan of padded counts (E <= kAlignThreads: one expert per thread)
  int padded = 0;
  if (tid < E) padded = (sh.cnt[tid] + block_m - 1) / block_m * block_m;
  int incl = padded;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  if (lane == 63) sh.wave_tot[wave] = incl;
  __syncthreads();
  int wave_base = 0;
  for (int w = 0; w < wave; ++w) wave_base += sh.wave_tot[w];
  const int excl = wave_base + incl - padded;
  if (tid < E) {
    sh.off[tid] = excl;
    offsets[tid] = excl;
  }
  if (tid == E - 1) {
    sh.off[E] = excl + padded;
    offsets[E] = excl + padded;
    *npp_out = excl + padded;
  }
  __syncthreads();

  // block -> expert map and sentinel padding, one expert per thread
  if (tid < E) {
    const int o0 = sh.off[tid], o1 = sh.off[tid + 1], c = sh.cnt[tid];
    for (int bb = o0 / block_m; bb < o1 / block_m; ++bb) block_expert[bb] = tid;
    for (int p = o0 + c; p < o1; ++p) sorted_ids[p] = MK;
  }

  // stable placement
  const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
  if (MK <= 64) {
    // one wave's worth: rank among equal experts of the earlier lanes only
    if (wave == 0) {
      int e = (lane < MK) ? ids[lane] : -1;
      e = (e >= E) ? -1 : e;
      const uint64_t same = equal_key_lanes(e, nbits, __ballot(e >= 0));
      if (e >= 0) sorted_ids[sh.off[e] + lanes_below(same)] = lane;
    }
    return;
  }
  // The waves' per-expert counts (counted with the totals above) become,
  // by a scan over the waves per expert, each wave's first position in the
  // expert's list; each wave then walks its range 64 lanes at a time, in
  // order, placing each assignment at its wave's running position plus its
  // rank among the equal experts of earlier lanes, and advances the running
  // positions.
  if (tid < E) {
    int c[kAlignWaves];  // all reads first: they go out together
#pragma unroll
    for (int w = 0; w < kAlignWaves; ++w) c[w] = sh.wcnt[w][tid];
    int run = sh.off[tid];
#pragma unroll
    for (int w = 0; w < kAlignWaves; ++w) {
      sh.wcnt[w][tid] = run;
      run += c[w];
    }
  }
  __syncthreads();
  for (int fb = f0; fb < f1; fb += 64 * kIdsPerLane) {
    int ev[kIdsPerLane];
#pragma unroll
    for (int i = 0; i < kIdsPerLane; ++i) {
      const int f = fb + 64 * i + lane;
      const int e = f < f1 ? ids[f] : -1;
      ev[i] = (e >= E) ? -1 : e;
    }
#pragma unroll
    for (int i = 0; i < kIdsPerLane; ++i) {
      if (fb + 64 * i >= f1) break;  // wave-uniform: the rest of the batch is past the range
      const int e = ev[i];
      const uint64_t same = equal_key_lanes(e, nbits, __ballot(e >= 0));
      const int before = lanes_below(same), tot = __builtin_popcountll(same);
      if (e >= 0) {
        // every lane reads the running position before the group's last lane
        // advances it (one wave: its LDS operations complete in order)
        const int base = sh.wcnt[wave][e];
        sorted_ids[base + before] = fb + 64 * i + lane;
        if (before == tot - 1) sh.wcnt[wave][e] = base + tot;
      }
    }
  }
}

// Grouping by a grid of workgroups for large batches (the one-workgroup
// kernel walks 64 assignments per wave step, so its time grows with M*k:
// ~80 us at M*k = 65536). Workgroup g places the contiguous segment
// [g*seg, (g+1)*seg) of the assignments. It needs each expert's total (for
// the padded offsets, which every workgroup computes alike) and each
// expert's count before its segment (where its part of the expert's list
// starts): it histograms all M*k ids itself, so no workgroup waits for
// another and no memory beyond the outputs is used. Inside the segment the
// placement is the one-workgroup kernel's: each wave a contiguous range,
// ballot ranks among equal experts, running positions in LDS. The outputs
// are identical to the one-workgroup kernel's.
struct AlignGridShared {
  int total[kMaxExperts];
  int before[kMaxExperts];
  int wave_tot[kAlignWaves];
  int wcnt[kAlignWaves][kMaxExperts];
};

__global__ __launch_bounds__(kAlignThreads) void align_grid_kernel(
    const int32_t* __restrict__ ids, int MK, int E, int block_m, int seg, int32_t* __restrict__ sorted_ids,
    int32_t* __restrict__ block_expert, int32_t* __restrict__ offsets, int32_t* __restrict__ npp_out) {
  __shared__ AlignGridShared sh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int s0 = blockIdx.x * seg;
  const int s1 = s0 + seg < MK ? s0 + seg : MK;
  if (tid < E) {
    sh.total[tid] = 0;
    sh.before[tid] = 0;
#pragma unroll
    for (int w = 0; w < kAlignWaves; ++w) sh.wcnt[w][tid] = 0;
  }
  __syncthreads();
  // each wave's own contiguous range of the segment; up to kWaveIdRegs ids
  // per lane it is loaded once, with the first histogram batch, and kept in
  // registers for the count and the placement
  const int wseg = ((s1 - s0 + kAlignWaves - 1) / kAlignWaves + 63) / 64 * 64;
  const int f0 = s0 + wave * wseg < s1 ? s0 + wave * wseg : s1;
  const int f1 = f0 + wseg < s1 ? f0 + wseg : s1;
  const bool in_regs = wseg <= 64 * kWaveIdRegs;
  int wv[kWaveIdRegs];
#pragma unroll
  for (int r = 0; r < kWaveIdRegs; ++r) {
    const int f = f0 + 64 * r + lane;
    wv[r] = ids[f < MK ? f : MK - 1];
  }
  // histograms of all ids and of the ids before the segment; the loads of a
  // batch are unconditional (index clamped) so they go out together
  for (int fb = 0; fb < MK; fb += kAlignThreads * kHistIdsPerLane) {
    int ev[kHistIdsPerLane];
#pragma unroll
    for (int i = 0; i < kHistIdsPerLane; ++i) {
      const int f = fb + i * kAlignThreads + tid;
      ev[i] = ids[f < MK ? f : MK - 1];
    }
#pragma unroll
    for (int i = 0; i < kHistIdsPerLane; ++i) {
      const int f = fb + i * kAlignThreads + tid;
      const int e = ev[i];
      if (f < MK && e >= 0 && e < E) {
        atomicAdd(&sh.total[e], 1);
        if (f < s0) atomicAdd(&sh.before[e], 1);
      }
    }
  }
  // the wave's per-expert counts
  if (in_regs) {
#pragma unroll
    for (int r = 0; r < kWaveIdRegs; ++r) {
      const int e = wv[r];
      if (f0 + 64 * r + lane < f1 && e >= 0 && e < E) atomicAdd(&sh.wcnt[wave][e], 1);
    }
  } else {
    for (int f = f0 + lane; f < f1; f += 64) {
      const int e = ids[f];
      if (e >= 0 && e < E) atomicAdd(&sh.wcnt[wave][e], 1);
    }
  }
  __syncthreads();

  // exclusive scan of the padded totals (one expert per thread)
  int padded = 0;
  if (tid < E) padded = (sh.total[tid] + block_m - 1) / block_m * block_m;
  int incl = padded;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  if (lane == 63) sh.wave_tot[wave] = incl;
  __syncthreads();
  int wave_base = 0;
  for (int w = 0; w < wave; ++w) wave_base += sh.wave_tot[w];
  const int excl = wave_base + incl - padded;

  // offsets, the block -> expert map and the sentinel padding: expert e is
  // written by workgroup e % gridDim.x
  if (tid < E && tid % gridDim.x == blockIdx.x) {
    const int o0 = excl, o1 = excl + padded, c = sh.total[tid];
    offsets[tid] = o0;
    for (int bb = o0 / block_m; bb < o1 / block_m; ++bb) block_expert[bb] = tid;
    for (int p = o0 + c; p < o1; ++p) sorted_ids[p] = MK;
  }
  if (tid == E - 1 && blockIdx.x == 0) {
    offsets[E] = excl + padded;
    *npp_out = excl + padded;
  }
  // each wave's first position in each expert's list: the expert's offset,
  // the segments before this one, the waves before this one
  if (tid < E) {
    int c[kAlignWaves];
#pragma unroll
    for (int w = 0; w < kAlignWaves; ++w) c[w] = sh.wcnt[w][tid];
    int run = excl + sh.before[tid];
#pragma unroll
    for (int w = 0; w < kAlignWaves; ++w) {
      sh.wcnt[w][tid] = run;
      run += c[w];
    }
  }
  __syncthreads();

  // stable placement of the wave's range, 64 assignments a step
  const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
  for (int fb = f0, r = 0; fb < f1; fb += 64, ++r) {
    const int f = fb + lane;
    int e = -1;
    if (in_regs) {
#pragma unroll
      for (int q = 0; q < kWaveIdRegs; ++q) e = q == r ? wv[q] : e;
    } else {
      e = ids[f < MK ? f : MK - 1];
    }
    e = (f >= f1 || e >= E) ? -1 : e;
    const uint64_t same = equal_key_lanes(e, nbits, __ballot(e >= 0));
    const int before = lanes_below(same), tot = __builtin_popcountll(same);
    if (e >= 0) {
      // every lane reads the running position before the group's last lane
      // advances it (one wave: its LDS operations complete in order)
      const int base = sh.wcnt[wave][e];
      sorted_ids[base + before] = f;
      if (before == tot - 1) sh.wcnt[wave][e] = base + tot;
    }
  }
}

__global__ __launch_bounds__(kAlignThreads) void align_kernel(
    const int32_t* __restrict__ ids, int MK, int E, int block_m, int32_t* __restrict__ sorted_ids,
    int32_t* __restrict__ block_expert, int32_t* __restrict__ offsets, int32_t* __restrict__ npp) {
  __shared__ AlignShared sh;
  align_body(sh, ids, MK, E, block_m, sorted_ids, block_expert, offsets, npp);
}

// Small batches (M <= 16): small_route in one workgroup (routing, ranks of
// the touched experts by an LDS bitmap, one block per touched expert), then
// the outputs from its tables. Measured at M = 9 on the 384-expert layer:
// 10.4 us with the general grouping (histogram, scan, ballot placement).
template <int VPL>
__global__ __launch_bounds__(kAlignThreads) void route_align_small_kernel(
    const float* __restrict__ logits, int M, int E, int k, int block_m, int32_t* __restrict__ topk_ids,
    float* __restrict__ topk_w, int32_t* __restrict__ sorted_ids, int32_t* __restrict__ block_expert,
    int32_t* __restrict__ offsets, int32_t* __restrict__ npp) {
  __shared__ SmallRoute sh;
  const int nd = small_route<VPL, kAlignThreads>(sh, logits, M, E, k);
  small_route_write<kAlignThreads>(sh, nd, M, E, k, block_m, topk_ids, topk_w, sorted_ids, block_expert, offsets,
                                   npp);
}

template <int VPL>
hipError_t launch_vpl(const float* logits, int M, int E, int k, int block_m, int32_t* topk_ids,
                      float* topk_w, int32_t* sorted_ids, int32_t* block_expert, int32_t* offsets,
                      int32_t* npp, hipStream_t stream) {
  if (M <= kSmallMaxTokens && M * k <= kSmallMaxAssign) {
    route_align_small_kernel<VPL><<<1, kAlignThreads, 0, stream>>>(
        logits, M, E, k, block_m, topk_ids, topk_w, sorted_ids, block_expert, offsets, npp);
    return hipGetLastError();
  }
  const int blocks = (M + kTopkWavesPerBlock - 1) / kTopkWavesPerBlock;
  topk_kernel<VPL><<<blocks, 64 * kTopkWavesPerBlock, 0, stream>>>(logits, M, E, k, topk_ids, topk_w);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int MK = M * k;
  if (MK >= kAlignGridMinIds) {
    // segments of at least kAlignGridSegIds assignments, at most
    // kAlignGridMaxBlocks workgroups (each histograms all M*k ids)
    const int64_t per = ((int64_t)MK + kAlignGridMaxBlocks - 1) / kAlignGridMaxBlocks;
    const int seg = (int)(per > kAlignGridSegIds ? (per + 1023) / 1024 * 1024 : kAlignGridSegIds);
    const int grid = (MK + seg - 1) / seg;
    align_grid_kernel<<<grid, kAlignThreads, 0, stream>>>(topk_ids, MK, E, block_m, seg, sorted_ids, block_expert,
                                                          offsets, npp);
  } else {
    align_kernel<<<1, kAlignThreads, 0, stream>>>(topk_ids, MK, E, block_m, sorted_ids, block_expert, offsets,
                                                  npp);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route_align(const float* logits, int M, int E, int k, int block_m,
                              int32_t* topk_ids, float* topk_weights, int32_t* sorted_ids,
                              int32_t* block_expert, int32_t* offsets, int32_t* npp, int64_t cap,
                              hipStream_t stream) {
  (void)cap;
  if (E <= 64)
    return launch_vpl<1>(logits, M, E, k, block_m, topk_ids, topk_weights, sorted_ids, block_expert, offsets, npp, stream);
  if (E <= 128)
    return launch_vpl<2>(logits, M, E, k, block_m, topk_ids, topk_weights, sorted_ids, block_expert, offsets, npp, stream);
  if (E <= 256)
    return launch_vpl<4>(logits, M, E, k, block_m, topk_ids, topk_weights, sorted_ids, block_expert, offsets, npp, stream);
  if (E <= 384)
    return launch_vpl<6>(logits, M, E, k, block_m, topk_ids, topk_weights, sorted_ids, block_expert, offsets, npp, stream);
  if (E <= 512)
    return launch_vpl<8>(logits, M, E, k, block_m, topk_ids, topk_weights, sorted_ids, block_expert, offsets, npp, stream);
  return launch_vpl<16>(logits, M, E, k, block_m, topk_ids, topk_weights, sorted_ids, block_expert, offsets, npp, stream);
}

}  // namespace moe

// Tiled grouped GEMM (FC1 and FC2) for batches whose experts hold tens to
// hundreds of rows: skewed routing, and large multi-stream batches.
//
// "The Throughput Lever: Quantifying the MoE GEMM and Mapping the Road to
// B300", section "The Result: Two Regimes": as the batch grows, the grouped
// GEMM turns from streaming the touched experts' weights into matrix work.
// What limits it on gfx950 is not the matrix core but the vector unit: the
// exact dequantisation widens every code (a few VALU operations per 8
// weights) and applies each group's fp16 scale to the fp32 MFMA result (one
// FMA per output and group, as many VALU cycles as the MFMA itself). Widened
// codes are shared by all rows of a tile, so the work per MFMA falls as the
// tile grows; the scale FMA does not.
//
// Work decomposition:
//   * a plan kernel cuts each expert's row range (block_m-padded, from
//     moe_route_align) into tiles of up to 64 rows (128 for the scale-before
//     kernel of fc_tile128.hip): a tile starts at every expert change and at
//     every 64-row boundary of the padded list, so an expert holding hundreds
//     of rows gets several 64-row tiles; a tile
//     counts only the 16-row sub-tiles that hold a row (padding is not
//     multiplied);
//   * a workgroup = one tile x 8 tile pairs (one per wave, full K); the
//     tile's activation chunk (up to 64 rows x 128 channels) is staged once
//     in a padded LDS double buffer and read by all 8 waves; two workgroups
//     share a CU (<= 128 VGPRs, 4 waves per SIMD: measured ~15% faster than
//     128-row tiles at 2 waves per SIMD, whose stalls nothing covers);
//   * per 32-channel group and 16-row sub-tile a wave spends one MFMA on the
//     -136 * sum(x) correction (the weights enter as q + 136) and one per
//     weight tile, then scales each result into its fp32 sum;
//   * the body is specialised for 1, 2 or 4 sub-tiles (a tile with 3 runs
//     the next size up with an empty one): the inner loop has no branches;
//   * weights of an expert with a single tile are streamed non-temporally,
//     those of an expert with several tiles are kept in the caches (its other
//     tiles re-read them);
//   * workgroup ids are dealt to the 8 XCDs so that all pair groups of a
//     tile run on one XCD (the tile's activations are read from that XCD's
//     L2) while consecutive tiles go to different XCDs.
// Epilogues are those of the other grouped kernels (FC1: bf16 SiLU(gate)*up;
// FC2: routing-weighted fp32 atomics into the accumulator FC1 clears).
#include "internal.h"
#include "device_common.h"
#include "fc_common.h"

namespace moe {
namespace MOE_FMT_NS {
namespace {

constexpr int kTW = 8;                     // waves (= tile pairs) per workgroup
constexpr int kTRowVecs = kChunkK / 8;     // 16-byte vectors of a row's chunk slice
constexpr int kTRowPad = kTRowVecs + 1;    // +16 B per row: rows start on different banks
constexpr int kTP = 2;                     // weight chunks in flight per wave (even: static ring slots)
constexpr int kTXcds = 8;

// ---------------------------------------------------------------------------
// Plan: one workgroup turns the block list into the tile list.
// tile_rows: 64 (this file's kernel) or 128 (the scale-before kernel).
__global__ __launch_bounds__(1024) void tile_plan_kernel(const int32_t* __restrict__ block_expert,
                                                        const int32_t* __restrict__ sorted_ids,
                                                        const int32_t* __restrict__ npp_p, int block_m, int MK,
                                                        int tile_rows, int max_tiles, int2* __restrict__ tiles,
                                                        int32_t* __restrict__ ntiles_out) {
  __shared__ int wave_cnt[16];
  __shared__ int base;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bpt = tile_rows / block_m;  // blocks per full tile
  const int nblk = *npp_p / block_m;
  if (tid == 0) base = 0;
  __syncthreads();
  for (int b0 = 0; b0 < nblk; b0 += 1024) {
    const int b = b0 + tid;
    int e = -1;
    bool head = false;
    if (b < nblk) {
      e = block_expert[b];
      head = (b % bpt == 0) || block_expert[b - 1] != e;  // b % bpt != 0 implies b >= 1
    }
    const unsigned long long m = __ballot(head);
    if (lane == 0) wave_cnt[wave] = __popcll(m);
    __syncthreads();
    int t = base + __popcll(m & ((1ull << lane) - 1ull));
    for (int w = 0; w < wave; ++w) t += wave_cnt[w];
    if (head && t < max_tiles) {
      // the tile runs to the next full-tile boundary or the end of the expert
      int nb = 1;
      while (nb < bpt - b % bpt && b + nb < nblk && block_expert[b + nb] == e) ++nb;
      // sub-tiles that hold a row: an expert's padding sits at the end of its
      // range, so they are a prefix of the tile's
      int nsub = nb * block_m / kTileRows;
      while (nsub > 1 && sorted_ids[b * block_m + (nsub - 1) * kTileRows] >= MK) --nsub;
      const bool reuse = (b > 0 && block_expert[b - 1] == e) || (b + nb < nblk && block_expert[b + nb] == e);
      tiles[t] = make_int2(b * block_m, nsub | (reuse ? kTileReuseBit : 0) | (e << kTileExpertShift));
    }
    __syncthreads();
    if (tid == 0) {
      int tot = 0;
      for (int w = 0; w < 16; ++w) tot += wave_cnt[w];
      base += tot;
    }
    __syncthreads();
  }
  if (tid == 0) *ntiles_out = base < max_tiles ? base : max_tiles;
}

// ---------------------------------------------------------------------------
// One workgroup's tile (rows row0 .. row0 + 16 * nsub of the sorted list,
// expert e) times this wave's tile pair, S >= nsub sub-tiles, weights loaded
// under cache policy kPolicy.
template <int S, bool kFc1, int kPolicy>
__device__ __forceinline__ void fc_tile_body(const FcArgs& a, const int e, const int pair, const int row0,
                                             const int nsub, uint4 (&xt)[2][kTileMaxRows][kTRowPad]) {
  constexpr int kThreads = 64 * kTW;
  constexpr int kItems = 16 * S * kTRowVecs;  // staged 16-byte vectors per chunk
  constexpr int kIPT = (kItems + kThreads - 1) / kThreads;
  constexpr int P = kTP;
  const int tid = threadIdx.x, lane = tid & 63;
  const int K = kFc1 ? a.H : a.I;
  const int N = kFc1 ? 2 * a.I : a.H;
  const int MK = a.M * a.k;
  const int n = K / kChunkK;
  const int32_t* rows = a.sorted_ids + row0;

  const uint8_t* wbase = a.wpacked + (int64_t)e * packed_bytes_per_expert(N, K) + (int64_t)pair * n * kPairChunkBytes;
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(wbase, (uint32_t)n * kPairChunkBytes);
  const uint32_t oq0 = 16u * lane, oq1 = kTileBytes + 16u * lane;
  const uint32_t os0 = kTileNibbleBytes + kScaleRowBytes * (lane & 15);
  const uint32_t os1 = kTileBytes + kTileNibbleBytes + kScaleRowBytes * (lane & 15);
  auto load_w = [&](int c) {
    const uint32_t base = (uint32_t)c * kPairChunkBytes;  // past the K range: zeros
    WChunk w;
    w.q0 = bload16<kPolicy>(wr, base + oq0);
    w.q1 = bload16<kPolicy>(wr, base + oq1);
    w.s0 = load_scales<kPolicy>(wr, base + os0);
    w.s1 = load_scales<kPolicy>(wr, base + os1);
    return w;
  };

  // The weight stream goes out first: it does not wait for the row ids that
  // the activation loads need (the scheduling barrier keeps those waits
  // below the loads).
  WChunk wb[P];
#pragma unroll
  for (int j = 0; j < P; ++j) wb[j] = load_w(j);
  __builtin_amdgcn_sched_barrier(0);

  // Staging: item i = (row i / 16, vector i % 16) of the chunk.
  const int rows_total = kFc1 ? a.M : MK;
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.act_in, (uint32_t)rows_total * (uint32_t)K * 2u);
  uint32_t soff[kIPT];
#pragma unroll
  for (int i = 0; i < kIPT; ++i) {
    const int item = tid + kThreads * i;
    const int r = item / kTRowVecs, v = item % kTRowVecs;
    const int f = (item < kItems && r < 16 * nsub) ? rows[r] : MK;
    const bool ok = f >= 0 && f < MK;
    soff[i] = ok ? ((uint32_t)(kFc1 ? f / a.k : f) * (uint32_t)K + 8u * v) * 2u : kOutOfRange;
  }
  auto load_x = [&](uint4 (&xg)[kIPT], int c) {
#pragma unroll
    for (int i = 0; i < kIPT; ++i)
      xg[i] = bload16(xr, (c < n && soff[i] != kOutOfRange) ? soff[i] + (uint32_t)c * (kChunkK * 2) : kOutOfRange);
  };
  // Unconditional: items past kItems (one sub-tile) land in rows 16..31,
  // which no MFMA reads; a branch here would let the compiler sink the
  // scale FMAs below it and keep every MFMA result of the chunk live.
  auto store_x = [&](const uint4 (&xg)[kIPT], int slot) {
#pragma unroll
    for (int i = 0; i < kIPT; ++i) {
      const int item = tid + kThreads * i;
      xt[slot][item / kTRowVecs][item % kTRowVecs] = xg[i];
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
  // Activation chunks are loaded kXD steps before they are stored to LDS
  // (kXD register sets alternating with the step parity; one for 4
  // sub-tiles, whose accumulators need the registers).
  constexpr int kXD = S >= 4 ? 1 : 2;
  uint4 xg[kXD][kIPT];
  load_x(xg[0], 0);
  store_x(xg[0], 0);
#pragma unroll
  for (int d = 0; d < kXD; ++d) load_x(xg[d], 1 + d);
  __syncthreads();

  // n is even (checked by the launcher), so the loop body has no branch.
  const int mrow = lane & 15, kv = lane >> 4;
  for (int c = 0; c < n; c += P) {
#pragma unroll
    for (int j = 0; j < P; ++j) {
      const int cc = c + j;
      {
        const int slot = j & 1;  // == cc & 1 since c is a multiple of the even P
        const WChunk w = wb[j];
        const uint32_t q0[4] = {w.q0.x, w.q0.y, w.q0.z, w.q0.w};
        const uint32_t q1[4] = {w.q1.x, w.q1.y, w.q1.z, w.q1.w};
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float g0 = group_scale(w.s0, g);
          const float g1 = group_scale(w.s1, g);
          const bf16x8_t b0 = dequant_group(q0[g], g0);
          const bf16x8_t b1 = dequant_group(q1[g], g1);
          if constexpr (kFmt == kFmtMxfp4) {
            // FP4: the scale is in the B operand, so each MFMA accumulates
            // straight into its sub-tile's sums (no vector work per output)
#pragma unroll
            for (int s = 0; s < S; ++s) {
              const bf16x8_t xv = as_bf16x8(xt[slot][16 * s + mrow][4 * g + kv]);
              acc0[s] = mfma16x16x32(xv, b0, acc0[s]);
              acc1[s] = mfma16x16x32(xv, b1, acc1[s]);
            }
            continue;
          }
          // Sub-tiles one after another, software-pipelined: step s issues
          // the MFMAs of sub-tile s (and the correction of s + 1), then the
          // scale FMAs of sub-tile s - 1, which run on the vector unit while
          // the matrix core works on step s. At most two sub-tiles are in
          // flight; more would only be hoisted into registers.
          bf16x8_t xv = as_bf16x8(xt[slot][mrow][4 * g + kv]);
          f32x4_t off = mfma16x16x32(xv, neg136, zero4);
          f32x4_t p0 = zero4, p1 = zero4;  // products of the previous sub-tile
#pragma unroll
          for (int s = 0; s < S; ++s) {
            bf16x8_t xn = xv;
            if (s + 1 < S) xn = as_bf16x8(xt[slot][16 * (s + 1) + mrow][4 * g + kv]);
            const f32x4_t t0 = mfma16x16x32(xv, b0, off);
            const f32x4_t t1 = mfma16x16x32(xv, b1, off);
            if (s + 1 < S) off = mfma16x16x32(xn, neg136, zero4);
            if (s > 0) {
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                acc0[s - 1][i] = __builtin_fmaf(p0[i], g0, acc0[s - 1][i]);
                acc1[s - 1][i] = __builtin_fmaf(p1[i], g1, acc1[s - 1][i]);
              }
            }
            p0 = t0;
            p1 = t1;
            xv = xn;
            __builtin_amdgcn_sched_barrier(0);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc0[S - 1][i] = __builtin_fmaf(p0[i], g0, acc0[S - 1][i]);
            acc1[S - 1][i] = __builtin_fmaf(p1[i], g1, acc1[S - 1][i]);
          }
        }
        wb[j] = load_w(cc + P);
        store_x(xg[j % kXD], (j + 1) & 1);  // chunk cc + 1 (zeros past the end)
        load_x(xg[j % kXD], cc + 1 + kXD);
        __syncthreads();
      }
    }
  }
  // This lane's row of every sub-tile (sub-tiles past nsub have none), read
  // here rather than kept live across the main loop.
  int frow[S];
  bool sact[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    sact[s] = s < nsub;
    frow[s] = sact[s] ? rows[16 * s + (lane & 15)] : MK;
  }
  fc_epilogue<S, kFc1>(a, pair, frow, sact, acc0, acc1, lane);
}

template <int S, bool kFc1>
__device__ __forceinline__ void fc_tile_dispatch_policy(const FcArgs& a, const int e, const int pair,
                                                        const int row0, const int nsub, const bool reuse,
                                                        uint4 (&xt)[2][kTileMaxRows][kTRowPad]) {
  if (reuse)
    fc_tile_body<S, kFc1, kPolicyDefault>(a, e, pair, row0, nsub, xt);
  else
    fc_tile_body<S, kFc1, kPolicyWeights>(a, e, pair, row0, nsub, xt);
}

template <bool kFc1>
__global__ __launch_bounds__(64 * kTW) __attribute__((amdgpu_waves_per_eu(4))) void fc_tile_kernel(FcArgs a) {
  __shared__ uint4 xt[2][kTileMaxRows][kTRowPad];
  constexpr int kThreads = 64 * kTW;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int N = kFc1 ? 2 * a.I : a.H;
  const int npg = N / kPairRows / kTW;  // pair groups per tile

  if constexpr (kFc1) {  // clear FC2's accumulator
    uint4* z = reinterpret_cast<uint4*>(a.acc);
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + tid; i < a.zero_words16; i += stride)
      z[i] = make_uint4(0, 0, 0, 0);
  }

  const int xcd = blockIdx.x % kTXcds, gi = blockIdx.x / kTXcds;
  const int tile = (gi / npg) * kTXcds + xcd;
  const int pair = (gi % npg) * kTW + wave;
  // the table has max_tiles entries (those past ntiles are not used): the
  // entry and the count are read in one round trip (the empty asm needs both
  // before the check, so the entry's load is not sunk below it)
  if (tile >= a.max_tiles) return;
  const int2 te = a.tiles[tile];
  const int ntiles = *a.ntiles;
  asm volatile("" ::"s"(te.x), "s"(te.y), "s"(ntiles));
  if (tile >= ntiles) return;
  const int row0 = __builtin_amdgcn_readfirstlane(te.x);
  const int meta = __builtin_amdgcn_readfirstlane(te.y);
  const int nsub = meta & kTileNsubMask;
  const bool reuse = (meta & kTileReuseBit) != 0;
  const int e = meta >> kTileExpertShift;
  if (e < 0 || e >= a.E || nsub < 1 || nsub > kTileMaxRows / kTileRows) return;

  if (nsub <= 1) fc_tile_dispatch_policy<1, kFc1>(a, e, pair, row0, nsub, reuse, xt);
  else if (nsub <= 2) fc_tile_dispatch_policy<2, kFc1>(a, e, pair, row0, nsub, reuse, xt);
  else fc_tile_dispatch_policy<4, kFc1>(a, e, pair, row0, nsub, reuse, xt);
}

}  // namespace

int64_t tile_grid_tiles(int64_t M, int64_t E, int64_t k, int64_t block_m, int64_t cap, int64_t tile_rows) {
  const int64_t bpt = tile_rows / block_m;
  const int64_t nblk = cap / block_m;
  const int64_t mk = M * k;
  const int64_t t = (nblk + bpt - 1) / bpt + (mk < E ? mk : E);
  return (t + kTXcds - 1) / kTXcds * kTXcds;
}

bool tile_path_supported(int64_t H, int64_t I) {
  // whole pair groups, and an even number of K chunks in both GEMMs
  return (2 * I / kPairRows) % kTW == 0 && (H / kPairRows) % kTW == 0 && (H / kChunkK) % kTP == 0 &&
         (I / kChunkK) % kTP == 0;
}

hipError_t launch_tile_plan(const FcArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(tile_plan_kernel, dim3(1), dim3(1024), 0, stream, a.block_expert, a.sorted_ids, a.npp,
                     a.block_m, a.M * a.k, a.tile_rows, a.max_tiles, a.tiles, a.ntiles);
  return hipGetLastError();
}

template <bool kFc1>
hipError_t launch_fc_tiled(const FcArgs& a, hipStream_t stream, hipEvent_t e0, hipEvent_t e1) {
  const int N = kFc1 ? 2 * a.I : a.H;
  const int64_t grid = (int64_t)a.max_tiles * (N / kPairRows / kTW);
  if (grid <= 0 || grid > 0x7FFFFFFF || a.max_tiles % kTXcds != 0) return hipErrorInvalidValue;
  launch_kernel(fc_tile_kernel<kFc1>, dim3((unsigned)grid), dim3(64 * kTW), 0, stream, e0, e1, a);
  return hipGetLastError();
}

template hipError_t launch_fc_tiled<true>(const FcArgs&, hipStream_t, hipEvent_t, hipEvent_t);
template hipError_t launch_fc_tiled<false>(const FcArgs&, hipStream_t, hipEvent_t, hipEvent_t);

}  // namespace MOE_FMT_NS
}  // namespace moe

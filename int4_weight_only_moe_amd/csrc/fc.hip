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
// With MXFP4 weights (this file compiled with MOE_WEIGHT_FORMAT = 1) the
// codes are widened to exact bf16 values already carrying the group's E8M0
// scale, so there is neither the -136 correction nor a scale after the
// product (fc_common.h: group_scale, dequant_group, group_c, group_add).
// FC1 epilogue: act_f = bf16(SiLU(gate) * up); gate and up of one output
// column land in the same lane because a pair is (gate tile r, up tile r).
// FC2 epilogue: acc[t] += w_f * y_f with fp32 atomics into a workspace
// accumulator that FC1 clears; a last small kernel rounds acc to bf16 once.
// (A "last arriving workgroup converts" scheme needs agent-scope fences, and
// on gfx950 each of those writes back and invalidates the L2.)
#include <atomic>

#include "internal.h"
#include "device_common.h"
#include "fc_common.h"
#include "route_common.h"

namespace moe {
namespace MOE_FMT_NS {
namespace {

template <int S, int KSPLIT, int P, int NCH, bool kFc1>
__global__ __launch_bounds__(64 * KSPLIT) __attribute__((amdgpu_waves_per_eu(S == 1 ? 4 : 1)))
void fc_kernel(FcArgs a) {
  constexpr int kThreads = 64 * KSPLIT;
  const int lane = threadIdx.x & 63;
  // wave index, blocks, experts and chunk ranges are wave-uniform: keep them
  // in scalar registers so the buffer descriptors built from them are too
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int N = kFc1 ? 2 * a.I : a.H;
  const int npairs = N / kPairRows;

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

// ---------------------------------------------------------------------------
// Wide variant for blocks of 32 or 64 rows (batches with tens of tokens per
// expert). Streaming each activation row once per tile pair, as fc_kernel
// does, multiplies the activation traffic by the number of pairs (128 for
// FC1 of the 384-expert layer); here one workgroup covers kWideNP pairs
// (one wave each, full K) and stages the block's activation chunk in LDS once
// for all of them. The -136*sum(x) correction of each (row, group) is summed
// while staging and enters the MFMA as its accumulator input, so no MFMA is
// spent on it. Workgroups are dealt to the 8 XCDs round-robin; the id
// mapping gives XCD x the blocks x, x+8, x+16, ... with all pair groups of a
// block on that XCD, back to back: a block's activations are read from that
// XCD's L2 by its pair groups, and an expert with many blocks (skewed
// routing) is spread over all XCDs instead of loading one of them.
//
// Per chunk step c (one barrier per step):
//   issue the activation loads of chunk c+P and the weight loads of c+P
//   (both rings P deep in registers, so a wait for one never drains the other),
//   run chunk c from LDS slot c%2, then store chunk c+1 into slot (c+1)%2.
constexpr int kWideNP = 16;                 // waves = tile pairs per workgroup
constexpr int kWideP = 2;                   // chunks in flight per wave (even: LDS slot parity is static)
constexpr int kRowVecs = kChunkK / 8;       // 16-byte vectors of a row's chunk slice
// A row's 16 vectors are stored XOR-swizzled with the row index (vector v of
// row r at v ^ (r % 16)): the A reads of a lane group (16 rows, the same
// vector) and the staging writes (one row's 16 vectors) hit distinct banks.
__device__ __forceinline__ int xswz(int row, int v) { return v ^ (row & 15); }

constexpr int kXcds = 8;

// The chunk loop and epilogue of one wide workgroup (block blk of expert e,
// this wave's pair), with the weight loads issued under cache policy kPolicy.
template <int S, bool kFc1, int kPolicy>
__device__ __forceinline__ void fc_wide_body(const FcArgs& a, const int e, const int pair, const int (&frow)[S],
                                             const int sf, const bool stager, const int srow, const int svec,
                                             uint4 (&xt)[2][16 * S][kRowVecs], f32x4_t (&xs4)[2][4][4 * S + 1]) {
  // A deeper ring does not fit: at 4 chunks the compiler spills, and a
  // scratch reload inside the loop waits for every weight load in flight.
  constexpr int P = kWideP;
  const int lane = threadIdx.x & 63;
  const int K = kFc1 ? a.H : a.I;
  const int N = kFc1 ? 2 * a.I : a.H;
  const int MK = a.M * a.k;

  const int n = K / kChunkK;
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
  // the activation loads and the sub-tile flags need (the scheduling barrier
  // keeps those waits below the loads).
  WChunk wb[P];
#pragma unroll
  for (int j = 0; j < P; ++j) wb[j] = load_w(j);
  __builtin_amdgcn_sched_barrier(0);
  // The row ids pass through empty volatile asm statements here: otherwise
  // the compiler hoists their uses (the same in both cache-policy copies of
  // this body) above the copies' branch, and so above the weight loads.
  int sfv = sf;
  asm volatile("" : "+v"(sfv));
  int frv[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    frv[s] = frow[s];
    asm volatile("" : "+v"(frv[s]));
  }

  bool sact[S];
#pragma unroll
  for (int s = 0; s < S; ++s) sact[s] = __builtin_amdgcn_readfirstlane(frv[s]) < MK;
  const int rows_total = kFc1 ? a.M : MK;
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.act_in, (uint32_t)rows_total * (uint32_t)K * 2u);
  const bool svalid = stager && sfv >= 0 && sfv < MK;
  const uint32_t soff = svalid ? ((uint32_t)(kFc1 ? sfv / a.k : sfv) * (uint32_t)K + 8u * svec) * 2u : kOutOfRange;
  auto load_x = [&](int c) { return bload16(xr, (c < n) ? soff + (uint32_t)c * (kChunkK * 2) : kOutOfRange); };
  // store one staged vector and its share of the group sum (4 vectors = 1 group)
  auto store_x = [&](uint4 v, int slot) {
    if (!stager) return;
    xt[slot][srow][xswz(srow, svec)] = v;
    const float corr = group_corr_quad(v);
    if ((svec & 3) == 0) reinterpret_cast<float*>(&xs4[slot][svec >> 2][0])[srow] = corr;
  };

  f32x4_t acc0[S], acc1[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    acc0[s] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    acc1[s] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  uint4 xg[P];
#pragma unroll
  for (int j = 0; j < P; ++j) xg[j] = load_x(j);
  store_x(xg[0], 0);
  __syncthreads();

  const int mrow = lane & 15, kv = lane >> 4;
  for (int c = 0; c < n; c += P) {
#pragma unroll
    for (int j = 0; j < P; ++j) {
      const int cc = c + j;
      if (cc < n) {
        const int slot = j & 1;  // == cc & 1 since c is a multiple of the even P
        xg[j] = load_x(cc + P);
        const WChunk w = wb[j];
        const uint32_t q0[4] = {w.q0.x, w.q0.y, w.q0.z, w.q0.w};
        const uint32_t q1[4] = {w.q1.x, w.q1.y, w.q1.z, w.q1.w};
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float g0 = group_scale(w.s0, g);
          const float g1 = group_scale(w.s1, g);
          const bf16x8_t b0 = dequant_group(q0[g], g0);
          const bf16x8_t b1 = dequant_group(q1[g], g1);
#pragma unroll
          for (int s = 0; s < S; ++s) {
            if (s > 0 && !sact[s]) continue;
            const bf16x8_t xv = as_bf16x8(xt[slot][16 * s + mrow][xswz(mrow, 4 * g + kv)]);
            if constexpr (kFmt == kFmtMxfp4) {  // scaled operand: accumulate in the MFMA
              acc0[s] = mfma16x16x32(xv, b0, acc0[s]);
              acc1[s] = mfma16x16x32(xv, b1, acc1[s]);
              continue;
            }
            const f32x4_t off = group_c(xs4[slot][g][4 * s + kv]);
            const f32x4_t t0 = mfma16x16x32(xv, b0, off);
            const f32x4_t t1 = mfma16x16x32(xv, b1, off);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              acc0[s][i] = group_add(acc0[s][i], t0[i], g0);
              acc1[s][i] = group_add(acc1[s][i], t1[i], g1);
            }
          }
          // keep the LDS reads of later groups from being hoisted (register pressure)
          __builtin_amdgcn_sched_barrier(0);
        }
        wb[j] = load_w(cc + P);
        if (cc + 1 < n) store_x(xg[(j + 1) % P], (j + 1) & 1);
        __syncthreads();
      }
    }
  }
  fc_epilogue<S, kFc1>(a, pair, frv, sact, acc0, acc1, lane);
}


template <int S, bool kFc1>
__global__ __launch_bounds__(64 * kWideNP) void fc_wide_kernel(FcArgs a) {
  constexpr int BM = 16 * S;
  constexpr int kThreads = 64 * kWideNP;
  constexpr int kItems = BM * kRowVecs;  // multiple of 64: whole waves stage or idle
  __shared__ uint4 xt[2][BM][kRowVecs];  // the block's activation chunk, double-buffered (swizzled)
  // -136 * group sums: [slot][group][4-row quad], one quad of padding per
  // group so that the four groups' stores of a row land in distinct banks
  __shared__ f32x4_t xs4[2][4][BM / 4 + 1];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int N = kFc1 ? 2 * a.I : a.H;
  const int npairs = N / kPairRows;
  const int MK = a.M * a.k;

  if constexpr (kFc1) {  // clear FC2's accumulator
    uint4* z = reinterpret_cast<uint4*>(a.acc);
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + tid; i < a.zero_words16; i += stride)
      z[i] = make_uint4(0, 0, 0, 0);
  }

  // the grid holds a multiple of 8 blocks; the ones past cap have no rows
  const int npg = npairs / kWideNP;
  const int xcd = blockIdx.x % kXcds, gi = blockIdx.x / kXcds;
  const int blk = (gi / npg) * kXcds + xcd;
  const int pair = (gi % npg) * kWideNP + wave;
  if ((int64_t)blk * BM >= a.cap) return;
  // All of the block's metadata is read in one round trip (the block list
  // entries of the neighbours too, for the cache policy below) before any
  // of it is used.
  // The loads are unconditional (indices clamped into range, the value then
  // dropped): a conditional load becomes a branch with a wait for every load
  // in flight.
  const int32_t* rows = a.sorted_ids + (int64_t)blk * BM;
  int frow[S];
#pragma unroll
  for (int s = 0; s < S; ++s) frow[s] = rows[16 * s + (lane & 15)];
  const bool stager = tid < kItems;
  const int srow = tid / kRowVecs, svec = tid % kRowVecs;
  const int sf0 = rows[stager ? srow : 0];
  const bool has_next = (int64_t)(blk + 1) * BM < a.cap;
  const int npp = __builtin_amdgcn_readfirstlane(*a.npp);
  const int e = __builtin_amdgcn_readfirstlane(a.block_expert[blk]);
  const int e_prev0 = __builtin_amdgcn_readfirstlane(a.block_expert[blk > 0 ? blk - 1 : blk]);
  const int e_next0 = __builtin_amdgcn_readfirstlane(a.block_expert[has_next ? blk + 1 : blk]);
  const int sf = stager ? sf0 : MK;
  const int e_prev = blk > 0 ? e_prev0 : -1;
  const int e_next = has_next ? e_next0 : -1;
  if (blk * BM >= npp) return;
  if (e < 0 || e >= a.E) return;

  // Weights are streamed non-temporally (read once per call) unless the
  // expert has more than one block: then its other blocks re-read them and
  // they are kept in the caches.
  const bool reuse = e_prev == e || ((blk + 1) * BM < npp && e_next == e);
  if (__builtin_amdgcn_readfirstlane((int)reuse))
    fc_wide_body<S, kFc1, kPolicyDefault>(a, e, pair, frow, sf, stager, srow, svec, xt, xs4);
  else
    fc_wide_body<S, kFc1, kPolicyWeights>(a, e, pair, frow, sf, stager, srow, svec, xt, xs4);
}

// FC1 of a small batch (M <= 16 tokens) with the routing and grouping done
// inside the kernel ("The Throughput Lever: Quantifying the MoE GEMM and
// Mapping the Road to B300", section "The B300 Analysis: When the Bottleneck
// Flips": at small batches the fixed per-step costs, a separate routing
// launch among them, weigh most).
//
// Prologue, once per workgroup: small_route (routing, ranks of the touched
// experts, block tables).
//
// Work: items (block, group of kRoutedSlots tile pairs), dealt round-robin
// to resident workgroups (one per CU). A workgroup's 16 waves are
// kRoutedSlots pairs x kRoutedKSplit K ranges. The batch's x rows (M <= 9 at
// H = 7168) are staged in LDS once, before the items: every block's rows are
// tokens of the batch, so each wave reads its A operand from there and keeps
// only weights in its register ring. The small items (the pairs of one
// block are split 32 ways) keep
// the last round short: with a few dozen experts touched, the wide kernel's
// 8 workgroups of 16 pairs per expert leave most CUs idle in a second round.
// A wave's last P chunk loads already fetch its next item's first chunks, so
// the weight stream does not drain across the partial-sum reduction and the
// epilogue.
//
// Workgroup 0 writes the routing and grouping outputs after its items,
// exactly as moe_route_align lays them out for block_m (FC2, their consumer,
// is the next kernel).
constexpr int kRoutedWaves = 16;
constexpr int kRoutedKSplit = 4;                            // waves per tile pair
constexpr int kRoutedSlots = kRoutedWaves / kRoutedKSplit;  // tile pairs per item
constexpr int kRoutedP = 2;                                 // weight chunks in flight per wave (divides NCH)
constexpr int kRoutedXPer = 9;               // x vectors staged per thread: M * H / 8 <= 9 * 1024
constexpr int kRoutedMaxXBytes = 128 * 1024;  // staged x rows (with the routing tables and partial sums: < 160 KB)

// One wave's share of an item: expert, tile pair, the row of lane % 16 and
// where its A operand starts in the staged rows.
struct RoutedWork {
  const uint8_t* w;  // this wave's first chunk of the pair
  uint32_t wbytes;   // bytes of a chunk to read: kPairChunkBytes, 0 for no item (reads zeros)
  int pair, frow;
  int xrow;          // LDS index of this lane's first 16 bytes (padding rows read token 0: never stored)
};

template <int VPL, int NCH>
__global__ __launch_bounds__(64 * kRoutedWaves) void fc1_routed_kernel(DecodeArgs d) {
  constexpr int P = kRoutedP, KS = kRoutedKSplit;
  constexpr int kThreads = 64 * kRoutedWaves;
  __shared__ SmallRoute sh;
  __shared__ f32x4_t red[kRoutedSlots][2][64];          // one K range's partial sums
  extern __shared__ uint4 xs[];                          // [M][H / 8 + 1]: the batch's x rows

  const FcArgs& a = d.fc;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kq = wave % KS, slot = wave / KS;
  const int M = a.M, E = a.E, k = a.k, MK = M * k, H = a.H;

  if (a.zero_words16 > 0) {  // clear FC2's accumulator when the grouped FC2 follows
    uint4* z = reinterpret_cast<uint4*>(a.acc);
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + tid; i < a.zero_words16; i += stride)
      z[i] = make_uint4(0, 0, 0, 0);
  }

  // The x rows: loads issued before the routing, stored to LDS after it
  // (rows padded by 16 bytes, so that rows start on different banks).
  const int hv = H / 8, row16 = hv + 1;
  const uint4* xg = reinterpret_cast<const uint4*>(a.act_in);
  uint4 xv[kRoutedXPer];
#pragma unroll
  for (int v = 0; v < kRoutedXPer; ++v) {
    const int i = tid + v * kThreads;
    xv[v] = i < M * hv ? xg[i] : make_uint4(0, 0, 0, 0);
  }
  const int nd = small_route<VPL, kThreads>(sh, d.logits, M, E, k);  // touched experts = blocks
#pragma unroll
  for (int v = 0; v < kRoutedXPer; ++v) {
    const int i = tid + v * kThreads;
    if (i < M * hv) xs[(i / hv) * row16 + i % hv] = xv[v];
  }
  __syncthreads();

  const int nkc = H / kChunkK;
  const int kc0 = kq * nkc / KS;
  const int n = NCH > 0 ? NCH : (kq + 1) * nkc / KS - kc0;  // this wave's chunks
  const int ipb = 2 * a.I / kPairRows / kRoutedSlots;        // items per block
  const int nitems = nd * ipb;
  const int64_t wexp = packed_bytes_per_expert(2 * a.I, H);
  const uint32_t oq0 = 16u * lane, oq1 = kTileBytes + 16u * lane;
  const uint32_t os0 = kTileNibbleBytes + kScaleRowBytes * (lane & 15);
  const uint32_t os1 = kTileBytes + kTileNibbleBytes + kScaleRowBytes * (lane & 15);

  auto work_of = [&](int item) {
    const int blk = item / ipb;
    RoutedWork r;
    r.pair = (item % ipb) * kRoutedSlots + slot;
    const int e = __builtin_amdgcn_readfirstlane(sh.blk_e[blk]);
    r.frow = sh.blk_rows[blk][lane & 15];
    r.w = a.wpacked + (int64_t)e * wexp + ((int64_t)r.pair * nkc + kc0) * kPairChunkBytes;
    r.wbytes = kPairChunkBytes;
    r.xrow = (r.frow < MK ? r.frow / k : 0) * row16 + kc0 * (kChunkK / 8) + (lane >> 4);
    return r;
  };
  // one buffer descriptor per chunk (scalar arithmetic); a chunk at or past
  // n has no bytes in range and reads zeros
  auto load_w = [&](const RoutedWork& r, int c) {
    const __amdgpu_buffer_rsrc_t wr =
        make_rsrc(r.w + (int64_t)c * kPairChunkBytes, c < n ? r.wbytes : 0u);
    WChunk w;
    w.q0 = bload16<kPolicyWeights>(wr, oq0);
    w.q1 = bload16<kPolicyWeights>(wr, oq1);
    w.s0 = load_scales<kPolicyWeights>(wr, os0);
    w.s1 = load_scales<kPolicyWeights>(wr, os1);
    return w;
  };
  // A operand of chunk c from the staged rows (a chunk past this wave's
  // range, whose weights read as zeros, re-reads chunk 0: any finite value)
  auto lds_x = [&](uint4 (&xa)[1][4], const RoutedWork& r, int c) {
    const int cc = c < n ? c : 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) xa[0][j] = xs[r.xrow + cc * (kChunkK / 8) + 4 * j];
  };

  const bf16x8_t neg136 = as_bf16x8(make_uint4(kNeg136Pair, kNeg136Pair, kNeg136Pair, kNeg136Pair));
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
  const bool sact[1] = {true};  // a touched expert has at least one row
  WChunk wb[P];
  int item = blockIdx.x;
  RoutedWork cur;
  if (item < nitems) {
    cur = work_of(item);
    if constexpr (NCH > 0) {
#pragma unroll
      for (int j = 0; j < P; ++j) wb[j] = load_w(cur, j);
    }
  }
  while (item < nitems) {
    const int next = item + (int)gridDim.x;
    const bool has_next = next < nitems;
    RoutedWork nx = cur;  // past the last item: loads of no bytes
    nx.wbytes = 0u;
    if (has_next) nx = work_of(next);
    f32x4_t acc0[1] = {zero4}, acc1[1] = {zero4};
    if constexpr (NCH > 0) {
      // straight-line (exact memory waits); the last P steps load the next
      // item's first chunks
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        uint4 xa[1][4];
        lds_x(xa, cur, c);
        mma_chunk<1>(wb[c % P], xa, sact, neg136, acc0, acc1);
        wb[c % P] = c + P < NCH ? load_w(cur, c + P) : load_w(nx, c + P - NCH);
        __builtin_amdgcn_sched_barrier(0);  // bound live ranges to one chunk
      }
    } else {
#pragma unroll
      for (int j = 0; j < P; ++j) wb[j] = load_w(cur, j);
      for (int c = 0; c < n; c += P) {
#pragma unroll
        for (int j = 0; j < P; ++j) {
          if (c + j < n) {
            uint4 xa[1][4];
            lds_x(xa, cur, c + j);
            mma_chunk<1>(wb[j], xa, sact, neg136, acc0, acc1);
          }
          wb[j] = load_w(cur, c + j + P);
        }
      }
    }
    // The K-range-0 wave of each pair adds the other ranges' partials in
    // range order, one range at a time through one LDS buffer (the LDS goes
    // to the staged rows), then runs the epilogue.
#pragma unroll
    for (int q = 1; q < KS; ++q) {
      if (kq == q) {
        red[slot][0][lane] = acc0[0];
        red[slot][1][lane] = acc1[0];
      }
      __syncthreads();
      if (kq == 0) {
        acc0[0] += red[slot][0][lane];
        acc1[0] += red[slot][1][lane];
      }
      __syncthreads();
    }
    if (kq == 0) {
      const int frow[1] = {cur.frow};
      fc_epilogue<1, true>(a, cur.pair, frow, sact, acc0, acc1, lane);
    }
    item = next;
    cur = nx;
  }

  if (blockIdx.x == 0)  // routing + grouping outputs, in block_m-row blocks
    small_route_write<kThreads>(sh, nd, M, E, k, d.block_m, d.topk_ids, d.topk_weights, d.sorted_ids,
                                d.block_expert, d.expert_offsets, d.npp_out);
}

// Workgroups of the routed FC1: one per compute unit (its register use
// allows one 16-wave workgroup per CU), at most one per work item.
// CU count of the current device, queried once per device (a benign race:
// every thread stores the same value).
constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];
inline int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < kMaxDevices) {
    const int c = g_cus[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 256;
  if (dev < kMaxDevices) g_cus[dev].store(cus, std::memory_order_relaxed);
  return cus;
}
inline int64_t routed_grid(int64_t max_items) {
  const int64_t cus = device_cus();
  return max_items < cus ? max_items : cus;
}

// Dynamic LDS of the routed FC1: the batch's x rows, padded.
inline uint32_t routed_x_bytes(int64_t M, int64_t H) { return (uint32_t)(M * (H / 8 + 1) * 16); }

// Raises the kernel's dynamic LDS limit (64 KB by default) once.
template <typename Kernel>
hipError_t allow_lds(Kernel kernel, uint32_t bytes) {
  static std::atomic<uint32_t> allowed{0};
  if (bytes <= 64 * 1024 || bytes <= allowed.load(std::memory_order_relaxed)) return hipSuccess;
  const hipError_t e =
      hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)kRoutedMaxXBytes);
  if (e == hipSuccess) allowed.store(kRoutedMaxXBytes, std::memory_order_relaxed);
  return e;
}

template <int VPL, int NCH>
hipError_t launch_routed(const DecodeArgs& d, unsigned grid, hipStream_t stream, hipEvent_t e0, hipEvent_t e1) {
  const uint32_t xbytes = routed_x_bytes(d.fc.M, d.fc.H);
  const hipError_t e = allow_lds(fc1_routed_kernel<VPL, NCH>, xbytes);
  if (e != hipSuccess) return e;
  launch_kernel(fc1_routed_kernel<VPL, NCH>, grid, 64 * kRoutedWaves, xbytes, stream, e0, e1, d);
  return hipGetLastError();
}

template <int VPL>
hipError_t launch_routed_vpl(const DecodeArgs& d, hipStream_t stream, hipEvent_t e0, hipEvent_t e1) {
  const int64_t MK = (int64_t)d.fc.M * d.fc.k;
  const int64_t nblk = MK < d.fc.E ? MK : d.fc.E;
  const unsigned grid = (unsigned)routed_grid(nblk * (2 * d.fc.I / kPairRows / kRoutedSlots));
  const int nkc = d.fc.H / kChunkK;
  // straight-line chunk loops for K ranges of 2 and 14 chunks (H = 1024, 7168)
  if (nkc == 2 * kRoutedKSplit) return launch_routed<VPL, 2>(d, grid, stream, e0, e1);
  if (nkc == 14 * kRoutedKSplit) return launch_routed<VPL, 14>(d, grid, stream, e0, e1);
  return launch_routed<VPL, 0>(d, grid, stream, e0, e1);
}

// block_m = 128 on the block kernels, which take blocks of up to 64 rows:
// each block is run as its two 64-row halves. half[h] = the expert of half
// h, or -1 where it holds no row (an expert's padding is at the end of its
// range, so a half whose first row is padding is all padding) or lies past
// the padded total.
__global__ __launch_bounds__(256) void half_block_kernel(const int32_t* __restrict__ block_expert,
                                                         const int32_t* __restrict__ sorted_ids,
                                                         const int32_t* __restrict__ npp_p, int MK, int64_t nhalf,
                                                         int32_t* __restrict__ half) {
  const int64_t h = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (h >= nhalf) return;
  int e = -1;
  if (h * 64 < *npp_p && sorted_ids[h * 64] < MK) e = block_expert[h >> 1];
  half[h] = e;
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
void launch(const FcArgs& a, unsigned grid, hipStream_t stream, hipEvent_t e0, hipEvent_t e1) {
  const int nkc = (kFc1 ? a.H : a.I) / kChunkK;
  constexpr int kNchFc1 = 56 / KSPLIT, kNchFc2 = 16 / KSPLIT;
  constexpr int kNch = kFc1 ? kNchFc1 : kNchFc2;
  if constexpr (S == 1 && kNch >= P) {  // unrolled code only fits registers for one sub-tile
    if (nkc == kNch * KSPLIT) {
      launch_kernel(fc_kernel<S, KSPLIT, P, kNch, kFc1>, grid, 64 * KSPLIT, 0, stream, e0, e1, a);
      return;
    }
  }
  launch_kernel(fc_kernel<S, KSPLIT, P, 0, kFc1>, grid, 64 * KSPLIT, 0, stream, e0, e1, a);
}

template <bool kFc1>
hipError_t launch_fc(const FcArgs& a, hipStream_t stream, hipEvent_t e0, hipEvent_t e1) {
  if (a.tiles) {  // tiled path: FC1 first writes the tile table FC2 reuses
    hipError_t err = hipSuccess;
    if constexpr (kFc1) err = launch_tile_plan(a, stream);
    // INT4 reads fp16 copies of its A rows (x for FC1, the activations for
    // FC2), each row scaled by a power of two
    FcArgs b = a;
    if constexpr (kFmt == kFmtInt4) {
      if (err == hipSuccess)
        err = launch_rowscale(a.act_in, kFc1 ? a.M : (int64_t)a.M * a.k, kFc1 ? a.H : a.I, a.a16, a.a16_exp, stream);
      b.act_in = a.a16;
      b.row_exp = a.a16_exp;
    }
    if (err == hipSuccess) err = launch_fc_prescaled<kFc1>(b, stream, e0, e1);
    if (err != hipSuccess || kFc1) return err;
    const int64_t n8 = (int64_t)a.M * a.H / 8;
    finalize_kernel<<<(unsigned)((n8 + 255) / 256), 256, 0, stream>>>(a.acc, a.out, n8);
    return hipGetLastError();
  }
  if (a.block_m == 128) {  // the 64-row kernels on each half of a block
    if (a.half_expert == nullptr || a.cap % 128 != 0) return hipErrorInvalidValue;
    const int64_t nhalf = a.cap / 64;
    half_block_kernel<<<(unsigned)((nhalf + 255) / 256), 256, 0, stream>>>(a.block_expert, a.sorted_ids, a.npp,
                                                                         a.M * a.k, nhalf, a.half_expert);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    FcArgs b = a;
    b.block_expert = a.half_expert;
    b.block_m = 64;
    return launch_fc<kFc1>(b, stream, e0, e1);
  }
  const int N = kFc1 ? 2 * a.I : a.H;
  const int64_t nblk = a.cap / a.block_m;
  const int64_t grid = nblk * (N / kPairRows);
  if (grid <= 0 || grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  const bool wide = (N / kPairRows) % kWideNP == 0;  // pairs split evenly over the wide workgroups
  const unsigned wgrid = (unsigned)((nblk + kXcds - 1) / kXcds * kXcds * (N / kPairRows / kWideNP));
  switch (a.block_m) {
    case 16: launch<1, 4, 3, kFc1>(a, (unsigned)grid, stream, e0, e1); break;
    case 32:
      if (wide) launch_kernel(fc_wide_kernel<2, kFc1>, wgrid, 64 * kWideNP, 0, stream, e0, e1, a);
      else launch<2, 4, 2, kFc1>(a, (unsigned)grid, stream, e0, e1);
      break;
    case 64:
      if (wide) launch_kernel(fc_wide_kernel<4, kFc1>, wgrid, 64 * kWideNP, 0, stream, e0, e1, a);
      else launch<4, 4, 2, kFc1>(a, (unsigned)grid, stream, e0, e1);
      break;
    default: return hipErrorInvalidValue;
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || kFc1) return err;
  const int64_t n8 = (int64_t)a.M * a.H / 8;
  finalize_kernel<<<(unsigned)((n8 + 255) / 256), 256, 0, stream>>>(a.acc, a.out, n8);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fc1(const FcArgs& a, hipStream_t stream, hipEvent_t ev_start, hipEvent_t ev_stop) {
  return launch_fc<true>(a, stream, ev_start, ev_stop);
}
hipError_t launch_fc2(const FcArgs& a, hipStream_t stream) { return launch_fc<false>(a, stream, nullptr, nullptr); }

bool routed_fc1_fits(int64_t M, int64_t E, int64_t H, int64_t I, int64_t k) {
  return M >= 1 && M <= kSmallMaxTokens && M * k <= kSmallMaxAssign && E <= kSmallMaxExperts &&
         (2 * I / kPairRows) % kRoutedSlots == 0 && M * (H / 8) <= (int64_t)kRoutedXPer * 64 * kRoutedWaves &&
         routed_x_bytes(M, H) <= (uint32_t)kRoutedMaxXBytes;
}

bool routed_fc1_preferred(int64_t M, int64_t E, int64_t H, int64_t I, int64_t k) {
  if (!routed_fc1_fits(M, E, H, I, k)) return false;
  // Per CU the routed kernel streams somewhat slower than the wide kernel;
  // it wins while the wide kernel's workgroups (16 pairs of one expert
  // each, for the expected number of distinct experts) would fill at most
  // 1.75 rounds of the CUs. On the 384-expert top-8 layer (measured, layer
  // call): M = 3 ... 7 by 4-8 %, M = 8 and 9 even (1.9 and 2.1 rounds).
  double miss = 1.0;  // probability that an expert is not among M tokens' top-k (uniform routing)
  for (int64_t t = 0; t < M; ++t) miss *= 1.0 - (double)k / (double)E;
  const double wide_wgs = (double)E * (1.0 - miss) * (double)(2 * I / kPairRows) / kWideNP;
  return wide_wgs <= 1.75 * device_cus();
}

hipError_t launch_fc1_routed(const DecodeArgs& d, hipStream_t stream, hipEvent_t ev_start, hipEvent_t ev_stop) {
  const int E = d.fc.E;
  if (E <= 64) return launch_routed_vpl<1>(d, stream, ev_start, ev_stop);
  if (E <= 128) return launch_routed_vpl<2>(d, stream, ev_start, ev_stop);
  if (E <= 256) return launch_routed_vpl<4>(d, stream, ev_start, ev_stop);
  if (E <= 384) return launch_routed_vpl<6>(d, stream, ev_start, ev_stop);
  if (E <= 512) return launch_routed_vpl<8>(d, stream, ev_start, ev_stop);
  return launch_routed_vpl<16>(d, stream, ev_start, ev_stop);
}

}  // namespace MOE_FMT_NS
}  // namespace moe

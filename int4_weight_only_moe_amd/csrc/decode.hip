// Decode path of the layer for tiny batches (M <= 4 tokens, M*k <= 64):
// two kernels instead of four.
//
// "The Throughput Lever: Quantifying the MoE GEMM and Mapping the Road to
// B300", section "The B300 Analysis: When the Bottleneck Flips": once the
// MoE GEMM runs at HBM speed, fixed per-step overheads (launches among them)
// dominate a decode step, and at M = 1 only ~8 of 384 experts are touched
// (section "The Result: Two Regimes"). On gfx950 every kernel boundary costs
// a few microseconds of dispatch and cache maintenance, so for M <= 4:
//
//   fc1_decode_kernel  each workgroup first routes the whole batch itself
//                      (one wave per token, top-k kept in LDS), takes the
//                      distinct experts in order of first occurrence and the
//                      rows of the block it owns, then runs the FC1 tile body
//                      of the grouped GEMM; workgroup 0 also writes the
//                      routing and grouping outputs (experts ascending) in
//                      the format moe_route_align produces. For one token
//                      every wave routes it only as far as its own slot and
//                      issues its weight loads before the row is staged.
//   fc2_decode_kernel  output-stationary FC2: one workgroup per (token,
//                      32-column tile pair of the output; for top-k > 8 one
//                      16-column tile), one wave per (routing slot j, tile)
//                      streaming the W2 tile of expert ids[t, j]; the k slot
//                      results of a tile meet in LDS and are summed in slot
//                      order with their routing weights, then rounded once to
//                      bf16. A pair per workgroup reads whole 2304-byte
//                      chunks, and at M = 1 gives 224 equal workgroups rather
//                      than 448 on 256 CUs. No atomics, no accumulator to
//                      clear, no finalize kernel, and the float result is
//                      deterministic. (The layer call also runs it after the
//                      grouped FC1 for small batches.)
// Each expert is read once per token that routes to it; with M <= 4 tokens
// and top-8 of 384 experts, repeats are rare, so the weight traffic stays the
// touched experts' bytes.
#include "internal.h"
#include "device_common.h"
#include "fc_common.h"
#include "route_common.h"

namespace moe {
namespace MOE_FMT_NS {
namespace {

constexpr int kDecKSplit = 4;   // FC1 waves per workgroup (split K)
// FC1 chunks in flight per wave (fewer for 3-4 rows: their sums need the registers)
constexpr int dec_p1(int rows) { return rows <= 2 ? 4 : 3; }

// The decode batch's routing in LDS (M <= 4 tokens, M*k <= 64 assignments).
struct DecodeRoute {
  int32_t ids[kDecodeMaxAssign];
  float w[kDecodeMaxAssign];
  int32_t list[kDecodeMaxAssign];                    // distinct experts, ascending
  int32_t cnt[kDecodeMaxAssign];                     // assignments per distinct expert
  int32_t rowf[kDecodeMaxAssign][kDecodeMaxTokens];  // their f, ascending
};

// FC1 of one (expert, tile pair) for the MR = M <= 4 tokens of the batch:
// D row r is token r, whether or not it routes to expert e (the MFMA computes
// 16 rows anyway; only the rows of tokens that route to e are stored). Lane
// l < 16 holds D rows 0..3 of column l of both tiles; lanes 16..63 hold
// padding rows, so only lanes 0..15 load scales and only the MR token rows
// are scaled into the sums. The A operand of lane l is the staged x row of
// token l % 16 (token 0 for padding rows: finite values whose D rows are
// never used). The accumulator input of each group's MFMA is the staged
// -136 * (group sum) of the four token rows (xcorr4[group] = one float per
// token, zero past M), so that every MFMA is a product with the weights.
// tokf: lane r < MR holds the assignment f of token r to expert e, or -1.
// pre() runs once the first weight loads are in flight; when it returns, the
// rows and corrections must be staged and visible to every wave (barrier).
template <int MR, int NCH, typename Pre>
__device__ __forceinline__ void fc1_decode_body(const DecodeArgs& d, const uint4* __restrict__ xs, int row16,
                                                const f32x4_t* __restrict__ xcorr4, const int e, const int pair,
                                                const int tokf, const int wave, const int lane, Pre&& pre) {
  const FcArgs& a = d.fc;
  const int H = a.H, I = a.I;
  const int nkc = H / kChunkK;
  // The waves take the pair's chunks in turn (wave w: chunks w, w + 4, ...),
  // so a workgroup reads its pair as one contiguous stream (measured: 4
  // separate 32 KB streams per workgroup left waves 1-3 far behind wave 0).
  const int n = NCH > 0 ? NCH : (nkc - wave + kDecKSplit - 1) / kDecKSplit;
  constexpr int64_t kStride = (int64_t)kDecKSplit * kPairChunkBytes;

  const uint8_t* wbase = a.wpacked + (int64_t)e * packed_bytes_per_expert(2 * I, H) +
                         ((int64_t)pair * nkc + wave) * kPairChunkBytes;
  const uint32_t oq0 = 16u * lane, oq1 = kTileBytes + 16u * lane;
  // INT4: lanes 16..63 read their scales out of range (zeros, no memory
  // access): the scale multiplies D rows, which lanes 0..15 hold. FP4: the
  // scale enters the B operand, whose column lane % 16 every lane supplies.
  const bool own_scales = kFmt == kFmtMxfp4 || lane < 16;
  const uint32_t os0 = own_scales ? kTileNibbleBytes + kScaleRowBytes * (lane & 15) : kOutOfRange;
  const uint32_t os1 = own_scales ? kTileBytes + kTileNibbleBytes + kScaleRowBytes * (lane & 15) : kOutOfRange;

  // x of this lane's row, at this wave's first chunk and this lane's K offset
  const int xrow = (lane & 15) < MR ? (lane & 15) : 0;
  const uint4* xl = xs + xrow * row16 + wave * (kChunkK / 8) + (lane >> 4);
  const f32x4_t* cr = xcorr4 + wave * (kChunkK / kGroup);  // this wave's first group

  // One buffer descriptor per chunk (scalar arithmetic), so the per-lane
  // offsets stay four constant registers; a chunk at or past n has no
  // bytes in range and reads zeros.
  auto load_w = [&](int c) {
    const __amdgpu_buffer_rsrc_t wr =
        make_rsrc(wbase + (int64_t)c * kStride, c < n ? (uint32_t)kPairChunkBytes : 0u);
    WChunk w;
    w.q0 = bload16<kPolicyWeights>(wr, oq0);
    w.q1 = bload16<kPolicyWeights>(wr, oq1);
    w.s0 = load_scales<kPolicyWeights>(wr, os0);
    w.s1 = load_scales<kPolicyWeights>(wr, os1);
    return w;
  };

  constexpr int P = dec_p1(MR);
  float acc0[MR], acc1[MR];
#pragma unroll
  for (int i = 0; i < MR; ++i) acc0[i] = acc1[i] = 0.f;

  auto chunk = [&](const WChunk& w, int c) {
    const uint32_t q0[4] = {w.q0.x, w.q0.y, w.q0.z, w.q0.w};
    const uint32_t q1[4] = {w.q1.x, w.q1.y, w.q1.z, w.q1.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x8_t xv = as_bf16x8(xl[c * kDecKSplit * (kChunkK / 8) + 4 * j]);
      const float g0 = group_scale(w.s0, j);
      const float g1 = group_scale(w.s1, j);
      const bf16x8_t b0 = dequant_group(q0[j], g0);
      const bf16x8_t b1 = dequant_group(q1[j], g1);
      const f32x4_t off = group_c(cr[c * kDecKSplit * (kChunkK / kGroup) + j]);
      const f32x4_t t0 = mfma16x16x32(xv, b0, off);
      const f32x4_t t1 = mfma16x16x32(xv, b1, off);
#pragma unroll
      for (int i = 0; i < MR; ++i) {
        acc0[i] = group_add(acc0[i], t0[i], g0);
        acc1[i] = group_add(acc1[i], t1[i], g1);
      }
    }
  };

  WChunk wb[P];
#pragma unroll
  for (int j = 0; j < P; ++j) wb[j] = load_w(j);
  pre();  // work that may overlap the first weight loads (it must leave xs staged)
  if constexpr (NCH > 0) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      chunk(wb[c % P], c);
      if (c + P < NCH) wb[c % P] = load_w(c + P);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    for (int c = 0; c < n; c += P) {
#pragma unroll
      for (int j = 0; j < P; ++j) {
        if (c + j < n) chunk(wb[j], c + j);
        wb[j] = load_w(c + j + P);
      }
    }
  }

  // K-split partials of the real rows meet in LDS; wave 0 finishes.
  __shared__ float red[kDecKSplit - 1][2][MR][16];
  if (wave > 0 && lane < 16) {
#pragma unroll
    for (int i = 0; i < MR; ++i) {
      red[wave - 1][0][i][lane] = acc0[i];
      red[wave - 1][1][i][lane] = acc1[i];
    }
  }
  __syncthreads();
  if (wave != 0 || lane >= 16) return;
#pragma unroll
  for (int w = 0; w < kDecKSplit - 1; ++w) {
#pragma unroll
    for (int i = 0; i < MR; ++i) {
      acc0[i] += red[w][0][i][lane];
      acc1[i] += red[w][1][i][lane];
    }
  }
#pragma unroll
  for (int i = 0; i < MR; ++i) {
    const int f = __builtin_amdgcn_readlane(tokf, i);  // token i's assignment to e
    if (f < 0) continue;
    const float g = acc0[i], u = acc1[i];
    const float v = g / (1.0f + __expf(-g)) * u;
    a.act_out[(int64_t)f * I + 16 * pair + lane] = (uint16_t)f32_to_bf16_bits(v);
  }
}

// x rows staged per thread before the routing (H = 7168: 896 16-byte vectors
// per row, at most 4 per thread); for M > 2 the registers this takes are
// needed by the routing, so the rows are loaded after it.
constexpr int kXPerThread = 4;
constexpr int kXEarlyRows = 2;

template <int VPL, int NCH, int MR>
__global__ __launch_bounds__(64 * kDecKSplit) __attribute__((amdgpu_waves_per_eu(4)))
void fc1_decode_kernel(DecodeArgs d) {
  __shared__ DecodeRoute sh;
  extern __shared__ uint4 xs[];  // [M][row16]: the batch's x rows, then xcorr
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int M = d.fc.M, E = d.fc.E, k = d.fc.k, H = d.fc.H;
  const int MK = M * k;
  const int npairs = d.fc.I / 16;
  const int blk = blockIdx.x / npairs;
  // Pair index rotated per slot (a bijection within each slot): a CU's
  // resident workgroups, blockIdx.x apart by the CU count, would otherwise all
  // read the same offset of different experts, whose bases are 64 KB
  // multiples; rotated, they read unrelated offsets (measured ~1 % faster).
  const int pair = (int)((blockIdx.x % npairs + (unsigned)blk * 37u) % (unsigned)npairs);
  const int hv = H / 8;        // 16-byte vectors per x row
  const int row16 = hv + 1;    // padded LDS row stride: rows start on different banks
  const int ng = H / kGroup;   // quantisation groups per row
  // [ng] x 4 tokens: -136 * group sums, zero for tokens past M
  f32x4_t* xcorr4 = reinterpret_cast<f32x4_t*>(xs + M * row16);
  float* xcorr = reinterpret_cast<float*>(xcorr4);
  const uint4* xg = reinterpret_cast<const uint4*>(d.fc.act_in);

  // One token: the logits go out first (the routing is the critical path),
  // then the x loads, which do not depend on the routing.
  float lg[VPL];
  if constexpr (MR == 1) topk_load<VPL>(d.logits, E, lg);
  constexpr bool kEarly = NCH > 0 && MR <= kXEarlyRows;
  uint4 xr[MR][kXPerThread];
  if constexpr (kEarly) {
    // unconditional (indices past the row read its last vector, which the
    // staging does not store): as a conditional load each would be waited for
    // where its branch joins, before the routing
#pragma unroll
    for (int r = 0; r < MR; ++r)
#pragma unroll
      for (int v = 0; v < kXPerThread; ++v) {
        const int i = threadIdx.x + v * 64 * kDecKSplit;
        xr[r][v] = xg[(int64_t)r * hv + (i < hv ? i : hv - 1)];
      }
  }

  // Staging of the rows and their group corrections, then a barrier.
  auto stage = [&]() {
    // Stage the rows and their group corrections: the 4 vectors of a group sit
    // in 4 consecutive threads (hv and the block size are multiples of 4, so a
    // quad is either wholly inside a row or wholly past its end).
    if constexpr (kEarly) {
  #pragma unroll
      for (int r = 0; r < MR; ++r)
  #pragma unroll
        for (int v = 0; v < kXPerThread; ++v) {
          const int i = threadIdx.x + v * 64 * kDecKSplit;
          const float corr = group_corr_quad(xr[r][v]);
          if (i < hv) {
            xs[r * row16 + i] = xr[r][v];
            if ((i & 3) == 0) xcorr[4 * (i >> 2) + r] = corr;
          }
        }
    } else {
      for (int i = threadIdx.x; i < M * hv; i += blockDim.x) {
        const uint4 v = xg[i];
        const int r = i / hv, c = i % hv;
        xs[r * row16 + c] = v;
        const float corr = group_corr_quad(v);
        if ((c & 3) == 0) xcorr[4 * (c >> 2) + r] = corr;
      }
    }
    if (M < kDecodeMaxTokens)
      for (int g = threadIdx.x; g < ng; g += blockDim.x)
        for (int r = M; r < kDecodeMaxTokens; ++r) xcorr[4 * g + r] = 0.f;
    __syncthreads();
  };
  // The grouping of the routed batch (from sh.ids, after the barrier):
  // workgroup 0 writes the routing and grouping outputs.
  auto group = [&](int& e, unsigned long long& firsts) {
    // Assignment f sits in lane f. `before` = earlier assignments of the same
    // expert (its row within the expert's block), `first` = first occurrence.
    // A token never repeats an expert, so for M = 1 every lane is a first.
    e = (lane < MK) ? sh.ids[lane] : -1;
    int before = 0, tot = 1;
    if (M > 1) {
      tot = 0;
      for (int j = 0; j < MK; ++j) {
        const int ej = __builtin_amdgcn_readlane(e, j);
        tot += (ej == e) ? 1 : 0;
        before += (j < lane && ej == e) ? 1 : 0;
      }
    }
    const bool first = e >= 0 && before == 0;
    firsts = __ballot(first);
    const int nd = __builtin_popcountll(firsts);

    if (blockIdx.x == 0) {  // routing + grouping outputs, block_m-padded like moe_route_align
      int rank = 0;         // distinct experts smaller than e: the ascending order
      for (int j = 0; j < MK; ++j) {
        const int ej = __builtin_amdgcn_readlane(e, j);
        rank += (((firsts >> j) & 1ull) && ej < e) ? 1 : 0;
      }
      const int B = d.block_m;
      if (wave == 0 && e >= 0) {
        sh.rowf[rank][before] = lane;
        if (first) {
          sh.list[rank] = e;
          sh.cnt[rank] = tot;
        }
      }
      __syncthreads();
      for (int i = threadIdx.x; i < MK; i += blockDim.x) {
        d.topk_ids[i] = sh.ids[i];
        d.topk_weights[i] = sh.w[i];
      }
      for (int x = threadIdx.x; x <= E; x += blockDim.x) {
        int below = 0;
        for (int q = 0; q < nd; ++q) below += (sh.list[q] < x) ? 1 : 0;
        d.expert_offsets[x] = B * below;  // every touched expert holds <= M <= B rows: one block
      }
      if (threadIdx.x == 0) *d.npp_out = B * nd;
      for (int pos = threadIdx.x; pos < nd * B; pos += blockDim.x) {
        const int q = pos / B, r = pos % B;
        d.sorted_ids[pos] = (r < sh.cnt[q]) ? sh.rowf[q][r] : MK;
      }
      for (int q = threadIdx.x; q < nd; q += blockDim.x) d.block_expert[q] = sh.list[q];
    }
    return nd;
  };

  if constexpr (MR == 1) {
    // One token: its k experts are distinct and workgroup blk takes slot blk.
    // Every wave routes the token itself and stops at its slot's take, so its
    // weight loads go out before the row is staged and without waiting for
    // the other slots; wave 0 of workgroup 0 routes completely (the routing
    // outputs).
    const bool full = blockIdx.x == 0 && wave == 0;
    uint32_t key[VPL];
    topk_keys_of<VPL>(lg, E, key);
    const int rounds = full ? k : blk + 1;
    __builtin_assume(rounds >= 1);  // else the logits loads are sunk below the x loads, into the rounds' branch
    const int eb = topk_route_keys<VPL>(key, 0, k, rounds, blk, full ? sh.ids : nullptr, sh.w);
    const int tokf = lane == 0 ? blk : -1;
    fc1_decode_body<MR, NCH>(d, xs, row16, xcorr4, eb, pair, tokf, wave, lane, [&]() {
      stage();
      if (blockIdx.x == 0) {
        int e;
        unsigned long long firsts;
        (void)group(e, firsts);
      }
    });
  } else {
    if (wave < M) topk_token<VPL>(d.logits, wave, E, k, sh.ids, sh.w);
    stage();
    int e;
    unsigned long long firsts;
    const int nd = group(e, firsts);
    if (blk >= nd) return;
    // FC1 takes the distinct experts in order of first occurrence: block blk is
    // the expert of the blk-th first occurrence
    unsigned long long mb = firsts;
    for (int i = 0; i < blk; ++i) mb &= mb - 1;
    const int eb = __builtin_amdgcn_readlane(e, __builtin_ctzll(mb));
    // lane r < M: the assignment of token r to expert eb (a token lists an expert at most once)
    int tokf = -1;
    if (lane < M)
      for (int j = 0; j < k; ++j) tokf = (sh.ids[lane * k + j] == eb) ? lane * k + j : tokf;
    fc1_decode_body<MR, NCH>(d, xs, row16, xcorr4, eb, pair, tokf, wave, lane, []() {});
  }
}

// One 16-row tile of a pair, for one activation row (D row 0, lanes 0..15):
// per group, one MFMA of the row with the codes (INT4: q + 136; FP4: the
// scaled values), all four issued back to back; then, for INT4, each group's
// -136 * (group sum) correction (cr, one float per group, the same for every
// lane) is added and the sum scaled; each group keeps its own running sum
// (no dependence between the groups).
__device__ __forceinline__ void mma_chunk_tile(uint4 q, uint2 sc, const uint4 (&xa)[4], const float4 cr,
                                               float (&accj)[4]) {
  const uint32_t qq[4] = {q.x, q.y, q.z, q.w};
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
  float g[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) g[j] = group_scale(sc, j);
  f32x4_t t[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) t[j] = mfma16x16x32(as_bf16x8(xa[j]), dequant_group(qq[j], g[j]), zero4);
  const float crj[4] = {cr.x, cr.y, cr.z, cr.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if constexpr (kFmt == kFmtMxfp4)
      accj[j] += t[j][0];  // the scale is in the B operand; FP4 needs no correction
    else
      accj[j] = __builtin_fmaf(t[j][0] + crj[j], g[j], accj[j]);
  }
}

// ROWV: 16-byte vectors of the activation row each lane stages, when the
// launcher knows it (I = 64 * 8 * ROWV); 0 = any I (staged by a loop).
// TPW = 16-column tiles per workgroup: 2 = both tiles of a pair (waves
// w < k take tile 0, the others tile 1), so that a workgroup reads the pair's
// chunks whole (2304 contiguous bytes) rather than every other 1152 bytes.
template <int ROWV, int KW, int TPW>  // KW: waves per workgroup the launch bounds allow (>= TPW * top_k)
__global__ __launch_bounds__(64 * KW) __attribute__((amdgpu_waves_per_eu(4)))
void fc2_decode_kernel(DecodeArgs d) {
  // The activation row (I bf16) of each routing slot is staged in LDS once,
  // with its -136 * (group sum) corrections; per chunk the A operand comes
  // from LDS, so registers hold only the weight stream.
  extern __shared__ uint4 xrows[];  // [k][I / 8], then the corrections [k][I / 32] (one float each)
  __shared__ float part[KW][16];
  const int lane = threadIdx.x & 63;
  const FcArgs& a = d.fc;
  const int H = a.H, I = a.I, k = a.k;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = w % k, hh = w / k;  // routing slot, tile within the workgroup
  const int ngrp = H / (16 * TPW);
  const int t = blockIdx.x / ngrp;
  const int tile = (blockIdx.x % ngrp) * TPW + hh;
  const int pair = tile >> 1, h = tile & 1;
  const bool stager = hh == 0;  // one wave per slot stages the row
  const int f = t * k + j;
  const int row16 = I / 8;
  const int ng = I / kGroup;
  // The activation row does not depend on the routing: its loads go out
  // before the wait for this slot's expert id (which the weight stream needs).
  const uint4* src = reinterpret_cast<const uint4*>(a.act_in) + (int64_t)f * row16;
  uint4 xs[ROWV > 0 ? ROWV : 1];
  if constexpr (ROWV > 0) {
    if (stager) {
#pragma unroll
      for (int r = 0; r < ROWV; ++r) xs[r] = src[lane + 64 * r];
    }
  }
  const int ef = __builtin_amdgcn_readfirstlane(d.topk_ids[f]);
  const bool ok = ef >= 0 && ef < a.E;  // always, for ids from the routing kernels
  const int e = ok ? ef : 0;
  const float wf = ok ? d.topk_weights[f] : 0.f;  // 0: an invalid id contributes nothing

  const int n = I / kChunkK;
  const uint8_t* wbase = a.wpacked + (int64_t)e * packed_bytes_per_expert(H, I) +
                         (int64_t)pair * n * kPairChunkBytes + h * kTileBytes;
  // Only D row 0 (lanes 0..15) is used: for INT4 lanes 16..63 read their
  // scales out of range (zeros, no memory access); FP4 scales enter the B
  // operand, whose column lane % 16 every lane supplies.
  const uint32_t oq = 16u * lane;
  const uint32_t os = (kFmt == kFmtMxfp4 || lane < 16) ? kTileNibbleBytes + kScaleRowBytes * (lane & 15) : kOutOfRange;
  uint4* dst = xrows + j * row16;
  float* corr = reinterpret_cast<float*>(xrows + k * row16) + j * ng;

  constexpr int P2 = KW > 8 ? 2 : 6;  // chunks in flight per wave: with 16 waves, 2 measured best (4: +3 %, 6: +13 %)
  uint4 qb[P2];
  uint2 sb[P2];
  auto load = [&](int slot, int c) {  // a chunk past the K range has no bytes in range: zeros
    const __amdgpu_buffer_rsrc_t wr =
        make_rsrc(wbase + (int64_t)c * kPairChunkBytes, c < n ? (uint32_t)kTileBytes : 0u);
    qb[slot] = bload16<kPolicyWeights>(wr, oq);
    sb[slot] = load_scales<kPolicyWeights>(wr, os);
  };
  // Issue order: the activation row, then the first P2 weight chunks, so that
  // staging the row waits only for its own loads.
  if constexpr (ROWV > 0) {
#pragma unroll
    for (int s = 0; s < P2; ++s) load(s, s);
    if (stager) {
#pragma unroll
      for (int r = 0; r < ROWV; ++r) {
        dst[lane + 64 * r] = xs[r];
        const float cg = group_corr_quad(xs[r]);
        if ((lane & 3) == 0) corr[(lane + 64 * r) >> 2] = cg;
      }
    }
  } else {
    if (stager) {
      // row16 is a multiple of 4: a quad of lanes is wholly inside the row or past it
      for (int i = lane; i < row16; i += 64) {
        const uint4 v = src[i];
        dst[i] = v;
        const float cg = group_corr_quad(v);
        if ((i & 3) == 0) corr[i >> 2] = cg;
      }
    }
#pragma unroll
    for (int s = 0; s < P2; ++s) load(s, s);
  }
  // With one tile per workgroup each wave reads back only the row it staged
  // itself (a wave's LDS operations complete in order): no barrier. With two,
  // the second tile's waves read rows the first tile's waves staged.
  if constexpr (TPW > 1) __syncthreads();
  // lane l reads K values 8*(l/16).. of each group; every A row is the token's
  // row (rows 1..15 of D are not used), so no lane needs a zero fill
  const uint4* xl = dst + (lane >> 4);

  // The LDS operands of chunk c + 1 are read before chunk c is computed
  // (the last chunk re-reads its own: no branch, no read past the row).
  const float4* corr4 = reinterpret_cast<const float4*>(corr);  // 4 groups = one chunk
  uint4 xn[4];
  float4 crn;
  auto lds_load = [&](int cc) {
#pragma unroll
    for (int g = 0; g < 4; ++g) xn[g] = xl[cc * (kChunkK / 8) + 4 * g];
    crn = corr4[cc];
  };
  lds_load(0);
  float accj[4] = {0.f, 0.f, 0.f, 0.f};
  // A loop, not straight-line code: unrolled, the scheduler hoists every
  // chunk's LDS reads and spills; looped, the memory waits stay exact because
  // the only loads in flight are the weight ring's.
  for (int c = 0; c < n; c += P2) {
#pragma unroll
    for (int s = 0; s < P2; ++s) {
      const int cc = c + s;
      if (cc < n) {
        uint4 xa[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) xa[g] = xn[g];
        const float4 cr = crn;
        lds_load(cc + 1 < n ? cc + 1 : cc);
        mma_chunk_tile(qb[s], sb[s], xa, cr, accj);
      }
      load(s, cc + P2);
    }
  }
  const float acc = (accj[0] + accj[1]) + (accj[2] + accj[3]);
  // D row 0 (the token) sits in lanes 0..15, element 0
  if (lane < 16) part[w][lane] = wf * acc;
  __syncthreads();
  if (threadIdx.x < 16 * TPW) {
    const int th = threadIdx.x >> 4, col = threadIdx.x & 15;
    float s = 0.f;
    for (int q = 0; q < k; ++q) s += part[th * k + q][col];
    a.out[(int64_t)t * H + 16 * ((blockIdx.x % ngrp) * TPW + th) + col] = (uint16_t)f32_to_bf16_bits(s);
  }
}

template <int VPL, int MR>
hipError_t launch_fc1_decode(const DecodeArgs& d, unsigned grid, uint32_t xlds, hipStream_t stream, hipEvent_t e0,
                             hipEvent_t e1) {
  // H = 7168 (56 chunks, 14 per wave): straight-line chunk code
  if (d.fc.H == 56 * kChunkK && (d.fc.H / 8 + 64 * kDecKSplit - 1) / (64 * kDecKSplit) <= kXPerThread)
    launch_kernel(fc1_decode_kernel<VPL, 56 / kDecKSplit, MR>, grid, 64 * kDecKSplit, xlds, stream, e0, e1, d);
  else
    launch_kernel(fc1_decode_kernel<VPL, 0, MR>, grid, 64 * kDecKSplit, xlds, stream, e0, e1, d);
  return hipGetLastError();
}

template <int VPL>
hipError_t launch_decode_vpl(const DecodeArgs& d, hipStream_t stream, hipEvent_t e0, hipEvent_t e1) {
  const int M = d.fc.M, E = d.fc.E, k = d.fc.k;
  const int nblk = M * k < E ? M * k : E;
  const unsigned grid1 = (unsigned)(nblk * (d.fc.I / 16));
  const uint32_t xlds = (uint32_t)decode_fc1_lds_bytes(M, d.fc.H);  // staged x rows + corrections
  hipError_t err = hipSuccess;
  // one token, or exactly four (the layer call sends two and three tokens
  // to the routed FC1)
  switch (M) {
    case 1: err = launch_fc1_decode<VPL, 1>(d, grid1, xlds, stream, e0, e1); break;
    case kDecodeMaxTokens: err = launch_fc1_decode<VPL, kDecodeMaxTokens>(d, grid1, xlds, stream, e0, e1); break;
    default: return hipErrorInvalidValue;
  }
  if (err != hipSuccess) return err;
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  DecodeArgs d2 = d;
  d2.fc.act_in = d.fc.act_out;
  d2.fc.wpacked = d.w2;
  return launch_fc2_tokens(d2, stream);
}

}  // namespace

// FC2 + combine, output-stationary: act rows d.fc.act_in [M*k, I] (row f =
// token t, slot j), expert ids and weights from d.topk_ids / d.topk_weights,
// W2 in d.fc.wpacked, bf16 output d.fc.out [M, H].
hipError_t launch_fc2_tokens(const DecodeArgs& d2, hipStream_t stream) {
  const int M = d2.fc.M, k = d2.fc.k;
  const bool i2048 = d2.fc.I == 2048;  // the 384-expert layer: 4 row vectors per lane
  const size_t lds = (size_t)decode_fc2_lds_bytes(d2.fc.I, k);  // the k activation rows + corrections
  if (k <= 8) {  // a whole pair per workgroup: 2k <= 16 waves (measured 12 % faster than one tile)
    const unsigned grid2 = (unsigned)(M * (d2.fc.H / 32));
    if (i2048) fc2_decode_kernel<4, 16, 2><<<grid2, 128 * k, lds, stream>>>(d2);
    else fc2_decode_kernel<0, 16, 2><<<grid2, 128 * k, lds, stream>>>(d2);
  } else {  // top_k > 8: one 16-column tile per workgroup, k <= 16 waves
    const unsigned grid2 = (unsigned)(M * (d2.fc.H / 16));
    fc2_decode_kernel<0, kMaxTopK, 1><<<grid2, 64 * k, lds, stream>>>(d2);
  }
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& d, hipStream_t stream, hipEvent_t e0, hipEvent_t e1) {
  const int E = d.fc.E;
  if (E <= 64) return launch_decode_vpl<1>(d, stream, e0, e1);
  if (E <= 128) return launch_decode_vpl<2>(d, stream, e0, e1);
  if (E <= 256) return launch_decode_vpl<4>(d, stream, e0, e1);
  if (E <= 384) return launch_decode_vpl<6>(d, stream, e0, e1);
  if (E <= 512) return launch_decode_vpl<8>(d, stream, e0, e1);
  return launch_decode_vpl<16>(d, stream, e0, e1);
}

}  // namespace MOE_FMT_NS
}  // namespace moe

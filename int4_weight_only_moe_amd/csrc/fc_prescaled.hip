// Grouped GEMM (FC1 and FC2) with the group scales applied before the
// product, on tiles of up to 128 rows: the large-batch regime.
//
// "The Throughput Lever: Quantifying the MoE GEMM and Mapping the Road to
// B300", section "The Result: Two Regimes": once every expert holds tens to
// hundreds of rows, the grouped GEMM is matrix work rather than a stream of
// weights. On gfx950 a kernel that applies each group's scale to the fp32
// MFMA result (one FMA per output and group, plus a correction MFMA per
// group), as the block kernels of fc.hip do, then runs out of vector issue
// slots. Here the weights enter the matrix core already scaled, so every
// MFMA accumulates straight into its output and the vector work per weight
// is shared by all rows of the tile:
//   * INT4: B = fp16(q * s'), one rounding of the exact product, where
//     s' = s * 2^-sigma and sigma is the per-weight-row exponent shift the
//     repack stores after the tiles (it keeps q * s' a normal fp16 below 2^15
//     for any finite scale; 2^sigma is applied exactly in the epilogue). The
//     A rows are fp16 copies of the bf16 activations, each row scaled by a
//     power of two so that its largest value lies in [2^14, 2^15) (exact:
//     fp16 holds every bf16 significand); the row's exponent is applied in
//     the epilogue. v_mfma_f32_16x16x32_f16 accumulates in fp32.
//   * MXFP4: the exact bf16 values code * 2^(s - 127) with the bf16 MFMA, A
//     the bf16 activations themselves.
// Work decomposition:
//   * a plan kernel cuts each expert's row range (block_m-padded, from
//     moe_route_align) into tiles of equal size counted from the expert's
//     first row, so an expert of up to 128 rows is one tile (its weights
//     are read once) and one holding hundreds of rows gets several; a tile
//     counts only the 16-row sub-tiles that hold a row (padding is not
//     multiplied), and carries a reuse flag when its expert has other tiles
//     (then the weights are read with the default cache policy, else
//     non-temporally);
//   * tiles of up to 128 rows of one expert: one tile pair per wave, 8
//     waves per workgroup, two workgroups per CU (four waves per SIMD,
//     <= 128 VGPRs, 74 KB of LDS each): while one workgroup waits at a
//     barrier or runs its epilogue, the other keeps the matrix core busy
//     (INT4's widened fp16 codes take registers: its bodies for 7 or 8
//     sub-tiles keep two A fragments in flight instead of three);
//   * the tile's activation chunk (up to 128 rows x 128 channels) is copied
//     from memory straight into LDS by gfx950's buffer loads to LDS (no
//     staging registers or stores), double-buffered; a row's sixteen 16-byte
//     vectors are stored XOR-swizzled with the row index, so the A reads of a
//     wave (16 rows, one vector each) hit 16 different bank groups;
//   * per 32-channel group a wave widens both tiles' codes once and runs
//     2 x S MFMAs (S = the tile's sub-tiles of 16 rows, at most 8: padding
//     sub-tiles are not multiplied);
//   * a workgroup's start costs one memory round trip: the first weight
//     chunks go out before the tile's row ids (they do not depend on them),
//     the row ids in one batch, and what the epilogue needs of each row
//     lands in LDS while the first chunks are in flight;
//   * per chunk step: the next chunk's rows go to LDS, the current chunk is
//     computed, the weight chunk after next is loaded, then one wait (the
//     rows and the next weight chunk; the newest weight loads stay in flight)
//     and one barrier. The waits are explicit: a workgroup fence would drain
//     every load in flight.
// Epilogues as in the other grouped kernels: FC1 stores bf16 SiLU(gate)*up,
// FC2 adds w_f * y_f into the fp32 accumulator with atomics.
#include "internal.h"
#include "device_common.h"
#include "fc_common.h"

namespace moe {
namespace MOE_FMT_NS {
namespace {

#ifndef MOE_PRESCALED_WAVES
#define MOE_PRESCALED_WAVES 8
#endif
constexpr int kBW = MOE_PRESCALED_WAVES;     // waves (= tile pairs) per workgroup
constexpr int kBVecs = kChunkK / 8;          // 16-byte vectors of a row's chunk slice
constexpr int kBMaxRows = prescaled_max_rows(kFmt);   // 128
constexpr int kCopyRows = 4 * kBW;                      // A rows one copy round of the workgroup covers
constexpr int kBSlotRows = (kBMaxRows + kCopyRows - 1) / kCopyRows * kCopyRows;  // whole rounds
constexpr int kBSlotVecs = kBSlotRows * kBVecs;         // one LDS slot: up to 128 rows x 16 vectors
constexpr int kBXcds = 8;
constexpr int kPlanMaxExperts = 1024;
constexpr int kBWLoads = 4;                  // vector loads per weight chunk (2 tiles' codes + scales)
#ifndef MOE_PRESCALED_APRE
#define MOE_PRESCALED_APRE 3
#endif
constexpr int kAPre = MOE_PRESCALED_APRE;    // A fragments in flight per group (INT4)
// Pipeline depth: chunks whose weights (registers) and rows (LDS slots) are
// in flight or resident at once; waves per SIMD (4: two workgroups per CU).
#ifndef MOE_PRESCALED_DEPTH
#define MOE_PRESCALED_DEPTH 2
#endif
#ifndef MOE_PRESCALED_WPE
#define MOE_PRESCALED_WPE 4
#endif
#ifndef MOE_PRESCALED_ASLOTS
#define MOE_PRESCALED_ASLOTS MOE_PRESCALED_DEPTH
#endif
constexpr int kDepth = MOE_PRESCALED_DEPTH;   // weight chunks held in registers
constexpr int kASlots = MOE_PRESCALED_ASLOTS; // activation chunks held in LDS
constexpr int kUnroll = kDepth == kASlots ? kDepth : kDepth * kASlots;  // lcm for depths 2..4 with |difference| 1
constexpr int kWpe = MOE_PRESCALED_WPE;
struct XSlots {
  uint4* x[kASlots];
};

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

// s_waitcnt immediate (gfx9 encoding): vmcnt <= v, lgkmcnt <= l, expcnt not waited for.
constexpr int waitcnt_imm(int v, int l) { return (v & 15) | ((v >> 4) << 14) | (7 << 4) | (l << 8); }

__device__ __forceinline__ f16x2_t as_f16x2(uint32_t u) { return __builtin_bit_cast(f16x2_t, u); }

// Eight INT4 codes (one dword of the tile layout: code 2p in bits [4p, 4p+4),
// code 2p+1 in bits [16+4p, 20+4p)) -> eight fp16 values fp16(q * s2), q = u - 8.
// A code at bits 0..3 of a half, OR-ed into fp16 1024.0 (ulp 1), gives
// 1032 + q; at bits 4..7, OR-ed into fp16 64.0 (ulp 1/16), 72 + q. Both
// differences are exact, so the only rounding is that of the product.
__device__ __forceinline__ f16x8_t dequant_int4_f16(uint32_t w, f16x2_t s2) {
  uint32_t m0 = 0x000F000Fu, m1 = 0x00F000F0u, c0 = 0x64006400u, c1 = 0x54005400u;
  asm("" : "+s"(m0));
  asm("" : "+s"(m1));
  asm("" : "+v"(c0));
  asm("" : "+v"(c1));
  uint32_t o0 = 0xE408E408u, o1 = 0xD480D480u;  // fp16 pairs (-1032, -1032), (-72, -72)
  asm("" : "+s"(o0));
  asm("" : "+s"(o1));
  const uint32_t t = w >> 8;
  const f16x2_t p0 = (as_f16x2((w & m0) | c0) + as_f16x2(o0)) * s2;
  const f16x2_t p1 = (as_f16x2((w & m1) | c1) + as_f16x2(o1)) * s2;
  const f16x2_t p2 = (as_f16x2((t & m0) | c0) + as_f16x2(o0)) * s2;
  const f16x2_t p3 = (as_f16x2((t & m1) | c1) + as_f16x2(o1)) * s2;
  return __builtin_shufflevector(__builtin_shufflevector(p0, p1, 0, 1, 2, 3),
                                 __builtin_shufflevector(p2, p3, 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
}

// ---------------------------------------------------------------------------
// Plan: one workgroup turns the block list into the tile list. Each
// expert's run of r blocks becomes n = ceil(r / bpt) tiles of as equal a
// size as whole blocks allow (bpt = tile_rows / block_m; tile_rows is 128
// rows by default), counted from the run's own first block: an expert of up to tile_rows
// rows is one tile and its weights are read once, and the tiles of a longer
// run are alike, so the XCDs they are dealt to get alike work. (Tiles cut at
// multiples of tile_rows of the whole list split most experts in two, each
// part reading the expert's weights; full tiles followed by one remainder
// alternated large and small tiles over the XCDs.)
__global__ __launch_bounds__(1024) void tile_plan_kernel(const int32_t* __restrict__ block_expert,
                                                        const int32_t* __restrict__ sorted_ids,
                                                        const int32_t* __restrict__ npp_p, int E, int block_m, int MK,
                                                        int tile_rows, int max_tiles, int2* __restrict__ tiles,
                                                        int32_t* __restrict__ ntiles_out) {
  __shared__ int run_blocks[kPlanMaxExperts];  // blocks per expert (each expert's blocks are one run)
  __shared__ int wave_cnt[16];
  __shared__ int wave_run[16];
  __shared__ int base, carry;  // tiles so far; the last run start of the blocks so far
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bpt = tile_rows / block_m;  // blocks per full tile
  const int nblk = *npp_p / block_m;
  for (int e = tid; e < E; e += 1024) run_blocks[e] = 0;
  if (tid == 0) {
    base = 0;
    carry = 0;
  }
  __syncthreads();
  for (int b = tid; b < nblk; b += 1024) {
    const int e = block_expert[b];
    if (e >= 0 && e < E) atomicAdd(&run_blocks[e], 1);
  }
  __syncthreads();
  for (int b0 = 0; b0 < nblk; b0 += 1024) {
    const int b = b0 + tid;
    int e = -1;
    bool run_head = false;
    if (b < nblk) {
      e = block_expert[b];
      run_head = b == 0 || block_expert[b - 1] != e;
    }
    // the first block of b's run: an inclusive max-scan of the run heads
    int rs = run_head ? b : -1;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(rs, d, 64);
      if (lane >= d) rs = max(rs, o);
    }
    if (lane == 63) wave_run[wave] = rs;
    __syncthreads();
    int first = carry;
    for (int w = 0; w < wave; ++w) first = max(first, wave_run[w]);
    first = max(first, rs);
    // tile j of the run starts at block floor(j * r / n): b starts a tile if
    // it is that start for j = ceil(pos * n / r)
    const int64_t pos = b - first;
    const int64_t r = (e >= 0 && e < E) ? run_blocks[e] : 0;
    const int64_t n = r > 0 ? (r + bpt - 1) / bpt : 1;
    const int64_t j = r > 0 ? (pos * n + r - 1) / r : 0;
    const bool head = b < nblk && pos < r && j * r / n == pos;
    const unsigned long long m = __ballot(head);
    if (lane == 0) wave_cnt[wave] = __popcll(m);
    __syncthreads();
    int t = base + __popcll(m & ((1ull << lane) - 1ull));
    for (int w = 0; w < wave; ++w) t += wave_cnt[w];
    if (head && t < max_tiles) {
      int nb = (int)((j + 1) * r / n - pos);
      nb = nb < nblk - b ? nb : nblk - b;
      // sub-tiles that hold a row: an expert's padding sits at the end of its
      // range, so they are a prefix of the tile's
      int nsub = nb * block_m / kTileRows;
      while (nsub > 1 && sorted_ids[b * block_m + (nsub - 1) * kTileRows] >= MK) --nsub;
      const bool reuse = n > 1;
      tiles[t] = make_int2(b * block_m, nsub | (reuse ? kTileReuseBit : 0) | (e << kTileExpertShift));
    }
    __syncthreads();
    if (tid == 0) {
      int tot = 0, last = carry;
      for (int w = 0; w < 16; ++w) {
        tot += wave_cnt[w];
        last = max(last, wave_run[w]);
      }
      base += tot;
      carry = last;
    }
    __syncthreads();
  }
  if (tid == 0) *ntiles_out = base < max_tiles ? base : max_tiles;
}

// (2^-sigma0, 2^-sigma1) for two rows' shifts (|sigma| <= 15: normal fp16 values).
__device__ __forceinline__ f16x2_t pow2_pair(int sigma0, int sigma1) {
  return f16x2_t{(_Float16)__builtin_ldexpf(1.0f, -sigma0), (_Float16)__builtin_ldexpf(1.0f, -sigma1)};
}

// The row id an A row of the tile reads: its token (FC1) or assignment (FC2).
template <bool kFc1>
__device__ __forceinline__ uint32_t a_row(int f, int k) { return (uint32_t)(kFc1 ? f / k : f); }

// What the epilogues need of each row of the tile, gathered into LDS while
// the workgroup's first chunks are in flight (rather than loaded after the
// main loop): the output offset (FC1: f * I into act; FC2: token * H into
// the accumulator; -1 for a padding row), FC2's routing weight and, for INT4,
// the A row's exponent.
struct TileRows {
  int32_t dst[kBSlotRows];
  float w[kBSlotRows];
  int32_t ex[kBSlotRows];
};
// INT4: the shifts of each wave's weight rows, per tile of its pair.
typedef int8_t PairSigmas[kBW][2][kTileRows];

// Epilogues of a tile pair. INT4 scales each output by 2^(row exponent +
// sigma of its weight row).
//
// FC1 multiplies with the operands swapped (the weights as the first MFMA
// operand), so the accumulators hold D transposed: lane L has A row L % 16
// and output columns 4 (L / 16) .. +3, and writes its 4 SiLU(gate) * up
// values as one 8-byte store.
template <int S>
__device__ __forceinline__ void prescaled_epilogue_fc1(const FcArgs& a, const int pair, const int nsub,
                                                       const f32x4_t (&acc0)[S], const f32x4_t (&acc1)[S],
                                                       const int lane, const TileRows& tr,
                                                       const int8_t (&sg)[2][kTileRows]) {
  const int c0 = 4 * (lane >> 4);
  int sg0[4] = {0, 0, 0, 0}, sg1[4] = {0, 0, 0, 0};
  if constexpr (kFmt == kFmtInt4) {
    const uint32_t d0 = *reinterpret_cast<const uint32_t*>(&sg[0][c0]);
    const uint32_t d1 = *reinterpret_cast<const uint32_t*>(&sg[1][c0]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sg0[i] = (int)(int8_t)(d0 >> (8 * i));
      sg1[i] = (int)(int8_t)(d1 >> (8 * i));
    }
  }
#pragma unroll
  for (int s = 0; s < S; ++s) {
    if (s >= nsub) continue;
    const int r = kTileRows * s + (lane & 15);
    const int dst = tr.dst[r];
    if (dst < 0) continue;
    const int ex = kFmt == kFmtInt4 ? tr.ex[r] : 0;
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float g = acc0[s][i], u = acc1[s][i];
      if constexpr (kFmt == kFmtInt4) {
        g = __builtin_ldexpf(g, ex + sg0[i]);
        u = __builtin_ldexpf(u, ex + sg1[i]);
      }
      // SiLU(g) * u; the reciprocal's rounding is far below the bf16 store's
      o[i] = f32_to_bf16_bits(g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u);
    }
    *reinterpret_cast<uint2*>(a.act_out + (uint32_t)(dst + 16 * pair + c0)) =
        make_uint2(o[0] | (o[1] << 16), o[2] | (o[3] << 16));
  }
}

// FC2: lane L has rows 4 (L / 16) + i and output column L % 16 of each tile.
template <int S>
__device__ __forceinline__ void prescaled_epilogue_fc2(const FcArgs& a, const int pair, const int nsub,
                                                       const f32x4_t (&acc0)[S], const f32x4_t (&acc1)[S],
                                                       const int lane, const TileRows& tr,
                                                       const int8_t (&sg)[2][kTileRows]) {
  const int col = lane & 15;
  int sig0 = 0, sig1 = 0;
  if constexpr (kFmt == kFmtInt4) {
    sig0 = sg[0][col];
    sig1 = sg[1][col];
  }
#pragma unroll
  for (int s = 0; s < S; ++s) {
    if (s >= nsub) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = kTileRows * s + 4 * (lane >> 4) + i;
      const int o = tr.dst[r];
      if (o < 0) continue;
      const float wt = tr.w[r];
      float v0 = acc0[s][i], v1 = acc1[s][i];
      if constexpr (kFmt == kFmtInt4) {
        const int x = tr.ex[r];
        v0 = __builtin_ldexpf(v0, x + sig0);
        v1 = __builtin_ldexpf(v1, x + sig1);
      }
      float* dst = a.acc + (uint32_t)(o + kPairRows * pair);  // < M * H < 2^31
      unsafeAtomicAdd(dst + col, wt * v0);
      unsafeAtomicAdd(dst + 16 + col, wt * v1);
    }
  }
}

// One workgroup's tile (rows row0 .. row0 + 16 * nsub of the sorted list,
// expert e) times this wave's tile pair; S >= nsub sub-tiles, weights under
// cache policy kPolicy.
template <int S, bool kFc1, int kPolicy>
__device__ __forceinline__ void prescaled_body(const FcArgs& a, const int e, const int pair, const int row0,
                                              const int nsub, const XSlots xs, uint32_t* xoffs, TileRows& tr,
                                              PairSigmas& psig) {
  constexpr int kD = (S * kTileRows + kCopyRows - 1) / kCopyRows;  // 1 KB copies per wave per chunk
  static_assert(S >= 1 && kD * kCopyRows <= kBSlotRows, "the copies fit the slot");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K = kFc1 ? a.H : a.I;
  const int N = kFc1 ? 2 * a.I : a.H;
  const int MK = a.M * a.k;
  const int n = K / kChunkK;
  const int32_t* rows = a.sorted_ids + row0;

  // Weight stream of the pair (a chunk past the K range reads zeros).
  const uint8_t* wbase = a.wpacked + (int64_t)e * packed_bytes_per_expert(N, K) + (int64_t)pair * n * kPairChunkBytes;
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(wbase, (uint32_t)n * kPairChunkBytes);
  const uint32_t oq0 = 16u * lane, oq1 = kTileBytes + 16u * lane;
  const uint32_t os0 = kTileNibbleBytes + kScaleRowBytes * (lane & 15);
  const uint32_t os1 = kTileBytes + kTileNibbleBytes + kScaleRowBytes * (lane & 15);
  auto load_w = [&](int c) {
    const uint32_t base = (uint32_t)c * kPairChunkBytes;
    WChunk w;
    w.q0 = bload16<kPolicy>(wr, base + oq0);
    w.q1 = bload16<kPolicy>(wr, base + oq1);
    w.s0 = load_scales<kPolicy>(wr, base + os0);
    w.s1 = load_scales<kPolicy>(wr, base + os1);
    return w;
  };
  WChunk wb[kDepth];
  // The first kDepth weight chunks do not depend on the tile's rows: they go
  // out before the row ids are read.
#pragma unroll
  for (int d = 0; d < kDepth; ++d) wb[d] = load_w(d);

  // The row ids: those of the A rows this lane copies and, for thread
  // t < 16 S, row t's for the epilogues. Indices are clamped into the tile so
  // that the loads are unconditional and go out together.
  const int last = kTileRows * nsub - 1;
  int fr[kD];
#pragma unroll
  for (int i = 0; i < kD; ++i) {
    const int r = 4 * (wave + kBW * i) + (lane >> 4);
    fr[i] = rows[r < last ? r : last];
  }
  const int rf0 = rows[tid < last ? tid : last];
  // INT4: the shifts of this wave's weight rows, lane l < 32: tile l / 16,
  // row l % 16 (FC1: gate column 16 pair + r, up column I + 16 pair + r;
  // FC2: row 32 pair + 16 t + r).
  int8_t sgv = 0;
  if constexpr (kFmt == kFmtInt4) {
    const int t = (lane / kTileRows) & 1, r = lane & (kTileRows - 1);
    const int nrow = kFc1 ? (t ? a.I : 0) + kTileRows * pair + r : kPairRows * pair + kTileRows * t + r;
    sgv = a.wsigma[(int64_t)e * N + nrow];
  }

  // A rows: copy i of this wave covers LDS rows 4 * (wave + 8i) .. +3 of a
  // slot; lane L writes row 4 * (wave + 8i) + L / 16, LDS vector L % 16,
  // which holds channel vector (L % 16) ^ (row % 16). Rows past the tile's
  // sub-tiles and padding entries read the tile's first row (their D rows are
  // not stored).
  const int rows_total = kFc1 ? a.M : MK;
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.act_in, (uint32_t)rows_total * (uint32_t)K * 2u);
  const uint32_t rid0 = a_row<kFc1>(rows[0], a.k);
  // The per-lane source offsets are kept in LDS (this thread's kD words,
  // copy-major so that a wave's accesses are consecutive words), not in
  // registers: they are needed only while the copies are issued.
  uint32_t* myoff = xoffs + tid;
#pragma unroll
  for (int i = 0; i < kD; ++i) {
    const int r = 4 * (wave + kBW * i) + (lane >> 4);
    const int f = r <= last ? fr[i] : MK;
    const uint32_t rid = (f >= 0 && f < MK) ? a_row<kFc1>(f, a.k) : rid0;
    const uint32_t v = (uint32_t)((lane & 15) ^ (r & 15));
    myoff[i * 64 * kBW] = (rid * (uint32_t)K + 8u * v) * 2u;
  }
  // The epilogue's row data (two more loads for thread t < 16 S), stored to
  // LDS before the prologue's barrier.
  const int rf = tid <= last ? rf0 : MK;
  int rdst = -1, rex = 0;
  float rw = 0.f;
  if (tid < kTileRows * S && rf >= 0 && rf < MK) {
    rdst = kFc1 ? rf * a.I : (rf / a.k) * a.H;  // < M * k * I, M * H < 2^31
    if constexpr (!kFc1) rw = a.topk_weights[rf];
    if constexpr (kFmt == kFmtInt4) rex = a.row_exp[kFc1 ? rf / a.k : rf];
  }
  typedef __attribute__((address_space(3))) void* lds_ptr_t;
  auto copy_rows = [&](int c, int slot) {
    uint32_t xoff[kD];
#pragma unroll
    for (int i = 0; i < kD; ++i) xoff[i] = myoff[i * 64 * kBW];
#pragma unroll
    for (int i = 0; i < kD; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr_t)(xs.x[slot] + (wave + kBW * i) * 64), 16,
                                               xoff[i], (uint32_t)c * (kChunkK * 2), 0, 0);
  };
  // LDS vector of this lane's A operand for group g of sub-tile 0 (slot 0):
  // row m = lane % 16, channel vector 4g + lane / 16, stored at vector
  // (4g + lane / 16) ^ m = 4 * (g ^ (m / 4)) + ((lane / 16) ^ (m % 4)).
  const uint32_t abase = (uint32_t)((lane & 15) * kBVecs + (((lane >> 4) ^ lane) & 3));
  const uint32_t am2 = (uint32_t)((lane & 15) >> 2);
  auto aoff = [&](int g) { return abase + 4u * ((uint32_t)g ^ am2); };

  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
  f32x4_t acc0[S], acc1[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    acc0[s] = zero4;
    acc1[s] = zero4;
  }

  // Chunk step c issues the rows of chunk c + kASlots - 1 into LDS, computes
  // chunk c, then loads the weights of chunk c + kDepth, and waits until the
  // rows and weights of chunk c + 1 have arrived: the newer loads may stay in
  // flight (kVmAfter of them: those issued after the later of the two). The
  // prologue has issued the weights of chunks 0 .. kDepth - 1, then issues
  // the rows of chunks 0 .. kASlots - 2 and waits for those of chunk 0.
  constexpr int kAfterW = (kDepth - 1) * (kD + kBWLoads);
  constexpr int kAfterRows = kBWLoads + (kASlots - 2) * (kD + kBWLoads);
  constexpr int kVmAfter = kAfterW < kAfterRows ? kAfterW : kAfterRows;
  static_assert(kVmAfter < 64, "vmcnt holds at most 63");
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int c = 0; c + 1 < kASlots; ++c) copy_rows(c, c);
  __builtin_amdgcn_sched_barrier(0);
  if (tid < kTileRows * S) {
    tr.dst[tid] = rdst;
    tr.w[tid] = rw;
    tr.ex[tid] = rex;
  }
  if constexpr (kFmt == kFmtInt4)
    if (lane < 2 * kTileRows) (&psig[wave][0][0])[lane] = sgv;
  __builtin_amdgcn_s_waitcnt(waitcnt_imm((kASlots - 2) * kD, 0));
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);

  // 2^-sigma of this lane's two weight rows (column lane % 16 of each tile).
  f16x2_t m2 = {(_Float16)1.0f, (_Float16)1.0f};
  if constexpr (kFmt == kFmtInt4) m2 = pow2_pair(psig[wave][0][lane & 15], psig[wave][1][lane & 15]);

  auto compute = [&](const WChunk& w, int slot) {
    const uint32_t q0[4] = {w.q0.x, w.q0.y, w.q0.z, w.q0.w};
    const uint32_t q1[4] = {w.q1.x, w.q1.y, w.q1.z, w.q1.w};
    f16x2_t s0lo, s0hi, s1lo, s1hi;
    if constexpr (kFmt == kFmtInt4) {  // s' = s * 2^-sigma for the four groups
      const f16x2_t m20 = __builtin_shufflevector(m2, m2, 0, 0), m21 = __builtin_shufflevector(m2, m2, 1, 1);
      s0lo = as_f16x2(w.s0.x) * m20;
      s0hi = as_f16x2(w.s0.y) * m20;
      s1lo = as_f16x2(w.s1.x) * m21;
      s1hi = as_f16x2(w.s1.y) * m21;
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      if constexpr (kFmt == kFmtInt4) {
        const f16x2_t t0 = g < 2 ? s0lo : s0hi, t1 = g < 2 ? s1lo : s1hi;
        const f16x2_t g0 = (g & 1) ? __builtin_shufflevector(t0, t0, 1, 1) : __builtin_shufflevector(t0, t0, 0, 0);
        const f16x2_t g1 = (g & 1) ? __builtin_shufflevector(t1, t1, 1, 1) : __builtin_shufflevector(t1, t1, 0, 0);
        // A fragments in a ring of kAP registers: the first kAP - 1
        // sub-tiles' rows are read before the widening, and sub-tile
        // s + kAP - 1's while sub-tile s's MFMAs are issued (two for seven
        // or eight sub-tiles: their accumulators take the registers)
        constexpr int kAP = S > 6 ? 2 : kAPre;
        const uint4* ap = xs.x[slot] + aoff(g);
        f16x8_t ar[kAP];
#pragma unroll
        for (int p = 0; p + 1 < kAP; ++p)
          if (p < S) ar[p] = __builtin_bit_cast(f16x8_t, ap[p * kTileRows * kBVecs]);
        __builtin_amdgcn_sched_barrier(0);
        const f16x8_t b0 = dequant_int4_f16(q0[g], g0);
        const f16x8_t b1 = dequant_int4_f16(q1[g], g1);
#pragma unroll
        for (int s = 0; s < S; ++s) {
          if (s + kAP - 1 < S)
            ar[(s + kAP - 1) % kAP] = __builtin_bit_cast(f16x8_t, ap[(s + kAP - 1) * kTileRows * kBVecs]);
          const f16x8_t xv = ar[s % kAP];
          if constexpr (kFc1) {  // D transposed (see the FC1 epilogue)
            acc0[s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(b0, xv, acc0[s], 0, 0, 0);
            acc1[s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(b1, xv, acc1[s], 0, 0, 0);
          } else {
            acc0[s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xv, b0, acc0[s], 0, 0, 0);
            acc1[s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xv, b1, acc1[s], 0, 0, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        // the next group's codes and rows are not hoisted above these MFMAs
        // (their registers would not fit next to the accumulators)
        __builtin_amdgcn_sched_barrier(0);
      } else {
        const bf16x8_t b0 = dequant_group(q0[g], group_scale(w.s0, g));
        const bf16x8_t b1 = dequant_group(q1[g], group_scale(w.s1, g));
#pragma unroll
        for (int s = 0; s < S; ++s) {
          const bf16x8_t xv = as_bf16x8(xs.x[slot][s * kTileRows * kBVecs + aoff(g)]);
          if constexpr (kFc1) {
            acc0[s] = mfma16x16x32(b0, xv, acc0[s]);
            acc1[s] = mfma16x16x32(b1, xv, acc1[s]);
          } else {
            acc0[s] = mfma16x16x32(xv, b0, acc0[s]);
            acc1[s] = mfma16x16x32(xv, b1, acc1[s]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // Chunk c uses weight buffer c % kDepth and slot c % kASlots (static in
  // the unrolled body). Steps past the last chunk (n need not be a multiple
  // of the unroll) are skipped.
  for (int c = 0; c < n; c += kUnroll) {
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      const int cc = c + j;
      if (kUnroll > 2 && cc >= n) break;
      // Rows of chunk cc + kASlots - 1 into the slot chunk cc - 1 used (every
      // wave passed the last barrier after its reads of that slot
      // completed). Past the last chunk the copy reads the next rows' data
      // (or nothing) into a slot no one reads.
      copy_rows(cc + kASlots - 1, (j + kASlots - 1) % kASlots);
      __builtin_amdgcn_sched_barrier(0);
      compute(wb[j % kDepth], j % kASlots);
      __builtin_amdgcn_sched_barrier(0);
      wb[j % kDepth] = load_w(cc + kDepth);
      __builtin_amdgcn_sched_barrier(0);
      // the rows and weights of chunk cc + 1 have arrived; newer loads may
      // stay in flight. lgkmcnt(0): this wave's reads of slot j are done
      // before anyone refills it.
      __builtin_amdgcn_s_waitcnt(waitcnt_imm(kVmAfter, 0));
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // no copy into LDS may outlive the workgroup
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));

  if constexpr (kFc1)
    prescaled_epilogue_fc1<S>(a, pair, nsub, acc0, acc1, lane, tr, psig[wave]);
  else
    prescaled_epilogue_fc2<S>(a, pair, nsub, acc0, acc1, lane, tr, psig[wave]);
}

template <int S, bool kFc1>
__device__ __forceinline__ void prescaled_policy(const FcArgs& a, const int e, const int pair, const int row0,
                                                const int nsub, const bool reuse, const XSlots xs,
                                                uint32_t* xoffs, TileRows& tr, PairSigmas& psig) {
  if (reuse)
    prescaled_body<S, kFc1, kPolicyDefault>(a, e, pair, row0, nsub, xs, xoffs, tr, psig);
  else
    prescaled_body<S, kFc1, kPolicyWeights>(a, e, pair, row0, nsub, xs, xoffs, tr, psig);
}

template <bool kFc1>
__global__ __launch_bounds__(64 * kBW) __attribute__((amdgpu_waves_per_eu(kWpe)))
void fc_prescaled_kernel(FcArgs a) {
  // the slots of the tile's activation chunks, as separate objects: the
  // compiler then knows that reads of one need not wait for copies into
  // another (with one array it drains every load before each chunk's reads)
  __shared__ uint4 xt0[kBSlotVecs];
  __shared__ uint4 xt1[kBSlotVecs];
  __shared__ uint4 xt2[kASlots > 2 ? kBSlotVecs : 1];
  __shared__ uint4 xt3[kASlots > 3 ? kBSlotVecs : 1];
  static_assert(kDepth >= 2 && kDepth <= 4 && kASlots >= 2 && kASlots <= 4, "two to four buffers");
  static_assert(kDepth == kASlots || kDepth - kASlots == 1 || kASlots - kDepth == 1, "unroll = lcm");
  XSlots xs;
  xs.x[0] = xt0;
  xs.x[1] = xt1;
  if constexpr (kASlots > 2) xs.x[2] = xt2;
  if constexpr (kASlots > 3) xs.x[3] = xt3;
  __shared__ uint32_t xoffs[64 * kBW * (kBSlotRows / kCopyRows)];  // each thread's copy source offsets
  __shared__ TileRows tr;
  __shared__ PairSigmas psig;
  constexpr int kThreads = 64 * kBW;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int N = kFc1 ? 2 * a.I : a.H;
  const int npg = N / kPairRows / kBW;  // pair groups per tile

  if constexpr (kFc1) {  // clear FC2's accumulator
    uint4* z = reinterpret_cast<uint4*>(a.acc);
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + tid; i < a.zero_words16; i += stride)
      z[i] = make_uint4(0, 0, 0, 0);
  }

  // workgroups dealt to the XCDs: all pair groups of a tile on one XCD,
  // consecutive tiles on different XCDs
  const int xcd = blockIdx.x % kBXcds, gi = blockIdx.x / kBXcds;
  const int tile = (gi / npg) * kBXcds + xcd;
  const int pair = (gi % npg) * kBW + wave;
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
  if (e < 0 || e >= a.E || nsub < 1 || nsub > a.tile_rows / kTileRows) return;

  // exactly the tile's sub-tiles are multiplied
  // (bodies for more sub-tiles than a tile can hold are not instantiated)
#define MOE_PRESCALED_CASE(S)                                                          \
  case S:                                                                              \
    if constexpr (S * kTileRows <= kBMaxRows)                                          \
      prescaled_policy<S, kFc1>(a, e, pair, row0, nsub, reuse, xs, xoffs, tr, psig);   \
    break;
  switch (nsub) {
    MOE_PRESCALED_CASE(1)
    MOE_PRESCALED_CASE(2)
    MOE_PRESCALED_CASE(3)
    MOE_PRESCALED_CASE(4)
    MOE_PRESCALED_CASE(5)
    MOE_PRESCALED_CASE(6)
    MOE_PRESCALED_CASE(7)
    MOE_PRESCALED_CASE(8)
  }
#undef MOE_PRESCALED_CASE
}

}  // namespace

int64_t tile_grid_tiles(int64_t M, int64_t E, int64_t k, int64_t block_m, int64_t cap, int64_t tile_rows) {
  const int64_t bpt = tile_rows / block_m;
  const int64_t nblk = cap / block_m;
  const int64_t mk = M * k;
  const int64_t t = (nblk + bpt - 1) / bpt + (mk < E ? mk : E);
  return (t + kBXcds - 1) / kBXcds * kBXcds;
}

hipError_t launch_tile_plan(const FcArgs& a, hipStream_t stream) {
  if (a.E > kPlanMaxExperts || a.block_m <= 0 || a.tile_rows % a.block_m != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(tile_plan_kernel, dim3(1), dim3(1024), 0, stream, a.block_expert, a.sorted_ids, a.npp, a.E,
                     a.block_m, a.M * a.k, a.tile_rows, a.max_tiles, a.tiles, a.ntiles);
  return hipGetLastError();
}

bool prescaled_supported(int64_t H, int64_t I) {
  // whole pair groups and an even number of K chunks in both GEMMs
  return (2 * I / kPairRows) % kBW == 0 && (H / kPairRows) % kBW == 0 && (H / kChunkK) % 2 == 0 &&
         (I / kChunkK) % 2 == 0;
}

template <bool kFc1>
hipError_t launch_fc_prescaled(const FcArgs& a, hipStream_t stream, hipEvent_t e0, hipEvent_t e1) {
  const int N = kFc1 ? 2 * a.I : a.H;
  const int64_t grid = (int64_t)a.max_tiles * (N / kPairRows / kBW);
  if (grid <= 0 || grid > 0x7FFFFFFF || a.max_tiles % kBXcds != 0) return hipErrorInvalidValue;
  launch_kernel(fc_prescaled_kernel<kFc1>, dim3((unsigned)grid), dim3(64 * kBW), 0, stream, e0, e1, a);
  return hipGetLastError();
}

template hipError_t launch_fc_prescaled<true>(const FcArgs&, hipStream_t, hipEvent_t, hipEvent_t);
template hipError_t launch_fc_prescaled<false>(const FcArgs&, hipStream_t, hipEvent_t, hipEvent_t);

}  // namespace MOE_FMT_NS
}  // namespace moe

#if MOE_WEIGHT_FORMAT == 0
// ---------------------------------------------------------------------------
// Format-independent helpers of the scale-before path, built once (INT4 unit).
namespace moe {
namespace {

constexpr int kRsWaves = 4;

// One wave per row: the largest |value| (bf16 bit patterns of finite values
// order as integers), e = floor(log2(max)) - 14, then every value times 2^-e
// converted to fp16. Every bf16 significand fits fp16's, so a scaled value
// of the normal fp16 range is exact; smaller ones (below 2^-28 of the row's
// largest) are truncated to fp16's subnormal spacing.
__global__ __launch_bounds__(64 * kRsWaves) void rowscale_kernel(const uint16_t* __restrict__ in, int64_t rows,
                                                                 int K, uint16_t* __restrict__ out,
                                                                 int32_t* __restrict__ exps) {
  const int64_t row = (int64_t)blockIdx.x * kRsWaves + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const uint4* src = reinterpret_cast<const uint4*>(in + row * K);
  uint4* dst = reinterpret_cast<uint4*>(out + row * K);
  const int nv = K / 8;
  uint32_t mx = 0;
  for (int i = lane; i < nv; i += 64) {
    const uint4 v = src[i];
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) mx = max(mx, max(d[j] & 0x7FFFu, (d[j] >> 16) & 0x7FFFu));
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off, 64));
  int ex = 0;
  if (mx != 0) {
    const int be = (int)(mx >> 7);
    // floor(log2) of the largest magnitude (a subnormal bf16 has exponent -133
    // plus the position of its leading mantissa bit)
    const int lg = be > 0 ? be - 127 : (31 - __builtin_clz(mx & 0x7Fu)) - 133;
    ex = lg - 14;
  }
  if (lane == 0) exps[row] = ex;
  for (int i = lane; i < nv; i += 64) {
    const uint4 v = src[i];
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float lo = __builtin_ldexpf(__uint_as_float(d[j] << 16), -ex);
      const float hi = __builtin_ldexpf(__uint_as_float(d[j] & 0xFFFF0000u), -ex);
      o[j] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
    }
    dst[i] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// The same with the whole row in registers (rows up to 64 * VPL * 8 values):
// every load of the row is issued at once and the row is read once. (The
// two-pass loop above keeps one 16-byte load per lane in flight, which held
// it to ~4.4 TB/s.)
template <int VPL>
__global__ __launch_bounds__(64 * kRsWaves) void rowscale_regs_kernel(const uint16_t* __restrict__ in, int64_t rows,
                                                                      int K, uint16_t* __restrict__ out,
                                                                      int32_t* __restrict__ exps) {
  const int64_t row = (int64_t)blockIdx.x * kRsWaves + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const uint4* src = reinterpret_cast<const uint4*>(in + row * K);
  uint4* dst = reinterpret_cast<uint4*>(out + row * K);
  const int nv = K / 8;
  uint4 v[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int idx = lane + 64 * i;
    v[i] = src[idx < nv ? idx : nv - 1];  // unconditional: the loads go out together
  }
  uint32_t mx = 0;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const uint32_t d[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) mx = max(mx, max(d[j] & 0x7FFFu, (d[j] >> 16) & 0x7FFFu));
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off, 64));
  int ex = 0;
  if (mx != 0) {
    const int be = (int)(mx >> 7);
    const int lg = be > 0 ? be - 127 : (31 - __builtin_clz(mx & 0x7Fu)) - 133;
    ex = lg - 14;
  }
  if (lane == 0) exps[row] = ex;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const uint32_t d[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float lo = __builtin_ldexpf(__uint_as_float(d[j] << 16), -ex);
      const float hi = __builtin_ldexpf(__uint_as_float(d[j] & 0xFFFF0000u), -ex);
      o[j] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
    }
    if (lane + 64 * i < nv) dst[lane + 64 * i] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// One thread per weight row: sigma = clamp(floor(log2(max_g |s|)) - 11, -15, 4).
__global__ __launch_bounds__(256) void row_sigma_kernel(const uint16_t* __restrict__ s, int64_t nrows, int G,
                                                        int8_t* __restrict__ sigma) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= nrows) return;
  const uint16_t* p = s + r * G;
  uint32_t mx = 0;
  for (int g = 0; g < G; ++g) mx = max(mx, (uint32_t)(p[g] & 0x7FFFu));
  int sg = 0;
  if (mx != 0) {
    const int be = (int)(mx >> 10);
    const int lg = be > 0 ? be - 15 : (31 - __builtin_clz(mx)) - 24;  // fp16 subnormal: m * 2^-24
    sg = min(max(lg - 11, -15), 4);
  }
  sigma[r] = (int8_t)sg;
}

}  // namespace

hipError_t launch_rowscale(const uint16_t* in, int64_t rows, int64_t K, uint16_t* out, int32_t* exps,
                           hipStream_t stream) {
  const int64_t blocks = (rows + kRsWaves - 1) / kRsWaves;
  if (blocks <= 0 || blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  const int64_t vpl = (K / 8 + 63) / 64;  // 16-byte vectors per lane
  if (vpl <= 2) rowscale_regs_kernel<2><<<(unsigned)blocks, 64 * kRsWaves, 0, stream>>>(in, rows, (int)K, out, exps);
  else if (vpl <= 4) rowscale_regs_kernel<4><<<(unsigned)blocks, 64 * kRsWaves, 0, stream>>>(in, rows, (int)K, out, exps);
  else if (vpl <= 8) rowscale_regs_kernel<8><<<(unsigned)blocks, 64 * kRsWaves, 0, stream>>>(in, rows, (int)K, out, exps);
  else if (vpl <= 14) rowscale_regs_kernel<14><<<(unsigned)blocks, 64 * kRsWaves, 0, stream>>>(in, rows, (int)K, out, exps);
  else if (vpl <= 16) rowscale_regs_kernel<16><<<(unsigned)blocks, 64 * kRsWaves, 0, stream>>>(in, rows, (int)K, out, exps);
  else rowscale_kernel<<<(unsigned)blocks, 64 * kRsWaves, 0, stream>>>(in, rows, (int)K, out, exps);
  return hipGetLastError();
}

hipError_t launch_row_sigma(const uint16_t* scales_f16, int E, int N, int K, int8_t* sigma, hipStream_t stream) {
  const int64_t rows = (int64_t)E * N;
  const int64_t blocks = (rows + 255) / 256;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  row_sigma_kernel<<<(unsigned)blocks, 256, 0, stream>>>(scales_f16, rows, K / kGroup, sigma);
  return hipGetLastError();
}

}  // namespace moe
#endif

// Internal declarations shared by the host-side entry points (abi.hip) and
// the kernel translation units. Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

namespace moe {

// Weight formats. kFmtInt4: INT4 codes (offset binary, q = u - 8), one fp16
// scale per 32 channels. kFmtMxfp4: FP4 e2m1 codes, one E8M0 scale
// (2^(s - 127)) per 32 channels. The grouped-GEMM sources (fc.hip,
// fc_prescaled.hip, decode.hip) are compiled once per format: MOE_WEIGHT_FORMAT
// selects it (the *_mxfp4.hip wrappers set 1), and their format-dependent
// code lives in the namespace MOE_FMT_NS.
constexpr int kFmtInt4 = 0;
constexpr int kFmtMxfp4 = 1;
#ifndef MOE_WEIGHT_FORMAT
#define MOE_WEIGHT_FORMAT 0
#endif
#if MOE_WEIGHT_FORMAT == 1
#define MOE_FMT_NS fmt_mxfp4
#else
#define MOE_FMT_NS fmt_int4
#endif
constexpr int kFmt = MOE_WEIGHT_FORMAT;  // the format this translation unit's kernels read

// Device layout of the repacked weights.
//   A "tile" is 16 rows x 128 input channels: 1024 bytes of codes followed
//   by the scales of 16 rows x 4 groups of 32 (fp16: 128 bytes, E8M0: 64).
//   A "pair" is two tiles read together by one wave: for W13 the gate rows
//   [16r, 16r+16) and the up rows I + [16r, 16r+16); for W2 the rows
//   [32r, 32r+16) and [32r+16, 32r+32).
//   Per expert: pairs in row order, each pair's K-chunks in K order, each
//   K-chunk holds the two tiles back to back.
constexpr int kGroup = 32;
constexpr int kTileRows = 16;
constexpr int kChunkK = 128;                 // input channels per tile
constexpr int kTileNibbleBytes = 1024;       // 16 x 128 / 2
__host__ __device__ constexpr int tile_scale_bytes(int fmt) { return fmt == kFmtMxfp4 ? 64 : 128; }
constexpr int kPairRows = 32;
// format-dependent sizes, of this translation unit's format (internal linkage)
constexpr int kTileScaleBytes = tile_scale_bytes(kFmt);
constexpr int kTileBytes = kTileNibbleBytes + kTileScaleBytes;
constexpr int kPairChunkBytes = 2 * kTileBytes;

__host__ __device__ constexpr int64_t packed_bytes_fmt(int fmt, int64_t N, int64_t K) {
  return (N / kPairRows) * (K / kChunkK) * 2 * (kTileNibbleBytes + tile_scale_bytes(fmt));
}
// INT4 blobs end with one int8 per weight row (E x N, canonical row order):
// sigma = clamp(floor(log2(max_g |s[n, g]|)) - 11, -15, 4), 0 for a row of
// zero scales. q * s * 2^-sigma is then a normal fp16 below 2^15 for every
// finite scale (the rounded-weight kernels use it; the others ignore it).
inline int64_t sigma_trailer_bytes(int fmt, int64_t E, int64_t N) { return fmt == kFmtInt4 ? E * N : 0; }
static __host__ __device__ inline int64_t packed_bytes_per_expert(int64_t N, int64_t K) {
  return packed_bytes_fmt(kFmt, N, K);
}

// Tiles of the tiled grouped GEMM (fc_prescaled.hip): up to 128 rows of one
// expert, in 16-row sub-tiles. Table entry: (first row in the sorted list,
// meta = sub-tiles | reuse flag | expert << 8). A sub-tile has kTileRows rows.
// Largest tile of the pre-scaled tiled kernel (fc_prescaled.hip): 128 rows
// for both formats (measured on the 384-expert layer against 96-row INT4
// tiles: M = 4096 -3.4 %, skewed routing -1.3 %, M <= 2048 and 8192 within
// +-0.5 %).
#ifndef MOE_PRESCALED_INT4_ROWS
#define MOE_PRESCALED_INT4_ROWS 128
#endif
__host__ __device__ constexpr int prescaled_max_rows(int fmt) {
  return fmt == kFmtMxfp4 ? 128 : MOE_PRESCALED_INT4_ROWS;
}
// Tile rows of the pre-scaled kernel for a block size: whole blocks per tile.
inline int prescaled_tile_rows(int fmt, int block_m) {
  const int r = prescaled_max_rows(fmt);
  return r % block_m == 0 ? r : block_m;
}
constexpr int kTileNsubMask = 15;
constexpr int kTileReuseBit = 16;
constexpr int kTileExpertShift = 8;
// Upper bound of the tile count for any block_m and tile size of at least 64
// rows (a tile starts at every expert change and every tile_rows rows of an
// expert's run of blocks).
inline int64_t tile_table_entries(int64_t M, int64_t k) { return 2 * M * k + 16; }

// The pre-scaled tiled kernel takes over from the block kernels once experts
// average this many assignments (and the shape divides into its pair
// groups). Measured on the 384-expert layer: at 16 (M = 768) it beats the
// wide block kernel by 2 %, at 21 (M = 1024) by 7 % with uniform routing
// and by 27 % with the skewed batch.
#ifndef MOE_PRESCALED_MIN_PER_EXPERT
#define MOE_PRESCALED_MIN_PER_EXPERT 16.0
#endif
inline bool prescaled_batch(int64_t M, int64_t E, int64_t k) {
  return (double)M * (double)k / (double)E >= MOE_PRESCALED_MIN_PER_EXPERT;
}

// Workspace layout of the forward:
// [acc fp32 M x H][act bf16 M*k x I][tile count int32 (16 B)][tile table int2]
// and, for batches the pre-scaled tiled kernel may take, the fp16 copies of
// the A rows (x [M, H] for FC1, then act [M*k, I] for FC2, in the same
// region) and their power-of-two row exponents.
struct WorkspaceLayout {
  int64_t acc_off, act_off, ntiles_off, tiles_off, a16_off, a16exp_off, total;
};
inline int64_t align256(int64_t v) { return (v + 255) & ~int64_t(255); }
inline WorkspaceLayout workspace_layout(int64_t M, int64_t E, int64_t H, int64_t I, int64_t k) {
  WorkspaceLayout w;
  w.acc_off = 0;
  w.act_off = align256(M * H * 4);
  w.ntiles_off = w.act_off + align256(M * k * I * 2);
  w.tiles_off = w.ntiles_off + 256;
  w.total = w.tiles_off + align256(tile_table_entries(M, k) * 8);
  w.a16_off = w.a16exp_off = 0;
  if (prescaled_batch(M, E, k)) {
    const int64_t a16_elems = M * H > M * k * I ? M * H : M * k * I;
    const int64_t a16_rows = M * k;  // >= M
    w.a16_off = w.total;
    w.a16exp_off = w.a16_off + align256(a16_elems * 2);
    w.total = w.a16exp_off + align256(a16_rows * 4);
  }
  return w;
}

// Kernel launchers (each returns the hipError_t of its launches).
hipError_t launch_route_align(const float* logits, int M, int E, int k, int block_m,
                              int32_t* topk_ids, float* topk_weights, int32_t* sorted_ids,
                              int32_t* block_expert, int32_t* offsets, int32_t* npp,
                              int64_t cap, hipStream_t stream);

// s: fp16 scales (kFmtInt4) or E8M0 bytes (kFmtMxfp4), [E, N, K/32].
hipError_t launch_repack(int fmt, const uint8_t* q, const void* s, int E, int N, int K, int kind,
                         uint8_t* packed, hipStream_t stream);
hipError_t launch_unpack(int fmt, const uint8_t* packed, int E, int N, int K, int kind, uint8_t* q,
                         void* s, hipStream_t stream);

struct FcArgs {
  const uint16_t* act_in;      // FC1: x [M, H]; FC2: act [M*k, I]
  const uint8_t* wpacked;      // repacked weights
  const int32_t* sorted_ids;   // [cap]
  const int32_t* block_expert; // [cap / block_m]
  const int32_t* npp;          // [1]
  const float* topk_weights;   // FC2 only, [M*k]
  uint16_t* act_out;           // FC1 only: act [M*k, I]
  float* acc;                  // fp32 [M, H]
  uint16_t* out;               // FC2 only: bf16 [M, H]
  int M, E, H, I, k, block_m;
  int64_t cap;
  int64_t zero_words16;         // FC1: 16-byte words of acc to clear
  // tiled paths only (tiles != nullptr): the tile table FC1's plan writes
  int2* tiles;                  // [max_tiles]
  int32_t* ntiles;              // [1]
  int max_tiles;                // grid tiles (a multiple of 8)
  int tile_rows;                // rows per tile (whole blocks)
  // INT4 weights only
  uint16_t* a16;                // fp16 copies of the A rows (workspace)
  int32_t* a16_exp;             // their row exponents
  const int32_t* row_exp;       // the A rows' exponents as the kernel reads them
  const int8_t* wsigma;         // per-weight-row shifts of the blob (E x N)
  // block_m = 128 on the block kernels (workspace, where the tile table
  // would be): the expert of each 64-row half of a block, -1 for a half
  // that holds no row
  int32_t* half_expert;
};

// Decode path (tiny batches): routing fused into FC1, output-stationary FC2.
constexpr int kMaxTopK = 16;
constexpr int kDecodeMaxTokens = 4;
constexpr int kDecodeMaxAssign = 64;  // M * k
// The decode kernels stage the batch's x rows (FC1) and the k activation
// rows of a token (FC2) in LDS; shapes whose rows do not fit take the
// general path.
// The staged rows also carry their -136 * (group sum) corrections: FC1 one
// float4 per group (the batch's 4 token slots), FC2 one float4 per group and
// row (the value replicated, the accumulator input of one MFMA).
constexpr int64_t kDecodeMaxStagedBytes = 64 * 1024;
inline int64_t decode_fc1_lds_bytes(int64_t M, int64_t H) { return M * (H / 8 + 1) * 16 + (H / 32) * 16; }
inline int64_t decode_fc2_lds_bytes(int64_t I, int64_t k) { return k * (I * 2 + (I / 32) * 4); }
inline bool decode_path_fits(int64_t M, int64_t H, int64_t I, int64_t k) {
  return M >= 1 && M <= kDecodeMaxTokens && M * k <= kDecodeMaxAssign &&
         decode_fc1_lds_bytes(M, H) <= kDecodeMaxStagedBytes && decode_fc2_lds_bytes(I, k) <= kDecodeMaxStagedBytes;
}
struct DecodeArgs {
  FcArgs fc;               // FC1 view: act_in = x, wpacked = W13, act_out = act, out = output
  const float* logits;     // [M, E]
  const uint8_t* w2;       // repacked W2
  int32_t* topk_ids;       // [M*k]
  float* topk_weights;     // [M*k]
  int32_t* sorted_ids;     // [cap], block_m-padded as by moe_route_align
  int32_t* block_expert;   // [cap / block_m]
  int32_t* expert_offsets; // [E + 1]
  int32_t* npp_out;        // [1]
  int block_m;
};
// Small batches take launch_fc2_tokens in moe_w4a16_layer: it reads each
// (token, slot)'s expert once, so an expert that several tokens share is
// read again, but it needs no accumulator, atomics or finalize kernel and
// splits into M * H / 32 equal workgroups (no partly filled last round).
// Taken up to 16 tokens while the M*k expert reads stay within 1.2x the
// expected number of distinct experts, E * (1 - (1 - k/E)^M) (on the
// 384-expert top-8 layer: M = 9 and 16 measured ~1 % faster, 24 and 32
// slower).
#ifndef MOE_TOKEN_FC2_MAX_TOKENS
#define MOE_TOKEN_FC2_MAX_TOKENS 16
#endif
constexpr int kTokenFc2MaxTokens = MOE_TOKEN_FC2_MAX_TOKENS;
inline bool token_fc2_fits(int64_t M, int64_t E, int64_t I, int64_t k) {
  if (M > kTokenFc2MaxTokens || k > 8 || decode_fc2_lds_bytes(I, k) > kDecodeMaxStagedBytes) return false;
  double miss = 1.0;  // probability that a given expert is not among M tokens' top-k (uniform routing)
  for (int64_t t = 0; t < M; ++t) miss *= 1.0 - (double)k / (double)E;
  return (double)(M * k) <= 1.2 * (double)E * (1.0 - miss);
}

// Launchers of the format-dependent kernels, declared for both formats
// (namespaces fmt_int4 and fmt_mxfp4); each is defined by that format's
// build of fc.hip, fc_prescaled.hip or decode.hip.
//   launch_fc1 / launch_fc2   grouped GEMM stages; ev_start / ev_stop (may be
//                             null) take FC1's own start and end timestamps
//                             (hipExtLaunchKernel), for timing the stage
//                             without extra packets
//   tile_grid_tiles, launch_tile_plan, prescaled_supported, launch_fc_prescaled
//                             the pre-scaled tiled grouped GEMM (fc_prescaled.hip)
//   launch_decode             routing fused into FC1 + output-stationary FC2
//                             for tiny batches; events as for launch_fc1
//   launch_fc2_tokens         FC2 + combine per token (output-stationary, no
//                             accumulator): act rows in d.fc.act_in, ids and
//                             weights in d.topk_ids / d.topk_weights, output
//                             d.fc.out
//   routed_fc1_fits, routed_fc1_preferred, launch_fc1_routed
//                             routing, grouping and FC1 in one kernel for up
//                             to 16 tokens (M*k <= 256, E <= 1024, the x rows
//                             within 128 KB of LDS: M <= 9 at H = 7168): fills every
//                             output moe_route_align fills (d.topk_ids ...
//                             d.npp_out, in d.block_m-row blocks) and FC1's
//                             activation rows, clears d.fc.zero_words16
//                             16-byte words of d.fc.acc (0: none);
//                             "preferred" = fits and the grouped wide kernel
//                             would leave CUs idle (queries the device)
#define MOE_FORMAT_LAUNCHERS \
  hipError_t launch_fc1(const FcArgs& a, hipStream_t stream, hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr); \
  hipError_t launch_fc2(const FcArgs& a, hipStream_t stream); \
  int64_t tile_grid_tiles(int64_t M, int64_t E, int64_t k, int64_t block_m, int64_t cap, int64_t tile_rows); \
  bool prescaled_supported(int64_t H, int64_t I); \
  template <bool kFc1> hipError_t launch_fc_prescaled(const FcArgs& a, hipStream_t stream, hipEvent_t e0, hipEvent_t e1); \
  hipError_t launch_tile_plan(const FcArgs& a, hipStream_t stream); \
  hipError_t launch_decode(const DecodeArgs& d, hipStream_t stream, hipEvent_t ev_start, hipEvent_t ev_stop); \
  hipError_t launch_fc2_tokens(const DecodeArgs& d, hipStream_t stream); \
  bool routed_fc1_fits(int64_t M, int64_t E, int64_t H, int64_t I, int64_t k); \
  bool routed_fc1_preferred(int64_t M, int64_t E, int64_t H, int64_t I, int64_t k); \
  hipError_t launch_fc1_routed(const DecodeArgs& d, hipStream_t stream, hipEvent_t ev_start, hipEvent_t ev_stop);
namespace fmt_int4 {
MOE_FORMAT_LAUNCHERS
}  // namespace fmt_int4
namespace fmt_mxfp4 {
MOE_FORMAT_LAUNCHERS
}  // namespace fmt_mxfp4

// fp16 copies of bf16 rows [rows, K], each scaled by 2^-e so that its
// largest magnitude lies in [2^14, 2^15) (e = 0 for an all-zero row); e goes
// to exps[row] (fc_prescaled.hip, INT4 build).
hipError_t launch_rowscale(const uint16_t* in, int64_t rows, int64_t K, uint16_t* out, int32_t* exps,
                           hipStream_t stream);
// One int8 per weight row (E x N) after the INT4 tiles: see sigma_trailer_bytes.
hipError_t launch_row_sigma(const uint16_t* scales_f16, int E, int N, int K, int8_t* sigma, hipStream_t stream);

// Launch with optional kernel-timestamp events.
template <typename... KArgs, typename... Args>
inline void launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, uint32_t shmem, hipStream_t s,
                          hipEvent_t ev_start, hipEvent_t ev_stop, Args... args) {
  if (ev_start || ev_stop)
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, s, ev_start, ev_stop, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, shmem, s, args...);
}

}  // namespace moe

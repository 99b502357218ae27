// Exported C entry points: host-side validation, sizes, and kernel launches.
// Every check runs before the first HIP call, so an invalid call launches
// nothing and touches no output.
#include <atomic>
#include <mutex>

#include "../../include/moe_w4a16.h"
#include "internal.h"

namespace {

using moe::kChunkK;
using moe::kGroup;
using moe::kPairRows;

constexpr int32_t kAbiVersion = 3;
constexpr int32_t kMaxExperts = 1024;
using moe::kMaxTopK;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
bool block_m_ok(int32_t b) { return b == 16 || b == 32 || b == 64 || b == 128; }

// One expert's repacked tensor (N rows of K channels, either format) stays
// below 2^31 bytes, so in-expert offsets fit 32 bits and E times it fits int64.
bool expert_bytes_ok(int32_t N, int32_t K) {
  return moe::packed_bytes_fmt(moe::kFmtInt4, N, K) < (int64_t(1) << 31);
}

// Size checks shared by the entry points. Returns MOE_OK or an error code.
int check_layer(int32_t M, int32_t E, int32_t H, int32_t I, int32_t k) {
  if (M < 0 || E <= 0 || H <= 0 || I <= 0 || k <= 0) return MOE_ERR_INVALID_ARG;
  if (E > kMaxExperts || k > kMaxTopK || k > E) return MOE_ERR_UNSUPPORTED;
  if (H % kChunkK != 0 || I % kChunkK != 0) return MOE_ERR_UNSUPPORTED;
  if (I > (int32_t(1) << 30) || !expert_bytes_ok(2 * I, H) || !expert_bytes_ok(H, I)) return MOE_ERR_UNSUPPORTED;
  const int64_t mk = (int64_t)M * k;
  const int64_t widest = H > I ? H : I;
  if (mk * widest >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int64_t capacity(int32_t M, int32_t E, int32_t k, int32_t block_m) {
  const int64_t mk = (int64_t)M * k;
  const int64_t touched = mk < E ? mk : E;
  const int64_t raw = mk + touched * (block_m - 1);
  return (raw + block_m - 1) / block_m * block_m;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

}  // namespace

// A launcher of the kernels for weight format `fmt` (moe::kFmtInt4 or
// moe::kFmtMxfp4).
#define FMT_CALL(fmt, fn, ...) \
  ((fmt) == moe::kFmtMxfp4 ? moe::fmt_mxfp4::fn(__VA_ARGS__) : moe::fmt_int4::fn(__VA_ARGS__))

extern "C" {

int32_t moe_w4a16_abi_version(void) { return kAbiVersion; }

const char* moe_w4a16_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument (null or misaligned pointer, or negative size)";
    case MOE_ERR_UNSUPPORTED: return "unsupported size (see the limits in moe_w4a16.h)";
    case MOE_ERR_CAPACITY: return "cap is smaller than moe_route_align_capacity() or not a multiple of block_m";
    case MOE_ERR_WORKSPACE: return "workspace is smaller than moe_w4a16_workspace_bytes()";
    case MOE_ERR_HIP: return "a HIP kernel launch failed";
    case MOE_ERR_SCRATCH:
      return "the batch needs more workspace than moe_w4a16_layer_noalloc's static scratch "
             "(MOE_W4A16_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int64_t moe_route_align_capacity(int32_t M, int32_t E, int32_t top_k, int32_t block_m) {
  if (M < 0 || E <= 0 || E > kMaxExperts || top_k <= 0 || top_k > E || top_k > kMaxTopK ||
      !block_m_ok(block_m))
    return -1;
  return capacity(M, E, top_k, block_m);
}

int moe_route_align(const float* logits, int32_t M, int32_t E, int32_t top_k, int32_t block_m,
                    int32_t* topk_ids, float* topk_weights, int32_t* sorted_token_ids,
                    int32_t* block_expert_ids, int32_t* expert_offsets, int32_t* num_tokens_post_pad,
                    int64_t cap, void* stream) {
  if (M < 0 || E <= 0 || top_k <= 0) return MOE_ERR_INVALID_ARG;
  if (E > kMaxExperts || top_k > E || top_k > kMaxTopK || !block_m_ok(block_m)) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)M * top_k >= (int64_t(1) << 30)) return MOE_ERR_UNSUPPORTED;
  if (M == 0) return MOE_OK;
  if (!logits || !topk_ids || !topk_weights || !sorted_token_ids || !block_expert_ids ||
      !expert_offsets || !num_tokens_post_pad)
    return MOE_ERR_INVALID_ARG;
  if (!aligned4(logits) || !aligned4(topk_ids) || !aligned4(topk_weights) || !aligned4(sorted_token_ids) ||
      !aligned4(block_expert_ids) || !aligned4(expert_offsets) || !aligned4(num_tokens_post_pad))
    return MOE_ERR_INVALID_ARG;
  if (cap < capacity(M, E, top_k, block_m) || cap % block_m != 0) return MOE_ERR_CAPACITY;
  return hip_status(moe::launch_route_align(logits, M, E, top_k, block_m, topk_ids, topk_weights,
                                            sorted_token_ids, block_expert_ids, expert_offsets,
                                            num_tokens_post_pad, cap, (hipStream_t)stream));
}

int64_t moe_w4a16_packed_bytes(int32_t E, int32_t N, int32_t K, int32_t group) {
  if (E <= 0 || N <= 0 || K <= 0 || group != kGroup || N % kPairRows != 0 || K % kChunkK != 0) return -1;
  if (E > kMaxExperts || !expert_bytes_ok(N, K)) return -1;
  return (int64_t)E * moe::packed_bytes_fmt(moe::kFmtInt4, N, K) + moe::sigma_trailer_bytes(moe::kFmtInt4, E, N);
}

int64_t moe_mxfp4_packed_bytes(int32_t E, int32_t N, int32_t K) {
  if (E <= 0 || N <= 0 || K <= 0 || N % kPairRows != 0 || K % kChunkK != 0) return -1;
  if (E > kMaxExperts || !expert_bytes_ok(N, K)) return -1;
  return (int64_t)E * moe::packed_bytes_fmt(moe::kFmtMxfp4, N, K);
}

static int check_repack(const void* a, const void* b, const void* c, int32_t E, int32_t N, int32_t K,
                        int32_t group, int32_t kind) {
  if (E <= 0 || N <= 0 || K <= 0) return MOE_ERR_INVALID_ARG;
  if (kind != 0 && kind != 1) return MOE_ERR_INVALID_ARG;
  if (group != kGroup || N % kPairRows != 0 || K % kChunkK != 0) return MOE_ERR_UNSUPPORTED;
  if (E > kMaxExperts || !expert_bytes_ok(N, K)) return MOE_ERR_UNSUPPORTED;
  if (kind == 0 && (N / 2) % 16 != 0) return MOE_ERR_UNSUPPORTED;
  if (!a || !b || !c) return MOE_ERR_INVALID_ARG;
  if (!aligned16(a) || !aligned16(b) || !aligned16(c)) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

int moe_w4a16_repack(const uint8_t* qweight, const uint16_t* scales_f16, int32_t E, int32_t N, int32_t K,
                     int32_t group, int32_t kind, void* packed, void* stream) {
  const int st = check_repack(qweight, scales_f16, packed, E, N, K, group, kind);
  if (st != MOE_OK) return st;
  return hip_status(moe::launch_repack(moe::kFmtInt4, qweight, scales_f16, E, N, K, kind, (uint8_t*)packed,
                                       (hipStream_t)stream));
}

int moe_mxfp4_repack(const uint8_t* qweight, const uint8_t* scales_e8m0, int32_t E, int32_t N, int32_t K,
                     int32_t kind, void* packed, void* stream) {
  const int st = check_repack(qweight, scales_e8m0, packed, E, N, K, kGroup, kind);
  if (st != MOE_OK) return st;
  return hip_status(moe::launch_repack(moe::kFmtMxfp4, qweight, scales_e8m0, E, N, K, kind, (uint8_t*)packed,
                                       (hipStream_t)stream));
}

int moe_w4a16_unpack(const void* packed, int32_t E, int32_t N, int32_t K, int32_t group, int32_t kind,
                     uint8_t* qweight, uint16_t* scales_f16, void* stream) {
  const int st = check_repack(packed, qweight, scales_f16, E, N, K, group, kind);
  if (st != MOE_OK) return st;
  return hip_status(moe::launch_unpack(moe::kFmtInt4, (const uint8_t*)packed, E, N, K, kind, qweight, scales_f16,
                                       (hipStream_t)stream));
}

int moe_mxfp4_unpack(const void* packed, int32_t E, int32_t N, int32_t K, int32_t kind, uint8_t* qweight,
                     uint8_t* scales_e8m0, void* stream) {
  const int st = check_repack(packed, qweight, scales_e8m0, E, N, K, kGroup, kind);
  if (st != MOE_OK) return st;
  return hip_status(moe::launch_unpack(moe::kFmtMxfp4, (const uint8_t*)packed, E, N, K, kind, qweight,
                                       scales_e8m0, (hipStream_t)stream));
}

int64_t moe_w4a16_workspace_bytes(int32_t M, int32_t E, int32_t H, int32_t I, int32_t top_k) {
  if (check_layer(M, E, H, I, top_k) != MOE_OK) return -1;
  return moe::workspace_layout(M, E, H, I, top_k).total;
}

int32_t moe_w4a16_preferred_block_m(int32_t M, int32_t E, int32_t H, int32_t I, int32_t top_k) {
  if (check_layer(M, E, H, I, top_k) != MOE_OK) return -1;
  // Measured on the 384-expert layer (M = 9 ... 1024): 32-row blocks (the
  // wide kernel, one LDS-staged activation chunk shared by 16 tile pairs)
  // beat 16-row blocks from M = 9 up, and 64-row blocks only pay off once an
  // expert averages more than ~24 rows. Batches of a few assignments keep
  // 16-row blocks: the wide kernel would launch too few workgroups.
  // From MOE_PRESCALED_MIN_PER_EXPERT on the pre-scaled tiled kernel runs,
  // whose tiles are up to 128 rows of whole blocks.
  const double per_expert = (double)M * top_k / E;
  if ((int64_t)M * top_k <= 32) return 16;
  if (moe::prescaled_batch(M, E, top_k) && moe::fmt_int4::prescaled_supported(H, I)) return 32;
  if (per_expert <= 24.0) return 32;
  return 64;
}

static int check_fc(int32_t M, int32_t E, int32_t H, int32_t I, int32_t top_k, int32_t block_m, int64_t cap,
                    int64_t workspace_bytes) {
  const int st = check_layer(M, E, H, I, top_k);
  if (st != MOE_OK) return st;
  if (!block_m_ok(block_m)) return MOE_ERR_UNSUPPORTED;
  if (M == 0) return MOE_OK;
  if (cap < capacity(M, E, top_k, block_m) || cap % block_m != 0) return MOE_ERR_CAPACITY;
  if (workspace_bytes < moe::workspace_layout(M, E, H, I, top_k).total) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

// The pre-scaled tiled grouped GEMM (fc_prescaled.hip) takes the batch from
// MOE_PRESCALED_MIN_PER_EXPERT assignments per expert on, where the shape
// divides into its pair groups and a block fits in its largest tile (a build
// with smaller INT4 tiles leaves 128-row blocks to the block kernels); the
// block kernels of fc.hip take the rest.
static bool use_tiled(int fmt, int32_t M, int32_t E, int32_t H, int32_t I, int32_t top_k, int32_t block_m) {
  return moe::prescaled_batch(M, E, top_k) && FMT_CALL(fmt, prescaled_supported, H, I) &&
         block_m <= moe::prescaled_max_rows(fmt);
}

// The weights a stage reads: the blob and, for INT4, its per-row shifts.
static void set_weights(moe::FcArgs& a, int fmt, const void* packed, int32_t N, int32_t K) {
  a.wpacked = (const uint8_t*)packed;
  a.wsigma = fmt == moe::kFmtInt4
                 ? (const int8_t*)(a.wpacked + (int64_t)a.E * moe::packed_bytes_fmt(moe::kFmtInt4, N, K))
                 : nullptr;
}

static moe::FcArgs fc_args(int fmt, int32_t M, int32_t E, int32_t H, int32_t I, int32_t top_k, int32_t block_m,
                           int64_t cap, const int32_t* sorted_ids, const int32_t* block_expert,
                           const int32_t* npp, void* workspace) {
  moe::FcArgs a{};
  const moe::WorkspaceLayout L = moe::workspace_layout(M, E, H, I, top_k);
  uint8_t* ws = (uint8_t*)workspace;
  a.sorted_ids = sorted_ids;
  a.block_expert = block_expert;
  a.npp = npp;
  a.acc = (float*)(ws + L.acc_off);
  a.act_out = (uint16_t*)(ws + L.act_off);
  a.M = M; a.E = E; a.H = H; a.I = I; a.k = top_k; a.block_m = block_m;
  // The block kernels' grid is sized from the padded total this batch can
  // reach, not from the caller's cap (route buffers may be allocated for a
  // larger batch): the rows past it are never part of the batch.
  const int64_t reach = capacity(M, E, top_k, block_m);
  a.cap = cap < reach ? cap : reach;
  a.zero_words16 = (int64_t)M * H * 4 / 16;
  if (use_tiled(fmt, M, E, H, I, top_k, block_m)) {
    a.tiles = (int2*)(ws + L.tiles_off);
    a.ntiles = (int32_t*)(ws + L.ntiles_off);
    a.tile_rows = moe::prescaled_tile_rows(fmt, block_m);
    // The grid is sized from the padded total this batch can reach, not from
    // the caller's cap (route buffers may be allocated for a larger batch):
    // the tile table in the workspace holds tile_table_entries(M, k) entries.
    a.max_tiles =
        (int)FMT_CALL(fmt, tile_grid_tiles, M, E, top_k, block_m, capacity(M, E, top_k, block_m), a.tile_rows);
    // the workspace has the fp16 row copies (prescaled_batch)
    a.a16 = (uint16_t*)(ws + L.a16_off);
    a.a16_exp = (int32_t*)(ws + L.a16exp_off);
  } else if (block_m == 128) {
    // The block kernels run each block as two 64-row halves, with a map of
    // the halves' experts where the tile table would be: cap / 64 <= 2 M k + 2
    // entries (cap being at most the batch's capacity, above).
    a.half_expert = (int32_t*)(ws + L.tiles_off);
  }
  return a;
}

static int fc1_impl(int fmt, const uint16_t* x_bf16, int32_t M, int32_t E, int32_t H, int32_t I, int32_t top_k,
                  int32_t block_m, const int32_t* sorted_token_ids, const int32_t* block_expert_ids,
                  const int32_t* num_tokens_post_pad, int64_t cap, const void* w13_packed, void* workspace,
                  int64_t workspace_bytes, void* stream) {
  int st = check_fc(M, E, H, I, top_k, block_m, cap, workspace_bytes);
  if (st != MOE_OK || M == 0) return st;
  if (!x_bf16 || !sorted_token_ids || !block_expert_ids || !num_tokens_post_pad || !w13_packed || !workspace)
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(x_bf16) || !aligned16(w13_packed) || !aligned16(workspace) || !aligned4(sorted_token_ids) ||
      !aligned4(block_expert_ids) || !aligned4(num_tokens_post_pad))
    return MOE_ERR_INVALID_ARG;
  moe::FcArgs a = fc_args(fmt, M, E, H, I, top_k, block_m, cap, sorted_token_ids, block_expert_ids,
                          num_tokens_post_pad, workspace);
  a.act_in = x_bf16;
  set_weights(a, fmt, w13_packed, 2 * I, H);
  return hip_status(FMT_CALL(fmt, launch_fc1, a, (hipStream_t)stream));
}

static int fc2_impl(int fmt, int32_t M, int32_t E, int32_t H, int32_t I, int32_t top_k, int32_t block_m,
                  const float* topk_weights, const int32_t* sorted_token_ids, const int32_t* block_expert_ids,
                  const int32_t* num_tokens_post_pad, int64_t cap, const void* w2_packed, void* workspace,
                  int64_t workspace_bytes, uint16_t* out_bf16, void* stream) {
  int st = check_fc(M, E, H, I, top_k, block_m, cap, workspace_bytes);
  if (st != MOE_OK || M == 0) return st;
  if (!topk_weights || !sorted_token_ids || !block_expert_ids || !num_tokens_post_pad || !w2_packed ||
      !workspace || !out_bf16)
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(w2_packed) || !aligned16(workspace) || !aligned16(out_bf16) || !aligned4(topk_weights) ||
      !aligned4(sorted_token_ids) || !aligned4(block_expert_ids) || !aligned4(num_tokens_post_pad))
    return MOE_ERR_INVALID_ARG;
  moe::FcArgs a = fc_args(fmt, M, E, H, I, top_k, block_m, cap, sorted_token_ids, block_expert_ids,
                          num_tokens_post_pad, workspace);
  a.act_in = a.act_out;  // FC2 reads the FC1 activations
  a.act_out = nullptr;
  set_weights(a, fmt, w2_packed, H, I);
  a.topk_weights = topk_weights;
  a.out = out_bf16;
  return hip_status(FMT_CALL(fmt, launch_fc2, a, (hipStream_t)stream));
}

static int forward_impl(int fmt, const uint16_t* x_bf16, int32_t M, int32_t E, int32_t H, int32_t I, int32_t top_k,
                      int32_t block_m, const float* topk_weights, const int32_t* sorted_token_ids,
                      const int32_t* block_expert_ids, const int32_t* expert_offsets,
                      const int32_t* num_tokens_post_pad, int64_t cap, const void* w13_packed,
                      const void* w2_packed, void* workspace, int64_t workspace_bytes, uint16_t* out_bf16,
                      void* stream) {
  int st = check_fc(M, E, H, I, top_k, block_m, cap, workspace_bytes);
  if (st != MOE_OK || M == 0) return st;
  if (!x_bf16 || !topk_weights || !sorted_token_ids || !block_expert_ids || !expert_offsets ||
      !num_tokens_post_pad || !w13_packed || !w2_packed || !workspace || !out_bf16)
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(x_bf16) || !aligned16(w13_packed) || !aligned16(w2_packed) || !aligned16(workspace) ||
      !aligned16(out_bf16) || !aligned4(topk_weights) || !aligned4(sorted_token_ids) ||
      !aligned4(block_expert_ids) || !aligned4(expert_offsets) || !aligned4(num_tokens_post_pad))
    return MOE_ERR_INVALID_ARG;
  st = fc1_impl(fmt, x_bf16, M, E, H, I, top_k, block_m, sorted_token_ids, block_expert_ids,
                num_tokens_post_pad, cap, w13_packed, workspace, workspace_bytes, stream);
  if (st != MOE_OK) return st;
  return fc2_impl(fmt, M, E, H, I, top_k, block_m, topk_weights, sorted_token_ids, block_expert_ids,
                  num_tokens_post_pad, cap, w2_packed, workspace, workspace_bytes, out_bf16, stream);
}

static int layer_impl(int fmt, const float* logits, const uint16_t* x_bf16, int32_t M, int32_t E, int32_t H, int32_t I,
                    int32_t top_k, int32_t block_m, int32_t* topk_ids, float* topk_weights,
                    int32_t* sorted_token_ids, int32_t* block_expert_ids, int32_t* expert_offsets,
                    int32_t* num_tokens_post_pad, int64_t cap, const void* w13_packed, const void* w2_packed,
                    void* workspace, int64_t workspace_bytes, uint16_t* out_bf16, void* stream,
                    void* const* stage_events) {
  int st = check_fc(M, E, H, I, top_k, block_m, cap, workspace_bytes);
  if (st != MOE_OK || M == 0) return st;
  if (!logits || !x_bf16 || !topk_ids || !topk_weights || !sorted_token_ids || !block_expert_ids ||
      !expert_offsets || !num_tokens_post_pad || !w13_packed || !w2_packed || !workspace || !out_bf16)
    return MOE_ERR_INVALID_ARG;
  if (!aligned4(logits) || !aligned16(x_bf16) || !aligned4(topk_ids) || !aligned4(topk_weights) ||
      !aligned4(sorted_token_ids) || !aligned4(block_expert_ids) || !aligned4(expert_offsets) ||
      !aligned4(num_tokens_post_pad) || !aligned16(w13_packed) || !aligned16(w2_packed) ||
      !aligned16(workspace) || !aligned16(out_bf16))
    return MOE_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  hipEvent_t ev0 = stage_events ? (hipEvent_t)stage_events[0] : nullptr;
  hipEvent_t ev1 = stage_events ? (hipEvent_t)stage_events[1] : nullptr;
  // The decode path for one token (measured on the 384-expert layer: decode
  // 42.9 vs routed 46.4 us at M = 1), and for four tokens where the routed
  // FC1 would not fill the device; the routed FC1 while few experts are
  // touched (82.7 vs 80.4 us at M = 2), and for two or three tokens wherever
  // the decode path fits (the routed kernel always fits there); else the
  // grouped kernels. The routed FC1 writes no tile table, so it is not
  // combined with the tiled grouped FC2.
  const bool tiled = use_tiled(fmt, M, E, H, I, top_k, block_m);
  const bool decode_fits = moe::decode_path_fits(M, H, I, top_k);
  const bool routed_pref = FMT_CALL(fmt, routed_fc1_preferred, M, E, H, I, top_k);
  const bool decode = decode_fits && (M == 1 || (M == moe::kDecodeMaxTokens && !routed_pref));
  const bool routed = !decode && !tiled &&
                      (routed_pref || (decode_fits && FMT_CALL(fmt, routed_fc1_fits, M, E, H, I, top_k)));
  if (decode) {
    moe::DecodeArgs d{};
    d.fc = fc_args(fmt, M, E, H, I, top_k, block_m, cap, sorted_token_ids, block_expert_ids, num_tokens_post_pad,
                   workspace);
    d.fc.act_in = x_bf16;
    d.fc.wpacked = (const uint8_t*)w13_packed;
    d.fc.topk_weights = topk_weights;
    d.fc.out = out_bf16;
    d.logits = logits;
    d.w2 = (const uint8_t*)w2_packed;
    d.topk_ids = topk_ids;
    d.topk_weights = topk_weights;
    d.sorted_ids = sorted_token_ids;
    d.block_expert = block_expert_ids;
    d.expert_offsets = expert_offsets;
    d.npp_out = num_tokens_post_pad;
    d.block_m = block_m;
    return hip_status(FMT_CALL(fmt, launch_decode, d, s, ev0, ev1));
  }
  const bool token_fc2 = moe::token_fc2_fits(M, E, I, top_k);
  if (routed) {  // routing and grouping inside FC1's workgroups
    moe::DecodeArgs d{};
    d.fc = fc_args(fmt, M, E, H, I, top_k, block_m, cap, sorted_token_ids, block_expert_ids, num_tokens_post_pad,
                   workspace);
    d.fc.act_in = x_bf16;
    d.fc.wpacked = (const uint8_t*)w13_packed;
    if (token_fc2) d.fc.zero_words16 = 0;  // the per-token FC2 has no accumulator
    d.logits = logits;
    d.topk_ids = topk_ids;
    d.topk_weights = topk_weights;
    d.sorted_ids = sorted_token_ids;
    d.block_expert = block_expert_ids;
    d.expert_offsets = expert_offsets;
    d.npp_out = num_tokens_post_pad;
    d.block_m = block_m;
    st = hip_status(FMT_CALL(fmt, launch_fc1_routed, d, s, ev0, ev1));
  } else {
    st = moe_route_align(logits, M, E, top_k, block_m, topk_ids, topk_weights, sorted_token_ids, block_expert_ids,
                         expert_offsets, num_tokens_post_pad, cap, stream);
    if (st != MOE_OK) return st;
    moe::FcArgs a = fc_args(fmt, M, E, H, I, top_k, block_m, cap, sorted_token_ids, block_expert_ids,
                            num_tokens_post_pad, workspace);
    a.act_in = x_bf16;
    set_weights(a, fmt, w13_packed, 2 * I, H);
    st = hip_status(FMT_CALL(fmt, launch_fc1, a, s, ev0, ev1));
  }
  if (st != MOE_OK) return st;
  if (token_fc2) {  // small batches: FC2 per token, no accumulator
    moe::DecodeArgs d2{};
    d2.fc = fc_args(fmt, M, E, H, I, top_k, block_m, cap, sorted_token_ids, block_expert_ids, num_tokens_post_pad,
                    workspace);
    d2.fc.act_in = d2.fc.act_out;  // FC1's activations
    d2.fc.act_out = nullptr;
    d2.fc.wpacked = (const uint8_t*)w2_packed;
    d2.fc.out = out_bf16;
    d2.topk_ids = topk_ids;
    d2.topk_weights = topk_weights;
    return hip_status(FMT_CALL(fmt, launch_fc2_tokens, d2, s));
  }
  return fc2_impl(fmt, M, E, H, I, top_k, block_m, topk_weights, sorted_token_ids, block_expert_ids,
                  num_tokens_post_pad, cap, w2_packed, workspace, workspace_bytes, out_bf16, stream);
}

int moe_w4a16_fc1(const uint16_t* x_bf16, int32_t M, int32_t E, int32_t H, int32_t I, int32_t top_k, int32_t block_m,
              const int32_t* sorted_token_ids, const int32_t* block_expert_ids, const int32_t* num_tokens_post_pad,
              int64_t cap, const void* w13_packed, void* workspace, int64_t workspace_bytes, void* stream) {
  return fc1_impl(moe::kFmtInt4, x_bf16, M, E, H, I, top_k, block_m, sorted_token_ids, block_expert_ids,
                  num_tokens_post_pad, cap, w13_packed, workspace, workspace_bytes, stream);
}

int moe_w4a16_fc2(int32_t M, int32_t E, int32_t H, int32_t I, int32_t top_k, int32_t block_m, const float* topk_weights,
              const int32_t* sorted_token_ids, const int32_t* block_expert_ids, const int32_t* num_tokens_post_pad,
              int64_t cap, const void* w2_packed, void* workspace, int64_t workspace_bytes, uint16_t* out_bf16,
              void* stream) {
  return fc2_impl(moe::kFmtInt4, M, E, H, I, top_k, block_m, topk_weights, sorted_token_ids, block_expert_ids,
                  num_tokens_post_pad, cap, w2_packed, workspace, workspace_bytes, out_bf16, stream);
}

int moe_w4a16_forward(const uint16_t* x_bf16, int32_t M, int32_t E, int32_t H, int32_t I, int32_t top_k, int32_t block_m,
                  const float* topk_weights, const int32_t* sorted_token_ids, const int32_t* block_expert_ids,
                  const int32_t* expert_offsets, const int32_t* num_tokens_post_pad, int64_t cap,
                  const void* w13_packed, const void* w2_packed, void* workspace, int64_t workspace_bytes,
                  uint16_t* out_bf16, void* stream) {
  return forward_impl(moe::kFmtInt4, x_bf16, M, E, H, I, top_k, block_m, topk_weights, sorted_token_ids, block_expert_ids,
                      expert_offsets, num_tokens_post_pad, cap, w13_packed, w2_packed, workspace, workspace_bytes,
                      out_bf16, stream);
}

int moe_w4a16_layer(const float* logits, const uint16_t* x_bf16, int32_t M, int32_t E, int32_t H, int32_t I,
                int32_t top_k, int32_t block_m, int32_t* topk_ids, float* topk_weights, int32_t* sorted_token_ids,
                int32_t* block_expert_ids, int32_t* expert_offsets, int32_t* num_tokens_post_pad, int64_t cap,
                const void* w13_packed, const void* w2_packed, void* workspace, int64_t workspace_bytes,
                uint16_t* out_bf16, void* stream, void* const* stage_events) {
  return layer_impl(moe::kFmtInt4, logits, x_bf16, M, E, H, I, top_k, block_m, topk_ids, topk_weights, sorted_token_ids,
                    block_expert_ids, expert_offsets, num_tokens_post_pad, cap, w13_packed, w2_packed, workspace,
                    workspace_bytes, out_bf16, stream, stage_events);
}

}  // extern "C"

// ---- the no-allocation layer call -----------------------------------------
// Its workspace: one static device array per GPU (the library allocates
// nothing). In host code `scratch` names a host-side stand-in, not device
// memory: the device address comes from hipGetSymbolAddress, once per device
// with that device current, and only that address is handed to kernels.
namespace {
constexpr int64_t kScratchBytes = MOE_W4A16_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxScratchDevices];
std::mutex g_scratch_mu;

// The current device's scratch address (resolved on the first call on it).
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MOE_ERR_HIP;
  if (dev >= kMaxScratchDevices) return MOE_ERR_UNSUPPORTED;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return MOE_OK;
}
}  // namespace

extern "C" {

int moe_w4a16_layer_noalloc(const float* logits, const uint16_t* x_bf16, int32_t M, int32_t E, int32_t H, int32_t I,
                            int32_t top_k, int32_t block_m, int32_t* topk_ids, float* topk_weights,
                            int32_t* sorted_token_ids, int32_t* block_expert_ids, int32_t* expert_offsets,
                            int32_t* num_tokens_post_pad, int64_t cap, const void* w13_packed, const void* w2_packed,
                            uint16_t* out_bf16, void* stream) {
  int st = check_layer(M, E, H, I, top_k);
  if (st != MOE_OK || M == 0) return st;
  const int64_t need = moe::workspace_layout(M, E, H, I, top_k).total;
  if (need > kScratchBytes) return MOE_ERR_SCRATCH;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != MOE_OK) return st;
  return layer_impl(moe::kFmtInt4, logits, x_bf16, M, E, H, I, top_k, block_m, topk_ids, topk_weights,
                    sorted_token_ids, block_expert_ids, expert_offsets, num_tokens_post_pad, cap, w13_packed,
                    w2_packed, ws, need, out_bf16, stream, nullptr);
}

int moe_mxfp4_fc1(const uint16_t* x_bf16, int32_t M, int32_t E, int32_t H, int32_t I, int32_t top_k, int32_t block_m,
              const int32_t* sorted_token_ids, const int32_t* block_expert_ids, const int32_t* num_tokens_post_pad,
              int64_t cap, const void* w13_packed, void* workspace, int64_t workspace_bytes, void* stream) {
  return fc1_impl(moe::kFmtMxfp4, x_bf16, M, E, H, I, top_k, block_m, sorted_token_ids, block_expert_ids,
                  num_tokens_post_pad, cap, w13_packed, workspace, workspace_bytes, stream);
}

int moe_mxfp4_fc2(int32_t M, int32_t E, int32_t H, int32_t I, int32_t top_k, int32_t block_m, const float* topk_weights,
              const int32_t* sorted_token_ids, const int32_t* block_expert_ids, const int32_t* num_tokens_post_pad,
              int64_t cap, const void* w2_packed, void* workspace, int64_t workspace_bytes, uint16_t* out_bf16,
              void* stream) {
  return fc2_impl(moe::kFmtMxfp4, M, E, H, I, top_k, block_m, topk_weights, sorted_token_ids, block_expert_ids,
                  num_tokens_post_pad, cap, w2_packed, workspace, workspace_bytes, out_bf16, stream);
}

int moe_mxfp4_forward(const uint16_t* x_bf16, int32_t M, int32_t E, int32_t H, int32_t I, int32_t top_k, int32_t block_m,
                  const float* topk_weights, const int32_t* sorted_token_ids, const int32_t* block_expert_ids,
                  const int32_t* expert_offsets, const int32_t* num_tokens_post_pad, int64_t cap,
                  const void* w13_packed, const void* w2_packed, void* workspace, int64_t workspace_bytes,
                  uint16_t* out_bf16, void* stream) {
  return forward_impl(moe::kFmtMxfp4, x_bf16, M, E, H, I, top_k, block_m, topk_weights, sorted_token_ids, block_expert_ids,
                      expert_offsets, num_tokens_post_pad, cap, w13_packed, w2_packed, workspace, workspace_bytes,
                      out_bf16, stream);
}

int moe_mxfp4_layer(const float* logits, const uint16_t* x_bf16, int32_t M, int32_t E, int32_t H, int32_t I,
                int32_t top_k, int32_t block_m, int32_t* topk_ids, float* topk_weights, int32_t* sorted_token_ids,
                int32_t* block_expert_ids, int32_t* expert_offsets, int32_t* num_tokens_post_pad, int64_t cap,
                const void* w13_packed, const void* w2_packed, void* workspace, int64_t workspace_bytes,
                uint16_t* out_bf16, void* stream, void* const* stage_events) {
  return layer_impl(moe::kFmtMxfp4, logits, x_bf16, M, E, H, I, top_k, block_m, topk_ids, topk_weights, sorted_token_ids,
                    block_expert_ids, expert_offsets, num_tokens_post_pad, cap, w13_packed, w2_packed, workspace,
                    workspace_bytes, out_bf16, stream, stage_events);
}

}  // extern "C"

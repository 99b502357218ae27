/* Host-side checks of the C ABI, built with AddressSanitizer and
 * UndefinedBehaviorSanitizer on the library's host code (test_abi_sanitize.py).
 *
 * Every call here is rejected by the library's own validation before any HIP
 * call: invalid or extreme sizes, null or misaligned pointers, short caps and
 * workspaces. The sanitizers watch the size arithmetic (signed overflow at
 * the int32/int64 edges) and every host access on those paths. The pointers
 * are a host array that the library never dereferences on a rejected call;
 * it runs on hosts without a GPU only, where a call that wrongly passed
 * validation would return MOE_ERR_HIP instead of its expected code.
 * Exit status: 0 when every check holds, 1 otherwise. */
#include <limits.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "moe_w4a16.h"

static int g_fails = 0;
static int g_checks = 0;

#define CHECK_EQ(expr, want)                                                                       \
  do {                                                                                             \
    const long long got_ = (long long)(expr);                                                      \
    const long long want_ = (long long)(want);                                                     \
    ++g_checks;                                                                                    \
    if (got_ != want_) {                                                                           \
      fprintf(stderr, "FAIL line %d: %s = %lld, want %lld\n", __LINE__, #expr, got_, want_);       \
      ++g_fails;                                                                                   \
    }                                                                                              \
  } while (0)

static unsigned char g_buf[4096] __attribute__((aligned(256)));
#define P ((void*)g_buf)
#define PI ((int32_t*)g_buf)
#define PF ((float*)g_buf)
#define PU16 ((uint16_t*)g_buf)
#define PU8 ((uint8_t*)g_buf)
#define P_ODD4 ((void*)(g_buf + 2))  /* not 4-byte aligned */
#define P_ODD16 ((void*)(g_buf + 8)) /* 4- but not 16-byte aligned */

/* INT4 bytes of one 16 x 128 tile: 1024 bytes of codes, 128 of scales; a
 * pair of tiles covers 32 rows. MXFP4 tiles carry 64 bytes of scales. */
static long long int4_expert_bytes(long long N, long long K) { return (N / 32) * (K / 128) * 2 * (1024 + 128); }
static long long mxfp4_expert_bytes(long long N, long long K) { return (N / 32) * (K / 128) * 2 * (1024 + 64); }

static long long capacity_formula(long long M, long long E, long long k, long long B) {
  const long long mk = M * k;
  const long long touched = mk < E ? mk : E;
  const long long raw = mk + touched * (B - 1);
  return (raw + B - 1) / B * B;
}

static void check_status_strings(void) {
  for (int s = -10; s <= 3; ++s) {
    const char* str = moe_w4a16_status_string(s);
    ++g_checks;
    if (!str || !str[0]) {
      fprintf(stderr, "FAIL: empty status string for %d\n", s);
      ++g_fails;
    }
  }
  CHECK_EQ(strcmp(moe_w4a16_status_string(MOE_OK), "ok"), 0);
  CHECK_EQ(strcmp(moe_w4a16_status_string(12345), "unknown status"), 0);
}

static void check_capacity(void) {
  CHECK_EQ(moe_route_align_capacity(0, 384, 8, 16), 0);
  CHECK_EQ(moe_route_align_capacity(-1, 384, 8, 16), -1);
  CHECK_EQ(moe_route_align_capacity(4, 0, 1, 16), -1);
  CHECK_EQ(moe_route_align_capacity(4, 1025, 8, 16), -1);
  CHECK_EQ(moe_route_align_capacity(4, 384, 0, 16), -1);
  CHECK_EQ(moe_route_align_capacity(4, 384, 17, 16), -1);
  CHECK_EQ(moe_route_align_capacity(4, 8, 9, 16), -1);
  CHECK_EQ(moe_route_align_capacity(4, 384, 8, 8), -1);
  CHECK_EQ(moe_route_align_capacity(4, 384, 8, 256), -1);
  CHECK_EQ(moe_route_align_capacity(4, 384, 8, 96), -1);
  CHECK_EQ(moe_route_align_capacity(INT32_MIN, 384, 8, 16), -1);
  CHECK_EQ(moe_route_align_capacity(4, INT32_MAX, 8, 16), -1);
  CHECK_EQ(moe_route_align_capacity(4, 384, INT32_MAX, 16), -1);
  CHECK_EQ(moe_route_align_capacity(4, 384, 8, INT32_MIN), -1);
  CHECK_EQ(moe_route_align_capacity(4096, 384, 8, 16), capacity_formula(4096, 384, 8, 16));
  CHECK_EQ(moe_route_align_capacity(1, 384, 8, 64), capacity_formula(1, 384, 8, 64));
  CHECK_EQ(moe_route_align_capacity(90, 384, 8, 128), capacity_formula(90, 384, 8, 128));
  /* the largest batch the capacity call accepts: int64 arithmetic throughout */
  CHECK_EQ(moe_route_align_capacity(INT32_MAX, 1024, 16, 64), capacity_formula(INT32_MAX, 1024, 16, 64));
  CHECK_EQ(moe_route_align_capacity(INT32_MAX, 1024, 16, 128), capacity_formula(INT32_MAX, 1024, 16, 128));
}

static void check_packed_bytes(void) {
  const long long pb = moe_w4a16_packed_bytes(384, 4096, 7168, 32);
  CHECK_EQ(pb, 384LL * int4_expert_bytes(4096, 7168) + 384LL * 4096);
  CHECK_EQ(moe_mxfp4_packed_bytes(384, 4096, 7168), 384LL * mxfp4_expert_bytes(4096, 7168));
  CHECK_EQ(moe_w4a16_packed_bytes(0, 4096, 7168, 32), -1);
  CHECK_EQ(moe_w4a16_packed_bytes(384, 4096, 7168, 16), -1);
  CHECK_EQ(moe_w4a16_packed_bytes(384, 48, 7168, 32), -1);
  CHECK_EQ(moe_w4a16_packed_bytes(384, 4096, 7000, 32), -1);
  CHECK_EQ(moe_w4a16_packed_bytes(-384, 4096, 7168, 32), -1);
  CHECK_EQ(moe_w4a16_packed_bytes(1025, 4096, 7168, 32), -1);
  /* extreme sizes: rejected, never wrapped */
  CHECK_EQ(moe_w4a16_packed_bytes(INT32_MAX, 4096, 7168, 32), -1);
  CHECK_EQ(moe_w4a16_packed_bytes(1, INT32_MAX - 31, INT32_MAX - 127, 32), -1);
  CHECK_EQ(moe_w4a16_packed_bytes(1024, INT32_MAX - 31, 128, 32), -1);
  CHECK_EQ(moe_mxfp4_packed_bytes(INT32_MAX, INT32_MAX - 31, INT32_MAX - 127), -1);
  CHECK_EQ(moe_mxfp4_packed_bytes(1025, 4096, 7168), -1);
  /* the per-expert limit's edge: 32 rows, K/128 tile pairs of 2304 bytes < 2^31 */
  const long long kmax = ((1LL << 31) - 1) / 2304 * 128;
  CHECK_EQ(moe_w4a16_packed_bytes(1, 32, (int32_t)kmax, 32), int4_expert_bytes(32, kmax) + 32);
  CHECK_EQ(moe_w4a16_packed_bytes(1, 32, (int32_t)(kmax + 128), 32), -1);
  CHECK_EQ(moe_w4a16_packed_bytes(1024, 32, (int32_t)kmax, 32), 1024LL * (int4_expert_bytes(32, kmax) + 32));
}

static void check_repack(void) {
  CHECK_EQ(moe_w4a16_repack(PU8, PU16, 2, 64, 128, 32, 2, P, NULL), MOE_ERR_INVALID_ARG);
  CHECK_EQ(moe_w4a16_repack(PU8, PU16, 2, 64, 128, 32, -1, P, NULL), MOE_ERR_INVALID_ARG);
  CHECK_EQ(moe_w4a16_repack(PU8, PU16, 2, 48, 128, 32, 1, P, NULL), MOE_ERR_UNSUPPORTED);
  CHECK_EQ(moe_w4a16_repack(PU8, PU16, 2, 64, 96, 32, 1, P, NULL), MOE_ERR_UNSUPPORTED);
  CHECK_EQ(moe_w4a16_repack(PU8, PU16, 2, 64, 128, 16, 1, P, NULL), MOE_ERR_UNSUPPORTED);
  CHECK_EQ(moe_w4a16_repack(NULL, PU16, 2, 64, 128, 32, 1, P, NULL), MOE_ERR_INVALID_ARG);
  CHECK_EQ(moe_w4a16_repack(PU8 + 8, PU16, 2, 64, 128, 32, 1, P, NULL), MOE_ERR_INVALID_ARG);
  CHECK_EQ(moe_w4a16_repack(PU8, PU16, 2, 64, 128, 32, 1, P_ODD16, NULL), MOE_ERR_INVALID_ARG);
  CHECK_EQ(moe_w4a16_repack(PU8, PU16, 0, 64, 128, 32, 1, P, NULL), MOE_ERR_INVALID_ARG);
  CHECK_EQ(moe_w4a16_repack(PU8, PU16, INT32_MIN, 64, 128, 32, 1, P, NULL), MOE_ERR_INVALID_ARG);
  CHECK_EQ(moe_w4a16_repack(PU8, PU16, INT32_MAX, INT32_MAX - 31, INT32_MAX - 127, 32, 1, P, NULL),
           MOE_ERR_UNSUPPORTED);
  CHECK_EQ(moe_w4a16_repack(PU8, PU16, 1025, 64, 128, 32, 1, P, NULL), MOE_ERR_UNSUPPORTED);
  CHECK_EQ(moe_w4a16_unpack(P, 2, 64, 128, 32, 0, NULL, PU16, NULL), MOE_ERR_INVALID_ARG);
  CHECK_EQ(moe_w4a16_unpack(P, 2, INT32_MAX - 31, INT32_MAX - 127, 32, 1, PU8, PU16, NULL), MOE_ERR_UNSUPPORTED);
  CHECK_EQ(moe_mxfp4_repack(PU8, PU8, 2, 64, 128, 2, P, NULL), MOE_ERR_INVALID_ARG);
  CHECK_EQ(moe_mxfp4_repack(PU8, PU8, 2, 48, 128, 1, P, NULL), MOE_ERR_UNSUPPORTED);
  CHECK_EQ(moe_mxfp4_repack(PU8, NULL, 2, 64, 128, 1, P, NULL), MOE_ERR_INVALID_ARG);
  CHECK_EQ(moe_mxfp4_repack(PU8, PU8 + 4, 2, 64, 128, 1, P, NULL), MOE_ERR_INVALID_ARG);
  CHECK_EQ(moe_mxfp4_repack(PU8, PU8, INT32_MAX, INT32_MAX - 31, INT32_MAX - 127, 1, P, NULL), MOE_ERR_UNSUPPORTED);
  CHECK_EQ(moe_mxfp4_unpack(P, 2, 64, 128, 0, NULL, PU8, NULL), MOE_ERR_INVALID_ARG);
  CHECK_EQ(moe_mxfp4_unpack(P, 2, 64, 128, 0, PU8, PU8 + 1, NULL), MOE_ERR_INVALID_ARG);
}

static void check_workspace_and_block_m(void) {
  CHECK_EQ(moe_w4a16_workspace_bytes(-1, 384, 7168, 2048, 8), -1);
  CHECK_EQ(moe_w4a16_workspace_bytes(4, 384, 7000, 2048, 8), -1);
  CHECK_EQ(moe_w4a16_workspace_bytes(4, 384, 7168, 2000, 8), -1);
  CHECK_EQ(moe_w4a16_workspace_bytes(1 << 20, 384, 7168, 2048, 8), -1); /* M*k*max(H, I) >= 2^31 */
  CHECK_EQ(moe_w4a16_workspace_bytes(INT32_MAX, 1024, 7168, 2048, 16), -1);
  CHECK_EQ(moe_w4a16_workspace_bytes(1, 1, INT32_MAX - 127, INT32_MAX - 127, 1), -1);
  CHECK_EQ(moe_w4a16_workspace_bytes(1, 1, 128, (1 << 30) + 128, 1), -1); /* 2*I past int32 */
  CHECK_EQ(moe_w4a16_workspace_bytes(1, 1, 1 << 20, 1 << 12, 1), -1);      /* one expert >= 2^31 bytes */
  CHECK_EQ(moe_w4a16_workspace_bytes(1, 1, 1 << 19, 1 << 10, 1) > 0, 1);
  CHECK_EQ(moe_w4a16_workspace_bytes(0, 384, 7168, 2048, 8) >= 0, 1);
  CHECK_EQ(moe_w4a16_workspace_bytes(4096, 384, 7168, 2048, 8) > 0, 1);
  CHECK_EQ(moe_w4a16_preferred_block_m(1, 384, 7168, 2048, 8), 16);
  CHECK_EQ(moe_w4a16_preferred_block_m(4096, 384, 7168, 2048, 8), 32);
  CHECK_EQ(moe_w4a16_preferred_block_m(4, 384, 7000, 2048, 8), -1);
  CHECK_EQ(moe_w4a16_preferred_block_m(INT32_MAX, 1024, 128, 128, 16), -1);
}

static void check_route_align(void) {
  const int64_t cap = moe_route_align_capacity(4, 384, 8, 16);
  CHECK_EQ(moe_route_align(NULL, 0, 384, 8, 16, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL), MOE_OK);
  CHECK_EQ(moe_route_align(PF, -1, 384, 8, 16, PI, PF, PI, PI, PI, PI, cap, NULL), MOE_ERR_INVALID_ARG);
  CHECK_EQ(moe_route_align(PF, 4, 1025, 8, 16, PI, PF, PI, PI, PI, PI, cap, NULL), MOE_ERR_UNSUPPORTED);
  CHECK_EQ(moe_route_align(PF, 4, 64, 17, 16, PI, PF, PI, PI, PI, PI, cap, NULL), MOE_ERR_UNSUPPORTED);
  CHECK_EQ(moe_route_align(PF, 4, 384, 8, 8, PI, PF, PI, PI, PI, PI, cap, NULL), MOE_ERR_UNSUPPORTED);
  CHECK_EQ(moe_route_align(PF, INT32_MAX, 1024, 16, 16, PI, PF, PI, PI, PI, PI, INT64_MAX, NULL),
           MOE_ERR_UNSUPPORTED);
  CHECK_EQ(moe_route_align(NULL, 4, 384, 8, 16, PI, PF, PI, PI, PI, PI, cap, NULL), MOE_ERR_INVALID_ARG);
  CHECK_EQ(moe_route_align(PF, 4, 384, 8, 16, PI, PF, PI, PI, PI, NULL, cap, NULL), MOE_ERR_INVALID_ARG);
  CHECK_EQ(moe_route_align((float*)P_ODD4, 4, 384, 8, 16, PI, PF, PI, PI, PI, PI, cap, NULL), MOE_ERR_INVALID_ARG);
  CHECK_EQ(moe_route_align(PF, 4, 384, 8, 16, PI, PF, PI, PI, PI, PI, cap - 16, NULL), MOE_ERR_CAPACITY);
  CHECK_EQ(moe_route_align(PF, 4, 384, 8, 16, PI, PF, PI, PI, PI, PI, cap + 1, NULL), MOE_ERR_CAPACITY);
  CHECK_EQ(moe_route_align(PF, 4, 384, 8, 16, PI, PF, PI, PI, PI, PI, INT64_MIN, NULL), MOE_ERR_CAPACITY);
}

typedef int (*fc1_fn)(const uint16_t*, int32_t, int32_t, int32_t, int32_t, int32_t, int32_t, const int32_t*,
                      const int32_t*, const int32_t*, int64_t, const void*, void*, int64_t, void*);
typedef int (*fc2_fn)(int32_t, int32_t, int32_t, int32_t, int32_t, int32_t, const float*, const int32_t*,
                      const int32_t*, const int32_t*, int64_t, const void*, void*, int64_t, uint16_t*, void*);
typedef int (*fwd_fn)(const uint16_t*, int32_t, int32_t, int32_t, int32_t, int32_t, int32_t, const float*,
                      const int32_t*, const int32_t*, const int32_t*, const int32_t*, int64_t, const void*,
                      const void*, void*, int64_t, uint16_t*, void*);
typedef int (*layer_fn)(const float*, const uint16_t*, int32_t, int32_t, int32_t, int32_t, int32_t, int32_t,
                        int32_t*, float*, int32_t*, int32_t*, int32_t*, int32_t*, int64_t, const void*, const void*,
                        void*, int64_t, uint16_t*, void*, void* const*);

/* The stage, forward and layer calls of one weight format. */
static void check_stages(fc1_fn fc1, fc2_fn fc2, fwd_fn fwd, layer_fn layer) {
  const int32_t M = 4, E = 384, H = 7168, I = 2048, k = 8, B = 16;
  const int64_t cap = moe_route_align_capacity(M, E, k, B);
  const int64_t ws = moe_w4a16_workspace_bytes(M, E, H, I, k);
  CHECK_EQ(fc1(PU16, M, E, H, I, k, B, PI, PI, PI, cap, P, P, ws - 16, NULL), MOE_ERR_WORKSPACE);
  CHECK_EQ(fc1(PU16, M, E, H, I, k, B, PI, PI, PI, cap - 16, P, P, ws, NULL), MOE_ERR_CAPACITY);
  CHECK_EQ(fc1(NULL, M, E, H, I, k, B, PI, PI, PI, cap, P, P, ws, NULL), MOE_ERR_INVALID_ARG);
  CHECK_EQ(fc1((uint16_t*)P_ODD16, M, E, H, I, k, B, PI, PI, PI, cap, P, P, ws, NULL), MOE_ERR_INVALID_ARG);
  CHECK_EQ(fc1(PU16, M, E, H, I, k, 256, PI, PI, PI, cap, P, P, ws, NULL), MOE_ERR_UNSUPPORTED);
  /* 128 passes the block_m check; the cap for 16-row blocks is too small for it */
  CHECK_EQ(fc1(PU16, M, E, H, I, k, 128, PI, PI, PI, cap, P, P, ws, NULL), MOE_ERR_CAPACITY);
  CHECK_EQ(fc1(NULL, 0, E, H, I, k, B, NULL, NULL, NULL, 0, NULL, NULL, 0, NULL), MOE_OK);
  CHECK_EQ(fc2(M, E, H, I, k, B, PF, PI, PI, PI, cap, P, P, ws, NULL, NULL), MOE_ERR_INVALID_ARG);
  CHECK_EQ(fc2(M, E, H, I, k, B, PF, PI, PI, PI, cap, P, P, ws, (uint16_t*)P_ODD16, NULL), MOE_ERR_INVALID_ARG);
  CHECK_EQ(fc2(M, E, H, I, k, B, PF, PI, PI, PI, cap, P, P, ws - 1, PU16, NULL), MOE_ERR_WORKSPACE);
  CHECK_EQ(fc2(M, E, H, 7000, k, B, PF, PI, PI, PI, cap, P, P, ws, PU16, NULL), MOE_ERR_UNSUPPORTED);
  CHECK_EQ(fwd(PU16, M, E, H, I, k, B, PF, PI, PI, PI, PI, cap, P, P, P, ws, (uint16_t*)P_ODD16, NULL),
           MOE_ERR_INVALID_ARG);
  CHECK_EQ(fwd(PU16, M, E, H, I, 0, B, PF, PI, PI, PI, PI, cap, P, P, P, ws, PU16, NULL), MOE_ERR_INVALID_ARG);
  CHECK_EQ(fwd(PU16, 1 << 20, E, H, I, k, B, PF, PI, PI, PI, PI, cap, P, P, P, ws, PU16, NULL),
           MOE_ERR_UNSUPPORTED);
  CHECK_EQ(fwd(PU16, INT32_MAX, 1024, 128, 128, 16, 64, PF, PI, PI, PI, PI, INT64_MAX, P, P, P, INT64_MAX, PU16,
               NULL),
           MOE_ERR_UNSUPPORTED);
  CHECK_EQ(fwd(PU16, M, E, H, I, k, B, PF, PI, PI, PI, PI, cap, P, NULL, P, ws, PU16, NULL), MOE_ERR_INVALID_ARG);
  CHECK_EQ(fwd(PU16, M, E, H, I, k, B, PF, PI, PI, PI, PI, INT64_MIN, P, P, P, ws, PU16, NULL), MOE_ERR_CAPACITY);
  CHECK_EQ(fwd(PU16, M, E, H, I, k, B, PF, PI, PI, PI, PI, cap, P, P, P, INT64_MIN, PU16, NULL), MOE_ERR_WORKSPACE);
  CHECK_EQ(layer(NULL, NULL, 0, E, H, I, k, B, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL, NULL, NULL, 0, NULL,
                 NULL, NULL),
           MOE_OK);
  CHECK_EQ(layer(PF, PU16, M, E, 7000, I, k, B, PI, PF, PI, PI, PI, PI, cap, P, P, P, ws, PU16, NULL, NULL),
           MOE_ERR_UNSUPPORTED);
  CHECK_EQ(layer(PF, PU16, M, E, H, I, k, B, PI, PF, PI, PI, PI, PI, cap - 16, P, P, P, ws, PU16, NULL, NULL),
           MOE_ERR_CAPACITY);
  CHECK_EQ(layer(PF, PU16, M, E, H, I, k, B, PI, PF, PI, PI, PI, PI, cap, P, P, P, ws - 1, PU16, NULL, NULL),
           MOE_ERR_WORKSPACE);
  CHECK_EQ(layer(NULL, PU16, M, E, H, I, k, B, PI, PF, PI, PI, PI, PI, cap, P, P, P, ws, PU16, NULL, NULL),
           MOE_ERR_INVALID_ARG);
  CHECK_EQ(layer(PF, (uint16_t*)P_ODD16, M, E, H, I, k, B, PI, PF, PI, PI, PI, PI, cap, P, P, P, ws, PU16, NULL,
                 NULL),
           MOE_ERR_INVALID_ARG);
  CHECK_EQ(layer(PF, PU16, M, 1025, H, I, k, B, PI, PF, PI, PI, PI, PI, cap, P, P, P, ws, PU16, NULL, NULL),
           MOE_ERR_UNSUPPORTED);
}

/* The no-allocation layer call: rejected sizes, and a batch past its scratch
 * (refused before the scratch address is looked up). */
static void check_noalloc(void) {
  const int64_t cap = moe_route_align_capacity(4, 384, 8, 16);
  CHECK_EQ(moe_w4a16_layer_noalloc(NULL, NULL, 0, 384, 7168, 2048, 8, 16, NULL, NULL, NULL, NULL, NULL, NULL, 0,
                                   NULL, NULL, NULL, NULL),
           MOE_OK);
  CHECK_EQ(moe_w4a16_layer_noalloc(PF, PU16, 4, 384, 7000, 2048, 8, 16, PI, PF, PI, PI, PI, PI, cap, P, P, PU16,
                                   NULL),
           MOE_ERR_UNSUPPORTED);
  CHECK_EQ(moe_w4a16_layer_noalloc(PF, PU16, -4, 384, 7168, 2048, 8, 16, PI, PF, PI, PI, PI, PI, cap, P, P, PU16,
                                   NULL),
           MOE_ERR_INVALID_ARG);
  const int64_t big = moe_route_align_capacity(32768, 384, 8, 16);
  CHECK_EQ(moe_w4a16_layer_noalloc(PF, PU16, 32768, 384, 7168, 2048, 8, 16, PI, PF, PI, PI, PI, PI, big, P, P, PU16,
                                   NULL),
           MOE_ERR_SCRATCH);
}

static void check_calib(void) {
  const int64_t g = moe_calib_read_granule();
  CHECK_EQ(g, 32768);
  uint32_t* sink = (uint32_t*)PI;
  CHECK_EQ(moe_calib_hbm_read(NULL, g, 1, sink, NULL), MOE_ERR_INVALID_ARG);
  CHECK_EQ(moe_calib_hbm_read(P, g, 1, NULL, NULL), MOE_ERR_INVALID_ARG);
  CHECK_EQ(moe_calib_hbm_read(P, 0, 1, sink, NULL), MOE_ERR_INVALID_ARG);
  CHECK_EQ(moe_calib_hbm_read(P, INT64_MIN, 1, sink, NULL), MOE_ERR_INVALID_ARG);
  CHECK_EQ(moe_calib_hbm_read(P, g - 16, 1, sink, NULL), MOE_ERR_INVALID_ARG);
  CHECK_EQ(moe_calib_hbm_read(P, INT64_MAX, 1, sink, NULL), MOE_ERR_INVALID_ARG);
  CHECK_EQ(moe_calib_hbm_read(P, g, 0, sink, NULL), MOE_ERR_INVALID_ARG);
  CHECK_EQ(moe_calib_hbm_read(P, g, INT32_MIN, sink, NULL), MOE_ERR_INVALID_ARG);
  CHECK_EQ(moe_calib_hbm_read(P, g, INT32_MAX, sink, NULL), MOE_ERR_INVALID_ARG);
  CHECK_EQ(moe_calib_hbm_read(PU8 + 8, g, 1, sink, NULL), MOE_ERR_INVALID_ARG);
  CHECK_EQ(moe_calib_mfma_f16(1, 1, NULL, NULL), MOE_ERR_INVALID_ARG);
  CHECK_EQ(moe_calib_mfma_f16(INT64_MIN, 1, (float*)PF, NULL), MOE_ERR_INVALID_ARG);
  CHECK_EQ(moe_calib_mfma_f16(1, 0, (float*)PF, NULL), MOE_ERR_INVALID_ARG);
  CHECK_EQ(moe_calib_mfma_f16(1, INT32_MAX, (float*)PF, NULL), MOE_ERR_INVALID_ARG);
}

int main(void) {
  CHECK_EQ(moe_w4a16_abi_version(), 3);
  check_status_strings();
  check_capacity();
  check_packed_bytes();
  check_repack();
  check_workspace_and_block_m();
  check_route_align();
  check_stages(moe_w4a16_fc1, moe_w4a16_fc2, moe_w4a16_forward, moe_w4a16_layer);
  check_stages(moe_mxfp4_fc1, moe_mxfp4_fc2, moe_mxfp4_forward, moe_mxfp4_layer);
  check_noalloc();
  check_calib();
  if (g_fails) {
    fprintf(stderr, "%d of %d checks failed\n", g_fails, g_checks);
    return 1;
  }
  printf("abi checks: %d passed\n", g_checks);
  return 0;
}

// Canonical INT4 or MXFP4 weights <-> the gfx950 tile layout the GEMM
// kernels stream.
//
// "The Throughput Lever: Quantifying the MoE GEMM and Mapping the Road to
// B300", section "Building the Benchmark", converts GPTQ-format INT4 weights
// once into the layout its kernel reads. This is the same one-time step for
// the layout of internal.h: per 16-row x 128-channel tile, lane L of a wave
// reads 16 bytes at offset 16*L; those hold, for row L % 16, the 8 channels
// 32*j + 8*(L/16) .. +7 of group j (j = 0..3) in dword j, code 2p in bits
// [4p, 4p+4) and code 2p+1 in bits [16+4p, 20+4p) so that one AND/OR per pair
// turns two codes into two bf16 values. The 128 bytes of scales that follow
// hold row r's 4 group scales at offset 8*r.
// MXFP4 (FP4 e2m1 codes, E8M0 scales): the same tiles with the codes in
// canonical byte order (gfx950's FP4 conversion takes a byte's low nibble
// first) and 64 bytes of scales, row r's 4 bytes at offset 4*r.
// An INT4 blob ends with one int8 exponent shift per weight row (internal.h,
// sigma_trailer_bytes), written here from the scales.
#include "internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

// Canonical row of row r (0..15) of tile h (0/1) of pair p.
__device__ __forceinline__ int64_t canon_row(int kind, int N, int p, int h, int r) {
  if (kind == 0) return (h == 0 ? 0 : N / 2) + 16 * p + r;  // W13: gate tile, up tile
  return 32 * p + 16 * h + r;                                 // W2: two halves of 32 rows
}

// Four canonical bytes (channels c0 .. c0+7, low nibble first) -> one device dword.
__device__ __forceinline__ uint32_t to_device_dword(uint32_t x) {
  uint32_t out = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    out |= ((x >> (8 * b)) & 0xFu) << (4 * b);
    out |= ((x >> (8 * b + 4)) & 0xFu) << (16 + 4 * b);
  }
  return out;
}
__device__ __forceinline__ uint32_t to_canonical_dword(uint32_t d) {
  uint32_t out = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    out |= ((d >> (4 * b)) & 0xFu) << (8 * b);
    out |= ((d >> (16 + 4 * b)) & 0xFu) << (8 * b + 4);
  }
  return out;
}

struct TileIndex {
  int64_t e, n, c0, dev_off;
  int L;
};

// Thread -> (expert, tile, lane): one thread per 16 device bytes of nibbles.
__device__ __forceinline__ bool tile_index(int fmt, int64_t gid, int E, int N, int K, int kind, TileIndex& ti,
                                           int64_t& canon_byte_row) {
  const int64_t nkc = K / kChunkK, npair = N / kPairRows;
  const int64_t per_expert = npair * nkc * 2 * 64;
  if (gid >= (int64_t)E * per_expert) return false;
  ti.e = gid / per_expert;
  int64_t rem = gid % per_expert;
  ti.L = (int)(rem % 64);
  const int64_t tile = rem / 64;  // (p * nkc + kc) * 2 + h
  const int h = (int)(tile % 2);
  const int64_t kc = (tile / 2) % nkc;
  const int p = (int)(tile / 2 / nkc);
  const int r = ti.L % 16, sb = ti.L / 16;
  ti.n = canon_row(kind, N, p, h, r);
  ti.c0 = kc * kChunkK + 8 * sb;  // channel of group j is c0 + 32*j
  ti.dev_off = ti.e * packed_bytes_fmt(fmt, N, K) + tile * (kTileNibbleBytes + tile_scale_bytes(fmt));
  canon_byte_row = (ti.e * N + ti.n) * (K / 2);
  return true;
}

__global__ __launch_bounds__(kThreads) void repack_kernel(int fmt, const uint8_t* __restrict__ q,
                                                          const void* __restrict__ s, int E, int N, int K,
                                                          int kind, uint8_t* __restrict__ packed) {
  const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  TileIndex ti;
  int64_t row;
  if (!tile_index(fmt, gid, E, N, K, kind, ti, row)) return;
  uint32_t d[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t x = *reinterpret_cast<const uint32_t*>(q + row + (ti.c0 + 32 * j) / 2);
    d[j] = fmt == kFmtMxfp4 ? x : to_device_dword(x);
  }
  *reinterpret_cast<uint4*>(packed + ti.dev_off + 16 * ti.L) = make_uint4(d[0], d[1], d[2], d[3]);
  if (ti.L < 16) {  // this lane also moves the 4 group scales of row ti.n
    const int64_t g0 = (ti.c0 - 8 * (ti.L / 16)) / kGroup;
    const int64_t srow = (ti.e * N + ti.n) * (K / kGroup) + g0;
    if (fmt == kFmtMxfp4)
      *reinterpret_cast<uint32_t*>(packed + ti.dev_off + kTileNibbleBytes + 4 * (ti.L % 16)) =
          *reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(s) + srow);
    else
      *reinterpret_cast<uint2*>(packed + ti.dev_off + kTileNibbleBytes + 8 * (ti.L % 16)) =
          *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(s) + srow);
  }
}

__global__ __launch_bounds__(kThreads) void unpack_kernel(int fmt, const uint8_t* __restrict__ packed, int E,
                                                          int N, int K, int kind, uint8_t* __restrict__ q,
                                                          void* __restrict__ s) {
  const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  TileIndex ti;
  int64_t row;
  if (!tile_index(fmt, gid, E, N, K, kind, ti, row)) return;
  const uint4 v = *reinterpret_cast<const uint4*>(packed + ti.dev_off + 16 * ti.L);
  const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int j = 0; j < 4; ++j)
    *reinterpret_cast<uint32_t*>(q + row + (ti.c0 + 32 * j) / 2) = fmt == kFmtMxfp4 ? d[j] : to_canonical_dword(d[j]);
  if (ti.L < 16) {
    const int64_t g0 = (ti.c0 - 8 * (ti.L / 16)) / kGroup;
    const int64_t srow = (ti.e * N + ti.n) * (K / kGroup) + g0;
    if (fmt == kFmtMxfp4)
      *reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(s) + srow) =
          *reinterpret_cast<const uint32_t*>(packed + ti.dev_off + kTileNibbleBytes + 4 * (ti.L % 16));
    else
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(s) + srow) =
          *reinterpret_cast<const uint2*>(packed + ti.dev_off + kTileNibbleBytes + 8 * (ti.L % 16));
  }
}

int64_t grid_for(int E, int N, int K) {
  const int64_t threads = (int64_t)E * (N / kPairRows) * (K / kChunkK) * 2 * 64;
  return (threads + kThreads - 1) / kThreads;
}

}  // namespace

hipError_t launch_repack(int fmt, const uint8_t* q, const void* s, int E, int N, int K, int kind,
                         uint8_t* packed, hipStream_t stream) {
  const int64_t blocks = grid_for(E, N, K);
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  repack_kernel<<<(unsigned)blocks, kThreads, 0, stream>>>(fmt, q, s, E, N, K, kind, packed);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || fmt != kFmtInt4) return err;
  // the per-row exponent shifts after the tiles (sigma_trailer_bytes)
  return launch_row_sigma(static_cast<const uint16_t*>(s), E, N, K,
                          reinterpret_cast<int8_t*>(packed + (int64_t)E * packed_bytes_fmt(fmt, N, K)), stream);
}

hipError_t launch_unpack(int fmt, const uint8_t* packed, int E, int N, int K, int kind, uint8_t* q, void* s,
                         hipStream_t stream) {
  const int64_t blocks = grid_for(E, N, K);
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  unpack_kernel<<<(unsigned)blocks, kThreads, 0, stream>>>(fmt, packed, E, N, K, kind, q, s);
  return hipGetLastError();
}

}  // namespace moe

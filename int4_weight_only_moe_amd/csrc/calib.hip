// Measurement helpers: what this GPU sustains, measured with plain kernels,
// so that a layer kernel's rate can be stated as a fraction of the attainable
// rate as well as of the published peaks. Not part of the layer.
//
//   calib_read_kernel  streams a buffer once with non-temporal 16-byte loads
//                      (the way the layer kernels stream their weights), each
//                      load instruction covering 4 KB contiguous per
//                      workgroup, 8 loads in flight per thread; the words are
//                      XOR-folded so that every load is used.
//   calib_mfma_kernel  back-to-back v_mfma_f32_16x16x32_f16 on register
//                      operands (the instruction the large-batch FC kernels
//                      issue), 8 independent accumulators per wave; the
//                      operands are fp16 values with full mantissas, since
//                      the matrix core's power, and so the clock it runs at
//                      under load, depends on the data.
#include "../../include/moe_w4a16.h"
#include "device_common.h"

namespace {

using moe::f32x4_t;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

constexpr int kCalibThreads = 256;
constexpr int kReadUnroll = 8;
constexpr int64_t kReadGranule = (int64_t)kCalibThreads * kReadUnroll * 16;  // bytes per block step
constexpr int kMfmaAcc = 8;
constexpr int32_t kMaxCalibWorkgroups = 1 << 20;

__global__ __launch_bounds__(kCalibThreads) void calib_read_kernel(const u32x4_t* __restrict__ src, int64_t nblk,
                                                                   uint32_t* __restrict__ sink) {
  u32x4_t acc = {0u, 0u, 0u, 0u};
  for (int64_t b = blockIdx.x; b < nblk; b += gridDim.x) {
    const u32x4_t* p = src + b * (kCalibThreads * kReadUnroll) + threadIdx.x;
    u32x4_t v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = __builtin_nontemporal_load(p + u * kCalibThreads);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u];
  }
  sink[(int64_t)blockIdx.x * kCalibThreads + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

// The fp16 operand value of (lane, element i, operand s): magnitude in
// [0.5, 1) with a hashed 10-bit mantissa and sign. The host computes the same
// values to check the kernel's sums.
__device__ __forceinline__ _Float16 calib_operand(uint32_t lane, uint32_t i, uint32_t s) {
  uint32_t h = lane * 0x9E3779B1u ^ (i + 8u * s) * 0x85EBCA77u;
  h ^= h >> 15;
  h *= 0x2C1B3C6Du;
  h ^= h >> 12;
  const uint16_t bits = (uint16_t)(((h >> 16) & 0x8000u) | 0x3800u | (h & 0x3FFu));
  return __builtin_bit_cast(_Float16, bits);
}

// The VGPR budget keeps the accumulators in ordinary VGPRs: with accumulation
// registers the allocator moved half of them every iteration.
__global__ __launch_bounds__(kCalibThreads) __attribute__((amdgpu_num_vgpr(64))) void calib_mfma_kernel(
    int64_t iters, float* __restrict__ sink) {
  const uint32_t lane = threadIdx.x & 63u;
  f16x8_t a[2], b[4];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int s = 0; s < 2; ++s) a[s][i] = calib_operand(lane, i, s);
#pragma unroll
    for (int s = 0; s < 4; ++s) b[s][i] = calib_operand(lane, i, 2 + s);
  }
  // accumulator 2j + i takes A operand i and B operand j
  f32x4_t c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0, c2 = c0, c3 = c0, c4 = c0, c5 = c0, c6 = c0, c7 = c0;
  for (int64_t it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[0], b[0], c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[1], b[0], c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[0], b[1], c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[1], b[1], c3, 0, 0, 0);
    c4 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[0], b[2], c4, 0, 0, 0);
    c5 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[1], b[2], c5, 0, 0, 0);
    c6 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[0], b[3], c6, 0, 0, 0);
    c7 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[1], b[3], c7, 0, 0, 0);
  }
  const f32x4_t acc[kMfmaAcc] = {c0, c1, c2, c3, c4, c5, c6, c7};
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kMfmaAcc; ++j) s += (acc[j][0] + acc[j][1]) + (acc[j][2] + acc[j][3]);
  sink[(int64_t)blockIdx.x * kCalibThreads + threadIdx.x] = s;
}

}  // namespace

extern "C" {

int64_t moe_calib_read_granule(void) { return kReadGranule; }

int moe_calib_hbm_read(const void* buf, int64_t bytes, int32_t workgroups, uint32_t* sink, void* stream) {
  if (buf == nullptr || sink == nullptr || bytes <= 0 || workgroups <= 0) return MOE_ERR_INVALID_ARG;
  if (bytes % kReadGranule != 0 || workgroups > kMaxCalibWorkgroups) return MOE_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(buf) & 15u) != 0 || (reinterpret_cast<uintptr_t>(sink) & 3u) != 0)
    return MOE_ERR_INVALID_ARG;
  hipLaunchKernelGGL(calib_read_kernel, dim3((unsigned)workgroups), dim3(kCalibThreads), 0, (hipStream_t)stream,
                     (const u32x4_t*)buf, bytes / kReadGranule, sink);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int moe_calib_mfma_f16(int64_t iters, int32_t workgroups, float* sink, void* stream) {
  if (sink == nullptr || iters < 0 || workgroups <= 0 || workgroups > kMaxCalibWorkgroups)
    return MOE_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(sink) & 3u) != 0) return MOE_ERR_INVALID_ARG;
  hipLaunchKernelGGL(calib_mfma_kernel, dim3((unsigned)workgroups), dim3(kCalibThreads), 0, (hipStream_t)stream,
                     iters, sink);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // extern "C"

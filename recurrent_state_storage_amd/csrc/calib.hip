// Bandwidth calibration kernels: the achievable HBM read, write and copy rates
// of this GPU, measured with the access pattern the decode kernels use (16-byte
// non-temporal loads and stores, fully coalesced). The decode path never calls
// them; a benchmark times them beside the decode kernels so that a kernel's
// bandwidth can be read against what the memory system delivers, not only
// against the data-sheet peak.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/rss_calib.h"
#include "device.h"

namespace rss {

constexpr int kCalibThreads = 256;
constexpr int kCalibUnroll = 4;   // 16-byte loads in flight per thread and round

__global__ __launch_bounds__(kCalibThreads) void calib_read_kernel(const f32x4* src, size_t n,
                                                                   float* sink) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const size_t stride = (size_t)gridDim.x * kCalibThreads * kCalibUnroll;
  for (size_t i = (size_t)blockIdx.x * kCalibThreads * kCalibUnroll + threadIdx.x; i < n; i += stride) {
    f32x4 v[kCalibUnroll];
#pragma unroll
    for (int u = 0; u < kCalibUnroll; ++u) {
      const size_t k = i + (size_t)u * kCalibThreads;
      v[u] = k < n ? __builtin_nontemporal_load(src + k) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < kCalibUnroll; ++u) acc += v[u];
  }
  // The sum is stored only if it equals a value the inputs are not expected to
  // produce, so the loads cannot be removed and (almost) nothing is written.
  const float s = acc.x + acc.y + acc.z + acc.w;
  if (s == -1234.5f) sink[0] = s;
}

__global__ __launch_bounds__(kCalibThreads) void calib_copy_kernel(const f32x4* src, f32x4* dst,
                                                                   size_t n) {
  const size_t stride = (size_t)gridDim.x * kCalibThreads * kCalibUnroll;
  for (size_t i = (size_t)blockIdx.x * kCalibThreads * kCalibUnroll + threadIdx.x; i < n; i += stride) {
    f32x4 v[kCalibUnroll];
#pragma unroll
    for (int u = 0; u < kCalibUnroll; ++u) {
      const size_t k = i + (size_t)u * kCalibThreads;
      if (k < n) v[u] = __builtin_nontemporal_load(src + k);
    }
#pragma unroll
    for (int u = 0; u < kCalibUnroll; ++u) {
      const size_t k = i + (size_t)u * kCalibThreads;
      if (k < n) __builtin_nontemporal_store(v[u], dst + k);
    }
  }
}

// Writes `n` 16-byte vectors of a fixed pattern (the value of each float is
// its vector index modulo 2^24 in the first lane, then 1, 2, 3), so a caller
// can check what was written.
__global__ __launch_bounds__(kCalibThreads) void calib_write_kernel(f32x4* dst, size_t n) {
  const size_t stride = (size_t)gridDim.x * kCalibThreads * kCalibUnroll;
  for (size_t i = (size_t)blockIdx.x * kCalibThreads * kCalibUnroll + threadIdx.x; i < n; i += stride) {
#pragma unroll
    for (int u = 0; u < kCalibUnroll; ++u) {
      const size_t k = i + (size_t)u * kCalibThreads;
      if (k < n) __builtin_nontemporal_store(f32x4{(float)(k & 0xffffffu), 1.f, 2.f, 3.f}, dst + k);
    }
  }
}

}  // namespace rss

namespace {
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
unsigned grid_of(int32_t blocks) { return blocks > 0 ? (unsigned)blocks : 4096u; }
}  // namespace

extern "C" {

int32_t rss_calib_read(const void* src, size_t bytes, float* sink, int32_t blocks, void* stream) {
  if (!src || !sink || !aligned16(src) || bytes % 16 || blocks < 0) return RSS_E_INVALID;
  if (bytes == 0) return RSS_OK;
  hipLaunchKernelGGL(rss::calib_read_kernel, dim3(grid_of(blocks)), dim3(rss::kCalibThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const rss::f32x4*>(src), bytes / 16,
                     sink);
  return hipGetLastError() == hipSuccess ? RSS_OK : RSS_E_HIP;
}

int32_t rss_calib_copy(const void* src, void* dst, size_t bytes, int32_t blocks, void* stream) {
  if (!src || !dst || !aligned16(src) || !aligned16(dst) || bytes % 16 || blocks < 0) return RSS_E_INVALID;
  if (bytes == 0) return RSS_OK;
  hipLaunchKernelGGL(rss::calib_copy_kernel, dim3(grid_of(blocks)), dim3(rss::kCalibThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const rss::f32x4*>(src),
                     static_cast<rss::f32x4*>(dst), bytes / 16);
  return hipGetLastError() == hipSuccess ? RSS_OK : RSS_E_HIP;
}

int32_t rss_calib_write(void* dst, size_t bytes, int32_t blocks, void* stream) {
  if (!dst || !aligned16(dst) || bytes % 16 || blocks < 0) return RSS_E_INVALID;
  if (bytes == 0) return RSS_OK;
  hipLaunchKernelGGL(rss::calib_write_kernel, dim3(grid_of(blocks)), dim3(rss::kCalibThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<rss::f32x4*>(dst), bytes / 16);
  return hipGetLastError() == hipSuccess ? RSS_OK : RSS_E_HIP;
}

}  // extern "C"

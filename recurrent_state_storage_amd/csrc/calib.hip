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

// One workgroup per tile, the decode kernels' shape of work: the tile's
// 16-byte non-temporal loads all issued at once (thread i takes vectors
// i, i + 256, ...), then `wvec` 16-byte vectors written per tile at
// dst[t * wvec + i], each carrying its thread's sum of the tile, so that the
// writes follow the reads as a decode's outputs and ring entries do. Tiles are
// dealt to the XCDs in runs of up to 512 KiB, as the decode kernels deal theirs
// (order 0), or in one contiguous range per XCD (order 1).
// COPY: the tile itself is written to dst (each thread stores the vectors it
// loaded, non-temporal), a decode kernel's read-then-write-back of a state tile.
// The other order a calibration may take: XCD x works through one contiguous
// range of tiles, x-th of eight, in address order.
__device__ __forceinline__ int xcd_range(int id, int n) {
  const int x = id % kXcds, q = n / kXcds, r = n % kXcds;
  return x * q + (x < r ? x : r) + id / kXcds;
}

template <int L, bool COPY>  // L: 16-byte loads per thread (tile bytes / 4096)
__global__ __launch_bounds__(kCalibThreads) void calib_tiles_kernel(const f32x4* src, f32x4* dst,
                                                                    int wvec, int order) {
  const int t = order ? xcd_range(blockIdx.x, gridDim.x)
                      : xcd_tile(blockIdx.x, gridDim.x, L * kCalibThreads * 16);
  const f32x4* tile = src + (size_t)t * (L * kCalibThreads);
  f32x4 v[L];
#pragma unroll
  for (int k = 0; k < L; ++k) v[k] = __builtin_nontemporal_load(tile + k * kCalibThreads + threadIdx.x);
  if constexpr (COPY) {
    f32x4* out = dst + (size_t)t * (L * kCalibThreads);
#pragma unroll
    for (int k = 0; k < L; ++k) __builtin_nontemporal_store(v[k], out + k * kCalibThreads + threadIdx.x);
    return;
  }
  f32x4 acc = v[0];
#pragma unroll
  for (int k = 1; k < L; ++k) acc += v[k];
  const float s = acc.x + acc.y + acc.z + acc.w;
  // Every thread's loads are used here: without this the compiler moves them
  // into the branch below, and threads that write nothing would read nothing.
  asm volatile("" ::"v"(s));
  if ((int)threadIdx.x < wvec)
    dst[(size_t)t * wvec + threadIdx.x] = f32x4{s, (float)threadIdx.x, (float)(t & 0xffffff), 1.f};
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

int32_t rss_calib_tiles(const void* src, size_t tile_bytes, int32_t n_tiles, void* dst,
                        int32_t write_bytes, int32_t order, void* stream) {
  if (tile_bytes != 4096 && tile_bytes != 8192 && tile_bytes != 16384 && tile_bytes != 32768 &&
      tile_bytes != 65536)
    return RSS_E_INVALID;
  const bool copy = (size_t)write_bytes == tile_bytes;
  if (!src || !aligned16(src) || n_tiles < 0 || write_bytes < 0 || write_bytes % 16 ||
      (write_bytes > 4096 && !copy) || (write_bytes > 0 && (!dst || !aligned16(dst))) ||
      (order != 0 && order != 1))
    return RSS_E_INVALID;
  if (n_tiles == 0) return RSS_OK;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const rss::f32x4* in = static_cast<const rss::f32x4*>(src);
  rss::f32x4* out = static_cast<rss::f32x4*>(dst);
  const int wvec = write_bytes / 16;
  const dim3 grid((unsigned)n_tiles), block(rss::kCalibThreads);
#define RSS_CALIB_TILES(L_)                                                             \
  do {                                                                                   \
    if (copy) hipLaunchKernelGGL((rss::calib_tiles_kernel<L_, true>), grid, block, 0, s, in, out, wvec, order); \
    else hipLaunchKernelGGL((rss::calib_tiles_kernel<L_, false>), grid, block, 0, s, in, out, wvec, order);     \
  } while (0)
  switch (tile_bytes / 4096) {
    case 1: RSS_CALIB_TILES(1); break;
    case 2: RSS_CALIB_TILES(2); break;
    case 4: RSS_CALIB_TILES(4); break;
    case 8: RSS_CALIB_TILES(8); break;
    default: RSS_CALIB_TILES(16); break;
  }
#undef RSS_CALIB_TILES
  return hipGetLastError() == hipSuccess ? RSS_OK : RSS_E_HIP;
}

}  // extern "C"

// Device helpers shared by the gfx950 kernels of librss.
//
// Tile geometry. One 256-thread workgroup (four 64-wide wavefronts) owns one
// (sequence, head) P x N tile, N fastest. Each thread reads 16 bytes per load:
// 4 fp32 or 8 bf16 consecutive columns. TPR = N / VEC threads cover a row,
// RPP = 256 / TPR rows are covered per pass, and up to kMaxPass passes are held
// in registers at once, so a 64 x 128 fp32 tile (32 KiB) is 8 loads per thread
// issued back to back. Rows never straddle a wavefront (TPR <= 64), so every
// row reduction is a butterfly of __shfl_xor inside a wavefront.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "limits.h"

namespace rss {

constexpr int kWaves = kThreads / 64;

// Error bits of the sticky device word (same values as the public header).
constexpr int kDevRollbackRange = 1;
constexpr int kDevRingOverflow = 2;
constexpr int kDevUncommitted = 4;

typedef uint16_t bf16_t;  // raw bf16 bits

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest, ties to even; NaN stays a (quiet) NaN.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<bf16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

template <typename T> __device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<bf16_t>(bf16_t v) { return bf16_to_f32(v); }

template <int N, bool LOW>
struct TileGeom {
  static constexpr int VEC = LOW ? 8 : 4;       // elements per 16-byte load
  static constexpr int TPR = N / VEC;            // threads per row
  static constexpr int RPP = kThreads / TPR;     // rows per pass
  static_assert(N % VEC == 0 && TPR >= 1 && TPR <= 64, "unsupported N");
  static_assert((TPR & (TPR - 1)) == 0, "N/VEC must be a power of two");
};

// Sum over the TPR consecutive lanes that share a row (fixed butterfly order).
template <int TPR>
__device__ __forceinline__ float row_sum(float v) {
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// 16-byte tile fragment: 4 fp32 or 8 bf16 values.
template <bool LOW> struct Frag;
template <> struct Frag<false> {
  float4 v;
  __device__ __forceinline__ float get(int i) const {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
  }
};
template <> struct Frag<true> {
  uint4 v;
  __device__ __forceinline__ float get(int i) const {
    const uint32_t w = i < 2 ? v.x : i < 4 ? v.y : i < 6 ? v.z : v.w;
    return (i & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
  }
};

__device__ __forceinline__ float4 ld16(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ uint4 ld16(const bf16_t* p) { return *reinterpret_cast<const uint4*>(p); }

// Ring slot of window position j (0 <= head < R, 0 <= j < R).
__device__ __forceinline__ int ring_slot(int head, int j, int R) {
  int s = head + j;
  return s >= R ? s - R : s;
}

}  // namespace rss

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

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Streaming 16-byte loads of checkpoint tiles: each byte is used once, so they
// are marked non-temporal to keep the caches for the small, reused data.
__device__ __forceinline__ float4 ld16(const float* p) {
  const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint4 ld16(const bf16_t* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st16(float* p, const float4& v) {
  __builtin_nontemporal_store(f32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<f32x4*>(p));
}

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) { return f32_to_bf16(v); }

// Reverse exclusive scan over the 64 lanes of a wavefront:
// returns sum_{m > lane} v_m, summed as a fixed tree (deterministic).
__device__ __forceinline__ float wave_suffix_excl(float v, int lane) {
  float s = __shfl_down(v, 1, 64);
  if (lane == 63) s = 0.f;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float t = __shfl_down(s, off, 64);
    if (lane + off < 64) s += t;
  }
  return s;
}

// 16-byte vectors of input elements (8 bf16 or 4 fp32) and their fp32 unpacking
// into LDS. Window rows are staged through these: row lengths are multiples of
// the vector width, so a vector never straddles two rows.
template <typename Tin> struct V16;
template <> struct V16<float> {
  typedef float4 T;
  static constexpr int VE = 4;
};
template <> struct V16<bf16_t> {
  typedef uint4 T;
  static constexpr int VE = 8;
};

template <typename Tin>
__device__ __forceinline__ typename V16<Tin>::T ldv(const Tin* p) {
  return *reinterpret_cast<const typename V16<Tin>::T*>(p);
}

__device__ __forceinline__ void st_lds_f32(float* d, const float4& v) {
  *reinterpret_cast<float4*>(d) = v;
}
__device__ __forceinline__ void st_lds_f32(float* d, const uint4& v) {
  *reinterpret_cast<float4*>(d) =
      make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                  __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u));
  *reinterpret_cast<float4*>(d + 4) =
      make_float4(__uint_as_float(v.z << 16), __uint_as_float(v.z & 0xffff0000u),
                  __uint_as_float(v.w << 16), __uint_as_float(v.w & 0xffff0000u));
}

__host__ __device__ constexpr int align4(int n) { return (n + 3) & ~3; }

// Ring slot of window position j (0 <= head < R, 0 <= j < R).
__device__ __forceinline__ int ring_slot(int head, int j, int R) {
  int s = head + j;
  return s >= R ? s - R : s;
}

}  // namespace rss

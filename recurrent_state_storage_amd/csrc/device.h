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

// fp32 -> bf16, round to nearest, ties to even; a NaN stays NaN (quiet bit set,
// sign and top payload bits kept); denormals are rounded, not flushed. gfx950's
// packed conversion (v_cvt_pk_bf16_f32, two values per instruction) does
// exactly this: it agrees with the bit-level definition (add 0x7fff plus the
// lowest kept bit, truncate; NaN -> (bits >> 16) | 0x40) on all 2^32 inputs.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return static_cast<bf16_t>(pack_bf16x2(f, 0.f) & 0xffffu);
}

template <typename T> __device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<bf16_t>(bf16_t v) { return bf16_to_f32(v); }

template <int N, bool LOW, int NT = kThreads>
struct TileGeom {
  static constexpr int VEC = LOW ? 8 : 4;       // elements per 16-byte load
  static constexpr int TPR = N / VEC;            // threads per row
  static constexpr int RPP = NT / TPR;           // rows per pass (NT threads per workgroup)
  static constexpr int SR = 64 / TPR;            // rows per pass in one wavefront
  static_assert(N % VEC == 0 && TPR >= 1 && TPR <= 64, "unsupported N");
  static_assert((TPR & (TPR - 1)) == 0, "N/VEC must be a power of two");
};

// Rows of a tile chunk held by one thread. A chunk is RPP * MP rows starting at
// `base`; wavefront w owns its MP * SR consecutive rows starting at
// base + w * MP * SR, and pass k of the wavefront covers the SR rows starting at
// base + w * MP * SR + k * SR (lane / TPR picks the row). Each wavefront thus
// loads whole, adjacent rows per 16-byte load (full cache lines) and its row
// outputs are contiguous.
template <int TPR, int MP>
struct RowMap {
  static constexpr int SR = 64 / TPR;
  int off;   // row offset of this thread inside the chunk, pass 0
  __device__ explicit RowMap(int tid) : off((tid >> 6) * MP * SR + (tid & 63) / TPR) {}
  __device__ int row(int base, int k) const { return base + k * SR + off; }
  // First row of pass k in this thread's wavefront (uniform across it).
  __device__ int wave_row(int base, int k, int wave) const { return base + (wave * MP + k) * SR; }
};

// Workgroup -> tile index, XCD-aware. The dispatcher hands consecutive
// workgroup ids to the eight XCDs in turn, each with its own L2. This bijection
// on [0, n) takes the ids in groups of 8 runs of 2^lc tiles, a run being the
// largest power-of-two number of tiles within 512 KiB: inside a group XCD x
// works through the x-th run. So each XCD streams runs of consecutive tiles
// (neighbouring heads, whose pointer words and ring entries share cache lines,
// go through one L2), while the eight XCDs together stay on one 4 MiB stretch
// of the state at a time. Measured on MI355X against one contiguous range per
// XCD (every tile of XCD x before those of XCD x + 1 in address order), 512 KiB
// runs beat both that and shorter or longer runs. Ids past the last whole group
// map to themselves.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_tile(int id, int n, int tile_bytes) {
  const int cl = tile_bytes > 1 ? 32 - __builtin_clz((unsigned)tile_bytes - 1u) : 0;  // ceil(log2)
  const int lc = cl < 19 ? 19 - cl : 0;                     // run of 2^lc tiles <= 512 KiB
  const int grp = kXcds << lc;                              // ids per group (a power of two)
  if (id >= (n & -grp)) return id;
  return (id & -grp) | ((id % kXcds) << lc) | ((id / kXcds) & ((1 << lc) - 1));
}

// ---- cross-lane exchanges ----------------------------------------------------
// xchg<BIT>(v) returns v of a partner lane whose id has the opposite bit BIT and
// the same higher bits: lane ^ 1 and lane ^ 2 (DPP quad permutes), lane ^ 7
// (DPP half-row mirror), lane ^ 8 (DPP row rotate by 8), lane ^ 16 (LDS-free
// ds_swizzle bit mode) and lane ^ 32 (ds_bpermute). The DPP forms are folded
// into the consuming add, so a butterfly step costs one VALU instruction.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, true));
}
template <int BIT> __device__ __forceinline__ float xchg(float v);
template <> __device__ __forceinline__ float xchg<0>(float v) { return dpp_f<0xB1>(v); }
template <> __device__ __forceinline__ float xchg<1>(float v) { return dpp_f<0x4E>(v); }
template <> __device__ __forceinline__ float xchg<2>(float v) { return dpp_f<0x141>(v); }
template <> __device__ __forceinline__ float xchg<3>(float v) { return dpp_f<0x128>(v); }
template <> __device__ __forceinline__ float xchg<4>(float v) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
}
template <> __device__ __forceinline__ float xchg<5>(float v) { return __shfl_xor(v, 32, 64); }

// Butterfly sum over the 2^NBITS lanes that agree in every bit >= NBITS, low
// bit first (with bits 0 and 1 already summed, the lane ^ 7 partner of bit 2
// holds the same value as lane ^ 4). Fixed order, so results are deterministic.
template <int NBITS>
__device__ __forceinline__ float lanes_sum(float v) {
  if constexpr (NBITS > 0) {
    v = lanes_sum<NBITS - 1>(v);
    v += xchg<NBITS - 1>(v);
  }
  return v;
}

template <int X> struct Log2 { static constexpr int v = 1 + Log2<X / 2>::v; };
template <> struct Log2<1> { static constexpr int v = 0; };

// Sum over the TPR consecutive lanes that share a row.
template <int TPR>
__device__ __forceinline__ float row_sum(float v) { return lanes_sum<Log2<TPR>::v>(v); }

// Sum over the 64 lanes, returned as a wavefront-uniform value: the 16-lane
// row butterfly above, then the GFX9 row broadcasts (lane 15 of row r into row
// r + 1 for rows 1 and 3, lane 31 into rows 2 and 3) leave the total in lane
// 63, which is read into a scalar register. No LDS round trip (the lane ^ 16 and
// lane ^ 32 exchanges of a full butterfly go through the LDS crossbar), fixed
// order, so deterministic.
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_rows(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWS, 0xf, false));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = lanes_sum<4>(v);
  v += dpp_rows<0x142, 0xa>(v);   // row_bcast:15
  v += dpp_rows<0x143, 0xc>(v);   // row_bcast:31
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Reduce-scatter of the 8 tile passes over a row group of TPR = 2^T lanes.
// On entry a[k] is this lane's partial dot for the row of pass k. Each step
// halves the values a lane keeps (by one lane-id bit, highest first) and adds
// the partner's copy of the half it keeps; after min(T, 3) steps the remaining
// low bits are summed by butterfly. On return a[0 .. NOUT-1], NOUT = 8 >> min(T,3),
// are complete row sums for passes kbase .. kbase + NOUT - 1; the lanes whose
// low T - min(T, 3) bits are zero own distinct rows and write them.
template <int BIT, int NV>
__device__ __forceinline__ void rs_step(float* a, int lr, int& kbase) {
  constexpr int H = NV / 2;
  const bool hi = (lr >> BIT) & 1;
#pragma unroll
  for (int m = 0; m < H; ++m) {
    const float send = hi ? a[m] : a[m + H];
    const float keep = hi ? a[m + H] : a[m];
    a[m] = keep + xchg<BIT>(send);
  }
  if (hi) kbase += H;
}

template <int TPR>
struct RowScatter {
  static constexpr int T = Log2<TPR>::v;
  static constexpr int S = T < 3 ? T : 3;
  static constexpr int NOUT = 8 >> S;
  static constexpr int WMASK = (1 << (T - S)) - 1;   // writer lanes: (lr & WMASK) == 0
  __device__ static __forceinline__ void run(float (&a)[8], int lr, int& kbase) {
    kbase = 0;
    if constexpr (T >= 1) rs_step<T - 1, 8>(a, lr, kbase);
    if constexpr (T >= 2) rs_step<T - 2, 4>(a, lr, kbase);
    if constexpr (T >= 3) rs_step<T - 3, 2>(a, lr, kbase);
    if constexpr (T > 3) a[0] = lanes_sum<T - 3>(a[0]);
  }
};

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
// Eight fp32 values stored as RNE bf16 (16 bytes, non-temporal).
__device__ __forceinline__ void st16_bf16x8(bf16_t* p, const float (&v)[8]) {
  u32x4 pk;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    pk[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
  __builtin_nontemporal_store(pk, reinterpret_cast<u32x4*>(p));
}

// Four bf16 values of a bf16 checkpoint (8 bytes, non-temporal) widened to
// fp32, and their RNE-packed store: the tile geometry of the fp32 state (4
// columns per thread) kept for a bf16-stored state.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float4 ld8_bf16x4(const bf16_t* p) {
  const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                     __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u));
}
__device__ __forceinline__ void st8_bf16x4(bf16_t* p, const float4& v) {
  const u32x2 pk = {pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)};
  __builtin_nontemporal_store(pk, reinterpret_cast<u32x2*>(p));
}

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) { return f32_to_bf16(v); }

// Reverse exclusive scan over the 64 lanes of a wavefront: returns
// sum_{m > lane} v_m as a fixed tree, with no LDS traffic: the wavefront shift
// (lane i takes v_{i+1}, lane 63 takes 0), the inclusive suffix within each
// 16-lane row by row shifts of 1, 2, 4 and 8 (lanes past the row's end read 0),
// then the totals of the higher rows, read into scalar registers, added per row.
template <int CTRL>
__device__ __forceinline__ float dpp_or_zero(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, true));
}
__device__ __forceinline__ float wave_suffix_excl(float v, int lane) {
  float x = dpp_or_zero<0x130>(v);   // wave_shl:1
  x += dpp_or_zero<0x101>(x);        // row_shl:1
  x += dpp_or_zero<0x102>(x);        // row_shl:2
  x += dpp_or_zero<0x104>(x);        // row_shl:4
  x += dpp_or_zero<0x108>(x);        // row_shl:8
  const float t1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
  const float t2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
  const float t3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
  const float s23 = t2 + t3, s123 = t1 + s23;
  const int row = lane >> 4;
  return x + (row == 0 ? s123 : row == 1 ? s23 : row == 2 ? t3 : 0.f);
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
// The same, non-temporal: for data read for the last time (a fold's ring rows).
template <typename Tin>
__device__ __forceinline__ typename V16<Tin>::T ldv_nt(const Tin* p) {
  return __builtin_bit_cast(typename V16<Tin>::T, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
}

// A 16-byte vector of input elements widened to fp32 in registers.
__device__ __forceinline__ void unpack16(const float4& v, float* d) {
  d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
}
__device__ __forceinline__ void unpack16(const uint4& v, float* d) {
  d[0] = __uint_as_float(v.x << 16); d[1] = __uint_as_float(v.x & 0xffff0000u);
  d[2] = __uint_as_float(v.y << 16); d[3] = __uint_as_float(v.y & 0xffff0000u);
  d[4] = __uint_as_float(v.z << 16); d[5] = __uint_as_float(v.z & 0xffff0000u);
  d[6] = __uint_as_float(v.w << 16); d[7] = __uint_as_float(v.w & 0xffff0000u);
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

// Direct global -> LDS 16-byte load (gfx950 global_load_lds_dwordx4): lane l of
// the wavefront writes its 16 bytes at lds_wave_base + 16 l. lds_wave_base must
// be uniform across the wavefront and 16-byte aligned. Completion is tracked by
// the vector-memory counter; wait for it before reading the LDS bytes.
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void gbl_void_t;
__device__ __forceinline__ void dma16(const void* g, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((gbl_void_t*)g, (lds_void_t*)lds_wave_base, 16, 0, 0);
}
// The same, marked non-temporal (read once: a call's own inputs). Lanes of one
// wavefront may mix the two forms under complementary exec masks: each writes
// its own lane's 16 bytes.
constexpr int kCachePolicyNt = 2;
__device__ __forceinline__ void dma16_nt(const void* g, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((gbl_void_t*)g, (lds_void_t*)lds_wave_base, 16, 0, kCachePolicyNt);
}

// Ring slot of window position j (0 <= head < R, 0 <= j < R).
__device__ __forceinline__ int ring_slot(int head, int j, int R) {
  int s = head + j;
  return s >= R ? s - R : s;
}

// Ring slot of window position j for 0 <= j < 2R (a verify that folds its
// committed window in the same pass stages up to R + K + 1 positions).
__device__ __forceinline__ int ring_slot2(int head, int j, int R) {
  int s = head + j;
  if (s >= R) s -= R;
  return s >= R ? s - R : s;
}

}  // namespace rss

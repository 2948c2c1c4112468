// Eager baseline: the per-token state rewrite ReplaySSM replaces.
//
// P1 ("La fiche qu'on réécrit à chaque token"): each decode step reads the
// previous state from HBM, applies a decay factor and a rank-1 update, computes
// the output and writes the whole state back; the kernel reads and writes the
// whole state for very little arithmetic, so HBM bandwidth is the limit.
//
//   a = exp(dt A_h);  S <- a S + dt outer(x, B);  y = S @ C
//
// In-place mode runs T tokens on S. Snapshot mode is the pre-ReplaySSM
// speculative rollback scheme (P3, "Почему это важно для индустрии": rollback
// needed state snapshots; P4, "Co się zmieniło?", item 4): the state is read
// from pool slot src_slot[b], and the state after token i is written to slot i.
//
// A bf16-stored state (the quantised eager state of P1, "Trois ennuis nés de
// la même fusion": rewritten, hence rounded, at every token) is widened to fp32,
// updated and read out in fp32, and stored back RNE-rounded (eager_bf16_kernel).
//
// Same tile geometries as the replay kernels: one 256-thread workgroup per
// fp32 (sequence, head) tile with 4-column fragments, two wavefronts with
// 8-column fragments per bf16 tile; row dots by reduce-scatter.
#include "device.h"
#include "launch.h"

namespace rss {

template <int N, typename Tin, bool POOL>
__global__ __launch_bounds__(kThreads) void eager_kernel(EagerArgs a) {
  using Geo = TileGeom<N, false>;
  constexpr int TPR = Geo::TPR, RPP = Geo::RPP;
  using Rows = RowMap<TPR, kMaxPass>;

  __shared__ float sa[kMaxNew];
  __shared__ float sdtv[kMaxNew];
  extern __shared__ __align__(16) float dyn[];  // xs[T][P], Bs[T][N], Cs[T][N]

  const int tid = threadIdx.x;
  const int H = a.H, P = a.P, G = a.G, T = a.T;
  const int bh = xcd_tile(blockIdx.x, gridDim.x, P * N * 4);
  const int b = bh / H, h = bh - b * H;
  const int g = h / (H / G);
  const size_t tile_elems = (size_t)P * N;

  float* src;
  float* const S = static_cast<float*>(a.S);
  if (POOL) {
    const int s = a.src_slot[b];
    if (s < 0 || s >= a.slots) {
      for (int e = tid; e < T * P; e += kThreads) {
        const int i = e / P, p = e - i * P;
        a.y[((size_t)(b * T + i) * H + h) * P + p] = __builtin_nanf("");
      }
      return;
    }
    src = S + (((size_t)b * a.slots + s) * H + h) * tile_elems;
  } else {
    src = S + (size_t)bh * tile_elems;
  }

  const int col = tid % TPR;
  const Rows rows(tid);
  Frag<false> fr[kMaxPass];
  auto load_chunk = [&](int base) {
#pragma unroll
    for (int k = 0; k < kMaxPass; ++k) {
      const int row = rows.row(base, k);
      if (row >= P) fr[k].v = float4{};
      else fr[k].v = ld16(src + row * N + col * 4);
    }
  };
  load_chunk(0);

  float* xs = dyn;
  float* Bs = dyn + T * P;
  float* Cs = Bs + T * N;
  const Tin* xin = static_cast<const Tin*>(a.x);
  const Tin* Bin = static_cast<const Tin*>(a.B);
  const Tin* Cin = static_cast<const Tin*>(a.C);
  for (int e = tid; e < T * P; e += kThreads) {
    const int i = e / P, p = e - i * P;
    xs[e] = to_f32(xin[((size_t)(b * T + i) * H + h) * P + p]);
  }
  for (int e = tid; e < T * N; e += kThreads) {
    const int i = e / N, c = e - i * N;
    const size_t off = ((size_t)(b * T + i) * G + g) * N + c;
    Bs[e] = to_f32(Bin[off]);
    Cs[e] = to_f32(Cin[off]);
  }
  if (tid < T) {
    const float d = a.dt[(size_t)(b * T + tid) * H + h];
    sdtv[tid] = d;
    sa[tid] = expf(d * a.A[h]);
  }
  __syncthreads();

  // Per token: every pass is updated (rows past P hold zeros, read a valid x
  // row and are never stored, so the pass loop has no branch), each row's dot
  // with C is reduce-scattered over the row's lanes (the replay's tree), and the
  // writer lanes store y; a snapshot slot, when asked for, is written as it
  // forms. In place, the state is stored once after the last token.
  using RS = RowScatter<TPR>;
  for (int base = 0; base < P; base += RPP * kMaxPass) {
    if (base > 0) load_chunk(base);
    int xrow[kMaxPass];
#pragma unroll
    for (int k = 0; k < kMaxPass; ++k) {
      const int row = rows.row(base, k);
      xrow[k] = row < P ? row : P - 1;
    }
    for (int i = 0; i < T; ++i) {
      const float ai = sa[i], di = sdtv[i];
      const float4 bv = *reinterpret_cast<const float4*>(&Bs[i * N + col * 4]);
      const float4 cv = *reinterpret_cast<const float4*>(&Cs[i * N + col * 4]);
      float part[kMaxPass];
#pragma unroll
      for (int k = 0; k < kMaxPass; ++k) {
        const float u = di * xs[i * P + xrow[k]];
        float4& s = fr[k].v;
        s.x = fmaf(u, bv.x, ai * s.x);
        s.y = fmaf(u, bv.y, ai * s.y);
        s.z = fmaf(u, bv.z, ai * s.z);
        s.w = fmaf(u, bv.w, ai * s.w);
        float acc = s.x * cv.x;
        acc = fmaf(s.y, cv.y, acc);
        acc = fmaf(s.z, cv.z, acc);
        part[k] = fmaf(s.w, cv.w, acc);
      }
      if (POOL) {
        float* dst = S + (((size_t)b * a.slots + i) * H + h) * tile_elems;
#pragma unroll
        for (int k = 0; k < kMaxPass; ++k) {
          const int row = rows.row(base, k);
          if (row < P) st16(dst + row * N + col * 4, fr[k].v);
        }
      }
      int kbase;
      RS::run(part, col, kbase);
      if ((col & RS::WMASK) == 0) {
        float* yo = a.y + ((size_t)(b * T + i) * H + h) * P;
#pragma unroll
        for (int m = 0; m < RS::NOUT; ++m) {
          const int row = rows.row(base, kbase + m);
          if (row < P) yo[row] = part[m];
        }
      }
    }
    if (!POOL) {
#pragma unroll
      for (int k = 0; k < kMaxPass; ++k) {
        const int row = rows.row(base, k);
        if (row < P) st16(src + row * N + col * 4, fr[k].v);
      }
    }
  }
}

// A bf16-stored state (eager in place only) in the bf16 tiles' geometry: two
// wavefronts per (sequence, head), 16-byte fragments of 8 columns, so each lane
// issues the same 16-byte loads and stores as the other kernels. The packed
// state stays in registers; per token every fragment is widened, updated in
// fp32, read out (y from the unrounded new state) and RNE-packed again, so the
// state is rounded after every token.
constexpr int kEagerLowThreads = 128;

template <int N, typename Tin>
__global__ __launch_bounds__(kEagerLowThreads) void eager_bf16_kernel(EagerArgs a) {
  constexpr int NT = kEagerLowThreads;
  using Geo = TileGeom<N, true, NT>;
  constexpr int TPR = Geo::TPR, RPP = Geo::RPP;
  using Rows = RowMap<TPR, kMaxPass>;

  __shared__ float sa[kMaxNew];
  __shared__ float sdtv[kMaxNew];
  extern __shared__ __align__(16) float dyn[];  // xs[T][P], Bs[T][N], Cs[T][N]

  const int tid = threadIdx.x;
  const int H = a.H, P = a.P, G = a.G, T = a.T;
  const int bh = xcd_tile(blockIdx.x, gridDim.x, P * N * 2);
  const int b = bh / H, h = bh - b * H;
  const int g = h / (H / G);
  bf16_t* st = static_cast<bf16_t*>(a.S) + (size_t)bh * P * N;

  const int col = tid % TPR;
  const Rows rows(tid);
  Frag<true> fr[kMaxPass];
  auto load_chunk = [&](int base) {
#pragma unroll
    for (int k = 0; k < kMaxPass; ++k) {
      const int row = rows.row(base, k);
      if (row >= P) fr[k].v = make_uint4(0u, 0u, 0u, 0u);
      else fr[k].v = ld16(st + row * N + col * 8);
    }
  };
  load_chunk(0);

  float* xs = dyn;
  float* Bs = dyn + T * P;
  float* Cs = Bs + T * N;
  const Tin* xin = static_cast<const Tin*>(a.x);
  const Tin* Bin = static_cast<const Tin*>(a.B);
  const Tin* Cin = static_cast<const Tin*>(a.C);
  for (int e = tid; e < T * P; e += NT) {
    const int i = e / P, p = e - i * P;
    xs[e] = to_f32(xin[((size_t)(b * T + i) * H + h) * P + p]);
  }
  for (int e = tid; e < T * N; e += NT) {
    const int i = e / N, c = e - i * N;
    const size_t off = ((size_t)(b * T + i) * G + g) * N + c;
    Bs[e] = to_f32(Bin[off]);
    Cs[e] = to_f32(Cin[off]);
  }
  if (tid < T) {
    const float d = a.dt[(size_t)(b * T + tid) * H + h];
    sdtv[tid] = d;
    sa[tid] = expf(d * a.A[h]);
  }
  __syncthreads();

  using RS = RowScatter<TPR>;
  for (int base = 0; base < P; base += RPP * kMaxPass) {
    if (base > 0) load_chunk(base);
    int xrow[kMaxPass];
#pragma unroll
    for (int k = 0; k < kMaxPass; ++k) {
      const int row = rows.row(base, k);
      xrow[k] = row < P ? row : P - 1;
    }
    for (int i = 0; i < T; ++i) {
      const float ai = sa[i], di = sdtv[i];
      float bv[8], cv[8];
      unpack16(*reinterpret_cast<const float4*>(&Bs[i * N + col * 8]), bv);
      unpack16(*reinterpret_cast<const float4*>(&Bs[i * N + col * 8 + 4]), bv + 4);
      unpack16(*reinterpret_cast<const float4*>(&Cs[i * N + col * 8]), cv);
      unpack16(*reinterpret_cast<const float4*>(&Cs[i * N + col * 8 + 4]), cv + 4);
      float part[kMaxPass];
#pragma unroll
      for (int k = 0; k < kMaxPass; ++k) {
        const float u = di * xs[i * P + xrow[k]];
        float sv[8];
        unpack16(fr[k].v, sv);
#pragma unroll
        for (int v = 0; v < 8; ++v) sv[v] = fmaf(u, bv[v], ai * sv[v]);
        float acc = sv[0] * cv[0];
#pragma unroll
        for (int v = 1; v < 8; ++v) acc = fmaf(sv[v], cv[v], acc);
        part[k] = acc;
        fr[k].v = make_uint4(pack_bf16x2(sv[0], sv[1]), pack_bf16x2(sv[2], sv[3]),
                             pack_bf16x2(sv[4], sv[5]), pack_bf16x2(sv[6], sv[7]));
      }
      int kbase;
      RS::run(part, col, kbase);
      if ((col & RS::WMASK) == 0) {
        float* yo = a.y + ((size_t)(b * T + i) * H + h) * P;
#pragma unroll
        for (int m = 0; m < RS::NOUT; ++m) {
          const int row = rows.row(base, kbase + m);
          if (row < P) yo[row] = part[m];
        }
      }
    }
#pragma unroll
    for (int k = 0; k < kMaxPass; ++k) {
      const int row = rows.row(base, k);
      if (row < P)
        __builtin_nontemporal_store(u32x4{fr[k].v.x, fr[k].v.y, fr[k].v.z, fr[k].v.w},
                                    reinterpret_cast<u32x4*>(st + row * N + col * 8));
    }
  }
}

template <int N, bool POOL>
static hipError_t eager_n(const EagerArgs& a, int batch, bool bf16_in, hipStream_t s) {
  const dim3 grid((unsigned)((size_t)batch * a.H)), block(kThreads);
  const size_t lds = (size_t)a.T * (a.P + 2 * N) * sizeof(float);
  if (bf16_in) hipLaunchKernelGGL((eager_kernel<N, bf16_t, POOL>), grid, block, lds, s, a);
  else hipLaunchKernelGGL((eager_kernel<N, float, POOL>), grid, block, lds, s, a);
  return hipGetLastError();
}

template <int N>
static hipError_t eager_s(const EagerArgs& a, int batch, bool bf16_in, bool bf16_state, hipStream_t s) {
  if (a.src_slot) return eager_n<N, true>(a, batch, bf16_in, s);
  if (bf16_state) {
    const size_t lds = (size_t)a.T * (a.P + 2 * N) * sizeof(float);
    const dim3 grid((unsigned)((size_t)batch * a.H)), block(kEagerLowThreads);
    if (bf16_in) hipLaunchKernelGGL((eager_bf16_kernel<N, bf16_t>), grid, block, lds, s, a);
    else hipLaunchKernelGGL((eager_bf16_kernel<N, float>), grid, block, lds, s, a);
    return hipGetLastError();
  }
  return eager_n<N, false>(a, batch, bf16_in, s);
}

hipError_t launch_eager(const EagerArgs& a, int batch, int N, bool bf16_in, bool bf16_state,
                        hipStream_t s) {
  if (bf16_state && a.src_slot) return hipErrorInvalidValue;  // snapshot pools are fp32
  switch (N) {
    case 16: return eager_s<16>(a, batch, bf16_in, bf16_state, s);
    case 32: return eager_s<32>(a, batch, bf16_in, bf16_state, s);
    case 64: return eager_s<64>(a, batch, bf16_in, bf16_state, s);
    case 128: return eager_s<128>(a, batch, bf16_in, bf16_state, s);
    case 256: return eager_s<256>(a, batch, bf16_in, bf16_state, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace rss

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
// la même fusion": rewritten, hence rounded, at every call) is widened to fp32
// on load, updated and read out in fp32, and stored back RNE-rounded.
//
// Same tile geometry as the replay kernels: one 256-thread workgroup per
// (sequence, head), 4-column fragments in registers, row dots by butterfly.
#include "device.h"
#include "launch.h"

namespace rss {

template <int N, typename Tin, bool SB16>
__global__ __launch_bounds__(kThreads) void eager_kernel(EagerArgs a) {
  using Geo = TileGeom<N, false>;
  constexpr int TPR = Geo::TPR, RPP = Geo::RPP;

  __shared__ float sa[kMaxNew];
  __shared__ float sdtv[kMaxNew];
  extern __shared__ __align__(16) float dyn[];  // xs[T][P], Bs[T][N], Cs[T][N]

  const int tid = threadIdx.x;
  const int H = a.H, P = a.P, G = a.G, T = a.T;
  const int bh = blockIdx.x;
  const int b = bh / H, h = bh - b * H;
  const int g = h / (H / G);
  const size_t tile_elems = (size_t)P * N;

  float* src;
  bf16_t* srcb = SB16 ? static_cast<bf16_t*>(a.S) + (size_t)bh * tile_elems : nullptr;
  float* const S = static_cast<float*>(a.S);
  if (SB16) {
    src = nullptr;
  } else if (a.src_slot) {
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

  const int col = tid % TPR, rsub = tid / TPR;
  Frag<false> fr[kMaxPass];
  auto load_chunk = [&](int base) {
#pragma unroll
    for (int k = 0; k < kMaxPass; ++k) {
      const int row = base + k * RPP + rsub;
      if (row >= P) fr[k].v = float4{};
      else if constexpr (SB16) fr[k].v = ld8_bf16x4(srcb + (size_t)row * N + col * 4);
      else fr[k].v = ld16(src + (size_t)row * N + col * 4);
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

  for (int base = 0; base < P; base += RPP * kMaxPass) {
    if (base > 0) load_chunk(base);
    for (int i = 0; i < T; ++i) {
      const float ai = sa[i], di = sdtv[i];
      const float4 bv = *reinterpret_cast<const float4*>(&Bs[i * N + col * 4]);
      const float4 cv = *reinterpret_cast<const float4*>(&Cs[i * N + col * 4]);
#pragma unroll
      for (int k = 0; k < kMaxPass; ++k) {
        if (base + k * RPP >= P) break;
        const int row = base + k * RPP + rsub;
        const float u = row < P ? di * xs[i * P + row] : 0.f;
        float4& s = fr[k].v;
        s.x = fmaf(u, bv.x, ai * s.x);
        s.y = fmaf(u, bv.y, ai * s.y);
        s.z = fmaf(u, bv.z, ai * s.z);
        s.w = fmaf(u, bv.w, ai * s.w);
        float part = s.x * cv.x;
        part = fmaf(s.y, cv.y, part);
        part = fmaf(s.z, cv.z, part);
        part = fmaf(s.w, cv.w, part);
        part = row_sum<TPR>(part);
        if (col == 0 && row < P) a.y[((size_t)(b * T + i) * H + h) * P + row] = part;
        if (!SB16 && a.src_slot && row < P) {
          float* dst = S + (((size_t)b * a.slots + i) * H + h) * tile_elems;
          *reinterpret_cast<float4*>(dst + (size_t)row * N + col * 4) = s;
        }
      }
    }
    if (!a.src_slot) {
#pragma unroll
      for (int k = 0; k < kMaxPass; ++k) {
        const int row = base + k * RPP + rsub;
        if (row >= P) continue;
        if constexpr (SB16) st8_bf16x4(srcb + (size_t)row * N + col * 4, fr[k].v);
        else *reinterpret_cast<float4*>(src + (size_t)row * N + col * 4) = fr[k].v;
      }
    }
  }
}

template <int N, bool SB16>
static hipError_t eager_n(const EagerArgs& a, int batch, bool bf16_in, hipStream_t s) {
  const dim3 grid((unsigned)((size_t)batch * a.H)), block(kThreads);
  const size_t lds = (size_t)a.T * (a.P + 2 * N) * sizeof(float);
  if (bf16_in) hipLaunchKernelGGL((eager_kernel<N, bf16_t, SB16>), grid, block, lds, s, a);
  else hipLaunchKernelGGL((eager_kernel<N, float, SB16>), grid, block, lds, s, a);
  return hipGetLastError();
}

template <int N>
static hipError_t eager_s(const EagerArgs& a, int batch, bool bf16_in, bool bf16_state, hipStream_t s) {
  return bf16_state ? eager_n<N, true>(a, batch, bf16_in, s) : eager_n<N, false>(a, batch, bf16_in, s);
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

// Replay kernels: decode (one new token) and speculative verify (K+1 tokens).
//
// Output of new token i, whose window position is t_i = n0 + i (n0 committed
// and earlier entries, then the new tokens 0..i):
//
//   y_i = exp(Lam_i) * (S_c @ C_i) + sum_{j <= t_i} exp(lam_i(j)) dt_j (B_j . C_i) x_j
//   lam_i(j) = sum_{m=j+1..t_i} l_m,   Lam_i = sum_{m=0..t_i} l_m,   l_m = dt_m A_h
//
// which is the eager recurrence unrolled from the checkpoint (P2, "L'astuce du
// checkpoint et du tampon": the recurrence is unrolled into an old checkpoint
// plus a buffer of recent inputs; P3, "Решение ReplaySSM": the output comes
// from checkpoint and buffer without writing a new state). Nothing of size
// P x N is written.
//
// One workgroup per (sequence, head). Every global load is issued in the first
// two memory round trips (the pointer word, then everything else), so a
// workgroup lives about two latencies whatever the window length:
//   1. read the (head, len) pointer word; issue the 16-byte non-temporal loads
//      of the checkpoint tile (the only large read);
//   2. issue, all at once, the window's x and B rows, the new tokens' C and the
//      window's (dt, l) pairs; then unpack them into LDS as fp32, and scan the
//      log-decays in one wavefront (a reverse tree sum: no prefix differences);
//   3. per (i, j) pair, one wavefront: w_ij = exp(lam) dt (B_j . C_i), and the
//      wavefront's share of sum_j w_ij x_j (wavefront w takes j = w mod 4);
//   4. consume the tile: per row a 16-byte fragment dot C_i, a butterfly over
//      the lanes sharing the row, y = exp(Lam) * dot + the four ring shares.
// The new tokens' x and B go to the ring straight from the staging registers.
// The checkpoint tile is read exactly once per call for all nt outputs.
#include <type_traits>

#include "device.h"
#include "launch.h"

namespace rss {

// Dynamic LDS layout of the replay kernel, in floats.
struct ReplayLds {
  int oX, oB, oC, oCF, oDC, oRing, total;
  __host__ __device__ ReplayLds(int R, int P, int N, int ntmax) {
    oX = 0;                          // window x rows    [R][P]
    oB = align4(R * P);              // window B rows    [R][N]
    oC = oB + R * N;                 // new tokens' C    [ntmax][N]
    oCF = oC + ntmax * N;            // exp(lam) * dt    [ntmax][R]
    oDC = oCF + ntmax * R;           // exp(Lam)         [ntmax]
    oRing = align4(oDC + ntmax);     // ring part, one share per wavefront [4][ntmax][P]
    total = oRing + 4 * ntmax * P;
  }
};

constexpr int kStageS = 4;  // scalar loads per thread and round (x rows when P % VE != 0)

template <int N, typename Tin, bool LOW, int NTMAX>
__global__ __launch_bounds__(kThreads) void replay_kernel(ReplayArgs a) {
  using Geo = TileGeom<N, LOW>;
  constexpr int VEC = Geo::VEC, TPR = Geo::TPR, RPP = Geo::RPP;
  constexpr int VE = V16<Tin>::VE;
  constexpr int NV = N / VE;                                   // vectors per B or C row
  constexpr int kStageC = (NTMAX * NV + kThreads - 1) / kThreads;
  // 16-byte loads per thread per staging round. One round holds a 16-entry
  // window of x and B at P = 64, N = 128 in bf16; longer windows take more rounds.
  constexpr int kStageX = NTMAX == 1 ? 1 : 2;
  constexpr int kStageB = NTMAX == 1 ? 1 : 2;
  using TileT = typename std::conditional<LOW, bf16_t, float>::type;
  using VT = typename V16<Tin>::T;

  extern __shared__ __align__(16) float lds[];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int H = a.H, P = a.P, G = a.G, R = a.R, nt = a.nt;
  const int bh = blockIdx.x;
  const int b = bh / H, h = bh - b * H;
  const int hpg = H / G, g = h / hpg;

  const int4 pt = a.ptr[bh];
  const int head = pt.x, n0 = pt.y;
  const int L = n0 + nt;

  if (head < 0 || head >= R || n0 < 0 || L > R) {  // ring full (no flush), or corrupt pointers
    if (tid == 0) atomicOr(a.err, kDevRingOverflow);
    for (int e = tid; e < nt * P; e += kThreads) {
      const int i = e / P, p = e - i * P;
      a.y[((size_t)(b * nt + i) * H + h) * P + p] = __builtin_nanf("");
    }
    return;
  }

  const ReplayLds lay(R, P, N, NTMAX);
  float* sX = lds + lay.oX;
  float* sB = lds + lay.oB;
  float* sC = lds + lay.oC;
  float* sCF = lds + lay.oCF;
  float* sDC = lds + lay.oDC;
  float* sRing = lds + lay.oRing;

  const Tin* xin = static_cast<const Tin*>(a.x);
  const Tin* Bin = static_cast<const Tin*>(a.B);
  const Tin* Cin = static_cast<const Tin*>(a.C);
  Tin* rx = static_cast<Tin*>(a.ring_x);
  Tin* rB = static_cast<Tin*>(a.ring_B);
  auto xrow = [&](int j) -> const Tin* {
    return j < n0 ? rx + ((size_t)bh * R + ring_slot(head, j, R)) * P
                  : xin + ((size_t)(b * nt + (j - n0)) * H + h) * P;
  };
  auto brow = [&](int j) -> const Tin* {
    return j < n0 ? rB + (((size_t)b * G + g) * R + ring_slot(head, j, R)) * N
                  : Bin + ((size_t)(b * nt + (j - n0)) * G + g) * N;
  };

  // 1. Checkpoint tile: first chunk of rows into registers.
  const int col = tid % TPR, rsub = tid / TPR;
  const TileT* tile = static_cast<const TileT*>(LOW ? a.ckpt_lo : static_cast<const void*>(a.ckpt))
                      + (size_t)bh * P * N;
  Frag<LOW> fr[kMaxPass];
  auto load_chunk = [&](int base) {
#pragma unroll
    for (int k = 0; k < kMaxPass; ++k) {
      const int r0 = base + k * RPP;
      if (r0 + RPP <= P) fr[k].v = ld16(tile + (size_t)(r0 + rsub) * N + col * VEC);  // whole pass
      else if (r0 + rsub < P) fr[k].v = ld16(tile + (size_t)(r0 + rsub) * N + col * VEC);
      else fr[k].v = decltype(fr[k].v){};
    }
  };
  load_chunk(0);

  // 2. Everything else in one round of loads, then unpack into LDS.
  const bool xvec = (P % VE) == 0;
  const int PV = xvec ? P / VE : 0;
  auto xdiv = [&](int q) { return (int)(((uint64_t)(uint32_t)q * a.xdiv) >> 32); };
  const int totXV = L * PV, totBV = L * NV, totCV = nt * NV;
  VT vx[kStageX], vb[kStageB], vc[kStageC];
  Tin sxs[kStageS];
#pragma unroll
  for (int m = 0; m < kStageB; ++m) {
    const int q = m * kThreads + tid;
    if (q < totBV) {
      const int j = q / NV, c = q - j * NV;
      vb[m] = ldv<Tin>(brow(j) + c * VE);
    }
  }
#pragma unroll
  for (int m = 0; m < kStageC; ++m) {
    const int q = m * kThreads + tid;
    if (q < totCV) {
      const int i = q / NV, c = q - i * NV;
      vc[m] = ldv<Tin>(Cin + ((size_t)(b * nt + i) * G + g) * N + c * VE);
    }
  }
  if (xvec) {
#pragma unroll
    for (int m = 0; m < kStageX; ++m) {
      const int q = m * kThreads + tid;
      if (q < totXV) {
        const int j = xdiv(q), c = q - j * PV;
        vx[m] = ldv<Tin>(xrow(j) + c * VE);
      }
    }
  } else {
#pragma unroll
    for (int m = 0; m < kStageS; ++m) {
      const int e = m * kThreads + tid;
      if (e < L * P) {
        const int j = xdiv(e);
        sxs[m] = xrow(j)[e - j * P];
      }
    }
  }
  const float Ah = a.A[h];
  float dtj = 0.f, lj = 0.f;
  if (tid < L) {  // wavefront 0: lane j holds window entry j's (dt, l)
    if (tid < n0) {
      const float2 v = a.ring_dl[(size_t)bh * R + ring_slot(head, tid, R)];
      dtj = v.x;
      lj = v.y;
    } else {
      dtj = a.dt[(size_t)(b * nt + (tid - n0)) * H + h];
      lj = dtj * Ah;
    }
  }

  const bool keepB = h == g * hpg;  // the group's first head keeps the group's B
#pragma unroll
  for (int m = 0; m < kStageB; ++m) {
    const int q = m * kThreads + tid;
    if (q < totBV) {
      st_lds_f32(sB + q * VE, vb[m]);
      const int j = q / NV;
      if (keepB && j >= n0)
        *reinterpret_cast<VT*>(rB + (((size_t)b * G + g) * R + ring_slot(head, j, R)) * N +
                               (q - j * NV) * VE) = vb[m];
    }
  }
#pragma unroll
  for (int m = 0; m < kStageC; ++m) {
    const int q = m * kThreads + tid;
    if (q < totCV) st_lds_f32(sC + q * VE, vc[m]);
  }
  if (xvec) {
#pragma unroll
    for (int m = 0; m < kStageX; ++m) {
      const int q = m * kThreads + tid;
      if (q < totXV) {
        st_lds_f32(sX + q * VE, vx[m]);
        const int j = xdiv(q);
        if (j >= n0)
          *reinterpret_cast<VT*>(rx + ((size_t)bh * R + ring_slot(head, j, R)) * P +
                                 (q - j * PV) * VE) = vx[m];
      }
    }
  } else {
#pragma unroll
    for (int m = 0; m < kStageS; ++m) {
      const int e = m * kThreads + tid;
      if (e < L * P) {
        sX[e] = to_f32(sxs[m]);
        const int j = xdiv(e);
        if (j >= n0) rx[((size_t)bh * R + ring_slot(head, j, R)) * P + (e - j * P)] = sxs[m];
      }
    }
  }
  // Long windows (rare): further staging rounds, loads then stores.
  for (int q0 = kStageB * kThreads; q0 < totBV; q0 += kStageB * kThreads) {
#pragma unroll
    for (int m = 0; m < kStageB; ++m) {
      const int q = q0 + m * kThreads + tid;
      if (q < totBV) { const int j = q / NV; vb[m] = ldv<Tin>(brow(j) + (q - j * NV) * VE); }
    }
#pragma unroll
    for (int m = 0; m < kStageB; ++m) {
      const int q = q0 + m * kThreads + tid;
      if (q < totBV) {
        st_lds_f32(sB + q * VE, vb[m]);
        const int j = q / NV;
        if (keepB && j >= n0)
          *reinterpret_cast<VT*>(rB + (((size_t)b * G + g) * R + ring_slot(head, j, R)) * N +
                                 (q - j * NV) * VE) = vb[m];
      }
    }
  }
  if (xvec) {
    for (int q0 = kStageX * kThreads; q0 < totXV; q0 += kStageX * kThreads) {
#pragma unroll
      for (int m = 0; m < kStageX; ++m) {
        const int q = q0 + m * kThreads + tid;
        if (q < totXV) { const int j = xdiv(q); vx[m] = ldv<Tin>(xrow(j) + (q - j * PV) * VE); }
      }
#pragma unroll
      for (int m = 0; m < kStageX; ++m) {
        const int q = q0 + m * kThreads + tid;
        if (q < totXV) {
          st_lds_f32(sX + q * VE, vx[m]);
          const int j = xdiv(q);
          if (j >= n0)
            *reinterpret_cast<VT*>(rx + ((size_t)bh * R + ring_slot(head, j, R)) * P +
                                   (q - j * PV) * VE) = vx[m];
        }
      }
    }
  } else {
    for (int e0 = kStageS * kThreads; e0 < L * P; e0 += kStageS * kThreads) {
#pragma unroll
      for (int m = 0; m < kStageS; ++m) {
        const int e = e0 + m * kThreads + tid;
        if (e < L * P) { const int j = xdiv(e); sxs[m] = xrow(j)[e - j * P]; }
      }
#pragma unroll
      for (int m = 0; m < kStageS; ++m) {
        const int e = e0 + m * kThreads + tid;
        if (e < L * P) {
          sX[e] = to_f32(sxs[m]);
          const int j = xdiv(e);
          if (j >= n0) rx[((size_t)bh * R + ring_slot(head, j, R)) * P + (e - j * P)] = sxs[m];
        }
      }
    }
  }

  // Log-decay scan in wavefront 0: lam_i(j) = sum_{j < m <= t_i} l_m, tree-summed.
  if (wave == 0) {
#pragma unroll
    for (int i = 0; i < NTMAX; ++i) {
      if (i >= nt) break;
      const int ti = n0 + i;
      const float u = lane <= ti ? lj : 0.f;
      const float lam = wave_suffix_excl(u, lane);
      if (lane < L) sCF[i * R + lane] = lane <= ti ? expf(lam) * dtj : 0.f;
      if (lane == 0) sDC[i] = expf(lam + u);
    }
    if (lane >= n0 && lane < L)  // the new tokens' (dt, l) into the ring
      a.ring_dl[(size_t)bh * R + ring_slot(head, lane, R)] = make_float2(dtj, lj);
  }
  __syncthreads();

  // 3. Wavefront w takes the window entries j = w (mod 4) of every output i:
  // w_ij = coef_ij (B_j . C_i), and its share of sum_j w_ij x_j, row p on lane p mod 64.
  constexpr int kRowsPerLane = kMaxP / 64;
  for (int i = 0; i < nt; ++i) {
    const int ti = n0 + i;
    float share[kRowsPerLane] = {};
    for (int j = wave; j <= ti; j += kWaves) {
      float part = 0.f;
#pragma unroll
      for (int n = lane; n < N; n += 64) part = fmaf(sB[j * N + n], sC[i * N + n], part);
      const float w = sCF[i * R + j] * wave_sum(part);
#pragma unroll
      for (int r = 0; r < kRowsPerLane; ++r)
        if (r * 64 + lane < P) share[r] = fmaf(w, sX[j * P + r * 64 + lane], share[r]);
    }
#pragma unroll
    for (int r = 0; r < kRowsPerLane; ++r)
      if (r * 64 + lane < P) sRing[(wave * NTMAX + i) * P + r * 64 + lane] = share[r];
  }
  __syncthreads();

  // 4. Consume the tile: per pass a 16-byte fragment dot C_i, reduce-scattered
  // over the row's lanes so that each writer lane finishes one row.
  using RS = RowScatter<TPR>;
  for (int base = 0; base < P; base += RPP * kMaxPass) {
    if (base > 0) load_chunk(base);
#pragma unroll
    for (int i = 0; i < NTMAX; ++i) {
      if (i >= nt) break;
      float cv[VEC];
#pragma unroll
      for (int v = 0; v < VEC; ++v) cv[v] = sC[i * N + col * VEC + v];
      float part[kMaxPass];
#pragma unroll
      for (int k = 0; k < kMaxPass; ++k) {
        float acc = 0.f;
#pragma unroll
        for (int v = 0; v < VEC; ++v) acc = fmaf(fr[k].get(v), cv[v], acc);
        part[k] = acc;
      }
      int kbase;
      RS::run(part, col, kbase);
      if ((col & RS::WMASK) == 0) {
#pragma unroll
        for (int m = 0; m < RS::NOUT; ++m) {
          const int row = base + (kbase + m) * RPP + rsub;
          if (row < P) {
            const float ring = (sRing[i * P + row] + sRing[(NTMAX + i) * P + row]) +
                               (sRing[(2 * NTMAX + i) * P + row] + sRing[(3 * NTMAX + i) * P + row]);
            a.y[((size_t)(b * nt + i) * H + h) * P + row] = fmaf(sDC[i], part[m], ring);
          }
        }
      }
    }
  }

  if (tid == 0) a.ptr[bh] = make_int4(head, L, a.set_tent ? nt : pt.z, 0);
}

template <int N, typename Tin, bool LOW, int NTMAX>
static hipError_t launch_one(const ReplayArgs& a, int batch, hipStream_t s) {
  const size_t lds = (size_t)ReplayLds(a.R, a.P, N, NTMAX).total * sizeof(float);
  auto kern = replay_kernel<N, Tin, LOW, NTMAX>;
  if (lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)((size_t)batch * a.H)), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

template <int N, typename Tin, bool LOW>
static hipError_t launch_nt(const ReplayArgs& a, int batch, hipStream_t s) {
  return a.nt == 1 ? launch_one<N, Tin, LOW, 1>(a, batch, s)
                   : launch_one<N, Tin, LOW, kMaxNew>(a, batch, s);
}

template <int N>
static hipError_t launch_n(const ReplayArgs& a, int batch, bool bf16_in, bool low, hipStream_t s) {
  if (bf16_in) return low ? launch_nt<N, bf16_t, true>(a, batch, s) : launch_nt<N, bf16_t, false>(a, batch, s);
  return low ? launch_nt<N, float, true>(a, batch, s) : launch_nt<N, float, false>(a, batch, s);
}

hipError_t launch_replay(const ReplayArgs& a, int batch, int N, bool bf16_in, bool low_copy,
                         hipStream_t s) {
  switch (N) {
    case 16: return launch_n<16>(a, batch, bf16_in, low_copy, s);
    case 32: return launch_n<32>(a, batch, bf16_in, low_copy, s);
    case 64: return launch_n<64>(a, batch, bf16_in, low_copy, s);
    case 128: return launch_n<128>(a, batch, bf16_in, low_copy, s);
    case 256: return launch_n<256>(a, batch, bf16_in, low_copy, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace rss

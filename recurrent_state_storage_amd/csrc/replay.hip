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
// One workgroup per (sequence, head):
//   1. issue the 16-byte loads of the checkpoint tile (the only large read);
//   2. while they fly: C_i into LDS, the window's (dt, l) pairs, the dot
//      products B_j . C_i (one wavefront per entry), the coefficients
//      exp(lam) dt (B.C) and the sums sum_j w_ij x_j, all in LDS; append the
//      new tokens to the ring;
//   3. consume the tile: per row a 16-byte fragment dot C_i, a butterfly over
//      the lanes of the row, and y = exp(Lam) * dot + ring part.
// The checkpoint tile is read exactly once per call for all nt outputs.
#include <type_traits>

#include "device.h"
#include "launch.h"

namespace rss {

template <int N, typename Tin, bool LOW, int NTMAX>
__global__ __launch_bounds__(kThreads) void replay_kernel(ReplayArgs a) {
  using Geo = TileGeom<N, LOW>;
  constexpr int VEC = Geo::VEC, TPR = Geo::TPR, RPP = Geo::RPP;
  constexpr int EPL = N >= 64 ? N / 64 : 1;
  using TileT = typename std::conditional<LOW, bf16_t, float>::type;

  __shared__ __align__(16) float sC[NTMAX][N];
  __shared__ float sl[kMaxRing];
  __shared__ float sdt[kMaxRing];
  __shared__ float sdot[NTMAX][kMaxRing];
  __shared__ float sw[NTMAX][kMaxRing];
  __shared__ float sdc[NTMAX];
  __shared__ float sring[NTMAX][kMaxP];

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

  const Tin* xin = static_cast<const Tin*>(a.x);
  const Tin* Bin = static_cast<const Tin*>(a.B);
  const Tin* Cin = static_cast<const Tin*>(a.C);
  Tin* rx = static_cast<Tin*>(a.ring_x);
  Tin* rB = static_cast<Tin*>(a.ring_B);

  // 1. Checkpoint tile: first chunk of rows into registers.
  const int col = tid % TPR, rsub = tid / TPR;
  const TileT* tile = static_cast<const TileT*>(LOW ? a.ckpt_lo : static_cast<const void*>(a.ckpt))
                      + (size_t)bh * P * N;
  Frag<LOW> fr[kMaxPass];
  auto load_chunk = [&](int base) {
#pragma unroll
    for (int k = 0; k < kMaxPass; ++k) {
      const int row = base + k * RPP + rsub;
      if (row < P) fr[k].v = ld16(tile + (size_t)row * N + col * VEC);
      else fr[k].v = decltype(fr[k].v){};
    }
  };
  load_chunk(0);

  // 2a. C of the new tokens, and (dt, l) of every window entry.
  const float Ah = a.A[h];
  for (int e = tid; e < nt * N; e += kThreads) {
    const int i = e / N, n = e - i * N;
    sC[i][n] = to_f32(Cin[((size_t)(b * nt + i) * G + g) * N + n]);
  }
  if (tid < L) {
    float dtj, lj;
    if (tid < n0) {
      const float2 v = a.ring_dl[(size_t)bh * R + ring_slot(head, tid, R)];
      dtj = v.x;
      lj = v.y;
    } else {
      dtj = a.dt[(size_t)(b * nt + (tid - n0)) * H + h];
      lj = dtj * Ah;
    }
    sdt[tid] = dtj;
    sl[tid] = lj;
  }
  __syncthreads();

  // 2b. B_j . C_i, one wavefront per window entry.
  for (int j = wave; j < L; j += kWaves) {
    const Tin* Bj = j < n0 ? rB + (((size_t)b * G + g) * R + ring_slot(head, j, R)) * N
                           : Bin + ((size_t)(b * nt + (j - n0)) * G + g) * N;
    float bv[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const int n = lane * EPL + e;
      bv[e] = n < N ? to_f32(Bj[n]) : 0.f;
    }
#pragma unroll
    for (int i = 0; i < NTMAX; ++i) {
      if (i >= nt) break;
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const int n = lane * EPL + e;
        if (n < N) part = fmaf(bv[e], sC[i][n], part);
      }
      part = wave_sum(part);
      if (lane == 0) sdot[i][j] = part;
    }
  }
  __syncthreads();

  // 2c. Coefficients w_ij = exp(lam_i(j)) dt_j (B_j.C_i) and exp(Lam_i), with
  // the log-decays summed from the newest entry backwards.
  for (int e = tid; e < nt * L; e += kThreads) {
    const int i = e / L, j = e - i * L;
    const int ti = n0 + i;
    float w = 0.f;
    if (j <= ti) {
      float lam = 0.f;
      for (int m = ti; m > j; --m) lam += sl[m];
      w = expf(lam) * sdt[j] * sdot[i][j];
    }
    sw[i][j] = w;
  }
  if (tid >= kThreads - NTMAX && tid - (kThreads - NTMAX) < nt) {
    const int i = tid - (kThreads - NTMAX);
    float lam = 0.f;
    for (int m = n0 + i; m >= 0; --m) lam += sl[m];
    sdc[i] = expf(lam);
  }
  __syncthreads();

  // 2d. Ring part sum_j w_ij x_j[p]; append the new tokens to the ring.
  for (int e = tid; e < nt * P; e += kThreads) {
    const int i = e / P, p = e - i * P;
    const int ti = n0 + i;
    float acc = 0.f;
    for (int j = 0; j <= ti; ++j) {
      const float xv = j < n0 ? to_f32(rx[((size_t)bh * R + ring_slot(head, j, R)) * P + p])
                              : to_f32(xin[((size_t)(b * nt + (j - n0)) * H + h) * P + p]);
      acc = fmaf(sw[i][j], xv, acc);
    }
    sring[i][p] = acc;
    rx[((size_t)bh * R + ring_slot(head, ti, R)) * P + p] = xin[((size_t)(b * nt + i) * H + h) * P + p];
  }
  if (h == g * hpg) {  // the group's first head keeps the group's B
    for (int e = tid; e < nt * N; e += kThreads) {
      const int i = e / N, n = e - i * N;
      rB[(((size_t)b * G + g) * R + ring_slot(head, n0 + i, R)) * N + n] =
          Bin[((size_t)(b * nt + i) * G + g) * N + n];
    }
  }
  if (tid < nt)
    a.ring_dl[(size_t)bh * R + ring_slot(head, n0 + tid, R)] = make_float2(sdt[n0 + tid], sl[n0 + tid]);
  __syncthreads();

  // 3. Consume the tile.
  for (int base = 0; base < P; base += RPP * kMaxPass) {
    if (base > 0) load_chunk(base);
#pragma unroll
    for (int k = 0; k < kMaxPass; ++k) {
      if (base + k * RPP >= P) break;
      const int row = base + k * RPP + rsub;
#pragma unroll
      for (int i = 0; i < NTMAX; ++i) {
        if (i >= nt) break;
        float part = 0.f;
#pragma unroll
        for (int v = 0; v < VEC; ++v) part = fmaf(fr[k].get(v), sC[i][col * VEC + v], part);
        part = row_sum<TPR>(part);
        if (col == 0 && row < P)
          a.y[((size_t)(b * nt + i) * H + h) * P + row] = fmaf(sdc[i], part, sring[i][row]);
      }
    }
  }

  if (tid == 0) a.ptr[bh] = make_int4(head, L, a.set_tent ? nt : pt.z, 0);
}

template <int N, typename Tin, bool LOW>
static hipError_t launch_nt(const ReplayArgs& a, int batch, hipStream_t s) {
  const dim3 grid((unsigned)((size_t)batch * a.H)), block(kThreads);
  if (a.nt == 1)
    hipLaunchKernelGGL((replay_kernel<N, Tin, LOW, 1>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((replay_kernel<N, Tin, LOW, kMaxNew>), grid, block, 0, s, a);
  return hipGetLastError();
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

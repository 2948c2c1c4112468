// Gated DeltaNet decode: eager baseline and replay from checkpoint + ring.
//
// P1 ("La fiche qu'on réécrit à chaque token") says GDN adds a delta-rule
// correction but writes its update in the same form as Mamba-2; P2 ("Des
// chiffres qui parlent d'eux-mêmes") says the method runs for Gated DeltaNet.
// Per head, with a d_v x d_k state S, scalar gate alpha_t and rate beta_t:
//
//   u_t = beta_t (v_t - alpha_t S_{t-1} k_t)
//   S_t = alpha_t S_{t-1} + u_t k_t^T          (the gated delta rule)
//   o_t = S_t q_t = alpha_t S_{t-1} q_t + (k_t . q_t) u_t
//
// i.e. the Mamba-2 step with x -> u, B -> k, dt -> 1 and log-decay log alpha.
// The ring keeps (k_j, u_j, log alpha_j) (with dt = 1 stored beside it), so the
// Mamba-2 flush kernel folds a GDN window unchanged. Replay forms
//   S_{t-1} z = exp(Lam) S_c z + sum_j exp(lam_j) (k_j . z) u_j   for z = k_t, q_t
// in one pass over the checkpoint tile (two row dots per row), with
// lam_j = sum of log alpha over the window entries after j, Lam over all of them.
//
// Kimi Delta Attention (KDA, named beside GDN on P1 "Des couches rapides sur le
// papier") is the same rule with one gate per key channel:
//   S_t = S_{t-1} Diag(alpha_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
//   u_t = beta_t (v_t - S_{t-1} (alpha_t * k_t)),  o_t = S_{t-1} (alpha_t * q_t) + (k_t . q_t) u_t
// The decays become per-channel suffix sums lam_j[n] (entries after j, the new
// token's gate included) and Lam[n]: replay dots the tile rows with
// exp(Lam) * k_t and exp(Lam) * q_t, and the ring term uses the channel-scaled
// keys k_j * exp(lam_j). The ring keeps log alpha_j as a row per entry.
#include "device.h"
#include "fold.h"
#include "launch.h"
#include "lds.h"

namespace rss {


template <int N, int MP, bool KDA, bool FOLD>
__global__ __launch_bounds__(kThreads) void gdn_replay_kernel(GdnArgs a) {
  using Geo = TileGeom<N, false>;
  constexpr int TPR = Geo::TPR, RPP = Geo::RPP;
  using Rows = RowMap<TPR, MP>;
  constexpr int NV = N / 4;
  constexpr int EPL = N >= 64 ? N / 64 : 1;
  using RS = RowScatter<TPR>;
  static_assert(MP % 8 == 0, "passes come in groups of 8");

  extern __shared__ __align__(16) float lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = a.H, P = a.P, R = a.R;
  const int bh = xcd_tile(blockIdx.x, gridDim.x, a.P * N * 4);
  const int b = bh / H, h = bh - b * H;

  float* tile = a.ckpt + (size_t)bh * P * N;
  const int col = tid % TPR;
  const Rows rows(tid);
  Frag<false> fr[MP];
  auto load_chunk = [&](int base) {
#pragma unroll
    for (int k = 0; k < MP; ++k) {
      const int row = rows.row(base, k);
      if (row < P) fr[k].v = ld16(tile + row * N + col * 4);
      else fr[k].v = float4{};
    }
  };
  load_chunk(0);
  // KDA: the gates are per channel and enter through the scaled vectors below,
  // so the scalar gate of the shared formulas is 1.
  const float alpha = KDA ? 1.f : a.alpha[bh], beta = a.beta[bh];

  const int4 pt = a.ptr[bh];
  const int head = pt.x, n0 = pt.y;
  const int L = n0 + 1;
  float* oout = a.o + (size_t)bh * P;
  if (head < 0 || head >= R || n0 < 0 || L > R) {  // ring full (no flush), or corrupt pointers
    if (tid == 0) atomicOr(a.err, kDevRingOverflow);
    for (int p = tid; p < P; p += kThreads) oout[p] = __builtin_nanf("");
    return;
  }
  // Fused fold: the token that fills the window also folds it (the new entry
  // included) into the tile already in registers and writes the tile, with the
  // flush's coefficients in the flush's order, so the result is bitwise the
  // separate flush's.
  const bool do_fold = FOLD && L >= a.fold_min_len && pt.z == 0;

  using Fold = MfmaFold<N, TPR, 4, MP>;
  const GdnLds lay(R, P, N, KDA, FOLD ? Fold::BUF : 0);
  float* sK = lds + lay.oK;
  float* sU = lds + lay.oU;
  float* sQ = lds + lay.oQ;
  float* sCF = lds + lay.oCF;
  float* sS = lds + lay.oS;
  float* sG = lds + lay.oG;
  float* sD = lds + lay.oD;
  float* sFC = lds + lay.oFC;
  // slot-major ring (slot s of every head of a sequence contiguous): this
  // head's rows at slot 0, then slot strides H P (u), H N (k, log-gates), H
  const int sus = H * P, sks = H * N;
  float* rg = KDA ? a.ring_g + (size_t)b * R * sks + h * N : nullptr;
  float* ru = a.ring_u + (size_t)b * R * sus + h * P;
  float* rk = a.ring_k + (size_t)b * R * sks + h * N;
  float2* rdl = a.ring_dl + (size_t)b * R * H + h;
  const float* kin = a.k + (size_t)bh * N;
  const float* qin = a.q + (size_t)bh * N;
  const float* vin = a.v + (size_t)bh * P;

  // Window k rows (ring, then k_t as row n0), u rows and v_t straight into
  // LDS; q_t and the log-decays through registers. The step's own inputs are
  // read once, so they go non-temporal; ring rows stay cached.
  const int totK = L * NV;
  for (int q0 = wave * 64; q0 < totK; q0 += kThreads) {
    const int q = q0 + lane;
    if (q < totK) {
      const int j = q / NV;
      if (j < n0) dma16(rk + ring_slot(head, j, R) * sks + (q - j * NV) * 4, sK + q0 * 4);
      else dma16_nt(kin + (q - j * NV) * 4, sK + q0 * 4);
    }
  }
  const bool uvec = (P % 4) == 0;
  float* sV = lds + lay.oV;
  if (uvec) {  // v_t, read by the writer lanes at the end of each tile chunk
    for (int q0 = wave * 64; q0 < P / 4; q0 += kThreads)
      if (q0 + lane < P / 4) dma16_nt(vin + (q0 + lane) * 4, sV + q0 * 4);
  } else {
    for (int p = tid; p < P; p += kThreads) sV[p] = __builtin_nontemporal_load(vin + p);
  }
  if (uvec) {
    const int PV = P / 4, totU = n0 * PV;
    for (int q0 = wave * 64; q0 < totU; q0 += kThreads) {
      const int q = q0 + lane;
      if (q < totU) {
        const int j = q / PV;
        dma16(ru + ring_slot(head, j, R) * sus + (q - j * PV) * 4, sU + q0 * 4);
      }
    }
  }
  if constexpr (KDA) {  // the committed entries' log-gate rows
    const int totG = n0 * NV;
    for (int q0 = wave * 64; q0 < totG; q0 += kThreads) {
      const int q = q0 + lane;
      if (q < totG) {
        const int j = q / NV;
        dma16(rg + ring_slot(head, j, R) * sks + (q - j * NV) * 4, sG + q0 * 4);
      }
    }
  }
  float qv = 0.f, av = 1.f;
  if (tid < N) qv = __builtin_nontemporal_load(qin + tid);
  if (KDA && tid < N) av = __builtin_nontemporal_load(a.alpha + (size_t)bh * N + tid);
  float2 dl = make_float2(0.f, 0.f);
  if (!KDA && tid < n0) dl = rdl[ring_slot(head, tid, R) * H];
  if (!uvec) {
    for (int e = tid; e < n0 * P; e += kThreads) {
      const int j = e / P;
      sU[e] = ru[ring_slot(head, j, R) * sus + (e - j * P)];
    }
  }
  if (tid < N) sQ[tid] = qv;
  if (!KDA && wave == 0) {  // exp(lam_j) over the committed entries, and exp(Lam)
    const float u = lane < n0 ? dl.y : 0.f;
    const float lam = wave_suffix_excl(u, lane);
    if (lane < n0) sCF[lane] = expf(lam);
    if (lane == 0) sCF[R] = expf(lam + u);
    if (FOLD) {  // the fold's coefficients over all L entries, as the flush forms them
      const float g = lane < n0 ? dl.y : logf(alpha);
      const float u2 = lane < L ? g : 0.f;
      const float lam2 = wave_suffix_excl(u2, lane);
      if (lane < lay.RS) sFC[lane] = lane < L ? expf(lam2) * 1.f : 0.f;
      if (lane == 0) sFC[lay.RS] = expf(lam2 + u2);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  if (FOLD && do_fold) {  // the fold reads entries in groups of four: rows past the window are zero
    const int F4 = align4(L);
    for (int q = tid; q < (F4 - L) * N; q += kThreads) sK[L * N + q] = 0.f;
    for (int q = tid; q < (F4 - L) * P; q += kThreads) sU[L * P + q] = 0.f;
  }
  __syncthreads();
  // the new entry's (1, log alpha) after the wait: a store before it would be waited for too
  if (!KDA && tid == 0) rdl[ring_slot(head, n0, R) * H] = make_float2(1.f, logf(alpha));
  if constexpr (KDA) {
    // Channel n (one thread each): lam_j[n] from the newest entry back, the new
    // token's gate included; scale the committed keys in place; exp(Lam[n]).
    if (tid < N) {
      const float gt = logf(av);
      rg[ring_slot(head, n0, R) * sks + tid] = gt;
      float acc = gt;
      for (int j = n0 - 1; j >= 0; --j) {
        sK[j * N + tid] *= expf(acc);
        acc += sG[j * N + tid];
      }
      sD[tid] = expf(acc);
    }
    if (tid < n0) sCF[tid] = 1.f;
    if (tid == 0) sCF[R] = 1.f;
    __syncthreads();
  }

  // k_t . q_t, and per wavefront its share of sum_j exp(lam_j)(k_j . z) u_j.
  if (wave == 0) {
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const int n = lane * EPL + e;
      if (n < N) part = fmaf(sK[n0 * N + n], sQ[n], part);
    }
    part = wave_sum(part);
    if (lane == 0) sCF[R + 1] = part;
  }
  {
    constexpr int kRowsPerLane = kMaxP / 64;
    float shk[kRowsPerLane] = {}, shq[kRowsPerLane] = {};
    for (int j = wave; j < n0; j += kWaves) {
      float pk = 0.f, pq = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const int n = lane * EPL + e;
        if (n < N) {
          const float kj = sK[j * N + n];
          pk = fmaf(kj, sK[n0 * N + n], pk);
          pq = fmaf(kj, sQ[n], pq);
        }
      }
      const float c = sCF[j];
      const float wk = c * wave_sum(pk), wq = c * wave_sum(pq);
#pragma unroll
      for (int r = 0; r < kRowsPerLane; ++r) {
        if (r * 64 + lane < P) {
          const float uj = sU[j * P + r * 64 + lane];
          shk[r] = fmaf(wk, uj, shk[r]);
          shq[r] = fmaf(wq, uj, shq[r]);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < kRowsPerLane; ++r) {
      if (r * 64 + lane < P) {
        sS[(wave * 2 + 0) * P + r * 64 + lane] = shk[r];
        sS[(wave * 2 + 1) * P + r * 64 + lane] = shq[r];
      }
    }
  }
  // k_t into the ring (every head owns its k)
  for (int q = tid; q < NV; q += kThreads)
    *reinterpret_cast<float4*>(rk + ring_slot(head, n0, R) * sks + q * 4) =
        *reinterpret_cast<const float4*>(sK + n0 * N + q * 4);
  __syncthreads();

  const float D = sCF[R], kq = sCF[R + 1];
  float kc[4], qc[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const float dn = KDA ? sD[col * 4 + v] : 1.f;
    kc[v] = dn * sK[n0 * N + col * 4 + v];
    qc[v] = dn * sQ[col * 4 + v];
  }
  float* unew = ru + ring_slot(head, n0, R) * sus;
  for (int base = 0; base < P; base += RPP * MP) {
    if (base > 0) load_chunk(base);
#pragma unroll
    for (int g8 = 0; g8 < MP; g8 += 8) {
      if (rows.wave_row(base, g8, wave) >= P) break;
      float pk[8], pq[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float4 s = fr[g8 + k].v;
        pk[k] = fmaf(s.w, kc[3], fmaf(s.z, kc[2], fmaf(s.y, kc[1], s.x * kc[0])));
        pq[k] = fmaf(s.w, qc[3], fmaf(s.z, qc[2], fmaf(s.y, qc[1], s.x * qc[0])));
      }
      int kb1, kb2;
      RS::run(pk, col, kb1);
      RS::run(pq, col, kb2);
      if ((col & RS::WMASK) == 0) {
#pragma unroll
        for (int m = 0; m < RS::NOUT; ++m) {
          const int row = rows.row(base, g8 + kb1 + m);
          if (row < P) {
            const float rk_ = (sS[0 * P + row] + sS[2 * P + row]) + (sS[4 * P + row] + sS[6 * P + row]);
            const float rq_ = (sS[1 * P + row] + sS[3 * P + row]) + (sS[5 * P + row] + sS[7 * P + row]);
            const float Sk = fmaf(D, pk[m], rk_);
            const float Sq = fmaf(D, pq[m], rq_);
            const float u = beta * (sV[row] - alpha * Sk);
            unew[row] = u;
            if (FOLD) sU[n0 * P + row] = u;
            oout[row] = fmaf(alpha, Sq, kq * u);
          }
        }
      }
    }
    if constexpr (FOLD) {
      __syncthreads();   // this chunk's new u rows are in LDS (do_fold is uniform)
      if (do_fold && rows.wave_row(base, 0, wave) < P) {
        // S <- D S + sum_j u_j outer (c_j k_j) on the matrix cores (the flush's
        // operands and order); KDA: D per key channel, and the keys in LDS are
        // already decayed per channel (c_j = 1).
        float Dc[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) Dc[v] = KDA ? sD[col * 4 + v] : sFC[lay.RS];
        Fold::run(rows.wave_row(base, 0, wave), P, align4(L), lds + lay.oW + wave * Fold::BUF, lane,
                  col, [&](int j, int c) { return KDA ? sK[j * N + c] : sFC[j] * sK[j * N + c]; },
                  [&](int j, int p) { return sU[j * P + p]; },
                  [&](int k, const float (&d)[4]) {
                    const float4 s = fr[k].v;
                    const int row = rows.row(base, k);
                    if (row < P)
                      st16(tile + row * N + col * 4,
                           make_float4(fmaf(Dc[0], s.x, d[0]), fmaf(Dc[1], s.y, d[1]),
                                       fmaf(Dc[2], s.z, d[2]), fmaf(Dc[3], s.w, d[3])));
                  });
      }
    }
  }
  if (tid == 0) {
    if (do_fold) a.ptr[bh] = make_int4(ring_slot(head, L, R), 0, 0, 0);
    else a.ptr[bh] = make_int4(head, L, 0, 0);
  }
}

// Eager gated delta rule: S <- alpha S + u k^T with u = beta (v - alpha S k),
// o = alpha (S q) + (k . q) u, on the state in place.
template <int N, int MP, bool KDA>
__global__ __launch_bounds__(kThreads) void gdn_eager_kernel(GdnEagerArgs a) {
  using Geo = TileGeom<N, false>;
  constexpr int TPR = Geo::TPR, RPP = Geo::RPP;
  using Rows = RowMap<TPR, MP>;
  constexpr int EPL = N >= 64 ? N / 64 : 1;
  using RS = RowScatter<TPR>;

  extern __shared__ __align__(16) float lds[];  // k [N], q [N], u [P], k.q, KDA gates [N]
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int P = a.P;
  const int bh = xcd_tile(blockIdx.x, gridDim.x, a.P * N * 4);
  float* tile = a.S + (size_t)bh * P * N;
  const int col = tid % TPR;
  const Rows rows(tid);
  Frag<false> fr[MP];
  auto load_chunk = [&](int base) {
#pragma unroll
    for (int k = 0; k < MP; ++k) {
      const int row = rows.row(base, k);
      if (row < P) fr[k].v = ld16(tile + row * N + col * 4);
      else fr[k].v = float4{};
    }
  };
  load_chunk(0);
  const float alpha = KDA ? 1.f : a.alpha[bh], beta = a.beta[bh];
  float* sk = lds;
  float* sq = lds + N;
  float* su = lds + 2 * N;
  float* skq = su + P;
  float* sa = skq + 1;
  for (int n = tid; n < N; n += kThreads) {
    sk[n] = a.k[(size_t)bh * N + n];
    sq[n] = a.q[(size_t)bh * N + n];
    if (KDA) sa[n] = a.alpha[(size_t)bh * N + n];
  }
  __syncthreads();
  if (wave == 0) {
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const int n = lane * EPL + e;
      if (n < N) part = fmaf(sk[n], sq[n], part);
    }
    part = wave_sum(part);
    if (lane == 0) *skq = part;
  }
  // Row dots use S (alpha * k) and S (alpha * q); the update decays column c by
  // its gate ac[c] (KDA) or every column by alpha (GDN: the gate is folded below).
  float kc[4], qc[4], kr[4], ac[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const float g = KDA ? sa[col * 4 + v] : 1.f;
    kr[v] = sk[col * 4 + v];
    kc[v] = g * kr[v];
    qc[v] = g * sq[col * 4 + v];
    ac[v] = KDA ? g : alpha;
  }
  const float* vin = a.v + (size_t)bh * P;
  float* oout = a.o + (size_t)bh * P;
  for (int base = 0; base < P; base += RPP * MP) {
    if (base > 0) load_chunk(base);
    __syncthreads();  // k . q ready; earlier readers of su are done
    const float kq = *skq;
#pragma unroll
    for (int g8 = 0; g8 < MP; g8 += 8) {
      if (rows.wave_row(base, g8, wave) >= P) break;
      float pk[8], pq[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float4 s = fr[g8 + k].v;
        pk[k] = fmaf(s.w, kc[3], fmaf(s.z, kc[2], fmaf(s.y, kc[1], s.x * kc[0])));
        pq[k] = fmaf(s.w, qc[3], fmaf(s.z, qc[2], fmaf(s.y, qc[1], s.x * qc[0])));
      }
      int kb1, kb2;
      RS::run(pk, col, kb1);
      RS::run(pq, col, kb2);
      if ((col & RS::WMASK) == 0) {
#pragma unroll
        for (int m = 0; m < RS::NOUT; ++m) {
          const int row = rows.row(base, g8 + kb1 + m);
          if (row < P) {
            const float u = beta * (vin[row] - alpha * pk[m]);
            su[row] = u;
            oout[row] = fmaf(alpha, pq[m], kq * u);
          }
        }
      }
    }
    __syncthreads();  // u of every row in this chunk is in LDS
#pragma unroll
    for (int k = 0; k < MP; ++k) {
      const int row = rows.row(base, k);
      if (row < P) {
        const float u = su[row];
        float4 s = fr[k].v;
        s.x = fmaf(u, kr[0], ac[0] * s.x);
        s.y = fmaf(u, kr[1], ac[1] * s.y);
        s.z = fmaf(u, kr[2], ac[2] * s.z);
        s.w = fmaf(u, kr[3], ac[3] * s.w);
        st16(tile + row * N + col * 4, s);
      }
    }
  }
}

template <int N, int MP, bool KDA, bool FOLD>
static hipError_t gdn_replay_one(const GdnArgs& a, int batch, hipStream_t s) {
  const size_t lds =
      (size_t)GdnLds(a.R, a.P, N, KDA, FOLD ? fold_buf_floats(N, 4, MP) : 0).total * sizeof(float);
  auto kern = gdn_replay_kernel<N, MP, KDA, FOLD>;
  if (lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)((size_t)batch * a.H)), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

// A folding launch holds 8 passes per chunk: the fold's accumulators need the
// registers the second half of a 16-pass chunk would take.
template <int N, bool KDA, bool FOLD>
static hipError_t gdn_replay_f(const GdnArgs& a, int batch, hipStream_t s) {
  return gdn_passes(a.P, N) == 16 && !FOLD ? gdn_replay_one<N, 16, KDA, FOLD>(a, batch, s)
                                           : gdn_replay_one<N, 8, KDA, FOLD>(a, batch, s);
}

template <int N, bool KDA>
static hipError_t gdn_replay_n(const GdnArgs& a, int batch, hipStream_t s) {
  return a.fold_min_len > 0 ? gdn_replay_f<N, KDA, true>(a, batch, s) : gdn_replay_f<N, KDA, false>(a, batch, s);
}

template <int N>
static hipError_t gdn_replay_k(const GdnArgs& a, int batch, bool kda, hipStream_t s) {
  return kda ? gdn_replay_n<N, true>(a, batch, s) : gdn_replay_n<N, false>(a, batch, s);
}

hipError_t launch_gdn_replay(const GdnArgs& a, int batch, int N, bool kda, hipStream_t s) {
  switch (N) {
    case 16: return gdn_replay_k<16>(a, batch, kda, s);
    case 32: return gdn_replay_k<32>(a, batch, kda, s);
    case 64: return gdn_replay_k<64>(a, batch, kda, s);
    case 128: return gdn_replay_k<128>(a, batch, kda, s);
    case 256: return gdn_replay_k<256>(a, batch, kda, s);
    default: return hipErrorInvalidValue;
  }
}

template <int N, int MP, bool KDA>
static hipError_t gdn_eager_one(const GdnEagerArgs& a, int batch, hipStream_t s) {
  const size_t lds = (size_t)(2 * N + a.P + 1 + (KDA ? N : 0)) * sizeof(float);
  hipLaunchKernelGGL((gdn_eager_kernel<N, MP, KDA>), dim3((unsigned)((size_t)batch * a.H)),
                     dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

template <int N, bool KDA>
static hipError_t gdn_eager_n(const GdnEagerArgs& a, int batch, hipStream_t s) {
  return gdn_passes(a.P, N) == 16 ? gdn_eager_one<N, 16, KDA>(a, batch, s)
                                  : gdn_eager_one<N, 8, KDA>(a, batch, s);
}

template <int N>
static hipError_t gdn_eager_k(const GdnEagerArgs& a, int batch, bool kda, hipStream_t s) {
  return kda ? gdn_eager_n<N, true>(a, batch, s) : gdn_eager_n<N, false>(a, batch, s);
}

hipError_t launch_gdn_eager(const GdnEagerArgs& a, int batch, int N, bool kda, hipStream_t s) {
  switch (N) {
    case 16: return gdn_eager_k<16>(a, batch, kda, s);
    case 32: return gdn_eager_k<32>(a, batch, kda, s);
    case 64: return gdn_eager_k<64>(a, batch, kda, s);
    case 128: return gdn_eager_k<128>(a, batch, kda, s);
    case 256: return gdn_eager_k<256>(a, batch, kda, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace rss

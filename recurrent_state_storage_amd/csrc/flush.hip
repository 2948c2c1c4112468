// Checkpoint fold (flush), state init and rollback kernels.
//
// Flush folds the window into the checkpoint once the buffer is full (P1,
// "Tenir le journal plutôt que le solde": the checkpoint is rewritten only when
// the buffer is full; P3, "Решение ReplaySSM": written rarely, once per window;
// P4's table: the checkpoint is written only when the buffer is emptied):
//
//   S_c <- exp(Lam) S_c + sum_{j<n} c_j outer(x_j, B_j),   c_j = exp(lam_j) dt_j
//   lam_j = sum_{m=j+1..n-1} l_m,   Lam = sum_{m=0..n-1} l_m
//
// This is the only kernel that writes a checkpoint. In dual-precision mode it
// also refreshes the bf16 read copy from the new fp32 master (P2, "Deux
// précisions pour le prix d'une"); the fold reads the master only. With a
// bf16-only checkpoint (the single low-precision checkpoint the dual mode is
// compared with) it folds from the bf16 values on the matrix cores (fold.h:
// with bf16 inputs c_j x_j enters as a bf16 hi/lo pair, 2^-18 relative) and
// stores the RNE-bf16 result: one rounding per window (P1, "Tenir le journal
// plutôt que le solde").
//
// With per-channel decays (Kimi Delta Attention) the scalars become vectors
// over the key channels n: S_c[:, n] <- exp(Lam[n]) S_c[:, n] + sum_j u_j
// k_j[n] exp(lam_j[n]), suffix sums taken per channel over the log-gate rows.
//
// Rollback (P2, "Un retour en arrière qui devient trivial") touches integers
// only: len -= n_drop, n_tent = 0.
#include <type_traits>

#include "device.h"
#include "fold.h"
#include "launch.h"
#include "lds.h"

namespace rss {

constexpr int kFlushStage = 2;  // 16-byte B loads per thread per staging round


// MF: the rank-n update runs on the matrix cores (fold.h); otherwise as fp32
// FMAs, one entry at a time in ascending order.
template <int N, typename Tin, int MODE, bool PCD, bool MF>
__global__ __launch_bounds__(kThreads) void flush_kernel(FlushArgs a) {
  constexpr bool DUAL = MODE == kCkptDual, B16 = MODE == kCkptBf16;
  using Geo = TileGeom<N, false>;
  constexpr int TPR = Geo::TPR, RPP = Geo::RPP;
  using Rows = RowMap<TPR, kMaxPass>;
  using Fold = MfmaFold<N, TPR, 4, kMaxPass>;
  constexpr int VE = V16<Tin>::VE;
  constexpr int NV = N / VE;
  using VT = typename V16<Tin>::T;

  extern __shared__ __align__(16) float lds[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = a.H, P = a.P, G = a.G, R = a.R;
  const int bh = xcd_tile(blockIdx.x, gridDim.x, a.P * N * (B16 ? 2 : 4));
  const int b = bh / H, h = bh - b * H;
  const int g = h / (H / G);
  const int4 pt = a.ptr[bh];
  const int head = pt.x, n = pt.y;
  const int th = a.min_len_dev ? a.min_len_dev[b] : a.min_len;
  if (n == 0 || n < th) return;
  if (head < 0 || head >= R || n < 0 || n > R) {  // corrupt pointers: never index with them
    if (tid == 0) atomicOr(a.err, kDevRingOverflow);
    return;
  }
  if (pt.z != 0) {  // tentative entries were never committed
    if (tid == 0) atomicOr(a.err, kDevUncommitted);
    return;
  }
  // A bf16-stored checkpoint with bf16 inputs folds on the bf16 matrix cores,
  // exactly as the decode that folds it in the same pass (fold.h).
  constexpr bool kB16Fold = MF && B16 && std::is_same<Tin, bf16_t>::value;
  const FlushLds lay(R, P, N, PCD, MF ? Fold::BUF : 0, kB16Fold ? fold_bt_elems(N, R) : 0);
  const int RS = lay.RS, LDB = lay.LDB, LDX = lay.LDX;
  const int F4 = align4(n);   // the matrix-core fold reads entries in groups of four
  float* sXT = lds + lay.oXT;
  float* sB = lds + lay.oB;
  float* sCF = lds + lay.oCF;
  float* sG = lds + lay.oG;
  float* sDc = lds + lay.oDc;
  const Tin* rx = static_cast<const Tin*>(a.ring_x);
  const Tin* rB = static_cast<const Tin*>(a.ring_B);
  // slot-major ring: slot s of every head (group) of a sequence is contiguous
  const Tin* rxh = rx + (size_t)b * R * H * P + h * P;
  const Tin* rBg = rB + (size_t)b * R * G * N + g * N;
  auto xrow = [&](int j) { return rxh + ring_slot(head, j, R) * (H * P); };
  auto brow = [&](int j) { return rBg + ring_slot(head, j, R) * (G * N); };

  // 1. Tile loads (the fp32 master, or the bf16 checkpoint widened to fp32).
  const int col = tid % TPR;
  const Rows rows(tid);
  float* tile = B16 ? nullptr : a.ckpt + (size_t)bh * P * N;
  bf16_t* tileb = B16 ? static_cast<bf16_t*>(a.ckpt_lo) + (size_t)bh * P * N : nullptr;
  Frag<false> fr[kMaxPass];
  auto ld_row = [&](int row) {
    if constexpr (B16) return ld8_bf16x4(tileb + (size_t)row * N + col * 4);
    else return ld16(tile + (size_t)row * N + col * 4);
  };
  auto load_chunk = [&](int base) {
#pragma unroll
    for (int k = 0; k < kMaxPass; ++k) {
      const int row = rows.row(base, k);
      if (row < P) fr[k].v = ld_row(row);
      else fr[k].v = float4{};
    }
  };
  load_chunk(0);

  // 2. Window B rows, x (transposed) and (dt, l), unpacked into LDS. The fold
  // is the last reader of these ring rows, so they are loaded non-temporal
  // (measured: dual-precision flush at batch 256 490 -> 478 us).
  float2 dl = make_float2(0.f, 0.f);
  if (!PCD && tid < n) dl = a.ring_dl[(size_t)b * R * H + ring_slot(head, tid, R) * H + h];
  if constexpr (PCD) {  // the window's per-channel log-decay rows
    const float* rg = a.ring_g + (size_t)b * R * H * N + h * N;
    for (int q = tid; q < n * (N / 4); q += kThreads) {
      const int j = q / (N / 4), c = q - j * (N / 4);
      *reinterpret_cast<float4*>(sG + j * N + c * 4) =
          *reinterpret_cast<const float4*>(rg + ring_slot(head, j, R) * (H * N) + c * 4);
    }
  }
  bf16_t* bt = reinterpret_cast<bf16_t*>(lds + lay.oBT);
  const int F16 = (n + 15) & ~15;
  if constexpr (kB16Fold) {
    // The bf16 fold's A operand straight from the ring: B rows transposed in
    // groups of 16 entries, bt[j / 16][c][j % 16] (zero for j >= n);
    // consecutive lanes take consecutive entries of one 8-column vector.
    for (int q = tid; q < F16 * NV; q += kThreads) {
      const int c8 = q / F16, j = q - c8 * F16;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (j < n) v = __builtin_bit_cast(u32x4, ldv_nt<Tin>(brow(j) + c8 * VE));
      bf16_t* dst = bt + ((j >> 4) * N + c8 * VE) * 16 + (j & 15);
#pragma unroll
      for (int e = 0; e < VE; ++e) dst[e * 16] = (bf16_t)((e & 1) ? v[e >> 1] >> 16 : v[e >> 1] & 0xffffu);
    }
  }
  const int totBV = kB16Fold ? 0 : n * NV;
  for (int q0 = 0; q0 < totBV; q0 += kFlushStage * kThreads) {
    VT vb[kFlushStage];
#pragma unroll
    for (int m = 0; m < kFlushStage; ++m) {
      const int q = q0 + m * kThreads + tid;
      if (q < totBV) { const int j = q / NV; vb[m] = ldv_nt<Tin>(brow(j) + (q - j * NV) * VE); }
    }
#pragma unroll
    for (int m = 0; m < kFlushStage; ++m) {
      const int q = q0 + m * kThreads + tid;
      if (q < totBV) { const int j = q / NV; st_lds_f32(sB + j * LDB + (q - j * NV) * VE, vb[m]); }
    }
  }
  if constexpr (MF) {
    // x one entry per row; the rows from n up to the next multiple of four
    // (read by the fold's last group of entries) are zero, in x and in B.
    if ((P % VE) == 0) {
      const int PV = P / VE;
      for (int q = tid; q < n * PV; q += kThreads) {
        const int j = q / PV, c = q - j * PV;
        st_lds_f32(sXT + j * LDX + c * VE, ldv_nt<Tin>(xrow(j) + c * VE));
      }
    } else {
      for (int q = tid; q < n * P; q += kThreads) {
        const int j = q / P, p = q - j * P;
        sXT[j * LDX + p] = to_f32(xrow(j)[p]);
      }
    }
    for (int q = tid; q < (F4 - n) * LDX; q += kThreads) sXT[n * LDX + q] = 0.f;
    if constexpr (!kB16Fold)
      for (int q = tid; q < (F4 - n) * LDB; q += kThreads) sB[n * LDB + q] = 0.f;
  } else if ((P % VE) == 0) {
    // x: thread -> (entry j = tid mod JP, column block tid / JP), JP =
    // 2^ceil(log2 n), so consecutive lanes write consecutive entries of a
    // transposed row.
    const int lgJP = n > 1 ? 32 - __clz(n - 1) : 0;
    const int JP = 1 << lgJP;
    const int jx = tid & (JP - 1);
    const int PV = P / VE;
    for (int c = tid >> lgJP; c < PV; c += kThreads >> lgJP) {
      if (jx < n) {
        float xv[VE];
        const VT v = ldv_nt<Tin>(xrow(jx) + c * VE);
        st_lds_f32(xv, v);
#pragma unroll
        for (int e = 0; e < VE; ++e) sXT[(c * VE + e) * RS + jx] = xv[e];
      }
    }
  } else {
    const int lgJP = n > 1 ? 32 - __clz(n - 1) : 0;
    const int JP = 1 << lgJP;
    const int jx = tid & (JP - 1);
    for (int p = tid >> lgJP; p < P; p += kThreads >> lgJP)
      if (jx < n) sXT[p * RS + jx] = to_f32(xrow(jx)[p]);
  }
  if (!PCD && wave == 0) {  // c_j = exp(sum_{j<m<n} l_m) dt_j and exp(Lam), tree-summed
    const float u = lane < n ? dl.y : 0.f;
    const float lam = wave_suffix_excl(u, lane);
    if (lane < n) sCF[lane] = expf(lam) * dl.x;
    if (lane == 0) sCF[RS] = expf(lam + u);
  }
  __syncthreads();
  if constexpr (MF && !PCD && !kB16Fold) {  // the fold's A operand: c_j B_j, scaled in place
    for (int q = tid; q < n * N; q += kThreads) {
      const int j = q / N, c = q - j * N;
      sB[j * LDB + c] *= sCF[j];
    }
    __syncthreads();
  }
  if constexpr (PCD) {
    // Channel c (one thread each): lam_j[c] from the newest entry back; the
    // decay goes into the staged key rows, exp(Lam[c]) scales tile column c.
    if (tid < N) {
      float acc = 0.f;
      for (int j = n - 1; j >= 0; --j) {
        sB[j * LDB + tid] *= expf(acc);
        acc += sG[j * N + tid];
      }
      sDc[tid] = expf(acc);
    }
    if (tid < n) sCF[tid] = 1.f;
    __syncthreads();
  }
  const float D = PCD ? 1.f : sCF[RS];
  float Dc[4] = {D, D, D, D};
  if constexpr (PCD) {
#pragma unroll
    for (int v = 0; v < 4; ++v) Dc[v] = sDc[col * 4 + v];
  }

  // 3. S <- D S + sum_j x_j outer (c_j B_j), in place.
  auto store_row = [&](int row, const float4& v) {
    if constexpr (B16) {
      st8_bf16x4(tileb + (size_t)row * N + col * 4, v);
    } else {
      st16(tile + (size_t)row * N + col * 4, v);
      if (DUAL) {
        bf16_t* lo = static_cast<bf16_t*>(a.ckpt_lo) + (size_t)bh * P * N + (size_t)row * N + col * 4;
        uint2 pk;
        pk.x = pack_bf16x2(v.x, v.y);
        pk.y = pack_bf16x2(v.z, v.w);
        *reinterpret_cast<uint2*>(lo) = pk;
      }
    }
  };
  for (int base = 0; base < P; base += RPP * kMaxPass) {
    if (base > 0) load_chunk(base);
    if constexpr (MF) {
      if (rows.wave_row(base, 0, wave) < P) {
        auto fin = [&](int k, const float (&d)[4]) {
          const float4 s = fr[k].v;
          const int row = rows.row(base, k);
          if (row < P)
            store_row(row, make_float4(fmaf(Dc[0], s.x, d[0]), fmaf(Dc[1], s.y, d[1]),
                                       fmaf(Dc[2], s.z, d[2]), fmaf(Dc[3], s.w, d[3])));
        };
        float* buf = lds + lay.oW + wave * Fold::BUF;
        if constexpr (kB16Fold) {
          Fold::run_b16(rows.wave_row(base, 0, wave), P, F16, bt, buf, lane, col,
                        [&](int j, int p) {  // v_j[p] = c_j x_j[p], zero past the window
                          const int jr = j < n ? j : 0;
                          const float v = sCF[jr] * sXT[jr * LDX + p];
                          return j < n ? v : 0.f;
                        },
                        fin);
        } else {
          Fold::run(rows.wave_row(base, 0, wave), P, F4, buf, lane, col,
                    [&](int j, int c) { return sB[j * LDB + c]; },
                    [&](int j, int p) { return sXT[j * LDX + p]; }, fin);
        }
      }
    } else {
#pragma unroll
      for (int k = 0; k < kMaxPass; ++k) {
        fr[k].v.x *= Dc[0];
        fr[k].v.y *= Dc[1];
        fr[k].v.z *= Dc[2];
        fr[k].v.w *= Dc[3];
      }
      // Rows past P read a valid row (results unused): every pass without a branch.
      const float* xr[kMaxPass];
#pragma unroll
      for (int k = 0; k < kMaxPass; ++k) {
        const int row = rows.row(base, k);
        xr[k] = sXT + (row < P ? row : P - 1) * RS;
      }
      for (int j = 0; j < n; ++j) {
        const float cj = sCF[j];
        const float4 t = *reinterpret_cast<const float4*>(&sB[j * LDB + col * 4]);
        const float b0 = cj * t.x, b1 = cj * t.y, b2 = cj * t.z, b3 = cj * t.w;
#pragma unroll
        for (int k = 0; k < kMaxPass; ++k) {
          const float xv = xr[k][j];
          float4& s = fr[k].v;
          s.x = fmaf(xv, b0, s.x); s.y = fmaf(xv, b1, s.y);
          s.z = fmaf(xv, b2, s.z); s.w = fmaf(xv, b3, s.w);
        }
      }
#pragma unroll
      for (int k = 0; k < kMaxPass; ++k) {
        const int row = rows.row(base, k);
        if (row < P) {
          if constexpr (B16) {
            st8_bf16x4(tileb + (size_t)row * N + col * 4, fr[k].v);
            continue;
          }
          st16(tile + (size_t)row * N + col * 4, fr[k].v);
          if (DUAL) {
            bf16_t* lo = static_cast<bf16_t*>(a.ckpt_lo) + (size_t)bh * P * N + (size_t)row * N + col * 4;
            uint2 pk;
            pk.x = pack_bf16x2(fr[k].v.x, fr[k].v.y);
            pk.y = pack_bf16x2(fr[k].v.z, fr[k].v.w);
            *reinterpret_cast<uint2*>(lo) = pk;
          }
        }
      }
    }
  }
  if (tid == 0) a.ptr[bh] = make_int4(ring_slot(head, n, R), 0, 0, 0);
}

template <int N, typename Tin, int MODE, bool PCD, bool MF>
static hipError_t flush_one(const FlushArgs& a, int batch, hipStream_t s) {
  constexpr bool kB16Fold = MF && MODE == kCkptBf16 && std::is_same<Tin, bf16_t>::value;
  const size_t lds = (size_t)FlushLds(a.R, a.P, N, PCD, MF ? fold_buf_floats(N, 4, kMaxPass) : 0,
                                      kB16Fold ? fold_bt_elems(N, a.R) : 0)
                         .total * sizeof(float);
  auto kern = flush_kernel<N, Tin, MODE, PCD, MF>;
  if (lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)((size_t)batch * a.H)), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

// The matrix-core fold serves the delta-rule layers (GDN, KDA) and the
// bf16-stored checkpoint, whose decode kernels fold the same way; the fp32 and
// dual-precision Mamba-2 checkpoints keep the FMA fold of their fused decode.
template <int N, typename Tin>
static hipError_t flush_t(const FlushArgs& a, int batch, int mode, bool delta, hipStream_t s) {
  switch (mode) {
    case kCkptF32:
      if (delta) return flush_one<N, Tin, kCkptF32, false, true>(a, batch, s);
      return flush_one<N, Tin, kCkptF32, false, false>(a, batch, s);
    case kCkptDual: return flush_one<N, Tin, kCkptDual, false, false>(a, batch, s);
    case kCkptBf16: return flush_one<N, Tin, kCkptBf16, false, true>(a, batch, s);
    default: return hipErrorInvalidValue;
  }
}

template <int N>
static hipError_t flush_n(const FlushArgs& a, int batch, bool bf16_in, int mode, int kind,
                          hipStream_t s) {
  if (kind == kFoldKda) {  // per-channel decay: fp32 rows and checkpoint only
    if (bf16_in || mode != kCkptF32) return hipErrorInvalidValue;
    return flush_one<N, float, kCkptF32, true, true>(a, batch, s);
  }
  if (kind == kFoldGdn) {
    if (bf16_in || mode != kCkptF32) return hipErrorInvalidValue;
    return flush_t<N, float>(a, batch, mode, true, s);
  }
  return bf16_in ? flush_t<N, bf16_t>(a, batch, mode, false, s)
                 : flush_t<N, float>(a, batch, mode, false, s);
}

hipError_t launch_flush(const FlushArgs& a, int batch, int N, bool bf16_in, int mode, int kind,
                        hipStream_t s) {
  switch (N) {
    case 16: return flush_n<16>(a, batch, bf16_in, mode, kind, s);
    case 32: return flush_n<32>(a, batch, bf16_in, mode, kind, s);
    case 64: return flush_n<64>(a, batch, bf16_in, mode, kind, s);
    case 128: return flush_n<128>(a, batch, bf16_in, mode, kind, s);
    case 256: return flush_n<256>(a, batch, bf16_in, mode, kind, s);
    default: return hipErrorInvalidValue;
  }
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void init_kernel(InitArgs a) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  const size_t i0 = (size_t)blockIdx.x * kThreads + threadIdx.x;
  const size_t nvec = a.n_state / 4;
  for (size_t i = i0; i < nvec; i += stride) {
    const float4 v = a.S0 ? reinterpret_cast<const float4*>(a.S0)[i] : float4{};
    if (a.ckpt) reinterpret_cast<float4*>(a.ckpt)[i] = v;
    if (a.ckpt_lo) {
      uint2 pk;
      pk.x = pack_bf16x2(v.x, v.y);
      pk.y = pack_bf16x2(v.z, v.w);
      reinterpret_cast<uint2*>(a.ckpt_lo)[i] = pk;
    }
  }
  for (size_t i = i0; i < a.n_ptr; i += stride) a.ptr[i] = make_int4(0, 0, 0, 0);
  if (i0 == 0) *a.err = 0;
}

hipError_t launch_init(const InitArgs& a, hipStream_t s) {
  const size_t work = a.n_state / 4 > a.n_ptr ? a.n_state / 4 : a.n_ptr;
  size_t blocks = (work + kThreads - 1) / kThreads;
  if (blocks > 8192) blocks = 8192;
  if (blocks == 0) blocks = 1;
  hipLaunchKernelGGL(init_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void rollback_kernel(RollbackArgs a) {
  const size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= a.n_ptr) return;
  const int b = (int)(i / a.H);
  const int nd = a.n_drop[b];
  const int4 p = a.ptr[i];
  if (nd < 0 || nd > p.z) {
    if (i % a.H == 0) atomicOr(a.err, kDevRollbackRange);
    return;
  }
  a.ptr[i] = make_int4(p.x, p.y - nd, 0, 0);
}

hipError_t launch_rollback(const RollbackArgs& a, hipStream_t s) {
  const size_t blocks = (a.n_ptr + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(rollback_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace rss

// The checkpoint fold on the matrix cores.
//
// A fold rewrites a P x N tile with the window's F entries (P1, "Tenir le
// journal plutôt que le solde": the checkpoint is rewritten once the buffer is
// full):
//
//   S[p, n] <- D[n] * S[p, n] + dS[p, n],   dS = sum_{j < F} x_j[p] * a_j[n]
//
// with a_j = c_j B_j (Mamba-2, c_j = exp(lam_j) dt_j; GDN: c_j = exp(lam_j),
// x -> u, B -> k) or the channel-decayed key (KDA, c_j = 1), and D the window's
// decay (one value, or one per key channel). dS is a real contraction over the
// window (K = F), so it runs on v_mfma_f32_16x16x4f32 (fp32 in, fp32
// accumulate), four entries per instruction:
//
//   dS^T[n, p] (16 x 16 block) += A[n, j] (16 x 4) * X[j, p] (4 x 16)
//
// Lane l supplies A[n = l % 16][j = l / 16] and X[j = l / 16][p = l % 16], and
// receives dS^T[n = 4 (l / 16) + v][p = l % 16] for v = 0..3: four adjacent
// columns of one row of dS. Entries past F are zero.
//
// The tile itself stays in the layout its coalesced loads deliver (RowMap:
// each wavefront holds MP * SR consecutive rows, a lane a 16-byte run of
// columns per row), which is not the accumulator layout. Each wavefront hands
// its dS blocks to its own lanes through a small LDS buffer (HR = 8 rows of N
// columns, 4 rows at N = 256, padded so writes and reads spread over the
// banks), HR rows at a time, and every lane then finishes its own values with
// one fused
// multiply-add: S = fma(D, S, dS). No other wavefront touches the buffer, so
// the hand-over needs no barrier (a wavefront's LDS accesses complete in
// order).
//
// A bf16-stored checkpoint with bf16 inputs folds with run_b16 instead: the
// same contraction on v_mfma_f32_16x16x32_bf16, sixteen entries per
// instruction, with c_j x_j carried as a bf16 (hi, lo) pair (2^-18 relative,
// far below the bf16 rounding of the stored result) and B_j exact. At fp32
// matrix rate that fold (8.6 GFLOP per launch at batch 256) would cost ~55 us
// of matrix-core time per launch; the bf16 form needs an eighth of it.
//
// The flush kernel and every kernel that folds inside a decode call these same
// routines with the same operands in the same order, so a fold gives the same
// bits wherever it runs.
#pragma once

#include "device.h"
#include "lds.h"

namespace rss {

template <int N, int TPR, int VEC, int MP>
struct MfmaFold {
  static constexpr int SR = 64 / TPR;           // rows per pass in a wavefront
  static constexpr int RW = MP * SR;            // rows of a wavefront per chunk
  static constexpr int NRB = (RW + 15) / 16;    // 16-row blocks per wavefront per chunk
  static constexpr int NCB = N / 16;            // 16-column blocks
  static constexpr int HR = N >= 256 ? 4 : 8;   // rows per hand-over round
  static constexpr int LD = N + 4;              // buffer row stride, in floats
  static constexpr int BUF = HR * LD;           // buffer floats per wavefront
  static_assert(N % 16 == 0 && RW % HR == 0, "unsupported tile geometry");
  static_assert(BUF == fold_buf_floats(N, VEC, MP), "LDS layout and fold disagree");

  // Computes dS for the rows of this wavefront's chunk and hands this lane its
  // share: fin(k, d) is called once per pass k of the lane whose row lies in a
  // computed row block, with d[v] = dS at column col * VEC + v (fin finishes the
  // tile values, S = fma(D, S, d), and may store them at once).
  // R0: first row of the wavefront's chunk (R0 < P). F4: the entry count
  // rounded up to a multiple of 4. aop(j, n) and xop(j, p) read the window's
  // operands for 0 <= j < F4 (entries at or past the true count must read as
  // zero), 0 <= n < N and R0 <= p < P. buf: this wavefront's BUF floats.
  template <typename AOp, typename XOp, typename Fin>
  __device__ static __forceinline__ void run(int R0, int P, int F4, float* buf, int lane, int col,
                                             AOp aop, XOp xop, Fin fin) {
    const int l15 = lane & 15, lg = lane >> 4;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      if (R0 + rb * 16 >= P) break;  // uniform: the rest of the chunk lies past the tile
      // rows past the tile (or past this wavefront's rows) read a valid row;
      // their results are never handed over
      const int pr = R0 + rb * 16 + l15 < P ? R0 + rb * 16 + l15 : P - 1;
      f32x4 acc[NCB];
#pragma unroll
      for (int c = 0; c < NCB; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int e = 0; e < F4; e += 4) {
        const int j = e + lg;
        const float xv = xop(j, pr);
#pragma unroll
        for (int c = 0; c < NCB; ++c)
          acc[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(aop(j, c * 16 + l15), xv, acc[c], 0, 0, 0);
      }
      hand_over(rb, acc, buf, lane, col, fin);
    }
  }

  // The same dS for a window of bf16 entries (x_j and B_j stored as bf16) on
  // v_mfma_f32_16x16x32_bf16, 16 entries per instruction:
  //
  //   dS^T[n, p] (16 x 16 block) += sum_{k < 32} A[n, k] X[k, p]
  //
  // k < 16 takes entry e0 + k with the high part of v_j[p] = c_j x_j[p], k >= 16
  // the same entry with the low part: v is formed in fp32 and split into
  // hi = bf16(v), lo = bf16(v - hi), so hi + lo carries v to 2^-18 relative;
  // A[n, k] = B_j[n] enters exactly, every product is exact in fp32 and the
  // sums are fp32. Lane l supplies A[n = l % 16][k = 8 (l / 16) .. + 7] and
  // X[k = 8 (l / 16) .. + 7][p = l % 16], so one 16-byte read of the
  // transposed B rows per instruction, and receives the fp32 path's layout.
  // bt: the window's B rows transposed in groups of 16 entries, bf16
  // [F16 / 16][N][16] (element (g, n, i) = B_{16 g + i}[n], zero past the
  // window), so the eight column blocks of one group lie at fixed offsets;
  // F16: the entry count rounded up to a multiple of 16. vop(j, p) returns
  // v_j[p] in fp32 (zero past the window).
  template <typename VOp, typename Fin>
  __device__ static __forceinline__ void run_b16(int R0, int P, int F16, const bf16_t* bt, float* buf,
                                                 int lane, int col, VOp vop, Fin fin) {
    typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
    const int l15 = lane & 15, lg = lane >> 4;
    const int jo = 8 * (lg & 1);     // this lane's first entry of a group of 16
    const bool low = lg >= 2;         // k-slices 16..31: the low parts
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      if (R0 + rb * 16 >= P) break;
      const int pr = R0 + rb * 16 + l15 < P ? R0 + rb * 16 + l15 : P - 1;
      f32x4 acc[NCB];
#pragma unroll
      for (int c = 0; c < NCB; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int e0 = 0; e0 < F16; e0 += 16) {
        u32x4 xw;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float v0 = vop(e0 + jo + 2 * q, pr), v1 = vop(e0 + jo + 2 * q + 1, pr);
          const uint32_t hi = pack_bf16x2(v0, v1);
          const uint32_t lo = pack_bf16x2(v0 - __uint_as_float(hi << 16), v1 - __uint_as_float(hi & 0xffff0000u));
          xw[q] = low ? lo : hi;
        }
        const bf16x8 X = __builtin_bit_cast(bf16x8, xw);
#pragma unroll
        for (int c = 0; c < NCB; ++c) {
          const u32x4 av = *reinterpret_cast<const u32x4*>(bt + ((e0 >> 4) * N + c * 16 + l15) * 16 + jo);
          acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), X, acc[c], 0, 0, 0);
        }
      }
      hand_over(rb, acc, buf, lane, col, fin);
    }
  }

 private:
  // Hand-over of row block rb in rounds of HR rows: the accumulator rows of the
  // round into the buffer, then every lane whose pass falls in those rows
  // reads its own columns and finishes them.
  template <typename Fin>
  __device__ static __forceinline__ void hand_over(int rb, const f32x4 (&acc)[NCB], float* buf, int lane,
                                                   int col, Fin& fin) {
    const int l15 = lane & 15, lg = lane >> 4;
    const int lrow = lane / TPR;
#pragma unroll
    for (int h = 0; h < 16 / HR; ++h) {
      if (rb * 16 + h * HR >= RW) break;
      if (l15 / HR == h) {
#pragma unroll
        for (int c = 0; c < NCB; ++c)
          *reinterpret_cast<f32x4*>(buf + (l15 % HR) * LD + c * 16 + 4 * lg) = acc[c];
      }
#pragma unroll
      for (int k = 0; k < MP; ++k) {
        const int qk = k * SR + lrow;
        if (qk / HR != rb * (16 / HR) + h) continue;
        const float* src = buf + (qk % HR) * LD + col * VEC;
        float d[VEC];
#pragma unroll
        for (int v4 = 0; v4 < VEC; v4 += 4) {
          const f32x4 t = *reinterpret_cast<const f32x4*>(src + v4);
#pragma unroll
          for (int v = 0; v < 4; ++v) d[v4 + v] = t[v];
        }
        fin(k, d);
      }
    }
  }
};

}  // namespace rss

// The ring terms of a verify on the matrix cores.
//
// A verify computes the outputs of nt tokens t_i = n0 + i at once from the
// checkpoint and the window (P2, "L'astuce du checkpoint et du tampon"; the
// speculative round of "Un retour en arrière qui devient trivial"). The
// window's part of output i is
//
//   z_i[p] = sum_{j <= t_i} w_ij x_j[p],   w_ij = coef_ij (B_j . C_i),
//
// coef_ij = exp(lam_i(j)) dt_j (zero for j > t_i). Over all outputs these are
// two small dense products, each a real contraction:
//
//   W[j, i] = sum_n B_j[n] C_i[n]   (window entries x outputs, K = N)
//   Z[p, i] = sum_j x_j[p] w_ij     (rows x outputs, K = window length)
//
// W runs on v_mfma_f32_16x16x32_bf16: B and C are bf16 inputs, so each
// product is exact in fp32 and the sums are fp32. Z runs on
// v_mfma_f32_16x16x4f32 (w is fp32). Both take a 16 x 16 output block per
// instruction sequence, outputs as the 16 columns (nt <= 9 of them used).
// Lane l supplies row l % 16 of the first operand and column l % 16 of the
// second, k-slice l / 16 of both; it receives rows 4 (l / 16) + r, r = 0..3, of
// column l % 16. Operand rows past the window or the outputs read a valid row
// (their results are never used) or zero where they enter a kept sum.
#pragma once

#include "device.h"

namespace rss {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// coef[i * RL + j] *= B_j . C_i for every window entry j < L and output i < nt.
// sB: the window's B rows, raw bf16 [L][N]; sCr: the outputs' C rows, raw bf16
// [nt][N]; both 16-byte aligned, N % 16 == 0. Wavefront w takes the blocks of
// 16 entries w, w + NW, ...
template <int N>
__device__ __forceinline__ void verify_weights_mfma(const bf16_t* sB, const bf16_t* sCr, float* coef,
                                                    int RL, int L, int nt, int wave, int NW, int lane) {
  const int l15 = lane & 15, kq = (lane >> 4) * 8;
  const int i = l15 < nt ? l15 : nt - 1;
  for (int blk = wave; blk * 16 < L; blk += NW) {
    const int j = blk * 16 + l15 < L ? blk * 16 + l15 : L - 1;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < N; kc += 32) {
      uint4 bv = make_uint4(0u, 0u, 0u, 0u), cv = make_uint4(0u, 0u, 0u, 0u);
      if (kc + kq < N) {  // N = 16: the upper half of K is zero
        bv = *reinterpret_cast<const uint4*>(sB + j * N + kc + kq);
        cv = *reinterpret_cast<const uint4*>(sCr + i * N + kc + kq);
      }
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, bv),
                                                    __builtin_bit_cast(bf16x8_t, cv), acc, 0, 0, 0);
    }
    if (l15 < nt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int jj = blk * 16 + (lane >> 4) * 4 + r;
        if (jj < L) coef[l15 * RL + jj] *= acc[r];
      }
    }
  }
}

// sRing[i * P + p] = sum_{j < L} x_j[p] coef[i * RL + j] for p < P, i < nt
// (coef holding w_ij, zero for j > t_i). sX: the window's x rows [L][P].
// Wavefront w takes the blocks of 16 rows w, w + NW, ...
template <typename Tin>
__device__ __forceinline__ void verify_shares_mfma(const Tin* sX, const float* coef, float* sRing, int RL,
                                                   int P, int L, int nt, int wave, int NW, int lane) {
  const int l15 = lane & 15, lq = lane >> 4;
  const bool out_ok = l15 < nt;
  for (int pb = wave; pb * 16 < P; pb += NW) {
    const int p = pb * 16 + l15 < P ? pb * 16 + l15 : P - 1;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < L; j0 += 4) {
      const int j = j0 + lq;
      const float xv = j < L ? to_f32(sX[j * P + p]) : 0.f;
      const float wv = j < L && out_ok ? coef[l15 * RL + j] : 0.f;
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xv, wv, acc, 0, 0, 0);
    }
    if (out_ok) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int pp = pb * 16 + lq * 4 + r;
        if (pp < P) sRing[l15 * P + pp] = acc[r];
      }
    }
  }
}

}  // namespace rss

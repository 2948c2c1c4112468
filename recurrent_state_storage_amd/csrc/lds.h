// Dynamic LDS layouts of the replay, flush and delta-rule kernels, shared by
// the kernels and by the host-side configuration check (a configuration whose
// layout exceeds kMaxLdsBytes is refused before any launch).
#pragma once

#include "device.h"

namespace rss {

constexpr int kMaxLdsBytes = 160 * 1024;  // LDS one gfx950 workgroup may allocate

// Floats of the per-wavefront hand-over buffer of the matrix-core fold
// (fold.h) for an N-column tile: 8 rows (4 at N = 256) of N columns, padded by
// 4 floats per row. (VEC and MP, the tile geometry, do not change it.)
__host__ __device__ constexpr int fold_buf_floats(int N, int VEC, int MP) {
  return (VEC > 0 && MP > 0) ? (N >= 256 ? 4 : 8) * (N + 4) : 0;
}

// bf16 elements of the transposed B rows the bf16 matrix-core fold reads
// (fold.h): N rows of the window's entries, padded to a multiple of 16.
__host__ __device__ constexpr int fold_bt_elems(int N, int R) { return N * ((R + 15) & ~15); }

// Row stride (floats) of a matrix-core fold operand staged in LDS: at least n,
// and 16 more than a multiple of 64, so the four window entries one
// instruction reads (one per group of 16 lanes) fall on different banks.
__host__ __device__ constexpr int fold_ld(int n) { return n + ((16 - n) & 63); }

// Dynamic LDS layout of the replay kernel, in 4-byte words. The window's x and
// B rows are kept raw (input dtype), exactly as the direct global->LDS loads
// deliver them; everything else is fp32. With a matrix-core fold (fold_buf >
// 0) the window rows are allocated in multiples of four (the fold reads entries
// in groups of four; the rows past the window are zeroed).
struct ReplayLds {
  int RA, oX, oB, oC, oCF, oDC, oCR, oRing, oFC, FD, oW, oBT, total;
  // fold_buf: floats of the matrix-core fold's hand-over buffer per wavefront
  // (0 when the kernel does not fold on the matrix cores); fold_bt: bf16
  // elements of the transposed B rows of the bf16 fold (0 without it).
  __host__ __device__ ReplayLds(int R, int P, int N, int ntmax, int tin_bytes, int nw,
                                int fold_buf = 0, int fold_bt = 0) {
    RA = fold_buf > 0 ? align4(R) : R;                 // allocated window rows
    oX = 0;                                            // raw window x [RA][P]
    oB = align4((RA * P * tin_bytes + 3) / 4);         // raw window B [RA][N]
    oC = oB + align4((RA * N * tin_bytes + 3) / 4);    // new tokens' C [ntmax][N]
    oCF = oC + ntmax * N;                              // exp(lam) * dt [ntmax][R]
    oDC = oCF + ntmax * R;                             // exp(Lam) [ntmax]
    oCR = align4(oDC + ntmax);                         // several bf16 tokens: their raw C [ntmax][N]
    oRing = oCR + (ntmax > 1 && tin_bytes == 2 ? align4((ntmax * N * 2 + 3) / 4) : 0);  // shares [nw][ntmax][P]
    oFC = oRing + nw * ntmax * P;                      // fused fold: c_j [align4(R)], then exp(Lam)
    FD = align4(R);                                    // index of exp(Lam) in the fold coefficients
    oW = align4(oFC + FD + 1);                         // fold hand-over buffers [nw][fold_buf]
    oBT = oW + nw * fold_buf;                          // bf16 fold: B rows transposed [align16(R)/16][N][16]
    total = oBT + align4((fold_bt + 1) / 2);
  }
};

// Dynamic LDS layout of the flush kernel, in floats. For the FMA fold, x is
// stored transposed (row p holds entries j = 0..R-1 contiguously, rows padded
// to a multiple of 4 words), so the window's x values of one row sit together;
// for the matrix-core fold (fold_buf > 0) x and the scaled B rows are stored
// one entry per row with fold_ld strides, the rows past the window zeroed.
struct FlushLds {
  int RS, LDX, LDB, oXT, oB, oCF, oDc, oG, oW, oBT, total;
  // fold_buf: floats of the matrix-core fold's hand-over buffer per wavefront
  // (0: the fold runs on the VALU). The per-channel log-decay rows are dead
  // once the decay walk has scaled the key rows, so the buffers share them.
  // fold_bt: bf16 elements of the transposed B rows of the bf16 fold (then the
  // B rows are not staged in fp32).
  __host__ __device__ FlushLds(int R, int P, int N, bool pcd, int fold_buf = 0, int fold_bt = 0) {
    RS = align4(R);
    const bool mf = fold_buf > 0;
    LDX = mf ? fold_ld(P) : 0;
    LDB = mf ? fold_ld(N) : N;
    oXT = 0;                                   // x: transposed [P][RS], or [RS][LDX]
    oB = mf ? RS * LDX : P * RS;               // window B rows [RS][LDB] (fp32)
    // the bf16 fold reads the B rows only transposed, bf16 [align16(R)/16][N][16],
    // staged in place of the fp32 rows
    oBT = oB;
    oCF = oB + (fold_bt > 0 ? align4((fold_bt + 1) / 2) : RS * LDB);  // c_j [RS], then exp(Lam) at [RS]
    oDc = align4(oCF + RS + 1);                // per-channel exp(Lam[n]) [N]
    oG = align4(oDc + (pcd ? N : 0));          // per-channel log-decay rows [R][N]
    oW = oG;                                   // fold hand-over buffers [4 wavefronts][fold_buf]
    const int g = pcd ? R * N : 0, w = kWaves * fold_buf;
    total = oG + (g > w ? g : w);
  }
};

// Tile passes the GDN / KDA kernels hold per chunk (N / 4 columns per lane
// group): 16 when the head has more rows than 8 passes cover, else 8.
__host__ __device__ constexpr int gdn_passes(int P, int N) { return P > 8 * (1024 / N) ? 16 : 8; }

// Dynamic LDS of the GDN / KDA replay kernel, in floats.
struct GdnLds {
  int RS, oK, oU, oQ, oV, oCF, oS, oD, oFC, oG, oW, total;
  // fold_buf: floats of the matrix-core fold's hand-over buffer per wavefront
  // (0 for a launch that does not fold). The window rows are allocated in
  // multiples of four (the fold reads entries in groups of four; the rows past
  // the window are zeroed). KDA's log-gate rows are dead once the decay walk
  // has scaled the key rows, so the buffers share them.
  __host__ __device__ GdnLds(int R, int P, int N, bool kda, int fold_buf = 0) {
    RS = align4(R);
    oK = 0;                   // window k rows [RS][N] (row n0 = k_t); KDA: scaled in place
    oU = RS * N;              // window u rows [RS][P]
    oQ = oU + RS * P;         // q_t [N]
    oV = align4(oQ + N);      // v_t [P] (the replay decode; 16-byte aligned)
    oCF = oV + P;             // exp(lam_j) [R], then exp(Lam), k_t . q_t
    oS = align4(oCF + R + 2); // shares [4 waves][2][P]: sum_j w u_j for z = k_t, q_t
    oD = oS + 8 * P;          // KDA: exp(Lam[n]) [N]
    oFC = oD + (kda ? N : 0); // fused fold (GDN): c_j [RS], then exp(Lam) at [RS]
    oG = align4(oFC + RS + 1); // KDA: committed log-gate rows [R][N]
    oW = oG;                  // fold hand-over buffers [4 wavefronts][fold_buf]
    const int g = kda ? R * N : 0, w = kWaves * fold_buf;
    total = oG + (g > w ? g : w);
  }
};

}  // namespace rss

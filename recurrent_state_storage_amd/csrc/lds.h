// Dynamic LDS layouts of the replay, flush and delta-rule kernels, shared by
// the kernels and by the host-side configuration check (a configuration whose
// layout exceeds kMaxLdsBytes is refused before any launch).
#pragma once

#include "device.h"

namespace rss {

constexpr int kMaxLdsBytes = 160 * 1024;  // LDS one gfx950 workgroup may allocate

// Floats of the per-wavefront hand-over buffer of the matrix-core fold
// (fold.h) for an N-column tile held as VEC columns per lane and MP passes:
// up to 16 rows of 16 * min(N / 16, 4) columns, padded by 4 floats per row.
__host__ __device__ constexpr int fold_buf_floats(int N, int VEC, int MP) {
  const int rw = MP * (64 / (N / VEC));
  const int ncb = N / 16;
  return (rw < 16 ? rw : 16) * (16 * (ncb < 4 ? ncb : 4) + 4);
}

// Dynamic LDS layout of the replay kernel, in 4-byte words. The window's x and
// B rows are kept raw (input dtype), exactly as the direct global->LDS loads
// deliver them; everything else is fp32.
struct ReplayLds {
  int oX, oB, oC, oCF, oDC, oRing, oFC, oW, total;
  // fold_buf: floats of the matrix-core fold's hand-over buffer per wavefront
  // (0 when the kernel does not fold on the matrix cores).
  __host__ __device__ ReplayLds(int R, int P, int N, int ntmax, int tin_bytes, int nw,
                                int fold_buf = 0) {
    oX = 0;                                            // raw window x [R][P]
    oB = align4((R * P * tin_bytes + 3) / 4);          // raw window B [R][N]
    oC = oB + align4((R * N * tin_bytes + 3) / 4);     // new tokens' C [ntmax][N]
    oCF = oC + ntmax * N;                              // exp(lam) * dt [ntmax][R]
    oDC = oCF + ntmax * R;                             // exp(Lam) [ntmax]
    oRing = align4(oDC + ntmax);                       // ring shares [nw][ntmax][P]
    oFC = oRing + nw * ntmax * P;                      // fused fold: c_j [R], then exp(Lam)
    oW = align4(oFC + R + 1);                          // fold hand-over buffers [nw][fold_buf]
    total = oW + nw * fold_buf;
  }
};

// Dynamic LDS layout of the flush kernel, in floats. x is stored transposed
// (row p holds entries j = 0..R-1 contiguously, rows padded to a multiple of 4
// words), so the window's x values of one row sit together.
struct FlushLds {
  int RS, oXT, oB, oCF, oDc, oG, oW, total;
  // fold_buf: floats of the matrix-core fold's hand-over buffer per wavefront
  // (0: the fold runs on the VALU). The per-channel log-decay rows are dead
  // once the decay walk has scaled the key rows, so the buffers share them.
  __host__ __device__ FlushLds(int R, int P, int N, bool pcd, int fold_buf = 0) {
    RS = align4(R);
    oXT = 0;                 // x transposed  [P][RS]
    oB = P * RS;             // window B rows [R][N]
    oCF = oB + R * N;        // c_j = exp(lam_j) dt_j [R], then exp(Lam)
    oDc = align4(oCF + R + 1);       // per-channel exp(Lam[n]) [N]
    oG = align4(oDc + (pcd ? N : 0));  // per-channel log-decay rows [R][N]
    oW = oG;                         // fold hand-over buffers [4 wavefronts][fold_buf]
    const int g = pcd ? R * N : 0, w = kWaves * fold_buf;
    total = oG + (g > w ? g : w);
  }
};

// Tile passes the GDN / KDA kernels hold per chunk (N / 4 columns per lane
// group): 16 when the head has more rows than 8 passes cover, else 8.
__host__ __device__ constexpr int gdn_passes(int P, int N) { return P > 8 * (1024 / N) ? 16 : 8; }

// Dynamic LDS of the GDN / KDA replay kernel, in floats.
struct GdnLds {
  int oK, oU, oQ, oCF, oS, oD, oFC, oG, oW, total;
  // fold_buf: floats of the matrix-core fold's hand-over buffer per wavefront
  // (0 for a launch that does not fold). KDA's log-gate rows are dead once the
  // decay walk has scaled the key rows, so the buffers share them.
  __host__ __device__ GdnLds(int R, int P, int N, bool kda, int fold_buf = 0) {
    oK = 0;                   // window k rows [R][N] (row n0 = k_t); KDA: scaled in place
    oU = R * N;               // window u rows [R][P]
    oQ = oU + R * P;          // q_t [N]
    oCF = oQ + N;             // exp(lam_j) [R], then exp(Lam), k_t . q_t
    oS = align4(oCF + R + 2); // shares [4 waves][2][P]: sum_j w u_j for z = k_t, q_t
    oD = oS + 8 * P;          // KDA: exp(Lam[n]) [N]
    oFC = oD + (kda ? N : 0); // fused fold (GDN): c_j [R], then exp(Lam)
    oG = align4(oFC + R + 1); // KDA: committed log-gate rows [R][N]
    oW = oG;                  // fold hand-over buffers [4 wavefronts][fold_buf]
    const int g = kda ? R * N : 0, w = kWaves * fold_buf;
    total = oG + (g > w ? g : w);
  }
};

}  // namespace rss

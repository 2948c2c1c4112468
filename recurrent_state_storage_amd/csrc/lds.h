// Dynamic LDS layouts of the replay, flush and delta-rule kernels, shared by
// the kernels and by the host-side configuration check (a configuration whose
// layout exceeds kMaxLdsBytes is refused before any launch).
#pragma once

#include "device.h"

namespace rss {

constexpr int kMaxLdsBytes = 160 * 1024;  // LDS one gfx950 workgroup may allocate

// Dynamic LDS layout of the replay kernel, in 4-byte words. The window's x and
// B rows are kept raw (input dtype), exactly as the direct global->LDS loads
// deliver them; everything else is fp32.
struct ReplayLds {
  int oX, oB, oC, oCF, oDC, oRing, oFC, RS, oXT, oCB, total;
  // fold_f32: room for the fused fold of a bf16-stored checkpoint, whose
  // operands are widened once: x transposed [P][RS] and c_j B_j [RS][N].
  __host__ __device__ ReplayLds(int R, int P, int N, int ntmax, int tin_bytes, int nw,
                                bool fold_f32 = false) {
    oX = 0;                                            // raw window x [R][P]
    oB = align4((R * P * tin_bytes + 3) / 4);          // raw window B [R][N]
    oC = oB + align4((R * N * tin_bytes + 3) / 4);     // new tokens' C [ntmax][N]
    oCF = oC + ntmax * N;                              // exp(lam) * dt [ntmax][R]
    oDC = oCF + ntmax * R;                             // exp(Lam) [ntmax]
    oRing = align4(oDC + ntmax);                       // ring shares [nw][ntmax][P]
    oFC = oRing + nw * ntmax * P;                      // fused fold: c_j [R], then exp(Lam)
    RS = align4(R);
    oXT = align4(oFC + R + 1);
    oCB = oXT + (fold_f32 ? P * RS : 0);
    total = fold_f32 ? oCB + RS * N : oFC + R + 1;
  }
};

// Dynamic LDS layout of the flush kernel, in floats. x is stored transposed
// (row p holds entries j = 0..R-1 contiguously, rows padded to a multiple of 4
// words), so the window's x values of one row sit together.
struct FlushLds {
  int RS, oXT, oB, oCF, oG, oDc, total;
  __host__ __device__ FlushLds(int R, int P, int N, bool pcd) {
    RS = align4(R);
    oXT = 0;                 // x transposed  [P][RS]
    oB = P * RS;             // window B rows [R][N]
    oCF = oB + R * N;        // c_j = exp(lam_j) dt_j [R], then exp(Lam)
    oG = align4(oCF + R + 1);        // per-channel log-decay rows [R][N]
    oDc = oG + (pcd ? R * N : 0);    // per-channel exp(Lam[n]) [N]
    total = oDc + (pcd ? N : 0);
  }
};

// Dynamic LDS of the GDN / KDA replay kernel, in floats.
struct GdnLds {
  int oK, oU, oQ, oCF, oS, oG, oD, oFC, total;
  __host__ __device__ GdnLds(int R, int P, int N, bool kda) {
    oK = 0;                   // window k rows [R][N] (row n0 = k_t); KDA: scaled in place
    oU = R * N;               // window u rows [R][P]
    oQ = oU + R * P;          // q_t [N]
    oCF = oQ + N;             // exp(lam_j) [R], then exp(Lam), k_t . q_t
    oS = align4(oCF + R + 2); // shares [4 waves][2][P]: sum_j w u_j for z = k_t, q_t
    oG = oS + 8 * P;          // KDA: committed log-gate rows [R][N]
    oD = oG + (kda ? R * N : 0);   // KDA: exp(Lam[n]) [N]
    oFC = oD + (kda ? N : 0);      // fused fold (GDN): c_j [R], then exp(Lam)
    total = oFC + R + 1;
  }
};

}  // namespace rss

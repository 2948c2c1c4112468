// Internal launch interface between the C ABI (rss_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "limits.h"

namespace rss {

// Decode (nt = 1) and speculative verify (nt = K+1) by replay.
struct ReplayArgs {
  float* ckpt;             // [Bt,H,P,N] fp32 master (written only by the fused fold)
  void* ckpt_lo;           // [Bt,H,P,N] bf16 read copy (dual mode), or the bf16-stored
                           // checkpoint (written only by its fused fold)
  void* ring_x;            // [Bt,R,H,P] (slot-major)
  void* ring_B;            // [Bt,R,G,N]
  float2* ring_dl;         // [Bt,R,H] (dt, dt*A)
  int4* ptr;               // [Bt,H] (head, len, n_tent, 0)
  const float* A;          // [H]
  int* err;                // sticky device word
  const void* x;           // [Bt,nt,H,P]
  const void* B;           // [Bt,nt,G,N]
  const void* C;           // [Bt,nt,G,N]
  const float* dt;         // [Bt,nt,H]
  float* y;                // [Bt,nt,H,P]
  int H, P, G, R, nt, set_tent;
  int fold_min_len;        // decode only: also fold windows that reach this length (0: never)
  const int* fold_min_len_dev;  // [Bt] per-sequence fold thresholds (overrides fold_min_len), or null
  uint64_t xdiv;           // ceil(2^32 / d): q / d == (q * xdiv) >> 32 for q < 2^16,
                           // d = P/VE (16-byte x vectors per row) or P (element path)
  int dual_fold;           // decode of a dual-precision layer with a fold: read the fp32
                           // master (outputs from its bf16 rounding), write master + copy
};
hipError_t launch_replay(const ReplayArgs& a, int batch, int N, bool bf16_in, bool low_copy,
                         hipStream_t s);

// Checkpoint precision modes (the public read_copy codes).
enum CkptMode { kCkptF32 = 0, kCkptDual = 1, kCkptBf16 = 2 };

// Fold the window into the checkpoint for sequences with len >= min_len.
struct FlushArgs {
  float* ckpt;             // fp32 checkpoint (null in kCkptBf16 mode)
  void* ckpt_lo;           // bf16 read copy (kCkptDual), or the bf16 checkpoint (kCkptBf16)
  const void* ring_x;
  const void* ring_B;
  const float2* ring_dl;
  const float* ring_g;     // per-channel log-decay rows [Bt,R,H,N] (KDA), else unused
  int4* ptr;
  int* err;
  int H, P, G, R, min_len;
  const int* min_len_dev;  // [Bt] per-sequence thresholds (overrides min_len), or null
};
// Layer kinds for the fold: Mamba-2, Gated DeltaNet (matrix-core fold), Kimi
// Delta Attention (matrix-core fold with per-channel decays).
enum FoldKind { kFoldMamba2 = 0, kFoldGdn = 1, kFoldKda = 2 };
hipError_t launch_flush(const FlushArgs& a, int batch, int N, bool bf16_in, int mode, int kind,
                        hipStream_t s);

// ckpt <- S0 (or 0), read copy <- bf16(ckpt), pointers and error word <- 0.
struct InitArgs {
  float* ckpt;             // null when the checkpoint is bf16 only
  void* ckpt_lo;           // bf16 copy or bf16 checkpoint (may be null)
  const float* S0;
  int4* ptr;
  int* err;
  size_t n_state;          // Bt*H*P*N (a multiple of 4)
  size_t n_ptr;            // Bt*H
};
hipError_t launch_init(const InitArgs& a, hipStream_t s);

// len -= n_drop[b], n_tent = 0 for every (b, h) with 0 <= n_drop[b] <= n_tent.
struct RollbackArgs {
  int4* ptr;
  const int* n_drop;
  int* err;
  int H;
  size_t n_ptr;
};
hipError_t launch_rollback(const RollbackArgs& a, hipStream_t s);

// Eager baseline: T tokens in place (src_slot == nullptr) or from pool slot
// src_slot[b] with a snapshot written to slot i after token i.
struct EagerArgs {
  void* S;                 // in-place state [Bt,H,P,N] (fp32, or bf16 when bf16_state),
                           // or the fp32 pool [Bt,slots,H,P,N]
  const int* src_slot;     // nullptr: in place
  const void* x;           // [Bt,T,H,P]
  const void* B;           // [Bt,T,G,N]
  const void* C;           // [Bt,T,G,N]
  const float* dt;         // [Bt,T,H]
  const float* A;          // [H]
  float* y;                // [Bt,T,H,P]
  int H, P, G, T, slots;
};
hipError_t launch_eager(const EagerArgs& a, int batch, int N, bool bf16_in, bool bf16_state,
                        hipStream_t s);

// Gated DeltaNet / KDA replay decode (one token) and the eager baselines.
struct GdnArgs {
  float* ckpt;             // [Bt,H,P,N] fp32, P = d_v, N = d_k
  float* ring_u;           // [Bt,R,H,P] (slot-major)
  float* ring_k;           // [Bt,R,H,N]
  float2* ring_dl;         // GDN: [Bt,R,H] (1, log alpha)
  float* ring_g;           // KDA: [Bt,R,H,N] log alpha per channel
  int4* ptr;               // [Bt,H]
  int* err;
  const float* q;          // [Bt,H,N]
  const float* k;          // [Bt,H,N]
  const float* v;          // [Bt,H,P]
  const float* beta;       // [Bt,H]
  const float* alpha;      // GDN [Bt,H]; KDA [Bt,H,N]
  float* o;                // [Bt,H,P]
  int H, P, R;
  int fold_min_len;        // also fold windows that reach this length (0: never)
};
hipError_t launch_gdn_replay(const GdnArgs& a, int batch, int N, bool kda, hipStream_t s);

struct GdnEagerArgs {
  float* S;                // [Bt,H,P,N], updated in place
  const float* q;
  const float* k;
  const float* v;
  const float* beta;
  const float* alpha;
  float* o;
  int H, P;
};
hipError_t launch_gdn_eager(const GdnEagerArgs& a, int batch, int N, bool kda, hipStream_t s);

}  // namespace rss

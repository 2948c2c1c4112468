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
// two memory round trips (tile and pointer word, then everything else), so a
// workgroup lives about two latencies whatever the window length:
//   1. issue the 16-byte non-temporal loads of the checkpoint tile (the only
//      large read), and read the (head, len) pointer word beside them;
//   2. issue, all at once, the window's x and B rows (direct global->LDS loads,
//      kept raw), the new tokens' C and the window's (dt, l) pairs; scan the
//      log-decays in one wavefront (a reverse tree sum: no prefix differences);
//   3. w_ij = exp(lam) dt (B_j . C_i) and sum_j w_ij x_j: for one token, per
//      entry j one wavefront (wavefront w takes j = w mod the number of
//      wavefronts) forms w_j and its share of the sum; for several bf16 tokens
//      both products run on the matrix cores (verify_mfma.h);
//   4. consume the tile: per pass a 16-byte fragment dot C_i (v_dot2_f32_bf16
//      for a bf16 tile), reduce-scattered over the lanes sharing the row,
//      y = exp(Lam) * dot + the ring shares.
// The new tokens' x and B rows are copied from LDS to the ring, and their
// (dt, l) pairs stored, after the loads have landed (a store issued before that
// wait would be waited for too). The checkpoint tile is read exactly once per
// call for all nt outputs. A bf16 tile is read by two-wavefront workgroups.
//
// Fused fold: a decode launched with a fold threshold also folds, in the same
// pass, every window the new token fills (the tile is already in registers),
// and writes the new checkpoint: the flush's extra read of the tile is saved.
// The threshold may differ per sequence, so that sequences whose windows are
// out of phase fold on different steps (a staggered schedule). A verify
// launched with a threshold folds the committed window it starts from instead.
// A bf16-stored checkpoint is folded the same way by the two-wavefront decode,
// on the matrix cores (fold.h) and stored RNE-bf16, as its separate flush does.
// The ring is slot-major (slot s of all heads of a sequence contiguous).
#include <type_traits>

#include "device.h"
#include "fold.h"
#include "verify_mfma.h"
#include "launch.h"
#include "lds.h"

namespace rss {

constexpr int kStageS = 4;  // scalar loads per thread and round (x rows when P % VE != 0)

// FOLD: 0 = no fold; 1 = fold windows that reach the threshold; 2 = the same for
// a dual-precision layer, from its fp32 master: the tile read is the master, the
// outputs use its RNE-bf16 rounding (bit for bit the read copy's values), and
// the fold writes the new master and its RNE-bf16 copy (decode only).
template <int N, typename Tin, bool LOW, int NTMAX, int FOLD, int NT>
__global__ __launch_bounds__(NT) void replay_kernel(ReplayArgs a) {
  constexpr bool kDual = FOLD == 2;
  static_assert(!kDual || (!LOW && NTMAX == 1), "dual fold: fp32 master tile, decode only");
  constexpr int NW = NT / 64;                                  // wavefronts per workgroup
  using Geo = TileGeom<N, LOW, NT>;
  constexpr int VEC = Geo::VEC, TPR = Geo::TPR, RPP = Geo::RPP;
  using Rows = RowMap<TPR, kMaxPass>;
  constexpr int VE = V16<Tin>::VE;
  constexpr int NV = N / VE;                                   // 16-byte vectors per B or C row
  constexpr int kStageC = (NTMAX * NV + NT - 1) / NT;
  constexpr int EPL = N >= 64 ? N / 64 : 1;                    // B elements per lane in a 64-lane dot
  using TileT = typename std::conditional<LOW, bf16_t, float>::type;
  using VT = typename V16<Tin>::T;

  extern __shared__ __align__(16) float lds[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = a.H, P = a.P, G = a.G, R = a.R, nt = a.nt;
  const int bh = xcd_tile(blockIdx.x, gridDim.x, a.P * N * (int)sizeof(TileT));
  const int b = bh / H, h = bh - b * H;
  const int hpg = H / G, g = h / hpg;

  // 1. Checkpoint tile: its address needs no pointer word, so its loads go
  // out first, in parallel with the pointer read.
  const TileT* tile = static_cast<const TileT*>(LOW ? a.ckpt_lo : static_cast<const void*>(a.ckpt)) +
                      (size_t)bh * P * N;
  const float Ah = a.A[h];
  const int col = tid % TPR;
  const Rows rows(tid);
  Frag<LOW> fr[kMaxPass];
  auto load_chunk = [&](int base) {
#pragma unroll
    for (int k = 0; k < kMaxPass; ++k) {
      const int row = rows.row(base, k);
      if (row < P) fr[k].v = ld16(tile + row * N + col * VEC);
      else fr[k].v = decltype(fr[k].v){};
    }
  };
  load_chunk(0);

  const int4 pt = a.ptr[bh];
  const int head = pt.x, n0 = pt.y;
  const int L = n0 + nt;

  // Fused fold (fp32 checkpoint, or a bf16-stored one in a decode): the tile
  // already in registers is folded and written back in this pass, exactly as a
  // separate flush would (same coefficients, same order). A decode folds its whole window, the new token
  // included, once that reaches the threshold; a verify folds the committed
  // window it starts from (never the tentative tokens it appends), as a flush
  // just before it would. Such a verify frees the committed slots for the new
  // entries, so its window may span up to R + K + 1 positions (all staged in
  // LDS before any slot is overwritten).
  // LDS is laid out for the nt tokens of this call (nt <= NTMAX).
  const int NTL = NTMAX == 1 ? 1 : nt;
  const int XR = (FOLD && NTMAX > 1) ? NTL : 0;         // extra staged rows
  const int RL = R + XR;                                 // staged rows (LDS layout)
  bool do_fold = false, tent = false;
  const int F = a.set_tent ? n0 : L;   // entries a fold takes
  if constexpr (FOLD) {
    const int th = a.fold_min_len_dev ? a.fold_min_len_dev[b] : a.fold_min_len;
    if (F >= th && F > 0 && n0 <= R) {
      if (pt.z == 0) do_fold = true;
      else tent = true;
    }
  }
  // (Only with one B row set per head: a group's B ring is written by its first
  // head while the other heads read it, so grouped layers never reuse a slot here.)
  const int cap = do_fold && XR && G == H ? (RL < 64 ? RL : 64) : R;
  if (head < 0 || head >= R || n0 < 0 || n0 > R || L > cap) {  // ring full (no flush), or corrupt pointers
    if (tid == 0) atomicOr(a.err, kDevRingOverflow);
    for (int e = tid; e < nt * P; e += NT) {
      const int i = e / P, p = e - i * P;
      a.y[((size_t)(b * nt + i) * H + h) * P + p] = __builtin_nanf("");
    }
    return;
  }
  if (tent && tid == 0) atomicOr(a.err, kDevUncommitted);  // never fold tentative entries

  using Fold = MfmaFold<N, TPR, VEC, kMaxPass>;
  // A bf16-stored checkpoint with bf16 inputs folds on the bf16 matrix cores
  // (fold.h), from the window's B rows transposed once per workgroup.
  constexpr bool kB16Fold = FOLD && LOW && std::is_same<Tin, bf16_t>::value;
  const ReplayLds lay(RL, P, N, NTL, (int)sizeof(Tin), NW, (FOLD && LOW) ? Fold::BUF : 0,
                      kB16Fold ? fold_bt_elems(N, RL) : 0);
  Tin* sX = reinterpret_cast<Tin*>(lds + lay.oX);
  Tin* sB = reinterpret_cast<Tin*>(lds + lay.oB);
  float* sC = lds + lay.oC;
  float* sCF = lds + lay.oCF;
  float* sDC = lds + lay.oDC;
  float* sFC = lds + lay.oFC;
  float* sRing = lds + lay.oRing;
  // Several bf16 tokens: the ring terms run on the matrix cores, from the raw C
  // rows (a single token keeps the wavefront dots, bitwise the decode's).
  constexpr bool kMfRing = NTMAX > 1 && std::is_same<Tin, bf16_t>::value;
  const bool mf_ring = kMfRing && nt > 1;
  bf16_t* sCr = reinterpret_cast<bf16_t*>(lds + lay.oCR);

  // Per-workgroup base pointers (uniform, held in scalar registers); every
  // per-lane offset below is a 32-bit int. The ring is slot-major: slot s of
  // every head of a sequence is contiguous, so one call's appends of all heads
  // land side by side.
  const int slx = H * P, slb = G * N;                                    // slot strides of x and B
  Tin* rx = static_cast<Tin*>(a.ring_x) + (size_t)b * R * slx + h * P;   // this head's x, slot 0
  Tin* rB = static_cast<Tin*>(a.ring_B) + (size_t)b * R * slb + g * N;   // this group's B, slot 0
  float2* rdl = a.ring_dl + (size_t)b * R * H + h;                       // (dt, l), slot stride H
  const Tin* xin = static_cast<const Tin*>(a.x) + ((size_t)b * nt * H + h) * P;
  const Tin* Bin = static_cast<const Tin*>(a.B) + ((size_t)b * nt * G + g) * N;
  const Tin* Cin = static_cast<const Tin*>(a.C) + ((size_t)b * nt * G + g) * N;
  const float* dtin = a.dt + (size_t)b * nt * H + h;
  float* yout = a.y + ((size_t)b * nt * H + h) * P;
  const int xstr = H * P, bstr = G * N;   // per-token strides of x and of B, C
  auto xrow = [&](int j) -> const Tin* {
    return j < n0 ? rx + ring_slot(head, j, R) * slx : xin + (j - n0) * xstr;
  };
  auto brow = [&](int j) -> const Tin* {
    return j < n0 ? rB + ring_slot(head, j, R) * slb : Bin + (j - n0) * bstr;
  };

  // 2. Window rows straight into LDS (direct global->LDS 16-byte loads: lane l
  // of a wavefront lands at the wavefront's LDS base + 16 l), C and (dt, l)
  // through registers. All issued before any wait. The call's own inputs are
  // read once, so they go non-temporal (measured: decode 185.0 -> 184.3 us at
  // batch 256); the ring rows, read again by the next calls, stay cached, except
  // in a verify that folds them (verify + fold 558.5 -> 555.3 us at batch 512;
  // a decode's fold did not gain).
  const bool last_read = NTMAX > 1 && do_fold;
  const bool xvec = (P % VE) == 0;
  const int PV = xvec ? P / VE : 0;
  auto xdiv = [&](int q) { return (int)(((uint64_t)(uint32_t)q * a.xdiv) >> 32); };
  const int totXV = L * PV, totBV = L * NV, totCV = nt * NV;
  for (int q0 = wave * 64; q0 < totBV; q0 += NT) {
    const int q = q0 + lane;
    if (q < totBV) {
      const int j = q / NV;
      if (j < n0 && !last_read) dma16(brow(j) + (q - j * NV) * VE, sB + q0 * VE);
      else dma16_nt(brow(j) + (q - j * NV) * VE, sB + q0 * VE);   // read for the last time
    }
  }
  Tin sxs[kStageS];
  if (xvec) {
    for (int q0 = wave * 64; q0 < totXV; q0 += NT) {
      const int q = q0 + lane;
      if (q < totXV) {
        const int j = xdiv(q);
        if (j < n0 && !last_read) dma16(xrow(j) + (q - j * PV) * VE, sX + q0 * VE);
        else dma16_nt(xrow(j) + (q - j * PV) * VE, sX + q0 * VE);
      }
    }
  } else {
#pragma unroll
    for (int m = 0; m < kStageS; ++m) {
      const int e = m * NT + tid;
      if (e < L * P) {
        const int j = xdiv(e);
        sxs[m] = xrow(j)[e - j * P];
      }
    }
  }
  VT vc[kStageC];
#pragma unroll
  for (int m = 0; m < kStageC; ++m) {
    const int q = m * NT + tid;
    if (q < totCV) {
      const int i = q / NV, c = q - i * NV;
      vc[m] = __builtin_bit_cast(VT, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Cin + i * bstr + c * VE)));
    }
  }
  // Wavefront 0: lane j holds window entry j's (dt, l). The new tokens' l =
  // dt * A is formed only after every load is in flight: consuming a load
  // waits for all loads issued before it.
  // (Separate registers for the two loads: one register written by two loads
  // in flight would serialise them.)
  float2 dl_ring = make_float2(0.f, 0.f);
  float dt_new = 0.f;
  if (tid < n0) dl_ring = rdl[ring_slot(head, tid, R) * H];
  if (tid >= n0 && tid < L) dt_new = __builtin_nontemporal_load(dtin + (tid - n0) * H);
#pragma unroll
  for (int m = 0; m < kStageC; ++m) {
    const int q = m * NT + tid;
    if (q < totCV) {
      st_lds_f32(sC + q * VE, vc[m]);
      if constexpr (kMfRing) {
        if (mf_ring) *reinterpret_cast<VT*>(sCr + q * VE) = vc[m];
      }
    }
  }
  if (!xvec) {
#pragma unroll
    for (int m = 0; m < kStageS; ++m) {
      const int e = m * NT + tid;
      if (e < L * P) sX[e] = sxs[m];
    }
    for (int e0 = kStageS * NT; e0 < L * P; e0 += kStageS * NT) {  // long windows
#pragma unroll
      for (int m = 0; m < kStageS; ++m) {
        const int e = e0 + m * NT + tid;
        if (e < L * P) { const int j = xdiv(e); sxs[m] = xrow(j)[e - j * P]; }
      }
#pragma unroll
      for (int m = 0; m < kStageS; ++m) {
        const int e = e0 + m * NT + tid;
        if (e < L * P) sX[e] = sxs[m];
      }
    }
  }

  // Log-decay scan in wavefront 0: lam_i(j) = sum_{j < m <= t_i} l_m, tree-summed.
  float2 dl_new = make_float2(0.f, 0.f);
  if (wave == 0) {
    const bool fresh = tid >= n0 && tid < L;
    const float dtj = fresh ? dt_new : dl_ring.x;
    const float lj = fresh ? dt_new * Ah : dl_ring.y;
#pragma unroll
    for (int i = 0; i < NTMAX; ++i) {
      if (i >= nt) break;
      const int ti = n0 + i;
      const float u = lane <= ti ? lj : 0.f;
      const float lam = wave_suffix_excl(u, lane);
      if (lane < L) sCF[i * RL + lane] = lane <= ti ? expf(lam) * dtj : 0.f;
      if (lane == 0) sDC[i] = expf(lam + u);
    }
    if constexpr (FOLD) {  // the fold's coefficients: window entries 0..F-1 (zero past them)
      const float u = lane < F ? lj : 0.f;
      const float lam = wave_suffix_excl(u, lane);
      if (lane < lay.FD) sFC[lane] = lane < F ? expf(lam) * dtj : 0.f;
      if (lane == 0) sFC[lay.FD] = expf(lam + u);
    }
    dl_new = make_float2(dtj, lj);
  }
  __builtin_amdgcn_s_waitcnt(0);  // the direct-to-LDS loads have landed
  if constexpr (FOLD && LOW && !kB16Fold) {
    if (do_fold) {  // the fold reads entries in groups of four: rows past the window are zero
      const int F4 = align4(F);
      for (int q = tid; q < (F4 - F) * P; q += NT) sX[F * P + q] = Tin(0);
      for (int q = tid; q < (F4 - F) * N; q += NT) sB[F * N + q] = Tin(0);
    }
  }
  __syncthreads();
  // The new tokens' (dt, l) into the ring, only now: on this target a store
  // counts in the same counter as the loads, so a store issued before the wait
  // above would have been waited for too.
  if (wave == 0 && lane >= n0 && lane < L) rdl[ring_slot2(head, lane, R) * H] = dl_new;
  // The new pointer word (this workgroup's own copy, read only at its start). A
  // verify stores it as soon as the loads have landed (measured at batch 512,
  // K = 4: 430 -> 424 us); a decode stores it last (183.1 against 182.6 us).
  if constexpr (NTMAX > 1) {
    if (tid == 0) {
      if (do_fold) a.ptr[bh] = make_int4(ring_slot(head, F, R), L - F, a.set_tent ? nt : 0, 0);
      else a.ptr[bh] = make_int4(head, L, a.set_tent ? nt : pt.z, 0);
    }
  }

  // The new tokens' x and B rows go from LDS to the ring. A verify's K + 1
  // rows per head go out non-temporal (measured at batch 512, K = 4: verify
  // 492 -> 482 us); a decode's single row is faster cached.
  auto put16 = [&](Tin* dst, const Tin* src) {
    const VT v = *reinterpret_cast<const VT*>(src);
    if constexpr (NTMAX > 1) __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), reinterpret_cast<u32x4*>(dst));
    else *reinterpret_cast<VT*>(dst) = v;
  };
  if (xvec) {
    for (int q = tid; q < nt * PV; q += NT) {
      const int i = q / PV, c = q - i * PV;
      put16(rx + ring_slot2(head, n0 + i, R) * slx + c * VE, sX + (n0 + i) * P + c * VE);
    }
  } else {
    for (int e = tid; e < nt * P; e += NT) {
      const int i = e / P, p = e - i * P;
      rx[ring_slot2(head, n0 + i, R) * slx + p] = sX[(n0 + i) * P + p];
    }
  }
  if (h == g * hpg) {  // the group's first head keeps the group's B
    for (int q = tid; q < nt * NV; q += NT) {
      const int i = q / NV, c = q - i * NV;
      put16(rB + ring_slot2(head, n0 + i, R) * slb + c * VE, sB + (n0 + i) * N + c * VE);
    }
  }

  // The bf16 fold's A operand: the window's B rows transposed in groups of 16
  // entries, bt[j / 16][n][j % 16] (zero for j >= F), 16-byte writes of eight.
  bf16_t* bt = reinterpret_cast<bf16_t*>(lds + lay.oBT);
  const int F16 = (F + 15) & ~15;
  if constexpr (kB16Fold) {
    if (do_fold) {
      for (int q = tid; q < N * (F16 / 8); q += NT) {
        const int n = q % N, j0 = (q / N) * 8;
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int ja = j0 + 2 * e, jb = ja + 1;
          const uint32_t lo = ja < F ? (uint32_t)sB[ja * N + n] : 0u;
          const uint32_t hi = jb < F ? (uint32_t)sB[jb * N + n] : 0u;
          w[e] = lo | (hi << 16);
        }
        *reinterpret_cast<u32x4*>(bt + ((j0 >> 4) * N + n) * 16 + (j0 & 15)) = w;
      }
    }
  }

  // 3. w_ij = coef_ij (B_j . C_i) for every output i and window entry j <= t_i,
  // and each wavefront's share of sum_j w_ij x_j (wavefront w takes j = w mod
  // the number of wavefronts; row p on lane p mod 64). Rows are visited in
  // blocks of 64 up to P only (a uniform bound), so short heads spend no
  // instructions on the rows they do not have.
  constexpr int kRowsPerLane = kMaxP / 64;
  const int nrb = (P + 63) >> 6;
  auto ring_shares = [&](auto&& weight) {
    for (int i = 0; i < nt; ++i) {
      const int ti = n0 + i;
      float share[kRowsPerLane] = {};
      for (int j = wave; j <= ti; j += NW) {
        const float w = weight(i, j);
#pragma unroll
        for (int r = 0; r < kRowsPerLane; ++r) {
          if (r >= nrb) break;
          if (r * 64 + lane < P) share[r] = fmaf(w, to_f32(sX[j * P + r * 64 + lane]), share[r]);
        }
      }
#pragma unroll
      for (int r = 0; r < kRowsPerLane; ++r) {
        if (r >= nrb) break;
        if (r * 64 + lane < P) sRing[(wave * NTL + i) * P + r * 64 + lane] = share[r];
      }
    }
  };
  if (NTMAX == 1 || nt == 1) {
    // One output: its wavefront computes each dot over 64 lanes (wave_sum), in
    // the loop that accumulates the shares.
    ring_shares([&](int i, int j) {
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const int n = lane * EPL + e;
        if (n < N) part = fmaf(to_f32(sB[j * N + n]), sC[i * N + n], part);
      }
      return sCF[i * RL + j] * wave_sum(part);
    });
  } else if (mf_ring) {
    verify_weights_mfma<N>(reinterpret_cast<const bf16_t*>(sB), sCr, sCF, RL, L, nt, wave, NW, lane);
    __syncthreads();
    verify_shares_mfma<Tin>(sX, sCF, sRing, RL, P, L, nt, wave, NW, lane);
  } else {
    // Several outputs: all (i, j) dots first, one 16-lane group per pair (16
    // pairs in flight per workgroup pass, each lane a contiguous slice of N
    // read as 16-byte vectors, a 4-step butterfly inside the group); the
    // group's first lane overwrites coef_ij with w_ij. Then the shares read
    // w_ij back. Pairs run over the (entry j, output i) rectangle, j = q / nt
    // by a multiply (q < 2^16 / nt); the corner j > t_i is skipped.
    constexpr int GL = 16, EPG = N / GL;
    const int gl = tid & (GL - 1);
    const int npairs = nt * L;
    const int magic = (65536 + nt - 1) / nt;
    for (int q = tid / GL; q < npairs; q += NT / GL) {
      const int j = (q * magic) >> 16, i = q - j * nt;
      if (j > n0 + i) continue;
      float bv[EPG], cv[EPG];
      if constexpr (EPG % VE == 0) {
#pragma unroll
        for (int v = 0; v < EPG; v += VE) unpack16(*reinterpret_cast<const VT*>(sB + j * N + gl * EPG + v), bv + v);
      } else {
#pragma unroll
        for (int e = 0; e < EPG; ++e) bv[e] = to_f32(sB[j * N + gl * EPG + e]);
      }
      if constexpr (EPG % 4 == 0) {
#pragma unroll
        for (int v = 0; v < EPG; v += 4) {
          const float4 t = *reinterpret_cast<const float4*>(sC + i * N + gl * EPG + v);
          cv[v] = t.x; cv[v + 1] = t.y; cv[v + 2] = t.z; cv[v + 3] = t.w;
        }
      } else {
#pragma unroll
        for (int e = 0; e < EPG; ++e) cv[e] = sC[i * N + gl * EPG + e];
      }
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < EPG; ++e) part = fmaf(bv[e], cv[e], part);
      part = lanes_sum<4>(part);
      if (gl == 0) sCF[i * RL + j] *= part;
    }
    __syncthreads();
    ring_shares([&](int i, int j) { return sCF[i * RL + j]; });
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
      if constexpr (LOW && std::is_same<Tin, bf16_t>::value) {
        // bf16 tile, bf16 C (the stored inputs: exact as bf16): two exact
        // products per v_dot2_f32_bf16, summed in fp32
        uint32_t cp[VEC / 2];
#pragma unroll
        for (int q = 0; q < VEC / 2; ++q) cp[q] = pack_bf16x2(cv[2 * q], cv[2 * q + 1]);
#pragma unroll
        for (int k = 0; k < kMaxPass; ++k) {
          const uint32_t w[4] = {fr[k].v.x, fr[k].v.y, fr[k].v.z, fr[k].v.w};
          float acc = 0.f;
#pragma unroll
          for (int q = 0; q < VEC / 2; ++q)
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[q]),
                                                  __builtin_bit_cast(bf16x2_t, cp[q]), acc, false);
          part[k] = acc;
        }
      } else if constexpr (kDual) {
        // the read copy's values: RNE-bf16 of the master, two per packed conversion
#pragma unroll
        for (int k = 0; k < kMaxPass; ++k) {
          const uint32_t lo = pack_bf16x2(fr[k].v.x, fr[k].v.y), hi = pack_bf16x2(fr[k].v.z, fr[k].v.w);
          const float q[4] = {__uint_as_float(lo << 16), __uint_as_float(lo & 0xffff0000u),
                              __uint_as_float(hi << 16), __uint_as_float(hi & 0xffff0000u)};
          float acc = 0.f;
#pragma unroll
          for (int v = 0; v < VEC; ++v) acc = fmaf(q[v], cv[v], acc);
          part[k] = acc;
        }
      } else {
#pragma unroll
        for (int k = 0; k < kMaxPass; ++k) {
          float acc = 0.f;
#pragma unroll
          for (int v = 0; v < VEC; ++v) acc = fmaf(fr[k].get(v), cv[v], acc);
          part[k] = acc;
        }
      }
      int kbase;
      RS::run(part, col, kbase);
      if ((col & RS::WMASK) == 0) {
#pragma unroll
        for (int m = 0; m < RS::NOUT; ++m) {
          const int row = rows.row(base, kbase + m);
          if (row < P) {
            float ring;
            if (mf_ring)
              ring = sRing[i * P + row];
            else if constexpr (NW == 4)
              ring = (sRing[i * P + row] + sRing[(NTL + i) * P + row]) +
                     (sRing[(2 * NTL + i) * P + row] + sRing[(3 * NTL + i) * P + row]);
            else
              ring = sRing[i * P + row] + sRing[(NTL + i) * P + row];
            // a verify's K+1 outputs per head go out non-temporal (measured: verify
            // 528 -> 520 us at batch 512; a decode's single output is faster cached)
            if constexpr (NTMAX > 1) __builtin_nontemporal_store(fmaf(sDC[i], part[m], ring), yout + i * xstr + row);
            else yout[i * xstr + row] = fmaf(sDC[i], part[m], ring);
          }
        }
      }
    }
    if constexpr (FOLD && LOW) {
      if (do_fold && rows.wave_row(base, 0, wave) < P) {
        // bf16-stored checkpoint: widened to fp32, folded on the matrix cores
        // (the flush's operands and order), stored RNE-bf16
        const float D = sFC[lay.FD];
        bf16_t* out = static_cast<bf16_t*>(a.ckpt_lo) + (size_t)bh * P * N;
        auto fin = [&](int k, const float (&d)[8]) {
          float o[8];
#pragma unroll
          for (int v = 0; v < 8; ++v) o[v] = fmaf(D, fr[k].get(v), d[v]);
          const int row = rows.row(base, k);
          if (row < P) st16_bf16x8(out + row * N + col * 8, o);
        };
        float* buf = lds + lay.oW + wave * Fold::BUF;
        if constexpr (kB16Fold) {
          Fold::run_b16(rows.wave_row(base, 0, wave), P, F16, bt, buf, lane, col,
                        [&](int j, int p) {  // v_j[p] = c_j x_j[p], zero past the window
                          const int jr = j < F ? j : 0;
                          const float v = sFC[jr] * to_f32(sX[jr * P + p]);
                          return j < F ? v : 0.f;
                        },
                        fin);
        } else {
          Fold::run(rows.wave_row(base, 0, wave), P, align4(F), buf, lane, col,
                    [&](int j, int c) { return sFC[j] * to_f32(sB[j * N + c]); },
                    [&](int j, int p) { return to_f32(sX[j * P + p]); }, fin);
        }
      }
    } else if constexpr (FOLD) {
      if (do_fold) {  // S <- exp(Lam) S + sum_j x_j outer (c_j B_j), j ascending
        const float D = sFC[lay.FD];
#pragma unroll
        for (int k = 0; k < kMaxPass; ++k) {
          fr[k].v.x *= D;
          fr[k].v.y *= D;
          fr[k].v.z *= D;
          fr[k].v.w *= D;
        }
        for (int j = 0; j < F; ++j) {
          const float cj = sFC[j];
          float bv[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) bv[v] = cj * to_f32(sB[j * N + col * 4 + v]);
#pragma unroll
          for (int k = 0; k < kMaxPass; ++k) {
            if (rows.wave_row(base, k, wave) >= P) break;
            const int r = rows.row(base, k);
            const int row = r < P ? r : P - 1;   // rows past P: result unused
            const float xv = to_f32(sX[j * P + row]);
            fr[k].v.x = fmaf(xv, bv[0], fr[k].v.x);
            fr[k].v.y = fmaf(xv, bv[1], fr[k].v.y);
            fr[k].v.z = fmaf(xv, bv[2], fr[k].v.z);
            fr[k].v.w = fmaf(xv, bv[3], fr[k].v.w);
          }
        }
        float* out = a.ckpt + (size_t)bh * P * N;
#pragma unroll
        for (int k = 0; k < kMaxPass; ++k) {
          const int row = rows.row(base, k);
          if (row < P) st16(out + row * N + col * 4, fr[k].v);
        }
        if constexpr (kDual) {  // the new read copy: RNE-bf16 of the new master
          bf16_t* lo = static_cast<bf16_t*>(a.ckpt_lo) + (size_t)bh * P * N;
#pragma unroll
          for (int k = 0; k < kMaxPass; ++k) {
            const int row = rows.row(base, k);
            if (row < P) st8_bf16x4(lo + row * N + col * 4, fr[k].v);
          }
        }
      }
    }
  }

  if constexpr (NTMAX == 1) {
    if (tid == 0) {
      if (do_fold) a.ptr[bh] = make_int4(ring_slot(head, F, R), L - F, a.set_tent ? nt : 0, 0);
      else a.ptr[bh] = make_int4(head, L, a.set_tent ? nt : pt.z, 0);
    }
  }
}

template <int N, typename Tin, bool LOW, int NTMAX, int FOLD, int NT = kThreads>
static hipError_t launch_one(const ReplayArgs& a, int batch, hipStream_t s) {
  constexpr int VEC = TileGeom<N, LOW, NT>::VEC;
  constexpr bool kB16Fold = FOLD && LOW && std::is_same<Tin, bf16_t>::value;
  const int RL = a.R + ((FOLD && NTMAX > 1) ? a.nt : 0);
  const size_t lds =
      (size_t)ReplayLds(RL, a.P, N, a.nt, (int)sizeof(Tin), NT / 64,
                        (FOLD && LOW) ? fold_buf_floats(N, VEC, kMaxPass) : 0,
                        kB16Fold ? fold_bt_elems(N, RL) : 0)
          .total * sizeof(float);
  auto kern = replay_kernel<N, Tin, LOW, NTMAX, FOLD, NT>;
  if (lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)((size_t)batch * a.H)), dim3(NT), lds, s, a);
  return hipGetLastError();
}

template <int N, typename Tin, bool LOW>
static hipError_t launch_nt(const ReplayArgs& a, int batch, hipStream_t s) {
  const bool fold = a.fold_min_len > 0 || a.fold_min_len_dev;
  if (a.nt != 1 || (fold && a.set_tent)) {   // verify (a folding verify of one token too)
    if constexpr (!LOW) {
      if (fold) return launch_one<N, Tin, LOW, kMaxNew, 1>(a, batch, s);
    } else {
      if (fold) return hipErrorInvalidValue;
    }
    return launch_one<N, Tin, LOW, kMaxNew, 0>(a, batch, s);
  }
  if constexpr (LOW) {
    // A bf16 tile is half the bytes: two wavefronts per (sequence, head) hold
    // it in the same 8 fragments per lane, and twice as many workgroups fit on
    // a CU, so twice the bytes are in flight. A fold writes the bf16 tile back:
    // only for a bf16-stored checkpoint (a dual-precision layer folds its fp32
    // master, which this kernel never reads).
    if (fold) return launch_one<N, Tin, LOW, 1, 1, 128>(a, batch, s);
    return launch_one<N, Tin, LOW, 1, 0, 128>(a, batch, s);
  } else {
    if (fold && a.dual_fold) return launch_one<N, Tin, LOW, 1, 2>(a, batch, s);
    if (fold) return launch_one<N, Tin, LOW, 1, 1>(a, batch, s);
    return launch_one<N, Tin, LOW, 1, 0>(a, batch, s);
  }
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

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
// précisions pour le prix d'une"); the fold reads the master only.
//
// Rollback (P2, "Un retour en arrière qui devient trivial") touches integers
// only: len -= n_drop, n_tent = 0.
#include "device.h"
#include "launch.h"

namespace rss {

constexpr int kFlushChunk = 16;  // window entries staged in LDS at a time

template <int N, typename Tin, bool DUAL>
__global__ __launch_bounds__(kThreads) void flush_kernel(FlushArgs a) {
  using Geo = TileGeom<N, false>;
  constexpr int TPR = Geo::TPR, RPP = Geo::RPP;
  constexpr int EC = kFlushChunk;

  __shared__ float sl[kMaxRing];
  __shared__ float sdt[kMaxRing];
  __shared__ float sc[kMaxRing];
  __shared__ float sD;
  extern __shared__ __align__(16) float dyn[];  // xs[EC][P] (c_j x_j), then Bs[EC][N]

  const int tid = threadIdx.x;
  const int H = a.H, P = a.P, G = a.G, R = a.R;
  const int bh = blockIdx.x;
  const int b = bh / H, h = bh - b * H;
  const int g = h / (H / G);
  const int4 pt = a.ptr[bh];
  const int head = pt.x, n = pt.y;
  if (n == 0 || n < a.min_len) return;
  if (head < 0 || head >= R || n < 0 || n > R) {  // corrupt pointers: never index with them
    if (tid == 0) atomicOr(a.err, kDevRingOverflow);
    return;
  }
  if (pt.z != 0) {  // tentative entries were never committed
    if (tid == 0) atomicOr(a.err, kDevUncommitted);
    return;
  }
  float* xs = dyn;
  float* Bs = dyn + EC * P;
  const Tin* rx = static_cast<const Tin*>(a.ring_x);
  const Tin* rB = static_cast<const Tin*>(a.ring_B);

  const int col = tid % TPR, rsub = tid / TPR;
  float* tile = a.ckpt + (size_t)bh * P * N;
  Frag<false> fr[kMaxPass];
  auto load_chunk = [&](int base) {
#pragma unroll
    for (int k = 0; k < kMaxPass; ++k) {
      const int row = base + k * RPP + rsub;
      if (row < P) fr[k].v = ld16(tile + (size_t)row * N + col * 4);
      else fr[k].v = float4{};
    }
  };
  load_chunk(0);

  if (tid < n) {
    const float2 v = a.ring_dl[(size_t)bh * R + ring_slot(head, tid, R)];
    sdt[tid] = v.x;
    sl[tid] = v.y;
  }
  __syncthreads();
  if (tid < n) {
    float lam = 0.f;
    for (int m = n - 1; m > tid; --m) lam += sl[m];
    sc[tid] = expf(lam) * sdt[tid];
  }
  if (tid == kThreads - 1) {
    float lam = 0.f;
    for (int m = n - 1; m >= 0; --m) lam += sl[m];
    sD = expf(lam);
  }
  __syncthreads();
  const float D = sD;

  for (int base = 0; base < P; base += RPP * kMaxPass) {
    if (base > 0) load_chunk(base);
    float4 acc[kMaxPass];
#pragma unroll
    for (int k = 0; k < kMaxPass; ++k) {
      acc[k].x = D * fr[k].v.x;
      acc[k].y = D * fr[k].v.y;
      acc[k].z = D * fr[k].v.z;
      acc[k].w = D * fr[k].v.w;
    }
    for (int j0 = 0; j0 < n; j0 += EC) {
      const int ne = min(EC, n - j0);
      if (j0 > 0 || base > 0) __syncthreads();  // earlier readers of xs/Bs are done
      for (int e = tid; e < ne * P; e += kThreads) {
        const int jj = e / P, p = e - jj * P;
        const int slot = ring_slot(head, j0 + jj, R);
        xs[jj * P + p] = sc[j0 + jj] * to_f32(rx[((size_t)bh * R + slot) * P + p]);
      }
      for (int e = tid; e < ne * N; e += kThreads) {
        const int jj = e / N, c = e - jj * N;
        const int slot = ring_slot(head, j0 + jj, R);
        Bs[jj * N + c] = to_f32(rB[(((size_t)b * G + g) * R + slot) * N + c]);
      }
      __syncthreads();
      for (int jj = 0; jj < ne; ++jj) {
        const float4 bv = *reinterpret_cast<const float4*>(&Bs[jj * N + col * 4]);
#pragma unroll
        for (int k = 0; k < kMaxPass; ++k) {
          if (base + k * RPP >= P) break;
          const int row = base + k * RPP + rsub;
          const float xv = row < P ? xs[jj * P + row] : 0.f;
          acc[k].x = fmaf(xv, bv.x, acc[k].x);
          acc[k].y = fmaf(xv, bv.y, acc[k].y);
          acc[k].z = fmaf(xv, bv.z, acc[k].z);
          acc[k].w = fmaf(xv, bv.w, acc[k].w);
        }
      }
    }
#pragma unroll
    for (int k = 0; k < kMaxPass; ++k) {
      const int row = base + k * RPP + rsub;
      if (row < P) {
        *reinterpret_cast<float4*>(tile + (size_t)row * N + col * 4) = acc[k];
        if (DUAL) {
          bf16_t* lo = static_cast<bf16_t*>(a.ckpt_lo) + (size_t)bh * P * N + (size_t)row * N + col * 4;
          uint2 pk;
          pk.x = (uint32_t)f32_to_bf16(acc[k].x) | ((uint32_t)f32_to_bf16(acc[k].y) << 16);
          pk.y = (uint32_t)f32_to_bf16(acc[k].z) | ((uint32_t)f32_to_bf16(acc[k].w) << 16);
          *reinterpret_cast<uint2*>(lo) = pk;
        }
      }
    }
  }
  if (tid == 0) a.ptr[bh] = make_int4(ring_slot(head, n, R), 0, 0, 0);
}

template <int N, typename Tin>
static hipError_t flush_dual(const FlushArgs& a, int batch, bool low, hipStream_t s) {
  const dim3 grid((unsigned)((size_t)batch * a.H)), block(kThreads);
  const size_t lds = (size_t)kFlushChunk * (a.P + N) * sizeof(float);
  if (low) hipLaunchKernelGGL((flush_kernel<N, Tin, true>), grid, block, lds, s, a);
  else hipLaunchKernelGGL((flush_kernel<N, Tin, false>), grid, block, lds, s, a);
  return hipGetLastError();
}

template <int N>
static hipError_t flush_n(const FlushArgs& a, int batch, bool bf16_in, bool low, hipStream_t s) {
  return bf16_in ? flush_dual<N, bf16_t>(a, batch, low, s) : flush_dual<N, float>(a, batch, low, s);
}

hipError_t launch_flush(const FlushArgs& a, int batch, int N, bool bf16_in, bool low_copy,
                        hipStream_t s) {
  switch (N) {
    case 16: return flush_n<16>(a, batch, bf16_in, low_copy, s);
    case 32: return flush_n<32>(a, batch, bf16_in, low_copy, s);
    case 64: return flush_n<64>(a, batch, bf16_in, low_copy, s);
    case 128: return flush_n<128>(a, batch, bf16_in, low_copy, s);
    case 256: return flush_n<256>(a, batch, bf16_in, low_copy, s);
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
    reinterpret_cast<float4*>(a.ckpt)[i] = v;
    if (a.ckpt_lo) {
      uint2 pk;
      pk.x = (uint32_t)f32_to_bf16(v.x) | ((uint32_t)f32_to_bf16(v.y) << 16);
      pk.y = (uint32_t)f32_to_bf16(v.z) | ((uint32_t)f32_to_bf16(v.w) << 16);
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

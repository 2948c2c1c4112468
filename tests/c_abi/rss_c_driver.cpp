// A plain C++ caller of librss: no torch, no Python. It allocates every buffer
// itself from rss_buffer_sizes, binds a layer, runs a decode loop and then
// speculative rounds through the C entry points, and writes the outputs, the
// final checkpoint and the pointers to a file, so that a test can check them
// against the fp64 oracle.
//
// usage: rss_c_driver <input> <output>
//   input  (little-endian): int32 header[16] = {magic 0x52535334, Bt, H, P, N,
//          G, W, R, T, has_S0, fused, K, rounds, bf16, read_copy, kind}; fp32
//          A[H]; fp32 S0[Bt*H*P*N] if has_S0; then per step t < T:
//          Mamba-2: x[Bt*H*P], B[Bt*G*N], C[Bt*G*N] (fp32, or raw bf16 bits if
//          bf16), fp32 dt[Bt*H]; Gated DeltaNet / KDA (fp32, K = rounds = 0):
//          q[Bt*H*N], k[Bt*H*N], v[Bt*H*P], beta[Bt*H], alpha[Bt*H] (GDN) or
//          [Bt*H*N] (KDA); then per round: x[Bt*(K+1)*H*P], B and
//          C[Bt*(K+1)*G*N] (same element type), fp32 dt[Bt*(K+1)*H], int32
//          n_drop[Bt].
//   output: fp32 y[T][Bt*H*P]; fp32 yr[rounds][Bt*(K+1)*H*P]; the ckpt
//          buffer's bytes (fp32, or bf16 with read_copy = RSS_STATE_BF16);
//          the ckpt_lo buffer's bytes (bf16, read_copy = RSS_COPY_BF16 only);
//          int32 ptr[Bt*H*4]; int32 device error word.
// fused = 0 runs rss_decode_step then rss_flush_checkpoint(W) every step;
// fused = 1 runs rss_decode_flush_step(W) (the rss_gdn_ / rss_kda_ forms for
// those kinds). A round is
// rss_verify_k_tokens_fold(W, K) then rss_rollback(n_drop). Exit status 0 only
// if every call returned RSS_OK.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <vector>

#include "rss.h"

namespace {

int fail(const char* what, int code) {
  std::fprintf(stderr, "rss_c_driver: %s failed (%d: %s)\n", what, code,
               code >= 0 && code < 16 ? rss_status_string(code) : "");
  return 1;
}

#define HIP_OK(call)                                                                   \
  do {                                                                                 \
    hipError_t e_ = (call);                                                            \
    if (e_ != hipSuccess) {                                                            \
      std::fprintf(stderr, "rss_c_driver: %s: %s\n", #call, hipGetErrorString(e_));    \
      return 1;                                                                        \
    }                                                                                  \
  } while (0)

bool read_all(FILE* f, void* dst, size_t bytes) { return std::fread(dst, 1, bytes, f) == bytes; }

}  // namespace

int main(int argc, char** argv) {
  if (argc != 3) {
    std::fprintf(stderr, "usage: %s <input> <output>\n", argv[0]);
    return 2;
  }
  FILE* in = std::fopen(argv[1], "rb");
  if (!in) return fail("open input", -1);
  int32_t hd[16];
  if (!read_all(in, hd, sizeof(hd)) || hd[0] != 0x52535334) return fail("input header", -1);
  const int Bt = hd[1], H = hd[2], P = hd[3], N = hd[4], G = hd[5], W = hd[6], R = hd[7],
            T = hd[8], has_s0 = hd[9], fused = hd[10], K = hd[11], rounds = hd[12], bf16 = hd[13],
            copy = hd[14], kind = hd[15];
  const bool delta = kind != RSS_KIND_MAMBA2;
  if (delta && (K || rounds || bf16 || copy)) return fail("input header (delta-rule layer)", -1);
  const size_t es = bf16 ? 2 : 4;  // bytes per x, B, C element
  const size_t nS = (size_t)Bt * H * P * N, nx = (size_t)Bt * H * P, nB = (size_t)Bt * G * N,
               ndt = (size_t)Bt * H;
  // delta rules: q, k [Bt*H*N], v [Bt*H*P], beta [Bt*H], alpha [Bt*H] or [Bt*H*N]
  const size_t nq = (size_t)Bt * H * N, nal = kind == RSS_KIND_KDA ? nq : ndt;
  const size_t step_bytes = delta ? (2 * nq + nx + ndt + nal) * 4 : (nx + 2 * nB) * es + ndt * 4;
  const size_t round_bytes = (size_t)(K + 1) * step_bytes + (size_t)Bt * 4;

  rss_config cfg = {Bt, H, P, N, G, W, R, K, bf16 ? RSS_DTYPE_BF16 : RSS_DTYPE_F32, copy, kind};
  rss_sizes sz;
  int st = rss_buffer_sizes(&cfg, &sz);
  if (st != RSS_OK) return fail("rss_buffer_sizes", st);

  std::vector<float> A(H), S0(has_s0 ? nS : 0);
  std::vector<unsigned char> steps((size_t)T * step_bytes), rnds((size_t)rounds * round_bytes);
  if (!read_all(in, A.data(), A.size() * 4) || !read_all(in, S0.data(), S0.size() * 4) ||
      !read_all(in, steps.data(), steps.size()) || !read_all(in, rnds.data(), rnds.size()))
    return fail("input body", -1);
  std::fclose(in);

  rss_buffers dev = {};
  void* p[8] = {};
  const size_t bytes[8] = {sz.ckpt, sz.ckpt_lo, sz.ring_x, sz.ring_B, sz.ring_dl, sz.ptr, sz.A, sz.dev_err};
  for (int i = 0; i < 8; ++i)
    if (bytes[i]) HIP_OK(hipMalloc(&p[i], bytes[i]));
  dev.ckpt = p[0];
  dev.ckpt_lo = p[1];
  dev.ring_x = p[2];
  dev.ring_B = p[3];
  dev.ring_dl = static_cast<float*>(p[4]);
  dev.ptr = static_cast<int32_t*>(p[5]);
  dev.A = static_cast<const float*>(p[6]);
  dev.dev_err = static_cast<int32_t*>(p[7]);
  if (sz.A) HIP_OK(hipMemcpy(p[6], A.data(), sz.A, hipMemcpyHostToDevice));

  // input buffers sized for a round of K + 1 tokens (a decode step uses the first)
  const size_t nt = (size_t)K + 1;
  float *dS0 = nullptr, *ddt, *dy;
  void *dx, *dB, *dC;
  int32_t* dndrop;
  if (has_s0) {
    HIP_OK(hipMalloc(&dS0, nS * 4));
    HIP_OK(hipMemcpy(dS0, S0.data(), nS * 4, hipMemcpyHostToDevice));
  }
  HIP_OK(hipMalloc(&dx, nt * nx * es));
  HIP_OK(hipMalloc(&dB, nt * nB * es));
  HIP_OK(hipMalloc(&dC, nt * nB * es));
  HIP_OK(hipMalloc(&ddt, nt * ndt * 4));
  HIP_OK(hipMalloc(&dy, nt * nx * 4));
  HIP_OK(hipMalloc(&dndrop, (size_t)Bt * 4 + 16));
  float *dq = nullptr, *dk = nullptr, *dv = nullptr, *dbeta = nullptr, *dalpha = nullptr;
  if (delta) {
    HIP_OK(hipMalloc(&dq, nq * 4));
    HIP_OK(hipMalloc(&dk, nq * 4));
    HIP_OK(hipMalloc(&dv, nx * 4));
    HIP_OK(hipMalloc(&dbeta, ndt * 4));
    HIP_OK(hipMalloc(&dalpha, nal * 4));
  }

  rss_layer* layer = nullptr;
  st = rss_layer_bind(&cfg, &dev, &layer);
  if (st != RSS_OK) return fail("rss_layer_bind", st);
  hipStream_t s;
  HIP_OK(hipStreamCreate(&s));
  st = rss_init_state(layer, dS0, s);
  if (st != RSS_OK) return fail("rss_init_state", st);

  std::vector<float> y((size_t)T * nx), yr((size_t)rounds * nt * nx);
  const unsigned char* src = steps.data();
  for (int t = 0; t < T && delta; ++t) {
    const float* f = reinterpret_cast<const float*>(src);
    HIP_OK(hipMemcpyAsync(dq, f, nq * 4, hipMemcpyHostToDevice, s));
    HIP_OK(hipMemcpyAsync(dk, f + nq, nq * 4, hipMemcpyHostToDevice, s));
    HIP_OK(hipMemcpyAsync(dv, f + 2 * nq, nx * 4, hipMemcpyHostToDevice, s));
    HIP_OK(hipMemcpyAsync(dbeta, f + 2 * nq + nx, ndt * 4, hipMemcpyHostToDevice, s));
    HIP_OK(hipMemcpyAsync(dalpha, f + 2 * nq + nx + ndt, nal * 4, hipMemcpyHostToDevice, s));
    src += step_bytes;
    const bool kda = kind == RSS_KIND_KDA;
    if (fused) {
      st = kda ? rss_kda_decode_flush_step(layer, W, dq, dk, dv, dbeta, dalpha, dy, s)
               : rss_gdn_decode_flush_step(layer, W, dq, dk, dv, dbeta, dalpha, dy, s);
      if (st != RSS_OK) return fail("rss_*_decode_flush_step", st);
    } else {
      st = kda ? rss_kda_decode_step(layer, dq, dk, dv, dbeta, dalpha, dy, s)
               : rss_gdn_decode_step(layer, dq, dk, dv, dbeta, dalpha, dy, s);
      if (st != RSS_OK) return fail("rss_*_decode_step", st);
      st = rss_flush_checkpoint(layer, W, s);
      if (st != RSS_OK) return fail("rss_flush_checkpoint", st);
    }
    HIP_OK(hipMemcpyAsync(y.data() + (size_t)t * nx, dy, nx * 4, hipMemcpyDeviceToHost, s));
  }
  for (int t = 0; t < T && !delta; ++t) {
    HIP_OK(hipMemcpyAsync(dx, src, nx * es, hipMemcpyHostToDevice, s));
    HIP_OK(hipMemcpyAsync(dB, src + nx * es, nB * es, hipMemcpyHostToDevice, s));
    HIP_OK(hipMemcpyAsync(dC, src + (nx + nB) * es, nB * es, hipMemcpyHostToDevice, s));
    HIP_OK(hipMemcpyAsync(ddt, src + (nx + 2 * nB) * es, ndt * 4, hipMemcpyHostToDevice, s));
    src += step_bytes;
    if (fused) {
      st = rss_decode_flush_step(layer, W, dx, dB, dC, ddt, dy, s);
      if (st != RSS_OK) return fail("rss_decode_flush_step", st);
    } else {
      st = rss_decode_step(layer, dx, dB, dC, ddt, dy, s);
      if (st != RSS_OK) return fail("rss_decode_step", st);
      st = rss_flush_checkpoint(layer, W, s);
      if (st != RSS_OK) return fail("rss_flush_checkpoint", st);
    }
    HIP_OK(hipMemcpyAsync(y.data() + (size_t)t * nx, dy, nx * 4, hipMemcpyDeviceToHost, s));
  }
  src = rnds.data();
  for (int r = 0; r < rounds; ++r) {
    HIP_OK(hipMemcpyAsync(dx, src, nt * nx * es, hipMemcpyHostToDevice, s));
    HIP_OK(hipMemcpyAsync(dB, src + nt * nx * es, nt * nB * es, hipMemcpyHostToDevice, s));
    HIP_OK(hipMemcpyAsync(dC, src + nt * (nx + nB) * es, nt * nB * es, hipMemcpyHostToDevice, s));
    HIP_OK(hipMemcpyAsync(ddt, src + nt * (nx + 2 * nB) * es, nt * ndt * 4, hipMemcpyHostToDevice, s));
    HIP_OK(hipMemcpyAsync(dndrop, src + nt * step_bytes, (size_t)Bt * 4, hipMemcpyHostToDevice, s));
    src += round_bytes;
    st = rss_verify_k_tokens_fold(layer, W, K, dx, dB, dC, ddt, dy, s);
    if (st != RSS_OK) return fail("rss_verify_k_tokens_fold", st);
    st = rss_rollback(layer, dndrop, s);
    if (st != RSS_OK) return fail("rss_rollback", st);
    HIP_OK(hipMemcpyAsync(yr.data() + (size_t)r * nt * nx, dy, nt * nx * 4, hipMemcpyDeviceToHost, s));
  }
  int32_t err = -1;
  st = rss_get_device_error(layer, &err, s);  // synchronises the stream
  if (st != RSS_OK) return fail("rss_get_device_error", st);
  std::vector<unsigned char> ck(sz.ckpt), cl(sz.ckpt_lo);
  std::vector<int32_t> ptr((size_t)Bt * H * 4);
  HIP_OK(hipMemcpy(ck.data(), p[0], sz.ckpt, hipMemcpyDeviceToHost));
  if (sz.ckpt_lo) HIP_OK(hipMemcpy(cl.data(), p[1], sz.ckpt_lo, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(ptr.data(), p[5], ptr.size() * 4, hipMemcpyDeviceToHost));

  FILE* out = std::fopen(argv[2], "wb");
  if (!out) return fail("open output", -1);
  const bool ok = std::fwrite(y.data(), 4, y.size(), out) == y.size() &&
                  std::fwrite(yr.data(), 4, yr.size(), out) == yr.size() &&
                  std::fwrite(ck.data(), 1, ck.size(), out) == ck.size() &&
                  std::fwrite(cl.data(), 1, cl.size(), out) == cl.size() &&
                  std::fwrite(ptr.data(), 4, ptr.size(), out) == ptr.size() &&
                  std::fwrite(&err, 4, 1, out) == 1;
  std::fclose(out);
  if (!ok) return fail("write output", -1);

  rss_layer_free(layer);
  HIP_OK(hipStreamDestroy(s));
  for (void* q : p)
    if (q) HIP_OK(hipFree(q));
  for (void* q : {(void*)dS0, dx, dB, dC, (void*)ddt, (void*)dy, (void*)dndrop, (void*)dq, (void*)dk,
                  (void*)dv, (void*)dbeta, (void*)dalpha})
    if (q) HIP_OK(hipFree(q));
  return 0;
}

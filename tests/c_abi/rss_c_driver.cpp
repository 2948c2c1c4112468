// A plain C++ caller of librss: no torch, no Python. It allocates every buffer
// itself from rss_buffer_sizes, binds a layer, runs a decode loop through the C
// entry points and writes the outputs, the final checkpoint and the pointers
// to a file, so that a test can check them against the fp64 oracle.
//
// usage: rss_c_driver <input> <output>
//   input  (little-endian): int32 header[11] = {magic 0x52535331, Bt, H, P, N,
//          G, W, R, T, has_S0, fused}; fp32 A[H]; fp32 S0[Bt*H*P*N] if has_S0;
//          then per step t < T: fp32 x[Bt*H*P], B[Bt*G*N], C[Bt*G*N], dt[Bt*H].
//   output: fp32 y[T][Bt*H*P]; fp32 ckpt[Bt*H*P*N]; int32 ptr[Bt*H*4];
//          int32 device error word.
// fused = 0 runs rss_decode_step then rss_flush_checkpoint(W) every step;
// fused = 1 runs rss_decode_flush_step(W). Exit status 0 only if every call
// returned RSS_OK.
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
  int32_t hd[11];
  if (!read_all(in, hd, sizeof(hd)) || hd[0] != 0x52535331) return fail("input header", -1);
  const int Bt = hd[1], H = hd[2], P = hd[3], N = hd[4], G = hd[5], W = hd[6], R = hd[7],
            T = hd[8], has_s0 = hd[9], fused = hd[10];
  const size_t nS = (size_t)Bt * H * P * N, nx = (size_t)Bt * H * P, nB = (size_t)Bt * G * N,
               ndt = (size_t)Bt * H;

  rss_config cfg = {Bt, H, P, N, G, W, R, 0, RSS_DTYPE_F32, RSS_COPY_NONE, RSS_KIND_MAMBA2};
  rss_sizes sz;
  int st = rss_buffer_sizes(&cfg, &sz);
  if (st != RSS_OK) return fail("rss_buffer_sizes", st);

  std::vector<float> A(H), S0(has_s0 ? nS : 0), steps((size_t)T * (nx + 2 * nB + ndt));
  if (!read_all(in, A.data(), A.size() * 4) || !read_all(in, S0.data(), S0.size() * 4) ||
      !read_all(in, steps.data(), steps.size() * 4))
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
  HIP_OK(hipMemcpy(p[6], A.data(), sz.A, hipMemcpyHostToDevice));

  float *dS0 = nullptr, *dx, *dB, *dC, *ddt, *dy;
  if (has_s0) {
    HIP_OK(hipMalloc(&dS0, nS * 4));
    HIP_OK(hipMemcpy(dS0, S0.data(), nS * 4, hipMemcpyHostToDevice));
  }
  HIP_OK(hipMalloc(&dx, nx * 4));
  HIP_OK(hipMalloc(&dB, nB * 4));
  HIP_OK(hipMalloc(&dC, nB * 4));
  HIP_OK(hipMalloc(&ddt, ndt * 4));
  HIP_OK(hipMalloc(&dy, nx * 4));

  rss_layer* layer = nullptr;
  st = rss_layer_bind(&cfg, &dev, &layer);
  if (st != RSS_OK) return fail("rss_layer_bind", st);
  hipStream_t s;
  HIP_OK(hipStreamCreate(&s));
  st = rss_init_state(layer, dS0, s);
  if (st != RSS_OK) return fail("rss_init_state", st);

  std::vector<float> y((size_t)T * nx);
  const float* src = steps.data();
  for (int t = 0; t < T; ++t) {
    HIP_OK(hipMemcpyAsync(dx, src, nx * 4, hipMemcpyHostToDevice, s));
    HIP_OK(hipMemcpyAsync(dB, src + nx, nB * 4, hipMemcpyHostToDevice, s));
    HIP_OK(hipMemcpyAsync(dC, src + nx + nB, nB * 4, hipMemcpyHostToDevice, s));
    HIP_OK(hipMemcpyAsync(ddt, src + nx + 2 * nB, ndt * 4, hipMemcpyHostToDevice, s));
    src += nx + 2 * nB + ndt;
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
  int32_t err = -1;
  st = rss_get_device_error(layer, &err, s);  // synchronises the stream
  if (st != RSS_OK) return fail("rss_get_device_error", st);
  std::vector<float> ck(nS);
  std::vector<int32_t> ptr((size_t)Bt * H * 4);
  HIP_OK(hipMemcpy(ck.data(), p[0], nS * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(ptr.data(), p[5], ptr.size() * 4, hipMemcpyDeviceToHost));

  FILE* out = std::fopen(argv[2], "wb");
  if (!out) return fail("open output", -1);
  const bool ok = std::fwrite(y.data(), 4, y.size(), out) == y.size() &&
                  std::fwrite(ck.data(), 4, ck.size(), out) == ck.size() &&
                  std::fwrite(ptr.data(), 4, ptr.size(), out) == ptr.size() &&
                  std::fwrite(&err, 4, 1, out) == 1;
  std::fclose(out);
  if (!ok) return fail("write output", -1);

  rss_layer_free(layer);
  HIP_OK(hipStreamDestroy(s));
  for (void* q : p)
    if (q) HIP_OK(hipFree(q));
  for (float* q : {dS0, dx, dB, dC, ddt, dy})
    if (q) HIP_OK(hipFree(q));
  return 0;
}

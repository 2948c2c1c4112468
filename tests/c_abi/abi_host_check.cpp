// Host-side check of the C ABI's validation, binding, sizing and call-order
// logic, built with AddressSanitizer and UndefinedBehaviorSanitizer and run on
// the CPU. The kernel launchers are replaced by the stubs below: they launch
// nothing, record the arguments the dispatch code handed them, and return
// success, so every documented status and every call sequence (verify, then
// rollback; calls out of order) runs through the real rss_api.cpp without a
// GPU. A sanitizer report or a failed check ends the program with a non-zero
// status.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <initializer_list>

#include "../../include/rss.h"
#include "../../recurrent_state_storage_amd/csrc/launch.h"

namespace {
int g_fail = 0;
int g_launches = 0;
rss::ReplayArgs g_last_replay;
bool g_last_replay_low = false;   // the replay launcher was asked for the bf16 tile geometry
rss::FlushArgs g_last_flush;
int g_last_flush_kind = -1;
}  // namespace

#define CHECK(cond)                                                        \
  do {                                                                     \
    if (!(cond)) {                                                         \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond);   \
      ++g_fail;                                                            \
    }                                                                      \
  } while (0)

// ---- stub launchers (same signatures as launch.h) ----------------------------
namespace rss {
hipError_t launch_replay(const ReplayArgs& a, int, int, bool, bool low, hipStream_t) {
  ++g_launches;
  g_last_replay = a;
  g_last_replay_low = low;
  return hipSuccess;
}
hipError_t launch_flush(const FlushArgs& a, int, int, bool, int, int kind, hipStream_t) {
  ++g_launches;
  g_last_flush = a;
  g_last_flush_kind = kind;
  return hipSuccess;
}
hipError_t launch_init(const InitArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_rollback(const RollbackArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_eager(const EagerArgs&, int, int, bool, bool, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_gdn_replay(const GdnArgs&, int, int, bool, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_gdn_eager(const GdnEagerArgs&, int, int, bool, hipStream_t) { ++g_launches; return hipSuccess; }
}  // namespace rss

// ---- helpers -------------------------------------------------------------------
static rss_config cfg_base() {
  rss_config c;
  c.batch = 4; c.nheads = 8; c.headdim = 64; c.dstate = 128; c.ngroups = 8; c.window = 16;
  c.capacity = 20; c.max_draft = 4; c.in_dtype = RSS_DTYPE_BF16; c.read_copy = RSS_COPY_NONE;
  c.kind = RSS_KIND_MAMBA2;
  return c;
}

// Aligned fake device addresses: the host code never dereferences them.
static void* fake(int i) { return reinterpret_cast<void*>((uintptr_t)0x100000 * (uintptr_t)(i + 1)); }

static rss_buffers bufs_for(const rss_config& c) {
  rss_buffers b;
  b.ckpt = fake(0);
  b.ckpt_lo = c.read_copy == RSS_COPY_BF16 ? fake(1) : nullptr;
  b.ring_x = fake(2);
  b.ring_B = fake(3);
  b.ring_dl = static_cast<float*>(fake(4));
  b.ptr = static_cast<int32_t*>(fake(5));
  b.A = static_cast<const float*>(fake(6));
  b.dev_err = static_cast<int32_t*>(fake(7));
  return b;
}

static int32_t sizes(const rss_config& c) {
  rss_sizes s;
  return rss_buffer_sizes(&c, &s);
}

int main() {
  // version and status strings
  CHECK(rss_version() > 0);
  for (int s = -3; s < 12; ++s) CHECK(rss_status_string(s) != nullptr && strlen(rss_status_string(s)) > 0);

  // sizes
  {
    rss_config c = cfg_base();
    rss_sizes s;
    CHECK(rss_buffer_sizes(&c, &s) == RSS_OK);
    CHECK(s.ckpt == (size_t)4 * 8 * 64 * 128 * 4 && s.ckpt_lo == 0);
    CHECK(s.ring_x == (size_t)4 * 8 * 20 * 64 * 2 && s.ring_B == (size_t)4 * 8 * 20 * 128 * 2);
    CHECK(s.ring_dl == (size_t)4 * 8 * 20 * 2 * 4 && s.ptr == (size_t)4 * 8 * 16);
    CHECK(rss_buffer_sizes(nullptr, &s) == RSS_E_INVALID);
    CHECK(rss_buffer_sizes(&c, nullptr) == RSS_E_INVALID);
    c.kind = RSS_KIND_KDA; c.max_draft = 0; c.in_dtype = RSS_DTYPE_F32;
    CHECK(rss_buffer_sizes(&c, &s) == RSS_OK && s.ring_dl == (size_t)4 * 8 * 20 * 128 * 4 && s.A == 0);
  }

  // invalid configurations: every documented class of error
  {
    struct Case { void (*f)(rss_config&); int32_t want; };
    const Case cases[] = {
        {[](rss_config& c) { c.dstate = 96; }, RSS_E_SHAPE},
        {[](rss_config& c) { c.dstate = 8; }, RSS_E_SHAPE},
        {[](rss_config& c) { c.headdim = 0; }, RSS_E_SHAPE},
        {[](rss_config& c) { c.headdim = 257; }, RSS_E_SHAPE},
        {[](rss_config& c) { c.nheads = 6; c.ngroups = 4; }, RSS_E_SHAPE},
        {[](rss_config& c) { c.ngroups = 0; }, RSS_E_SHAPE},
        {[](rss_config& c) { c.batch = -1; }, RSS_E_SHAPE},
        {[](rss_config& c) { c.batch = 0x7fffffff; c.nheads = 2; c.ngroups = 2; }, RSS_E_SHAPE},
        {[](rss_config& c) { c.window = 0; }, RSS_E_SHAPE},
        {[](rss_config& c) { c.capacity = 65; }, RSS_E_SHAPE},
        {[](rss_config& c) { c.capacity = 19; }, RSS_E_CAPACITY},
        {[](rss_config& c) { c.max_draft = 8; c.capacity = 30; }, RSS_E_CAPACITY},
        {[](rss_config& c) { c.max_draft = -1; }, RSS_E_CAPACITY},
        {[](rss_config& c) { c.in_dtype = 7; }, RSS_E_DTYPE},
        {[](rss_config& c) { c.read_copy = 3; }, RSS_E_DTYPE},
        {[](rss_config& c) { c.kind = 3; }, RSS_E_INVALID},
        {[](rss_config& c) { c.kind = RSS_KIND_GDN; c.max_draft = 0; }, RSS_E_DTYPE},
        {[](rss_config& c) { c.kind = RSS_KIND_GDN; c.in_dtype = RSS_DTYPE_F32; }, RSS_E_CAPACITY},
        {[](rss_config& c) { c.headdim = 256; c.dstate = 256; c.window = 57; c.capacity = 64;
                             c.max_draft = 7; c.in_dtype = RSS_DTYPE_F32; }, RSS_E_SHAPE},
    };
    for (const Case& k : cases) {
      rss_config c = cfg_base();
      k.f(c);
      CHECK(sizes(c) == k.want);
      rss_layer* h = reinterpret_cast<rss_layer*>(0x1);
      rss_buffers b = bufs_for(cfg_base());
      CHECK(rss_layer_bind(&c, &b, &h) == k.want && h == nullptr);
    }
  }

  // binding: null and misaligned buffers, and a good bind
  {
    rss_config c = cfg_base();
    rss_layer* h = nullptr;
    CHECK(rss_layer_bind(&c, nullptr, &h) == RSS_E_INVALID);
    CHECK(rss_layer_bind(&c, nullptr, nullptr) == RSS_E_INVALID);
    for (int which = 0; which < 7; ++which) {
      for (int mis = 0; mis < 2; ++mis) {
        rss_buffers b = bufs_for(c);
        void** slots[] = {&b.ckpt, &b.ring_x, &b.ring_B, reinterpret_cast<void**>(&b.ring_dl),
                          reinterpret_cast<void**>(&b.ptr), reinterpret_cast<void**>(const_cast<float**>(&b.A)),
                          reinterpret_cast<void**>(&b.dev_err)};
        *slots[which] = mis ? static_cast<char*>(*slots[which]) + 4 : nullptr;
        CHECK(rss_layer_bind(&c, &b, &h) == RSS_E_INVALID && h == nullptr);
      }
    }
    rss_config dual = cfg_base();
    dual.read_copy = RSS_COPY_BF16;
    rss_buffers b = bufs_for(c);   // no ckpt_lo
    CHECK(rss_layer_bind(&dual, &b, &h) == RSS_E_INVALID);
    b = bufs_for(dual);
    CHECK(rss_layer_bind(&dual, &b, &h) == RSS_OK && h != nullptr);
    CHECK(rss_layer_free(h) == RSS_OK);
    CHECK(rss_layer_free(nullptr) == RSS_OK);
  }

  // a Mamba-2 layer: argument errors, call order, and what reaches the launcher
  {
    rss_config c = cfg_base();
    rss_buffers b = bufs_for(c);
    rss_layer* h = nullptr;
    CHECK(rss_layer_bind(&c, &b, &h) == RSS_OK);
    void* A = fake(9);
    char* Am = static_cast<char*>(A) + 4;
    const float* dt = static_cast<const float*>(A);
    float* y = static_cast<float*>(fake(10));
    const int32_t* dev_i = static_cast<const int32_t*>(fake(11));
    int32_t v = 0;
    CHECK(rss_rollback(h, dev_i, nullptr) == RSS_E_ORDER);
    CHECK(rss_decode_step(h, nullptr, A, A, dt, y, nullptr) == RSS_E_INVALID);
    CHECK(rss_decode_step(h, Am, A, A, dt, y, nullptr) == RSS_E_INVALID);
    CHECK(rss_decode_step(nullptr, A, A, A, dt, y, nullptr) == RSS_E_INVALID);
    CHECK(rss_verify_k_tokens(h, 5, A, A, A, dt, y, nullptr) == RSS_E_CAPACITY);
    CHECK(rss_verify_k_tokens(h, -1, A, A, A, dt, y, nullptr) == RSS_E_INVALID);
    CHECK(rss_verify_k_tokens_fold(h, 0, 2, A, A, A, dt, y, nullptr) == RSS_E_INVALID);
    CHECK(rss_verify_k_tokens_fold(h, 16, 5, A, A, A, dt, y, nullptr) == RSS_E_CAPACITY);
    CHECK(rss_flush_checkpoint(h, 0, nullptr) == RSS_E_INVALID);
    CHECK(rss_decode_flush_step(h, 0, A, A, A, dt, y, nullptr) == RSS_E_INVALID);
    CHECK(rss_decode_flush_step_each(h, nullptr, A, A, A, dt, y, nullptr) == RSS_E_INVALID);
    CHECK(rss_decode_flush_step_each(h, reinterpret_cast<const int32_t*>(Am), A, A, A, dt, y, nullptr) ==
          RSS_E_INVALID);
    CHECK(rss_flush_checkpoint_each(h, nullptr, nullptr) == RSS_E_INVALID);
    CHECK(rss_rollback(h, nullptr, nullptr) == RSS_E_INVALID);
    CHECK(rss_init_state(h, reinterpret_cast<const float*>(Am), nullptr) == RSS_E_INVALID);
    CHECK(rss_get_device_error(nullptr, &v, nullptr) == RSS_E_INVALID);
    CHECK(rss_get_device_error(h, nullptr, nullptr) == RSS_E_INVALID);
    CHECK(rss_gdn_decode_step(h, static_cast<const float*>(A), dt, dt, dt, dt, y, nullptr) == RSS_E_INVALID);
    CHECK(g_launches == 0);

    // good calls reach the launcher with the bound buffers
    CHECK(rss_init_state(h, nullptr, nullptr) == RSS_OK);
    CHECK(rss_decode_step(h, A, A, A, dt, y, nullptr) == RSS_OK);
    CHECK(g_last_replay.ckpt == b.ckpt && g_last_replay.ring_x == b.ring_x && g_last_replay.nt == 1);
    CHECK(g_last_replay.H == c.nheads && g_last_replay.P == c.headdim && g_last_replay.R == c.capacity);
    CHECK(g_last_replay.fold_min_len == 0 && g_last_replay.set_tent == 0);
    CHECK(rss_decode_flush_step(h, 16, A, A, A, dt, y, nullptr) == RSS_OK);
    CHECK(g_last_replay.fold_min_len == 16);
    CHECK(rss_flush_checkpoint(h, 16, nullptr) == RSS_OK && g_last_flush.min_len == 16);
    CHECK(g_last_flush_kind == rss::kFoldMamba2);
    // verify: a round stays pending until its rollback
    CHECK(rss_verify_k_tokens(h, 4, A, A, A, dt, y, nullptr) == RSS_OK && g_last_replay.nt == 5);
    CHECK(g_last_replay.set_tent == 1);
    CHECK(rss_decode_step(h, A, A, A, dt, y, nullptr) == RSS_E_ORDER);
    CHECK(rss_flush_checkpoint(h, 16, nullptr) == RSS_E_ORDER);
    CHECK(rss_verify_k_tokens(h, 4, A, A, A, dt, y, nullptr) == RSS_E_ORDER);
    CHECK(rss_rollback(h, dev_i, nullptr) == RSS_OK);
    CHECK(rss_rollback(h, dev_i, nullptr) == RSS_E_ORDER);
    CHECK(rss_verify_k_tokens_fold(h, 16, 4, A, A, A, dt, y, nullptr) == RSS_OK);
    CHECK(g_last_replay.fold_min_len == 16 && g_last_replay.nt == 5);
    CHECK(rss_rollback(h, dev_i, nullptr) == RSS_OK);
    // the ring-index division helper the kernels use: q / d == (q * xdiv) >> 32
    {
      const uint64_t d = c.headdim / 8;   // 16-byte bf16 vectors per x row
      for (uint32_t q = 0; q < (1u << 16); ++q) CHECK((uint32_t)((q * g_last_replay.xdiv) >> 32) == q / d);
    }
    CHECK(rss_layer_free(h) == RSS_OK);
  }

  // grouped B rows and the verify-fold capacity rules
  {
    rss_config big = cfg_base();
    big.window = 50; big.capacity = 60;
    rss_buffers b = bufs_for(big);
    rss_layer* h = nullptr;
    void* A = fake(9);
    const float* dt = static_cast<const float*>(A);
    float* y = static_cast<float*>(fake(10));
    CHECK(rss_layer_bind(&big, &b, &h) == RSS_OK);
    CHECK(rss_verify_k_tokens_fold(h, 50, 4, A, A, A, dt, y, nullptr) == RSS_E_CAPACITY);
    CHECK(rss_layer_free(h) == RSS_OK);
    rss_config grp = cfg_base();
    grp.ngroups = 4; grp.window = 8; grp.capacity = 12;
    b = bufs_for(grp);
    CHECK(rss_layer_bind(&grp, &b, &h) == RSS_OK);
    CHECK(rss_verify_k_tokens_fold(h, 8, 4, A, A, A, dt, y, nullptr) == RSS_E_CAPACITY);
    CHECK(rss_layer_free(h) == RSS_OK);
  }

  // delta-rule layers
  for (int kind : {RSS_KIND_GDN, RSS_KIND_KDA}) {
    rss_config c = cfg_base();
    c.kind = kind; c.max_draft = 0; c.in_dtype = RSS_DTYPE_F32;
    rss_buffers b = bufs_for(c);
    b.A = nullptr;   // unused by the delta rules
    rss_layer* h = nullptr;
    CHECK(rss_layer_bind(&c, &b, &h) == RSS_OK);
    const float* f = static_cast<const float*>(fake(9));
    float* o = static_cast<float*>(fake(10));
    auto dec = kind == RSS_KIND_GDN ? rss_gdn_decode_step : rss_kda_decode_step;
    auto other = kind == RSS_KIND_GDN ? rss_kda_decode_step : rss_gdn_decode_step;
    auto fold = kind == RSS_KIND_GDN ? rss_gdn_decode_flush_step : rss_kda_decode_flush_step;
    CHECK(dec(h, f, f, f, f, f, o, nullptr) == RSS_OK);
    CHECK(other(h, f, f, f, f, f, o, nullptr) == RSS_E_INVALID);
    CHECK(dec(h, nullptr, f, f, f, f, o, nullptr) == RSS_E_INVALID);
    CHECK(fold(h, 0, f, f, f, f, f, o, nullptr) == RSS_E_INVALID);
    CHECK(fold(h, 16, f, f, f, f, f, o, nullptr) == RSS_OK);
    CHECK(rss_decode_step(h, f, f, f, f, o, nullptr) == RSS_E_INVALID);
    CHECK(rss_flush_checkpoint(h, 16, nullptr) == RSS_OK);
    CHECK(g_last_flush_kind == (kind == RSS_KIND_GDN ? rss::kFoldGdn : rss::kFoldKda));
    auto eager = kind == RSS_KIND_GDN ? rss_gdn_eager_step : rss_kda_eager_step;
    CHECK(eager(&c, nullptr, f, f, f, f, f, o, nullptr) == RSS_E_INVALID);
    CHECK(eager(&c, o, f, f, f, f, f, o, nullptr) == RSS_OK);
    CHECK(eager(nullptr, o, f, f, f, f, f, o, nullptr) == RSS_E_INVALID);
    CHECK(rss_layer_free(h) == RSS_OK);
  }

  // eager baselines
  {
    rss_config c = cfg_base();
    void* S = fake(12);
    void* x = fake(9);
    const float* dt = static_cast<const float*>(x);
    float* y = static_cast<float*>(fake(10));
    const int32_t* slot = static_cast<const int32_t*>(fake(11));
    CHECK(rss_eager_step(&c, nullptr, x, x, x, dt, dt, y, 1, nullptr) == RSS_E_INVALID);
    CHECK(rss_eager_step(&c, S, x, x, x, dt, dt, y, 0, nullptr) == RSS_E_INVALID);
    CHECK(rss_eager_step(&c, S, x, x, x, dt, dt, y, 9, nullptr) == RSS_E_INVALID);
    CHECK(rss_eager_step(&c, S, x, x, x, dt, dt, y, 1, nullptr) == RSS_OK);
    CHECK(rss_eager_verify(&c, static_cast<float*>(S), nullptr, 4, x, x, x, dt, dt, y, nullptr) == RSS_E_INVALID);
    CHECK(rss_eager_verify(&c, static_cast<float*>(S), slot, 8, x, x, x, dt, dt, y, nullptr) == RSS_E_INVALID);
    CHECK(rss_eager_verify(&c, static_cast<float*>(S), slot, 4, x, x, x, dt, dt, y, nullptr) == RSS_OK);
    c.read_copy = RSS_STATE_BF16;
    CHECK(rss_eager_verify(&c, static_cast<float*>(S), slot, 4, x, x, x, dt, dt, y, nullptr) == RSS_E_DTYPE);
    c.read_copy = 5;
    CHECK(rss_eager_step(&c, S, x, x, x, dt, dt, y, 1, nullptr) == RSS_E_DTYPE);
  }

  // an empty batch: buffers may be null, calls succeed and launch nothing
  {
    rss_config c = cfg_base();
    c.batch = 0;
    rss_buffers b = bufs_for(c);
    b.ckpt = b.ring_x = b.ring_B = nullptr;
    b.ring_dl = nullptr;
    b.ptr = nullptr;
    rss_layer* h = nullptr;
    CHECK(rss_layer_bind(&c, &b, &h) == RSS_OK);
    const int before = g_launches;
    CHECK(rss_decode_step(h, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == RSS_OK);
    CHECK(rss_flush_checkpoint(h, 16, nullptr) == RSS_OK);
    CHECK(rss_verify_k_tokens(h, 2, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == RSS_OK);
    CHECK(rss_rollback(h, nullptr, nullptr) == RSS_OK);
    CHECK(g_launches == before);
    CHECK(rss_layer_free(h) == RSS_OK);
  }

  // dual precision: the one-pass fold from the fp32 master only on a token the
  // handle knows fills every window; the replay of the copy + the flush otherwise
  {
    rss_config c = cfg_base();
    c.read_copy = RSS_COPY_BF16;
    const int W = c.window;
    rss_buffers b = bufs_for(c);
    rss_layer* h = nullptr;
    CHECK(rss_layer_bind(&c, &b, &h) == RSS_OK);
    void* A = fake(9);
    const float* dt = static_cast<const float*>(A);
    float* y = static_cast<float*>(fake(10));
    const int32_t* dev_i = static_cast<const int32_t*>(fake(11));
    auto fused = [&](int min_len, bool one_pass) {
      const int before = g_launches;
      CHECK(rss_decode_flush_step(h, min_len, A, A, A, dt, y, nullptr) == RSS_OK);
      if (one_pass) {
        CHECK(g_launches == before + 1);
        CHECK(g_last_replay.dual_fold == 1 && !g_last_replay_low && g_last_replay.fold_min_len == min_len);
        CHECK(g_last_replay.ckpt == b.ckpt && g_last_replay.ckpt_lo == b.ckpt_lo);
      } else {
        CHECK(g_launches == before + 2);   // the replay of the copy, then the flush
        CHECK(g_last_replay.dual_fold == 0 && g_last_replay_low && g_last_replay.fold_min_len == 0);
        CHECK(g_last_flush.min_len == min_len);
      }
    };
    fused(W, false);                          // bound, never initialised: windows unknown
    CHECK(rss_init_state(h, nullptr, nullptr) == RSS_OK);
    for (int t = 0; t < W - 1; ++t) CHECK(rss_decode_step(h, A, A, A, dt, y, nullptr) == RSS_OK);
    fused(W, true);                           // the W-th token fills every window
    for (int t = 0; t < W - 1; ++t) fused(W, false);
    fused(W, true);
    fused(1, true);                           // a fold every token
    CHECK(rss_verify_k_tokens(h, 4, A, A, A, dt, y, nullptr) == RSS_OK);
    CHECK(rss_rollback(h, dev_i, nullptr) == RSS_OK);
    for (int t = 0; t < 2 * W; ++t) fused(W, false);   // windows uneven after the round
    CHECK(rss_flush_checkpoint(h, 1, nullptr) == RSS_OK);  // every window folded: in step
    for (int t = 0; t < W - 1; ++t) fused(W, false);
    fused(W, true);
    CHECK(rss_decode_flush_step_each(h, dev_i, A, A, A, dt, y, nullptr) == RSS_OK);
    CHECK(g_last_replay.dual_fold == 0);
    for (int t = 0; t < 2 * W; ++t) fused(W, false);   // per-sequence thresholds: unknown again
    CHECK(rss_init_state(h, nullptr, nullptr) == RSS_OK);
    for (int t = 0; t < c.capacity; ++t) CHECK(rss_decode_step(h, A, A, A, dt, y, nullptr) == RSS_OK);
    fused(W, false);                          // the ring is full: that token would overflow
    CHECK(rss_layer_free(h) == RSS_OK);
  }

  if (g_fail) {
    fprintf(stderr, "%d checks failed\n", g_fail);
    return 1;
  }
  printf("abi host checks passed (%d stub launches)\n", g_launches);
  return 0;
}

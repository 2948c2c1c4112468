// C ABI of librss: argument validation, call-order tracking and dispatch to the
// gfx950 kernels. Every check that the host can make happens here, before any
// launch, so a failing call leaves device state untouched.
#include <hip/hip_runtime_api.h>

#include <new>

#include "../../include/rss.h"
#include "launch.h"
#include "lds.h"

struct rss_layer {
  rss_config cfg;
  rss_buffers dev;
  int pending_verify;  // a verify round is waiting for its rollback
  // What the host knows of the windows: lock_len >= 0 when every sequence's
  // window holds exactly lock_len committed entries and none tentative (from
  // rss_init_state on, through plain decodes and folds of every window), -1 when
  // unknown (after speculative rounds or per-sequence thresholds). It only picks
  // a launch plan: every fold is still decided on the device from the pointers.
  int lock_len;
};

// A decode appended one entry to every window, and folded those that reached
// min_len (0: no fold).
static void lock_decode(rss_layer* l, int32_t min_len) {
  if (l->lock_len < 0 || l->lock_len >= l->cfg.capacity) {  // unknown, or the ring overflows
    l->lock_len = -1;
    return;
  }
  const int n = l->lock_len + 1;
  l->lock_len = (min_len > 0 && n >= min_len) ? 0 : n;
}

// A flush folded every window holding at least min_len entries.
static void lock_flush(rss_layer* l, int32_t min_len) {
  if (min_len == 1 || (l->lock_len >= 0 && l->lock_len >= min_len)) l->lock_len = 0;
}

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool supported_n(int32_t n) { return n == 16 || n == 32 || n == 64 || n == 128 || n == 256; }

int32_t check_shape(const rss_config* c) {
  if (!c) return RSS_E_INVALID;
  if (c->batch < 0 || c->nheads < 1 || c->ngroups < 1) return RSS_E_SHAPE;
  if (c->nheads % c->ngroups) return RSS_E_SHAPE;
  if (c->headdim < 1 || c->headdim > rss::kMaxP) return RSS_E_SHAPE;
  if (!supported_n(c->dstate)) return RSS_E_SHAPE;
  if ((int64_t)c->batch * c->nheads > 0x7fffffffLL) return RSS_E_SHAPE;
  if (c->in_dtype != RSS_DTYPE_F32 && c->in_dtype != RSS_DTYPE_BF16) return RSS_E_DTYPE;
  return RSS_OK;
}

// Largest dynamic LDS any kernel of this layer allocates per workgroup.
size_t layer_lds_bytes(const rss_config* c) {
  const int R = c->capacity, P = c->headdim, N = c->dstate;
  size_t m = 0;
  auto upd = [&m](int words) { if ((size_t)words * 4 > m) m = (size_t)words * 4; };
  if (c->kind == RSS_KIND_MAMBA2) {
    const int tin = c->in_dtype == RSS_DTYPE_BF16 ? 2 : 4;
    upd(rss::ReplayLds(R, P, N, 1, tin, c->read_copy == RSS_COPY_NONE ? 4 : 2).total);
    if (c->max_draft > 0) upd(rss::ReplayLds(R, P, N, c->max_draft + 1, tin, 4).total);
    // the bf16-stored checkpoint folds on the matrix cores (a decode that would
    // not fit runs its fold as the flush launch instead, so only the flush counts)
    const bool mf = c->read_copy == RSS_STATE_BF16;
    upd(rss::FlushLds(R, P, N, false, mf ? rss::fold_buf_floats(N, 4, rss::kMaxPass) : 0,
                      mf && tin == 2 ? rss::fold_bt_elems(N, R) : 0).total);
  } else {
    const bool kda = c->kind == RSS_KIND_KDA;
    upd(rss::GdnLds(R, P, N, kda, rss::fold_buf_floats(N, 4, rss::gdn_passes(P, N))).total);
    upd(rss::FlushLds(R, P, N, kda, rss::fold_buf_floats(N, 4, rss::kMaxPass)).total);
  }
  return m;
}

bool valid_mode(int32_t m) { return m == RSS_COPY_NONE || m == RSS_COPY_BF16 || m == RSS_STATE_BF16; }

int32_t check_config(const rss_config* c) {
  int32_t st = check_shape(c);
  if (st) return st;
  if (!valid_mode(c->read_copy)) return RSS_E_DTYPE;
  if (c->kind != RSS_KIND_MAMBA2 && c->kind != RSS_KIND_GDN && c->kind != RSS_KIND_KDA)
    return RSS_E_INVALID;
  if (c->kind != RSS_KIND_MAMBA2) {  // delta rules: one key per head, fp32, no read copy, no drafts
    if (c->ngroups != c->nheads) return RSS_E_SHAPE;
    if (c->in_dtype != RSS_DTYPE_F32 || c->read_copy != RSS_COPY_NONE) return RSS_E_DTYPE;
    if (c->max_draft != 0) return RSS_E_CAPACITY;
  }
  if (c->window < 1 || c->capacity < c->window || c->capacity > rss::kMaxRing) return RSS_E_SHAPE;
  if (c->max_draft < 0 || c->max_draft > rss::kMaxNew - 1) return RSS_E_CAPACITY;
  if (c->capacity < c->window + c->max_draft) return RSS_E_CAPACITY;
  // one sequence's ring rows (slot-major: R slots of H rows) stay within 32-bit
  // element offsets, as the kernels index them
  const int64_t row = c->headdim > c->dstate ? c->headdim : c->dstate;
  if ((int64_t)c->capacity * c->nheads * row > 0x7fffffffLL) return RSS_E_SHAPE;
  if (layer_lds_bytes(c) > (size_t)rss::kMaxLdsBytes) return RSS_E_SHAPE;
  return RSS_OK;
}

size_t in_bytes(const rss_config* c) { return c->in_dtype == RSS_DTYPE_BF16 ? 2 : 4; }

int32_t launch_status(hipError_t e) { return e == hipSuccess ? RSS_OK : RSS_E_HIP; }

// The fp32 checkpoint (null with a bf16-only checkpoint) and the bf16 tile the
// kernels read (the read copy, or the bf16-only checkpoint itself).
float* ckpt_f32(const rss_layer* l) {
  return l->cfg.read_copy == RSS_STATE_BF16 ? nullptr : static_cast<float*>(l->dev.ckpt);
}
void* ckpt_bf16(const rss_layer* l) {
  return l->cfg.read_copy == RSS_STATE_BF16 ? l->dev.ckpt : l->dev.ckpt_lo;
}

bool inputs_ok(const void* x, const void* B, const void* C, const void* dt, const void* y) {
  return x && B && C && dt && y && aligned16(x) && aligned16(B) && aligned16(C) &&
         aligned16(dt) && aligned16(y);
}

}  // namespace

extern "C" {

int32_t rss_version(void) { return 10600; }

const char* rss_status_string(int32_t s) {
  switch (s) {
    case RSS_OK: return "ok";
    case RSS_E_INVALID: return "invalid argument (null or misaligned pointer, bad value)";
    case RSS_E_SHAPE: return "unsupported or inconsistent sizes";
    case RSS_E_DTYPE: return "unknown dtype or read-copy mode";
    case RSS_E_CAPACITY: return "ring capacity too small (R < W + K_max) or K > K_max";
    case RSS_E_ORDER: return "call order violated (verify round uncommitted, or no round to roll back)";
    case RSS_E_HIP: return "HIP runtime call or kernel launch failed";
    default: return "unknown status";
  }
}

int32_t rss_buffer_sizes(const rss_config* c, rss_sizes* out) {
  if (!out) return RSS_E_INVALID;
  const int32_t st = check_config(c);
  if (st) return st;
  const size_t Bt = c->batch, H = c->nheads, P = c->headdim, N = c->dstate, G = c->ngroups,
               R = c->capacity;
  out->ckpt = Bt * H * P * N * (c->read_copy == RSS_STATE_BF16 ? 2 : 4);
  out->ckpt_lo = c->read_copy == RSS_COPY_BF16 ? Bt * H * P * N * 2 : 0;
  out->ring_x = Bt * H * R * P * in_bytes(c);
  out->ring_B = Bt * G * R * N * in_bytes(c);
  out->ring_dl = Bt * H * R * (c->kind == RSS_KIND_KDA ? N : 2) * 4;
  out->ptr = Bt * H * 4 * 4;
  out->A = c->kind == RSS_KIND_MAMBA2 ? H * 4 : 0;
  out->dev_err = 4;
  return RSS_OK;
}

int32_t rss_layer_bind(const rss_config* c, const rss_buffers* d, rss_layer** out) {
  if (!out) return RSS_E_INVALID;
  *out = nullptr;
  const int32_t st = check_config(c);
  if (st) return st;
  if (!d) return RSS_E_INVALID;
  if (!d->dev_err || !aligned16(d->dev_err)) return RSS_E_INVALID;
  if (c->kind == RSS_KIND_MAMBA2 && (!d->A || !aligned16(d->A))) return RSS_E_INVALID;  // delta rules: unused
  if (c->batch > 0) {  // with no sequences the per-sequence buffers may be empty (NULL)
    const void* req[] = {d->ckpt, d->ring_x, d->ring_B, d->ring_dl, d->ptr};
    for (const void* p : req)
      if (!p || !aligned16(p)) return RSS_E_INVALID;
    if (c->read_copy == RSS_COPY_BF16 && (!d->ckpt_lo || !aligned16(d->ckpt_lo)))
      return RSS_E_INVALID;
  }
  rss_layer* l = new (std::nothrow) rss_layer;
  if (!l) return RSS_E_INVALID;
  l->cfg = *c;
  l->dev = *d;
  if (c->read_copy != RSS_COPY_BF16) l->dev.ckpt_lo = nullptr;
  l->pending_verify = 0;
  l->lock_len = -1;
  *out = l;
  return RSS_OK;
}

int32_t rss_layer_free(rss_layer* l) {
  delete l;
  return RSS_OK;
}

int32_t rss_init_state(rss_layer* l, const float* S0, void* stream) {
  if (!l) return RSS_E_INVALID;
  if (S0 && !aligned16(S0)) return RSS_E_INVALID;
  const rss_config& c = l->cfg;
  rss::InitArgs a;
  a.ckpt = ckpt_f32(l);
  a.ckpt_lo = ckpt_bf16(l);
  a.S0 = S0;
  a.ptr = reinterpret_cast<int4*>(l->dev.ptr);
  a.err = l->dev.dev_err;
  a.n_state = (size_t)c.batch * c.nheads * c.headdim * c.dstate;
  a.n_ptr = (size_t)c.batch * c.nheads;
  l->pending_verify = 0;
  l->lock_len = 0;
  return launch_status(rss::launch_init(a, static_cast<hipStream_t>(stream)));
}

static int32_t replay_call(rss_layer* l, int nt, int set_tent, int fold_min_len,
                           const int32_t* fold_each, const void* x, const void* B, const void* C,
                           const float* dt, float* y, void* stream, int dual_fold = 0) {
  const rss_config& c = l->cfg;
  if (c.batch == 0) return RSS_OK;
  rss::ReplayArgs a;
  a.ckpt = ckpt_f32(l);
  a.ckpt_lo = ckpt_bf16(l);
  a.ring_x = l->dev.ring_x;
  a.ring_B = l->dev.ring_B;
  a.ring_dl = reinterpret_cast<float2*>(l->dev.ring_dl);
  a.ptr = reinterpret_cast<int4*>(l->dev.ptr);
  a.A = l->dev.A;
  a.err = l->dev.dev_err;
  a.x = x;
  a.B = B;
  a.C = C;
  a.dt = dt;
  a.y = y;
  a.H = c.nheads;
  a.P = c.headdim;
  a.G = c.ngroups;
  a.R = c.capacity;
  a.nt = nt;
  a.set_tent = set_tent;
  a.fold_min_len = fold_min_len;
  a.fold_min_len_dev = fold_each;
  const int ve = c.in_dtype == RSS_DTYPE_BF16 ? 8 : 4;  // elements per 16-byte vector
  const uint64_t d = c.headdim % ve == 0 ? (uint64_t)(c.headdim / ve) : (uint64_t)c.headdim;
  a.xdiv = ((1ull << 32) + d - 1) / d;
  a.dual_fold = dual_fold;
  // a dual fold reads the fp32 master in the fp32 tile geometry
  return launch_status(rss::launch_replay(a, c.batch, c.dstate, c.in_dtype == RSS_DTYPE_BF16,
                                          !dual_fold && c.read_copy != RSS_COPY_NONE,
                                          static_cast<hipStream_t>(stream)));
}

int32_t rss_decode_step(rss_layer* l, const void* x, const void* B, const void* C, const float* dt,
                        float* y, void* stream) {
  if (!l || l->cfg.kind != RSS_KIND_MAMBA2) return RSS_E_INVALID;
  if (l->cfg.batch > 0 && !inputs_ok(x, B, C, dt, y)) return RSS_E_INVALID;
  if (l->pending_verify) return RSS_E_ORDER;
  const int32_t st = replay_call(l, 1, 0, 0, nullptr, x, B, C, dt, y, stream);
  if (st == RSS_OK) lock_decode(l, 0);
  return st;
}

static int32_t flush_call(rss_layer* l, int32_t min_len, const int32_t* each, void* stream);

// The fp32-geometry decode of a dual fold (four wavefronts) within the LDS budget.
static bool dual_fold_fits(const rss_config& c) {
  const int tin = c.in_dtype == RSS_DTYPE_BF16 ? 2 : 4;
  return (size_t)rss::ReplayLds(c.capacity, c.headdim, c.dstate, 1, tin, 4, 0, 0).total * 4 <=
         (size_t)rss::kMaxLdsBytes;
}

static int32_t decode_fold(rss_layer* l, int32_t min_len, const int32_t* each, const void* x,
                           const void* B, const void* C, const float* dt, float* y, void* stream) {
  if (!l || l->cfg.kind != RSS_KIND_MAMBA2) return RSS_E_INVALID;
  if (l->cfg.batch > 0 && !inputs_ok(x, B, C, dt, y)) return RSS_E_INVALID;
  if (l->pending_verify) return RSS_E_ORDER;
  const rss_config& c = l->cfg;
  // Two launches where the fold cannot ride on the replay: dual precision (the
  // replay reads the copy, the fold the fp32 master), or a bf16-stored
  // checkpoint whose widened fold operands would not fit the LDS budget.
  bool separate = c.read_copy == RSS_COPY_BF16;
  if (c.read_copy == RSS_STATE_BF16) {
    const int tin = c.in_dtype == RSS_DTYPE_BF16 ? 2 : 4;
    const size_t lds = (size_t)rss::ReplayLds(c.capacity, c.headdim, c.dstate, 1, tin, 2,
                                              rss::fold_buf_floats(c.dstate, 8, rss::kMaxPass),
                                              tin == 2 ? rss::fold_bt_elems(c.dstate, c.capacity) : 0)
                           .total * 4;
    separate = lds > (size_t)rss::kMaxLdsBytes;
  }
  int32_t st;
  if (separate && c.read_copy == RSS_COPY_BF16 && !each && l->lock_len >= 0 &&
      l->lock_len < c.capacity && l->lock_len + 1 >= min_len && dual_fold_fits(c)) {
    // Dual precision, every window filled by this token: one pass reads the fp32
    // master (which the fold needs anyway) instead of the copy, takes the outputs
    // from its RNE-bf16 rounding (the copy's values) and writes master and copy.
    st = replay_call(l, 1, 0, min_len, nullptr, x, B, C, dt, y, stream, 1);
  } else if (separate) {
    st = replay_call(l, 1, 0, 0, nullptr, x, B, C, dt, y, stream);
    if (st == RSS_OK) st = flush_call(l, min_len, each, stream);
  } else {
    st = replay_call(l, 1, 0, min_len, each, x, B, C, dt, y, stream);
  }
  if (st == RSS_OK) {
    if (each) l->lock_len = -1;
    else lock_decode(l, min_len);
  }
  return st;
}

int32_t rss_decode_flush_step(rss_layer* l, int32_t min_len, const void* x, const void* B,
                              const void* C, const float* dt, float* y, void* stream) {
  if (min_len < 1) return RSS_E_INVALID;
  return decode_fold(l, min_len, nullptr, x, B, C, dt, y, stream);
}

int32_t rss_decode_flush_step_each(rss_layer* l, const int32_t* min_len, const void* x,
                                   const void* B, const void* C, const float* dt, float* y,
                                   void* stream) {
  if (!l) return RSS_E_INVALID;
  if (l->cfg.batch > 0 && (!min_len || !aligned16(min_len))) return RSS_E_INVALID;
  return decode_fold(l, 1, min_len, x, B, C, dt, y, stream);
}

int32_t rss_verify_k_tokens(rss_layer* l, int32_t K, const void* x, const void* B, const void* C,
                            const float* dt, float* y, void* stream) {
  if (!l || l->cfg.kind != RSS_KIND_MAMBA2) return RSS_E_INVALID;
  if (l->cfg.batch > 0 && !inputs_ok(x, B, C, dt, y)) return RSS_E_INVALID;
  if (K < 0) return RSS_E_INVALID;
  if (K > l->cfg.max_draft) return RSS_E_CAPACITY;
  if (l->pending_verify) return RSS_E_ORDER;
  const int32_t st = replay_call(l, K + 1, 1, 0, nullptr, x, B, C, dt, y, stream);
  if (st == RSS_OK) {
    l->pending_verify = 1;
    l->lock_len = -1;
  }
  return st;
}

int32_t rss_verify_k_tokens_fold(rss_layer* l, int32_t min_len, int32_t K, const void* x,
                                 const void* B, const void* C, const float* dt, float* y,
                                 void* stream) {
  if (!l || l->cfg.kind != RSS_KIND_MAMBA2) return RSS_E_INVALID;
  if (min_len < 1) return RSS_E_INVALID;
  if (l->cfg.batch > 0 && !inputs_ok(x, B, C, dt, y)) return RSS_E_INVALID;
  if (K < 0) return RSS_E_INVALID;
  if (K > l->cfg.max_draft) return RSS_E_CAPACITY;
  if (l->pending_verify) return RSS_E_ORDER;
  const rss_config& c = l->cfg;
  if (c.read_copy == RSS_COPY_NONE) {
    // The fold frees the committed slots in the same pass, so a window of up to
    // R + K + 1 positions is staged at once: it must fit one wavefront's scan
    // (64 lanes) and the LDS budget.
    if (c.capacity + K + 1 > 64) return RSS_E_CAPACITY;
    // Grouped B rows are shared by the group's heads, so no slot may be reused
    // within the call: the window must fit R even before its fold.
    if (c.ngroups != c.nheads && c.capacity < min_len + 2 * K + 1) return RSS_E_CAPACITY;
    const int tin = c.in_dtype == RSS_DTYPE_BF16 ? 2 : 4;
    const size_t lds = (size_t)rss::ReplayLds(c.capacity + K + 1, c.headdim, c.dstate,
                                              K + 1, tin, 4).total * 4;
    if (lds > (size_t)rss::kMaxLdsBytes) return RSS_E_SHAPE;
  }
  int32_t st;
  if (c.read_copy != RSS_COPY_NONE) {  // the replay reads a bf16 tile: fold first, separately
    st = flush_call(l, min_len, nullptr, stream);
    if (st == RSS_OK) st = replay_call(l, K + 1, 1, 0, nullptr, x, B, C, dt, y, stream);
  } else {
    st = replay_call(l, K + 1, 1, min_len, nullptr, x, B, C, dt, y, stream);
  }
  if (st == RSS_OK) {
    l->pending_verify = 1;
    l->lock_len = -1;
  }
  return st;
}

int32_t rss_rollback(rss_layer* l, const int32_t* n_drop, void* stream) {
  if (!l) return RSS_E_INVALID;
  if (l->cfg.batch > 0 && (!n_drop || !aligned16(n_drop))) return RSS_E_INVALID;
  if (!l->pending_verify) return RSS_E_ORDER;
  const rss_config& c = l->cfg;
  l->pending_verify = 0;
  if (c.batch == 0) return RSS_OK;
  rss::RollbackArgs a;
  a.ptr = reinterpret_cast<int4*>(l->dev.ptr);
  a.n_drop = n_drop;
  a.err = l->dev.dev_err;
  a.H = c.nheads;
  a.n_ptr = (size_t)c.batch * c.nheads;
  return launch_status(rss::launch_rollback(a, static_cast<hipStream_t>(stream)));
}

int32_t rss_flush_checkpoint(rss_layer* l, int32_t min_len, void* stream) {
  if (!l) return RSS_E_INVALID;
  if (min_len < 1) return RSS_E_INVALID;
  const int32_t st = flush_call(l, min_len, nullptr, stream);
  if (st == RSS_OK) lock_flush(l, min_len);
  return st;
}

int32_t rss_flush_checkpoint_each(rss_layer* l, const int32_t* min_len, void* stream) {
  if (!l) return RSS_E_INVALID;
  if (l->cfg.batch > 0 && (!min_len || !aligned16(min_len))) return RSS_E_INVALID;
  const int32_t st = flush_call(l, 1, min_len, stream);
  if (st == RSS_OK) l->lock_len = -1;
  return st;
}

static int32_t flush_call(rss_layer* l, int32_t min_len, const int32_t* each, void* stream) {
  if (l->pending_verify) return RSS_E_ORDER;
  const rss_config& c = l->cfg;
  if (c.batch == 0) return RSS_OK;
  rss::FlushArgs a;
  a.ckpt = ckpt_f32(l);
  a.ckpt_lo = ckpt_bf16(l);
  a.ring_x = l->dev.ring_x;
  a.ring_B = l->dev.ring_B;
  a.ring_dl = reinterpret_cast<const float2*>(l->dev.ring_dl);
  a.ptr = reinterpret_cast<int4*>(l->dev.ptr);
  a.err = l->dev.dev_err;
  a.H = c.nheads;
  a.P = c.headdim;
  a.G = c.ngroups;
  a.R = c.capacity;
  a.min_len = min_len;
  a.min_len_dev = each;
  a.ring_g = c.kind == RSS_KIND_KDA ? l->dev.ring_dl : nullptr;
  const int kind = c.kind == RSS_KIND_KDA ? rss::kFoldKda
                   : c.kind == RSS_KIND_GDN ? rss::kFoldGdn : rss::kFoldMamba2;
  return launch_status(rss::launch_flush(a, c.batch, c.dstate, c.in_dtype == RSS_DTYPE_BF16,
                                         c.read_copy, kind, static_cast<hipStream_t>(stream)));
}

static int32_t delta_decode(rss_layer* l, int32_t kind, int32_t fold_min_len, const float* q,
                            const float* k, const float* v, const float* beta, const float* alpha,
                            float* o, void* stream) {
  if (!l || l->cfg.kind != kind) return RSS_E_INVALID;
  const rss_config& c = l->cfg;
  if (c.batch > 0 && (!inputs_ok(q, k, v, beta, o) || !alpha || !aligned16(alpha)))
    return RSS_E_INVALID;
  if (l->pending_verify) return RSS_E_ORDER;
  if (c.batch == 0) return RSS_OK;
  rss::GdnArgs a;
  a.ckpt = static_cast<float*>(l->dev.ckpt);
  a.ring_u = static_cast<float*>(l->dev.ring_x);
  a.ring_k = static_cast<float*>(l->dev.ring_B);
  a.ring_dl = reinterpret_cast<float2*>(l->dev.ring_dl);
  a.ring_g = l->dev.ring_dl;
  a.ptr = reinterpret_cast<int4*>(l->dev.ptr);
  a.err = l->dev.dev_err;
  a.q = q;
  a.k = k;
  a.v = v;
  a.beta = beta;
  a.alpha = alpha;
  a.o = o;
  a.H = c.nheads;
  a.P = c.headdim;
  a.R = c.capacity;
  a.fold_min_len = fold_min_len;
  const int32_t st = launch_status(rss::launch_gdn_replay(a, c.batch, c.dstate, kind == RSS_KIND_KDA,
                                                          static_cast<hipStream_t>(stream)));
  if (st == RSS_OK) lock_decode(l, fold_min_len);
  return st;
}

int32_t rss_gdn_decode_step(rss_layer* l, const float* q, const float* k, const float* v,
                            const float* beta, const float* alpha, float* o, void* stream) {
  return delta_decode(l, RSS_KIND_GDN, 0, q, k, v, beta, alpha, o, stream);
}

int32_t rss_gdn_decode_flush_step(rss_layer* l, int32_t min_len, const float* q, const float* k,
                                  const float* v, const float* beta, const float* alpha, float* o,
                                  void* stream) {
  if (min_len < 1) return RSS_E_INVALID;
  return delta_decode(l, RSS_KIND_GDN, min_len, q, k, v, beta, alpha, o, stream);
}

int32_t rss_kda_decode_step(rss_layer* l, const float* q, const float* k, const float* v,
                            const float* beta, const float* alpha, float* o, void* stream) {
  return delta_decode(l, RSS_KIND_KDA, 0, q, k, v, beta, alpha, o, stream);
}

int32_t rss_kda_decode_flush_step(rss_layer* l, int32_t min_len, const float* q, const float* k,
                                  const float* v, const float* beta, const float* alpha, float* o,
                                  void* stream) {
  if (min_len < 1) return RSS_E_INVALID;
  return delta_decode(l, RSS_KIND_KDA, min_len, q, k, v, beta, alpha, o, stream);
}

static int32_t delta_eager(const rss_config* c, bool kda, float* S, const float* q, const float* k,
                           const float* v, const float* beta, const float* alpha, float* o,
                           void* stream) {
  if (!c) return RSS_E_INVALID;
  if (c->batch < 0 || c->nheads < 1 || c->headdim < 1 || c->headdim > rss::kMaxP) return RSS_E_SHAPE;
  if (!supported_n(c->dstate)) return RSS_E_SHAPE;
  if ((int64_t)c->batch * c->nheads > 0x7fffffffLL) return RSS_E_SHAPE;
  if (c->batch == 0) return RSS_OK;
  if (!S || !aligned16(S) || !inputs_ok(q, k, v, beta, o) || !alpha || !aligned16(alpha))
    return RSS_E_INVALID;
  rss::GdnEagerArgs a;
  a.S = S;
  a.q = q;
  a.k = k;
  a.v = v;
  a.beta = beta;
  a.alpha = alpha;
  a.o = o;
  a.H = c->nheads;
  a.P = c->headdim;
  return launch_status(rss::launch_gdn_eager(a, c->batch, c->dstate, kda,
                                             static_cast<hipStream_t>(stream)));
}

int32_t rss_gdn_eager_step(const rss_config* c, float* S, const float* q, const float* k,
                           const float* v, const float* beta, const float* alpha, float* o,
                           void* stream) {
  return delta_eager(c, false, S, q, k, v, beta, alpha, o, stream);
}

int32_t rss_kda_eager_step(const rss_config* c, float* S, const float* q, const float* k,
                           const float* v, const float* beta, const float* alpha, float* o,
                           void* stream) {
  return delta_eager(c, true, S, q, k, v, beta, alpha, o, stream);
}

int32_t rss_get_device_error(rss_layer* l, int32_t* host_code, void* stream) {
  if (!l || !host_code) return RSS_E_INVALID;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t v = 0;
  if (hipMemcpyAsync(&v, l->dev.dev_err, sizeof(v), hipMemcpyDeviceToHost, s) != hipSuccess)
    return RSS_E_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return RSS_E_HIP;
  *host_code = v;
  return RSS_OK;
}

static int32_t eager_call(const rss_config* c, void* S, const int32_t* src_slot, int32_t slots,
                          int32_t T, const void* x, const void* B, const void* C, const float* dt,
                          const float* A, float* y, void* stream) {
  const int32_t st = check_shape(c);
  if (st) return st;
  if (!valid_mode(c->read_copy)) return RSS_E_DTYPE;
  const bool bf16_state = c->read_copy == RSS_STATE_BF16;
  if (bf16_state && slots > 0) return RSS_E_DTYPE;  // snapshot pools are fp32
  if (T < 1 || T > rss::kMaxNew) return RSS_E_INVALID;
  if (!A || !aligned16(A)) return RSS_E_INVALID;
  if (c->batch == 0) return RSS_OK;
  if (!S || !aligned16(S) || !inputs_ok(x, B, C, dt, y)) return RSS_E_INVALID;
  rss::EagerArgs a;
  a.S = S;
  a.src_slot = src_slot;
  a.x = x;
  a.B = B;
  a.C = C;
  a.dt = dt;
  a.A = A;
  a.y = y;
  a.H = c->nheads;
  a.P = c->headdim;
  a.G = c->ngroups;
  a.T = T;
  a.slots = slots;
  return launch_status(rss::launch_eager(a, c->batch, c->dstate, c->in_dtype == RSS_DTYPE_BF16,
                                         bf16_state, static_cast<hipStream_t>(stream)));
}

int32_t rss_eager_step(const rss_config* c, void* S, const void* x, const void* B, const void* C,
                       const float* dt, const float* A, float* y, int32_t T, void* stream) {
  return eager_call(c, S, nullptr, 0, T, x, B, C, dt, A, y, stream);
}

int32_t rss_eager_verify(const rss_config* c, float* pool, const int32_t* src_slot, int32_t K,
                         const void* x, const void* B, const void* C, const float* dt,
                         const float* A, float* y, void* stream) {
  if (K < 0 || K > rss::kMaxNew - 1) return RSS_E_INVALID;
  if (c && c->batch > 0 && (!src_slot || !aligned16(src_slot))) return RSS_E_INVALID;
  return eager_call(c, pool, src_slot, K + 1, K + 1, x, B, C, dt, A, y, stream);
}

}  // extern "C"

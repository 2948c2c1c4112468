/*
 * rss.h — C ABI of the ReplaySSM decode library for AMD MI355X (gfx950).
 *
 * A Mamba-2 SSM layer in decode keeps, per (sequence b, head h), a P x N fp32
 * state. The eager step reads that state, decays it, adds a rank-1 update,
 * reads the output and writes the whole state back (P1, "La fiche qu'on
 * réécrit à chaque token"):
 *
 *     a = exp(dt*A_h);  S <- a*S + dt*outer(x, B);  y = S @ C
 *
 * ReplaySSM instead keeps a checkpoint S_c plus a ring of the inputs that
 * followed it, computes each output from both without writing a state, and
 * folds the ring into the checkpoint only when it is full (P1, "Tenir le
 * journal plutôt que le solde"; P2, "L'astuce du checkpoint et du tampon";
 * P3, "Решение ReplaySSM"; P4's table, row "Ruch pamięci stanu"). Rolling back
 * rejected speculative tokens moves ring pointers only (P2, "Un retour en
 * arrière qui devient trivial"). An optional bf16 read copy of the checkpoint
 * serves outputs while the fp32 master alone feeds the fold (P2, "Deux
 * précisions pour le prix d'une").
 *
 * Page key: P1 = "NVIDIA réécrit le stockage d'état des modèles hybrides"
 * (blog.thibaultmonteiro.fr); P2 = "ReplaySSM : l'IA qui cesse de réécrire son
 * passé" (irisproject.cloud); P3 = "ReplaySSM: Rethinking State Storage for
 * Faster Hybrid-Model Decoding" (aikraft.ru); P4 = "NVIDIA i Princeton
 * eliminują wąskie gardła dekodowania w hybrydowych modelach SSM"
 * (ainews.tenesys.com).
 *
 * Conventions for every call
 * --------------------------
 *  - Notation: batch Bt, heads H, head dim P, state dim N, groups G (H % G ==
 *    0; head h uses group g = h / (H/G)), window W, ring capacity R, largest
 *    draft K_max.
 *  - Memory: the caller allocates and owns every device buffer and passes raw
 *    device pointers; all tensors are dense, row-major, with the layouts given
 *    below, and every pointer must be 16-byte aligned. The library allocates
 *    no device memory and frees nothing of the caller's; its only allocation is
 *    the small host-side rss_layer handle.
 *  - Streams: `stream` is a hipStream_t (NULL = the null stream). Every call
 *    only enqueues work and returns; nothing synchronises except
 *    rss_get_device_error. A handle must be used from one stream at a time.
 *  - Errors: every call returns an rss_status. Anything detectable on the
 *    host is checked before any launch and leaves device state untouched.
 *    Violations only the device can see (they depend on device-resident
 *    pointers or counts) leave that (sequence, head) unchanged, write NaN to
 *    its outputs, and OR a bit into the layer's sticky device error word.
 *  - dtypes: dt, A, y, the checkpoint and the ring's (dt, decay) pairs are
 *    fp32. x, B, C (and the ring's copies of x and B) are fp32 or bf16 as the
 *    config says.
 *  - Supported sizes: N in {16, 32, 64, 128, 256}; 1 <= P <= 256; Bt, H >= 1
 *    (Bt = 0 is accepted and launches nothing); 1 <= W <= R <= 64;
 *    0 <= K_max <= 7 and R >= W + K_max. The window's rows are staged in LDS,
 *    of which one gfx950 workgroup may hold 160 KiB: a configuration whose
 *    kernels would need more is refused with RSS_E_SHAPE. Only
 *    the largest shapes reach it: at P = N = 256, fp32 x/B/C with K_max > 0
 *    allow R <= 58 and a KDA layer R <= 48; bf16 x/B/C and GDN allow R = 64.
 */
#ifndef RSS_H_
#define RSS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum rss_status {
  RSS_OK = 0,
  RSS_E_INVALID = 1,  /* null pointer, misaligned pointer, bad enum, bad value */
  RSS_E_SHAPE = 2,    /* sizes outside the supported set or inconsistent     */
  RSS_E_DTYPE = 3,    /* unknown dtype or read-copy code                      */
  RSS_E_CAPACITY = 4, /* R < W + K_max, or K > K_max                          */
  RSS_E_ORDER = 5,    /* call order: decode/verify/flush while a verify round
                         is uncommitted, or rollback with no round pending    */
  RSS_E_HIP = 6       /* a HIP runtime call or kernel launch failed           */
} rss_status;

enum { RSS_DTYPE_F32 = 0, RSS_DTYPE_BF16 = 1 };
/* Checkpoint precision (rss_config.read_copy):
 *   RSS_COPY_NONE   fp32 checkpoint, read and folded in fp32;
 *   RSS_COPY_BF16   dual precision: fp32 master for the fold plus a bf16 copy
 *                   for reads (P2, "Deux précisions pour le prix d'une");
 *   RSS_STATE_BF16  a single bf16 checkpoint: read in bf16, folded in fp32
 *                   from the bf16 values and rounded back to bf16 at every
 *                   fold. This is the low-precision point the dual mode is
 *                   measured against: a quantised state accumulates one
 *                   rounding per rewrite (P1, "Trois ennuis nés de la même
 *                   fusion"), and ReplaySSM rewrites it once per window
 *                   instead of once per token (P1, "Tenir le journal plutôt
 *                   que le solde"). `ckpt` then holds bf16 [Bt,H,P,N] and
 *                   `ckpt_lo` is unused. For the eager entry points it means
 *                   an eager state stored in bf16 (rounded every token). */
enum { RSS_COPY_NONE = 0, RSS_COPY_BF16 = 1, RSS_STATE_BF16 = 2 };

/* Layer types. A Gated DeltaNet layer (P1, "La fiche qu'on réécrit à chaque
 * token": GDN's delta-rule update has the same form) uses P = d_v, N = d_k,
 * G = H (one key per head), fp32 inputs, no read copy; its ring holds
 * (u_t, k_t, (1, log alpha_t)) in ring_x, ring_B and ring_dl, and A is unused.
 * A Kimi Delta Attention layer (KDA, P1 "Des couches rapides sur le papier")
 * has the same rules and layout except that its gate has one value per key
 * channel: ring_dl then holds a log-gate row per entry, fp32 [Bt, R, H, N]. */
enum { RSS_KIND_MAMBA2 = 0, RSS_KIND_GDN = 1, RSS_KIND_KDA = 2 };

/* Bits of the sticky device error word. */
enum {
  RSS_DEV_ROLLBACK_RANGE = 1, /* rollback n_drop[b] < 0 or > n_tent           */
  RSS_DEV_RING_OVERFLOW = 2,  /* an append would exceed R entries              */
  RSS_DEV_UNCOMMITTED = 4     /* flush met tentative entries (never committed) */
};

typedef struct rss_config {
  int32_t batch;     /* Bt */
  int32_t nheads;    /* H  */
  int32_t headdim;   /* P  */
  int32_t dstate;    /* N  */
  int32_t ngroups;   /* G  */
  int32_t window;    /* W: flush threshold the caller intends to use        */
  int32_t capacity;  /* R: ring slots per (sequence, head)                   */
  int32_t max_draft; /* K_max                                                */
  int32_t in_dtype;  /* RSS_DTYPE_*: storage of x, B, C and their ring copies */
  int32_t read_copy; /* checkpoint precision: RSS_COPY_NONE / _BF16, RSS_STATE_BF16 */
  int32_t kind;      /* RSS_KIND_*: layer type                               */
} rss_config;

/*
 * Device buffers of one layer (all device pointers, caller-owned):
 *   ckpt     fp32 [Bt, H, P, N]   checkpoint S_c (the fp32 master); bf16
 *                                 [Bt, H, P, N] when read_copy = RSS_STATE_BF16
 *   ckpt_lo  bf16 [Bt, H, P, N]   read copy; NULL unless read_copy = BF16
 *   ring_x   in_dtype [Bt, R, H, P]   buffered x_j
 *   ring_B   in_dtype [Bt, R, G, N]   buffered B_j (one copy per group)
 *   ring_dl  fp32 [Bt, R, H, 2]   buffered (dt_j, dt_j * A_h); KDA:
 *                                 fp32 [Bt, R, H, N] log-gate rows
 *            The ring is slot-major: slot s of every head (group) of a
 *            sequence is contiguous, so the entries one call appends for all
 *            heads of a sequence sit side by side. One sequence's ring,
 *            R * H * max(P, N) elements, must stay below 2^31
 *            (RSS_E_SHAPE otherwise).
 *   ptr      int32 [Bt, H, 4]     per (sequence, head): head slot, window
 *                                 length len, tentative count n_tent, 0.
 *                                 Every head of a sequence holds the same
 *                                 values; each kernel workgroup owns its own
 *                                 (b, h) copy, so no two workgroups race.
 *   A        fp32 [H]             A_h (negative); unused (may be NULL) for
 *                                 GDN and KDA
 *   dev_err  int32 [1]            sticky device error word
 */
typedef struct rss_buffers {
  void* ckpt;
  void* ckpt_lo;
  void* ring_x;
  void* ring_B;
  float* ring_dl;
  int32_t* ptr;
  const float* A;
  int32_t* dev_err;
} rss_buffers;

/* Byte sizes of the buffers above for a config (0 for an absent buffer). */
typedef struct rss_sizes {
  size_t ckpt, ckpt_lo, ring_x, ring_B, ring_dl, ptr, A, dev_err;
} rss_sizes;

typedef struct rss_layer rss_layer;

/* Library version (major*10000 + minor*100 + patch). */
int32_t rss_version(void);

/* Human-readable text of a status code; never NULL, static storage. */
const char* rss_status_string(int32_t status);

/* Validate cfg and fill *out with the byte size of every buffer. */
int32_t rss_buffer_sizes(const rss_config* cfg, rss_sizes* out);

/* Validate cfg and the buffer pointers, and create a host handle that records
 * them (no device work, no device allocation). *out receives the handle, or
 * NULL on error. The buffers must outlive the handle. */
int32_t rss_layer_bind(const rss_config* cfg, const rss_buffers* dev, rss_layer** out);

/* Destroy a handle (NULL is accepted). Device buffers are not touched. */
int32_t rss_layer_free(rss_layer* layer);

/* Start every sequence from S0 (device fp32 [Bt,H,P,N]; NULL = zeros): the
 * checkpoint becomes S0 (RNE-bf16(S0) when read_copy = RSS_STATE_BF16), the
 * read copy RNE-bf16(S0), the rings empty
 * (head = len = n_tent = 0) and the device error word 0. The prefill that
 * produces S0 is outside this library. */
int32_t rss_init_state(rss_layer* layer, const float* S0, void* stream);

/* One plain decode token for every sequence: append (x_t, B_t, dt_t,
 * dt_t*A_h) at ring slot (head + len) mod R, len += 1, and write
 *   y_t = exp(Lam_c) * S_c @ C_t + sum_{j in window} exp(lam_j) dt_j (B_j.C_t) x_j
 * (lam_j: summed log-decays of the entries after j; Lam_c: of the whole
 * window). No state is written (P2, "L'astuce du checkpoint et du tampon";
 * P3, "Решение ReplaySSM"). With read_copy = BF16 the S_c term reads the bf16
 * copy. Inputs: x [Bt,H,P], B and C [Bt,G,N] (in_dtype), dt [Bt,H] fp32;
 * output y [Bt,H,P] fp32. Device error RSS_DEV_RING_OVERFLOW if len = R
 * (flush was not called). RSS_E_ORDER while a verify round is uncommitted. */
int32_t rss_decode_step(rss_layer* layer, const void* x, const void* B, const void* C,
                        const float* dt, float* y, void* stream);

/* rss_decode_step followed by rss_flush_checkpoint(min_len), in one pass where
 * it can be: a sequence whose window reaches min_len entries with this token is
 * folded while its checkpoint tile is already loaded for the output, and the
 * new checkpoint is written, so the flush's second read of the tile is saved
 * (the fold writes the state only once per window, P1 "Tenir le journal plutôt
 * que le solde"). Results equal the two separate calls bit for bit (dual
 * precision: outputs up to rounding, see below). A bf16-stored checkpoint
 * (RSS_STATE_BF16) is folded in the same pass too, unless its fold operands,
 * widened to fp32 in LDS, would not fit the budget (P = N = 256 with a long
 * window): then the fold runs as the separate flush launch, with the same
 * results. With read_copy = BF16 the replay reads the bf16 copy while the fold
 * needs the fp32 master. When the handle knows that this token fills every
 * window (all sequences in step: since rss_init_state or an
 * rss_flush_checkpoint(1), only plain decodes and folds of every window, no
 * verify round and no per-sequence thresholds), one pass reads the fp32 master
 * instead of the copy: the outputs come from the master's RNE-bf16 rounding,
 * bit for bit the copy's values, summed in another order (equal to the
 * separate calls' up to rounding), and the new master and copy are written,
 * bit for bit as the flush writes them. Otherwise the dual-precision fold is
 * the separate flush launch after the replay of the copy. On steps
 * where no sequence folds the call costs what rss_decode_step does, so a
 * caller may simply use it for every token. min_len >= 1; errors as
 * rss_decode_step, plus RSS_DEV_UNCOMMITTED if a window to fold still holds
 * tentative entries (that sequence is then not folded). */
int32_t rss_decode_flush_step(rss_layer* layer, int32_t min_len, const void* x, const void* B,
                              const void* C, const float* dt, float* y, void* stream);

/* rss_decode_flush_step with a threshold per sequence: min_len is device int32
 * [Bt] (values below 1 act as 1), read by the launch, so sequences whose
 * windows are out of phase fold on different steps. Setting min_len[b] =
 * 1 + (b mod W) for the first window and W afterwards staggers the folds: every
 * step then writes about Bt/W checkpoints instead of all Bt on one step in W,
 * which flattens the per-step time (the fold still happens once per window per
 * sequence, P1 "Tenir le journal plutôt que le solde"). Errors as
 * rss_decode_flush_step; RSS_E_INVALID if min_len is null or misaligned. */
int32_t rss_decode_flush_step_each(rss_layer* layer, const int32_t* min_len, const void* x,
                                   const void* B, const void* C, const float* dt, float* y,
                                   void* stream);

/* Fold the ring into the checkpoint for every sequence whose window holds at
 * least min_len >= 1 entries (P1, "Tenir le journal plutôt que le solde":
 * rewritten only when the buffer is full; P3: once per window):
 *   S_c <- exp(Lam_c) S_c + sum_j exp(lam_j) dt_j outer(x_j, B_j)
 * then head <- (head + len) mod R, len <- 0, and in dual mode the read copy
 * becomes RNE-bf16 of the new fp32 master. With read_copy = RSS_STATE_BF16 the
 * fold starts from the bf16 checkpoint's values (fp32 arithmetic) and stores
 * RNE-bf16 of the result. Other sequences are untouched.
 * RSS_E_ORDER while a verify round is uncommitted. */
int32_t rss_flush_checkpoint(rss_layer* layer, int32_t min_len, void* stream);

/* rss_flush_checkpoint with a threshold per sequence (device int32 [Bt], values
 * below 1 act as 1): sequence b is folded if its window holds >= min_len[b]
 * entries. RSS_E_INVALID if min_len is null or misaligned. */
int32_t rss_flush_checkpoint_each(rss_layer* layer, const int32_t* min_len, void* stream);

/* Speculative verify of K+1 tokens per sequence (the last sampled token and K
 * drafts; 0 <= K <= K_max): append all K+1 as tentative entries (n_tent =
 * K+1) and write the K+1 outputs, output i being the decode output of token i
 * over the committed window plus tokens 0..i (P3, "Почему это важно для
 * индустрии": drafts are added to the buffer). One pass over S_c serves all K+1 outputs.
 * Layouts: x [Bt,K+1,H,P], B and C [Bt,K+1,G,N], dt [Bt,K+1,H], y
 * [Bt,K+1,H,P]. Device error RSS_DEV_RING_OVERFLOW if len + K + 1 > R.
 * RSS_E_ORDER if a previous round is still uncommitted. */
int32_t rss_verify_k_tokens(rss_layer* layer, int32_t K, const void* x, const void* B,
                            const void* C, const float* dt, float* y, void* stream);

/* rss_flush_checkpoint(min_len) followed by rss_verify_k_tokens(K), in one pass
 * where it can be: a sequence whose committed window holds >= min_len entries
 * (min_len >= 1) has that window folded into its checkpoint while the tile is
 * loaded for the K+1 outputs, and the new checkpoint is written; the K+1 new
 * entries then start the next window. The checkpoint, ring and pointers equal
 * the two separate calls' bit for bit; the outputs are computed from the
 * unfolded checkpoint and the whole window, equal up to rounding. A speculative
 * loop of this call and rss_rollback needs no separate flush: a window the
 * accepted drafts fill is folded by the next round. R >= W + K_max still
 * bounds the ring between rounds, where a window may hold up to W + K entries,
 * so call rss_flush_checkpoint(W) before returning to plain decode. During the
 * call a folding sequence stages up to R + K + 1 positions, the committed ones
 * read before their slots are reused. With read_copy = BF16 or RSS_STATE_BF16
 * the fold runs as a separate
 * flush launch first. Errors as rss_verify_k_tokens and rss_flush_checkpoint,
 * plus RSS_E_CAPACITY if R + K + 1 > 64, or if G < H and R < min_len + 2K + 1
 * (heads of a group share B rows, so no slot is reused within the call: a
 * grouped layer needs room for a full window plus two rounds), and
 * RSS_E_SHAPE if the staged window would exceed the LDS budget (fp32
 * checkpoint only). */
int32_t rss_verify_k_tokens_fold(rss_layer* layer, int32_t min_len, int32_t K, const void* x,
                                 const void* B, const void* C, const float* dt, float* y,
                                 void* stream);

/* Commit a verify round: per sequence drop the n_drop[b] newest tentative
 * entries (0 <= n_drop[b] <= n_tent; n_drop = K - accepted drafts) and keep
 * the rest: len -= n_drop[b], n_tent = 0. Pointer arithmetic only; no
 * checkpoint or ring bytes are touched (P2, "Un retour en arrière qui devient
 * trivial"; P1: rejected tokens leave the buffer without harming the
 * checkpoint). n_drop: device int32 [Bt], written by the caller's sampler.
 * Out-of-range n_drop sets RSS_DEV_ROLLBACK_RANGE and leaves that sequence
 * unchanged. RSS_E_ORDER if no round is pending. Callers then flush(W). */
int32_t rss_rollback(rss_layer* layer, const int32_t* n_drop, void* stream);

/* Gated DeltaNet decode of one token for every sequence (kind = RSS_KIND_GDN),
 * by replay: with S_{t-1} = checkpoint + window, and per head
 *   u_t = beta_t (v_t - alpha_t S_{t-1} k_t),   o_t = alpha_t S_{t-1} q_t + (k_t.q_t) u_t,
 * which is the gated delta rule S_t = alpha_t S_{t-1}(I - beta_t k_t k_t^T) +
 * beta_t v_t k_t^T read out as o_t = S_t q_t, without writing S_t. Appends
 * (u_t, k_t, (1, log alpha_t)) to the ring; rss_flush_checkpoint folds GDN
 * windows like Mamba-2 ones. Layouts: q, k [Bt,H,N]; v [Bt,H,P]; beta, alpha
 * [Bt,H]; o [Bt,H,P]; all fp32. Ring overflow as rss_decode_step. */
int32_t rss_gdn_decode_step(rss_layer* layer, const float* q, const float* k, const float* v,
                            const float* beta, const float* alpha, float* o, void* stream);

/* rss_gdn_decode_step followed by rss_flush_checkpoint(min_len), in one pass:
 * a sequence whose window reaches min_len >= 1 entries with this token has it
 * folded (the new entry included) into the tile already loaded for the output,
 * and the new checkpoint written. Results equal the two calls bit for bit. */
int32_t rss_gdn_decode_flush_step(rss_layer* layer, int32_t min_len, const float* q,
                                  const float* k, const float* v, const float* beta,
                                  const float* alpha, float* o, void* stream);

/* Eager gated delta rule (the GDN baseline): S [Bt,H,P,N] fp32 updated in
 * place, S <- alpha S + u k^T, o = S q, layouts as rss_gdn_decode_step. Uses
 * cfg's batch, nheads, headdim (d_v) and dstate (d_k). */
int32_t rss_gdn_eager_step(const rss_config* cfg, float* S, const float* q, const float* k,
                           const float* v, const float* beta, const float* alpha, float* o,
                           void* stream);

/* Kimi Delta Attention decode of one token for every sequence (kind =
 * RSS_KIND_KDA), by replay: the gated delta rule with one gate per key channel,
 *   S_t = S_{t-1} Diag(alpha_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *   u_t = beta_t (v_t - S_{t-1} (alpha_t * k_t)),
 *   o_t = S_t q_t = S_{t-1} (alpha_t * q_t) + (k_t . q_t) u_t,
 * with S_{t-1} the checkpoint (each key channel n decayed by the product of its
 * gates) plus the window, never written. Appends (u_t, k_t, log alpha_t) to the
 * ring; rss_flush_checkpoint folds KDA windows with per-channel decays.
 * Layouts: q, k, alpha [Bt,H,N]; v [Bt,H,P]; beta [Bt,H]; o [Bt,H,P]; all
 * fp32; 0 < alpha < 1. Ring overflow as rss_decode_step. */
int32_t rss_kda_decode_step(rss_layer* layer, const float* q, const float* k, const float* v,
                            const float* beta, const float* alpha, float* o, void* stream);

/* rss_kda_decode_step followed by rss_flush_checkpoint(min_len), in one pass,
 * as rss_gdn_decode_flush_step; results equal the two calls bit for bit. */
int32_t rss_kda_decode_flush_step(rss_layer* layer, int32_t min_len, const float* q,
                                  const float* k, const float* v, const float* beta,
                                  const float* alpha, float* o, void* stream);

/* Eager KDA step (its baseline): S [Bt,H,P,N] fp32 updated in place by the rule
 * above, layouts as rss_kda_decode_step; uses cfg's batch, nheads, headdim
 * (d_v) and dstate (d_k). */
int32_t rss_kda_eager_step(const rss_config* cfg, float* S, const float* q, const float* k,
                           const float* v, const float* beta, const float* alpha, float* o,
                           void* stream);

/* Copy the sticky device error word to *host_code (synchronises `stream`). */
int32_t rss_get_device_error(rss_layer* layer, int32_t* host_code, void* stream);

/* Eager baseline (P1, "La fiche qu'on réécrit à chaque token"): for T >= 1
 * tokens per sequence run S <- a S + dt outer(x,B), y = S @ C in order,
 * reading and writing the full state. S fp32 [Bt,H,P,N] is updated in place;
 * with cfg->read_copy = RSS_STATE_BF16, S is bf16 [Bt,H,P,N]: each token
 * computes in fp32 from the stored bf16 values, takes y from the fp32 result
 * and stores RNE-bf16 of it (the per-token rounding of a quantised eager
 * state, P1 "Trois ennuis nés de la même fusion").
 * Layouts: x [Bt,T,H,P], B and C [Bt,T,G,N], dt [Bt,T,H], y [Bt,T,H,P]; A [H].
 * Uses cfg's batch, nheads, headdim, dstate, ngroups, in_dtype and read_copy
 * (RSS_COPY_BF16 is treated as RSS_COPY_NONE: an eager state has no copy).
 * 1 <= T <= 8. */
int32_t rss_eager_step(const rss_config* cfg, void* S, const void* x, const void* B,
                       const void* C, const float* dt, const float* A, float* y,
                       int32_t T, void* stream);

/* Eager speculative baseline with per-token state snapshots, the rollback
 * scheme ReplaySSM removes (P3, "Почему это важно для индустрии"; P4, "Co się
 * zmieniło?", item 4): pool fp32 [Bt, K+1, H, P, N]. Sequence b starts from slot
 * src_slot[b] (device int32 [Bt], 0 <= src_slot[b] <= K), runs K+1 eager
 * tokens and writes the state after token i to slot i (the read completes
 * before any write, so src_slot may be any slot). Rolling back to n_acc
 * accepted drafts is then "next round reads slot n_acc". Layouts as in
 * rss_eager_step with T = K+1; 0 <= K <= 7. An out-of-range src_slot[b]
 * writes NaN outputs for that sequence and leaves its slots unchanged.
 * The pool is fp32 only: RSS_E_DTYPE if cfg->read_copy = RSS_STATE_BF16. */
int32_t rss_eager_verify(const rss_config* cfg, float* pool, const int32_t* src_slot,
                         int32_t K, const void* x, const void* B, const void* C,
                         const float* dt, const float* A, float* y, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RSS_H_ */

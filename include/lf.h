/*
 * lf.h -- C ABI of the batch-1 FP16 decode library (liblf.so), MI355X / gfx950.
 *
 * One decode step of a dense pre-norm decoder (RMSNorm, QKV with rotary
 * embedding, causal attention over an fp16 KV cache, output projection, SwiGLU
 * FFN, final norm, lm_head, next-token choice) runs as ONE persistent GPU
 * kernel; lf_generate runs n such steps in one launch and feeds each sampled
 * token back on the device, without returning to the host between tokens.
 *
 * Source pages: "KOG LaneFormer-2B & the monokernel" (shivam2003.com),
 * sections "The problem" (batch-1 decode streams every weight once per token
 * through matrix-vector products), "Pillar 3 - the monokernel runtime" (the
 * whole decode pass, sampling included, in one resident kernel that hands the
 * token back only when it is produced), "Compile-time work partition" (a fixed
 * grid of one block per compute unit with a static assignment of work) and
 * "The fused operations, briefly".
 *
 * Conventions for every entry point:
 *   - Return 0 (LF_OK) or a negative LF_E* code; no exception crosses the ABI.
 *     lf_last_error(state) (or lf_last_error(NULL) before a state exists)
 *     returns a text description of the last failure on this thread.
 *   - Pointers named *_dev are device pointers (hipMalloc or torch CUDA tensors),
 *     all others host pointers.  fp16 means IEEE binary16.
 *   - Calls are synchronous with respect to the state's stream: they enqueue on
 *     it and wait for completion before returning.  One state per host thread.
 */
#ifndef LF_H
#define LF_H
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  LF_OK = 0,
  LF_EINVAL = -1,      /* bad configuration, null or misaligned pointer */
  LF_ENOMEM = -2,      /* device allocation failed */
  LF_EHIP = -3,        /* HIP runtime or launch failure (incl. co-residency refused) */
  LF_ERANGE = -4,      /* pos >= max_seq, token outside [0, vocab), n out of range */
  LF_ETIMEOUT = -5,    /* a bounded in-kernel wait expired; the kernel exited cleanly */
  LF_EUNSUPPORTED = -6 /* valid but not implemented (e.g. head_dim not 64, 96 or 128) */
};

/* config.flags */
#define LF_HIDDEN_IO 1u  /* no embedding / lm_head: the layers run on a hidden vector
                            set with lf_set_hidden and read with lf_get_hidden */
#define LF_STATS 4u      /* record per-workgroup wait time (lf_get_stats) */
#define LF_GUMBEL 8u     /* with temperature > 0: Gumbel-max sampling instead of the
                            nucleus (top_p unused).  "KOG LaneFormer-2B & the
                            monokernel", "The fused operations, briefly": the token
                            is argmax_i(logit_i / T + g_i), g_i = -ln(-ln u_i),
                            u_i = (2 (x0 >> 9) + 1) 2^-24 from the first word of
                            the Philox4x32-10 block with key (seed lo, seed hi) and
                            counter (pos, i, 1, 0); ln is the library's defined
                            logarithm (lf_test_logdef); lowest index on ties.  Each
                            lm_head workgroup publishes its best score, so no
                            workgroup reads the whole logit vector. */

typedef struct lf_state lf_state;

typedef struct {
  int32_t n_layers, d_model, n_heads, n_kv_heads, head_dim, ffn_dim, vocab, max_seq;   /* head_dim 64, 96 or 128 */
  float rms_eps;       /* RMSNorm epsilon, inside the square root (1e-5) */
  float rope_base;     /* rotary base (10000) */
  float temperature;   /* 0: greedy argmax; > 0: nucleus (or, with LF_GUMBEL, Gumbel-max) sampling */
  float top_p;         /* nucleus mass fraction in (0, 1] when temperature > 0 (not LF_GUMBEL) */
  uint64_t seed;       /* Philox4x32-10 key of the sampler */
  uint32_t flags;      /* LF_HIDDEN_IO | LF_STATS | LF_GUMBEL */
  int32_t sliding_window;   /* > 0: the layers in window_layers attend to the last
                               sliding_window positions only (rows pos-W+1..pos);
                               0: every layer attends to all earlier positions.
                               "KOG LaneFormer-2B & the monokernel", "Pillar 1". */
  uint64_t window_layers;   /* bit l set: layer l (< 64) uses the window */
} lf_config;

/* One layer's weights: fp16 device pointers, row-major [out][in]:
 *   attn_norm, ffn_norm [d]; wq [n_heads*head_dim][d] (row h*head_dim + j is
 *   dimension j of query head h); wk, wv [n_kv_heads*head_dim][d];
 *   wo [d][n_heads*head_dim]; w_gate, w_up [ffn_dim][d]; w_down [d][ffn_dim]. */
typedef struct {
  const void *attn_norm, *wq, *wk, *wv, *wo, *ffn_norm, *w_gate, *w_up, *w_down;
} lf_layer_weights;

/* Model weights: tok_emb, lm_head [vocab][d] (untied), final_norm [d]; all fp16
 * device pointers (NULL with LF_HIDDEN_IO).  layers: host array of n_layers. */
typedef struct {
  const void *tok_emb, *final_norm, *lm_head;
  const lf_layer_weights *layers;
} lf_weights;

/* Validate the config, repack the weights into library-owned device memory (the
 * caller may free its copies afterwards; each RMSNorm gain vector is folded into
 * the columns of the projection after it, the weight pre-transform of the
 * pages' "Weight streaming" section), allocate the KV cache (zeroed),
 * activations and synchronisation words, and build the static work plan.
 * stream: a hipStream_t (NULL = default stream).  On success *out owns all of it.
 * Errors: LF_EINVAL (config, null pointer), LF_EUNSUPPORTED, LF_ENOMEM, LF_EHIP. */
int lf_model_create(const lf_config *config, const lf_weights *weights, void *stream,
                    lf_state **out);

/* Free everything the state owns.  NULL is ignored. */
void lf_model_destroy(lf_state *st);

/* One decode step in one launch ("KOG LaneFormer-2B & the monokernel", "Pillar 3
 * - the monokernel runtime": the whole pass, the token choice included, in one
 * resident kernel): consume `token` at position `pos`, write K/V at pos, compute
 * logits, choose the next token (RNG counter = pos) and store it as the pending
 * (next, pos + 1) for lf_generate.  next_token (host, nullable)
 * receives it.  With LF_HIDDEN_IO: token is ignored, the layers run on the hidden
 * vector and *next_token = -1.
 * Errors: LF_ERANGE (pos outside [0, max_seq), token outside [0, vocab)),
 * LF_ETIMEOUT, LF_EHIP. */
int lf_decode_step(lf_state *st, int32_t token, int32_t pos, int32_t *next_token);

/* n decode steps from the pending (token, pos) in ONE launch; each sampled token
 * is fed back on the device, so no kernel boundary or host round trip separates
 * tokens (same page, "Pillar 3 - the monokernel runtime" and "The arithmetic that
 * forces this").  out_tokens (host, n entries) receives the sampled
 * tokens.  Errors: LF_ERANGE (no pending token, n < 1, pos + n > max_seq),
 * LF_ETIMEOUT, LF_EHIP. */
int lf_generate(lf_state *st, int32_t n, int32_t *out_tokens);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same n
 * decode steps in ONE launch as lf_generate, with the same kernel and results,
 * that allocates nothing -- no hipMalloc, hipFree or allocating library call.
 * The per-launch scratch (exchange words, progress and error words, argmax
 * partials, the token slot; lf_query(st, LF_Q_SCRATCH_BYTES) bytes) lives in
 * the library's static device array of LF_Q_SCRATCH_MAX bytes (4 MiB), one per
 * GPU, held until the process ends; it is cleared by a fill kernel at each
 * call.  Every state on a GPU shares that GPU's array: calls that overlap on
 * one GPU race.  out_tokens_dev (device, n int32 entries, caller-owned)
 * receives the sampled tokens; the pending (token, pos) advances as with
 * lf_generate.  Errors: LF_EINVAL (NULL, LF_HIDDEN_IO), LF_ERANGE (no pending
 * token, n < 1, pos + n > max_seq), LF_EUNSUPPORTED (the state needs more
 * scratch than the array holds), LF_ETIMEOUT, LF_EHIP. */
int lf_generate_noalloc(lf_state *st, int32_t n, int32_t *out_tokens_dev);

/* Teacher-forced prompt in ONE launch: tokens[i] (host array) is consumed at
 * position pos0 + i and its K/V written; no logits, no sampling, and the pending
 * token is cleared (follow with lf_set_position or lf_decode_step).
 * Errors: LF_ERANGE (token outside [0, vocab), pos0 + n > max_seq), LF_ETIMEOUT, LF_EHIP. */
int lf_prefill(lf_state *st, const int32_t *tokens, int32_t n, int32_t pos0);

/* Set the pending (token, pos) used by the next lf_generate. */
int lf_set_position(lf_state *st, int32_t token, int32_t pos);

/* Text of the last failure of a call on this thread ("" if none). */
const char *lf_last_error(const lf_state *st);

/* Logits (fp32, vocab entries) of the last step.  dst is a device pointer when
 * dst_is_device != 0, else a host pointer. */
int lf_get_logits(lf_state *st, float *dst, int dst_is_device);

/* Copy n cache rows (positions pos0 .. pos0+n-1) of one layer from / to device
 * buffers k_dev, v_dev laid out [n][n_kv_heads][head_dim] fp16.  Prefilled keys
 * are used as given (no rotary embedding is applied to them). */
int lf_kv_fill(lf_state *st, int32_t layer, int32_t pos0, int32_t n, const void *k_dev,
               const void *v_dev);
int lf_kv_read(lf_state *st, int32_t layer, int32_t pos0, int32_t n, void *k_dev, void *v_dev);

/* LF_HIDDEN_IO: set the fp32 [d] input of the first layer / read the fp32 [d]
 * residual after the last layer (device pointers). */
int lf_set_hidden(lf_state *st, const float *x_dev);
int lf_get_hidden(lf_state *st, float *x_dev);

/* LF_STATS: 16 uint64 per workgroup for the last launch, in 100 MHz ticks:
 * [0] wave 0 time polling other workgroups, [1] number of polls, [2] XCD id,
 * [3] kernel time, [4] input staging, [5] waiting for the stream waves,
 * [6] epilogues and publishing, [7] attention, [8] lm_head + token choice,
 * [9] stream wave 1 waiting for phase inputs, [10] stream wave 1 consuming,
 * [11] pieces stream wave 1 consumed, [12..15] zero.  bytes >= 128 * grid. */
int lf_get_stats(lf_state *st, void *dst, size_t bytes);

/* Grid size (workgroups = compute units used) and words of the launch plan. */
int lf_query(const lf_state *st, int32_t what);
#define LF_Q_GRID 0
#define LF_Q_THREADS 1
#define LF_Q_LDS_BYTES 2
#define LF_Q_SCRATCH_BYTES 3   /* scratch lf_generate_noalloc uses for this state */
#define LF_Q_SCRATCH_MAX 4     /* bytes of the static scratch array */
#define LF_Q_KV_PF 5           /* stream waves per attention unit whose first K/V tile is prefetched into LDS */
#define LF_Q_GU_PF 6           /* pieces per stream wave of projection LF_Q_PF_KIND prefetched into LDS */
#define LF_Q_WAVE_W 7          /* + k, k = 0..6: share weight of stream wave k + 1 (a workgroup's rows of a
                                  projection go to its seven stream waves in proportion to these weights, no
                                  wave taking more whole rounds of 8 pieces than an equal share would, plus
                                  one where that is 8 or more) */
#define LF_Q_WAVE_W_KINDS 14   /* bit mask of the projections split by those weights (QKV 1, O 2, gate/up 4,
                                  down 8, lm_head 16); the others are split equally */
#define LF_Q_PF_KIND 15        /* the projection LF_Q_GU_PF prefetches: 1 output projection, 2 gate/up */

/* Test hooks, device pointers, on `stream`:
 * lf_test_expdef: y[i] = E(x[i]) with the library's defined exponential.
 * lf_test_sample: for each case c < m, the token the in-kernel sampler picks
 * from logits_dev[c*n .. c*n+n) with (temperature, top_p, seed) and RNG counter
 * pos_dev[c]; tokens_dev[c] receives it. */
int lf_test_expdef(const float *x_dev, float *y_dev, int64_t n, void *stream);
/* lf_test_logdef: y[i] = L(x[i]), the library's defined natural logarithm, for
 * positive normal x (the Gumbel noise's only use; other inputs are not defined).
 * lf_test_sample_gumbel: for each case c < m, the LF_GUMBEL token of
 * logits_dev[c*n .. c*n+n) at temperature T and RNG counter pos_dev[c].
 * All return LF_EINVAL on NULL pointers, n < 1 or T <= 0, LF_EHIP on a HIP error,
 * and wait for the stream. */
int lf_test_logdef(const float *x_dev, float *y_dev, int64_t n, void *stream);
int lf_test_sample_gumbel(const float *logits_dev, int32_t n, float temperature, uint64_t seed,
                          const int32_t *pos_dev, int32_t m, int32_t *tokens_dev, void *stream);
int lf_test_sample(const float *logits_dev, int32_t n, float temperature, float top_p,
                   uint64_t seed, const int32_t *pos_dev, int32_t m, int32_t *tokens_dev,
                   void *stream);

#ifdef __cplusplus
}
#endif
#endif

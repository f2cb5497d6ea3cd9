/*
 * lf_oracle.h -- plain, slow CPU reference of the batch-1 decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  This library exists to check the GPU path.  Only
 * the tests, the smoke check and the CPU-baseline leg of the benchmark may load
 * it; the product path never does.  It shares no code, header, table or
 * constant with the GPU library.
 *
 * What it computes (a Llama-style pre-norm decoder, fp32 arithmetic, fp16
 * weights and fp16 KV cache):
 *   x   = fp32(E[token])
 *   per layer:  h = rmsnorm(x, g_attn);  q = Wq h;  k = Wk h;  v = Wv h
 *               rope(q), rope(k) at position pos (rotate-half pairs)
 *               K[pos] = fp16(k);  V[pos] = fp16(v)
 *               o = causal softmax attention of q over K[0..pos], V[0..pos]
 *               x = x + Wo o
 *               h = rmsnorm(x, g_ffn);  a = silu(Wg h) * (Wu h);  x = x + Wd a
 *   logits = Wlm rmsnorm(x, g_final)
 *   next token: greedy argmax (lowest index on ties), or temperature / top-p
 *               nucleus sampling with integer masses and a Philox4x32-10 draw.
 *
 * Sources: "KOG LaneFormer-2B & the monokernel" (shivam2003.com), sections
 * "The problem" (each token streams all weights through GEMVs), "The fused
 * operations, briefly" (dot products with fp32 accumulation, cross-CU softmax
 * correction of attention, sampling at the end of the pass) and "Pillar 1"
 * (Llama-2 lineage, GQA).  The pages never write the block out; the block above
 * is the plainest reading, and every step below names the reading it takes.
 *
 * Conventions: every matrix is fp16 (raw IEEE binary16 bits, uint16_t),
 * row-major [out][in], host memory.  The KV cache is [layer][pos][kv_head][dh]
 * fp16 bits, owned by the caller.  All functions return 0 on success or a
 * negative value on a bad argument.
 */
#ifndef LF_ORACLE_H
#define LF_ORACLE_H
#include <stdint.h>
#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t n_layers, d_model, n_heads, n_kv_heads, head_dim, ffn_dim, vocab, max_seq;
  float rms_eps, rope_base;
  int32_t sliding_window;   /* 0: every layer attends to all earlier positions */
  int32_t reserved;
  uint64_t window_layers;   /* bit l set: layer l attends to the last sliding_window positions */
} orc_config;

typedef struct {
  const uint16_t *attn_norm, *wq, *wk, *wv, *wo, *ffn_norm, *w_gate, *w_up, *w_down;
} orc_layer;

typedef struct {
  const uint16_t *tok_emb, *final_norm, *lm_head;
  const orc_layer *layers;
} orc_weights;

/* ---- scalar building blocks ---- */
float    orc_f16_to_f32(uint16_t h);
uint16_t orc_f32_to_f16(float f);                 /* round to nearest, ties to even */
void     orc_f16_to_f32_n(const uint16_t *src, float *dst, size_t n);
void     orc_f32_to_f16_n(const float *src, uint16_t *dst, size_t n);

/* y[r] = sum_k W[r][k] * x[k], fp32, summed in column order. */
void orc_gemv(const uint16_t *W, const float *x, int32_t rows, int32_t cols, float *y);
/* y_i = g_i * (x_i / sqrtf(sum_j x_j^2 / d + eps)) */
void orc_rmsnorm(const float *x, const uint16_t *g, int32_t d, float eps, float *y);
/* in-place rotate-half RoPE of one head vector of length dh at position pos */
void orc_rope(float *v, int32_t dh, int32_t pos, float base);
/* attention of n_heads query heads at position pos over cache rows 0..pos of one layer
 * (rows pos-window+1..pos when window > 0).
 * q: [n_heads][dh] fp32; kc, vc: layer base of the cache [max_seq][n_kv][dh]; o: [n_heads][dh]. */
void orc_attention(const float *q, const uint16_t *kc, const uint16_t *vc, int32_t pos,
                   int32_t n_heads, int32_t n_kv_heads, int32_t dh, int32_t window, float *o);
float orc_silu(float z);

/* ---- the decoder ---- */
/* one layer at position pos on the fp32 residual x (in place); writes K/V at pos. */
int orc_layer_forward(const orc_config *c, const orc_layer *w, uint16_t *kc_layer,
                      uint16_t *vc_layer, float *x, int32_t pos, int32_t layer);
/* the window layer l attends over: c->sliding_window if bit l of c->window_layers is set, else 0 */
int32_t orc_layer_window(const orc_config *c, int32_t layer);
/* full decode step: embed token, all layers, final norm, lm_head -> logits[V]. */
int orc_decode_step(const orc_config *c, const orc_weights *w, uint16_t *kcache,
                    uint16_t *vcache, int32_t token, int32_t pos, float *logits);
/* second path: no KV cache; recomputes every position 0..n-1 of tokens[] with full
 * causal attention (K/V still rounded to fp16) and returns the logits of the last one. */
int orc_forward_nocache(const orc_config *c, const orc_weights *w, const int32_t *tokens,
                        int32_t n, float *logits);

/* ---- next-token selection ---- */
int32_t  orc_argmax(const float *logits, int32_t n);           /* lowest index on ties */
float    orc_expdef(float x);                                  /* defined exp, x <= 0 */
/* the 11 binary32 constants of orc_expdef: log2(e), ln2 hi, ln2 lo, 1/0! .. 1/7! */
void     orc_expdef_constants(float out[11]);
void     orc_expdef_n(const float *x, float *y, size_t n);
void     orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);
float    orc_logdef(float x);                                  /* defined ln, x > 0 normal */
void     orc_logdef_n(const float *x, float *y, size_t n);
float    orc_gumbel_noise(uint64_t seed, int32_t pos, int32_t i);  /* -L(-L(u_i)) */
int32_t  orc_sample_gumbel(const float *logits, int32_t n, float temperature, uint64_t seed,
                           int32_t pos);                       /* argmax(z + g) */
/* temperature == 0 -> argmax; else nucleus sampling keyed by (seed, pos). */
int32_t  orc_sample(const float *logits, int32_t n, float temperature, float top_p,
                    uint64_t seed, int32_t pos);
/* details of the nucleus draw for tests: masses q[n] (u64), K (nucleus size),
 * C_V, C_N, the draw t, and the chosen token. */
int32_t  orc_sample_detail(const float *logits, int32_t n, float temperature, float top_p,
                           uint64_t seed, int32_t pos, uint64_t *q_out, int32_t *nucleus_size,
                           uint64_t *c_v, uint64_t *c_n, uint64_t *t_draw, uint8_t *in_nucleus);

/* n steps from (token, pos): out[i] = next token of step i; logits_hist [n][V] nullable. */
int orc_generate(const orc_config *c, const orc_weights *w, uint16_t *kcache, uint16_t *vcache,
                 int32_t token, int32_t pos, int32_t n, float temperature, float top_p,
                 uint64_t seed, int32_t *out, float *logits_hist);

/* thread count used by the GEMV loops (results do not depend on it). */
void orc_set_threads(int32_t n);
int32_t orc_get_threads(void);

#ifdef __cplusplus
}
#endif
#endif

/*
 * lf_oracle.cpp -- plain, slow CPU reference of the batch-1 decode step.
 *
 * TEST INFRASTRUCTURE ONLY: called by the tests, the smoke check and the
 * CPU-baseline leg of the benchmark, never by the product path.  No code,
 * header, table or constant is shared with the GPU library.
 *
 * Build: g++ -O2 -fopenmp -ffp-contract=off (no fused multiply-add except the
 * explicit fmaf calls of the defined exp), so each line below is one IEEE
 * operation in the order written.
 *
 * Source pages: "KOG LaneFormer-2B & the monokernel" (shivam2003.com): "The
 * problem" and "A worked bandwidth ceiling" (each token streams every weight
 * once through matrix-vector products), "The fused operations, briefly" (fp32
 * accumulation of dot products; attention split over the sequence and merged
 * with an online-softmax correction, which is an exact identity, so a single
 * pass is used here; sampling closes the pass) and "Pillar 1" (Llama-2 lineage,
 * grouped-query attention).  Readings where the pages are silent are named at
 * each function.
 */
#include "lf_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#include <vector>
#include <algorithm>
#ifdef _OPENMP
#include <omp.h>
#endif

static int g_threads = 1;

extern "C" void orc_set_threads(int32_t n) { g_threads = n < 1 ? 1 : n; }
extern "C" int32_t orc_get_threads(void) { return g_threads; }

/* ------------------------------------------------------------------ fp16 */

/* binary16 -> binary32, exact: value = (1024 + m) * 2^(e-25) for normals,
 * m * 2^-24 for subnormals. */
extern "C" float orc_f16_to_f32(uint16_t h) {
  const int sign = (h >> 15) & 1;
  const int e = (h >> 10) & 0x1f;
  const int m = h & 0x3ff;
  float v;
  if (e == 0) {
    v = ldexpf((float)m, -24);
  } else if (e == 31) {
    v = m ? NAN : INFINITY;
  } else {
    v = ldexpf((float)(1024 + m), e - 25);
  }
  return sign ? -v : v;
}

/* binary32 -> binary16, round to nearest, ties to even. */
extern "C" uint16_t orc_f32_to_f16(float f) {
  uint32_t b;
  memcpy(&b, &f, 4);
  const uint16_t sign = (uint16_t)((b >> 16) & 0x8000u);
  const uint32_t a = b & 0x7fffffffu;
  if (a >= 0x7f800000u) return sign | (a > 0x7f800000u ? 0x7e00 : 0x7c00); /* NaN / inf */
  if (a >= 0x477ff000u) return sign | 0x7c00;      /* |f| >= 65520 rounds to inf */
  if (a < 0x38800000u) {                           /* |f| < 2^-14: fp16 subnormal or zero */
    float s = fabsf(f) * 16777216.0f;              /* exact: |f| / 2^-24, below 1024 */
    return sign | (uint16_t)rintf(s);              /* RNE to an integer count of 2^-24 */
  }
  uint32_t e = (a >> 23) - 127 + 15;               /* 1..30 */
  uint32_t m = a & 0x7fffffu;
  uint32_t h = (e << 10) | (m >> 13);
  uint32_t rem = m & 0x1fffu;
  if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h += 1;  /* carry into exponent is correct */
  return sign | (uint16_t)h;
}

extern "C" void orc_f16_to_f32_n(const uint16_t *src, float *dst, size_t n) {
  for (size_t i = 0; i < n; ++i) dst[i] = orc_f16_to_f32(src[i]);
}
extern "C" void orc_f32_to_f16_n(const float *src, uint16_t *dst, size_t n) {
  for (size_t i = 0; i < n; ++i) dst[i] = orc_f32_to_f16(src[i]);
}

/* 65536-entry decode table built from orc_f16_to_f32 (same values, faster). */
static const float *f16tab() {
  static std::vector<float> tab;
  if (tab.empty()) {
    std::vector<float> t(65536);
    for (uint32_t i = 0; i < 65536; ++i) t[i] = orc_f16_to_f32((uint16_t)i);
    tab.swap(t);
  }
  return tab.data();
}

/* --------------------------------------------------------------- blocks */

/* Matrix-vector product, fp32 accumulation in column order ("The fused
 * operations": dot products accumulate in FP32). */
extern "C" void orc_gemv(const uint16_t *W, const float *x, int32_t rows, int32_t cols, float *y) {
  const float *T = f16tab();
#pragma omp parallel for schedule(static) num_threads(g_threads)
  for (int32_t r = 0; r < rows; ++r) {
    const uint16_t *w = W + (size_t)r * cols;
    float acc = 0.0f;
    for (int32_t k = 0; k < cols; ++k) acc += T[w[k]] * x[k];
    y[r] = acc;
  }
}

/* RMSNorm, eps inside the square root: y_i = g_i * (x_i / sqrt(mean(x^2) + eps)). */
extern "C" void orc_rmsnorm(const float *x, const uint16_t *g, int32_t d, float eps, float *y) {
  float ss = 0.0f;
  for (int32_t j = 0; j < d; ++j) ss += x[j] * x[j];
  const float r = sqrtf(ss / (float)d + eps);
  for (int32_t i = 0; i < d; ++i) y[i] = orc_f16_to_f32(g[i]) * (x[i] / r);
}

/* Rotary embedding, rotate-half pairing (i, i + dh/2).  The pages do not fix a
 * convention; any one shared by both sides is correct for random weights.
 * Angle theta_i = base^(-2i/dh) and phase p*theta_i in fp64, cos/sin rounded to fp32. */
extern "C" void orc_rope(float *v, int32_t dh, int32_t pos, float base) {
  const int32_t half = dh / 2;
  for (int32_t i = 0; i < half; ++i) {
    const double theta = pow((double)base, -2.0 * (double)i / (double)dh);
    const double phi = (double)pos * theta;
    const float c = (float)cos(phi), s = (float)sin(phi);
    const float a = v[i], b = v[i + half];
    v[i] = a * c - b * s;
    v[i + half] = b * c + a * s;
  }
}

/* Causal attention of one position over cache rows 0..pos, or with window > 0
 * over the last `window` of them, rows max(0, pos - window + 1)..pos (sliding-
 * window attention, "KOG LaneFormer-2B & the monokernel", "Pillar 1": it bounds
 * the KV rows a step reads).  Query head h uses
 * KV head h / (n_heads / n_kv_heads) (contiguous groups).  Scores scaled by
 * 1/sqrt(dh), softmax with max subtraction, o = sum_j a_j v_j.  A split over
 * the sequence merged by online-softmax correction is the same quantity, so one
 * pass is used. */
extern "C" void orc_attention(const float *q, const uint16_t *kc, const uint16_t *vc, int32_t pos,
                              int32_t n_heads, int32_t n_kv_heads, int32_t dh, int32_t window, float *o) {
  const int32_t group = n_heads / n_kv_heads;
  const int32_t j_lo = window > 0 && pos + 1 > window ? pos + 1 - window : 0;
  kc += (size_t)j_lo * n_kv_heads * dh;   /* the rows the window keeps, renumbered from 0 */
  vc += (size_t)j_lo * n_kv_heads * dh;
  const int32_t n = pos + 1 - j_lo;
  const float scale = 1.0f / sqrtf((float)dh);
  std::vector<float> s(n);
  for (int32_t h = 0; h < n_heads; ++h) {
    const int32_t g = h / group;
    const float *qh = q + (size_t)h * dh;
    for (int32_t j = 0; j < n; ++j) {
      const uint16_t *kj = kc + ((size_t)j * n_kv_heads + g) * dh;
      float acc = 0.0f;
      for (int32_t e = 0; e < dh; ++e) acc += qh[e] * orc_f16_to_f32(kj[e]);
      s[j] = acc * scale;
    }
    float m = s[0];
    for (int32_t j = 1; j < n; ++j) m = s[j] > m ? s[j] : m;
    float l = 0.0f;
    for (int32_t j = 0; j < n; ++j) { s[j] = expf(s[j] - m); l += s[j]; }
    float *oh = o + (size_t)h * dh;
    for (int32_t e = 0; e < dh; ++e) oh[e] = 0.0f;
    for (int32_t j = 0; j < n; ++j) {
      const float a = s[j] / l;
      const uint16_t *vj = vc + ((size_t)j * n_kv_heads + g) * dh;
      for (int32_t e = 0; e < dh; ++e) oh[e] += a * orc_f16_to_f32(vj[e]);
    }
  }
}

extern "C" float orc_silu(float z) { return z / (1.0f + expf(-z)); }

static bool cfg_ok(const orc_config *c) {
  return c && c->n_layers > 0 && c->d_model > 0 && c->n_heads > 0 && c->n_kv_heads > 0 &&
         c->n_heads % c->n_kv_heads == 0 && c->head_dim > 0 && c->head_dim % 2 == 0 &&
         c->ffn_dim > 0 && c->max_seq > 0;
}

/* One pre-norm decoder layer at position pos (Llama-2 lineage, "Pillar 1"). */
extern "C" int32_t orc_layer_window(const orc_config *c, int32_t layer) {
  const bool on = c->sliding_window > 0 && layer >= 0 && layer < 64 && ((c->window_layers >> layer) & 1u);
  return on ? c->sliding_window : 0;
}

extern "C" int orc_layer_forward(const orc_config *c, const orc_layer *w, uint16_t *kc,
                                 uint16_t *vc, float *x, int32_t pos, int32_t layer) {
  if (!cfg_ok(c) || !w || !kc || !vc || !x || pos < 0 || pos >= c->max_seq) return -1;
  const int32_t d = c->d_model, hq = c->n_heads, hkv = c->n_kv_heads, dh = c->head_dim,
                f = c->ffn_dim;
  std::vector<float> h(d), q((size_t)hq * dh), k((size_t)hkv * dh), v((size_t)hkv * dh),
      o((size_t)hq * dh), y(d), g(f), u(f), a(f);
  orc_rmsnorm(x, w->attn_norm, d, c->rms_eps, h.data());
  orc_gemv(w->wq, h.data(), hq * dh, d, q.data());
  orc_gemv(w->wk, h.data(), hkv * dh, d, k.data());
  orc_gemv(w->wv, h.data(), hkv * dh, d, v.data());
  for (int32_t i = 0; i < hq; ++i) orc_rope(q.data() + (size_t)i * dh, dh, pos, c->rope_base);
  for (int32_t i = 0; i < hkv; ++i) orc_rope(k.data() + (size_t)i * dh, dh, pos, c->rope_base);
  uint16_t *krow = kc + (size_t)pos * hkv * dh, *vrow = vc + (size_t)pos * hkv * dh;
  for (int32_t i = 0; i < hkv * dh; ++i) { krow[i] = orc_f32_to_f16(k[i]); vrow[i] = orc_f32_to_f16(v[i]); }
  orc_attention(q.data(), kc, vc, pos, hq, hkv, dh, orc_layer_window(c, layer), o.data());
  orc_gemv(w->wo, o.data(), d, hq * dh, y.data());
  for (int32_t i = 0; i < d; ++i) x[i] = x[i] + y[i];
  orc_rmsnorm(x, w->ffn_norm, d, c->rms_eps, h.data());
  orc_gemv(w->w_gate, h.data(), f, d, g.data());
  orc_gemv(w->w_up, h.data(), f, d, u.data());
  for (int32_t j = 0; j < f; ++j) a[j] = orc_silu(g[j]) * u[j];
  orc_gemv(w->w_down, a.data(), d, f, y.data());
  for (int32_t i = 0; i < d; ++i) x[i] = x[i] + y[i];
  return 0;
}

extern "C" int orc_decode_step(const orc_config *c, const orc_weights *w, uint16_t *kcache,
                               uint16_t *vcache, int32_t token, int32_t pos, float *logits) {
  if (!cfg_ok(c) || !w || !w->tok_emb || !w->lm_head || !w->final_norm || !logits) return -1;
  if (token < 0 || token >= c->vocab || pos < 0 || pos >= c->max_seq) return -2;
  const int32_t d = c->d_model;
  const size_t layer_stride = (size_t)c->max_seq * c->n_kv_heads * c->head_dim;
  std::vector<float> x(d), h(d);
  orc_f16_to_f32_n(w->tok_emb + (size_t)token * d, x.data(), d);
  for (int32_t l = 0; l < c->n_layers; ++l) {
    int rc = orc_layer_forward(c, &w->layers[l], kcache + l * layer_stride,
                               vcache + l * layer_stride, x.data(), pos, l);
    if (rc) return rc;
  }
  orc_rmsnorm(x.data(), w->final_norm, d, c->rms_eps, h.data());
  orc_gemv(w->lm_head, h.data(), c->vocab, d, logits);
  return 0;
}

/* Second, cache-free path: all positions of the prefix are recomputed layer by
 * layer and each attends causally over the fp16-rounded keys/values of its
 * predecessors.  Shares only the building blocks above with the cached path. */
extern "C" int orc_forward_nocache(const orc_config *c, const orc_weights *w, const int32_t *tokens,
                                   int32_t n, float *logits) {
  if (!cfg_ok(c) || !w || !tokens || n <= 0 || n > c->max_seq || !logits) return -1;
  const int32_t d = c->d_model, hq = c->n_heads, hkv = c->n_kv_heads, dh = c->head_dim,
                f = c->ffn_dim;
  const int32_t group = hq / hkv;
  const float scale = 1.0f / sqrtf((float)dh);
  std::vector<float> X((size_t)n * d);
  for (int32_t i = 0; i < n; ++i) {
    if (tokens[i] < 0 || tokens[i] >= c->vocab) return -2;
    orc_f16_to_f32_n(w->tok_emb + (size_t)tokens[i] * d, X.data() + (size_t)i * d, d);
  }
  std::vector<float> h(d), Q((size_t)n * hq * dh), Kf((size_t)n * hkv * dh), Vf((size_t)n * hkv * dh),
      o((size_t)hq * dh), y(d), g(f), u(f), a(f), s(n);
  for (int32_t l = 0; l < c->n_layers; ++l) {
    const orc_layer *L = &w->layers[l];
    for (int32_t i = 0; i < n; ++i) {
      float *xi = X.data() + (size_t)i * d;
      orc_rmsnorm(xi, L->attn_norm, d, c->rms_eps, h.data());
      float *qi = Q.data() + (size_t)i * hq * dh, *ki = Kf.data() + (size_t)i * hkv * dh,
            *vi = Vf.data() + (size_t)i * hkv * dh;
      orc_gemv(L->wq, h.data(), hq * dh, d, qi);
      orc_gemv(L->wk, h.data(), hkv * dh, d, ki);
      orc_gemv(L->wv, h.data(), hkv * dh, d, vi);
      for (int32_t t = 0; t < hq; ++t) orc_rope(qi + (size_t)t * dh, dh, i, c->rope_base);
      for (int32_t t = 0; t < hkv; ++t) orc_rope(ki + (size_t)t * dh, dh, i, c->rope_base);
      for (int32_t e = 0; e < hkv * dh; ++e) {   /* the cache holds fp16; so does this path */
        ki[e] = orc_f16_to_f32(orc_f32_to_f16(ki[e]));
        vi[e] = orc_f16_to_f32(orc_f32_to_f16(vi[e]));
      }
    }
    const int32_t win = orc_layer_window(c, l);
    for (int32_t i = 0; i < n; ++i) {
      const int32_t jl = win > 0 && i + 1 > win ? i + 1 - win : 0;   /* first key in the window */
      for (int32_t t = 0; t < hq; ++t) {
        const int32_t gk = t / group;
        const float *qt = Q.data() + ((size_t)i * hq + t) * dh;
        for (int32_t j = jl; j <= i; ++j) {
          const float *kj = Kf.data() + ((size_t)j * hkv + gk) * dh;
          float acc = 0.0f;
          for (int32_t e = 0; e < dh; ++e) acc += qt[e] * kj[e];
          s[j] = acc * scale;
        }
        float m = s[jl];
        for (int32_t j = jl + 1; j <= i; ++j) m = s[j] > m ? s[j] : m;
        float lsum = 0.0f;
        for (int32_t j = jl; j <= i; ++j) { s[j] = expf(s[j] - m); lsum += s[j]; }
        float *ot = o.data() + (size_t)t * dh;
        for (int32_t e = 0; e < dh; ++e) ot[e] = 0.0f;
        for (int32_t j = jl; j <= i; ++j) {
          const float p = s[j] / lsum;
          const float *vj = Vf.data() + ((size_t)j * hkv + gk) * dh;
          for (int32_t e = 0; e < dh; ++e) ot[e] += p * vj[e];
        }
      }
      float *xi = X.data() + (size_t)i * d;
      orc_gemv(L->wo, o.data(), d, hq * dh, y.data());
      for (int32_t e = 0; e < d; ++e) xi[e] = xi[e] + y[e];
      orc_rmsnorm(xi, L->ffn_norm, d, c->rms_eps, h.data());
      orc_gemv(L->w_gate, h.data(), f, d, g.data());
      orc_gemv(L->w_up, h.data(), f, d, u.data());
      for (int32_t j = 0; j < f; ++j) a[j] = orc_silu(g[j]) * u[j];
      orc_gemv(L->w_down, a.data(), d, f, y.data());
      for (int32_t e = 0; e < d; ++e) xi[e] = xi[e] + y[e];
    }
  }
  orc_rmsnorm(X.data() + (size_t)(n - 1) * d, w->final_norm, d, c->rms_eps, h.data());
  orc_gemv(w->lm_head, h.data(), c->vocab, d, logits);
  return 0;
}

/* ------------------------------------------------------------- sampling */

/* Greedy choice: largest logit, the lowest index among equal maxima. */
extern "C" int32_t orc_argmax(const float *logits, int32_t n) {
  int32_t best = 0;
  for (int32_t i = 1; i < n; ++i)
    if (logits[i] > logits[best]) best = i;
  return best;
}

/* Defined exponential E(x) for x <= 0, identical on any IEEE-754 machine:
 *   k = rint(x * log2(e));  r = x - k ln2 (two-constant Cody-Waite, each step one fma);
 *   p = degree-7 Taylor polynomial of e^r in Horner form (fma);  E = p * 2^k.
 * Constants are the nearest binary32 values of log2(e), ln 2, the remainder
 * ln 2 - LN2_HI, and 1/n!; derived from the exact values, not from any libm. */
static const float EXP_L2E = 0x1.715476p+0f;      /* log2(e) */
static const float EXP_LN2_HI = 0x1.62e430p-1f;   /* ln 2 rounded to binary32 */
static const float EXP_LN2_LO = -0x1.05c610p-29f; /* ln 2 - EXP_LN2_HI, rounded */
static const float EXP_C[8] = {1.0f, 1.0f, 0x1.0p-1f, 0x1.555556p-3f, 0x1.555556p-5f,
                               0x1.111112p-7f, 0x1.6c16c2p-10f, 0x1.a01a02p-13f}; /* 1/n! */

extern "C" float orc_expdef(float x) {
  const float k = rintf(x * EXP_L2E);
  float r = fmaf(-k, EXP_LN2_HI, x);
  r = fmaf(-k, EXP_LN2_LO, r);
  float p = EXP_C[7];
  for (int n = 6; n >= 0; --n) p = fmaf(p, r, EXP_C[n]);
  return ldexpf(p, (int)k);
}

extern "C" void orc_expdef_n(const float *x, float *y, size_t n) {
  for (size_t i = 0; i < n; ++i) y[i] = orc_expdef(x[i]);
}

extern "C" void orc_expdef_constants(float out[11]) {
  out[0] = EXP_L2E; out[1] = EXP_LN2_HI; out[2] = EXP_LN2_LO;
  for (int i = 0; i < 8; ++i) out[3 + i] = EXP_C[i];
}

/* Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy
 * as 1, 2, 3", SC'11): ten rounds of the 4x32 Philox round, the key bumped by
 * the two Weyl constants between rounds. */
extern "C" void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u, W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
  uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3], k0 = key[0], k1 = key[1];
  for (int round = 0; round < 10; ++round) {
    if (round > 0) { k0 += W0; k1 += W1; }
    const uint64_t p0 = (uint64_t)M0 * c0, p1 = (uint64_t)M1 * c2;
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    const uint32_t n0 = hi1 ^ c1 ^ k0, n1 = lo1, n2 = hi0 ^ c3 ^ k1, n3 = lo0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* Temperature / top-p sampling with integer masses (reading of the pages'
 * on-device sampling, made bit-reproducible):
 *   z_i = logit_i * (float)(1/T);  z* = max z;
 *   q_i = floor(E(z_i - z*) * 2^32), 0 when z_i - z* < -23;  C_V = sum q_i;
 *   order tokens by (z desc, index asc); M* = ceil(top_p * C_V) in fp64;
 *   the nucleus is the shortest prefix of that order whose mass reaches M* (>= 1 token);
 *   Philox4x32-10 with key (seed lo, seed hi) and counter (pos, 0, 0, 0) gives x0, x1;
 *   t = floor(((x1 << 32) | x0) * C_N / 2^64), C_N the nucleus mass;
 *   the token is the first nucleus member in ascending index order whose running
 *   nucleus mass exceeds t. */
extern "C" int32_t orc_sample_detail(const float *logits, int32_t n, float temperature, float top_p,
                                     uint64_t seed, int32_t pos, uint64_t *q_out,
                                     int32_t *nucleus_size, uint64_t *c_v, uint64_t *c_n,
                                     uint64_t *t_draw, uint8_t *in_nucleus) {
  if (n <= 0) return -1;
  if (!(temperature > 0.0f)) return orc_argmax(logits, n);
  const float invT = (float)(1.0 / (double)temperature);
  std::vector<float> z(n);
  for (int32_t i = 0; i < n; ++i) z[i] = logits[i] * invT;
  float zmax = z[0];
  for (int32_t i = 1; i < n; ++i) zmax = z[i] > zmax ? z[i] : zmax;
  std::vector<uint64_t> q(n);
  uint64_t CV = 0;
  for (int32_t i = 0; i < n; ++i) {
    const float dz = z[i] - zmax;
    q[i] = dz < -23.0f ? 0 : (uint64_t)(orc_expdef(dz) * 4294967296.0f);
    CV += q[i];
  }
  std::vector<int32_t> order(n);
  for (int32_t i = 0; i < n; ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
    if (z[a] != z[b]) return z[a] > z[b];
    return a < b;
  });
  const uint64_t Mstar = (uint64_t)ceil((double)top_p * (double)CV);
  int32_t K = 0;
  uint64_t cum = 0;
  do { cum += q[order[K]]; ++K; } while (K < n && cum < Mstar);
  std::vector<uint8_t> inN(n, 0);
  for (int32_t k = 0; k < K; ++k) inN[order[k]] = 1;
  uint64_t CN = 0;
  for (int32_t i = 0; i < n; ++i) if (inN[i]) CN += q[i];
  const uint32_t ctr[4] = {(uint32_t)pos, 0u, 0u, 0u};
  const uint32_t key[2] = {(uint32_t)(seed & 0xffffffffu), (uint32_t)(seed >> 32)};
  uint32_t x[4];
  orc_philox4x32_10(ctr, key, x);
  const uint64_t r = ((uint64_t)x[1] << 32) | x[0];
  const uint64_t t = (uint64_t)(((unsigned __int128)r * CN) >> 64);
  int32_t tok = -1;
  uint64_t run = 0;
  for (int32_t i = 0; i < n; ++i) {
    if (!inN[i]) continue;
    run += q[i];
    if (run > t) { tok = i; break; }
  }
  if (q_out) memcpy(q_out, q.data(), sizeof(uint64_t) * n);
  if (nucleus_size) *nucleus_size = K;
  if (c_v) *c_v = CV;
  if (c_n) *c_n = CN;
  if (t_draw) *t_draw = t;
  if (in_nucleus) memcpy(in_nucleus, inN.data(), n);
  return tok;
}

extern "C" int32_t orc_sample(const float *logits, int32_t n, float temperature, float top_p,
                              uint64_t seed, int32_t pos) {
  return orc_sample_detail(logits, n, temperature, top_p, seed, pos, nullptr, nullptr, nullptr,
                           nullptr, nullptr, nullptr);
}

/* Defined natural logarithm L(x) for positive normal binary32 x, identical on any
 * IEEE-754 machine (every step one correctly rounded operation or one fma):
 *   x = m 2^e with m in [sqrt(1/2), sqrt(2)) (read from the bits);  f = m - 1 (exact);
 *   s = f / (2 + f);  ln(1 + f) = 2 atanh(s) = 2s + 2s R(s^2) with
 *   R(w) = w/3 + w^2/5 + ... + w^6/13 in Horner form;  L = e ln2_hi + (e ln2_lo + ln(1+f)).
 * Constants are the nearest binary32 values of ln 2 (split hi / lo) and 1/(2k+1). */
static const float LOG_SQRT2 = 0x1.6a09e6p+0f;     /* sqrt(2) rounded */
static const float LOG_LN2_HI = 0x1.62e430p-1f;    /* ln 2 rounded to binary32 */
static const float LOG_LN2_LO = -0x1.05c610p-29f;  /* ln 2 - LOG_LN2_HI, rounded */
static const float LOG_C[6] = {0x1.555556p-2f, 0x1.99999ap-3f, 0x1.24924ap-3f,
                               0x1.c71c72p-4f, 0x1.745d18p-4f, 0x1.3b13b2p-4f}; /* 1/3 .. 1/13 */

extern "C" float orc_logdef(float x) {
  uint32_t bits;
  memcpy(&bits, &x, 4);
  int e = (int)(bits >> 23) - 127;
  const uint32_t mb = (bits & 0x7fffffu) | 0x3f800000u;
  float m;
  memcpy(&m, &mb, 4);
  if (m > LOG_SQRT2) { m = m * 0.5f; e += 1; }
  const float f = m - 1.0f;
  const float s = f / (2.0f + f);
  const float w = s * s;
  float r = LOG_C[5];
  for (int k = 4; k >= 0; --k) r = fmaf(r, w, LOG_C[k]);
  r = r * w;
  const float s2 = s + s;
  const float l1p = fmaf(s2, r, s2);
  const float ef = (float)e;
  return fmaf(ef, LOG_LN2_HI, fmaf(ef, LOG_LN2_LO, l1p));
}

extern "C" void orc_logdef_n(const float *x, float *y, size_t n) {
  for (size_t i = 0; i < n; ++i) y[i] = orc_logdef(x[i]);
}

/* Gumbel noise of vocabulary entry i at RNG counter pos (reading of the pages'
 * Gumbel-max sampling, made bit-reproducible): Philox4x32-10 with key (seed lo,
 * seed hi) and counter (pos, i, 1, 0) gives x0; u = (2 (x0 >> 9) + 1) 2^-24, a
 * binary32 value strictly inside (0, 1); g = -L(-L(u)). */
extern "C" float orc_gumbel_noise(uint64_t seed, int32_t pos, int32_t i) {
  const uint32_t ctr[4] = {(uint32_t)pos, (uint32_t)i, 1u, 0u};
  const uint32_t key[2] = {(uint32_t)(seed & 0xffffffffu), (uint32_t)(seed >> 32)};
  uint32_t x[4];
  orc_philox4x32_10(ctr, key, x);
  const float u = (float)(2u * (x[0] >> 9) + 1u) * 0x1.0p-24f;
  return -orc_logdef(-orc_logdef(u));
}

/* Gumbel-max sampling ("KOG LaneFormer-2B & the monokernel", "The fused
 * operations, briefly"): the token is argmax_i (z_i + g_i) with z_i = logit_i *
 * (float)(1/T) and g_i the noise above, the lowest index among equal maxima.
 * The sum is one binary32 addition.  Returns -1 for n <= 0; T <= 0 is greedy. */
extern "C" int32_t orc_sample_gumbel(const float *logits, int32_t n, float temperature, uint64_t seed,
                                     int32_t pos) {
  if (n <= 0) return -1;
  if (!(temperature > 0.0f)) return orc_argmax(logits, n);
  const float invT = (float)(1.0 / (double)temperature);
  int32_t best = 0;
  float bv = -INFINITY;
  for (int32_t i = 0; i < n; ++i) {
    const float y = logits[i] * invT + orc_gumbel_noise(seed, pos, i);
    if (y > bv) { bv = y; best = i; }
  }
  return best;
}

extern "C" int orc_generate(const orc_config *c, const orc_weights *w, uint16_t *kcache,
                            uint16_t *vcache, int32_t token, int32_t pos, int32_t n,
                            float temperature, float top_p, uint64_t seed, int32_t *out,
                            float *logits_hist) {
  if (!cfg_ok(c) || !out || n < 0) return -1;
  std::vector<float> logits(c->vocab);
  for (int32_t i = 0; i < n; ++i) {
    int rc = orc_decode_step(c, w, kcache, vcache, token, pos + i, logits.data());
    if (rc) return rc;
    if (logits_hist) memcpy(logits_hist + (size_t)i * c->vocab, logits.data(), sizeof(float) * c->vocab);
    token = orc_sample(logits.data(), c->vocab, temperature, top_p, seed, pos + i);
    out[i] = token;
  }
  return 0;
}

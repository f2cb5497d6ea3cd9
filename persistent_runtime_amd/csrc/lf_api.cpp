// lf_api.cpp -- the C ABI of include/lf.h: configuration checks, weight repack,
// allocation of the KV cache / activations / synchronisation words, the static
// launch plan, and the single cooperative launch per lf_decode_step /
// lf_generate call.
//
// The pages fix the work partition at compile time and never leave the kernel
// mid-token ("KOG LaneFormer-2B & the monokernel", sections "Compile-time work
// partition" and "Pillar 3"); here the partition is fixed when the state is
// created: contiguous row blocks of every matrix per workgroup, and
// (KV head, key chunk) attention units derived from the position.  Weights are
// transformed once, ahead of decoding, as the pages' section "Weight streaming"
// does it: rows are repacked so the rotary pairs (i, i + head_dim/2) of each
// head and the SwiGLU pairs (gate j, up j) sit in adjacent rows and every row
// block holds whole pairs, and each RMSNorm gain vector is folded into the
// columns of the projection that follows it.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/lf.h"
#include "lf_internal.h"

namespace {

thread_local std::string g_err;

int fail(std::string *dst, int code, const std::string &msg) {
  g_err = msg;
  if (dst) *dst = msg;
  return code;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace

struct lf_state {
  lf_config cfg{};
  hipStream_t stream = nullptr;
  int device = 0;
  lf::Params P{};
  std::vector<void *> allocs;
  int out_cap = 0, in_cap = 0;
  void *xbuf = nullptr;        // tagged exchange words (cleared whenever the level numbering restarts)
  size_t xbuf_bytes = 0;
  unsigned level_base = 0;
  int pending_token = -1, pending_pos = 0;
  bool has_pending = false;
  std::string err;
};

namespace {

int hip_fail(lf_state *st, hipError_t e, const char *what) {
  std::string m = std::string(what) + ": " + hipGetErrorString(e);
  return fail(st ? &st->err : nullptr, LF_EHIP, m);
}

void *dev_alloc(lf_state *st, size_t bytes, hipError_t *e) {
  void *p = nullptr;
  *e = hipMalloc(&p, bytes ? bytes : 16);
  if (*e != hipSuccess) return nullptr;
  st->allocs.push_back(p);
  return p;
}

int validate(const lf_config *c) {
  if (!c) return fail(nullptr, LF_EINVAL, "config is NULL");
  const bool hidden = (c->flags & LF_HIDDEN_IO) != 0;
  if (c->n_layers < 1 || c->d_model < 8 || c->n_heads < 1 || c->n_kv_heads < 1 || c->ffn_dim < 1 ||
      c->max_seq < 1)
    return fail(nullptr, LF_EINVAL, "sizes must be positive");
  if (c->d_model % 8 || c->ffn_dim % 8)
    return fail(nullptr, LF_EINVAL, "d_model and ffn_dim must be multiples of 8");
  if (c->d_model > 8192) return fail(nullptr, LF_EUNSUPPORTED, "d_model above 8192");
  if (c->n_heads % c->n_kv_heads)
    return fail(nullptr, LF_EINVAL, "n_heads must be a multiple of n_kv_heads");
  if (c->n_heads / c->n_kv_heads > 8) return fail(nullptr, LF_EUNSUPPORTED, "more than 8 query heads per KV head");
  if (c->head_dim != 64 && c->head_dim != 96 && c->head_dim != 128)
    return fail(nullptr, LF_EUNSUPPORTED, "head_dim must be 64, 96 or 128");
  if (c->sliding_window < 0) return fail(nullptr, LF_EINVAL, "sliding_window must be >= 0");
  if (c->sliding_window > 0) {
    // the layer mask is one 64-bit word: bit l selects layer l
    if (c->n_layers > 64) return fail(nullptr, LF_EUNSUPPORTED, "sliding windows need n_layers <= 64");
    if (c->n_layers < 64 && (c->window_layers >> c->n_layers) != 0)
      return fail(nullptr, LF_EINVAL, "window_layers has bits at or above n_layers");
  }
  if (!hidden && (c->vocab < 2 || c->vocab % 2))
    return fail(nullptr, LF_EINVAL, "vocab must be even and at least 2");
  if (!(c->rms_eps >= 0.0f) || !(c->rope_base > 0.0f)) return fail(nullptr, LF_EINVAL, "bad rms_eps or rope_base");
  if (!(c->temperature >= 0.0f)) return fail(nullptr, LF_EINVAL, "temperature must be >= 0");
  if (c->temperature > 0.0f && !(c->flags & LF_GUMBEL) && !(c->top_p > 0.0f))
    return fail(nullptr, LF_EINVAL, "top_p must be > 0");
  if (!hidden && c->temperature > 0.0f && !(c->flags & LF_GUMBEL) && c->vocab > lf::kSampMaxVocab)
    return fail(nullptr, LF_EUNSUPPORTED, "nucleus sampling supports vocabularies up to 393216");
  if (c->flags & ~(LF_HIDDEN_IO | LF_STATS | LF_GUMBEL)) return fail(nullptr, LF_EINVAL, "unknown flag bits");
  return LF_OK;
}

hipError_t copy_rows_strided(void *dst, size_t dpitch, const void *src, size_t spitch, size_t width,
                             size_t height, hipStream_t s) {
  if (height == 0) return hipSuccess;
  return hipMemcpy2DAsync(dst, dpitch, src, spitch, width, height, hipMemcpyDeviceToDevice, s);
}

// Restart the level numbering: progress words and every tagged
// exchange word go back to zero (no level is ever zero), level_base to 0.
hipError_t reset_levels(lf_state *st) {
  const lf::Params &P = st->P;
  hipError_t e;
  if ((e = hipMemsetAsync(P.progress, 0, sizeof(unsigned) * P.G, st->stream)) != hipSuccess) return e;
  if ((e = hipMemsetAsync(st->xbuf, 0, st->xbuf_bytes, st->stream)) != hipSuccess) return e;
  st->level_base = 0;
  return hipSuccess;
}

int do_launch(lf_state *st, int token0, int pos0, int n, std::vector<int> *out, bool prefill = false) {
  lf::Params &P = st->P;
  P.levels_per_token = lf::PH_PER_LAYER * P.L + ((P.hidden_io || prefill) ? 0 : 2 + (P.nuc_grid ? lf::kNucLevels : 0));
  const unsigned need = (unsigned)(n + 1) * (unsigned)P.levels_per_token;
  hipError_t e;
  if ((unsigned long long)st->level_base + need >= 0x7fffffffull) {
    if ((e = reset_levels(st)) != hipSuccess) return hip_fail(st, e, "reset levels");
  }
  P.n_tokens = n;
  P.trace_token = n / 2;
  P.token0 = token0;
  P.pos0 = pos0;
  P.level_base = st->level_base;
  if ((e = hipMemsetAsync(P.err, 0, 4 * sizeof(unsigned), st->stream)) != hipSuccess)
    return hip_fail(st, e, "clear error word");
  if ((e = lf::launch_monokernel(P, prefill, st->stream)) != hipSuccess) return hip_fail(st, e, "cooperative launch");
  if ((e = hipStreamSynchronize(st->stream)) != hipSuccess) return hip_fail(st, e, "kernel execution");
  unsigned herr[4];
  if ((e = hipMemcpy(herr, P.err, sizeof(herr), hipMemcpyDeviceToHost)) != hipSuccess)
    return hip_fail(st, e, "read error word");
  if (herr[0]) {
    // a bounded wait expired: the grid drained; restart the level numbering
    (void)reset_levels(st);
    (void)hipStreamSynchronize(st->stream);
    char buf[160];
    std::snprintf(buf, sizeof buf, "in-kernel wait timed out (workgroup %u, level %u)", herr[1], herr[2]);
    return fail(&st->err, LF_ETIMEOUT, buf);
  }
  st->level_base += (unsigned)n * (unsigned)P.levels_per_token;
  if (herr[3]) return fail(&st->err, LF_EHIP, "the token choice produced no valid token (non-finite logits?)");
  if (out && !P.hidden_io && !prefill) {
    out->resize(n);
    if ((e = hipMemcpy(out->data(), P.out_tokens, sizeof(int) * n, hipMemcpyDeviceToHost)) != hipSuccess)
      return hip_fail(st, e, "read tokens");
  }
  return LF_OK;
}

// Where lf_generate_noalloc puts the per-launch scratch inside the static
// array: the exchange words at the same offsets as in the state's own buffer,
// then the progress words, the error words, the argmax partials and the token
// slot.  Returns the bytes used; with base != null also fills P's pointers.
size_t noalloc_layout(const lf_state *st, char *base, lf::Params *P) {
  const lf::Params &S = st->P;
  auto rel = [&](const void *p) -> unsigned long long * {
    return reinterpret_cast<unsigned long long *>(base + ((const char *)p - (const char *)st->xbuf));
  };
  size_t off = align_up(st->xbuf_bytes, 256);
  const size_t prog = off;
  off += align_up((size_t)S.G * 4, 256);
  const size_t errw = off;
  off += 256;
  const size_t lmv = off;
  off += align_up((size_t)S.G * 4, 256);
  const size_t lmi = off;
  off += align_up((size_t)S.G * 4, 256);
  const size_t tok = off;
  off += 256;
  if (base && P) {
    P->xmid_t = rel(S.xmid_t);
    P->xout_t = rel(S.xout_t);
    P->q_t = rel(S.q_t);
    P->kc_t = rel(S.kc_t);
    P->vc_t = rel(S.vc_t);
    P->part_t = rel(S.part_t);
    P->o_t = rel(S.o_t);
    P->a_t = rel(S.a_t);
    if (S.nuc_hist) {
      P->nuc_hist = rel(S.nuc_hist);
      P->nuc_btot = rel(S.nuc_btot);
      P->nuc_cand = rel(S.nuc_cand);
      P->nuc_zmax = rel(S.nuc_zmax);
    }
    P->progress = reinterpret_cast<unsigned *>(base + prog);
    P->err = reinterpret_cast<unsigned *>(base + errw);
    P->lm_val = reinterpret_cast<float *>(base + lmv);
    P->lm_idx = reinterpret_cast<int *>(base + lmi);
    P->tok_slot = reinterpret_cast<int *>(base + tok);
  }
  return off;
}

}  // namespace

extern "C" {

const char *lf_last_error(const lf_state *st) { return st ? st->err.c_str() : g_err.c_str(); }

void lf_model_destroy(lf_state *st) {
  if (!st) return;
  for (void *p : st->allocs) (void)hipFree(p);
  delete st;
}

int lf_model_create(const lf_config *config, const lf_weights *w, void *stream, lf_state **out) {
  if (!out) return fail(nullptr, LF_EINVAL, "out is NULL");
  *out = nullptr;
  int rc = validate(config);
  if (rc) return rc;
  const lf_config &c = *config;
  const bool hidden = (c.flags & LF_HIDDEN_IO) != 0;
  if (!w || !w->layers) return fail(nullptr, LF_EINVAL, "weights are NULL");
  if (!hidden && (!w->tok_emb || !w->lm_head || !w->final_norm))
    return fail(nullptr, LF_EINVAL, "tok_emb, final_norm and lm_head are required");
  for (int l = 0; l < c.n_layers; ++l) {
    const lf_layer_weights &L = w->layers[l];
    if (!L.attn_norm || !L.wq || !L.wk || !L.wv || !L.wo || !L.ffn_norm || !L.w_gate || !L.w_up || !L.w_down)
      return fail(nullptr, LF_EINVAL, "a layer weight pointer is NULL");
  }

  lf_state *st = new lf_state();
  st->cfg = c;
  st->stream = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  auto bail = [&](int code) {
    g_err = st->err;
    lf_model_destroy(st);
    return code;
  };
  if ((e = hipGetDevice(&st->device)) != hipSuccess) return bail(hip_fail(st, e, "hipGetDevice"));
  // the device address of lf_generate_noalloc's static scratch on this device
  if ((e = lf::noalloc_scratch_init(st->device)) != hipSuccess)
    return bail(hip_fail(st, e, "hipGetSymbolAddress(scratch)"));
  int ncu = 0, coop = 0;
  (void)hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, st->device);
  (void)hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, st->device);
  if (!coop) return bail(fail(&st->err, LF_EHIP, "device does not support cooperative launch"));
  int G = ncu;
  if (const char *s = std::getenv("LF_GRID")) {
    int g = std::atoi(s);
    if (g >= 1 && g <= ncu) G = g;
  }

  lf::Params &P = st->P;
  const int d = c.d_model, Hq = c.n_heads, Hkv = c.n_kv_heads, dh = c.head_dim, F = c.ffn_dim;
  const int V = hidden ? 0 : c.vocab;
  P.L = c.n_layers; P.d = d; P.Hq = Hq; P.Hkv = Hkv; P.dh = dh; P.F = F; P.V = V;
  P.max_seq = c.max_seq; P.G = G; P.qpg = Hq / Hkv; P.nqkv = (Hq + 2 * Hkv) * dh;
  P.eps = c.rms_eps;
  P.inv_sqrt_dh = 1.0f / std::sqrt((float)dh);
  P.sampling = (hidden || !(c.temperature > 0.0f)) ? lf::SAMPLE_GREEDY
               : (c.flags & LF_GUMBEL)              ? lf::SAMPLE_GUMBEL
                                                    : lf::SAMPLE_NUCLEUS;
  P.inv_temp = P.sampling ? (float)(1.0 / (double)c.temperature) : 0.0f;
  P.top_p = c.top_p;
  P.seed = c.seed;
  P.flags = c.flags;
  P.hidden_io = hidden ? 1 : 0;
  P.window = c.sliding_window;
  P.attn_unit_tiles = lf::kWaves - 1;   // one tile per stream wave
  P.attn_split_tiles = 3;
  P.attn_qsplit = 1;
  // Stream waves 1-3 share their SIMDs with waves 5-7 and are served first
  // (measured: they finish a phase first, waves 5-7 last, wave 4, beside the
  // mostly idle sync wave, in between), so they take ~7% more pieces and
  // waves 5-7 ~7% fewer, within the round caps of wave_counts.
  {
    static const int kWaveW[lf::kNcwHost] = {274, 274, 274, 256, 238, 238, 238};
    for (int k = 0; k < lf::kNcwHost; ++k) P.wave_w[k] = kWaveW[k];
  }
  P.wave_w_kinds = 31;
  if (const char *s = std::getenv("LF_WAVE_W_KINDS")) P.wave_w_kinds = std::atoi(s) & 31;
  if (const char *s = std::getenv("LF_WAVE_W")) {   // seven ':'-separated weights, 64 .. 1024
    int v[lf::kNcwHost], n = 0;
    for (const char *p = s; *p && n < lf::kNcwHost;) {
      v[n++] = std::atoi(p);
      while (*p && *p != ':') ++p;
      if (*p == ':') ++p;
    }
    bool ok = n == lf::kNcwHost;
    for (int k = 0; k < n; ++k) ok = ok && v[k] >= 64 && v[k] <= 1024;
    if (ok)
      for (int k = 0; k < lf::kNcwHost; ++k) P.wave_w[k] = v[k];
  }
  if (const char *s = std::getenv("LF_ATTN_QSPLIT")) P.attn_qsplit = std::atoi(s) != 0 ? 1 : 0;
  // Workgroups without attention units hold back the output projection's first
  // ring round ~3.5 us (350 ticks of the 100 MHz clock), about one attention
  // pass at short contexts, so that the K/V loads meet a quieter memory system.
  P.o_refill_delay = 350;
  if (const char *s = std::getenv("LF_O_REFILL_DELAY_NS")) P.o_refill_delay = (unsigned)(std::atof(s) / 10.0);
  if (const char *s = std::getenv("LF_ATTN_UNIT_TILES")) {
    const int v = std::atoi(s);
    if (v >= 1 && v <= lf::kWaves - 1) P.attn_unit_tiles = v;
  }
  if (const char *s = std::getenv("LF_ATTN_SPLIT_TILES")) {
    const int v = std::atoi(s);
    if (v >= 1 && v <= lf::kWaves - 1) P.attn_split_tiles = v;
  }
  P.window_layers = c.sliding_window > 0 ? c.window_layers : 0ull;
  P.levels_per_token = lf::PH_PER_LAYER * c.n_layers + (hidden ? 0 : 2);
  double tmo_ms = 2000.0;
  if (const char *s = std::getenv("LF_TIMEOUT_MS")) tmo_ms = std::atof(s);
  P.timeout_ticks = (unsigned long long)(tmo_ms * 1e5);   // s_memrealtime runs at 100 MHz

  // ---- packed weights
  const size_t rowB_d = (size_t)d * 2;
  const size_t sz_qkv = align_up((size_t)P.nqkv * rowB_d, 256);
  const size_t sz_o = align_up((size_t)d * Hq * dh * 2, 256);
  const size_t sz_gu = align_up((size_t)2 * F * rowB_d, 256);
  const size_t sz_d = align_up((size_t)d * F * 2, 256);
  const size_t per_layer = sz_qkv + sz_o + sz_gu + sz_d;
  const size_t sz_head = hidden ? 0 : 2 * align_up((size_t)V * rowB_d, 256);
  char *wb = (char *)dev_alloc(st, per_layer * c.n_layers + sz_head, &e);
  if (!wb) return bail(fail(&st->err, LF_ENOMEM, "weight buffer allocation failed"));
  hipStream_t s = st->stream;
  const int half = dh / 2;
  for (int l = 0; l < c.n_layers; ++l) {
    const lf_layer_weights &L = w->layers[l];
    char *base = wb + per_layer * l;
    char *qkv = base, *wo = qkv + sz_qkv, *wgu = wo + sz_o, *wd = wgu + sz_gu;
    // q and k heads: packed row (h*dh + 2i) = source row (h*dh + i), (h*dh + 2i + 1) = (h*dh + i + dh/2)
    for (int part = 0; part < 2; ++part) {
      const char *src = (const char *)(part == 0 ? L.wq : L.wk);
      const int nh = part == 0 ? Hq : Hkv;
      char *dst0 = qkv + (part == 0 ? 0 : (size_t)Hq * dh * rowB_d);
      for (int h = 0; h < nh; ++h) {
        const char *sh = src + (size_t)h * dh * rowB_d;
        char *dsth = dst0 + (size_t)h * dh * rowB_d;
        if ((e = copy_rows_strided(dsth, 2 * rowB_d, sh, rowB_d, rowB_d, half, s)) != hipSuccess ||
            (e = copy_rows_strided(dsth + rowB_d, 2 * rowB_d, sh + (size_t)half * rowB_d, rowB_d, rowB_d, half,
                                   s)) != hipSuccess)
          return bail(hip_fail(st, e, "repack q/k rows"));
      }
    }
    if ((e = hipMemcpyAsync(qkv + (size_t)(Hq + Hkv) * dh * rowB_d, L.wv, (size_t)Hkv * dh * rowB_d,
                            hipMemcpyDeviceToDevice, s)) != hipSuccess)
      return bail(hip_fail(st, e, "copy v rows"));
    if ((e = hipMemcpyAsync(wo, L.wo, (size_t)d * Hq * dh * 2, hipMemcpyDeviceToDevice, s)) != hipSuccess)
      return bail(hip_fail(st, e, "copy wo"));
    if ((e = copy_rows_strided(wgu, 2 * rowB_d, L.w_gate, rowB_d, rowB_d, F, s)) != hipSuccess ||
        (e = copy_rows_strided(wgu + rowB_d, 2 * rowB_d, L.w_up, rowB_d, rowB_d, F, s)) != hipSuccess)
      return bail(hip_fail(st, e, "interleave gate/up rows"));
    if ((e = hipMemcpyAsync(wd, L.w_down, (size_t)d * F * 2, hipMemcpyDeviceToDevice, s)) != hipSuccess)
      return bail(hip_fail(st, e, "copy w_down"));
    // RMSNorm is g * x / rms(x) and the projection after it is linear, so the
    // gains are folded into the projection's columns here and the kernel
    // scales the row sums by 1 / rms.
    if ((e = lf::launch_scale_columns(qkv, (size_t)P.nqkv, d, L.attn_norm, s)) != hipSuccess ||
        (e = lf::launch_scale_columns(wgu, (size_t)2 * F, d, L.ffn_norm, s)) != hipSuccess)
      return bail(hip_fail(st, e, "fold norm gains"));
  }
  if (!hidden) {
    char *base = wb + per_layer * c.n_layers;
    char *lm = base, *emb = lm + align_up((size_t)V * rowB_d, 256);
    if ((e = hipMemcpyAsync(lm, w->lm_head, (size_t)V * rowB_d, hipMemcpyDeviceToDevice, s)) != hipSuccess ||
        (e = hipMemcpyAsync(emb, w->tok_emb, (size_t)V * rowB_d, hipMemcpyDeviceToDevice, s)) != hipSuccess ||
        (e = lf::launch_scale_columns(lm, (size_t)V, d, w->final_norm, s)) != hipSuccess)
      return bail(hip_fail(st, e, "copy embedding / lm_head"));
    P.lm_head = lm;
    P.tok_emb = emb;
  }
  P.wbase = wb;
  P.layer_stride = per_layer;
  P.part_off[lf::LW_QKV] = 0;
  P.part_off[lf::LW_O] = sz_qkv;
  P.part_off[lf::LW_GU] = sz_qkv + sz_o;
  P.part_off[lf::LW_D] = sz_qkv + sz_o + sz_gu;

  // ---- KV cache, rotary table, activations, sync words
  P.kv_tiles = (c.max_seq + lf::kKvTile - 1) / lf::kKvTile;
  const size_t kv_elems = (size_t)c.n_layers * Hkv * P.kv_tiles * lf::kKvTile * dh;
  P.kcache = dev_alloc(st, kv_elems * 2, &e);
  P.vcache = P.kcache ? dev_alloc(st, kv_elems * 2, &e) : nullptr;
  if (!P.vcache) return bail(fail(&st->err, LF_ENOMEM, "KV cache allocation failed"));
  (void)hipMemsetAsync(P.kcache, 0, kv_elems * 2, s);
  (void)hipMemsetAsync(P.vcache, 0, kv_elems * 2, s);

  std::vector<float> rope((size_t)c.max_seq * half * 2);
  for (int p = 0; p < c.max_seq; ++p)
    for (int i = 0; i < half; ++i) {
      const double theta = std::pow((double)c.rope_base, -2.0 * (double)i / (double)dh);
      const double phi = (double)p * theta;
      rope[((size_t)p * half + i) * 2 + 0] = (float)std::cos(phi);
      rope[((size_t)p * half + i) * 2 + 1] = (float)std::sin(phi);
    }
  float *drope = (float *)dev_alloc(st, rope.size() * 4, &e);
  if (!drope) return bail(fail(&st->err, LF_ENOMEM, "rotary table allocation failed"));
  if ((e = hipMemcpy(drope, rope.data(), rope.size() * 4, hipMemcpyHostToDevice)) != hipSuccess)
    return bail(hip_fail(st, e, "upload rotary table"));
  P.rope = drope;

  int smax = G / Hkv;
  if (smax > lf::kMaxSplit) smax = lf::kMaxSplit;
  if (smax < 1) smax = 1;
  const size_t part_gen = (size_t)Hkv * smax * P.qpg * (dh + 2);
  // small buffers, each 256-byte aligned, in one arena
  struct Slot { void **dst; size_t bytes; };
  void *x_hidden, *x_out, *logits, *lm_val, *lm_idx, *progress, *tok_slot, *errw, *stats;
  Slot slots[] = {
      {&x_hidden, (size_t)d * 4}, {&x_out, (size_t)d * 4}, {&logits, (size_t)(V > 0 ? V : 1) * 4},
      {&lm_val, (size_t)G * 4}, {&lm_idx, (size_t)G * 4}, {&progress, (size_t)G * 4},
      {&tok_slot, 16}, {&errw, 16},
      {&stats, (size_t)G * (lf::kStatWords + (lf::kTrace ? lf::kTraceSlots * (5 * c.n_layers + 2) : 0)) * 8}};
  size_t arena = 0;
  for (auto &sl : slots) arena += align_up(sl.bytes, 256);
  char *ar = (char *)dev_alloc(st, arena, &e);
  if (!ar) return bail(fail(&st->err, LF_ENOMEM, "activation arena allocation failed"));
  (void)hipMemsetAsync(ar, 0, arena, s);
  size_t off = 0;
  for (auto &sl : slots) { *sl.dst = ar + off; off += align_up(sl.bytes, 256); }
  P.x_hidden = (float *)x_hidden; P.x_out = (float *)x_out; P.logits = (float *)logits;
  P.lm_val = (float *)lm_val; P.lm_idx = (int *)lm_idx; P.progress = (unsigned *)progress;
  P.tok_slot = (int *)tok_slot; P.err = (unsigned *)errw;
  P.stats = (unsigned long long *)stats;
  P.stat_stride = lf::kStatWords + (lf::kTrace ? lf::kTraceSlots * (5 * c.n_layers + 2) : 0);
  // tagged exchange words, two generations each, in one zeroed allocation
  {
    struct TSlot { unsigned long long **dst; size_t words; };
    TSlot ts[] = {{&P.xmid_t, (size_t)d}, {&P.xout_t, (size_t)d}, {&P.q_t, (size_t)Hq * dh},
                  {&P.kc_t, (size_t)Hkv * dh / 2}, {&P.vc_t, (size_t)Hkv * dh / 2}, {&P.part_t, part_gen},
                  {&P.o_t, (size_t)Hq * dh / 2}, {&P.a_t, (size_t)F / 2}};
    // each buffer: two generations, then one staging round of padding (staging
    // reads whole rounds; the words past a vector's end are ignored)
    const size_t pad_words = lf::kStageRound > lf::kStageRoundWide ? lf::kStageRound : lf::kStageRoundWide;
    size_t bytes = 0;
    for (auto &t : ts) bytes += align_up((2 * t.words + pad_words) * 8, 256);
    // the nucleus draw over the grid: one generation each (its levels order every
    // reader of one token before any writer of the next)
    const bool nuc = P.sampling == lf::SAMPLE_NUCLEUS && !hidden;
    P.nuc_cmax = 2 * ((V / 2 + G - 1) / G);
    TSlot tn[] = {{&P.nuc_hist, (size_t)lf::kSampBins * G * 2}, {&P.nuc_btot, (size_t)lf::kSampBins * 2},
                  {&P.nuc_cand, (size_t)G * (3 + (size_t)P.nuc_cmax / 2)}, {&P.nuc_zmax, (size_t)G}};
    if (nuc)
      for (auto &t : tn) bytes += align_up(t.words * 8, 256);
    char *xb = (char *)dev_alloc(st, bytes, &e);
    if (!xb) return bail(fail(&st->err, LF_ENOMEM, "exchange buffer allocation failed"));
    (void)hipMemsetAsync(xb, 0, bytes, s);
    size_t o2 = 0;
    for (auto &t : ts) { *t.dst = (unsigned long long *)(xb + o2); o2 += align_up((2 * t.words + pad_words) * 8, 256); }
    for (auto &t : tn) {
      if (!nuc) { *t.dst = nullptr; continue; }
      *t.dst = (unsigned long long *)(xb + o2);
      o2 += align_up(t.words * 8, 256);
    }
    // (workgroup 0's list bookkeeping holds at most kSampBins workgroups; rows
    // are listed as 16-bit offsets within a workgroup's block)
    P.nuc_grid = nuc && G <= lf::kSampBins && P.nuc_cmax <= 65536 &&
                 !(std::getenv("LF_NUC_WG0") && std::atoi(std::getenv("LF_NUC_WG0")) != 0) ? 1 : 0;
    P.part_gen = part_gen;
    st->xbuf = xb;
    st->xbuf_bytes = bytes;
  }
  st->out_cap = 1;
  P.out_tokens = (int *)dev_alloc(st, sizeof(int) * 1, &e);
  st->in_cap = 1;
  P.in_tokens = (const int *)dev_alloc(st, sizeof(int) * 1, &e);
  if (!P.out_tokens || !P.in_tokens) return bail(fail(&st->err, LF_ENOMEM, "token buffer allocation failed"));

  // ---- LDS layout: [h | part] (also attention / sampler scratch), red, ctl, rings
  int rows_max = 0, rows_k[5];
  {
    const int units[5] = {P.nqkv / 2, d, F / 2, d / 2, hidden ? 0 : V / 2};
    const int upr[5] = {2, 1, 4, 2, 2};   // rows per partition unit (as in the kernel)
    // with the K/V tile prefetch, up to a quarter of the grid runs attention
    // only and the QKV rows go to the other workgroups
    const char *kvpf = std::getenv("LF_KV_PF");
    const bool kvpf_asked = kvpf && std::atoll(kvpf) > 0;
    for (int k = 0; k < 5; ++k) {
      const int g = k == 1 ? G - lf::o_rows_skip_max(G, Hkv, P.qpg, P.attn_qsplit)   // the output projection's workgroups
                           : (k == 0 && kvpf_asked ? G - G / 4 : G);
      const int r = upr[k] * ((units[k] + g - 1) / g);
      rows_k[k] = r;
      rows_max = r > rows_max ? r : rows_max;
    }
  }
  int hmax = d;
  if (Hq * dh > hmax) hmax = Hq * dh;
  if (F > hmax) hmax = F;
  // a staged vector of fp16 pairs is written in whole staging rounds of 32-bit words
  const auto round_up = [](size_t w, size_t r) { return (w + r - 1) / r * r; };
  const size_t o_words = round_up((size_t)Hq * dh / 2, lf::kStageRound);
  const size_t a_words = round_up((size_t)F / 2, lf::kStageRoundWide);   // the SwiGLU vector's wider rounds
  const size_t round_up_words = o_words > a_words ? o_words : a_words;
  size_t h_b = align_up((size_t)hmax * 2 + 1024, 16);   // + one piece of slack for masked lanes
  if (round_up_words * 4 > h_b) h_b = align_up(round_up_words * 4, 16);
  // an RMSNorm input is written as fp16 elements in whole rounds of words
  const size_t d_elems = round_up((size_t)d, lf::kStageRound);
  if (d_elems * 2 > h_b) h_b = align_up(d_elems * 2, 16);
  // partial row sums [row][8] per phase kind, each kind's area sized for its own rows
  size_t part_floats = 0;
  for (int k = 0; k < 5; ++k) {
    P.psum_off[k] = (int)part_floats;
    part_floats += align_up((size_t)rows_k[k] * 8, 4);
  }
  const size_t part_b = align_up(part_floats * 4, 16);
  // attention scratch: queries, current K/V row, per-wave (m, l) and per-wave o
  const size_t attn_b = (size_t)lf::attn_lds(P.qpg, dh).bytes;
  // the nucleus draw's scratch overlays the staged input and the attention area
  const size_t samp_b = P.sampling == lf::SAMPLE_NUCLEUS ? (size_t)lf::kSampBytes : 0;
  // h, then the attention area; the sampler scratch (after the last layer) overlays both
  size_t region_a = align_up(h_b, 256);
  if (samp_b > region_a + attn_b) region_a = align_up(samp_b - attn_b, 256);
  P.lds_h = 0;
  P.lds_attn = (int)region_a;
  P.lds_red = (int)align_up((size_t)P.lds_attn + attn_b, 256);
  P.lds_ctl = P.lds_red + 256;
  P.lds_xown = P.lds_ctl + lf::kCtlBytes;
  P.lds_xres = (int)align_up((size_t)P.lds_xown + (size_t)rows_max * 4, 16);
  P.lds_part = (int)align_up((size_t)P.lds_xres + (size_t)rows_max * 4, 256);   // per kind: [rows][8]
  P.lds_trace = (int)align_up((size_t)P.lds_part + part_b, 256);
  size_t lds_end = align_up((size_t)P.lds_trace + (lf::kTrace ? (size_t)lf::kTraceSlots * (5 * c.n_layers + 2) * 8 : 0), 256);
  P.psum_total = (int)part_floats;
  P.hmax = hmax;
  int lds_limit = 0;
  (void)hipDeviceGetAttribute(&lds_limit, hipDeviceAttributeMaxSharedMemoryPerBlock, st->device);
  if (lds_limit <= 0) lds_limit = 65536;
  if ((long long)lds_end > lds_limit)
    return bail(fail(&st->err, LF_EUNSUPPORTED, "shape needs more LDS than a workgroup can hold"));
  // The LDS left over can hold the first K/V tile of up to seven stream waves
  // of an attention unit (LF_KV_PF: how many), then the projection prefetch
  // below.  The tile prefetch is off by default: measured end to end, the
  // attention that ends ~0.5 us sooner does not move the layer's end (the next
  // exchange absorbs it) while the other workgroups stream more QKV rows.
  {
    const int nvh = (dh + 63) / 64;
    P.kv_pf_tile = (dh / 8 + 8 * nvh) * 1024;
    long long fit = ((long long)lds_limit - (long long)lds_end) / P.kv_pf_tile;
    long long want = 0;
    if (const char *s = std::getenv("LF_KV_PF")) want = std::atoll(s);
    if (want < 0 || P.qpg > 4) want = 0;   // the unit variant for more query heads reads no prefetch
    P.kv_pf = (int)(want < fit ? want : fit);
    if (P.kv_pf > 0) P.attn_qsplit = 0;   // the tile prefetch maps units to KV heads directly
    P.lds_kvpf = (int)lds_end;
    lds_end += (size_t)P.kv_pf * P.kv_pf_tile;
  }
  // The LDS left over can hold the first pieces of each stream wave's share of
  // one projection, loaded while attention runs.  By default that is the output
  // projection, where a wave's share (at the largest weight) is more than one
  // ring round and the pieces that fit take a whole round off the phase (all of
  // it fitting, the ring's refill after attention starts on gate/up).  Where
  // the share fits the ring (one round) it is off: measured, 4 pieces on the
  // 2.2B decode cost 2.8%.  LF_GU_PF (pieces per wave) with LF_PF_KIND (2 gate/up, the
  // default then; 1 output projection) overrides the rule.  A gate/up
  // prefetch costs more than it saves (its burst delays the output
  // projection's input).
  {
    const long long per_piece = (long long)lf::kNcwHost * 1024;
    long long fit = ((long long)lds_limit - (long long)lds_end) / per_piece;
    long long want = 0;
    if (const char *s = std::getenv("LF_GU_PF")) {
      want = std::atoll(s);
      P.pf_kind = 2;
      if (const char *k = std::getenv("LF_PF_KIND")) P.pf_kind = std::atoi(k) == 1 ? 1 : 2;
    } else {
      const int og = G - lf::o_rows_skip_max(G, Hkv, P.qpg, P.attn_qsplit);
      const long long o_pieces = (long long)((d + og - 1) / og) * ((Hq * dh + 511) / 512);
      int wmax = 0, wsum = 0;
      for (int k = 0; k < lf::kNcwHost; ++k) {
        wmax = P.wave_w[k] > wmax ? P.wave_w[k] : wmax;
        wsum += P.wave_w[k];
      }
      // a wave's pieces: its weighted share, capped (as the kernel splits them)
      // at the whole rounds of an equal share, plus one round from 8 rounds on
      const long long eq = (o_pieces + lf::kNcwHost - 1) / lf::kNcwHost;
      const long long r = (eq + lf::kRingSlots - 1) / lf::kRingSlots;
      const long long cap = lf::kRingSlots * (r + (r >= 8 ? 1 : 0));
      long long share = (o_pieces * wmax + wsum - 1) / wsum;
      if (share > cap) share = cap;
      // on where it takes a whole round off the phase (ring rounds left after
      // the pieces that fit)
      const long long rounds = (share + lf::kRingSlots - 1) / lf::kRingSlots;
      const long long left = share > fit ? share - fit : 0;
      P.pf_kind = 1;
      if (eq > lf::kRingSlots && (left + lf::kRingSlots - 1) / lf::kRingSlots < rounds) want = fit;
    }
    if (want < 0) want = 0;
    P.pf_n = (int)(want < fit ? want : fit);
    P.lds_pf = (int)lds_end;
  }
  P.lds_bytes = (int)(lds_end + (size_t)P.pf_n * lf::kNcwHost * 1024);
  P.plain_launch = (std::getenv("LF_PLAIN_LAUNCH") && std::atoi(std::getenv("LF_PLAIN_LAUNCH")) != 0) ? 1 : 0;
  for (int pf = 0; pf < 2; ++pf) {
    if ((e = hipFuncSetAttribute(lf::monokernel_symbol(pf != 0, P.qpg), hipFuncAttributeMaxDynamicSharedMemorySize,
                                 P.lds_bytes)) != hipSuccess)
      return bail(hip_fail(st, e, "set dynamic LDS size"));
    int nblk = 0;
    if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nblk, lf::monokernel_symbol(pf != 0, P.qpg), lf::kThreads,
                                                          P.lds_bytes)) != hipSuccess)
      return bail(hip_fail(st, e, "occupancy query"));
    if (nblk < 1) return bail(fail(&st->err, LF_EHIP, "the kernel cannot be resident on a compute unit"));
  }
  if ((e = hipStreamSynchronize(s)) != hipSuccess) return bail(hip_fail(st, e, "create"));
  *out = st;
  g_err.clear();
  return LF_OK;
}

int lf_set_position(lf_state *st, int32_t token, int32_t pos) {
  if (!st) return fail(nullptr, LF_EINVAL, "state is NULL");
  if (pos < 0 || pos >= st->cfg.max_seq) return fail(&st->err, LF_ERANGE, "pos outside [0, max_seq)");
  if (!st->P.hidden_io && (token < 0 || token >= st->cfg.vocab))
    return fail(&st->err, LF_ERANGE, "token outside [0, vocab)");
  st->pending_token = token;
  st->pending_pos = pos;
  st->has_pending = true;
  return LF_OK;
}

int lf_decode_step(lf_state *st, int32_t token, int32_t pos, int32_t *next_token) {
  if (!st) return fail(nullptr, LF_EINVAL, "state is NULL");
  if (pos < 0 || pos >= st->cfg.max_seq) return fail(&st->err, LF_ERANGE, "pos outside [0, max_seq)");
  if (st->P.hidden_io) {
    int rc = do_launch(st, 0, pos, 1, nullptr);
    if (rc) return rc;
    if (next_token) *next_token = -1;
    return LF_OK;
  }
  if (token < 0 || token >= st->cfg.vocab) return fail(&st->err, LF_ERANGE, "token outside [0, vocab)");
  std::vector<int> out;
  int rc = do_launch(st, token, pos, 1, &out);
  if (rc) return rc;
  if (next_token) *next_token = out[0];
  if (pos + 1 < st->cfg.max_seq) {
    st->pending_token = out[0];
    st->pending_pos = pos + 1;
    st->has_pending = true;
  } else {
    st->has_pending = false;
  }
  return LF_OK;
}

int lf_generate(lf_state *st, int32_t n, int32_t *out_tokens) {
  if (!st) return fail(nullptr, LF_EINVAL, "state is NULL");
  if (st->P.hidden_io) return fail(&st->err, LF_EINVAL, "lf_generate needs a vocabulary");
  if (!out_tokens) return fail(&st->err, LF_EINVAL, "out_tokens is NULL");
  if (!st->has_pending) return fail(&st->err, LF_ERANGE, "no pending token: call lf_decode_step or lf_set_position");
  if (n < 1 || st->pending_pos + n > st->cfg.max_seq)
    return fail(&st->err, LF_ERANGE, "n < 1 or pos + n > max_seq");
  if (n > st->out_cap) {
    hipError_t e;
    int *p = (int *)dev_alloc(st, sizeof(int) * n, &e);
    if (!p) return fail(&st->err, LF_ENOMEM, "token buffer allocation failed");
    st->P.out_tokens = p;
    st->out_cap = n;
  }
  std::vector<int> out;
  int rc = do_launch(st, st->pending_token, st->pending_pos, n, &out);
  if (rc) return rc;
  std::memcpy(out_tokens, out.data(), sizeof(int) * n);
  st->pending_pos += n;
  st->pending_token = out[n - 1];
  st->has_pending = st->pending_pos < st->cfg.max_seq;
  return LF_OK;
}

int lf_generate_noalloc(lf_state *st, int32_t n, int32_t *out_tokens_dev) {
  if (!st) return fail(nullptr, LF_EINVAL, "state is NULL");
  if (st->P.hidden_io) return fail(&st->err, LF_EINVAL, "lf_generate_noalloc needs a vocabulary");
  if (!out_tokens_dev) return fail(&st->err, LF_EINVAL, "out_tokens_dev is NULL");
  if (!st->has_pending) return fail(&st->err, LF_ERANGE, "no pending token: call lf_decode_step or lf_set_position");
  if (n < 1 || st->pending_pos + n > st->cfg.max_seq)
    return fail(&st->err, LF_ERANGE, "n < 1 or pos + n > max_seq");
  char *base = static_cast<char *>(lf::noalloc_scratch(st->device));
  if (!base) return fail(&st->err, LF_EHIP, "the static scratch of this device was never looked up");
  const size_t need = noalloc_layout(st, nullptr, nullptr);
  if (need > lf::kNoallocScratchBytes) {
    char buf[200];
    std::snprintf(buf, sizeof buf, "this state needs %zu bytes of launch scratch; the static array holds %zu",
                  need, lf::kNoallocScratchBytes);
    return fail(&st->err, LF_EUNSUPPORTED, buf);
  }
  lf::Params P = st->P;
  noalloc_layout(st, base, &P);
  P.out_tokens = out_tokens_dev;
  P.levels_per_token = lf::PH_PER_LAYER * P.L + 2 + (P.nuc_grid ? lf::kNucLevels : 0);
  P.n_tokens = n;
  P.trace_token = n / 2;
  P.token0 = st->pending_token;
  P.pos0 = st->pending_pos;
  P.level_base = 0;   // the words are cleared below: the numbering restarts at every call
  hipError_t e;
  // a fill kernel (not a memset node, so the sequence may be captured in a graph)
  if ((e = lf::launch_zero(base, need, st->stream)) != hipSuccess) return hip_fail(st, e, "clear scratch");
  if ((e = lf::launch_monokernel(P, false, st->stream)) != hipSuccess) return hip_fail(st, e, "cooperative launch");
  if ((e = hipStreamSynchronize(st->stream)) != hipSuccess) return hip_fail(st, e, "kernel execution");
  unsigned herr[4];
  if ((e = hipMemcpy(herr, P.err, sizeof(herr), hipMemcpyDeviceToHost)) != hipSuccess)
    return hip_fail(st, e, "read error word");
  if (herr[0]) {
    char buf[160];
    std::snprintf(buf, sizeof buf, "in-kernel wait timed out (workgroup %u, level %u)", herr[1], herr[2]);
    return fail(&st->err, LF_ETIMEOUT, buf);
  }
  if (herr[3]) return fail(&st->err, LF_EHIP, "the token choice produced no valid token (non-finite logits?)");
  int last = 0;
  if ((e = hipMemcpy(&last, out_tokens_dev + (n - 1), sizeof(int), hipMemcpyDeviceToHost)) != hipSuccess)
    return hip_fail(st, e, "read last token");
  st->pending_pos += n;
  st->pending_token = last;
  st->has_pending = st->pending_pos < st->cfg.max_seq;
  return LF_OK;
}

int lf_prefill(lf_state *st, const int32_t *tokens, int32_t n, int32_t pos0) {
  if (!st) return fail(nullptr, LF_EINVAL, "state is NULL");
  if (st->P.hidden_io) return fail(&st->err, LF_EINVAL, "lf_prefill needs a vocabulary");
  if (!tokens && n > 0) return fail(&st->err, LF_EINVAL, "tokens is NULL");
  if (n < 0 || pos0 < 0 || pos0 + n > st->cfg.max_seq)
    return fail(&st->err, LF_ERANGE, "n < 0 or positions outside [0, max_seq)");
  for (int i = 0; i < n; ++i)
    if (tokens[i] < 0 || tokens[i] >= st->cfg.vocab) return fail(&st->err, LF_ERANGE, "token outside [0, vocab)");
  if (n == 0) return LF_OK;
  hipError_t e;
  if (n > st->in_cap) {
    int *p = (int *)dev_alloc(st, sizeof(int) * n, &e);
    if (!p) return fail(&st->err, LF_ENOMEM, "token buffer allocation failed");
    st->P.in_tokens = p;
    st->in_cap = n;
  }
  if ((e = hipMemcpy(const_cast<int *>(st->P.in_tokens), tokens, sizeof(int) * n, hipMemcpyHostToDevice)) !=
      hipSuccess)
    return hip_fail(st, e, "upload prompt tokens");
  int rc = do_launch(st, tokens[0], pos0, n, nullptr, true);
  if (rc) return rc;
  st->has_pending = false;
  return LF_OK;
}

int lf_get_logits(lf_state *st, float *dst, int dst_is_device) {
  if (!st || !dst) return fail(st ? &st->err : nullptr, LF_EINVAL, "NULL argument");
  if (st->P.hidden_io) return fail(&st->err, LF_EINVAL, "no logits with LF_HIDDEN_IO");
  hipError_t e = hipMemcpy(dst, st->P.logits, sizeof(float) * st->P.V,
                           dst_is_device ? hipMemcpyDeviceToDevice : hipMemcpyDeviceToHost);
  return e == hipSuccess ? LF_OK : hip_fail(st, e, "copy logits");
}

static int kv_copy(lf_state *st, int32_t layer, int32_t pos0, int32_t n, void *k, void *v, bool fill) {
  if (!st || !k || !v) return fail(st ? &st->err : nullptr, LF_EINVAL, "NULL argument");
  if (layer < 0 || layer >= st->cfg.n_layers || pos0 < 0 || n < 0 || pos0 + n > st->cfg.max_seq)
    return fail(&st->err, LF_ERANGE, "layer / position range outside the cache");
  hipError_t e = lf::launch_kv_copy(st->P, layer, pos0, n, k, v, fill, st->stream);
  if (e != hipSuccess) return hip_fail(st, e, fill ? "kv fill" : "kv read");
  e = hipStreamSynchronize(st->stream);
  return e == hipSuccess ? LF_OK : hip_fail(st, e, "kv copy");
}

int lf_kv_fill(lf_state *st, int32_t layer, int32_t pos0, int32_t n, const void *k, const void *v) {
  return kv_copy(st, layer, pos0, n, const_cast<void *>(k), const_cast<void *>(v), true);
}

int lf_kv_read(lf_state *st, int32_t layer, int32_t pos0, int32_t n, void *k, void *v) {
  return kv_copy(st, layer, pos0, n, k, v, false);
}

int lf_set_hidden(lf_state *st, const float *x) {
  if (!st || !x) return fail(st ? &st->err : nullptr, LF_EINVAL, "NULL argument");
  if (!st->P.hidden_io) return fail(&st->err, LF_EINVAL, "state was not created with LF_HIDDEN_IO");
  hipError_t e = hipMemcpy(st->P.x_hidden, x, sizeof(float) * st->P.d, hipMemcpyDeviceToDevice);
  return e == hipSuccess ? LF_OK : hip_fail(st, e, "set hidden");
}

int lf_get_hidden(lf_state *st, float *x) {
  if (!st || !x) return fail(st ? &st->err : nullptr, LF_EINVAL, "NULL argument");
  if (!st->P.hidden_io) return fail(&st->err, LF_EINVAL, "state was not created with LF_HIDDEN_IO");
  hipError_t e = hipMemcpy(x, st->P.x_out, sizeof(float) * st->P.d, hipMemcpyDeviceToDevice);
  return e == hipSuccess ? LF_OK : hip_fail(st, e, "get hidden");
}

int lf_get_stats(lf_state *st, void *dst, size_t bytes) {
  if (!st || !dst) return fail(st ? &st->err : nullptr, LF_EINVAL, "NULL argument");
  size_t need = (size_t)st->P.G * lf::kStatWords * 8;
  if (lf::kTrace && bytes >= (size_t)st->P.G * st->P.stat_stride * 8) need = (size_t)st->P.G * st->P.stat_stride * 8;
  if (bytes < need) return fail(&st->err, LF_EINVAL, "stats buffer too small");
  hipError_t e = hipMemcpy(dst, st->P.stats, need, hipMemcpyDeviceToHost);
  return e == hipSuccess ? LF_OK : hip_fail(st, e, "copy stats");
}

int lf_query(const lf_state *st, int32_t what) {
  if (!st) return LF_EINVAL;
  switch (what) {
    case LF_Q_GRID: return st->P.G;
    case LF_Q_THREADS: return lf::kThreads;
    case LF_Q_LDS_BYTES: return st->P.lds_bytes;
    case LF_Q_SCRATCH_BYTES: return (int)noalloc_layout(st, nullptr, nullptr);
    case LF_Q_SCRATCH_MAX: return (int)lf::kNoallocScratchBytes;
    case LF_Q_KV_PF: return st->P.kv_pf;
    case LF_Q_GU_PF: return st->P.pf_n;
    case LF_Q_WAVE_W_KINDS: return st->P.wave_w_kinds;
    case LF_Q_PF_KIND: return st->P.pf_kind;
    default:
      if (what >= LF_Q_WAVE_W && what < LF_Q_WAVE_W + lf::kNcwHost) return st->P.wave_w[what - LF_Q_WAVE_W];
      return LF_EINVAL;
  }
}

int lf_test_expdef(const float *x, float *y, int64_t n, void *stream) {
  if ((!x || !y) && n > 0) return fail(nullptr, LF_EINVAL, "NULL argument");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = lf::launch_test_expdef(x, y, n, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  return e == hipSuccess ? LF_OK : hip_fail(nullptr, e, "lf_test_expdef");
}

int lf_test_logdef(const float *x, float *y, int64_t n, void *stream) {
  if ((!x || !y) && n > 0) return fail(nullptr, LF_EINVAL, "NULL argument");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = lf::launch_test_logdef(x, y, n, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  return e == hipSuccess ? LF_OK : hip_fail(nullptr, e, "lf_test_logdef");
}

int lf_test_sample_gumbel(const float *logits, int32_t n, float temperature, uint64_t seed, const int32_t *pos,
                          int32_t m, int32_t *tokens, void *stream) {
  if (!logits || !pos || !tokens || n < 1 || m < 0) return fail(nullptr, LF_EINVAL, "bad argument");
  if (!(temperature > 0.0f)) return fail(nullptr, LF_EINVAL, "temperature must be > 0");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const float inv_temp = (float)(1.0 / (double)temperature);
  hipError_t e = lf::launch_test_gumbel(logits, n, inv_temp, seed, pos, m, tokens, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  return e == hipSuccess ? LF_OK : hip_fail(nullptr, e, "lf_test_sample_gumbel");
}

int lf_test_sample(const float *logits, int32_t n, float temperature, float top_p, uint64_t seed,
                   const int32_t *pos, int32_t m, int32_t *tokens, void *stream) {
  if (!logits || !pos || !tokens || n < 1 || m < 0) return fail(nullptr, LF_EINVAL, "bad argument");
  if (!(temperature > 0.0f) || !(top_p > 0.0f)) return fail(nullptr, LF_EINVAL, "temperature and top_p must be > 0");
  if (n > lf::kSampMaxVocab) return fail(nullptr, LF_EUNSUPPORTED, "nucleus sampling supports up to 393216 logits");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const float inv_temp = (float)(1.0 / (double)temperature);
  hipError_t e = lf::launch_test_sample(logits, n, inv_temp, top_p, seed, pos, m, tokens, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  return e == hipSuccess ? LF_OK : hip_fail(nullptr, e, "lf_test_sample");
}

}  // extern "C"

// lf_internal.h -- parameter block shared by the host planner (lf_api.cpp) and
// the persistent kernel (lf_kernel.hip).  Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lf {

constexpr int kThreads = 512;          // 8 wave64s per workgroup
constexpr int kWaves = kThreads / 64;
constexpr int kNcwHost = kWaves - 1;   // stream waves per workgroup
constexpr int kMaxSplit = 64;          // most split-K chunks per KV head
// The KV cache of one (layer, KV head) is a run of tiles of kKvTile positions,
// each 128 * head_dim bytes for K and for V:
//   K tile [head_dim / 8][64 keys][8 dims]: one 16-byte vector is 8 dims of one
//     key, and a 1-KB piece is the same 8 dims of all 64 keys, so a wave64 load
//     puts one key in each lane;
//   V tile [8 key groups][head_dim][8 keys]: one 16-byte vector is one dim of 8
//     consecutive keys, and a 1-KB piece is 64 dims of one key group, so a wave64
//     load puts one dim in each lane.
// Both make every load of a tile a contiguous 1-KB piece.
constexpr int kKvTile = 64;
// Element (position j, dim e) of a K / V tile run, in fp16 elements from its start.
__host__ __device__ constexpr size_t k_elem(int dh, int j, int e) {
  return (size_t)(j >> 6) * (size_t)(64 * dh) + (size_t)((e >> 3) * 512 + (j & 63) * 8 + (e & 7));
}
__host__ __device__ constexpr size_t v_elem(int dh, int j, int e) {
  return (size_t)(j >> 6) * (size_t)(64 * dh) + (size_t)(((j & 63) >> 3) * dh * 8 + e * 8 + (j & 7));
}
// Workgroups 0 .. n-1 merge the attention heads' split-K partials (unit c = 0
// of head g runs on workgroup g); they are the last to finish attention, so
// with enough workgroups they get no rows of the output projection.
__host__ __device__ constexpr int o_rows_skip(int G, int Hkv) { return G > 2 * Hkv ? Hkv : 0; }
// The most workgroups that may skip them: with short heads split by query heads
// (one unit per query head while 2 Hkv qpg <= G), every unit's workgroup.
__host__ __device__ constexpr int o_rows_skip_max(int G, int Hkv, int qpg, int qsplit) {
  return qsplit && qpg > 1 && 2 * Hkv * qpg <= G ? o_rows_skip(G, Hkv * qpg) : o_rows_skip(G, Hkv);
}
constexpr int kStatWords = 16;         // uint64 statistics per workgroup (LF_STATS)
// LF_TRACE builds also record, for one token, three timestamps per phase and
// workgroup: input staged, stream waves done, published.
#ifdef LF_TRACE
constexpr bool kTrace = true;
#else
constexpr bool kTrace = false;
#endif
#ifndef LF_RING_SLOTS
#define LF_RING_SLOTS 8
#endif
constexpr int kCtlBytes = 1024;           // LDS bytes of a workgroup's control block
constexpr int kTraceSlots = 16;          // timestamps per phase (LF_TRACE builds)
constexpr int kStageRound = 64 * 40;      // tagged words one staging round reads (buffers are padded to it)
constexpr int kStageRoundWide = 64 * 56;  // the SwiGLU vector's staging round
constexpr int kRingSlots = LF_RING_SLOTS;  // 1-KB pieces in flight per stream wave (register ring)
constexpr int kSampBins = 256;             // bins of z* - z in the nucleus draw
constexpr int kSampBytes = 60 * 1024;      // LDS of the nucleus draw (after the lm_head)
constexpr int kSampSegs = 6144;            // 64-index segments the nucleus draw's token search can hold
constexpr int kSampMaxVocab = kSampSegs * 64;

// Attention scratch in LDS (an area of its own, so the sync wave may stage the
// next phase's input while the stream waves run attention): fp16 queries [qpg][dh], fp32 current K and V rows [dh] each, fp16
// softmax weights [kWaves][8][64], per-wave (m, l) [kWaves][8][2] and per-wave
// o [kWaves][qpg][dh].  Byte offsets.
struct AttnLds {
  int q16, kcur, vcur, p16, wml, wo, bytes;
};
__host__ __device__ inline AttnLds attn_lds(int qpg, int dh) {
  AttnLds a{};
  a.q16 = 0;
  a.kcur = (qpg * dh * 2 + 15) & ~15;
  a.vcur = a.kcur + dh * 4;
  a.p16 = (a.vcur + dh * 4 + 15) & ~15;
  a.wml = a.p16 + kWaves * 8 * kKvTile * 2;
  a.wo = a.wml + kWaves * 8 * 2 * 4;
  a.bytes = a.wo + kWaves * qpg * dh * 4;
  return a;
}

// Phases of one layer; each completes one "level" of the dependency chain.
enum Phase { PH_QKV = 1, PH_ATTN = 2, PH_O = 3, PH_GU = 4, PH_D = 5, PH_PER_LAYER = 5 };

// Offsets (bytes) of one layer's pieces inside the packed weight buffer; layer l
// starts at wbase + l * layer_stride.
enum LayerPart { LW_QKV = 0, LW_O, LW_GU, LW_D, LW_COUNT };

// Next-token choice: argmax, the nucleus draw (over the lm_head workgroups, or
// by workgroup 0 alone), or Gumbel-max (every lm_head workgroup publishes its
// best noised score, workgroup 0 reduces them).
enum SampleMode { SAMPLE_GREEDY = 0, SAMPLE_NUCLEUS = 1, SAMPLE_GUMBEL = 2 };
// Dependency levels the nucleus draw over the grid adds between the lm_head's
// level and the token's.
constexpr int kNucLevels = 3;

struct Params {
  // shape
  int L, d, Hq, Hkv, dh, F, V, max_seq, G, qpg, nqkv;
  float eps, inv_sqrt_dh, inv_temp, top_p;
  unsigned long long seed;
  unsigned flags;
  int hidden_io, sampling;   // sampling: a SampleMode
  int window;                          // sliding-window length (0: none)
  int attn_unit_tiles;                 // most KV tiles a KV head keeps in one unit (1 .. 7)
  int attn_split_tiles;                // tiles per unit once a head is split (1 .. 7)
  int attn_qsplit;                     // 1: a KV head in one unit is split by query heads (GQA)
  int pf_kind;                         // the projection whose first pieces the LDS prefetch takes (2 gate/up, 1 O)
  int wave_w[kNcwHost];                // relative shares of a workgroup's pieces per stream wave (1 .. 7)
  int wave_w_kinds;                    // bit k: phase kind k uses wave_w (else equal shares)
  int pf_n;                            // pieces per stream wave of projection pf_kind prefetched into LDS during attention
  int kv_pf;                           // stream waves whose first K/V tile is prefetched into LDS (0: off)
  int kv_pf_tile;                      // LDS bytes of one prefetched tile
  unsigned o_refill_delay;             // ticks (100 MHz) a workgroup without attention units waits
                                       // after the QKV phase before prefetching the output projection
  unsigned long long window_layers;    // bit l: layer l attends over the window
  int levels_per_token;
  // weights (library-owned, packed)
  // Per layer: Wqkv [(Hq+2Hkv)*dh][d] (q/k rows pair-interleaved per head:
  // i, i+dh/2), Wo [d][Hq*dh], Wgu [2F][d] (row 2j = gate j, 2j+1 = up j),
  // Wd [d][F]; all fp16.  The RMSNorm gains that precede a projection are
  // folded into its columns (Wqkv and Wgu by the layer's attention / FFN norm
  // gains, lm_head by the final norm gain), each product rounded to fp16 once.
  const char *wbase;
  unsigned long long layer_stride;
  unsigned long long part_off[LW_COUNT];
  const void *tok_emb, *lm_head;
  // state
  void *kcache, *vcache;   // fp16 [L][Hkv][kv_tiles] tiles of kKvTile positions (k_elem / v_elem)
  int kv_tiles;            // tiles per (layer, KV head): ceil(max_seq / kKvTile)
  const float *rope;       // [max_seq][dh/2][2] (cos, sin)
  float *x_hidden;         // fp32 [d] layer-0 input (LF_HIDDEN_IO, written by the host)
  float *x_out;            // fp32 [d] residual after the last layer (LF_HIDDEN_IO, read by the host)
  // Exchange words between workgroups: {payload in bits 0..31, level tag in
  // bits 32..63}, two generations selected by layer parity.  A consumer accepts
  // a word only when its tag is the level it waits for.
  unsigned long long *xmid_t, *xout_t;   // [2][d] fp32 residual after O / after down
  unsigned long long *q_t;               // [2][Hq*dh] fp32 post-rotary queries
  unsigned long long *kc_t, *vc_t;       // [2][Hkv*dh/2] fp16 pairs of the current K row
                                         //   (dims i, i+dh/2) and V row (dims 2j, 2j+1)
  unsigned long long *part_t;            // [2][part_gen] split-K partials (m, l, o[dh])
  unsigned long long *o_t;               // [2][Hq*dh/2] fp16 pairs of the merged attention output
  unsigned long long *a_t;               // [2][F/2] fp16 pairs of the SwiGLU output
  unsigned long long part_gen;           // words per generation of part_t
  // the nucleus draw over the grid (nucleus sampling; null otherwise): each
  // workgroup's masses per bin [256][G][2], bin totals [256][2], records
  // [G][3 + nuc_cmax / 2] (count, mass before the boundary bin, the boundary
  // bin's rows two a word), largest logits [G]
  unsigned long long *nuc_hist, *nuc_btot, *nuc_cand, *nuc_zmax;
  int nuc_cmax;                          // most lm_head rows of one workgroup
  int nuc_grid;                          // 1: the draw over the grid, 0: workgroup 0 alone
  float *logits;           // fp32 [V]
  float *lm_val;           // [G] per-workgroup max logit
  int *lm_idx;             // [G] its index
  unsigned *progress;      // [G] last completed level of each workgroup
  int *tok_slot;           // [1] token chosen by the last step
  int *out_tokens;         // [n_tokens]
  const int *in_tokens;    // [n_tokens] teacher-forced tokens (prefill launches)
  unsigned *err;           // [4] {code, workgroup, level, 0}
  unsigned long long *stats;  // [G][stat_stride]: kStatWords counters, then (LF_TRACE builds) a phase trace
  int stat_stride, trace_token;
  // this launch
  int n_tokens, token0, pos0;
  unsigned level_base;
  unsigned long long timeout_ticks;
  int plain_launch;        // 1: ordinary launch instead of a cooperative one
  // LDS layout (byte offsets into dynamic shared memory)
  int lds_h, lds_attn, lds_part, lds_red, lds_ctl, lds_xown, lds_xres, lds_trace, lds_pf, lds_kvpf, lds_bytes;
  int psum_off[5];                     // LDS partial row sums: each phase kind's first float
  int psum_total, hmax;                // floats of all kinds' partial row sums
};

hipError_t launch_monokernel(const Params &p, bool prefill, hipStream_t stream);
// The entry point that allocates nothing keeps its per-launch scratch in a
// static device array of this many bytes (one per GPU).
constexpr size_t kNoallocScratchBytes = (size_t)4 << 20;
// Look up the array's device address on `device` (current) once; later calls
// return at once.  noalloc_scratch: that address, or null before the lookup.
hipError_t noalloc_scratch_init(int device);
void *noalloc_scratch(int device);
// Zero `bytes` (a multiple of 8) at p with a fill kernel on `stream`.
hipError_t launch_zero(void *p, size_t bytes, hipStream_t stream);
// w[r][c] = fp16(w[r][c] * g[c]) for an fp16 matrix of `rows` rows of `cols`
// elements (cols % 8 == 0, w 16-byte aligned, g 2-byte aligned).
hipError_t launch_scale_columns(void *w, size_t rows, int cols, const void *g, hipStream_t stream);
// Copy n cache positions pos0.. of layer l between natural [n][Hkv][dh] fp16
// buffers k, v and the tiled cache (to_cache: into the cache, else out of it).
hipError_t launch_kv_copy(const Params &p, int l, int pos0, int n, void *k, void *v, bool to_cache,
                          hipStream_t stream);
hipError_t launch_test_expdef(const float *x, float *y, int64_t n, hipStream_t stream);
hipError_t launch_test_logdef(const float *x, float *y, int64_t n, hipStream_t stream);
hipError_t launch_test_gumbel(const float *logits, int n, float inv_temp, unsigned long long seed, const int *pos,
                              int m, int *tokens, hipStream_t stream);
hipError_t launch_test_sample(const float *logits, int n, float inv_temp, float top_p,
                              unsigned long long seed, const int *pos, int m, int *tokens,
                              hipStream_t stream);
const void *monokernel_symbol(bool prefill, int qpg);   // the instance for qpg query heads per KV head

}  // namespace lf

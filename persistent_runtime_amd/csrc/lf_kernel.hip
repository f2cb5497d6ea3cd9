// lf_kernel.hip -- the persistent batch-1 decode kernel for gfx950 (MI355X).
//
// One workgroup (8 wave64s) per compute unit runs the whole decode pass, every
// layer and the next-token choice, for n tokens in a single launch ("KOG
// LaneFormer-2B & the monokernel", sections "Pillar 3 - the monokernel runtime"
// and "Compile-time work partition").  Work is partitioned statically: every
// matrix is cut into contiguous row blocks, one per workgroup, fixed for the
// life of the state; attention is cut into (KV head, key chunk) units, and a
// short GQA head into one unit per query head.
//
// Roles inside a workgroup.  Wave 0 is the SYNC wave: after each phase it adds
// the stream waves' partial row sums and runs the phase's epilogue (rotary
// embedding and the KV-cache append, the residual add, SiLU(gate) * up, the
// lm_head's local argmax), stores the outputs as tagged exchange words and
// stores its progress word; with temperature and top-p, every workgroup's sync
// wave takes part in the nucleus draw over its own lm_head rows.  Waves 1..7 are STREAM waves: each walks its own
// contiguous slice of the workgroup's weight rows, phase after phase, layer
// after layer, token after token, through a ring of eight 1-KB pieces held in
// registers the compiler never allocates (v224..v255), loaded with
// non-temporal 16-byte global loads; the loop that consumes a phase's rounds
// and refills each slot as it is freed is inline assembly, and the first
// round of the next phase is issued as soon as a phase is done, so those loads
// are in flight while its input is still being produced ("Weight streaming -
// keeping HBM saturated").  All eight waves stage each phase's input vector
// into LDS together, and the stream waves also run the attention units.
//
// Synchronisation between workgroups.  No grid barrier and no counter.  The
// vectors passed between phases are 64-bit words that carry their payload and
// the dependency level that produced it, and an aligned 8-byte store is
// single-copy atomic: a consumer re-reads a vector until every word carries
// the level it waits for, so the data are their own flag and a producer never
// waits for its stores before announcing them ("Cross-GPU synchronization
// without atomics": consumers poll the memory the producer writes).  Split-K
// attention partials are merged by a fixed unit per KV head that waits on the
// partials' tags.  Untagged data (logits, the per-workgroup argmax partials,
// the chosen token) use the per-workgroup progress words, stored after the
// producer's stores complete; the nucleus draw instead polls each workgroup's
// largest logit as a tagged word stored after that progress word.  Every wait is bounded: on expiry the workgroup
// writes the error word and returns, every other wait sees it and returns too,
// so the grid always drains.
//
// Matrix-vector products run on the vector ALUs with v_dot2_f32_f16 (fp16 x
// fp16 products, fp32 accumulation) and cross-lane sums, not on MFMA: at batch 1
// there is no dense contraction to feed matrix cores ("The fused operations,
// briefly").
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstddef>
#include <mutex>

#include "lf_internal.h"

namespace lf {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// The parameter block as seen by the kernel: in the constant (kernel argument)
// address space, read with scalar loads.
typedef const __attribute__((address_space(4))) Params KP;

// The same parameter block through an opaque pointer: field reads after this
// point cannot be hoisted above it, so a region re-reads the few fields it uses
// instead of keeping every field of the block live in scalar registers for the
// whole kernel (they would crowd out the stream loop's state).
__device__ __forceinline__ KP &fresh(KP &P) {
  KP *p = &P;
  asm volatile("" : "+s"(p));
  return *p;
}

constexpr int kNcw = kWaves - 1;       // stream waves per workgroup
constexpr int kRing = kRingSlots;      // 1-KB pieces each stream wave keeps in flight (registers)
constexpr int kMaxQpg = 8;             // query heads per KV head supported
enum Kind { K_QKV = 0, K_O = 1, K_GU = 2, K_D = 3, K_LM = 4, K_COUNT = 5 };
// sync-wave activities timed with LF_STATS: staging, waiting for the stream
// waves, epilogue + publish, attention, lm_head + token choice
enum StatPhase { ST_STAGE = 0, ST_STREAMS = 1, ST_EPI = 2, ST_ATTN = 3, ST_LM = 4, kStatPhases = 5 };

// Thread index through an opaque copy: the kernel's outer token and layer loops
// would otherwise let the compiler hoist every per-thread address of every phase
// out of them and spill the lot.
__device__ __forceinline__ int tid_x() {
  int t = (int)threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}
__device__ __forceinline__ int lane_id() { return tid_x() & 63; }
// The wave index is uniform: keep it (and all work derived from it) scalar.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(tid_x() >> 6); }

// Eight fp16 products accumulated in fp32 with four v_dot2_f32_f16.  The halves
// are taken by bit-casting the whole 16-byte vector and shuffling pairs out of
// it: hipcc mis-compiles a bit-cast of a single ext-vector element (w.y) into a
// read of element 0.
__device__ __forceinline__ float dot8(u32x4 w, u32x4 h, float acc) {
  const f16x8 a = __builtin_bit_cast(f16x8, w), b = __builtin_bit_cast(f16x8, h);
  acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(a, a, 0, 1), __builtin_shufflevector(b, b, 0, 1), acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(a, a, 2, 3), __builtin_shufflevector(b, b, 2, 3), acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(a, a, 4, 5), __builtin_shufflevector(b, b, 4, 5), acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(a, a, 6, 7), __builtin_shufflevector(b, b, 6, 7), acc, false);
  return acc;
}

#define LF_DPP(v, ctrl, rmask) \
  __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, (v)), (ctrl), (rmask), 0xf, false))

// Wave-wide sum with DPP row operations; the total ends up in lane 63.
__device__ __forceinline__ float wave_sum_to63(float v) {
  v += LF_DPP(v, 0xB1, 0xf);    // quad_perm [1,0,3,2]
  v += LF_DPP(v, 0x4E, 0xf);    // quad_perm [2,3,0,1]
  v += LF_DPP(v, 0x141, 0xf);   // row_half_mirror
  v += LF_DPP(v, 0x140, 0xf);   // row_mirror
  v += LF_DPP(v, 0x142, 0xa);   // row_bcast:15 into rows 1 and 3
  v += LF_DPP(v, 0x143, 0xc);   // row_bcast:31 into rows 2 and 3
  return v;
}
// Wave-wide sum, the same value in every lane.
__device__ __forceinline__ float wave_sum(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wave_sum_to63(v)), 63));
}
// DPP move whose disabled lanes keep their own value (an identity for max / min).
#define LF_DPP_KEEP(v, ctrl, rmask) \
  __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, (v)), __builtin_bit_cast(int, (v)), (ctrl), (rmask), 0xf, false)
// Wave-wide max / min with the same DPP row steps as wave_sum_to63, the result
// read back from lane 63 into every lane.
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, __builtin_bit_cast(float, LF_DPP_KEEP(v, 0xB1, 0xf)));
  v = fmaxf(v, __builtin_bit_cast(float, LF_DPP_KEEP(v, 0x4E, 0xf)));
  v = fmaxf(v, __builtin_bit_cast(float, LF_DPP_KEEP(v, 0x141, 0xf)));
  v = fmaxf(v, __builtin_bit_cast(float, LF_DPP_KEEP(v, 0x140, 0xf)));
  v = fmaxf(v, __builtin_bit_cast(float, LF_DPP_KEEP(v, 0x142, 0xa)));
  v = fmaxf(v, __builtin_bit_cast(float, LF_DPP_KEEP(v, 0x143, 0xc)));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
__device__ __forceinline__ unsigned wave_min_u32(unsigned v) {
  v = min(v, (unsigned)LF_DPP_KEEP(v, 0xB1, 0xf));
  v = min(v, (unsigned)LF_DPP_KEEP(v, 0x4E, 0xf));
  v = min(v, (unsigned)LF_DPP_KEEP(v, 0x141, 0xf));
  v = min(v, (unsigned)LF_DPP_KEEP(v, 0x140, 0xf));
  v = min(v, (unsigned)LF_DPP_KEEP(v, 0x142, 0xa));
  v = min(v, (unsigned)LF_DPP_KEEP(v, 0x143, 0xc));
  return (unsigned)__builtin_amdgcn_readlane((int)v, 63);
}
// Wave-wide argmax of (value, index) pairs held one per lane (index >= 0):
// the largest value, and among lanes holding it the smallest index.
__device__ __forceinline__ void wave_argmax(float &best, int &bi) {
  const float m = wave_max(best);
  bi = (int)wave_min_u32(best == m ? (unsigned)bi : 0xffffffffu);
  best = m;
}
// Whether no active lane has p set (one compare into a scalar lane mask).
__device__ __forceinline__ bool wave_none(bool p) { return __builtin_amdgcn_ballot_w64(p) == 0ull; }
// One DPP move of a 64-bit value (two 32-bit moves); lanes without a source
// read 0.
#define LF_DPP_U64(v, ctrl, rmask)                                                                     \
  (((unsigned long long)(unsigned)__builtin_amdgcn_update_dpp(0, (int)(unsigned)((v) >> 32), (ctrl), (rmask), \
                                                              0xf, false)                                \
    << 32) |                                                                                             \
   (unsigned)__builtin_amdgcn_update_dpp(0, (int)(unsigned)(v), (ctrl), (rmask), 0xf, false))
__device__ __forceinline__ unsigned long long lane63_u64(unsigned long long v) {
  const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)v, 63);
  const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(v >> 32), 63);
  return ((unsigned long long)hi << 32) | lo;
}
// Wave-wide sum of 64-bit integers with the same DPP row steps as wave_sum_to63
// (integer sums are exact in any order), read back from lane 63 into every lane.
__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v) {
  v += LF_DPP_U64(v, 0xB1, 0xf);
  v += LF_DPP_U64(v, 0x4E, 0xf);
  v += LF_DPP_U64(v, 0x141, 0xf);
  v += LF_DPP_U64(v, 0x140, 0xf);
  v += LF_DPP_U64(v, 0x142, 0xa);
  v += LF_DPP_U64(v, 0x143, 0xc);
  return lane63_u64(v);
}
// Inclusive prefix sums over the 64 lanes: shifts right by 1, 2, 4 and 8 lanes
// within each row of 16, then lane 15 of a row added into the next row (rows 1
// and 3) and lane 31 into rows 2 and 3.
__device__ __forceinline__ unsigned long long wave_scan_u64(unsigned long long v) {
  v += LF_DPP_U64(v, 0x111, 0xf);   // row_shr:1
  v += LF_DPP_U64(v, 0x112, 0xf);   // row_shr:2
  v += LF_DPP_U64(v, 0x114, 0xf);   // row_shr:4
  v += LF_DPP_U64(v, 0x118, 0xf);   // row_shr:8
  v += LF_DPP_U64(v, 0x142, 0xa);   // row_bcast:15
  v += LF_DPP_U64(v, 0x143, 0xc);   // row_bcast:31
  return v;
}
__device__ __forceinline__ unsigned wave_scan_u32(unsigned v) {
  v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false);
  v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false);
  v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false);
  v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false);
  v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);
  v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);
  return v;
}

__device__ __forceinline__ void block_range(int total, int parts, int b, int &p0, int &p1) {
  const int base = total / parts, rem = total % parts;
  p0 = b * base + (b < rem ? b : rem);
  p1 = p0 + base + (b < rem ? 1 : 0);
}

__device__ __forceinline__ unsigned long long now_ticks() { return __builtin_amdgcn_s_memrealtime(); }

// ---------------------------------------------------------------- device-scope accesses
// Data exchanged between workgroups: coherent at device scope (sc1), so a
// consumer on another XCD never reads a stale line of its own L2.
__device__ __forceinline__ float ld_dev(const float *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned ld_dev(const unsigned *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int ld_dev(const int *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long ld_dev(const unsigned long long *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(unsigned *p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(int *p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev_h(void *base, size_t i, float v) {
  const _Float16 h = (_Float16)v;
  __hip_atomic_store(reinterpret_cast<unsigned short *>(base) + i, __builtin_bit_cast(unsigned short, h),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Tagged exchange words: payload in bits 0..31, level tag in bits 32..63.  An
// aligned 8-byte store / load is single-copy atomic, so a word whose tag is the
// awaited level carries that level's payload: no fence or store acknowledgement
// is needed between producing data and announcing it.
typedef unsigned long long u64;
__device__ __forceinline__ u64 tag_f(float v, unsigned tag) {
  return (u64)__float_as_uint(v) | ((u64)tag << 32);
}
__device__ __forceinline__ u64 tag_h2(float a, float b, unsigned tag) {
  f16x2 h;
  h.x = (_Float16)a;
  h.y = (_Float16)b;
  return (u64)__builtin_bit_cast(unsigned, h) | ((u64)tag << 32);
}
__device__ __forceinline__ unsigned tag_of(u64 w) { return (unsigned)(w >> 32); }
__device__ __forceinline__ float pay_f(u64 w) { return __uint_as_float((unsigned)w); }
__device__ __forceinline__ void st_tag(u64 *p, u64 w) {
  __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Exchange words through a pointer typed as global memory.  A pointer passed
// through an empty asm statement (to fix where its address is computed) loses
// what the compiler knew of its address space, and a generic pointer's accesses
// become FLAT instructions, which also count in lgkmcnt: every later wait for an
// LDS access would then wait for them too.  This type keeps them global.
typedef __attribute__((address_space(1))) u64 gu64;
__device__ __forceinline__ void st_tag(gu64 *p, u64 w) {
  __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ u64 ld_dev(const gu64 *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// LDS words shared between the waves of one workgroup.
__device__ __forceinline__ unsigned lds_ld(const unsigned *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_st(unsigned *p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// Complete this wave's earlier LDS accesses (e.g. before a flag that announces them).
__device__ __forceinline__ void lds_drain() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt not waited on
  asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------- LDS control block

struct Geo {            // one phase kind's row block in this workgroup
  int r0, nrows, kv, ppr;   // first row, rows, 16-B vectors per row, 1-KB pieces per row
};

// A stream wave's pieces of one phase kind: n pieces from piece kp of row `row`.
struct Slice {
  int n, row, kp, pad_;
};

struct Ctl {
  unsigned abort;           // the sync wave gave up (the error word is set)
  unsigned done[kWaves];    // per stream wave: last GEMV phase (1-based) it finished
  int status;               // outcome of a barrier-based wait
  unsigned abar;            // arrivals at the stream waves' barrier (kNcw per barrier)
  int na;                   // workgroups 0 .. na-1 run attention with prefetched tiles (no QKV rows)
  int pad[4];
  float ssw[kWaves];        // per wave: sum of squares of its share of an RMSNorm input
  Geo geo[K_COUNT];
  // The partition of every phase kind among the stream waves, fixed for the
  // launch: computed once so that no phase divides by the pieces per row.
  Slice slice[K_COUNT][kNcw];
  // The first pieces of each stream wave's share of projection P.pf_kind,
  // prefetched into its own LDS area before the phase (slice[] then holds the rest).
  Slice pf[kNcw];
};
static_assert(sizeof(Ctl) <= kCtlBytes, "workgroup control block exceeds its LDS space");

// ---------------------------------------------------------------- global sync (wave 0)

struct Sync {
  KP *P;
  Ctl *ctl;
  unsigned long long spin;    // ticks spent polling other workgroups
  unsigned long long waits;
  unsigned long long tm[kStatPhases];   // sync-wave time by activity (LF_STATS)
  int trace_k;                               // LF_TRACE: phase slot being staged, else -1
  bool timed;                                // LF_STATS: activity timers on
};

// Add the ticks since t0 to activity k; returns the current tick.
__device__ __forceinline__ unsigned long long lap(Sync &s, int k, unsigned long long t0) {
  if (!s.timed) return 0ull;
  const unsigned long long t1 = now_ticks();
  s.tm[k] += t1 - t0;
  return t1;
}
// The current tick when activity timers are on (LF_STATS), else 0.
__device__ __forceinline__ unsigned long long stamp(const Sync &s) { return s.timed ? now_ticks() : 0ull; }

// LF_TRACE builds: timestamp j (0 input staged, 1 streams done, 2 published;
// stream wave 1: 3 input seen, 4 first round done, 5 done; wave 0: 6 staging
// started, 7 tagged input complete, 8 its first poll back, 9 its poll round
// trips (a count), and for the QKV phase 12 the layer loop's top, 11 after the
// row block's read; attention, wave 1: 6
// unit start, 7 first barrier passed, 3 queries staged, 8 first keys loaded,
// 10 first scores, 4 keys done, 9 waves' states in LDS, 5 partial stored, and
// in a merging unit 11 merge start, 12 the waves' folded states in LDS, 13
// heads merged and stored)
// of phase k (5l + {QKV, attention, O, gate/up, down}; 5L lm_head; 5L+1 token).
// Timestamps collect in LDS and are copied out when the kernel ends, so that
// tracing adds no global stores (and no store waits) to the path it measures.
typedef __attribute__((address_space(3))) unsigned long long lds_u64;
__device__ __forceinline__ lds_u64 *trace_row(KP &P, int k) {
  extern __shared__ __align__(16) unsigned char lf_dyn_lds[];
  return (lds_u64 *)(lf_dyn_lds + P.lds_trace) + kTraceSlots * k;
}
__device__ __forceinline__ void trace(KP &P, int t, int k, int j) {
  if (kTrace && t == P.trace_token && lane_id() == 0) trace_row(P, k)[j] = now_ticks();
}
// stamp j of phase slot k, if k >= 0 (lane 0 only)
__device__ __forceinline__ void trace_at(KP &P, int k, int j) {
  if (kTrace && k >= 0 && lane_id() == 0) trace_row(P, k)[j] = now_ticks();
}

// Mark a loaded value as used.  A load whose result is never read stays
// "in flight" for the compiler, and where paths merge it then waits for every
// memory access issued since (stores included) before it reuses the register.
// Retiring the value where it is already in (it was requested before the loads
// just waited for) costs no wait.
__device__ __forceinline__ void retire(unsigned v) { asm volatile("" ::"v"(v)); }

// The bound of a wait started at t0 has expired: record the first such event in
// the error word (any lane may call; one wins).  Also true once another
// workgroup has recorded an error: err0 is the error word as read with the
// polled data, in the same batch of loads, so that checking it adds no memory
// round trip to a retry.
__device__ __forceinline__ bool expired(KP &P, unsigned long long t0, unsigned level, unsigned err0) {
  if (now_ticks() - t0 <= P.timeout_ticks) return err0 != 0u;
  unsigned zero = 0u;
  if (__hip_atomic_compare_exchange_strong(&P.err[0], &zero, 1u, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT)) {
    st_dev(&P.err[1], (unsigned)blockIdx.x);
    st_dev(&P.err[2], level);
  }
  return true;
}

// Wave 0 only: poll progress[first .. first+count) >= level.  Returns false when
// the bound expired or another workgroup reported an error.
__device__ __forceinline__ bool poll_level(Sync &s, int first, int count, unsigned level) {
  KP &P = *s.P;
  const unsigned long long t0 = now_ticks();
  bool ok = false;
  for (;;) {
    bool behind = false;
    const unsigned e = ld_dev(&P.err[0]);
    // up to 256 words a pass with every load in flight (clamped indices; the
    // copies past count are ignored), not one round trip per 64 words
    for (int i0 = 0; i0 < count; i0 += 4 * 64) {
      unsigned v[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) v[k] = ld_dev(&P.progress[first + min(i0 + 64 * k + lane_id(), count - 1)]);
#pragma unroll
      for (int k = 0; k < 4; ++k) behind |= i0 + 64 * k + lane_id() < count && v[k] < level;
    }
    if (wave_none(behind)) {
      retire(e);
      ok = true;
      break;
    }
    if (expired(P, t0, level, e)) break;
  }
  s.spin += now_ticks() - t0;
  s.waits += 1;
  return ok;
}

// Wave 0 only: announce `level` for this workgroup.  The level's data are tagged
// words, so the announcement need not wait for them to land: a consumer that
// sees the progress word early re-reads until the tags match.
__device__ __forceinline__ void publish_fast(KP &P, unsigned level) {
  if (lane_id() == 0) st_dev(&P.progress[blockIdx.x], level);
}

// Wave 0 only: announce `level` after every store of this wave has completed
// (for the untagged data of the lm_head and token levels).
__device__ __forceinline__ void publish_sync(KP &P, unsigned level) {
  __builtin_amdgcn_s_waitcnt(0);
  asm volatile("" ::: "memory");
  if (lane_id() == 0) st_dev(&P.progress[blockIdx.x], level);
}

// Wave 0: announce a level whose data other workgroups read as tagged words.
__device__ __forceinline__ void publish_vec(KP &P, unsigned level) { publish_fast(P, level); }

// All waves: barrier-based wait (wave 0 polls).  Used where the whole workgroup
// works together (attention, nucleus sampling).  With `acquire`, wave 0 takes an
// agent-scope acquire fence so the workgroup may read untagged data with plain
// loads.
__device__ __forceinline__ bool wait_all_waves(Sync &s, int first, int count, unsigned level,
                                               bool acquire = false) {
  if (wave_id() == 0) {
    const bool ok = poll_level(s, first, count, level);
    if (ok && acquire) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      __builtin_amdgcn_s_waitcnt(0);
    }
    if (lane_id() == 0) s.ctl->status = ok ? 1 : 2;
  }
  __syncthreads();
  const bool ok = s.ctl->status == 1;
  __syncthreads();
  return ok;
}

// ---------------------------------------------------------------- staging (wave 0)

constexpr int kStageBatch = kStageRound / 64;   // words per lane in one staging round

// ---- cooperative staging (all waves)

// Workgroup barrier that waits for no memory operation: the stream waves keep
// their ring loads in flight across it.  A wave that has ended no longer
// counts, so a wave that gives up releases the others.
__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// How a GEMV phase's input vector reaches LDS: a tagged residual to normalise
// (RMS: fp32 words -> fp16 h, sum of squares), tagged fp16 pairs (PAIRS: 32-bit
// words -> h), or, for the first layer's input, plain memory read by the sync
// wave alone (PLAIN).  n words at src, each carrying `tag` once valid.
enum StageMode { SM_RMS = 0, SM_PAIRS = 1, SM_PLAIN = 2 };
struct StageSpec {
  const u64 *src;
  int n, mode;
  unsigned tag;
  int cap0, capn;   // RMS: words [cap0, cap0 + capn) are also kept in fp32, in cap[0 .. capn)
  float *cap;
};

// One wave's share of a tagged vector src[0..n): the 64-word slots
// [w ns / 8, (w + 1) ns / 8) of the vector's ns slots, read up to kCoopChunk
// slots at once and re-read until every word carries `tag`; then use(i, word,
// real) for every word of the share (real: i < n).  Only the pass that finds
// the words valid hands them over, so a retry costs one bare round trip, and
// the eight waves' passes run side by side.  The buffer must be readable up to
// n rounded up to whole slots.  Each pass reads the error word with the data.
constexpr int kCoopChunk = 8;
template <class F>
__device__ __forceinline__ bool coop_fetch(KP &P, const u64 *src, int n, unsigned tag, int wave, F &&use,
                                           int trk = -1) {
  const int lane = lane_id();
  const unsigned long long t0 = now_ticks();
  int polls = 0;   // LF_TRACE: round trips of the last chunk
  const int ns = (n + 63) >> 6;
  const int s0 = wave * ns / kWaves, s1 = (wave + 1) * ns / kWaves;
  for (int c0 = s0; c0 < s1; c0 += kCoopChunk) {
    const int m = min(kCoopChunk, s1 - c0);
    const u64 *rp = src + 64 * c0 + lane;
    for (;;) {
      // The error word first: loads complete in order, so once the words are
      // in, no load of this loop is left in flight (a load still in flight
      // into a register the code reuses later would make that reuse wait for
      // every access issued since, stores included).
      const unsigned e = ld_dev(&P.err[0]);
      u64 v[kCoopChunk];
#pragma unroll
      for (int k = 0; k < kCoopChunk; ++k) v[k] = k < m ? ld_dev(rp + 64 * k) : ((u64)tag << 32);
      bool bad = false;
#pragma unroll
      for (int k = 0; k < kCoopChunk; ++k) bad |= 64 * (c0 + k) + lane < n && tag_of(v[k]) != tag;
      if (kTrace && trk >= 0) {
        if (polls == 0) trace_at(P, trk, 8);   // first poll back
        ++polls;
      }
      if (wave_none(bad)) {
        retire(e);
#pragma unroll
        for (int k = 0; k < kCoopChunk; ++k) {
          const int i = 64 * (c0 + k) + lane;
          if (k < m) use(i, v[k], i < n);
        }
        break;
      }
      if (expired(P, t0, tag, e)) return false;
    }
  }
  if (kTrace && trk >= 0 && lane == 0) trace_row(P, trk)[9] = (unsigned long long)polls;
  return true;
}

// All waves (of a workgroup with rows in the phase): stage the phase's input
// vector into LDS h.  Tagged inputs are split over the eight waves; a plain
// input is read by the sync wave alone.  For RMSNorm inputs each wave leaves
// the sum of squares of its share in ctl->ssw.  On a timeout the wave sets the
// abort flag.  The caller then meets the other waves at wg_barrier().
__device__ __forceinline__ void coop_stage(KP &P, Ctl *ctl, const StageSpec &sp, int wave, _Float16 *h,
                                           int trk = -1) {
  const int lane = lane_id();
  bool ok = true;
  if (sp.mode == SM_RMS) {
    float ss = 0.0f;
    ok = coop_fetch(P, sp.src, sp.n, sp.tag, wave, [&](int i, u64 w, bool real) __attribute__((always_inline)) {
      const float x = pay_f(w);
      ss += real ? x * x : 0.0f;
      h[i] = (_Float16)x;
      if ((unsigned)(i - sp.cap0) < (unsigned)sp.capn) sp.cap[i - sp.cap0] = x;
    }, trk);
    ss = wave_sum(ss);
    if (lane == 0) ctl->ssw[wave] = ss;
  } else if (sp.mode == SM_PAIRS) {
    unsigned *dst = reinterpret_cast<unsigned *>(h);
    ok = coop_fetch(P, sp.src, sp.n, sp.tag, wave,
                    [&](int i, u64 w, bool) __attribute__((always_inline)) { dst[i] = (unsigned)w; }, trk);
  }
  if (!ok && lane == 0) lds_st(&ctl->abort, 1u);
  lds_drain();
}

// Sync wave, after the barrier of an RMSNorm stage: 1 / rms from the waves'
// sums of squares (added in wave order).
__device__ __forceinline__ float coop_inv_rms(const Ctl *ctl, int d, float eps) {
  float ss = 0.0f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) ss += ctl->ssw[w];
  return 1.0f / sqrtf(ss / (float)d + eps);
}

// The input of GEMV phase `kind` of layer l of token t (gen: the layer's buffer
// generation, lvl: the layer's base level; for K_LM, lvl is the level of the
// last layer's down projection).  The residual stream's rows that this
// workgroup's epilogues add to are kept in fp32 as they arrive: its
// output-projection rows of the layer input in xo, its down-projection rows of
// x after attention in xd (two buffers: a workgroup may still read xd for the
// previous layer's down projection while its waves fetch the next layer input).
__device__ __forceinline__ StageSpec stage_spec(const KP &P, const Ctl *ctl, int kind, int t, int l, int gen,
                                                unsigned lvl, float *xo, float *xd) {
  StageSpec sp;
  const int L = P.L, d = P.d;
  sp.src = nullptr;
  sp.n = d;
  sp.mode = SM_RMS;
  sp.tag = lvl;
  sp.cap0 = sp.capn = 0;
  sp.cap = xo;
  switch (kind) {
    case K_QKV:
      if (l > 0) {
        sp.src = P.xout_t + (size_t)((t * L + l - 1) & 1) * d;
        sp.cap0 = __builtin_amdgcn_readfirstlane(ctl->geo[K_O].r0);
        sp.capn = __builtin_amdgcn_readfirstlane(ctl->geo[K_O].nrows);
      } else {
        sp.mode = SM_PLAIN;
      }
      break;
    case K_O:
      sp.src = P.o_t + (size_t)gen * (P.Hq * P.dh / 2);
      sp.n = P.Hq * P.dh / 2;
      sp.mode = SM_PAIRS;
      sp.tag = lvl + PH_ATTN;
      break;
    case K_GU:
      sp.src = P.xmid_t + (size_t)gen * d;
      sp.tag = lvl + PH_O;
      sp.cap0 = __builtin_amdgcn_readfirstlane(ctl->geo[K_D].r0);
      sp.capn = __builtin_amdgcn_readfirstlane(ctl->geo[K_D].nrows);
      sp.cap = xd;
      break;
    case K_D:
      sp.src = P.a_t + (size_t)gen * (P.F / 2);
      sp.n = P.F / 2;
      sp.mode = SM_PAIRS;
      sp.tag = lvl + PH_GU;
      break;
    default:   // K_LM
      sp.src = P.xout_t + (size_t)((t * L + L - 1) & 1) * d;
      break;
  }
  return sp;
}

// The same for a layer-0 input: an fp16 embedding row or the host's fp32
// vector.  Returns 1 / rms.
// One source type per instance, and every load unconditional (indices clamped
// into the row), so that all of a round's loads are in flight at once: a
// guarded load, or a choice of source inside the loop, made the compiler wait
// for each load in turn (40 round trips for a 2560-element row).
template <class T>
__device__ __forceinline__ float stage_rmsnorm_plain(const T *x, int d, float eps, _Float16 *h) {
  const int lane = lane_id();
  float ss = 0.0f;
  for (int base = 0; base < d; base += 64 * kStageBatch) {
    float v[kStageBatch];
#pragma unroll
    for (int j = 0; j < kStageBatch; ++j) v[j] = (float)x[min(base + 64 * j + lane, d - 1)];
#pragma unroll
    for (int j = 0; j < kStageBatch; ++j) {
      const int i = base + 64 * j + lane;
      if (i < d) {
        ss += v[j] * v[j];
        h[i] = (_Float16)v[j];
      }
    }
  }
  return 1.0f / sqrtf(wave_sum(ss) / (float)d + eps);
}

// ---------------------------------------------------------------- stream waves

// Weight rows of phase kind k in layer l for this workgroup: row r0 of its block.
__device__ __forceinline__ const void *layer_part(KP &P, int l, int part) {
  return P.wbase + (size_t)l * P.layer_stride + P.part_off[part];
}

// Weight rows of phase kind k in layer l for this workgroup: row r0 of its block.
// Pure address arithmetic (no loads), so crossing a phase never drains the
// stream wave's load pipeline.
__device__ __forceinline__ const unsigned char *phase_base(KP &P, const Geo &g, int kind, int l) {
  const void *w;
  switch (kind) {
    case K_QKV: w = layer_part(P, l, LW_QKV); break;
    case K_O: w = layer_part(P, l, LW_O); break;
    case K_GU: w = layer_part(P, l, LW_GU); break;
    case K_D: w = layer_part(P, l, LW_D); break;
    default: w = P.lm_head; break;
  }
  return reinterpret_cast<const unsigned char *>(w) + (size_t)g.r0 * g.kv * 16;
}

// A phase kind's partial row sums in LDS: [rows][8], slot 7 unused.
__device__ __forceinline__ float *kind_part(float *part, int off) { return part + off; }

// A phase kind's row block, read from LDS into wave-uniform (scalar) registers.
__device__ __forceinline__ Geo uniform_geo(const Ctl *ctl, int kind) {
  const Geo g = ctl->geo[kind];
  return Geo{__builtin_amdgcn_readfirstlane(g.r0), __builtin_amdgcn_readfirstlane(g.nrows),
             __builtin_amdgcn_readfirstlane(g.kv), __builtin_amdgcn_readfirstlane(g.ppr)};
}

__device__ __forceinline__ Slice uniform_slice(const Ctl *ctl, int kind, int cw) {
  const Slice sl = ctl->slice[kind][cw];
  return Slice{__builtin_amdgcn_readfirstlane(sl.n), __builtin_amdgcn_readfirstlane(sl.row),
               __builtin_amdgcn_readfirstlane(sl.kp), 0};
}

// Stream wave cw's share [lo, hi) of the np pieces of a row block (contiguous).
// The stream waves' shares of a workgroup's np pieces (counts n[0 .. kNcw)).
// Waves sharing a SIMD do not stream equally fast (the lower-numbered wave of
// each pair finishes first), so the shares follow the weights ww; but each
// wave's pieces are padded to whole rounds of kRing, and a round that holds one
// real piece costs nearly a full round, so no wave gets more rounds than its
// equal share needs (one more once that share is eight rounds or more).  The
// pieces the caps leave over go back to the waves below their caps, lowest
// weight last.
__device__ __forceinline__ void wave_counts(int np, const int *ww, int *n) {
  int wt = 0;
  for (int k = 0; k < kNcw; ++k) wt += ww[k];
  int w0 = 0, sum = 0, cap[kNcw];
  for (int k = 0; k < kNcw; ++k) {
    const int eq = ((k + 1) * np) / kNcw - (k * np) / kNcw;
    const int r = (eq + kRing - 1) / kRing;
    cap[k] = kRing * (r + (r >= 8 ? 1 : 0));
    const int lo = (int)((long long)np * w0 / wt);
    w0 += ww[k];
    const int hi = (int)((long long)np * w0 / wt);
    n[k] = min(hi - lo, cap[k]);
    sum += n[k];
  }
  for (int pass = 0; pass < 2 && sum < np; ++pass)   // (one pass suffices: the caps hold np)
    for (int k = 0; k < kNcw && sum < np; ++k) {
      const int add = min(cap[k] - n[k], np - sum);
      n[k] += add;
      sum += add;
    }
}

static_assert((kRing & (kRing - 1)) == 0 && kRing <= 32, "ring depth must be a power of two <= 32");
static_assert(kRing == 8, "the hand-scheduled stream rounds hold exactly eight pieces");

// ---------------------------------------------------------------- stream rounds in assembly
//
// The compiler does not model a load that stays in flight across a loop edge:
// a ring carried around a loop is moved between registers behind a wait for
// every load of the round.  The stream waves' ring therefore lives in
// registers the compiler never allocates (the kernel caps its own allocation
// at 208 VGPRs): v224..v255 hold the eight pieces in flight (slot k in
// v[224+4k : 227+4k]), v216..v223 two input-vector buffers, v208..v215
// temporaries.  Loads into the ring and every use of it are inline assembly
// with explicit waits; the compiler's own waits stay correct because loads
// complete in order (an extra ring load only makes them wait longer).

// Every VGPR the ring code owns, named as clobbered so that the kernel's VGPR
// count includes them (they are outside the compiler's allocation).
#define LF_RING_VGPRS "v208", "v209", "v210", "v211", "v212", "v213", "v214", "v215", "v216", "v217", "v218", "v219", "v220", "v221", "v222", "v223", "v224", "v225", "v226", "v227", "v228", "v229", "v230", "v231", "v232", "v233", "v234", "v235", "v236", "v237", "v238", "v239", "v240", "v241", "v242", "v243", "v244", "v245", "v246", "v247", "v248", "v249", "v250", "v251", "v252", "v253", "v254", "v255"

// Load one 1-KB piece (16 bytes per lane at base + off) into ring slot k.
#define LF_RING_LOAD(K, R)                                                                           \
  case K:                                                                                           \
    asm volatile("global_load_dwordx4 v[" #R "], %0, %1 nt" ::"v"(off), "s"(base)                   \
                 : "memory", LF_RING_VGPRS);                                                        \
    break;
__device__ __forceinline__ void ring_load(int k, const unsigned char *base, unsigned off) {
  switch (k) {
    LF_RING_LOAD(0, 224:227)
    LF_RING_LOAD(1, 228:231)
    LF_RING_LOAD(2, 232:235)
    LF_RING_LOAD(3, 236:239)
    LF_RING_LOAD(4, 240:243)
    LF_RING_LOAD(5, 244:247)
    LF_RING_LOAD(6, 248:251)
    LF_RING_LOAD(7, 252:255)
    default: break;
  }
}
#undef LF_RING_LOAD

// Request the input vector of the next slot (its piece kp is sQ) from LDS
// into v[H] and advance sQ to the next piece of the row (0 after the row's
// last piece, whose lanes past the valid vectors re-read the last one).
#define LF_HX(H)                                                                                    \
  "s_cmp_eq_u32 %[sQ], %[ppm1]\n"                                                                   \
  "s_cselect_b64 vcc, -1, 0\n"                                                                      \
  "v_cndmask_b32 v214, %[loff], %[toff], vcc\n"                                                     \
  "s_lshl_b32 %[sT1], %[sQ], 10\n"                                                                  \
  "s_add_u32 %[sT1], %[sT1], %[hb]\n"                                                               \
  "v_add_u32 v214, %[sT1], v214\n"                                                                  \
  "ds_read_b128 v[" #H "], v214\n"                                                                  \
  "s_add_u32 %[sT1], %[sQ], 1\n"                                                                    \
  "s_cmp_eq_u32 %[sQ], %[ppm1]\n"                                                                   \
  "s_cselect_b32 %[sQ], 0, %[sT1]\n"

// Use ring slot K (registers R0..R3, input vector H0..H3) once at most W loads
// issued after its own are still in flight.  A padding piece (index >= n) is
// skipped.  The row's last piece is masked to its valid lanes (tm); at a row
// end (the row's last piece, or the wave's last piece) the wave sum goes to
// part[pa] from lane 63 and pa advances one row.  The products are summed in
// the same order as the C dot.
#define LF_USE(T, K, W, R0, R1, R2, R3, H0, H1, H2, H3)                                                \
  "s_waitcnt vmcnt(" #W ")\n"                                                                       \
  "s_add_u32 %[sT1], %[sI], " #K "\n"                                                               \
  "s_cmp_lt_u32 %[sT1], %[n]\n"                                                                     \
  "s_cbranch_scc0 .Lu" #T #K "e%=\n"                                                                   \
  "s_cmp_eq_u32 %[kpc], %[ppm1]\n"                                                                  \
  "s_cbranch_scc1 .Lu" #T #K "t%=\n"                                                                   \
  "v_dot2c_f32_f16 %[acc], v" #R0 ", v" #H0 "\n"                                                   \
  "v_dot2c_f32_f16 %[acc], v" #R1 ", v" #H1 "\n"                                                   \
  "v_dot2c_f32_f16 %[acc], v" #R2 ", v" #H2 "\n"                                                   \
  "v_dot2c_f32_f16 %[acc], v" #R3 ", v" #H3 "\n"                                                   \
  "s_add_u32 %[sT0], %[sT1], 1\n"                                                                   \
  "s_cmp_eq_u32 %[sT0], %[n]\n"                                                                     \
  "s_cbranch_scc0 .Lu" #T #K "a%=\n"                                                                   \
  "s_branch .Lu" #T #K "r%=\n"                                                                         \
  ".Lu" #T #K "t%=:\n"                                                                                 \
  "s_mov_b64 %[sE], exec\n"                                                                         \
  "s_mov_b64 exec, %[tm]\n"                                                                         \
  "v_dot2c_f32_f16 %[acc], v" #R0 ", v" #H0 "\n"                                                   \
  "v_dot2c_f32_f16 %[acc], v" #R1 ", v" #H1 "\n"                                                   \
  "v_dot2c_f32_f16 %[acc], v" #R2 ", v" #H2 "\n"                                                   \
  "v_dot2c_f32_f16 %[acc], v" #R3 ", v" #H3 "\n"                                                   \
  "s_mov_b64 exec, %[sE]\n"                                                                         \
  ".Lu" #T #K "r%=:\n"                                                                                 \
  "s_nop 4\n"                                                                                       \
  "v_add_f32_dpp %[acc], %[acc], %[acc] quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n" \
  "s_nop 1\n"                                                                                       \
  "v_add_f32_dpp %[acc], %[acc], %[acc] quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n" \
  "s_nop 1\n"                                                                                       \
  "v_add_f32_dpp %[acc], %[acc], %[acc] row_half_mirror row_mask:0xf bank_mask:0xf bound_ctrl:1\n"  \
  "s_nop 1\n"                                                                                       \
  "v_add_f32_dpp %[acc], %[acc], %[acc] row_mirror row_mask:0xf bank_mask:0xf bound_ctrl:1\n"       \
  "v_mov_b32 v215, 0\n"                                                                             \
  "s_nop 1\n"                                                                                       \
  "v_mov_b32_dpp v215, %[acc] row_bcast:15 row_mask:0xa bank_mask:0xf\n"                            \
  "v_add_f32 %[acc], %[acc], v215\n"                                                                \
  "v_mov_b32 v215, 0\n"                                                                             \
  "s_nop 1\n"                                                                                       \
  "v_mov_b32_dpp v215, %[acc] row_bcast:31 row_mask:0xc bank_mask:0xf\n"                            \
  "v_add_f32 %[acc], %[acc], v215\n"                                                                \
  "v_mov_b32 v214, %[pa]\n"                                                                         \
  "s_mov_b64 %[sE], exec\n"                                                                         \
  "s_mov_b64 exec, %[m63]\n"                                                                        \
  "ds_write_b32 v214, %[acc]\n"                                                                     \
  "s_mov_b64 exec, %[sE]\n"                                                                         \
  "s_add_u32 %[pa], %[pa], 32\n"                                                                    \
  "v_mov_b32 %[acc], 0\n"                                                                           \
  ".Lu" #T #K "a%=:\n"                                                                                 \
  "s_add_u32 %[sT1], %[kpc], 1\n"                                                                   \
  "s_cmp_eq_u32 %[kpc], %[ppm1]\n"                                                                  \
  "s_cselect_b32 %[kpc], 0, %[sT1]\n"                                                               \
  ".Lu" #T #K "e%=:\n"

// Refill ring slot K (registers RR) with the next piece of the phase (address
// v[208:209] plus the lane offset; the row's last piece clamps lanes past its
// valid vectors), or with a padding re-read (v[212:213]) when none is left.
#define LF_REFILL(K, RR)                                                                            \
  "s_cmp_eq_u32 %[ileft], 0\n"                                                                      \
  "s_cbranch_scc1 .Lf" #K "d%=\n"                                                                   \
  "s_cmp_eq_u32 %[ikp], %[ppm1]\n"                                                                  \
  "s_cselect_b64 vcc, -1, 0\n"                                                                      \
  "v_cndmask_b32 v214, %[loff], %[toff], vcc\n"                                                     \
  "v_add_co_u32 v210, vcc, v208, v214\n"                                                            \
  "v_addc_co_u32 v211, vcc, 0, v209, vcc\n"                                                         \
  "global_load_dwordx4 v[" #RR "], v[210:211], off nt\n"                                            \
  "s_sub_u32 %[ileft], %[ileft], 1\n"                                                               \
  "s_cmp_eq_u32 %[ikp], %[ppm1]\n"                                                                  \
  "s_cbranch_scc1 .Lf" #K "n%=\n"                                                                   \
  "s_add_u32 %[ikp], %[ikp], 1\n"                                                                   \
  "v_add_co_u32 v208, vcc, 0x400, v208\n"                                                           \
  "v_addc_co_u32 v209, vcc, 0, v209, vcc\n"                                                         \
  "s_branch .Lf" #K "e%=\n"                                                                         \
  ".Lf" #K "n%=:\n"                                                                                 \
  "s_mov_b32 %[ikp], 0\n"                                                                           \
  "v_mov_b32 v214, %[adh]\n"                                                                        \
  "v_add_co_u32 v208, vcc, %[adl], v208\n"                                                          \
  "v_addc_co_u32 v209, vcc, v214, v209, vcc\n"                                                      \
  "s_branch .Lf" #K "e%=\n"                                                                         \
  ".Lf" #K "d%=:\n"                                                                                 \
  "global_load_dwordx4 v[" #RR "], v[212:213], off nt\n"                                            \
  ".Lf" #K "e%=:\n"

// Slot K of a round: request the next slot's input vector (NH) unless K is the
// last slot, wait for this slot's (all LDS accesses but the newest done), use
// it, and refill the slot if the round is not the phase's last.
#define LF_SLOT_REFILL(K, NH, R0, R1, R2, R3, H0, H1, H2, H3, RR)                                   \
  LF_HX(NH) "s_waitcnt lgkmcnt(1)\n" LF_USE(R, K, 7, R0, R1, R2, R3, H0, H1, H2, H3) LF_REFILL(K, RR)
#define LF_SLOT_LAST(K, W, NH, R0, R1, R2, R3, H0, H1, H2, H3)                                      \
  LF_HX(NH) "s_waitcnt lgkmcnt(1)\n" LF_USE(L, K, W, R0, R1, R2, R3, H0, H1, H2, H3)

// The LDS byte address of a pointer into this workgroup's LDS.
__device__ __forceinline__ unsigned lds_addr(const void *p) {
  return (unsigned)(size_t)((const __attribute__((address_space(3))) char *)p);
}

// One phase of a stream wave: its n pieces (n >= 1) in rounds of eight.  The
// first round is in the ring on entry (the previous phase's prefetch); every
// round but the last refills each slot as soon as its piece is used, with the
// phase's pieces from ip (issue piece kp ikp, ileft real pieces left) and
// padding re-reads of dummy; the last round only uses its pieces.  No load
// issued here is in flight on exit.
struct RoundArgs {
  unsigned n, nr, kpc, ppm1, hb, pa, ikp, ileft;
  unsigned long long ip, dummy, adv, tm;
  unsigned loff, toff;
};
__device__ __forceinline__ void stream_rounds(const RoundArgs &a, float &acc) {
  unsigned kpc = a.kpc, pa = a.pa, ikp = a.ikp, ileft = a.ileft;
  unsigned sR, sI, sQ, sT0, sT1;
  unsigned long long sE;
  const unsigned ipl = (unsigned)a.ip, iph = (unsigned)(a.ip >> 32);
  const unsigned dml = (unsigned)a.dummy, dmh = (unsigned)(a.dummy >> 32);
  const unsigned adl = (unsigned)a.adv, adh = (unsigned)(a.adv >> 32);
  const unsigned long long m63 = 1ull << 63;
  asm volatile(
      "v_mov_b32 v208, %[ipl]\n"
      "v_mov_b32 v209, %[iph]\n"
      "v_mov_b32 v213, %[dmh]\n"
      "v_add_co_u32 v212, vcc, %[dml], %[loff]\n"
      "v_addc_co_u32 v213, vcc, 0, v213, vcc\n"
      "s_mov_b32 %[sR], 0\n"
      "s_mov_b32 %[sI], 0\n"
      ".Lr%=:\n"
      "s_mov_b32 %[sQ], %[kpc]\n"
      LF_HX(216:219)
      "s_add_u32 %[sT1], %[sR], 1\n"
      "s_cmp_lt_u32 %[sT1], %[nr]\n"
      "s_cbranch_scc0 .Ll%=\n"
      LF_SLOT_REFILL(0, 220:223, 224, 225, 226, 227, 216, 217, 218, 219, 224:227)
      LF_SLOT_REFILL(1, 216:219, 228, 229, 230, 231, 220, 221, 222, 223, 228:231)
      LF_SLOT_REFILL(2, 220:223, 232, 233, 234, 235, 216, 217, 218, 219, 232:235)
      LF_SLOT_REFILL(3, 216:219, 236, 237, 238, 239, 220, 221, 222, 223, 236:239)
      LF_SLOT_REFILL(4, 220:223, 240, 241, 242, 243, 216, 217, 218, 219, 240:243)
      LF_SLOT_REFILL(5, 216:219, 244, 245, 246, 247, 220, 221, 222, 223, 244:247)
      LF_SLOT_REFILL(6, 220:223, 248, 249, 250, 251, 216, 217, 218, 219, 248:251)
      "s_waitcnt lgkmcnt(0)\n"
      LF_USE(R, 7, 7, 252, 253, 254, 255, 220, 221, 222, 223) LF_REFILL(7, 252:255)
      "s_add_u32 %[sR], %[sR], 1\n"
      "s_add_u32 %[sI], %[sI], 8\n"
      "s_branch .Lr%=\n"
      ".Ll%=:\n"
      LF_SLOT_LAST(0, 7, 220:223, 224, 225, 226, 227, 216, 217, 218, 219)
      LF_SLOT_LAST(1, 6, 216:219, 228, 229, 230, 231, 220, 221, 222, 223)
      LF_SLOT_LAST(2, 5, 220:223, 232, 233, 234, 235, 216, 217, 218, 219)
      LF_SLOT_LAST(3, 4, 216:219, 236, 237, 238, 239, 220, 221, 222, 223)
      LF_SLOT_LAST(4, 3, 220:223, 240, 241, 242, 243, 216, 217, 218, 219)
      LF_SLOT_LAST(5, 2, 216:219, 244, 245, 246, 247, 220, 221, 222, 223)
      LF_SLOT_LAST(6, 1, 220:223, 248, 249, 250, 251, 216, 217, 218, 219)
      "s_waitcnt lgkmcnt(0)\n"
      LF_USE(L, 7, 0, 252, 253, 254, 255, 220, 221, 222, 223)
      "s_waitcnt lgkmcnt(0)\n"
      : [acc] "+v"(acc), [kpc] "+s"(kpc), [pa] "+s"(pa), [ikp] "+s"(ikp), [ileft] "+s"(ileft),
        [sR] "=&s"(sR), [sI] "=&s"(sI), [sQ] "=&s"(sQ), [sT0] "=&s"(sT0), [sT1] "=&s"(sT1), [sE] "=&s"(sE)
      : [n] "s"(a.n), [nr] "s"(a.nr), [ppm1] "s"(a.ppm1), [hb] "s"(a.hb), [ipl] "s"(ipl), [iph] "s"(iph),
        [dml] "s"(dml), [dmh] "s"(dmh), [adl] "s"(adl), [adh] "s"(adh), [tm] "s"(a.tm), [m63] "s"(m63),
        [loff] "v"(a.loff), [toff] "v"(a.toff)
      : "vcc", "scc", "memory", LF_RING_VGPRS);
}
#undef LF_HX
#undef LF_USE
#undef LF_REFILL
#undef LF_SLOT_REFILL
#undef LF_SLOT_LAST



// A stream wave's weights in flight: kRing 16-byte vectors per lane (one 1-KB
// piece per slot), loaded with non-temporal global loads straight into
// registers.  Each wave's pieces of a phase are padded with dummy pieces (a
// re-read of one cached vector) to a whole number of rounds of kRing, so a phase
// always starts at slot 0, every slot is loaded and consumed unconditionally,
// every register index is a compile-time constant, and the compiler's wait
// counters (loads complete in order) wait for exactly the oldest slot.
//
// The issue side runs one round ahead of the consume side and walks GEMV phases
// q = 0, 1, ... of the launch (token t = q / ngp, phase g = q % ngp; g < 4L is
// (layer g/4, kind g%4), else the lm_head).  A piece is 64 consecutive vectors
// of one row (the last piece of a row may be partial: its idle lanes re-read
// the row's last vector).  All cursor state is wave-uniform.
struct Streamer {
  KP *P;
  const Ctl *ctl;
  int cw, ngp, qend;
  int q, left, pad, kp, ppr, tailv;   // phase, real / dummy pieces left in it, piece in row, pieces per row,
                                      // vectors in a row's last piece
  long long adv_last;                 // bytes from a row's last piece to the next row
  const unsigned char *ptr;           // next real piece (lane 0's address)
  const unsigned char *dummy;         // the 1 KB that padding pieces re-read
  bool timed;                                 // LF_STATS on stream wave 1
  int trace_k;                                // LF_TRACE: phase slot of the traced token, else -1
  unsigned long long t_ready, t_work, pieces;

  // advance to the first GEMV phase >= q_ in which this wave has pieces
  __device__ __forceinline__ void locate(int q_) {
    q = q_;
    KP &Q = fresh(*P);
    while (q < qend) {
      const int g = q % ngp;
      const bool lm = g >= 4 * Q.L;
      const int kind = lm ? K_LM : (g & 3);
      const int l = lm ? 0 : (g >> 2);
      const Geo ge = uniform_geo(ctl, kind);
      const Slice sl = uniform_slice(ctl, kind, cw);
      if (sl.n > 0) {
        const int row = sl.row;
        left = sl.n;
        pad = (kRing - left % kRing) % kRing;
        kp = sl.kp;
        ppr = ge.ppr;
        tailv = ge.kv - (ge.ppr - 1) * 64;
        adv_last = (long long)ge.kv * 16 - (long long)(ge.ppr - 1) * 1024;
        ptr = phase_base(Q, ge, kind, l) + ((size_t)row * ge.kv * 16 + (size_t)kp * 1024);
        return;
      }
      ++q;
    }
  }

  // load the next piece (real or dummy) into slot k
  __device__ __forceinline__ void issue(int k) {
    const int lane = lane_id();
    const bool real = q < qend && left > 0;
    const bool last = kp == ppr - 1;
    const unsigned off = (unsigned)((last ? min(lane, tailv - 1) : lane) * 16);
    ring_load(k, real ? ptr : dummy, off);
    if (real) {
      --left;
      if (last) {
        kp = 0;
        ptr += adv_last;
      } else {
        ++kp;
        ptr += 1024;
      }
    } else if (q < qend) {
      --pad;
    }
  }
  // one round: slots 0 .. kRing-1, then move to the next phase if this one is done
  __device__ __forceinline__ void next_phase_if_done() {
    if (q < qend && left == 0 && pad == 0) locate(q + 1);
  }
  // refill every slot with the next round of pieces
  __device__ __forceinline__ void refill() {
#pragma unroll
    for (int k = 0; k < kRing; ++k) issue(k);
    next_phase_if_done();
  }
};

// Whether stream wave st has pieces in phase kind (then stream_phase ends with a
// round whose refill the caller may defer).
__device__ __forceinline__ bool st_has_rounds(const Streamer &st, int kind, const Ctl *ctl) {
  return uniform_slice(ctl, kind, st.cw).n > 0;
}

// LDS prefetch of one projection (P.pf_kind: the output projection or gate/up).
// During attention most workgroups have nothing to stream but the output
// projection's first round, so each stream wave copies the first pieces of its
// share of that projection for layer l into an LDS area of its own with
// direct-to-LDS loads (lane i's 16 bytes to byte 16 i of the piece's KB).  They
// complete in order with the wave's other loads; the phase waits for them
// before it reads the area.
__device__ __forceinline__ unsigned char *pf_area(const KP &P, int cw) {
  extern __shared__ __align__(16) unsigned char lf_dyn_lds[];
  return lf_dyn_lds + P.lds_pf + (size_t)cw * P.pf_n * 1024;
}
__device__ __forceinline__ Slice uniform_pf(const Ctl *ctl, int cw) {
  const Slice sl = ctl->pf[cw];
  return Slice{__builtin_amdgcn_readfirstlane(sl.n), __builtin_amdgcn_readfirstlane(sl.row),
               __builtin_amdgcn_readfirstlane(sl.kp), 0};
}
__device__ __forceinline__ void lds_prefetch(KP &P, const Ctl *ctl, int cw, int l) {
  const Slice ps = uniform_pf(ctl, cw);
  if (ps.n <= 0) return;
  const int kind = P.pf_kind;
  const Geo ge = uniform_geo(ctl, kind);
  const int lane = lane_id();
  const int tailv = ge.kv - (ge.ppr - 1) * 64;
  const long long adv_last = (long long)ge.kv * 16 - (long long)(ge.ppr - 1) * 1024;
  const unsigned char *p = phase_base(P, ge, kind, l) + ((size_t)ps.row * ge.kv * 16 + (size_t)ps.kp * 1024);
  unsigned char *dst = pf_area(P, cw);
  int kp = ps.kp;
  for (int j = 0; j < ps.n; ++j) {
    const bool last = kp == ge.ppr - 1;
    const int v = last ? min(lane, tailv - 1) : lane;
    __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1))) *)(p + v * 16),
                                     (void __attribute__((address_space(3))) *)(dst + j * 1024), 16, 0, 2);
    if (last) {
      kp = 0;
      p += adv_last;
    } else {
      ++kp;
      p += 1024;
    }
  }
}
// Use the prefetched pieces: per-lane dot products over each piece, a wave sum
// into part[row][cw] at every row end and at the wave's last piece (when no
// ring pieces follow).  Returns the running sum of a row the ring part goes on
// with.
__device__ __forceinline__ float pf_consume(const KP &P, const Ctl *ctl, int cw, const _Float16 *h, float *pk,
                                               const Geo &ge, bool ring_follows) {
  const Slice ps = uniform_pf(ctl, cw);
  float acc = 0.0f;
  if (ps.n <= 0) return acc;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  const int lane = lane_id();
  const int tailv = ge.kv - (ge.ppr - 1) * 64;
  const unsigned char *src = pf_area(P, cw) + lane * 16;
  const unsigned char *hb = reinterpret_cast<const unsigned char *>(h);
  int kp = ps.kp, row = ps.row;
  for (int j = 0; j < ps.n; ++j) {
    const bool last = kp == ge.ppr - 1;
    const int v = last ? min(lane, tailv - 1) : lane;
    const u32x4 w = *reinterpret_cast<const u32x4 *>(src + j * 1024);
    const u32x4 x = *reinterpret_cast<const u32x4 *>(hb + kp * 1024 + v * 16);
    if (!last || lane < tailv) acc = dot8(w, x, acc);
    if (last || (j == ps.n - 1 && !ring_follows)) {
      const float sum = wave_sum(acc);
      if (lane == 0) pk[row * 8 + cw] = sum;
      acc = 0.0f;
    }
    if (last) {
      kp = 0;
      ++row;
    } else {
      ++kp;
    }
  }
  return acc;
}

// A stream wave's share of GEMV phase q: consume its pieces round by round from
// the register ring, refilling each slot as it is freed, and leave one partial
// row sum per (row, wave) in part[row * 8 + cw].  Returns false if the sync wave
// aborted.
__device__ __forceinline__ bool stream_phase(Streamer &st, int q, int kind, Ctl *ctl, _Float16 *h, float *part,
                                             const StageSpec &sp, bool defer_last_refill = false) {
  const Geo ge = uniform_geo(ctl, kind);
  const Slice sl = uniform_slice(ctl, kind, st.cw);
  // the dependency wait happens on wave 0; here only its LDS announcement
  const bool timed = st.timed;
  unsigned long long t0 = timed ? now_ticks() : 0ull;
  if (ge.nrows > 0 || sp.capn > 0) {
    // this wave's share of the input vector, then the workgroup barrier
    coop_stage(*st.P, ctl, sp, st.cw + 1, h);
    wg_barrier();
    if (lds_ld(&ctl->abort)) return false;
  }
  if (timed) {
    const unsigned long long t1 = now_ticks();
    st.t_ready += t1 - t0;
    t0 = t1;
  }
  const int lane = lane_id();
  const int trk = kTrace && st.cw == 0 && st.trace_k >= 0 ? st.trace_k : -1;
  trace_at(*st.P, trk, 3);
  const int ppr = ge.ppr, tailv = ge.kv - (ge.ppr - 1) * 64;
  const int n = sl.n;
  const int nr = (n + kRing - 1) / kRing;
  float acc = 0.0f;
  if (kind == st.P->pf_kind && st.P->pf_n > 0)
    acc = pf_consume(*st.P, ctl, st.cw, h, kind_part(part, fresh(*st.P).psum_off[kind]), ge, nr > 0);
  if (nr > 0) {
    // The ring holds this phase's first round.  If the phase has more pieces
    // than one round, the streamer still points into this phase: its cursor
    // (the ninth piece) is where the rounds continue.
    RoundArgs ra;
    ra.n = (unsigned)n;
    ra.nr = (unsigned)nr;
    ra.kpc = (unsigned)sl.kp;
    ra.ppm1 = (unsigned)(ppr - 1);
    ra.hb = lds_addr(h);
    ra.pa = lds_addr(kind_part(part, fresh(*st.P).psum_off[kind]) + sl.row * 8 + st.cw);
    const bool more = n > kRing;
    ra.ikp = more ? (unsigned)st.kp : 0u;
    ra.ileft = more ? (unsigned)st.left : 0u;
    ra.ip = reinterpret_cast<unsigned long long>(more ? st.ptr : st.dummy);
    ra.dummy = reinterpret_cast<unsigned long long>(st.dummy);
    ra.adv = (unsigned long long)st.adv_last;
    ra.tm = tailv >= 64 ? ~0ull : ((1ull << tailv) - 1ull);
    ra.loff = (unsigned)(lane * 16);
    ra.toff = (unsigned)(min(lane, tailv - 1) * 16);
    stream_rounds(ra, acc);
    if (more) {   // the rounds issued the rest of this phase's pieces
      st.left = 0;
      st.pad = 0;
      st.next_phase_if_done();
    }
    lds_drain();
    trace_at(*st.P, trk, 5);
    if (lane == 0) lds_st(&ctl->done[st.cw], (unsigned)(q + 1));
    if (!defer_last_refill) st.refill();   // else the caller refills (st.refill()) later
  }
  if (nr == 0 && lane == 0) lds_st(&ctl->done[st.cw], (unsigned)(q + 1));
  if (timed) {
    st.t_work += now_ticks() - t0;
    st.pieces += (unsigned long long)n;
  }
  return true;
}

// ---------------------------------------------------------------- sync-wave phase pieces

// Sum of the stream waves' partials of one row, in wave order: the row's eight
// partial slots are read at once.  Each phase kind has its own slots, zeroed
// when the kernel starts, and the partition of a kind among the stream waves
// is fixed for the launch: a slot of a wave that does not touch the row is
// never written and stays zero, so no slot needs a check.
__device__ __forceinline__ float row_value(const float *part, int row) {
  const float4 p0 = reinterpret_cast<const float4 *>(part + row * 8)[0];
  const float4 p1 = reinterpret_cast<const float4 *>(part + row * 8)[1];
  return ((((((p0.x + p0.y) + p0.z) + p0.w) + p1.x) + p1.y) + p1.z);
}


// Wave 0: wait until every stream wave finished GEMV phase q.  Returns false
// if the abort flag is set instead: a stream wave leaves the kernel only after
// setting or seeing it (a bounded wait of its own expired), so it may never
// report the phase done.
__device__ __forceinline__ bool wait_streams(const Ctl *ctl, int q) {
  for (;;) {
    const bool behind = lane_id() < kNcw && lds_ld(&ctl->done[lane_id()]) < (unsigned)(q + 1);
    if (wave_none(behind)) break;
    if (lds_ld(&ctl->abort)) return false;
    __builtin_amdgcn_s_sleep(1);
  }
  asm volatile("" ::: "memory");
  return true;
}


// ---------------------------------------------------------------- attention

// The cached keys attended at position pos are [kb, pos) (kb = 0, or the
// window's first key pos - W + 1); the key at pos itself comes from the QKV
// phase's tagged words.  The cached keys lie in tiles t0 .. t0 + nt - 1 of
// kKvTile positions, split into S units of at most tpu consecutive tiles (unit
// c takes tiles from t0 + c tpu): one unit per KV head while its nt tiles are
// at most ut (at most kNcw: one tile per stream wave), so no merge; past that
// ceil(nt / us) units, at most G / Hkv and kMaxSplit.  A head that is split
// anyway gains from short units (a CU keeps only ~60 KB of loads in flight, so
// a unit's load time grows with its tiles), while one that fits in one unit
// would pay a merge exchange to split.  Unit 0 also takes the current key.
// A KV head that fits in one unit is further split by query heads (qs, GQA):
// Q units of qpg / Q query heads each read the same tiles, so a wave scores one
// query head instead of qpg, while enough workgroups are left (2 Hkv qpg <= G).
// Units: H = Hkv Q "unit heads" (unit head v: KV head v / Q, query heads
// v qpg / Q ..), S chunks each; unit u is (v, c) = (u mod H, u / H).
struct AttnPart {
  int S, tpu, t0, nt, kb, Q, H;
};
__device__ __forceinline__ AttnPart attn_part(int kb, int pos, int G, int Hkv, int qpg, int qs, int ut, int us) {
  AttnPart a;
  a.kb = kb;
  int smax = G / Hkv;
  if (smax > kMaxSplit) smax = kMaxSplit;
  if (smax < 1) smax = 1;
  if (pos > kb) {
    a.t0 = kb / kKvTile;
    a.nt = (pos - 1) / kKvTile - a.t0 + 1;
    int S = a.nt <= ut ? 1 : (a.nt + us - 1) / us;
    if (S > smax) S = smax;
    a.tpu = (a.nt + S - 1) / S;
    a.S = (a.nt + a.tpu - 1) / a.tpu;   // no unit is left without tiles
  } else {
    a.t0 = a.nt = a.tpu = 0;
    a.S = 1;
  }
  a.Q = qs && a.S == 1 && qpg > 1 && 2 * Hkv * qpg <= G ? qpg : 1;
  a.H = Hkv * a.Q;
  return a;
}

// r = hd * dh + rem: shifts and masks when dh is a power of two (a uniform
// branch), a division otherwise (head_dim 96).
__device__ __forceinline__ void head_split(int r, int dh, int &hd, int &rem) {
  if ((dh & (dh - 1)) == 0) {
    hd = r >> __builtin_ctz((unsigned)dh);
    rem = r & (dh - 1);
  } else {
    hd = r / dh;
    rem = r - hd * dh;
  }
}

// Whether layer l attends over a sliding window (bit l of the window mask).
__device__ __forceinline__ bool layer_windowed(const KP &P, int l) {
  return P.window > 0 && l < 64 && ((P.window_layers >> l) & 1ull);
}

// The attention split of one position for full layers ([0]) and windowed
// layers ([1]).
struct AttnSplit {
  AttnPart a[2];
  __device__ __forceinline__ AttnSplit(const KP &P, int pos, int G) {
    const int n = pos + 1, W = P.window;
    a[0] = attn_part(0, pos, G, P.Hkv, P.qpg, P.attn_qsplit, P.attn_unit_tiles, P.attn_split_tiles);
    a[1] = attn_part(W > 0 && n > W ? n - W : 0, pos, G, P.Hkv, P.qpg, P.attn_qsplit, P.attn_unit_tiles,
                     P.attn_split_tiles);
  }
};

// A buffer resource over `bytes` bytes from p: loads past the end return zero.
typedef __amdgpu_buffer_rsrc_t Rsrc;
__device__ __forceinline__ Rsrc make_rsrc(const void *p, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}
// 16 bytes of a KV tile run at byte offset off, device-scope (sc1) and
// non-temporal (nt).  A line of a tile also holds positions that are written
// after an earlier step has read the line, so the load must not be served from
// a copy this XCD's L2 kept from that earlier read.
#ifndef LF_KV_AUX
#define LF_KV_AUX (16 | 2)
#endif
__device__ __forceinline__ u32x4 kv_load(Rsrc r, unsigned off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, LF_KV_AUX);
}

// Barrier of the seven stream waves (the sync wave takes no part in attention):
// each wave completes its LDS accesses, counts itself in, and waits until the
// count reaches the next multiple of kNcw.  No wave waits for its global stores.
__device__ __forceinline__ void stream_barrier(Ctl *ctl) {
  lds_drain();
  unsigned old = 0u;
  if (lane_id() == 0)
    old = __hip_atomic_fetch_add(&ctl->abar, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  old = __builtin_amdgcn_readfirstlane(old);
  const unsigned target = (old / kNcw + 1u) * kNcw;
  while (lds_ld(&ctl->abar) < target && !lds_ld(&ctl->abort)) __builtin_amdgcn_s_sleep(0);
  asm volatile("" ::: "memory");
}

// K/V tile prefetch.  The cached tiles of a unit do not depend on the step's
// queries, so a workgroup that runs attention and streams no QKV rows copies
// each of its first P.kv_pf stream waves' first tile into LDS during the QKV
// phase (direct-to-LDS loads, device-scope and non-temporal like kv_load): K
// pieces 0 .. dh/8-1, then V pieces (key group kg, half hh) at dh/8 + kg nvh + hh,
// each holding what lane i of that wave's tile load would hold.
__device__ __forceinline__ bool kv_pf_wave(const KP &P, const Ctl *ctl, int u, int kwv, int tfirst, int te) {
  return P.kv_pf > 0 && P.qpg <= 4 && u == (int)blockIdx.x && u < ctl->na && kwv < P.kv_pf && tfirst < te;
}
__device__ __forceinline__ unsigned char *kv_pf_area(const KP &P, int kwv) {
  extern __shared__ __align__(16) unsigned char lf_dyn_lds[];
  return lf_dyn_lds + P.lds_kvpf + (size_t)kwv * P.kv_pf_tile;
}
__device__ __forceinline__ void kv_prefetch(KP &P, const Ctl *ctl, int l, int u, const AttnPart &ap, int kwv) {
  const int Hkv = P.Hkv, dh = P.dh;
  const int g = u % Hkv, c = u / Hkv;
  const int ta = ap.t0 + c * ap.tpu;
  const int te = min(ta + ap.tpu, ap.t0 + ap.nt);
  const int t = ta + kwv;
  if (!kv_pf_wave(P, ctl, u, kwv, t, te)) return;
  const int lane = lane_id();
  const int nck = dh >> 3, nvh = (dh + 63) >> 6;
  const size_t tile_b = (size_t)128 * dh;
  const size_t off = (((size_t)l * Hkv + g) * P.kv_tiles + (size_t)t) * tile_b;
  const unsigned char *kb = reinterpret_cast<const unsigned char *>(P.kcache) + off;
  const unsigned char *vb = reinterpret_cast<const unsigned char *>(P.vcache) + off;
  unsigned char *dst = kv_pf_area(P, kwv);
  for (int k = 0; k < nck; ++k)
    __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1))) *)(kb + k * 1024 + lane * 16),
                                     (void __attribute__((address_space(3))) *)(dst + k * 1024), 16, 0, 16 | 2);
  for (int kg = 0; kg < 8; ++kg)
    for (int hh = 0; hh < nvh; ++hh)
      __builtin_amdgcn_global_load_lds(
          (const void __attribute__((address_space(1))) *)(vb + (size_t)(kg * dh + min(hh * 64 + lane, dh - 1)) * 16),
          (void __attribute__((address_space(3))) *)(dst + (nck + kg * nvh + hh) * 1024), 16, 0, 16 | 2);
}

// Lanes 2i of the result hold the fp16 pair (x of lane 2i, x of lane 2i + 1).
__device__ __forceinline__ unsigned pair_up(_Float16 x) {
  const unsigned lo = (unsigned)__builtin_bit_cast(unsigned short, x);
  const unsigned hi = (unsigned)__builtin_amdgcn_update_dpp(0, (int)lo, 0xF5, 0xf, 0xf, false);   // quad_perm [1,1,3,3]
  return lo | (hi << 16);
}

// fp16 pair m (elements 2m, 2m + 1) of a 16-byte vector.
__device__ __forceinline__ f16x2 pair_of(u32x4 w, int m) {
  const f16x8 a = __builtin_bit_cast(f16x8, w);
  switch (m) {
    case 0: return __builtin_shufflevector(a, a, 0, 1);
    case 1: return __builtin_shufflevector(a, a, 2, 3);
    case 2: return __builtin_shufflevector(a, a, 4, 5);
    default: return __builtin_shufflevector(a, a, 6, 7);
  }
}

// One split-K unit (KV head g, tile chunk c) of layer l at position pos, run by
// the seven stream waves.  These are the pages' three attention stages ("The
// fused operations, briefly"): attention over one run of cache tiles per unit,
// the cross-unit softmax correction, then (next phase) the output projection.
//
// Stream wave w takes the unit's tiles w - 1, w + 6, ...; its first tile's K and
// V pieces are requested before the queries are awaited.  The waves that hold
// no tile poll the queries (a wave's loads complete in order, so behind 32 KB
// of tile pieces a poll would wait for them) into the unit's own LDS area.
// Scores: lane j holds key j of the tile (K tile layout); the query sits in one
// register per head, lane i holding its dim pair i, and each pair reaches every
// lane by v_readlane, so a score is 64 dot2 products with no cross-lane sum
// and no LDS access; the tile's maximum is one wave reduction.  The fp16
// softmax weights are paired by one DPP move and read the same way, and lane e
// accumulates output dims e and e + 64 as dot2 products of its V pieces (one
// dim of 8 keys, V tile layout).  Each wave keeps an online softmax (m, l, o)
// per query head.  Wave 1 combines the waves' states into the unit's partial
// (tagged words), and in unit c = 0 of each KV head the waves merge the group's
// S partials (waiting on their tags) into the fp16 output o_t.  The current
// position's K/V row comes from the tagged exchange words, not from the cache
// (whose row for this step may still be in flight); the last stream wave of
// unit 0 folds it in.  Returns false if a bounded wait expired.
// kQ: a bound on the query heads per KV head (qpg <= kQ), so that an MHA
// model's unit keeps one head's state in registers and no loop over heads.
template <int kQ>
__device__ __forceinline__ bool attn_unit(KP &P0, Ctl *ctl, int l, int gen, unsigned tag_q, unsigned tag_a, int pos,
                                          int u, const AttnPart &ap, unsigned char *lds, int trk = -1) {
  static_assert(kQ <= kMaxQpg, "query heads per KV head");
  KP &P = fresh(P0);
  const int wave = wave_id(), lane = lane_id();
  if (kTrace && wave == 1) trace_at(P, trk, 8);
  const int dh = P.dh, Hkv = P.Hkv, half = dh / 2;
  const int S = ap.S;
  const int qpg = P.qpg / ap.Q;                      // this unit's query heads
  const int vg = u % ap.H, c = u / ap.H;             // chunk c = 0 of unit head vg runs on workgroup vg
  const int g = vg / ap.Q;                           // its KV head
  const AttnLds al = attn_lds(qpg, dh);
  _Float16 *q16 = reinterpret_cast<_Float16 *>(lds + al.q16);   // [qpg][dh]
  float *kcur = reinterpret_cast<float *>(lds + al.kcur);        // [dh]
  float *vcur = reinterpret_cast<float *>(lds + al.vcur);        // [dh]
  float *wml = reinterpret_cast<float *>(lds + al.wml);          // [kWaves][kMaxQpg][2] per-wave (m, l)
  float *wo = reinterpret_cast<float *>(lds + al.wo);            // [kWaves][qpg][dh] per-wave o
  const unsigned long long t0 = now_ticks();
  bool bad = false;
  constexpr int kKW = kNcw;
  const int kwv = wave - 1;
  const int ta = ap.t0 + c * ap.tpu;                   // this unit's tiles [ta, te)
  const int te = min(ta + ap.tpu, ap.t0 + ap.nt);
  const int tfirst = ta + kwv;
  const int nck = dh >> 3;              // K pieces per tile
  const int nvh = (dh + 63) >> 6;       // V pieces per key group
  const unsigned tile_b = (unsigned)(128 * dh);
  const size_t run_b = (size_t)P.kv_tiles * tile_b;
  const size_t run0 = ((size_t)l * Hkv + g) * run_b;
  const Rsrc rk = make_rsrc(reinterpret_cast<const char *>(P.kcache) + run0, (unsigned)run_b);
  const Rsrc rv = make_rsrc(reinterpret_cast<const char *>(P.vcache) + run0, (unsigned)run_b);
  // K piece k of a tile: 16 bytes per lane at k KB + 16 lane.  V piece (kg, hh):
  // dim hh * 64 + lane of key group kg (lanes past head_dim re-read its last dim)
  const unsigned koff = (unsigned)lane * 16u;
  const unsigned voff0 = (unsigned)min(lane, dh - 1) * 16u;
  const unsigned voff1 = (unsigned)min(64 + lane, dh - 1) * 16u;
  // With more than four query heads per KV head the V pieces are requested once
  // the scores are done (in the K pieces' registers), so that the heads' states
  // fit without spilling.
  constexpr bool kPreV = kQ <= 4;
  u32x4 kr[16], vr[8][2];
  auto load_v = [&](int t) __attribute__((always_inline)) {
    const unsigned tb = (unsigned)t * tile_b;
#pragma unroll
    for (int kg = 0; kg < 8; ++kg) {
      const unsigned gb = tb + (unsigned)(kg * dh * 16);
      vr[kg][0] = kv_load(rv, gb + voff0);
      if (nvh > 1) vr[kg][1] = kv_load(rv, gb + voff1);
    }
  };
  auto load_tile = [&](int t) __attribute__((always_inline)) {
    const unsigned tb = (unsigned)t * tile_b;
#pragma unroll
    for (int k = 0; k < 16; ++k)
      if (k < nck) kr[k] = kv_load(rk, tb + (unsigned)k * 1024u + koff);
    if (kPreV) load_v(t);
  };
  if (kTrace && wave == 1) trace_at(P, trk, 6);
  // The first tile, when it was prefetched into LDS during the QKV phase (only
  // with V requested up front: the other variant has no registers to spare).
  if (kPreV && kv_pf_wave(P, ctl, u, kwv, tfirst, te)) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the direct-to-LDS loads have landed
    const unsigned char *pft = kv_pf_area(P, kwv) + lane * 16;
#pragma unroll
    for (int k = 0; k < 16; ++k)
      if (k < nck) kr[k] = *reinterpret_cast<const u32x4 *>(pft + k * 1024);
#pragma unroll
    for (int kg = 0; kg < 8; ++kg) {
      vr[kg][0] = *reinterpret_cast<const u32x4 *>(pft + (nck + kg * nvh) * 1024);
      if (nvh > 1) vr[kg][1] = *reinterpret_cast<const u32x4 *>(pft + (nck + kg * nvh + 1) * 1024);
    }
  } else if (tfirst < te) {
    if (kTrace && wave == 1) trace_at(P, trk, 2);
    load_tile(tfirst);
  }
  if (kTrace && wave == 1) trace_at(P, trk, 0);
  {
    // The queries (to fp16) and, in unit 0, the current K and V pairs: one
    // tagged word each, polled by the stream waves that hold no tile (with a
    // tile in every wave, all of them).  Each thread requests up to four words
    // at once and re-reads the stale ones.
    const u64 *qsrc = P.q_t + (size_t)gen * P.Hq * dh + (size_t)vg * qpg * dh;
    const size_t nw = (size_t)Hkv * half;
    const int nq = qpg * dh;
    const int nwords = nq + (c == 0 ? dh : 0);
    const int busy = min(te - ta, kKW);                  // stream waves holding a tile
    const int p0 = busy < kKW ? busy : 0;                // first polling stream wave
    const int npt = (kKW - p0) * 64;                     // polling threads
    const int me = kwv - p0;
    auto word = [&](int i) __attribute__((always_inline)) -> const u64 * {
      if (i < nq) return qsrc + i;
      if (i < nq + half) return P.kc_t + gen * nw + (size_t)g * half + (i - nq);
      return P.vc_t + gen * nw + (size_t)g * half + (i - nq - half);
    };
    if (me >= 0) {
      for (int i0 = me * 64 + lane; i0 < nwords; i0 += npt * 4) {
        u64 w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int i = i0 + k * npt;
          w[k] = i < nwords ? ld_dev(word(i)) : ((u64)tag_q << 32);
        }
        for (;;) {
          bool stale = false;
#pragma unroll
          for (int k = 0; k < 4; ++k) stale |= tag_of(w[k]) != tag_q;
          if (!stale) break;
          const unsigned e = ld_dev(&P.err[0]);
#pragma unroll
          for (int k = 0; k < 4; ++k)
            if (tag_of(w[k]) != tag_q) w[k] = ld_dev(word(i0 + k * npt));
          if (expired(P, t0, tag_q, e)) {
            bad = true;
            break;
          }
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int i = i0 + k * npt;
          if (i >= nwords) continue;
          if (i < nq) {
            q16[i] = (_Float16)pay_f(w[k]);
          } else if (i < nq + half) {   // a K word pairs dims (e, e + dh/2)
            const f16x2 hv = __builtin_bit_cast(f16x2, (unsigned)w[k]);
            kcur[i - nq] = (float)hv.x;
            kcur[i - nq + half] = (float)hv.y;
          } else {                      // a V word pairs dims (2e, 2e + 1)
            const int e = i - nq - half;
            const f16x2 hv = __builtin_bit_cast(f16x2, (unsigned)w[k]);
            vcur[2 * e] = (float)hv.x;
            vcur[2 * e + 1] = (float)hv.y;
          }
        }
      }
    }
    if (bad) lds_st(&ctl->abort, 1u);
  }
  if (kTrace && wave == kWaves - 1) trace_at(P, trk, 1);
  stream_barrier(ctl);
  if (lds_ld(&ctl->abort)) return false;
  const int trw = wave == 1 ? trk : -1;
  trace_at(P, trw, 3);

  const float scale = P.inv_sqrt_dh;
  float m[kQ], ls[kQ], o0[kQ], o1[kQ];
  unsigned qv[kQ];   // lane i: the fp16 query pair (2i, 2i + 1) of head h
#pragma unroll
  for (int h = 0; h < kQ; ++h) {
    m[h] = -INFINITY;
    ls[h] = o0[h] = o1[h] = 0.0f;
    qv[h] = h < qpg && lane < half ? reinterpret_cast<const unsigned *>(q16 + h * dh)[lane] : 0u;
  }
  for (int t = tfirst; t < te; t += kKW) {
    if (t != tfirst) load_tile(t);
    const int j = t * kKvTile + lane;
    const bool valid = j >= ap.kb && j < pos;
    unsigned pp[kQ];   // even lanes: fp16 softmax weights of keys (lane, lane + 1)
    // scores and the online-softmax update (every tile of the run holds at
    // least one cached key, so the new maximum is finite)
#pragma unroll
    for (int h = 0; h < kQ; ++h) {
      if (h < qpg) {
        float s = 0.0f;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          if (k < nck) {
#pragma unroll
            for (int mm = 0; mm < 4; ++mm) {
              const unsigned q2 = (unsigned)__builtin_amdgcn_readlane((int)qv[h], 4 * k + mm);
              s = __builtin_amdgcn_fdot2(pair_of(kr[k], mm), __builtin_bit_cast(f16x2, q2), s, false);
            }
          }
        }
        s = valid ? s * scale : -INFINITY;
        const float mn = fmaxf(m[h], wave_max(s));
        const float alpha = __expf(m[h] - mn);   // 0 while m is -inf
        const _Float16 ph = (_Float16)__expf(s - mn);
        ls[h] = ls[h] * alpha + (float)ph;
        o0[h] *= alpha;
        o1[h] *= alpha;
        m[h] = mn;
        pp[h] = pair_up(ph);
      }
    }
    if (kTrace && wave == 1 && t == tfirst) trace_at(P, trk, 10);
    if (!kPreV) load_v(t);
    // weights x V: lane e accumulates dims e and e + 64 over the tile's keys
#pragma unroll
    for (int h = 0; h < kQ; ++h) {
      if (h < qpg) {
#pragma unroll
        for (int kg = 0; kg < 8; ++kg) {
#pragma unroll
          for (int mm = 0; mm < 4; ++mm) {
            const f16x2 w2 = __builtin_bit_cast(f16x2, (unsigned)__builtin_amdgcn_readlane((int)pp[h], 8 * kg + 2 * mm));
            o0[h] = __builtin_amdgcn_fdot2(pair_of(vr[kg][0], mm), w2, o0[h], false);
            if (nvh > 1) o1[h] = __builtin_amdgcn_fdot2(pair_of(vr[kg][1], mm), w2, o1[h], false);
          }
        }
      }
    }
  }
  if (c == 0 && wave == kWaves - 1) {
    // the current key, from the staged tagged words (its weight rounded to fp16
    // like every cached key's)
    const int e2 = lane < half ? 2 * lane : 0;
#pragma unroll
    for (int h = 0; h < kQ; ++h) {
      if (h < qpg) {
        const _Float16 *qh = q16 + h * dh;
        const float x = lane < half ? (float)qh[e2] * kcur[e2] + (float)qh[e2 + 1] * kcur[e2 + 1] : 0.0f;
        const float s = wave_sum(x) * scale;
        const float mn = fmaxf(m[h], s);
        const float alpha = __expf(m[h] - mn);
        const float p = (float)(_Float16)__expf(s - mn);
        ls[h] = ls[h] * alpha + (lane == 0 ? p : 0.0f);
        o0[h] = o0[h] * alpha + p * vcur[min(lane, dh - 1)];
        o1[h] = o1[h] * alpha + (nvh > 1 ? p * vcur[min(64 + lane, dh - 1)] : 0.0f);
        m[h] = mn;
      }
    }
  }
  trace_at(P, trw, 4);
  // the waves' states -> LDS (a wave without keys leaves m = -inf, l = 0)
#pragma unroll
  for (int h = 0; h < kQ; ++h) {
    if (h < qpg) {
      const float lt = wave_sum(ls[h]);
      if (lane == 0) {
        wml[(wave * kMaxQpg + h) * 2 + 0] = m[h];
        wml[(wave * kMaxQpg + h) * 2 + 1] = lt;
      }
      float *ow = wo + (size_t)(wave * qpg + h) * dh;
      if (lane < dh) ow[lane] = o0[h];
      if (64 + lane < dh) ow[64 + lane] = o1[h];
    }
  }
  // (taken before the barrier: none of it depends on the other waves)
  const bool act = lane < half;   // lane holds output dims 2 lane, 2 lane + 1
  const int e0 = act ? 2 * lane : 0;
  const int stride = dh + 2;
  gu64 *pg = (gu64 *)(P.part_t + (size_t)gen * P.part_gen);
  gu64 *o_out = (gu64 *)(P.o_t + (size_t)gen * (P.Hq * dh / 2) + ((size_t)vg * qpg * dh + e0) / 2);
  asm volatile("" : "+s"(pg), "+v"(o_out));
  // Wave 1: combine the stream waves' states of head h (m, l, o for this lane's
  // two dims) left in wml / wo.  Every read is in bounds for every lane (e0 = 0
  // on lanes past the head dims), so the seven states load together.
  auto combine = [&](int h, float &M, float &Ls, float &a0, float &a1) __attribute__((always_inline)) {
    float mw[kKW], lw[kKW];
    float2 ow[kKW];
#pragma unroll
    for (int w = 0; w < kKW; ++w) {
      mw[w] = wml[((w + 1) * kMaxQpg + h) * 2];
      lw[w] = wml[((w + 1) * kMaxQpg + h) * 2 + 1];
      ow[w] = *reinterpret_cast<const float2 *>(&wo[((w + 1) * qpg + h) * dh + e0]);
    }
    M = mw[0];
#pragma unroll
    for (int w = 1; w < kKW; ++w) M = fmaxf(M, mw[w]);
    Ls = a0 = a1 = 0.0f;
#pragma unroll
    for (int w = 0; w < kKW; ++w) {
      const float sw = mw[w] == -INFINITY ? 0.0f : __expf(mw[w] - M);
      Ls += sw * lw[w];
      a0 += sw * ow[w].x;
      a1 += sw * ow[w].y;
    }
  };
  stream_barrier(ctl);
  if (wave == 1) {
    trace_at(P, trw, 9);
    gu64 *dst = pg + (size_t)(vg * S + c) * qpg * stride;   // partials of unit head vg in chunk order
    for (int h = 0; h < qpg; ++h) {
      float M, Ls, a0, a1;
      combine(h, M, Ls, a0, a1);
      if (S == 1) {
        // the unit holds every key of the head: its state is the head's output
        if (act) {
          const float il = 1.0f / Ls;
          st_tag(o_out + (size_t)h * dh / 2, tag_h2(a0 * il, a1 * il, tag_a));
        }
        continue;
      }
      if (act) {
        st_tag(&dst[h * stride + 2 + e0], tag_f(a0, tag_a));
        st_tag(&dst[h * stride + 2 + e0 + 1], tag_f(a1, tag_a));
      }
      if (lane == 0) {
        st_tag(&dst[h * stride + 0], tag_f(M, tag_a));
        st_tag(&dst[h * stride + 1], tag_f(Ls, tag_a));
      }
    }
    trace_at(P, trw, 5);
  }
  if (c == 0 && S > 1) {
    // The merging unit (c = 0 of each KV head), all stream waves.  Stream wave w polls
    // chunks w - 1, w + 6, ... of the group (their (m, l) and this lane's two o
    // dims, up to four chunks' words in flight at once, each pass re-reading
    // every stale word: one round trip per pass), folds them into one online
    // softmax state per head and leaves it in wml / wo; wave 1 then combines
    // the seven states into the head's output.
    stream_barrier(ctl);   // wave 1 has read the unit's own states: wml / wo are free
    if (wave == 1) trace_at(P, trw, 11);
    {
      const gu64 *src = pg + (size_t)vg * S * qpg * stride;
      const u64 tagw = (u64)tag_a << 32;
      for (int h = 0; h < qpg; ++h) {
        float M = -INFINITY, Ls = 0.0f, a0 = 0.0f, a1 = 0.0f;
        for (int cb = kwv; cb < S; cb += 4 * kKW) {
          u64 w[4][4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bool use = cb + kKW * i < S;
            const gu64 *q = src + ((size_t)(cb + kKW * i) * qpg + h) * stride;
            w[i][0] = use ? ld_dev(q) : tagw;
            w[i][1] = use ? ld_dev(q + 1) : tagw;
            w[i][2] = use ? ld_dev(q + 2 + e0) : tagw;
            w[i][3] = use ? ld_dev(q + 3 + e0) : tagw;
          }
          for (;;) {
            // (words not read carry the tag already, so they are never stale)
            bool stale = false;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
              for (int k = 0; k < 4; ++k) stale |= tag_of(w[i][k]) != tag_a;
            if (wave_none(stale)) break;
            const unsigned e = ld_dev(&P.err[0]);
            // (addresses recomputed here, not held across the loop)
            const gu64 *pb = src + ((size_t)cb * qpg + h) * stride;
            asm volatile("" : "+v"(pb));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const gu64 *q = pb + (size_t)kKW * i * qpg * stride;
              if (tag_of(w[i][0]) != tag_a) w[i][0] = ld_dev(q);
              if (tag_of(w[i][1]) != tag_a) w[i][1] = ld_dev(q + 1);
              if (tag_of(w[i][2]) != tag_a) w[i][2] = ld_dev(q + 2 + e0);
              if (tag_of(w[i][3]) != tag_a) w[i][3] = ld_dev(q + 3 + e0);
            }
            if (expired(P, t0, tag_a, e)) {
              bad = true;
              break;
            }
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (cb + kKW * i < S) {
              const float mc = pay_f(w[i][0]);
              const float Mn = fmaxf(M, mc);
              const float sa = M == -INFINITY ? 0.0f : __expf(M - Mn);
              const float sb = mc == -INFINITY ? 0.0f : __expf(mc - Mn);
              Ls = Ls * sa + pay_f(w[i][1]) * sb;
              a0 = a0 * sa + pay_f(w[i][2]) * sb;
              a1 = a1 * sa + pay_f(w[i][3]) * sb;
              M = Mn;
            }
          }
        }
        if (lane == 0) {
          wml[(wave * kMaxQpg + h) * 2 + 0] = M;
          wml[(wave * kMaxQpg + h) * 2 + 1] = Ls;
        }
        if (act) *reinterpret_cast<float2 *>(&wo[(wave * qpg + h) * dh + e0]) = make_float2(a0, a1);
      }
      if (bad && lane == 0) lds_st(&ctl->abort, 1u);
    }
    stream_barrier(ctl);
    if (wave == 1) {
      if (trw >= 0) trace_at(P, trw, 12);
      for (int h = 0; h < qpg; ++h) {
        float M, Ls, a0, a1;
        combine(h, M, Ls, a0, a1);
        if (act) {
          const float il = 1.0f / Ls;
          st_tag(o_out + (size_t)h * dh / 2, tag_h2(a0 * il, a1 * il, tag_a));
        }
      }
      trace_at(P, trw, 13);
    }
  }
  stream_barrier(ctl);
  return !lds_ld(&ctl->abort);
}

// The kernel is instantiated per attention variant (kQ: the query heads per KV
// head rounded up to 1, 2, 4 or 8), so each holds one copy of the unit: the
// largest variant's registers would otherwise set every model's spills.
__host__ __device__ constexpr int kq_of(int qpg) { return qpg <= 1 ? 1 : qpg == 2 ? 2 : qpg <= 4 ? 4 : kMaxQpg; }

// ---------------------------------------------------------------- sampler

// Defined exponential for x <= 0, bit-identical on any IEEE machine: k = rint(x
// log2 e); r = x - k ln2 by a two-constant Cody-Waite step with fma; degree-7
// Taylor polynomial of e^r (Horner, fma); scale by 2^k.  Constants are the
// nearest binary32 values of log2(e), ln 2, (ln 2 - that value) and 1/n!.
__device__ __forceinline__ float expdef(float x) {
#pragma clang fp contract(off)
  const float k = __builtin_rintf(x * 0x1.715476p+0f);
  float r = __builtin_fmaf(-k, 0x1.62e430p-1f, x);
  r = __builtin_fmaf(-k, -0x1.05c610p-29f, r);
  float p = 0x1.a01a02p-13f;
  p = __builtin_fmaf(p, r, 0x1.6c16c2p-10f);
  p = __builtin_fmaf(p, r, 0x1.111112p-7f);
  p = __builtin_fmaf(p, r, 0x1.555556p-5f);
  p = __builtin_fmaf(p, r, 0x1.555556p-3f);
  p = __builtin_fmaf(p, r, 0x1.0p-1f);
  p = __builtin_fmaf(p, r, 1.0f);
  p = __builtin_fmaf(p, r, 1.0f);
  return __builtin_ldexpf(p, (int)k);
}

// Philox4x32-10 (Salmon et al., SC'11): 10 rounds, key bumped by the Weyl
// constants between rounds.
__device__ __forceinline__ void philox4x32_10(unsigned c[4], unsigned k0, unsigned k1) {
  for (int round = 0; round < 10; ++round) {
    if (round > 0) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
    const unsigned hi0 = __umulhi(0xD2511F53u, c[0]), lo0 = 0xD2511F53u * c[0];
    const unsigned hi1 = __umulhi(0xCD9E8D57u, c[2]), lo1 = 0xCD9E8D57u * c[2];
    const unsigned n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0; c[1] = lo1; c[2] = n2; c[3] = lo0;
  }
}

// Defined natural logarithm of a positive normal x, the same bits on any
// IEEE-754 machine (each step one correctly rounded operation or one fma):
// x = m 2^e with m in [sqrt(1/2), sqrt(2)), f = m - 1 (exact), s = f / (2 + f),
// ln(1 + f) = 2 atanh(s) = 2s + 2s (w/3 + w^2/5 + ... + w^6/13) with w = s^2,
// plus e ln 2 split into a binary32 high part and the rounded remainder.
__device__ __forceinline__ float logdef(float x) {
#pragma clang fp contract(off)
  const unsigned bits = __float_as_uint(x);
  int e = (int)(bits >> 23) - 127;
  float m = __uint_as_float((bits & 0x7fffffu) | 0x3f800000u);
  if (m > 0x1.6a09e6p+0f) {
    m = m * 0.5f;
    e += 1;
  }
  const float f = m - 1.0f;
  const float s = __fdiv_rn(f, 2.0f + f);
  const float w = s * s;
  float r = 0x1.3b13b2p-4f;                  // 1/13
  r = __builtin_fmaf(r, w, 0x1.745d18p-4f);  // 1/11
  r = __builtin_fmaf(r, w, 0x1.c71c72p-4f);  // 1/9
  r = __builtin_fmaf(r, w, 0x1.24924ap-3f);  // 1/7
  r = __builtin_fmaf(r, w, 0x1.99999ap-3f);  // 1/5
  r = __builtin_fmaf(r, w, 0x1.555556p-2f);  // 1/3
  r = r * w;
  const float s2 = s + s;
  const float ef = (float)e;
  return __builtin_fmaf(ef, 0x1.62e430p-1f, __builtin_fmaf(ef, -0x1.05c610p-29f, __builtin_fmaf(s2, r, s2)));
}

// Gumbel noise of vocabulary entry i at RNG counter pos: the first word x0 of
// the Philox4x32-10 block with counter (pos, i, 1, 0) (the nucleus draw uses
// (pos, 0, 0, 0)), u = (2 (x0 >> 9) + 1) 2^-24 strictly inside (0, 1) and exact
// in binary32, g = -ln(-ln u) with the defined logarithm.
__device__ __forceinline__ float gumbel_noise(unsigned long long seed, int pos, int i) {
  unsigned c[4] = {(unsigned)pos, (unsigned)i, 1u, 0u};
  philox4x32_10(c, (unsigned)(seed & 0xffffffffull), (unsigned)(seed >> 32));
  const float u = (float)(2u * (c[0] >> 9) + 1u) * 0x1.0p-24f;
  return -logdef(-logdef(u));
}

// Gumbel-max score of one logit ("KOG LaneFormer-2B & the monokernel", "The
// fused operations, briefly"): z + g with z = logit * (1/T), one rounded
// product and one rounded sum.  The token is the argmax of the scores (lowest
// index among equal maxima): a draw from softmax(z) without normalising it.
__device__ __forceinline__ float gumbel_score(float logit, float inv_temp, unsigned long long seed, int pos,
                                              int i) {
#pragma clang fp contract(off)
  const float z = logit * inv_temp;
  return z + gumbel_noise(seed, pos, i);
}

// Plain loads: the caller has taken an agent-scope acquire fence after the
// logits were published, so this XCD's caches hold no stale copy of them, and
// the sampler's repeated passes then hit in L2.
__device__ __forceinline__ float scale_logit(float logit, float inv_temp) {
#pragma clang fp contract(off)
  float z = logit * inv_temp;
  return z == 0.0f ? 0.0f : z;   // one zero: -0 and +0 order as equal
}
__device__ __forceinline__ float scaled_logit(const float *logits, int i, float inv_temp) {
  return scale_logit(logits[i], inv_temp);
}

__device__ __forceinline__ unsigned long long mass_of(float z, float zmax) {
#pragma clang fp contract(off)
  const float dz = z - zmax;
  if (dz < -23.0f) return 0ull;
  // E(dz) 2^32 lies in [0, 2^32]: truncation to an integer is one u32 conversion
  // below 2^32 (the same value as a u64 one); 2^32 itself (dz = 0) is set apart
  const float v = expdef(dz) * 4294967296.0f;
  return v >= 4294967296.0f ? (1ull << 32) : (unsigned long long)(unsigned)v;
}

// Order key: larger key = earlier in (z descending, index ascending) order.
__device__ __forceinline__ unsigned long long order_key(float z, int i) {
  unsigned b = __float_as_uint(z);
  b = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((unsigned long long)b << 32) | (unsigned long long)(0xffffffffu - (unsigned)i);
}

// Nucleus draw scratch.  Pass 1 histograms the positive masses over 256 bins of
// d = z* - z (a monotone function of z, so every element of a lower bin comes
// earlier in the (z desc, index asc) order); the bin that holds the nucleus
// boundary is then the only one whose order matters, and its elements (the
// candidates, up to kSampCap) are kept in LDS for the radix select.
constexpr int kSampCap = 2048;
constexpr float kSampBinScale = 256.0f / 24.0f;   // d in [0, 23] -> bins 0 .. 245
#ifndef LF_SAMP_BATCH
#define LF_SAMP_BATCH 32
#endif
constexpr int kSampBatch = LF_SAMP_BATCH;   // rounds whose logits one thread requests at once
struct SampLds {
  // (after the radix select these three arrays, contiguous, hold the segment
  // sums of the token search: up to kSampSegs segments of 64 indices)
  unsigned long long hm[kWaves][kSampBins];   // per-wave bin masses (pass 1)
  unsigned long long ck[kSampCap];            // candidates' order keys
  unsigned long long cq[kSampCap];            // candidates' masses
  unsigned long long mass[256];               // bin totals, then one radix pass's digit masses
  unsigned char cown[kSampCap];               // (the draw over the grid) each candidate's workgroup
  unsigned long long wtot[kWaves];
  unsigned long long sel[4];
  float fred[kWaves];
  int ibc[4];
  unsigned ncand;
};
static_assert(sizeof(SampLds) <= kSampBytes, "nucleus scratch exceeds its LDS space");
static_assert(offsetof(SampLds, ck) == sizeof(unsigned long long) * kWaves * kSampBins &&
                  offsetof(SampLds, cq) == offsetof(SampLds, ck) + sizeof(unsigned long long) * kSampCap &&
                  kWaves * kSampBins + 2 * kSampCap == kSampSegs,
              "segment sums overlay the bin histograms and the candidate list");

__device__ __forceinline__ unsigned long long block_sum_u64(unsigned long long v, SampLds *s) {
  v = wave_sum_u64(v);
  if (lane_id() == 0) s->wtot[wave_id()] = v;
  __syncthreads();
  unsigned long long t = 0;
  for (int w = 0; w < kWaves; ++w) t += s->wtot[w];
  __syncthreads();
  return t;
}

// Bin of a positive-mass element (d = z* - z <= 23).
__device__ __forceinline__ int samp_bin(float z, float zmax) {
#pragma clang fp contract(off)
  const int b = (int)((zmax - z) * kSampBinScale);
  return b < kSampBins - 1 ? b : kSampBins - 1;
}

// Temperature / top-p nucleus sampling with integer masses, by one workgroup:
// z = logit * inv_temp; q_i = floor(E(z_i - z*) * 2^32) (0 below -23); the
// nucleus is the shortest prefix of the (z desc, index asc) order whose mass
// reaches ceil(top_p * C_V) in fp64; the Philox draw t = floor(r * C_N / 2^64)
// with r from counter (pos, 0, 0, 0); the token is the first nucleus member in
// index order whose running mass exceeds t.  Thread t owns indices t + 512 k
// (coalesced reads) and re-reads their logits in each pass.  The boundary is
// found in two steps: the bin histogram gives the boundary bin and the mass of
// the bins before it; an 8-pass radix select on a 64-bit (z, index) order key
// then runs over that bin's candidates only (or, when they do not fit in LDS,
// over every element of the bin).  The token: each wave sums its 64 nucleus
// masses per round k (64 consecutive indices), an exclusive scan over the
// (round, wave) sums in index order finds the segment holding t, and a wave
// scan inside it the index.
// Wave 0: the first entry i of the order i = 0, 1, .. (entry m[desc ? 255 - i : i]
// of 256) at which base + the inclusive sum of the entries reaches need; returns
// its slot in m and, in *before, base + the sum of the entries ahead of it.  Lane
// l holds entries 4l .. 4l + 3 of the order; one 64-bit wave scan of the lane
// totals and a ballot find it.  Falls back to the last entry if none does.
__device__ __forceinline__ int scan_reach(const unsigned long long *m, bool desc, unsigned long long base,
                                          unsigned long long need, unsigned long long *before) {
  const int lane = lane_id();
  unsigned long long e[4], tot = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = 4 * lane + k;
    e[k] = m[desc ? 255 - i : i];
    tot += e[k];
  }
  unsigned long long incl = wave_scan_u64(tot);
  unsigned long long run = base + incl - tot;   // before this lane's first entry
  int hit = -1;
  unsigned long long hb = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (hit < 0 && e[k] > 0 && run + e[k] >= need) {
      hit = 4 * lane + k;
      hb = run;
    }
    run += e[k];
  }
  const unsigned long long mask = __builtin_amdgcn_ballot_w64(hit >= 0);
  int idx;
  unsigned long long bef;
  if (mask) {
    const int src = __builtin_ctzll(mask);
    idx = __builtin_amdgcn_readlane(hit, src);
    bef = ((unsigned long long)(unsigned)__builtin_amdgcn_readlane((int)(hb >> 32), src) << 32) |
          (unsigned)__builtin_amdgcn_readlane((int)(unsigned)hb, src);
  } else {
    // (unreachable for consistent inputs: the entries hold at least need)
    idx = 255;
    bef = base + lane63_u64(incl);
  }
  *before = bef;
  return desc ? 255 - idx : idx;
}

// Temperature / top-p nucleus sampling with integer masses, by one workgroup:
// z = logit * inv_temp; q_i = floor(E(z_i - z*) * 2^32) (0 below -23); the
// nucleus is the shortest prefix of the (z desc, index asc) order whose mass
// reaches ceil(top_p * C_V) in fp64; the Philox draw t = floor(r * C_N / 2^64)
// with r from counter (pos, 0, 0, 0); the token is the first nucleus member in
// index order whose running mass exceeds t.  Thread t owns indices t + 512 k
// (coalesced reads, eight rounds' loads in flight at once) and re-reads their
// logits in each pass.  The boundary is found in two steps: the bin histogram
// gives the boundary bin and the mass of the bins before it; an 8-pass radix
// select on a 64-bit (z, index) order key then runs over that bin's candidates
// only (or, when they do not fit in LDS, over every element of the bin).  The
// token: each wave sums its 64 nucleus masses per round k (64 consecutive
// indices), an exclusive scan over the (round, wave) sums in index order finds
// the segment holding t, and a wave scan inside it the index.
// lm_max (nullable): the n_lm per-workgroup maxima of the logits, from which z*
// is taken (the maximum of the rounded products is the rounded product of the
// maximum) instead of a pass over every logit.
__device__ __forceinline__ int sample_topp(const float *logits, int V, float inv_temp, float top_p,
                                           unsigned long long seed, int pos, SampLds *s,
                                           lds_u64 *tr = nullptr, const float *lm_max = nullptr, int n_lm = 0) {
  const int tid = tid_x(), wave = wave_id(), lane = lane_id();
  auto stamp_at = [&](int j) __attribute__((always_inline)) {   // LF_TRACE builds: stage times
    if (kTrace && tr && tid == 0) tr[j] = now_ticks();
  };
  stamp_at(3);
  const int nr = (V + kThreads - 1) / kThreads;   // rounds
  // body(k, i, z) for every round k (index i) of this thread, kSampBatch rounds'
  // logits requested at once
  auto each = [&](auto &&body) __attribute__((always_inline)) {
    for (int k0 = 0; k0 < nr; k0 += kSampBatch) {
      // (unconditional loads, clamped into range: a guarded load makes the
      // compiler wait for it at the end of its branch)
      float zc[kSampBatch];
#pragma unroll
      for (int u = 0; u < kSampBatch; ++u)
        zc[u] = scaled_logit(logits, min((k0 + u) * kThreads + tid, V - 1), inv_temp);
#pragma unroll
      for (int u = 0; u < kSampBatch; ++u) {
        const int i = (k0 + u) * kThreads + tid;
        if (k0 + u < nr && i < V) body(k0 + u, i, zc[u]);
      }
    }
  };
  float zm = -INFINITY;
  if (lm_max) {
#pragma clang fp contract(off)
    for (int i = tid; i < n_lm; i += kThreads) zm = fmaxf(zm, lm_max[i]);
    zm = zm * inv_temp;
  } else {
    each([&](int, int, float z) __attribute__((always_inline)) { zm = fmaxf(zm, z); });
  }
  zm = wave_max(zm);
  if (lane == 0) s->fred[wave] = zm;
  for (int i = tid; i < kWaves * kSampBins; i += kThreads) (&s->hm[0][0])[i] = 0ull;
  if (tid == 0) s->ncand = 0u;
  __syncthreads();
  float zmax = -INFINITY;
  for (int w = 0; w < kWaves; ++w) zmax = fmaxf(zmax, s->fred[w]);
  stamp_at(4);
  // pass 1: total mass and the per-wave bin histograms of the positive masses
  unsigned long long part = 0;
  each([&](int, int, float z) __attribute__((always_inline)) {
    const unsigned long long q = mass_of(z, zmax);
    part += q;
    if (q) atomicAdd(&s->hm[wave][samp_bin(z, zmax)], q);
  });
  const unsigned long long CV = block_sum_u64(part, s);   // (its barriers also publish the histograms)
  const unsigned long long Mstar = (unsigned long long)ceil((double)top_p * (double)CV);
  stamp_at(5);
  for (int b = tid; b < kSampBins; b += kThreads) {
    unsigned long long m = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) m += s->hm[w][b];
    s->mass[b] = m;
  }
  __syncthreads();
  if (wave == 0) {
    // the first bin whose cumulative mass reaches M* (the bins hold C_V >= M*)
    unsigned long long cum;
    const int beta = scan_reach(s->mass, false, 0ull, Mstar, &cum);
    if (lane == 0) {
      s->sel[0] = (unsigned long long)beta;
      s->sel[1] = cum;
    }
  }
  __syncthreads();
  const int beta = (int)s->sel[0];
  unsigned long long above = s->sel[1];
  // the boundary bin's elements (positive mass) into the candidate list (the
  // bin first: it is cheap, and only the boundary bin's masses are needed)
  each([&](int, int i, float z) __attribute__((always_inline)) {
    if (samp_bin(z, zmax) != beta) return;
    const unsigned long long q = mass_of(z, zmax);
    if (q) {
      const unsigned c = atomicAdd(&s->ncand, 1u);
      if (c < (unsigned)kSampCap) {
        s->ck[c] = order_key(z, i);
        s->cq[c] = q;
      }
    }
  });
  __syncthreads();
  const unsigned ncand = s->ncand;
  const bool listed = ncand <= (unsigned)kSampCap;
  stamp_at(6);
  // radix select on the order key among the boundary bin's elements
  unsigned long long prefix = 0, pmask = 0;
  for (int shift = 56; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += kThreads) s->mass[i] = 0;
    __syncthreads();
    auto add = [&](unsigned long long key, unsigned long long q) __attribute__((always_inline)) {
      if ((key & pmask) == prefix) atomicAdd(&s->mass[(int)((key >> shift) & 255ull)], q);
    };
    if (listed) {
      for (unsigned c = (unsigned)tid; c < ncand; c += kThreads) add(s->ck[c], s->cq[c]);
    } else {
      each([&](int, int i, float z) __attribute__((always_inline)) {
        if (samp_bin(z, zmax) != beta) return;
        const unsigned long long q = mass_of(z, zmax);
        if (q) add(order_key(z, i), q);
      });
    }
    __syncthreads();
    if (wave == 0) {
      // digits in descending key order (earliest first): the first whose
      // cumulative mass reaches M* holds the boundary
      unsigned long long bef;
      const int pick = scan_reach(s->mass, true, above, Mstar, &bef);
      if (lane == 0) {
        s->sel[0] = prefix | ((unsigned long long)pick << shift);
        s->sel[1] = pmask | (255ull << shift);
        s->sel[2] = bef;
      }
    }
    __syncthreads();
    prefix = s->sel[0];
    pmask = s->sel[1];
    above = s->sel[2];
    __syncthreads();
  }
  const unsigned long long kappa = prefix;   // the boundary element's key: the nucleus is key >= kappa
  stamp_at(7);
  // nucleus masses summed per (round, wave) segment of 64 consecutive indices
  // (members: every element of a bin before the boundary bin, and in it those
  // with key >= kappa; a positive mass lies in bins 0 .. 245, so an element of
  // a later bin or without mass contributes nothing)
  unsigned long long *segs = &s->hm[0][0];
  unsigned long long local = 0;
  auto segment = [&](int k, float z) __attribute__((always_inline)) {
    const int i = k * kThreads + tid;
    const int bn = samp_bin(z, zmax);
    const bool member = i < V && (bn < beta || (bn == beta && order_key(z, i) >= kappa));
    const unsigned long long q = member ? mass_of(z, zmax) : 0ull;
    local += q;
    const unsigned long long sg = wave_sum_u64(q);
    if (lane == 0) segs[k * kWaves + wave] = sg;   // segment (k, wave): indices 512 k + 64 wave ..
  };
  for (int k0 = 0; k0 < nr; k0 += kSampBatch) {
    float zc[kSampBatch];
#pragma unroll
    for (int u = 0; u < kSampBatch; ++u) zc[u] = scaled_logit(logits, min((k0 + u) * kThreads + tid, V - 1), inv_temp);
#pragma unroll
    for (int u = 0; u < kSampBatch; ++u)
      if (k0 + u < nr) segment(k0 + u, zc[u]);
  }
  if (tid == 0) s->ibc[0] = -1;
  const unsigned long long CN = block_sum_u64(local, s);
  stamp_at(8);
  unsigned ctr[4] = {(unsigned)pos, 0u, 0u, 0u};
  philox4x32_10(ctr, (unsigned)(seed & 0xffffffffull), (unsigned)(seed >> 32));
  const unsigned long long r = ((unsigned long long)ctr[1] << 32) | ctr[0];
  const unsigned long long t = __umul64hi(r, CN);
  if (wave == 0) {
    // the segment holding t: exclusive scan of the nr * 8 segment sums in index order
    const int nseg = nr * kWaves;
    unsigned long long base = 0;
    for (int c0 = 0; c0 < nseg; c0 += 64) {
      const int c = c0 + lane;
      const unsigned long long v = c < nseg ? segs[c] : 0ull;
      unsigned long long incl = wave_scan_u64(v);
      const unsigned long long ex = base + incl - v;
      if (v > 0 && ex <= t && t < ex + v) {
        s->sel[0] = (unsigned long long)c;
        s->sel[1] = ex;
      }
      base += lane63_u64(incl);
    }
  }
  __syncthreads();
  const int seg = (int)s->sel[0];
  if (wave == seg % kWaves) {
    // inside the segment: the lane whose inclusive running mass first exceeds t
    const int k = seg / kWaves, i = k * kThreads + tid;
    unsigned long long q = 0;
    if (i < V) {
      const float z = scaled_logit(logits, i, inv_temp);
      if (order_key(z, i) >= kappa) q = mass_of(z, zmax);
    }
    unsigned long long incl = wave_scan_u64(q);
    const unsigned long long ex = s->sel[1] + incl - q;
    if (q > 0 && ex <= t && t < ex + q) s->ibc[0] = i;
  }
  __syncthreads();
  const int tok = s->ibc[0];
  stamp_at(9);
  if (kTrace && tr && tid == 0) tr[10] = ncand;
  __syncthreads();
  return tok;
}

// ---------------------------------------------------------------- the nucleus draw over the grid
//
// The same draw as sample_topp (the same integer masses, bins, order keys and
// Philox draw, so the same token), with the per-logit work spread over the
// lm_head workgroups, each over its own block of rows (consecutive indices,
// ascending with the workgroup), and workgroup 0 handling the aggregates.  The
// sync waves only; each step is one tagged exchange (a 64-bit value is a pair
// of tagged words, low then high), at the levels after the lm_head's (the
// largest logit z* of each workgroup comes tagged with the lm_head's level):
//   +1  each workgroup's masses per bin            hist [bin][G][2]
//   +2  the bin totals, bin j summed by workgroup j mod G   btot [bin][2]
//   then every workgroup finds the boundary bin beta from the totals, and
//   +3  each workgroup's record: its mass in the bins before beta and its rows
//       in bin beta (16-bit offsets)                 cand [G][3 + cmax / 2]
// Workgroup 0 then reads the records and the listed rows' logits, finds the
// boundary key kappa, adds each workgroup's members in bin beta to its mass
// before beta, and finds the workgroup and the row holding the draw.  With more
// than kSampCap candidates it finds kappa, and the workgroups' members in bin
// beta, by scanning every logit itself (slow, exact).

__device__ __forceinline__ void st_tag64(u64 *p, unsigned long long v, unsigned tag) {
  st_tag(p, ((u64)tag << 32) | (unsigned)v);
  st_tag(p + 1, ((u64)tag << 32) | (unsigned)(v >> 32));
}

// Wave 0: the n tagged words at addr(i), i < n, re-read until every one carries
// tag, then use(i, payload) for each (kCoopChunk slots of 64 words at a time).
template <int kChunk = kCoopChunk, class A, class F>
__device__ __forceinline__ bool wave_fetch(KP &P, int n, unsigned tag, A &&addr, F &&use) {
  const int lane = lane_id();
  const unsigned long long t0 = now_ticks();
  for (int b0 = 0; b0 < n; b0 += 64 * kChunk) {
    u64 v[kChunk];
    for (;;) {
      const unsigned e = ld_dev(&P.err[0]);
#pragma unroll
      for (int k = 0; k < kChunk; ++k) v[k] = ld_dev(addr(min(b0 + 64 * k + lane, n - 1)));
      bool bad = false;
#pragma unroll
      for (int k = 0; k < kChunk; ++k) bad |= b0 + 64 * k + lane < n && tag_of(v[k]) != tag;
      if (wave_none(bad)) {
        retire(e);
        break;
      }
      if (expired(P, t0, tag, e)) return false;
    }
#pragma unroll
    for (int k = 0; k < kChunk; ++k)
      if (b0 + 64 * k + lane < n) use(b0 + 64 * k + lane, (unsigned)v[k]);
  }
  return true;
}

// Wave 0 of workgroup 0: the radix select of sample_topp over the candidate
// list (keys ck, masses cq, n of them): the key of the nucleus boundary, given
// the mass `above` before bin beta.  rescan: instead of the list, every logit of
// bin beta (more candidates than the list holds).
__device__ __forceinline__ unsigned long long nuc_kappa(SampLds *s, unsigned n, bool rescan, const float *logits,
                                                        int V, float inv_temp, float zmax, int beta,
                                                        unsigned long long above, unsigned long long Mstar) {
  const int lane = lane_id();
  unsigned long long prefix = 0, pmask = 0;
  for (int shift = 56; shift >= 0; shift -= 8) {
    for (int i = lane; i < 256; i += 64) s->mass[i] = 0;
    lds_drain();
    auto add = [&](unsigned long long key, unsigned long long q) __attribute__((always_inline)) {
      if ((key & pmask) == prefix) atomicAdd(&s->mass[(int)((key >> shift) & 255ull)], q);
    };
    if (!rescan) {
      // 64 candidates a round; when every matching lane has the same digit (the
      // high bytes of nearby keys), one wave sum and one add instead of 64 adds
      // to one LDS word
      for (unsigned c0 = 0; c0 < n; c0 += 64) {
        const unsigned c = c0 + (unsigned)lane;
        const unsigned long long key = c < n ? s->ck[c] : 0ull, q = c < n ? s->cq[c] : 0ull;
        const bool m = c < n && (key & pmask) == prefix;
        const int dg = (int)((key >> shift) & 255ull);
        const unsigned long long mm = __builtin_amdgcn_ballot_w64(m);
        if (mm == 0ull) continue;
        const int d0 = __builtin_amdgcn_readlane(dg, __builtin_ctzll(mm));
        if (__builtin_amdgcn_ballot_w64(m && dg != d0) == 0ull) {
          const unsigned long long sum = wave_sum_u64(m ? q : 0ull);
          if (lane == 0) atomicAdd(&s->mass[d0], sum);
        } else if (m) {
          atomicAdd(&s->mass[dg], q);
        }
      }
    } else {
      for (int i = lane; i < V; i += 64) {
        const float z = scaled_logit(logits, i, inv_temp);
        if (samp_bin(z, zmax) != beta) continue;
        const unsigned long long q = mass_of(z, zmax);
        if (q) add(order_key(z, i), q);
      }
    }
    lds_drain();
    unsigned long long bef;
    const int pick = scan_reach(s->mass, true, above, Mstar, &bef);
    prefix |= (unsigned long long)pick << shift;
    pmask |= 255ull << shift;
    above = bef;
  }
  return prefix;
}

// Wave 0 of workgroup 0: kappa from the candidate list (keys ck, masses cq, n of
// them, all in bin beta) without eight radix passes: a histogram of the
// candidates' masses over 256 sub-bins of bin beta (sub-bin = floor(256 (d -
// beta)) with d = (z* - z) kSampBinScale, the bin's own formula refined, so a
// lower sub-bin holds larger z), the sub-bin where the running mass from
// `above` reaches Mstar, then that sub-bin's candidates ordered by key (each
// lane ranks one against the others).  Returns false (kappa unset) when that
// sub-bin holds more than 64 candidates (ties in z): then the radix select.
__device__ __forceinline__ int nuc_sub(float z, float zmax, int beta) {
#pragma clang fp contract(off)
  const float d = (zmax - z) * kSampBinScale - (float)beta;
  const int sb = (int)(d * 256.0f);
  return sb < 0 ? 0 : (sb > 255 ? 255 : sb);
}
// (s->mass holds the candidates' masses per sub-bin on entry)
__device__ __forceinline__ bool nuc_kappa_fine(SampLds *s, unsigned n, float zmax, int beta, unsigned long long above,
                                               unsigned long long Mstar, unsigned long long *kappa) {
  const int lane = lane_id();
  auto sub_of = [&](unsigned long long key) __attribute__((always_inline)) -> int {
    unsigned b = (unsigned)(key >> 32);
    b = (b & 0x80000000u) ? (b & 0x7fffffffu) : ~b;   // the order key's float bits back
    return nuc_sub(__uint_as_float(b), zmax, beta);
  };
  unsigned long long before;
  const int sb = scan_reach(s->mass, false, above, Mstar, &before);
  // the sub-bin's candidates into ibc-free scratch: indices into ck / cq (wave ballots)
  unsigned *pick = reinterpret_cast<unsigned *>(&s->hm[7][0]);   // up to 64 entries
  unsigned m = 0;
  for (unsigned c0 = 0; c0 < n; c0 += 64) {
    const unsigned c = c0 + (unsigned)lane;
    const bool in = c < n && sub_of(s->ck[c]) == sb;
    const unsigned long long mm = __builtin_amdgcn_ballot_w64(in);
    const unsigned k = m + (unsigned)__builtin_popcountll(mm & ((1ull << lane) - 1ull));
    if (in && k < 64u) pick[k] = c;
    m += (unsigned)__builtin_popcountll(mm);
  }
  if (m > 64u) return false;
  lds_drain();
  // lane j < m: candidate j; its running mass before it = before + the masses of
  // the sub-bin's larger keys
  const bool act = (unsigned)lane < m;
  const unsigned me = act ? pick[lane] : 0u;
  const unsigned long long key = act ? s->ck[me] : 0ull, q = act ? s->cq[me] : 0ull;
  unsigned long long run = before;
  for (unsigned j = 0; j < m; ++j) {
    const unsigned o = pick[j];
    const unsigned long long ko = s->ck[o];
    if (ko > key) run += s->cq[o];
  }
  const bool hit = act && run < Mstar && run + q >= Mstar;
  const unsigned long long hm = __builtin_amdgcn_ballot_w64(hit);
  if (hm == 0ull) return false;   // (unreachable for consistent masses)
  const int src = __builtin_ctzll(hm);
  *kappa = ((unsigned long long)(unsigned)__builtin_amdgcn_readlane((int)(key >> 32), src) << 32) |
           (unsigned)__builtin_amdgcn_readlane((int)(unsigned)key, src);
  return true;
}

// Every workgroup's sync wave, after the lm_head level lvl: the steps above.
// Returns the token in workgroup 0 (-1 elsewhere), or -2 when a wait expired.
__device__ __forceinline__ int nucleus_grid(KP &P, Sync &sy, Ctl *ctl, int b, int G, unsigned lvl, int pos,
                                            unsigned char *lds, int trk = -1) {
  const int lane = lane_id();
  // LF_TRACE stamps (slot trk): 3 z* known, 4 bins written, 5 bin totals written,
  // 6 boundary bin known, 7 record written; workgroup 0: 12 the heads in, 13 the
  // lists in, 8 the candidates' keys, 14 kappa known, 10 the masses, 11 the
  // token found; [15] the candidate count
  auto stamp_at = [&](int j) __attribute__((always_inline)) { trace_at(P, trk, j); };
  SampLds *s = reinterpret_cast<SampLds *>(lds);
  unsigned long long *hist = &s->hm[0][0];                       // this workgroup's bins (256)
  // fetched payloads and workgroup 0's list bookkeeping (5 G + G + kSampCap / 2
  // words at most: below hm[7], which the sub-bin search uses)
  unsigned *tmp = reinterpret_cast<unsigned *>(&s->hm[1][0]);
  const Geo ge = uniform_geo(ctl, K_LM);
  const int V = P.V, cmax = P.nuc_cmax, cstride = 3 + cmax / 2;
  const float inv_temp = P.inv_temp;
  // z*: the lm_head workgroups' maxima, tagged words stored after their logits
  // were complete (the acquire fence then orders the plain logit loads below)
  float zm = -INFINITY;
  if (!wave_fetch(P, G, lvl, [&](int i) { return (const u64 *)P.nuc_zmax + i; },
                  [&](int, unsigned w) { zm = fmaxf(zm, __uint_as_float(w)); }))
    return -2;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  __builtin_amdgcn_s_waitcnt(0);
  float zmax;
  {
#pragma clang fp contract(off)
    zmax = wave_max(zm) * inv_temp;
  }
  stamp_at(3);
  // +1: masses per bin of this workgroup's rows
  for (int j = lane; j < kSampBins; j += 64) hist[j] = 0ull;
  lds_drain();
  for (int i = lane; i < ge.nrows; i += 64) {
    const float z = scaled_logit(P.logits, ge.r0 + i, inv_temp);
    const unsigned long long q = mass_of(z, zmax);
    if (q) atomicAdd(&hist[samp_bin(z, zmax)], q);
  }
  lds_drain();
  for (int j = lane; j < kSampBins; j += 64) st_tag64(P.nuc_hist + ((size_t)j * G + b) * 2, hist[j], lvl + 1u);
  stamp_at(4);
  // +2: the totals of bins b, b + G, ...
  for (int j = b; j < kSampBins; j += G) {
    const u64 *src = P.nuc_hist + (size_t)j * G * 2;
    if (!wave_fetch(P, 2 * G, lvl + 1u, [&](int i) { return src + i; },
                    [&](int i, unsigned w) { tmp[i] = w; }))
      return -2;
    lds_drain();
    unsigned long long v = 0;
    for (int w = lane; w < G; w += 64) v += ((unsigned long long)tmp[2 * w + 1] << 32) | tmp[2 * w];
    v = wave_sum_u64(v);
    lds_drain();
    if (lane == 0) st_tag64(P.nuc_btot + (size_t)j * 2, v, lvl + 2u);
  }
  stamp_at(5);
  // every workgroup: the bin totals, their sum C_V, the target mass M* =
  // ceil(top_p C_V) and the boundary bin beta (the same values everywhere)
  if (!wave_fetch(P, 2 * kSampBins, lvl + 2u, [&](int i) { return P.nuc_btot + i; },
                  [&](int i, unsigned w) { tmp[i] = w; }))
    return -2;
  lds_drain();
  unsigned long long cv = 0;
  for (int j = lane; j < kSampBins; j += 64) {
    const unsigned long long m = ((unsigned long long)tmp[2 * j + 1] << 32) | tmp[2 * j];
    s->mass[j] = m;
    cv += m;
  }
  cv = wave_sum_u64(cv);
  lds_drain();
  const unsigned long long Mstar = (unsigned long long)ceil((double)P.top_p * (double)cv);
  unsigned long long above;   // the mass of the bins before beta
  const int beta = scan_reach(s->mass, false, 0ull, Mstar, &above);
  stamp_at(6);
  // +3: this workgroup's record: word 0 the count of its rows in bin beta (with
  // a nonzero mass), words 1-2 the mass of its rows in the bins before beta,
  // words 3.. those rows as 16-bit offsets from its first row, two a word
  {
    u64 *cb = P.nuc_cand + (size_t)b * cstride;
    unsigned short *off16 = reinterpret_cast<unsigned short *>(tmp);
    unsigned cnt = 0;
    for (int i0 = 0; i0 < ge.nrows; i0 += 64) {
      const int i = i0 + lane;
      bool c = false;
      if (i < ge.nrows) {
        const float z = scaled_logit(P.logits, ge.r0 + i, inv_temp);
        c = mass_of(z, zmax) != 0 && samp_bin(z, zmax) == beta;
      }
      const unsigned long long m = __builtin_amdgcn_ballot_w64(c);
      if (c) off16[cnt + (unsigned)__builtin_popcountll(m & ((1ull << lane) - 1ull))] = (unsigned short)i;
      cnt += (unsigned)__builtin_popcountll(m);
    }
    lds_drain();
    for (unsigned j = (unsigned)lane; 2 * j < cnt; j += 64) {
      const unsigned lo = off16[2 * j], hi = 2 * j + 1 < cnt ? off16[2 * j + 1] : 0u;
      st_tag(cb + 3 + j, ((u64)(lvl + 3u) << 32) | lo | (hi << 16));
    }
    unsigned long long pre = 0;
    for (int j = lane; j < beta; j += 64) pre += hist[j];
    pre = wave_sum_u64(pre);
    lds_drain();
    if (lane == 0) {
      st_tag64(cb + 1, pre, lvl + 3u);
      st_tag(cb, ((u64)(lvl + 3u) << 32) | cnt);
    }
  }
  stamp_at(7);
  if (b != 0) return -1;

  // ---- workgroup 0: every record's head (count, mass before beta)
  unsigned *head = tmp, *cpre = tmp + 3 * G, *wpre = tmp + 4 * G, *wmap = tmp + 5 * G;
  const int qb = (V / 2) / G, rb = (V / 2) % G;   // workgroup w's first row: 2 (w qb + min(w, rb))
  if (!wave_fetch<16>(P, 3 * G, lvl + 3u,
                  [&](int i) { return (const u64 *)P.nuc_cand + (size_t)(i / 3) * cstride + i % 3; },
                  [&](int i, unsigned v) { head[i] = v; }))
    return -2;
  lds_drain();
  // exclusive prefixes over the workgroups of the counts (cpre) and of the list
  // words (wpre); each workgroup's nucleus mass starts as its mass before beta
  unsigned long long *sums = &s->hm[0][0];
  unsigned run = 0, wrun = 0;
  for (int w0 = 0; w0 < G; w0 += 64) {
    const int w = w0 + lane;
    const unsigned v = w < G ? head[3 * w] : 0u, vw = (v + 1u) >> 1;
    const unsigned incl = wave_scan_u32(v), winc = wave_scan_u32(vw);
    if (w < G) {
      cpre[w] = run + incl - v;
      wpre[w] = wrun + winc - vw;
      sums[w] = ((unsigned long long)head[3 * w + 2] << 32) | head[3 * w + 1];
    }
    run += (unsigned)__builtin_amdgcn_readlane((int)incl, 63);
    wrun += (unsigned)__builtin_amdgcn_readlane((int)winc, 63);
  }
  lds_drain();
  const unsigned total = run, nw = wrun;
  const bool rescan = total > (unsigned)kSampCap;
  for (int j = lane; j < 256; j += 64) s->mass[j] = 0ull;
  lds_drain();
  stamp_at(12);
  if (kTrace && trk >= 0 && lane == 0) trace_row(P, trk)[15] = total;
  if (!rescan && total > 0) {
    // the list words: word i belongs to workgroup wmap[i]; candidate c (in
    // workgroup then row order) gets its row in ck[c]
    for (int w = lane; w < G; w += 64) {
      const unsigned n = (head[3 * w] + 1u) >> 1;
      for (unsigned k = 0; k < n; ++k) wmap[wpre[w] + k] = (unsigned)w;
    }
    lds_drain();
    if (!wave_fetch<16>(P, (int)nw, lvl + 3u,
                        [&](int i) {
                          // (clamped: a word index always stays inside the record area)
                          const unsigned w = min(wmap[i], (unsigned)G - 1u);
                          return (const u64 *)P.nuc_cand + (size_t)w * cstride + 3 +
                                 min((unsigned)i - wpre[w], (unsigned)cstride - 4u);
                        },
                        [&](int i, unsigned v) {
                          const unsigned w = wmap[i], k = 2u * ((unsigned)i - wpre[w]), c = cpre[w] + k;
                          const unsigned r0 = 2u * (w * (unsigned)qb + min(w, (unsigned)rb));
                          s->ck[c] = r0 + (v & 0xffffu);
                          s->cown[c] = (unsigned char)w;
                          if (k + 1u < head[3 * w]) {
                            s->ck[c + 1] = r0 + (v >> 16);
                            s->cown[c + 1] = (unsigned char)w;
                          }
                        }))
      return -2;
    lds_drain();
    stamp_at(13);
    // the candidates' logits (plain loads, kB per lane in flight), their order
    // keys and masses, and their masses per sub-bin of bin beta
    constexpr int kB = 16;
    for (unsigned c0 = 0; c0 < total; c0 += 64 * kB) {
      int row[kB];
      float lg[kB];
#pragma unroll
      for (int k = 0; k < kB; ++k) {
        const unsigned c = c0 + 64 * k + (unsigned)lane;
        row[k] = c < total ? (int)s->ck[c] : 0;
        lg[k] = P.logits[row[k]];
      }
#pragma unroll
      for (int k = 0; k < kB; ++k) {
        const unsigned c = c0 + 64 * k + (unsigned)lane;
        if (c < total) {
          const float z = scale_logit(lg[k], inv_temp);
          const unsigned long long q = mass_of(z, zmax);
          s->ck[c] = order_key(z, row[k]);
          s->cq[c] = q;
          atomicAdd(&s->mass[nuc_sub(z, zmax, beta)], q);
        }
      }
    }
    lds_drain();
  }
  stamp_at(8);
  unsigned long long kappa = 0;
  if (rescan || !nuc_kappa_fine(s, total, zmax, beta, above, Mstar, &kappa))
    kappa = nuc_kappa(s, total, rescan, P.logits, V, inv_temp, zmax, beta, above, Mstar);
  stamp_at(14);
  // add each workgroup's members in bin beta (key >= kappa) to its mass
  if (!rescan) {
    for (unsigned c = (unsigned)lane; c < total; c += 64)
      if (s->ck[c] >= kappa) atomicAdd(&sums[s->cown[c]], s->cq[c]);
  } else {
    const int cut = rb * (qb + 1);
    auto owner = [&](int r) __attribute__((always_inline)) -> int {
      const int p = r >> 1;
      return p < cut ? p / (qb + 1) : rb + (p - cut) / qb;
    };
    for (int i = lane; i < V; i += 64) {
      const float z = scaled_logit(P.logits, i, inv_temp);
      if (samp_bin(z, zmax) != beta || order_key(z, i) < kappa) continue;
      const unsigned long long q = mass_of(z, zmax);
      if (q) atomicAdd(&sums[owner(i)], q);
    }
  }
  lds_drain();
  unsigned long long cn = 0;
  for (int w = lane; w < G; w += 64) cn += sums[w];
  cn = wave_sum_u64(cn);
  stamp_at(10);
  auto member_mass = [&](int r) __attribute__((always_inline)) -> unsigned long long {
    const float z = scaled_logit(P.logits, r, inv_temp);
    const int bn = samp_bin(z, zmax);
    return (bn < beta || (bn == beta && order_key(z, r) >= kappa)) ? mass_of(z, zmax) : 0ull;
  };
  // the draw t, the workgroup holding it, then its row
  unsigned ctr[4] = {(unsigned)pos, 0u, 0u, 0u};
  philox4x32_10(ctr, (unsigned)(P.seed & 0xffffffffull), (unsigned)(P.seed >> 32));
  const unsigned long long r = ((unsigned long long)ctr[1] << 32) | ctr[0];
  const unsigned long long t = __umul64hi(r, cn);
  // exclusive scans in index order: the workgroup w with ex <= t < ex + v, then its row
  auto find = [&](int n, auto &&val, unsigned long long base, unsigned long long &at) __attribute__((always_inline)) {
    int hit = -1;
    for (int c0 = 0; c0 < n; c0 += 64) {
      const unsigned long long v = c0 + lane < n ? val(c0 + lane) : 0ull;
      unsigned long long incl = wave_scan_u64(v);
      const unsigned long long ex = base + incl - v;
      const unsigned long long m = __builtin_amdgcn_ballot_w64(v > 0 && ex <= t && t < ex + v);
      if (m) {
        const int src = __builtin_ctzll(m);
        hit = c0 + src;
        at = ((unsigned long long)(unsigned)__builtin_amdgcn_readlane((int)(ex >> 32), src) << 32) |
             (unsigned)__builtin_amdgcn_readlane((int)(unsigned)ex, src);
        break;
      }
      base += lane63_u64(incl);
    }
    return hit;
  };
  unsigned long long wbase = 0, rbase = 0;
  const int w = find(G, [&](int i) { return sums[i]; }, 0ull, wbase);
  if (w < 0) return 0;   // (unreachable: the workgroups' masses add up to C_N > t)
  int p0, p1;
  block_range(V / 2, G, w, p0, p1);
  const int row = find(2 * (p1 - p0), [&](int i) { return member_mass(2 * p0 + i); }, wbase, rbase);
  stamp_at(11);
  return row < 0 ? 0 : 2 * p0 + row;
}

// ---------------------------------------------------------------- the kernel

// kPrefill: teacher-forced prompt tokens read from in_tokens[], no logits and no
// sampling; each token's first layer waits until every workgroup finished the
// previous token.
//
// Dependency levels of token t, layer l (lvl = level of the previous layer's
// down projection): QKV lvl+1, attention lvl+2, O lvl+3, gate/up lvl+4, down
// lvl+5; after the last layer, lm_head lvl+1 and the chosen token lvl+2.  The
// vectors between phases travel as tagged words in generation (t*L + l) & 1.
// A workgroup reads a phase's input only if it has rows in that phase, so each
// read is followed by an output that every later phase depends on; a buffer of
// one generation is rewritten two layers later, after every reader of it.
template <bool kPrefill, int kQ>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_num_vgpr(104))) lf_monokernel(Params Parg) {
  // Parg is the only argument: read it where the dispatch placed it, at the
  // start of the kernel-argument segment (never through a copy).
  (void)Parg;
  KP &P = *(KP *)(__builtin_amdgcn_kernarg_segment_ptr());
  extern __shared__ __align__(16) unsigned char smem[];
  _Float16 *hl = reinterpret_cast<_Float16 *>(smem + P.lds_h);
  float *part = reinterpret_cast<float *>(smem + P.lds_part);
  Ctl *ctl = reinterpret_cast<Ctl *>(smem + P.lds_ctl);
  float *xown = reinterpret_cast<float *>(smem + P.lds_xown); // residual rows: output projection
  float *xres = reinterpret_cast<float *>(smem + P.lds_xres); // residual rows: down projection
  unsigned char *alds = smem + P.lds_h;                       // sampler scratch (over the staged input)
  unsigned char *attn_scratch = smem + P.lds_attn;            // attention scratch (stream waves)
  const int b = blockIdx.x, G = P.G, wave = wave_id(), lane = lane_id();
  const int L = P.L, d = P.d, dh = P.dh;
  const bool has_lm = !kPrefill && !P.hidden_io;
  const int ngp = 4 * L + (has_lm ? 1 : 0);        // GEMV phases per token
  const _Float16 *emb = reinterpret_cast<const _Float16 *>(P.tok_emb);

  // this workgroup's row block of every phase kind: contiguous partition units
  // (row pairs, so each rotary pair has one producer; gate/up in units of two
  // pairs, so one SwiGLU word has one producer; the output projection in single
  // rows, over the workgroups that merge no attention head)
  if (tid_x() == 0) {
    const int units[K_COUNT] = {P.nqkv / 2, d, P.F / 2, d / 2, P.V / 2};
    const int upr[K_COUNT] = {2, 1, 4, 2, 2};
    const int kvs[K_COUNT] = {d / 8, P.Hq * dh / 8, d / 8, P.F / 8, d / 8};
    // (the units of the launch's first position: with query-split heads every
    // unit's workgroup, else the merging ones)
    const AttnSplit asp0(P, P.pos0, G);
    const int nskip = o_rows_skip(G, asp0.a[0].H);
    // Workgroups that run attention with prefetched tiles stream no QKV rows:
    // the units of the launch's last position (the most), if they are few.
    int na = 0;
    if (P.kv_pf > 0) {
      const int pl = P.pos0 + P.n_tokens - 1;
      const AttnSplit asp(P, pl, G);
      int smax = asp.a[0].S > asp.a[1].S ? asp.a[0].S : asp.a[1].S;
      if (P.window > 0) {   // a window's tile count moves by one with the position
        const AttnPart w1 = attn_part(0, P.window + kKvTile, G, P.Hkv, P.qpg, P.attn_qsplit, P.attn_unit_tiles,
                                      P.attn_split_tiles);
        if (w1.S > smax) smax = w1.S;
      }
      na = P.Hkv * smax;
      if (4 * na > G) na = 0;
    }
    ctl->na = na;
    int ww[kNcw], weq[kNcw];
    for (int k = 0; k < kNcw; ++k) {
      ww[k] = P.wave_w[k];
      weq[k] = 1;
    }
    for (int k = 0; k < K_COUNT; ++k) {
      int p0 = 0, p1 = 0;
      if (k == K_QKV) {
        if (b >= na) block_range(units[k], G - na, b - na, p0, p1);
      } else if (k != K_O) {
        block_range(units[k], G, b, p0, p1);
      } else if (b >= nskip) {
        block_range(units[k], G - nskip, b - nskip, p0, p1);
      }
      const Geo ge = Geo{upr[k] * p0, upr[k] * (p1 - p0), kvs[k], (kvs[k] + 63) / 64};
      ctl->geo[k] = ge;
      int wn[kNcw];
      wave_counts(ge.nrows * ge.ppr, ((P.wave_w_kinds >> k) & 1) ? ww : weq, wn);
      for (int cw = 0; cw < kNcw; ++cw) {
        int lo, hi;
        lo = hi = 0;
        for (int c = 0; c <= cw; ++c) {
          lo = hi;
          hi += wn[c];
        }
        if (k == P.pf_kind) {
          const int npf = min(hi - lo, P.pf_n);
          ctl->pf[cw] = Slice{npf, npf > 0 ? lo / ge.ppr : 0, npf > 0 ? lo % ge.ppr : 0, 0};
          lo += npf;
        }
        const int row = lo < hi ? lo / ge.ppr : 0;
        ctl->slice[k][cw] = Slice{hi - lo, row, lo < hi ? lo - row * ge.ppr : 0, 0};
      }
    }
    if (kTrace)
      for (int i = 0; i < kTraceSlots * (5 * L + 2); ++i) trace_row(P, 0)[i] = 0ull;
    ctl->abort = 0;
    ctl->abar = 0;
    for (int w = 0; w < kWaves; ++w) ctl->done[w] = 0;
    ctl->status = 0;
  }
  for (int i = tid_x(); i < P.psum_total; i += kThreads) part[i] = 0.0f;
  __syncthreads();

  Sync sy{&P, ctl, 0ull, 0ull, {0ull, 0ull, 0ull, 0ull, 0ull}, -1, (P.flags & 4u) != 0};
  const unsigned long long kt0 = now_ticks();

  if (wave > 0) {
    // ======================= stream waves =======================
    Streamer st;
    st.P = &P;
    st.ctl = ctl;
    st.cw = wave - 1;
    st.ngp = ngp;
    st.qend = P.n_tokens * ngp;
    st.timed = (P.flags & 4u) && st.cw == 0;
    st.t_ready = st.t_work = st.pieces = 0;
    st.trace_k = -1;
    {
      // padding pieces re-read 1 KB of layer 0's weights; spread over 64 KB so
      // that the chip's padding reads do not all queue at one L2 channel
      const long long nkb = (long long)P.layer_stride / 1024;
      const long long kb = (long long)((b * kWaves + wave) & 63) % (nkb > 0 ? nkb : 1);
      st.dummy = reinterpret_cast<const unsigned char *>(P.wbase) + kb * 1024;
    }
    st.left = st.pad = st.kp = 0;
    st.ppr = 1;
    st.tailv = 64;
    st.adv_last = 0;
    st.ptr = st.dummy;
    st.locate(0);
#pragma unroll
    for (int k = 0; k < kRing; ++k) st.issue(k);
    st.next_phase_if_done();
    for (int t = 0; t < P.n_tokens; ++t) {
      const int pos = P.pos0 + t;
      const unsigned lv0 = P.level_base + (unsigned)t * (unsigned)P.levels_per_token;
      AttnSplit asp(P, pos, G);
      // The token's GEMV phases (four per layer, then the lm_head) in one loop,
      // so that the phase code exists once: a layer's instruction footprint then
      // stays within the instruction cache.
#pragma clang loop unroll(disable)
      for (int g = 0; g < ngp; ++g) {
        const bool lm = g >= 4 * L;
        const int kind = lm ? K_LM : (g & 3);
        const int l = lm ? L : (g >> 2);
        const unsigned lvl = lv0 + (unsigned)(l * PH_PER_LAYER);
        const int gen = (t * L + l) & 1;
        const bool qkv = kind == K_QKV;
        st.trace_k = t == P.trace_token ? 5 * l + (qkv || lm ? 0 : kind + 1) : -1;
        // The refill after the QKV phase (the O phase's first round) waits until
        // after attention: this wave's loads complete in order, so attention's
        // K/V loads would otherwise queue behind it.
        const bool qkv_rounds = qkv && st_has_rounds(st, K_QKV, ctl);
        if (qkv && P.kv_pf > 0 && b < asp.a[layer_windowed(P, l) ? 1 : 0].H * asp.a[layer_windowed(P, l) ? 1 : 0].S)
          kv_prefetch(P, ctl, l, b, asp.a[layer_windowed(P, l) ? 1 : 0], st.cw);
        if (!stream_phase(st, t * ngp + g, kind, ctl, hl, part, stage_spec(P, ctl, kind, t, l, gen, lvl, xown, xres),
                          qkv))
          return;
        if (qkv) {
          const AttnPart &ap = asp.a[layer_windowed(P, l) ? 1 : 0];
          if (lds_ld(&ctl->abort)) return;
          if (b < ap.H * ap.S) {
            for (int u = b; u < ap.H * ap.S; u += G)
              if (!attn_unit<kQ>(P, ctl, l, gen, lvl + PH_QKV, lvl + PH_ATTN, pos, u, ap, attn_scratch,
                                 u == b && t == P.trace_token ? 5 * l + 1 : -1))
                return;
          } else if (2 * ap.H * ap.S <= G) {
            // a workgroup without attention units, while attention runs on few:
            // hold back the output projection's first round for a while, so that
            // the K/V loads meet less traffic
            const unsigned t_qkv = (unsigned)now_ticks();
            while ((unsigned)now_ticks() - t_qkv < P.o_refill_delay) __builtin_amdgcn_s_sleep(2);
          }
          if (qkv_rounds) st.refill();
          if (P.pf_n > 0) lds_prefetch(P, ctl, st.cw, l);
        }
      }
      if (has_lm && b == 0 && P.sampling == SAMPLE_NUCLEUS && !P.nuc_grid) {
        const unsigned lvl_lm = lv0 + (unsigned)(L * PH_PER_LAYER) + 1u;
        if (lds_ld(&ctl->abort)) return;
        if (!wait_all_waves(sy, 0, G, lvl_lm, true)) return;
        sample_topp(P.logits, P.V, P.inv_temp, P.top_p, P.seed, pos, reinterpret_cast<SampLds *>(alds),
                    t == P.trace_token ? trace_row(P, 5 * L + 1) : nullptr, P.lm_val, G);
      }
    }
    if (st.timed && lane == 0) {
      P.stats[b * P.stat_stride + 9] = st.t_ready;
      P.stats[b * P.stat_stride + 10] = st.t_work;
      P.stats[b * P.stat_stride + 11] = st.pieces;
    }
    return;
  }

  // ======================= sync wave (wave 0) =======================
  auto fail = [&]() __attribute__((always_inline)) {
    if (lane == 0) lds_st(&ctl->abort, 1u);
  };
  const int nq = P.Hq * dh, nk = P.Hkv * dh, half = dh / 2;
  const size_t nkw = (size_t)P.Hkv * half;   // words per generation of kc_t / vc_t
  int token = P.token0;
  for (int t = 0; t < P.n_tokens; ++t) {
    const int pos = P.pos0 + t;
    const unsigned lv0 = P.level_base + (unsigned)t * (unsigned)P.levels_per_token;
    if (kPrefill) token = P.in_tokens[t];
    const AttnSplit asp(P, pos, G);
    for (int l = 0; l < L; ++l) {
      if (kTrace) trace(P, t, 5 * l + 0, 12);
      KP &Pl = fresh(P);
      sy.P = &Pl;
      const unsigned lvl = lv0 + (unsigned)(l * PH_PER_LAYER);
      const int q0 = t * ngp + 4 * l;
      const int gen = (t * L + l) & 1;

      // ---------------- attention norm + QKV + rotary + KV append
      {
        const Geo ge = uniform_geo(ctl, K_QKV);
        if (l == 0 && t > 0) {
          if (kPrefill || Pl.hidden_io) {
            // the previous token is finished everywhere (its reads included)
            if (!poll_level(sy, 0, G, lv0)) { fail(); return; }
          } else {
            if (!poll_level(sy, 0, 1, lv0)) { fail(); return; }
            token = ld_dev(Pl.tok_slot);
          }
          // Nothing left in flight into the layer loop: the loads above are in
          // already (the token's own round trip aside), and a load the compiler
          // still counts as pending would make each layer's staging wait for
          // the previous layer's stores.
          __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
          asm volatile("" ::: "memory");
        }
        trace(Pl, t, 5 * l + 0, 11);
        unsigned long long tq = stamp(sy);
        sy.trace_k = t == Pl.trace_token ? 5 * l : -1;
        trace(Pl, t, 5 * l + 0, 6);
        float inv = 0.0f;   // 1 / rms of the layer input: scales the row sums
        const StageSpec sp = stage_spec(Pl, ctl, K_QKV, t, l, gen, lvl, xown, xres);
        if (ge.nrows > 0 || sp.capn > 0) {
          if (l > 0) {
            coop_stage(Pl, ctl, sp, 0, hl, sy.trace_k);
          } else {
            inv = Pl.hidden_io ? stage_rmsnorm_plain(Pl.x_hidden, d, Pl.eps, hl)
                               : stage_rmsnorm_plain(emb + (size_t)token * d, d, Pl.eps, hl);
            lds_drain();
          }
          trace(Pl, t, 5 * l + 0, 7);
          wg_barrier();
          if (lds_ld(&ctl->abort)) return;
          if (l > 0) inv = coop_inv_rms(ctl, d, Pl.eps);
        }
        tq = lap(sy, ST_STAGE, tq);
        trace(Pl, t, 5 * l + 0, 0);
        // Rotary factors of this lane's first row pair, loaded before the wait
        // for the stream waves (after the input is staged: the staging polls go
        // out first at the layer's start).
        float cs0 = 0.0f, sn0 = 0.0f;
        if (lane < ge.nrows / 2) {
          const int r = ge.r0 + 2 * lane;
          if (r < nq + nk) {
            int hd, rem;
            head_split(r < nq ? r : r - nq, dh, hd, rem);
            const int k = rem >> 1;
            cs0 = Pl.rope[((size_t)pos * half + k) * 2 + 0];
            sn0 = Pl.rope[((size_t)pos * half + k) * 2 + 1];
          }
        }
        const float *pk = kind_part(part, Pl.psum_off[K_QKV]);
        if (!wait_streams(ctl, q0)) return;
        tq = lap(sy, ST_STREAMS, tq);
        trace(Pl, t, 5 * l + 0, 1);
        const unsigned tag = lvl + PH_QKV;
        // this layer's tile runs of the cache (k_elem / v_elem within a run)
        const size_t run = (size_t)Pl.kv_tiles * kKvTile * dh;
        _Float16 *kc = reinterpret_cast<_Float16 *>(Pl.kcache) + (size_t)l * Pl.Hkv * run;
        _Float16 *vc = reinterpret_cast<_Float16 *>(Pl.vcache) + (size_t)l * Pl.Hkv * run;
        for (int i = lane; i < ge.nrows / 2; i += 64) {
          const float a = row_value(pk, 2 * i) * inv, bb = row_value(pk, 2 * i + 1) * inv;
          const int r = ge.r0 + 2 * i;
          if (r < nq + nk) {
            // q / k rows come in rotary pairs (dims k, k + dh/2 of head hd)
            const int rr = r < nq ? r : r - nq;
            int hd, rem;
            head_split(rr, dh, hd, rem);
            const int k = rem >> 1;
            const float cs = i == lane ? cs0 : Pl.rope[((size_t)pos * half + k) * 2 + 0];
            const float sn = i == lane ? sn0 : Pl.rope[((size_t)pos * half + k) * 2 + 1];
            const float y0 = a * cs - bb * sn, y1 = bb * cs + a * sn;
            if (r < nq) {
              u64 *qd = Pl.q_t + (size_t)gen * nq + (size_t)hd * dh;
              st_tag(qd + k, tag_f(y0, tag));
              st_tag(qd + k + half, tag_f(y1, tag));
            } else {
              st_dev_h(kc, (size_t)hd * run + k_elem(dh, pos, k), y0);
              st_dev_h(kc, (size_t)hd * run + k_elem(dh, pos, k + half), y1);
              st_tag(Pl.kc_t + gen * nkw + (size_t)hd * half + k, tag_h2(y0, y1, tag));
            }
          } else {
            const int rv = r - nq - nk;   // V rows in natural order, pairs (rv, rv + 1)
            const u64 w = tag_h2(a, bb, tag);
            int gv, ev;
            head_split(rv, dh, gv, ev);
            st_dev_h(vc, (size_t)gv * run + v_elem(dh, pos, ev), a);
            st_dev_h(vc, (size_t)gv * run + v_elem(dh, pos, ev + 1), bb);
            st_tag(Pl.vc_t + gen * nkw + (size_t)(rv / 2), w);
          }
        }
        publish_fast(Pl, tag);
        trace(Pl, t, 5 * l + 0, 2);
        lap(sy, ST_EPI, tq);
      }

      // (attention runs on the stream waves alone, in an LDS area of its own:
      // the sync wave goes on to poll the output projection's input)

      // ---------------- output projection + residual
      {
        const Geo ge = uniform_geo(ctl, K_O);
        unsigned long long tk = stamp(sy);
        sy.trace_k = t == Pl.trace_token ? 5 * l + 2 : -1;
        trace(Pl, t, 5 * l + 2, 6);
        if (ge.nrows > 0) {
          coop_stage(Pl, ctl, stage_spec(Pl, ctl, K_O, t, l, gen, lvl, xown, xres), 0, hl, sy.trace_k);
          trace(Pl, t, 5 * l + 2, 7);
          wg_barrier();
          if (lds_ld(&ctl->abort)) return;
        }
        tk = lap(sy, ST_STAGE, tk);
        trace(Pl, t, 5 * l + 2, 0);
        // Before the wait (none of it depends on the stream waves): the output
        // words and the residual of this lane's first row.
        const float *pk = kind_part(part, Pl.psum_off[K_O]);
        u64 *xm = Pl.xmid_t + (size_t)gen * d;
        const int hio = Pl.hidden_io;
        auto residual = [&](int i) __attribute__((always_inline)) {
          const int r = ge.r0 + i;
          return l > 0 ? xown[i] : (hio ? Pl.x_hidden[r] : (float)emb[(size_t)token * d + r]);
        };
        const float xin0 = lane < ge.nrows ? residual(lane) : 0.0f;
        // Every store this wave made before (KV cache rows, tagged words) has
        // completed before anything it publishes from here on: later steps
        // read the cache rows with plain loads.  They were issued a whole
        // projection ago, so this wait is short.
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
        asm volatile("" ::: "memory");
        if (!wait_streams(ctl, q0 + 1)) return;
        tk = lap(sy, ST_STREAMS, tk);
        trace(Pl, t, 5 * l + 2, 1);
        const unsigned tag = lvl + PH_O;
        for (int i = lane; i < ge.nrows; i += 64) {
          const int r = ge.r0 + i;
          const float xin = i == lane ? xin0 : residual(i);
          const float x = xin + row_value(pk, i);
          st_tag(xm + r, tag_f(x, tag));
        }
        publish_vec(Pl, tag);
        trace(Pl, t, 5 * l + 2, 2);
        lap(sy, ST_EPI, tk);
      }

      // ---------------- FFN norm + gate/up + SwiGLU
      {
        const Geo ge = uniform_geo(ctl, K_GU);
        unsigned long long tk = stamp(sy);
        sy.trace_k = t == Pl.trace_token ? 5 * l + 3 : -1;
        trace(Pl, t, 5 * l + 3, 6);
        float inv = 0.0f;
        const StageSpec sp = stage_spec(Pl, ctl, K_GU, t, l, gen, lvl, xown, xres);
        if (ge.nrows > 0 || sp.capn > 0) {
          coop_stage(Pl, ctl, sp, 0, hl, sy.trace_k);
          trace(Pl, t, 5 * l + 3, 7);
          wg_barrier();
          if (lds_ld(&ctl->abort)) return;
          inv = coop_inv_rms(ctl, d, Pl.eps);
        }
        tk = lap(sy, ST_STAGE, tk);
        trace(Pl, t, 5 * l + 3, 0);
        const float *pk = kind_part(part, Pl.psum_off[K_GU]);
        gu64 *ad = (gu64 *)(Pl.a_t + (size_t)gen * (Pl.F / 2));
        asm volatile("" : "+s"(ad));   // computed now, not after the wait
        if (!wait_streams(ctl, q0 + 2)) return;
        tk = lap(sy, ST_STREAMS, tk);
        trace(Pl, t, 5 * l + 3, 1);
        const unsigned tag = lvl + PH_GU;
        for (int i = lane; i < ge.nrows / 4; i += 64) {
          // rows 4i..4i+3 = gate j, up j, gate j+1, up j+1 with j = r0/2 + 2i
          const float g0 = row_value(pk, 4 * i) * inv, u0 = row_value(pk, 4 * i + 1) * inv;
          const float g1 = row_value(pk, 4 * i + 2) * inv, u1 = row_value(pk, 4 * i + 3) * inv;
          const float s0 = __fdividef(g0, 1.0f + __expf(-g0)), s1 = __fdividef(g1, 1.0f + __expf(-g1));
          st_tag(ad + ge.r0 / 4 + i, tag_h2(s0 * u0, s1 * u1, tag));
        }
        publish_vec(Pl, tag);
        trace(Pl, t, 5 * l + 3, 2);
        lap(sy, ST_EPI, tk);
      }

      // ---------------- down projection + residual
      {
        const Geo ge = uniform_geo(ctl, K_D);
        unsigned long long tk = stamp(sy);
        sy.trace_k = t == Pl.trace_token ? 5 * l + 4 : -1;
        trace(Pl, t, 5 * l + 4, 6);
        if (ge.nrows > 0) {
          coop_stage(Pl, ctl, stage_spec(Pl, ctl, K_D, t, l, gen, lvl, xown, xres), 0, hl, sy.trace_k);
          trace(Pl, t, 5 * l + 4, 7);
          wg_barrier();
          if (lds_ld(&ctl->abort)) return;
        }
        tk = lap(sy, ST_STAGE, tk);
        trace(Pl, t, 5 * l + 4, 0);
        // before the wait: output words, this lane's first residual
        const float *pk = kind_part(part, Pl.psum_off[K_D]);
        u64 *xo = Pl.xout_t + (size_t)gen * d;
        const bool host_out = Pl.hidden_io && l == L - 1;
        const float xo0 = lane < ge.nrows ? xres[lane] : 0.0f;
        if (!wait_streams(ctl, q0 + 3)) return;
        tk = lap(sy, ST_STREAMS, tk);
        trace(Pl, t, 5 * l + 4, 1);
        const unsigned tag = lvl + PH_D;
        for (int i = lane; i < ge.nrows; i += 64) {
          const int r = ge.r0 + i;
          const float x = (i == lane ? xo0 : xres[i]) + row_value(pk, i);
          st_tag(xo + r, tag_f(x, tag));
          if (host_out) Pl.x_out[r] = x;
        }
        publish_vec(Pl, tag);
        trace(Pl, t, 5 * l + 4, 2);
        lap(sy, ST_EPI, tk);
      }
    }
    sy.P = &P;
    if (!has_lm) continue;

    // ---------------- final norm + lm_head + local argmax
    const unsigned lvl_lm = lv0 + (unsigned)(L * PH_PER_LAYER) + 1u;
    const int qlm = t * ngp + 4 * L;
    const unsigned long long tlm = stamp(sy);
    {
      const Geo ge = uniform_geo(ctl, K_LM);
      float inv = 0.0f;
      if (ge.nrows > 0) {
        coop_stage(P, ctl, stage_spec(P, ctl, K_LM, t, L, 0, lvl_lm - 1u, xown, xres), 0, hl);
        trace(P, t, 5 * L, 7);
        wg_barrier();
        if (lds_ld(&ctl->abort)) return;
        inv = coop_inv_rms(ctl, d, P.eps);
      }
      trace(P, t, 5 * L, 0);
      const float *pk = kind_part(part, P.psum_off[K_LM]);
      if (!wait_streams(ctl, qlm)) return;
      trace(P, t, 5 * L, 1);
      float best = -INFINITY;
      int bi = 0x7fffffff;
      const bool gumbel = P.sampling == SAMPLE_GUMBEL;
      for (int i = lane; i < ge.nrows; i += 64) {
        const float y = row_value(pk, i) * inv;
        st_dev(&P.logits[ge.r0 + i], y);
        // Gumbel-max: this workgroup's best score z + g instead of its best logit
        const float sc = gumbel ? gumbel_score(y, P.inv_temp, P.seed, pos, ge.r0 + i) : y;
        if (sc > best || (sc == best && ge.r0 + i < bi)) { best = sc; bi = ge.r0 + i; }
      }
      wave_argmax(best, bi);
      if (lane == 0) {
        st_dev(&P.lm_val[b], best);
        st_dev(&P.lm_idx[b], bi);
      }
      publish_sync(P, lvl_lm);
      // the nucleus draw over the grid polls the maxima as tagged words (the
      // logits' stores are complete: publish_sync waited for them)
      if (P.nuc_grid && lane == 0) st_tag(P.nuc_zmax + b, tag_f(best, lvl_lm));
      trace(P, t, 5 * L, 2);
    }

    // ---------------- next token
    if (P.sampling == SAMPLE_NUCLEUS && P.nuc_grid) {
      // the nucleus draw over the grid: every workgroup's sync wave takes part
      trace(P, t, 5 * L + 1, 0);
      int tok = nucleus_grid(P, sy, ctl, b, G, lvl_lm, pos, alds, t == P.trace_token ? 5 * L + 1 : -1);
      if (tok == -2) {
        fail();
        return;
      }
      if (b == 0) {
        if (tok < 0 || tok >= P.V) {   // never expected; keeps the next embedding read in bounds
          if (lane == 0) st_dev(&P.err[3], 1u);
          tok = 0;
        }
        if (lane == 0) {
          st_dev(P.tok_slot, tok);
          P.out_tokens[t] = tok;
        }
        publish_sync(P, lvl_lm + 1u + (unsigned)kNucLevels);
      }
      trace(P, t, 5 * L + 1, 2);
    } else if (b == 0) {
      int tok;
      if (P.sampling == SAMPLE_NUCLEUS) {
        trace(P, t, 5 * L + 1, 0);
        if (!wait_all_waves(sy, 0, G, lvl_lm, true)) { fail(); return; }
        trace(P, t, 5 * L + 1, 1);
        tok = sample_topp(P.logits, P.V, P.inv_temp, P.top_p, P.seed, pos, reinterpret_cast<SampLds *>(alds),
                          t == P.trace_token ? trace_row(P, 5 * L + 1) : nullptr, P.lm_val, G);
      } else {
        if (!poll_level(sy, 0, G, lvl_lm)) {
          fail();
          return;
        }
        // every workgroup's (max, index): all loads in flight at once (clamped
        // indices; entries past G are ignored), then the comparisons
        float best = -INFINITY;
        int bi = 0x7fffffff;
        for (int i0 = 0; i0 < G; i0 += 4 * 64) {
          float v[4];
          int ix[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int i = min(i0 + 64 * k + lane, G - 1);
            v[k] = ld_dev(&P.lm_val[i]);
            ix[k] = ld_dev(&P.lm_idx[i]);
          }
#pragma unroll
          for (int k = 0; k < 4; ++k)
            if (i0 + 64 * k + lane < G && (v[k] > best || (v[k] == best && ix[k] < bi))) {
              best = v[k];
              bi = ix[k];
            }
        }
        wave_argmax(best, bi);
        tok = bi;
      }
      if (tok < 0 || tok >= P.V) {   // never expected; keeps the next embedding read in bounds
        if (lane == 0) st_dev(&P.err[3], 1u);
        tok = 0;
      }
      if (lane == 0) {
        st_dev(P.tok_slot, tok);
        P.out_tokens[t] = tok;
      }
      publish_sync(P, lvl_lm + 1u);
      trace(P, t, 5 * L + 1, 2);
    }
    lap(sy, ST_LM, tlm);
  }
  if (kTrace)
    for (int i = lane; i < kTraceSlots * (5 * L + 2); i += 64)
      P.stats[(size_t)b * P.stat_stride + kStatWords + i] = trace_row(P, 0)[i];
  if ((P.flags & 4u) && lane == 0) {
    unsigned xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    unsigned long long *o = P.stats + (size_t)b * P.stat_stride;
    o[0] = sy.spin;
    o[1] = sy.waits;
    o[2] = xcc & 0xfu;
    o[3] = now_ticks() - kt0;
    for (int k = 0; k < kStatPhases; ++k) o[4 + k] = sy.tm[k];
  }
}

__global__ void lf_test_expdef_kernel(const float *x, float *y, long long n) {
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long long)gridDim.x * blockDim.x)
    y[i] = expdef(x[i]);
}

__global__ void __launch_bounds__(kThreads) lf_test_sample_kernel(const float *logits, int n, float inv_temp,
                                                                 float top_p, unsigned long long seed,
                                                                 const int *pos, int *tokens) {
  extern __shared__ __align__(16) unsigned char samp_lds[];
  SampLds &s = *reinterpret_cast<SampLds *>(samp_lds);
  const int c = blockIdx.x;
  const int tok = sample_topp(logits + (size_t)c * n, n, inv_temp, top_p, seed, pos[c], &s);
  if (threadIdx.x == 0) tokens[c] = tok;
}

__global__ void lf_test_logdef_kernel(const float *x, float *y, long long n) {
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long long)gridDim.x * blockDim.x)
    y[i] = logdef(x[i]);
}

// One case per workgroup: the Gumbel-max token of logits[c*n .. c*n+n) at
// counter pos[c], from the same score function as the decode kernel.
__global__ void __launch_bounds__(kThreads) lf_test_gumbel_kernel(const float *logits, int n, float inv_temp,
                                                                 unsigned long long seed, const int *pos,
                                                                 int *tokens) {
  __shared__ float wbest[kWaves];
  __shared__ int wbi[kWaves];
  const int c = blockIdx.x;
  const float *lg = logits + (size_t)c * n;
  float best = -INFINITY;
  int bi = 0x7fffffff;
  for (int i = threadIdx.x; i < n; i += kThreads) {
    const float sc = gumbel_score(lg[i], inv_temp, seed, pos[c], i);
    if (sc > best || (sc == best && i < bi)) { best = sc; bi = i; }
  }
  wave_argmax(best, bi);
  if (lane_id() == 0) {
    wbest[wave_id()] = best;
    wbi[wave_id()] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kWaves; ++w)
      if (wbest[w] > best || (wbest[w] == best && wbi[w] < bi)) { best = wbest[w]; bi = wbi[w]; }
    tokens[c] = bi;
  }
}

// Natural [n][Hkv][dh] fp16 rows (positions pos0..) <-> the tiled cache of one
// layer (kc, vc: the layer's first tile run; run: elements per run), one
// thread per element.
__global__ void __launch_bounds__(256) lf_kv_copy_kernel(_Float16 *kc, _Float16 *vc, _Float16 *k, _Float16 *v,
                                                         long long n_elems, int Hkv, int dh, int pos0,
                                                         long long run, int to_cache) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n_elems; i += (long long)gridDim.x * 256) {
    const int e = (int)(i % dh);
    const long long r = i / dh;
    const int g = (int)(r % Hkv);
    const int j = pos0 + (int)(r / Hkv);
    const size_t ki = (size_t)g * run + k_elem(dh, j, e), vi = (size_t)g * run + v_elem(dh, j, e);
    if (to_cache) {
      kc[ki] = k[i];
      vc[vi] = v[i];
    } else {
      k[i] = kc[ki];
      v[i] = vc[vi];
    }
  }
}

// Weight packing: scale every column of an fp16 matrix (rows x 8*cols8,
// 16-byte aligned) by the fp16 gain of that column (any 2-byte alignment),
// eight elements per thread.
__global__ void __launch_bounds__(256) lf_scale_columns_kernel(f16x8 *w, long long n8, int cols8,
                                                               const _Float16 *g) {
  for (long long v = (long long)blockIdx.x * 256 + threadIdx.x; v < n8; v += (long long)gridDim.x * 256) {
    const _Float16 *gg = g + (v % cols8) * 8;
    f16x8 x = w[v];
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = (_Float16)((float)x[k] * (float)gg[k]);
    w[v] = x;
  }
}

// Clears n 64-bit words (the scratch of the entry point that allocates nothing).
__global__ void __launch_bounds__(256) lf_zero_kernel(unsigned long long *p, long long n) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256) p[i] = 0ull;
}

}  // namespace

// Device memory of lf_generate_noalloc: one array per GPU (every device that
// loads this code object holds its own copy until the process ends).  Host code
// never names it directly: the array's host-side symbol is not a device
// address, so kernels and copies use the address hipGetSymbolAddress returns
// for the current device, kept per device in g_scratch_ptr.
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch_init(int device) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[device]) return hipSuccess;
  void *p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  g_scratch_ptr[device] = p;
  return hipSuccess;
}

void *noalloc_scratch(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  return g_scratch_ptr[device];
}

hipError_t launch_zero(void *p, size_t bytes, hipStream_t stream) {
  const long long n = (long long)(bytes / 8);
  if (n == 0) return hipSuccess;
  long long blocks = (n + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(lf_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     reinterpret_cast<unsigned long long *>(p), n);
  return hipGetLastError();
}

const void *monokernel_symbol(bool prefill, int qpg) {
  switch (kq_of(qpg)) {
    case 1: return prefill ? reinterpret_cast<const void *>(&lf_monokernel<true, 1>)
                           : reinterpret_cast<const void *>(&lf_monokernel<false, 1>);
    case 2: return prefill ? reinterpret_cast<const void *>(&lf_monokernel<true, 2>)
                           : reinterpret_cast<const void *>(&lf_monokernel<false, 2>);
    case 4: return prefill ? reinterpret_cast<const void *>(&lf_monokernel<true, 4>)
                           : reinterpret_cast<const void *>(&lf_monokernel<false, 4>);
    default: return prefill ? reinterpret_cast<const void *>(&lf_monokernel<true, kMaxQpg>)
                            : reinterpret_cast<const void *>(&lf_monokernel<false, kMaxQpg>);
  }
}

hipError_t launch_monokernel(const Params &p, bool prefill, hipStream_t stream) {
  void *args[] = {const_cast<Params *>(&p)};
  if (p.plain_launch)
    return hipLaunchKernel(monokernel_symbol(prefill, p.qpg), dim3(p.G), dim3(kThreads), args, (size_t)p.lds_bytes,
                           stream);
  return hipLaunchCooperativeKernel(monokernel_symbol(prefill, p.qpg), dim3(p.G), dim3(kThreads), args,
                                    (unsigned)p.lds_bytes, stream);
}

hipError_t launch_kv_copy(const Params &p, int l, int pos0, int n, void *k, void *v, bool to_cache,
                          hipStream_t stream) {
  const long long n_elems = (long long)n * p.Hkv * p.dh;
  if (n_elems <= 0) return hipSuccess;
  if (l < 0 || l >= p.L || pos0 < 0 || pos0 + n > p.kv_tiles * kKvTile) return hipErrorInvalidValue;
  const long long run = (long long)p.kv_tiles * kKvTile * p.dh;
  _Float16 *kc = reinterpret_cast<_Float16 *>(p.kcache) + (size_t)l * p.Hkv * run;
  _Float16 *vc = reinterpret_cast<_Float16 *>(p.vcache) + (size_t)l * p.Hkv * run;
  long long blocks = (n_elems + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(lf_kv_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, kc, vc,
                     reinterpret_cast<_Float16 *>(k), reinterpret_cast<_Float16 *>(v), n_elems, p.Hkv, p.dh, pos0,
                     run, to_cache ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_scale_columns(void *w, size_t rows, int cols, const void *g, hipStream_t stream) {
  if (cols <= 0 || cols % 8 || reinterpret_cast<uintptr_t>(w) % 16 || reinterpret_cast<uintptr_t>(g) % 2)
    return hipErrorInvalidValue;
  const long long n8 = (long long)rows * (cols / 8);
  if (n8 == 0) return hipSuccess;
  long long blocks = (n8 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(lf_scale_columns_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     reinterpret_cast<f16x8 *>(w), n8, cols / 8, reinterpret_cast<const _Float16 *>(g));
  return hipGetLastError();
}

hipError_t launch_test_expdef(const float *x, float *y, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  long long blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(lf_test_expdef_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, x, y, (long long)n);
  return hipGetLastError();
}

hipError_t launch_test_logdef(const float *x, float *y, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  long long blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(lf_test_logdef_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, x, y, (long long)n);
  return hipGetLastError();
}

hipError_t launch_test_gumbel(const float *logits, int n, float inv_temp, unsigned long long seed, const int *pos,
                              int m, int *tokens, hipStream_t stream) {
  if (m <= 0) return hipSuccess;
  hipLaunchKernelGGL(lf_test_gumbel_kernel, dim3(m), dim3(kThreads), 0, stream, logits, n, inv_temp, seed, pos,
                     tokens);
  return hipGetLastError();
}

hipError_t launch_test_sample(const float *logits, int n, float inv_temp, float top_p, unsigned long long seed,
                              const int *pos, int m, int *tokens, hipStream_t stream) {
  if (m <= 0) return hipSuccess;
  static bool attr = false;
  if (!attr) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&lf_test_sample_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(SampLds));
    if (e != hipSuccess) return e;
    attr = true;
  }
  hipLaunchKernelGGL(lf_test_sample_kernel, dim3(m), dim3(kThreads), sizeof(SampLds), stream, logits, n, inv_temp,
                     top_p, seed, pos, tokens);
  return hipGetLastError();
}

}  // namespace lf

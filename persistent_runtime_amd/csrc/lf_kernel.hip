// lf_kernel.hip -- the persistent batch-1 decode kernel for gfx950 (MI355X).
//
// One workgroup (8 wave64s) per compute unit runs the whole decode pass, every
// layer and the next-token choice, for n tokens in a single launch ("KOG
// LaneFormer-2B & the monokernel", sections "Pillar 3 - the monokernel runtime"
// and "Compile-time work partition").  Work is partitioned statically: every
// matrix is cut into contiguous row blocks, one per workgroup, fixed for the
// life of the state; attention is cut into (KV head, key chunk) units.
//
// Synchronisation.  There is no grid barrier.  Each workgroup owns one 32-bit
// progress word holding the last dependency level it completed; a level is one
// phase of one layer of one token, numbered monotonically across launches.  A
// consumer waits until the words of the producers it depends on reach the
// level it needs ("Cross-GPU synchronization without atomics": consumers poll
// memory the producer publishes, instead of an atomic-counter barrier).  The
// producer's wave 0 writes every datum the level publishes, then issues an
// agent-scope release fence and stores the level; the consumer's wave 0 polls
// with agent-scope loads, issues an agent-scope acquire fence, and releases its
// workgroup through a barrier.  Split-K attention partials are merged by the
// last-arriving unit of each KV head (an atomic ticket), so the merge costs no
// extra level.  Every wait is bounded: on expiry the workgroup records an error
// word and returns, and every other wait sees the error word and returns too,
// so the grid always drains.
//
// Matrix-vector products run on the vector ALUs with v_dot2_f32_f16 (fp16 x
// fp16 products, fp32 accumulation) and cross-lane sums, not on MFMA: at batch 1
// there is no dense contraction to feed matrix cores ("The fused operations,
// briefly").  Weights are read once per token with non-temporal 128-bit loads,
// 1 KB contiguous per wave instruction; the first batch of each phase is issued
// before the dependency wait so the weight stream overlaps the wait ("Weight
// streaming - keeping HBM saturated").
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lf_internal.h"

namespace lf {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kMaxQpg = 8;     // query heads per KV head supported
constexpr int kMaxDpl = 2;     // head dims per lane (head_dim <= 128)
constexpr int kMaxDPerThread = 16;  // d_model <= 16 * 512

// Thread index through an opaque copy: the kernel's outer token and layer loops
// would otherwise let the compiler hoist every per-thread address of every phase
// out of them and spill the lot.
__device__ __forceinline__ int tid_x() {
  int t = (int)threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}
__device__ __forceinline__ int lane_id() { return tid_x() & 63; }
__device__ __forceinline__ int wave_id() { return tid_x() >> 6; }

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

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}
__device__ __forceinline__ unsigned wave_min_u32(unsigned v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = min(v, (unsigned)__shfl_xor((int)v, m, 64));
  return v;
}
__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += (unsigned long long)__shfl_xor((long long)v, m, 64);
  return v;
}

// Sum over the workgroup, same order on every call (deterministic).
__device__ __forceinline__ float block_sum(float v, float *red) {
  v = wave_sum(v);
  if (lane_id() == 0) red[wave_id()] = v;
  __syncthreads();
  float t = 0.0f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) t += red[w];
  __syncthreads();
  return t;
}

__device__ __forceinline__ void block_range(int total, int parts, int b, int &p0, int &p1) {
  const int base = total / parts, rem = total % parts;
  p0 = b * base + (b < rem ? b : rem);
  p1 = p0 + base + (b < rem ? 1 : 0);
}

__device__ __forceinline__ unsigned long long now_ticks() { return __builtin_amdgcn_s_memrealtime(); }

// ------------------------------------------------------------------ sync

struct Sync {
  const Params *P;
  int *bcast;                 // LDS int used to broadcast the wait outcome
  unsigned long long spin;    // ticks spent waiting (wave 0)
  unsigned long long waits;
};

// Wait until progress[first .. first+count) >= level.  All threads call it.
// Wave 0 polls with agent-scope relaxed loads, then takes an agent-scope acquire
// fence; the barrier hands the result to the other waves.  Returns false if the
// wait timed out or another workgroup reported an error.
__device__ __forceinline__ bool wait_level(Sync &s, int first, int count, unsigned level) {
  const Params &P = *s.P;
  if (tid_x() < 64) {
    const unsigned long long t0 = now_ticks();
    int status = 0;
    unsigned it = 0;
    for (;;) {
      unsigned mn = 0xffffffffu;
      for (int i = tid_x(); i < count; i += 64)
        mn = min(mn, __hip_atomic_load(&P.progress[first + i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      mn = wave_min_u32(mn);
      if (mn >= level) { status = 1; break; }
      if ((++it & 15u) == 0 &&
          __hip_atomic_load(&P.err[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) {
        status = 2;
        break;
      }
      if (now_ticks() - t0 > P.timeout_ticks) {
        if (tid_x() == 0) {
          unsigned zero = 0u;
          if (__hip_atomic_compare_exchange_strong(&P.err[0], &zero, 1u, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT)) {
            __hip_atomic_store(&P.err[1], (unsigned)blockIdx.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&P.err[2], level, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
        status = 2;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    if (status == 1) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    __builtin_amdgcn_s_waitcnt(0);
    s.spin += now_ticks() - t0;
    s.waits += 1;
    if (tid_x() == 0) *s.bcast = status;
  }
  __syncthreads();
  const bool ok = *s.bcast == 1;
  __syncthreads();
  return ok;
}

// Publish `level` for this workgroup.  Called by wave 0 only, after wave 0 itself
// wrote every global datum the level stands for.
__device__ __forceinline__ void publish(const Params &P, unsigned level) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  if (tid_x() == 0)
    __hip_atomic_store(&P.progress[blockIdx.x], level, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------ prologues

// h = fp16(g * (x / sqrt(mean(x^2) + eps))) into LDS; x is fp32 or fp16 in global.
__device__ __forceinline__ void rmsnorm_to_lds(const float *x32, const _Float16 *x16, const _Float16 *g, int d, float eps,
                               _Float16 *h, float *red) {
  float v[kMaxDPerThread];
  float ss = 0.0f;
#pragma unroll
  for (int k = 0; k < kMaxDPerThread; ++k) {
    const int i = tid_x() + k * kThreads;
    v[k] = 0.0f;
    if (i < d) v[k] = x32 ? x32[i] : (float)x16[i];
    ss += v[k] * v[k];
  }
  const float total = block_sum(ss, red);
  const float r = sqrtf(total / (float)d + eps);
#pragma unroll
  for (int k = 0; k < kMaxDPerThread; ++k) {
    const int i = tid_x() + k * kThreads;
    if (i < d) h[i] = (_Float16)((float)g[i] * (v[k] / r));
  }
  __syncthreads();
}

// Copy an fp16 vector of n elements (n % 8 == 0) from global to LDS.
__device__ __forceinline__ void copy16_to_lds(const _Float16 *src, int n, _Float16 *h) {
  const u32x4 *s = reinterpret_cast<const u32x4 *>(src);
  u32x4 *dst = reinterpret_cast<u32x4 *>(h);
  for (int i = tid_x(); i < n / 8; i += kThreads) dst[i] = s[i];
  __syncthreads();
}

// ------------------------------------------------------------------ GEMV

// Rows [0, nrows) of a row-major fp16 matrix with kv 16-byte vectors per row,
// times the fp16 vector in LDS.  Work items are (row, chunk) with a chunk of
// 64*CV vectors; wave w takes items w, w+8, ...; the lane-sum of each item goes
// to part[item].  pre() (the dependency wait and the input prologue) runs after
// the first batch of weight loads has been issued.
template <int CV, class Pre>
__device__ __forceinline__ bool gemv_rows(const u32x4 *__restrict__ W, int kv, int nrows, int nc, const u32x4 *hl,
                          float *part, Pre &&pre) {
  constexpr int U = (16 / CV) > 0 ? (16 / CV) : 1;
  const int wave = wave_id(), lane = lane_id();
  const int nitems = nrows * nc;
  const int nb = (nitems + kWaves * U - 1) / (kWaves * U);
  u32x4 buf[U][CV];
  auto load = [&](int bi) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = (bi * U + u) * kWaves + wave;
      const int r = i / nc, c = i - r * nc;
#pragma unroll
      for (int k = 0; k < CV; ++k) {
        const int v = c * 64 * CV + 64 * k + lane;
        if (i < nitems && v < kv)
          buf[u][k] = __builtin_nontemporal_load(W + (size_t)r * kv + v);
        else
          buf[u][k] = (u32x4){0u, 0u, 0u, 0u};
      }
    }
  };
  if (nb > 0) load(0);
  if (!pre()) return false;
  for (int bi = 0; bi < nb; ++bi) {
    if (bi > 0) load(bi);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = (bi * U + u) * kWaves + wave;
      const int r = i / nc, c = i - r * nc;
      (void)r;
      float acc = 0.0f;
#pragma unroll
      for (int k = 0; k < CV; ++k) {
        const int v = c * 64 * CV + 64 * k + lane;
        if (v < kv) acc = dot8(buf[u][k], hl[v], acc);
      }
      acc = wave_sum(acc);
      if (i < nitems && lane == 0) part[i] = acc;
    }
  }
  return true;
}

// Chunk shape for a row of kv vectors: CV = 4 vectors per lane when the row
// fits in 4 per lane, else 8, and as many chunks as needed.
__device__ __forceinline__ void gemv_shape(int kv, int &cv, int &nc) {
  const int per_lane = (kv + 63) / 64;
  cv = per_lane <= 4 ? 4 : 8;
  nc = (per_lane + cv - 1) / cv;
}

template <class Pre>
__device__ __forceinline__ bool gemv_dispatch(const void *W, int kv, int nrows, const _Float16 *hl, float *part,
                                              Pre &&pre) {
  int cv, nc;
  gemv_shape(kv, cv, nc);
  const u32x4 *w = reinterpret_cast<const u32x4 *>(W);
  const u32x4 *h = reinterpret_cast<const u32x4 *>(hl);
  if (cv == 4) return gemv_rows<4>(w, kv, nrows, nc, h, part, pre);
  return gemv_rows<8>(w, kv, nrows, nc, h, part, pre);
}

// Row sum of the chunk partials (chunk order fixed).
__device__ __forceinline__ float row_value(const float *part, int row, int nc) {
  float y = 0.0f;
  for (int c = 0; c < nc; ++c) y += part[row * nc + c];
  return y;
}

__device__ __forceinline__ int chunks_for(int kv) {
  int cv, nc;
  gemv_shape(kv, cv, nc);
  return nc;
}

// ------------------------------------------------------------------ attention

__device__ __forceinline__ void attn_split(int n, int G, int Hkv, int &S, int &Lc) {
  int smax = G / Hkv;
  if (smax < 1) smax = 1;
  S = (n + kMinKeysPerUnit - 1) / kMinKeysPerUnit;
  if (S > smax) S = smax;
  if (S < 1) S = 1;
  Lc = (n + S - 1) / S;
}

// One split-K unit (KV head g, key chunk c) of layer l at position pos: partial
// (m, l, o) for the qpg query heads of group g, written to attn_part; the last
// unit of the group to arrive merges all partials into o16 (wave 0).
__device__ __forceinline__ void attn_unit(const Params &P, int l, int pos, int u, int S, int Lc, unsigned char *lds,
                          float *red) {
  const int tid = tid_x(), wave = wave_id(), lane = lane_id();
  const int qpg = P.qpg, dh = P.dh, Hkv = P.Hkv;
  const int dpl = dh / 64;
  const int g = u / S, c = u - g * S;
  const int n = pos + 1;
  const int j0 = c * Lc;
  const int j1 = min(n, j0 + Lc);
  float *qs = reinterpret_cast<float *>(lds);      // [qpg][dh]
  float *sc = qs + qpg * dh;                        // [qpg][kAttnBlock]
  float *ored = sc + qpg * kAttnBlock;              // [kWaves][qpg][dh]
  for (int i = tid; i < qpg * dh; i += kThreads) qs[i] = P.q[(size_t)g * qpg * dh + i];
  __syncthreads();
  const size_t lstride = (size_t)P.max_seq * Hkv * dh;
  const _Float16 *Kl = reinterpret_cast<const _Float16 *>(P.kcache) + (size_t)l * lstride;
  const _Float16 *Vl = reinterpret_cast<const _Float16 *>(P.vcache) + (size_t)l * lstride;
  float m_run[kMaxQpg], l_run[kMaxQpg], oacc[kMaxQpg][kMaxDpl];
#pragma unroll
  for (int h = 0; h < kMaxQpg; ++h) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.0f;
#pragma unroll
    for (int e = 0; e < kMaxDpl; ++e) oacc[h][e] = 0.0f;
  }
  for (int sb = j0; sb < j1; sb += kAttnBlock) {
    const int nb = min(kAttnBlock, j1 - sb);
    if (tid < nb) {
      const u32x4 *kr = reinterpret_cast<const u32x4 *>(Kl + ((size_t)(sb + tid) * Hkv + g) * dh);
      float s[kMaxQpg];
#pragma unroll
      for (int h = 0; h < kMaxQpg; ++h) s[h] = 0.0f;
      for (int e8 = 0; e8 < dh / 8; ++e8) {
        const f16x8 kv = __builtin_bit_cast(f16x8, kr[e8]);
#pragma unroll
        for (int h = 0; h < kMaxQpg; ++h) {
          if (h < qpg) {
            const float *qh = qs + h * dh + e8 * 8;
#pragma unroll
            for (int i = 0; i < 8; ++i) s[h] += qh[i] * (float)kv[i];
          }
        }
      }
#pragma unroll
      for (int h = 0; h < kMaxQpg; ++h)
        if (h < qpg) sc[h * kAttnBlock + tid] = s[h] * P.inv_sqrt_dh;
    }
    __syncthreads();
    float m_new[kMaxQpg], alpha[kMaxQpg];
#pragma unroll
    for (int h = 0; h < kMaxQpg; ++h) {
      if (h < qpg) {
        float v = tid < nb ? sc[h * kAttnBlock + tid] : -INFINITY;
        v = wave_max(v);
        if (lane == 0) red[wave * kMaxQpg + h] = v;
      }
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < kMaxQpg; ++h) {
      m_new[h] = m_run[h];
      alpha[h] = 0.0f;
      if (h < qpg) {
        float mb = -INFINITY;
        for (int w = 0; w < kWaves; ++w) mb = fmaxf(mb, red[w * kMaxQpg + h]);
        m_new[h] = fmaxf(m_run[h], mb);
        alpha[h] = __expf(m_run[h] - m_new[h]);
      }
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < kMaxQpg; ++h) {
      if (h < qpg) {
        float p = 0.0f;
        if (tid < nb) {
          p = __expf(sc[h * kAttnBlock + tid] - m_new[h]);
          sc[h * kAttnBlock + tid] = p;
        }
        p = wave_sum(p);
        if (lane == 0) red[wave * kMaxQpg + h] = p;
      }
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < kMaxQpg; ++h) {
      if (h < qpg) {
        float lb = 0.0f;
        for (int w = 0; w < kWaves; ++w) lb += red[w * kMaxQpg + h];
        l_run[h] = l_run[h] * alpha[h] + lb;
#pragma unroll
        for (int e = 0; e < kMaxDpl; ++e) oacc[h][e] *= alpha[h];
      }
      m_run[h] = m_new[h];
    }
    for (int jj = wave; jj < nb; jj += kWaves) {
      const _Float16 *vr = Vl + ((size_t)(sb + jj) * Hkv + g) * dh + lane * dpl;
      float v0, v1 = 0.0f;
      if (dpl == 2) {
        const f16x2 vv = *reinterpret_cast<const f16x2 *>(vr);
        v0 = (float)vv.x;
        v1 = (float)vv.y;
      } else {
        v0 = (float)vr[0];
      }
#pragma unroll
      for (int h = 0; h < kMaxQpg; ++h) {
        if (h < qpg) {
          const float p = sc[h * kAttnBlock + jj];
          oacc[h][0] += p * v0;
          oacc[h][1] += p * v1;
        }
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int h = 0; h < kMaxQpg; ++h)
    if (h < qpg) {
#pragma unroll
      for (int e = 0; e < kMaxDpl; ++e)
        if (e < dpl) ored[(wave * qpg + h) * dh + lane * dpl + e] = oacc[h][e];
    }
  __syncthreads();
  if (wave == 0) {
    const int stride = dh + 2;
    float *dst = P.attn_part + (size_t)u * qpg * stride;
    for (int h = 0; h < qpg; ++h) {
      for (int e = lane; e < dh; e += 64) {
        float o = 0.0f;
        for (int w = 0; w < kWaves; ++w) o += ored[(w * qpg + h) * dh + e];
        dst[h * stride + 2 + e] = o;
      }
      if (lane == 0) {
        dst[h * stride + 0] = m_run[h];
        dst[h * stride + 1] = l_run[h];
      }
    }
    // Arrival ticket of group g: the unit that completes the count merges.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    unsigned old = 0;
    if (lane == 0)
      old = __hip_atomic_fetch_add(&P.tickets[l * Hkv + g], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    old = __shfl(old, 0, 64);
    if (old == (unsigned)(S - 1)) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      const float *src = P.attn_part + (size_t)g * S * qpg * stride;
      _Float16 *o16 = reinterpret_cast<_Float16 *>(P.o16) + (size_t)g * qpg * dh;
      for (int h = 0; h < qpg; ++h) {
        float M = -INFINITY;
        for (int cc = 0; cc < S; ++cc) M = fmaxf(M, src[(cc * qpg + h) * stride + 0]);
        float Lsum = 0.0f;
        for (int cc = 0; cc < S; ++cc) {
          const float *pp = src + (cc * qpg + h) * stride;
          Lsum += __expf(pp[0] - M) * pp[1];
        }
        for (int e = lane; e < dh; e += 64) {
          float o = 0.0f;
          for (int cc = 0; cc < S; ++cc) {
            const float *pp = src + (cc * qpg + h) * stride;
            o += __expf(pp[0] - M) * pp[2 + e];
          }
          o16[h * dh + e] = (_Float16)(o / Lsum);
        }
      }
      if (lane == 0)
        __hip_atomic_store(&P.tickets[l * Hkv + g], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __syncthreads();
}

// ------------------------------------------------------------------ sampler

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

__device__ __forceinline__ float scaled_logit(const float *logits, int i, float inv_temp) {
#pragma clang fp contract(off)
  float z = logits[i] * inv_temp;
  return z == 0.0f ? 0.0f : z;   // one zero: -0 and +0 order as equal
}

__device__ __forceinline__ unsigned long long mass_of(float z, float zmax) {
#pragma clang fp contract(off)
  const float dz = z - zmax;
  if (dz < -23.0f) return 0ull;
  return (unsigned long long)(expdef(dz) * 4294967296.0f);
}

// Order key: larger key = earlier in (z descending, index ascending) order.
__device__ __forceinline__ unsigned long long order_key(float z, int i) {
  unsigned b = __float_as_uint(z);
  b = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((unsigned long long)b << 32) | (unsigned long long)(0xffffffffu - (unsigned)i);
}

struct SampLds {
  unsigned long long mass[256];
  unsigned cnt[256];
  unsigned long long wtot[kWaves];
  unsigned long long sel[4];   // prefix, mask, mass_above, misc
  float fred[kWaves];
  int ibc[4];
};

__device__ __forceinline__ unsigned long long block_sum_u64(unsigned long long v, SampLds *s) {
  v = wave_sum_u64(v);
  if (lane_id() == 0) s->wtot[wave_id()] = v;
  __syncthreads();
  unsigned long long t = 0;
  for (int w = 0; w < kWaves; ++w) t += s->wtot[w];
  __syncthreads();
  return t;
}

// Temperature / top-p nucleus sampling with integer masses, by one workgroup:
// z = logit * inv_temp; q_i = floor(E(z_i - z*) * 2^32) (0 below -23); the
// nucleus is the shortest prefix of the (z desc, index asc) order whose mass
// reaches ceil(top_p * C_V) in fp64, found by an 8-pass radix select on a 64-bit
// order key; the Philox draw t = floor(r * C_N / 2^64) with r from counter
// (pos, 0, 0, 0); the token is the first nucleus member in index order whose
// running mass exceeds t.
__device__ __forceinline__ int sample_topp(const float *logits, int V, float inv_temp, float top_p,
                           unsigned long long seed, int pos, SampLds *s) {
  const int tid = tid_x();
  float zm = -INFINITY;
  for (int i = tid; i < V; i += kThreads) zm = fmaxf(zm, scaled_logit(logits, i, inv_temp));
  zm = wave_max(zm);
  if (lane_id() == 0) s->fred[wave_id()] = zm;
  __syncthreads();
  float zmax = -INFINITY;
  for (int w = 0; w < kWaves; ++w) zmax = fmaxf(zmax, s->fred[w]);
  __syncthreads();
  unsigned long long part = 0;
  for (int i = tid; i < V; i += kThreads) part += mass_of(scaled_logit(logits, i, inv_temp), zmax);
  const unsigned long long CV = block_sum_u64(part, s);
  const unsigned long long Mstar = (unsigned long long)ceil((double)top_p * (double)CV);
  unsigned long long prefix = 0, pmask = 0, above = 0;
  for (int shift = 56; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += kThreads) { s->mass[i] = 0; s->cnt[i] = 0; }
    __syncthreads();
    for (int i = tid; i < V; i += kThreads) {
      const float z = scaled_logit(logits, i, inv_temp);
      const unsigned long long key = order_key(z, i);
      if ((key & pmask) == prefix) {
        const int dg = (int)((key >> shift) & 255ull);
        atomicAdd(&s->mass[dg], mass_of(z, zmax));
        atomicAdd(&s->cnt[dg], 1u);
      }
    }
    __syncthreads();
    if (tid == 0) {
      unsigned long long cum = 0;
      int pick = -1, lowest = -1;
      unsigned long long cum_lowest = 0;
      for (int dg = 255; dg >= 0; --dg) {
        if (s->cnt[dg] == 0) continue;
        if (above + cum + s->mass[dg] >= Mstar) { pick = dg; break; }
        lowest = dg;
        cum_lowest = cum;
        cum += s->mass[dg];
      }
      if (pick < 0) { pick = lowest; cum = cum_lowest; }   // mass never reached: take every token
      s->sel[0] = prefix | ((unsigned long long)pick << shift);
      s->sel[1] = pmask | (255ull << shift);
      s->sel[2] = above + cum;
    }
    __syncthreads();
    prefix = s->sel[0];
    pmask = s->sel[1];
    above = s->sel[2];
    __syncthreads();
  }
  const unsigned long long kappa = prefix;
  // nucleus mass; each thread owns a contiguous index block for the final scan
  const int blk = (V + kThreads - 1) / kThreads;
  const int i0 = min(V, tid * blk), i1 = min(V, i0 + blk);
  unsigned long long local = 0;
  for (int i = i0; i < i1; ++i) {
    const float z = scaled_logit(logits, i, inv_temp);
    if (order_key(z, i) >= kappa) local += mass_of(z, zmax);
  }
  const unsigned long long CN = block_sum_u64(local, s);
  unsigned ctr[4] = {(unsigned)pos, 0u, 0u, 0u};
  philox4x32_10(ctr, (unsigned)(seed & 0xffffffffull), (unsigned)(seed >> 32));
  const unsigned long long r = ((unsigned long long)ctr[1] << 32) | ctr[0];
  const unsigned long long t = __umul64hi(r, CN);
  // exclusive scan of the per-thread masses (thread order = index order)
  unsigned long long incl = local;
  for (int off = 1; off < 64; off <<= 1) {
    const unsigned long long y = (unsigned long long)__shfl_up((long long)incl, off, 64);
    if (lane_id() >= off) incl += y;
  }
  if (lane_id() == 63) s->wtot[wave_id()] = incl;
  if (tid == 0) s->ibc[0] = -1;
  __syncthreads();
  unsigned long long base = 0;
  for (int w = 0; w < wave_id(); ++w) base += s->wtot[w];
  const unsigned long long excl = base + incl - local;
  if (local > 0 && excl <= t && t < excl + local) {
    unsigned long long run = excl;
    for (int i = i0; i < i1; ++i) {
      const float z = scaled_logit(logits, i, inv_temp);
      if (order_key(z, i) < kappa) continue;
      run += mass_of(z, zmax);
      if (run > t) { s->ibc[0] = i; break; }
    }
  }
  __syncthreads();
  const int tok = s->ibc[0];
  __syncthreads();
  return tok;
}

// ------------------------------------------------------------------ the kernel

// kPrefill: teacher-forced prompt tokens read from in_tokens[], no logits and no
// sampling; each token's first layer waits for the previous token's last layer.
template <bool kPrefill>
__global__ void __launch_bounds__(kThreads, 1) lf_monokernel(Params P) {
  extern __shared__ __align__(16) unsigned char smem[];
  _Float16 *hl = reinterpret_cast<_Float16 *>(smem + P.lds_h);
  float *part = reinterpret_cast<float *>(smem + P.lds_part);
  float *red = reinterpret_cast<float *>(smem + P.lds_red);   // 64 floats + 16 ints
  int *ibc = reinterpret_cast<int *>(red + 64);
  unsigned char *alds = smem + P.lds_attn;
  const int b = blockIdx.x, G = P.G, wave = wave_id(), lane = lane_id();
  Sync sy{&P, ibc, 0ull, 0ull};
  const unsigned long long kt0 = now_ticks();
  const int d = P.d, dh = P.dh;
  const int kv_d = d / 8;
  const _Float16 *emb = reinterpret_cast<const _Float16 *>(P.tok_emb);
  bool ok = true;

  for (int t = 0; t < P.n_tokens && ok; ++t) {
    const int pos = P.pos0 + t;
    const unsigned lv0 = P.level_base + (unsigned)t * (unsigned)P.levels_per_token;
    int token = kPrefill ? P.in_tokens[t] : P.token0;
    for (int l = 0; l < P.L && ok; ++l) {
      const LayerW &W = P.layers[l];
      const unsigned lvl = lv0 + (unsigned)(l * PH_PER_LAYER);
      const _Float16 *attn_norm = reinterpret_cast<const _Float16 *>(W.attn_norm);
      const _Float16 *ffn_norm = reinterpret_cast<const _Float16 *>(W.ffn_norm);

      // ---------------- QKV + rotary + KV append
      {
        int p0, p1;
        block_range(P.nqkv / 2, G, b, p0, p1);
        const int r0 = 2 * p0, nrows = 2 * (p1 - p0);
        auto pre = [&]() __attribute__((always_inline)) -> bool {
          if (l == 0) {
            if (kPrefill) {
              if (t > 0 && !wait_level(sy, 0, G, lv0)) return false;
            } else if (t > 0 && !P.hidden_io) {
              if (!wait_level(sy, 0, 1, lv0)) return false;
              token = *P.tok_slot;
            }
            if (P.hidden_io)
              rmsnorm_to_lds(P.x_hidden, nullptr, attn_norm, d, P.eps, hl, red);
            else
              rmsnorm_to_lds(nullptr, emb + (size_t)token * d, attn_norm, d, P.eps, hl, red);
          } else {
            if (!wait_level(sy, 0, G, lvl)) return false;
            rmsnorm_to_lds(P.x_out, nullptr, attn_norm, d, P.eps, hl, red);
          }
          return true;
        };
        const u32x4 *wq = reinterpret_cast<const u32x4 *>(W.wqkv) + (size_t)r0 * kv_d;
        if (!gemv_dispatch(wq, kv_d, nrows, hl, part, pre)) { ok = false; break; }
        __syncthreads();
        if (wave == 0) {
          const int nc = chunks_for(kv_d);
          const int half = dh / 2;
          const int nq = P.Hq * dh, nk = P.Hkv * dh;
          const size_t kvrow = ((size_t)l * P.max_seq + pos) * (size_t)nk;
          _Float16 *kc = reinterpret_cast<_Float16 *>(P.kcache) + kvrow;
          _Float16 *vc = reinterpret_cast<_Float16 *>(P.vcache) + kvrow;
          for (int i = lane; i < nrows / 2; i += 64) {
            const float a = row_value(part, 2 * i, nc), bb = row_value(part, 2 * i + 1, nc);
            const int r = r0 + 2 * i;
            if (r < nq + nk) {
              const int rr = r < nq ? r : r - nq;
              const int hd = rr / dh, k = (rr % dh) / 2;
              const float cs = P.rope[((size_t)pos * half + k) * 2 + 0];
              const float sn = P.rope[((size_t)pos * half + k) * 2 + 1];
              const float y0 = a * cs - bb * sn, y1 = bb * cs + a * sn;
              if (r < nq) {
                P.q[hd * dh + k] = y0;
                P.q[hd * dh + k + half] = y1;
              } else {
                kc[hd * dh + k] = (_Float16)y0;
                kc[hd * dh + k + half] = (_Float16)y1;
              }
            } else {
              const int rv = r - nq - nk;
              vc[rv] = (_Float16)a;
              vc[rv + 1] = (_Float16)bb;
            }
          }
          publish(P, lvl + PH_QKV);
        }
      }

      // ---------------- attention (split-K, last arriver merges)
      {
        if (!wait_level(sy, 0, G, lvl + PH_QKV)) { ok = false; break; }
        int S, Lc;
        attn_split(pos + 1, G, P.Hkv, S, Lc);
        const int units = P.Hkv * S;
        for (int u = b; u < units; u += G) attn_unit(P, l, pos, u, S, Lc, alds, red);
        if (wave == 0) publish(P, lvl + PH_ATTN);
      }

      // ---------------- output projection + residual
      {
        int p0, p1;
        block_range(d / 2, G, b, p0, p1);
        const int r0 = 2 * p0, nrows = 2 * (p1 - p0);
        const int kv = P.Hq * dh / 8;
        auto pre = [&]() __attribute__((always_inline)) -> bool {
          if (!wait_level(sy, 0, G, lvl + PH_ATTN)) return false;
          copy16_to_lds(reinterpret_cast<const _Float16 *>(P.o16), P.Hq * dh, hl);
          return true;
        };
        const u32x4 *wo = reinterpret_cast<const u32x4 *>(W.wo) + (size_t)r0 * kv;
        if (!gemv_dispatch(wo, kv, nrows, hl, part, pre)) { ok = false; break; }
        __syncthreads();
        if (wave == 0) {
          const int nc = chunks_for(kv);
          for (int i = lane; i < nrows; i += 64) {
            const int r = r0 + i;
            float xin;
            if (l > 0) xin = P.x_out[r];
            else if (P.hidden_io) xin = P.x_hidden[r];
            else xin = (float)emb[(size_t)token * d + r];
            P.x_mid[r] = xin + row_value(part, i, nc);
          }
          publish(P, lvl + PH_O);
        }
      }

      // ---------------- FFN norm + gate/up + SwiGLU
      {
        int p0, p1;
        block_range(P.F, G, b, p0, p1);
        const int r0 = 2 * p0, nrows = 2 * (p1 - p0);
        auto pre = [&]() __attribute__((always_inline)) -> bool {
          if (!wait_level(sy, 0, G, lvl + PH_O)) return false;
          rmsnorm_to_lds(P.x_mid, nullptr, ffn_norm, d, P.eps, hl, red);
          return true;
        };
        const u32x4 *wgu = reinterpret_cast<const u32x4 *>(W.wgu) + (size_t)r0 * kv_d;
        if (!gemv_dispatch(wgu, kv_d, nrows, hl, part, pre)) { ok = false; break; }
        __syncthreads();
        if (wave == 0) {
          const int nc = chunks_for(kv_d);
          _Float16 *a16 = reinterpret_cast<_Float16 *>(P.a16);
          for (int i = lane; i < nrows / 2; i += 64) {
            const float gt = row_value(part, 2 * i, nc), up = row_value(part, 2 * i + 1, nc);
            const float sg = gt / (1.0f + __expf(-gt));
            a16[p0 + i] = (_Float16)(sg * up);
          }
          publish(P, lvl + PH_GU);
        }
      }

      // ---------------- down projection + residual
      {
        int p0, p1;
        block_range(d / 2, G, b, p0, p1);
        const int r0 = 2 * p0, nrows = 2 * (p1 - p0);
        const int kv = P.F / 8;
        auto pre = [&]() __attribute__((always_inline)) -> bool {
          if (!wait_level(sy, 0, G, lvl + PH_GU)) return false;
          copy16_to_lds(reinterpret_cast<const _Float16 *>(P.a16), P.F, hl);
          return true;
        };
        const u32x4 *wd = reinterpret_cast<const u32x4 *>(W.wd) + (size_t)r0 * kv;
        if (!gemv_dispatch(wd, kv, nrows, hl, part, pre)) { ok = false; break; }
        __syncthreads();
        if (wave == 0) {
          const int nc = chunks_for(kv);
          for (int i = lane; i < nrows; i += 64) {
            const int r = r0 + i;
            P.x_out[r] = P.x_mid[r] + row_value(part, i, nc);
          }
          publish(P, lvl + PH_D);
        }
      }
    }
    if (kPrefill || !ok || P.hidden_io) continue;

    // ---------------- final norm + lm_head + local argmax
    const unsigned lvl_lm = lv0 + (unsigned)(P.L * PH_PER_LAYER) + 1u;
    {
      int p0, p1;
      block_range(P.V / 2, G, b, p0, p1);
      const int r0 = 2 * p0, nrows = 2 * (p1 - p0);
      auto pre = [&]() __attribute__((always_inline)) -> bool {
        if (!wait_level(sy, 0, G, lvl_lm - 1u)) return false;
        rmsnorm_to_lds(P.x_out, nullptr, reinterpret_cast<const _Float16 *>(P.final_norm), d, P.eps, hl, red);
        return true;
      };
      const u32x4 *wl = reinterpret_cast<const u32x4 *>(P.lm_head) + (size_t)r0 * kv_d;
      if (!gemv_dispatch(wl, kv_d, nrows, hl, part, pre)) { ok = false; break; }
      __syncthreads();
      if (wave == 0) {
        const int nc = chunks_for(kv_d);
        float best = -INFINITY;
        int bi = 0x7fffffff;
        for (int i = lane; i < nrows; i += 64) {
          const float y = row_value(part, i, nc);
          P.logits[r0 + i] = y;
          if (y > best || (y == best && r0 + i < bi)) { best = y; bi = r0 + i; }
        }
        for (int m = 32; m >= 1; m >>= 1) {
          const float ov = __shfl_xor(best, m, 64);
          const int oi = __shfl_xor(bi, m, 64);
          if (ov > best || (ov == best && oi < bi)) { best = ov; bi = oi; }
        }
        if (lane == 0) { P.lm_val[b] = best; P.lm_idx[b] = bi; }
        publish(P, lvl_lm);
      }
    }

    // ---------------- next token (workgroup 0)
    if (b == 0) {
      if (!wait_level(sy, 0, G, lvl_lm)) { ok = false; break; }
      int tok;
      if (P.sampling) {
        tok = sample_topp(P.logits, P.V, P.inv_temp, P.top_p, P.seed, pos, reinterpret_cast<SampLds *>(alds));
      } else {
        float best = -INFINITY;
        int bi = 0x7fffffff;
        for (int i = tid_x(); i < G; i += kThreads) {
          const float v = P.lm_val[i];
          const int ix = P.lm_idx[i];
          if (v > best || (v == best && ix < bi)) { best = v; bi = ix; }
        }
        for (int m = 32; m >= 1; m >>= 1) {
          const float ov = __shfl_xor(best, m, 64);
          const int oi = __shfl_xor(bi, m, 64);
          if (ov > best || (ov == best && oi < bi)) { best = ov; bi = oi; }
        }
        if (lane == 0) { red[wave] = best; ibc[4 + wave] = bi; }
        __syncthreads();
        best = red[0];
        bi = ibc[4];
        for (int w = 1; w < kWaves; ++w)
          if (red[w] > best || (red[w] == best && ibc[4 + w] < bi)) { best = red[w]; bi = ibc[4 + w]; }
        __syncthreads();
        tok = bi;
      }
      if (tok < 0 || tok >= P.V) {   // never expected; keeps the next embedding read in bounds
        if (tid_x() == 0) __hip_atomic_store(&P.err[3], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        tok = 0;
      }
      if (wave == 0) {
        if (lane == 0) {
          *P.tok_slot = tok;
          P.out_tokens[t] = tok;
        }
        publish(P, lvl_lm + 1u);
      }
    }
  }
  if ((P.flags & 4u) && tid_x() == 0) {
    unsigned xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    P.stats[b * 4 + 0] = sy.spin;
    P.stats[b * 4 + 1] = sy.waits;
    P.stats[b * 4 + 2] = xcc & 0xfu;
    P.stats[b * 4 + 3] = now_ticks() - kt0;
  }
}

__global__ void lf_test_expdef_kernel(const float *x, float *y, long long n) {
  for (long long i = (long long)blockIdx.x * blockDim.x + tid_x(); i < n; i += (long long)gridDim.x * blockDim.x)
    y[i] = expdef(x[i]);
}

__global__ void __launch_bounds__(kThreads) lf_test_sample_kernel(const float *logits, int n, float inv_temp,
                                                                 float top_p, unsigned long long seed,
                                                                 const int *pos, int *tokens) {
  __shared__ SampLds s;
  const int c = blockIdx.x;
  const int tok = sample_topp(logits + (size_t)c * n, n, inv_temp, top_p, seed, pos[c], &s);
  if (tid_x() == 0) tokens[c] = tok;
}

}  // namespace

const void *monokernel_symbol(bool prefill) {
  return prefill ? reinterpret_cast<const void *>(&lf_monokernel<true>)
                 : reinterpret_cast<const void *>(&lf_monokernel<false>);
}

hipError_t launch_monokernel(const Params &p, bool prefill, hipStream_t stream) {
  void *args[] = {const_cast<Params *>(&p)};
  return hipLaunchCooperativeKernel(monokernel_symbol(prefill), dim3(p.G), dim3(kThreads), args,
                                    (unsigned)p.lds_bytes, stream);
}

hipError_t launch_test_expdef(const float *x, float *y, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  long long blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(lf_test_expdef_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, x, y, (long long)n);
  return hipGetLastError();
}

hipError_t launch_test_sample(const float *logits, int n, float inv_temp, float top_p, unsigned long long seed,
                              const int *pos, int m, int *tokens, hipStream_t stream) {
  if (m <= 0) return hipSuccess;
  hipLaunchKernelGGL(lf_test_sample_kernel, dim3(m), dim3(kThreads), 0, stream, logits, n, inv_temp, top_p,
                     seed, pos, tokens);
  return hipGetLastError();
}

}  // namespace lf

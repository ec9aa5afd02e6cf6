// ksa_attention.h -- device bodies of the decode attention kernels:
// decode attention of every query head over a token list of its KV head (the
// selected blocks of the Kinetics explainer, section 五; one token set shared
// by every head of a sequence, LessIsMore explainer, section 五; or the dense
// range [0, T), Kinetics explainer, section 四).  Kernels that own a
// (sequence, KV head) row call attn_row_valu or attn_row_mfma on it.
//
// Work decomposition.  A (sequence b, KV head g) row's token list is a
// sequence of "virtual positions" p = 0..L-1 (block list: p -> token
// idx[p / Bs] * Bs + p % Bs; token list: p -> idx[p]; dense: p -> p).  It is
// cut into chunks of CH positions.  `splits` workgroups share a row; each
// covers a contiguous run of chunks and its waves take the run's chunks
// round-robin.
//
// Inside a wave, a group of LPT lanes (a "slot") holds one token row: each
// lane owns 16 bytes (8 bf16 or 4 fp32 channels) of K and V, so one 16-byte
// load per lane reads 64/LPT consecutive-position rows and a Bs-aligned block
// of 16 bf16 tokens is four fully used 1 KB loads.  All G query heads of the
// group are handled by the same lanes, so each K/V byte is read once per
// group (the GQA sharing the LessIsMore explainer's kernel relies on).
//
// Numerics.  q is pre-scaled by sm_scale*log2(e); logits accumulate in fp32
// (bf16 x bf16 products are exact), the per-slot online softmax keeps
// (m, l, acc) in the log2 domain with hardware exp2, and P stays fp32 for the
// P.V accumulation.  States are merged slot -> wave -> workgroup -> split in
// a fixed order, so results are bitwise repeatable; the split merge is done
// by the row's last workgroup to finish (no separate merge launch).
//
// Pipelining.  The workgroup's slice of the index list is staged in LDS once;
// while a wave computes one chunk, the K/V loads of its next
// kPrefetchChunks chunks are in flight (a ring of register buffers).
#pragma once

#include <float.h>

#include <type_traits>

#include "ksa_device.h"
#include "ksa_internal.h"

namespace ksa {

// waves a workgroup may have (the LDS merge arrays are sized for it)
#ifndef KSA_MAX_WAVES
#define KSA_MAX_WAVES 8
#endif
constexpr int kMaxWaves = KSA_MAX_WAVES;
constexpr int kMaxSplits = 4096;  // workgroups per row (arrival counts are 16-bit)
// Launch-plan knobs: workgroups per CU the split count aims at, and the
// fewest chunks a wave is planned to stream.  One workgroup per CU is the
// measured best for the short rows of a shared token set (c4 shape: 2 / 3 /
// 4 per CU took 34.8 / 44.7 / 50.8 us against 29.4): a workgroup's fixed
// costs (index staging, pipeline fill, the wave and split merges) outweigh
// the extra bytes in flight once a row's 2048 tokens are cut finer.
#ifndef KSA_PLAN_WGS_PER_CU
#define KSA_PLAN_WGS_PER_CU 1
#endif
#ifndef KSA_PLAN_MIN_CHUNKS
#define KSA_PLAN_MIN_CHUNKS 8
#endif
// chunks whose K/V loads are in flight while a wave computes another
#ifndef KSA_ATTN_PREFETCH
#define KSA_ATTN_PREFETCH 1
#endif
constexpr int kPrefetchChunks = KSA_ATTN_PREFETCH;
// the same for the MFMA body (one chunk in flight is the measured best for
// the token-set and block shapes it serves)
#ifndef KSA_MFMA_PREFETCH
#define KSA_MFMA_PREFETCH 1
#endif
constexpr int kMfmaPrefetch = KSA_MFMA_PREFETCH;
// K/V rows are streamed once per call: nontemporal loads keep them from
// displacing reusable lines in L2 and the Infinity Cache.
#ifndef KSA_NT_LOADS
#define KSA_NT_LOADS 1
#endif
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* idx;
  int count;       // idx entries per row (block list) or per sequence (token list)
  Dims d;
  int ltot;        // virtual positions per row
  int bs_shift;    // log2(Bs) when Bs is a power of two, else -1
  int splits, cps;
  float qscale;    // sm_scale * log2(e)
  float* out;
  float* lse;
  float* part_acc; // [rows, splits, G, D]
  float* part_ml;  // [rows, splits, G, 2]
  // split rows: one arrival word per row, [tag:48 | arrivals:16]; the
  // workgroup that completes a row's count merges the row (see merge_waves)
  unsigned long long* arrive;
  unsigned long long tag;  // this call's 47-bit tag (bit 47 clear)
  // paged cache (kind 3): pages of each sequence's logical blocks, lengths
  const int32_t* table;    // [B, tstride]
  const int32_t* seq_lens; // [B]
  int tstride;             // max_blocks
  int page_rows;           // Hkv * Bs: token rows per page
  // dense (kind 2) on MFMA: the order keys of the raw logits of history
  // tokens t < vhist go to vkeys [B, Hq, vkstride] (the vote's scores); a
  // paged dense walk sets vhist per row from vbudget and vwindow
  uint32_t* vkeys;
  int vkstride;
  int vhist;
  int vbudget, vwindow;
  // kind 4 (one token list per query head): the rows are query heads
  // (d.Hkv = Hq, d.G = 1) and row (b, h) reads KV head h / kv_div
  int kv_div;
};

// Kernel arguments of one attention call (host side).  kind: 0 = selected
// blocks, 1 = shared token list, 2 = dense range [0, T), 3 = blocks of a
// paged cache (logical ids and their pages staged in LDS; the per-row
// length is set by the kernel), 4 = a token list per query head, 5 = a
// shared token list over a paged cache (ids and pool rows staged in LDS).
inline AttnArgs make_attn_args(const Dims& d, int kind, const void* q, const void* k, const void* v,
                               const int32_t* idx, int count, float* out, float* lse,
                               void* workspace, const AttnPlan& plan) {
  AttnArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.idx = idx;
  a.count = count;
  a.d = d;
  a.ltot = (kind == 0 || kind == 3) ? count * d.Bs : (kind == 2 ? d.T : count);
  a.bs_shift = -1;
  if ((kind == 0 || kind == 3) && (d.Bs & (d.Bs - 1)) == 0) {
    int sh = 0;
    while ((1 << sh) < d.Bs) ++sh;
    a.bs_shift = sh;
  }
  a.splits = plan.splits;
  a.cps = plan.cps;
  a.qscale = d.scale * kLog2e;
  a.out = out;
  a.lse = lse;
  const size_t rows = (size_t)d.B * d.Hkv;
  // workspace of a split plan: arrival words, then the partial states
  a.arrive = (unsigned long long*)workspace;
  a.part_acc = workspace ? (float*)((char*)workspace + arrival_bytes(rows)) : nullptr;
  a.part_ml = workspace ? a.part_acc + rows * plan.splits * d.G * d.D : nullptr;
  a.tag = 0;
  a.table = nullptr;
  a.seq_lens = nullptr;
  a.tstride = 0;
  a.page_rows = d.Hkv * d.Bs;
  a.vkeys = nullptr;
  a.vkstride = 0;
  a.vhist = 0;
  a.vbudget = 0;
  a.vwindow = 0;
  a.kv_div = 1;
  return a;
}

// Token rows of the NI rows a lane loads for chunk c (token ids; for a paged
// cache, rows page * page_rows + r of the pool seen from the KV head's first
// row).  Indices of the workgroup's range are staged in LDS (s_idx, entries
// from e0 on; pages in s_pg for kind 3).
template <int KIND, int CH, int SPW, int NI>
__device__ __forceinline__ void resolve_chunk(const AttnArgs& a, const int* s_idx, const int* s_pg,
                                              int e0, int slot, int c, int* tok, bool* ok) {
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int p = c * CH + i * SPW + slot;
    if constexpr (KIND == 2) {
      ok[i] = p < a.d.T;
      tok[i] = ok[i] ? p : 0;
    } else if constexpr (KIND == 1 || KIND == 4) {
      ok[i] = p < a.ltot;
      const int at = min(max(p - e0, 0), kIdxStage - 1);  // in range whenever ok
      tok[i] = ok[i] ? s_idx[at] : 0;
    } else if constexpr (KIND == 5 || KIND == 6) {
      // a token list over a paged cache (5: shared by the sequence's heads, 6:
      // one per query head): s_idx holds the token ids (negative: padding,
      // skipped), s_pg their pool rows
      const int at = min(max(p - e0, 0), kIdxStage - 1);
      ok[i] = p < a.ltot && s_idx[at] >= 0 && s_idx[at] < a.d.T;
      tok[i] = ok[i] ? s_pg[at] : 0;
    } else {
      ok[i] = p < a.ltot;
      int q, r;
      if (a.bs_shift >= 0) {
        q = p >> a.bs_shift;
        r = p & ((1 << a.bs_shift) - 1);
      } else {
        q = p / a.d.Bs;
        r = p - q * a.d.Bs;
      }
      const int at = min(max(q - e0, 0), kIdxStage - 1);  // in range whenever ok
      const int blk = ok[i] ? s_idx[at] : 0;
      const int t = blk * a.d.Bs + r;
      ok[i] = ok[i] && t < a.d.T && (KIND != 3 || blk >= 0);  // paged lists pad with -1
      if constexpr (KIND == 3)
        tok[i] = ok[i] ? s_pg[at] * a.page_rows + r : 0;
      else
        tok[i] = ok[i] ? t : 0;
    }
  }
}

template <typename T>
__device__ __forceinline__ uint4 ld_kv(const T* p) {
#if KSA_NT_LOADS
  return ld16_stream(p);
#else
  return ld16(p);
#endif
}

template <typename T, int D, int KIND, int CH, int SPW, int NI>
__device__ __forceinline__ void load_chunk(const AttnArgs& a, const int* s_idx, const int* s_pg,
                                           int e0, int slot, int c, const T* kbase,
                                           const T* vbase, uint4* kr, uint4* vr, bool* okr) {
  int tok[NI];
  resolve_chunk<KIND, CH, SPW, NI>(a, s_idx, s_pg, e0, slot, c, tok, okr);
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    kr[i] = ld_kv(kbase + (int64_t)tok[i] * D);
    vr[i] = ld_kv(vbase + (int64_t)tok[i] * D);
  }
}

// bf16 logits on v_dot2c_f32_bf16: q and K stay packed (no widening), two
// exact products per instruction, and the scale is applied to the lane
// group's sum; fp32 keeps the widened, pre-scaled q of the FMA chain.
#ifndef KSA_VALU_DOT2
#define KSA_VALU_DOT2 1
#endif
template <typename T>
constexpr bool kDot2 = KSA_VALU_DOT2 && std::is_same<T, uint16_t>::value;

template <typename T, int D, int G, int NI, int LPT>
__device__ __forceinline__ void compute_chunk(const float (&qv)[G][KV<T>::EPL], const uint4 (&qb)[G],
                                              float qscale, const uint4* kc, const uint4* vc,
                                              const bool* okc, float* m, float* l,
                                              float (&acc)[G][KV<T>::EPL]) {
  constexpr int EPL = KV<T>::EPL;
  // logits of the NI tokens for every head of the group
  float s[NI][G];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    if constexpr (kDot2<T>) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float p = dot2_bf16(qb[h].x, kc[i].x, 0.f);
        p = dot2_bf16(qb[h].y, kc[i].y, p);
        p = dot2_bf16(qb[h].z, kc[i].z, p);
        p = dot2_bf16(qb[h].w, kc[i].w, p);
        s[i][h] = group_sum<LPT>(p) * qscale;
      }
    } else {
      float f[EPL];
      KV<T>::widen(kc[i], f);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float p = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) p = fmaf(qv[h][e], f[e], p);
        s[i][h] = group_sum<LPT>(p);
      }
    }
  }
  // online softmax update, once per chunk
  float alpha[G];
  bool rescale = false;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float mx = m[h];
#pragma unroll
    for (int i = 0; i < NI; ++i)
      if (okc[i]) mx = fmaxf(mx, s[i][h]);
    alpha[h] = fast_exp2(m[h] - mx);
    rescale |= alpha[h] != 1.f;
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const float p = okc[i] ? fast_exp2(s[i][h] - mx) : 0.f;
      s[i][h] = p;
      ps += p;
    }
    l[h] = fmaf(l[h], alpha[h], ps);
    m[h] = mx;
  }
  // the accumulators change only when some running max moved (a factor of
  // exactly 1 leaves them as they are, so skipping it is exact); after the
  // first chunks that is rare, and the test is one wave-wide ballot
  if (__ballot(rescale)) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] *= alpha[h];
  }
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    float f[EPL];
    KV<T>::widen(vc[i], f);
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(s[i][h], f[e], acc[h][e]);
  }
}

// Arrival at a split row's word: returns how many of the row's workgroups
// (this one included) have arrived in this call.  The word holds
// [tag:48 | count:16]; a word whose tag is not this call's (left by an
// earlier call, which re-tags it with bit 47 set, or never written) starts
// the count afresh, so the workspace needs no clearing between calls.
__device__ __forceinline__ int arrive_at_row(unsigned long long* w, unsigned long long tag) {
  unsigned long long old = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (;;) {
    const bool mine = (old >> 16) == tag;
    const unsigned long long want = mine ? old + 1ull : ((tag << 16) | 1ull);
    if (__hip_atomic_compare_exchange_strong(w, &old, want, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT))
      return (int)(want & 0xFFFFull);
  }
}

// Partial states cross workgroups (and XCDs, whose L2 caches are not
// coherent with each other) as agent-scope atomic stores and loads, which
// the hardware keeps coherent device-wide without writing back or
// invalidating the L2 (an agent-scope fence does both, and costs ~0.7 us per
// workgroup per XCD under load).  Each wave waits until its stores are
// complete before the row's arrival word is updated, and the merging
// workgroup reads the states only after it has seen the last arrival.
__device__ __forceinline__ void st_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_stores_complete() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Merges the per-wave softmax states of a workgroup (staged in LDS) and
// writes the row's output.  When the row is split over several workgroups,
// each writes its partial state to the workspace and arrives at the row's
// word; the workgroup that arrives last merges the row's partial states in
// split order (fixed: bitwise repeatable) and re-tags the word for the next
// call.
template <int D, int G, int NWMAX = kMaxWaves>
__device__ __forceinline__ void merge_waves(const AttnArgs& a, int row, int b, int g, int split,
                                            int nw, const float (*s_m)[G], const float (*s_l)[G],
                                            const float (*s_acc)[G][D]) {
  const Dims& d = a.d;
  __shared__ int s_last;
  for (int o = threadIdx.x; o < G * D; o += blockDim.x) {
    const int h = o / D, e = o - (o / D) * D;
    // every wave's state read at once (unrolled to NWMAX), combined in
    // wave order
    float mw[NWMAX], lw[NWMAX], aw[NWMAX];
#pragma unroll
    for (int w = 0; w < NWMAX; ++w) {
      const int ww = min(w, nw - 1);
      mw[w] = s_m[ww][h];
      lw[w] = s_l[ww][h];
      aw[w] = s_acc[ww][h][e];
    }
    float M = -FLT_MAX;
#pragma unroll
    for (int w = 0; w < NWMAX; ++w)
      if (w < nw) M = fmaxf(M, mw[w]);
    float L = 0.f, A = 0.f;
#pragma unroll
    for (int w = 0; w < NWMAX; ++w) {
      if (w < nw) {
        const float sc = fast_exp2(mw[w] - M);
        L = fmaf(lw[w], sc, L);
        A = fmaf(aw[w], sc, A);
      }
    }
    if (a.splits == 1) {
      const int64_t oh = (int64_t)b * d.Hq + g * G + h;
      a.out[oh * D + e] = A / L;
      if (e == 0 && a.lse) a.lse[oh] = (M + log2f(L)) * kLn2;
    } else {
      const int64_t pi = ((int64_t)row * a.splits + split) * G + h;
      st_coherent(a.part_acc + pi * D + e, A);
      if (e == 0) {
        st_coherent(a.part_ml + pi * 2, M);
        st_coherent(a.part_ml + pi * 2 + 1, L);
      }
    }
  }
  if (a.splits == 1) return;
  wait_stores_complete();
  __syncthreads();
  if (threadIdx.x == 0) s_last = arrive_at_row(a.arrive + row, a.tag) == a.splits;
  __syncthreads();
  if (!s_last) return;
  // the partial states of kMergeBatch splits are loaded before any is used
  // (one round trip per batch rather than per split); the arithmetic keeps
  // the split order: max over splits, then the rescaled sums in split order
  constexpr int kMergeBatch = 8;
  for (int o = threadIdx.x; o < G * D; o += blockDim.x) {
    const int h = o / D, e = o - (o / D) * D;
    const int64_t p0 = (int64_t)row * a.splits * G + h;
    float M = -FLT_MAX, L = 0.f, A = 0.f;
    if (a.splits <= kMergeBatch) {
      float pm[kMergeBatch], pl[kMergeBatch], pa[kMergeBatch];
#pragma unroll
      for (int s = 0; s < kMergeBatch; ++s) {
        const int64_t pi = p0 + (int64_t)min(s, a.splits - 1) * G;
        pm[s] = ld_coherent(a.part_ml + pi * 2);
        pl[s] = ld_coherent(a.part_ml + pi * 2 + 1);
        pa[s] = ld_coherent(a.part_acc + pi * D + e);
      }
#pragma unroll
      for (int s = 0; s < kMergeBatch; ++s)
        if (s < a.splits) M = fmaxf(M, pm[s]);
#pragma unroll
      for (int s = 0; s < kMergeBatch; ++s) {
        if (s < a.splits) {
          const float sc = fast_exp2(pm[s] - M);
          L = fmaf(pl[s], sc, L);
          A = fmaf(pa[s], sc, A);
        }
      }
    } else {
      for (int s0 = 0; s0 < a.splits; s0 += kMergeBatch) {
        float pm[kMergeBatch];
#pragma unroll
        for (int s = 0; s < kMergeBatch; ++s)
          pm[s] = ld_coherent(a.part_ml + (p0 + (int64_t)min(s0 + s, a.splits - 1) * G) * 2);
#pragma unroll
        for (int s = 0; s < kMergeBatch; ++s)
          if (s0 + s < a.splits) M = fmaxf(M, pm[s]);
      }
      for (int s0 = 0; s0 < a.splits; s0 += kMergeBatch) {
        float pm[kMergeBatch], pl[kMergeBatch], pa[kMergeBatch];
#pragma unroll
        for (int s = 0; s < kMergeBatch; ++s) {
          const int64_t pi = p0 + (int64_t)min(s0 + s, a.splits - 1) * G;
          pm[s] = ld_coherent(a.part_ml + pi * 2);
          pl[s] = ld_coherent(a.part_ml + pi * 2 + 1);
          pa[s] = ld_coherent(a.part_acc + pi * D + e);
        }
#pragma unroll
        for (int s = 0; s < kMergeBatch; ++s) {
          if (s0 + s < a.splits) {
            const float sc = fast_exp2(pm[s] - M);
            L = fmaf(pl[s], sc, L);
            A = fmaf(pa[s], sc, A);
          }
        }
      }
    }
    const int64_t oh = (int64_t)b * d.Hq + g * G + h;
    a.out[oh * D + e] = A / L;
    if (e == 0 && a.lse) a.lse[oh] = (M + log2f(L)) * kLn2;
  }
  // every arrival of this call is in: the word takes a tag no call uses
  if (threadIdx.x == 0)
    __hip_atomic_store(a.arrive + row, ((~a.tag) & 0xFFFFFFFFFFFFull) << 16, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

// Copies n int32 from global memory to LDS, the whole workgroup taking turns:
// each thread issues up to kStageBatch loads before it waits for any (a
// loop of load-then-store would wait for each load in turn).
constexpr int kStageBatch = 8;
template <typename F>
__device__ __forceinline__ void stage_batches(int n, F body) {
  for (int base = 0; base < n; base += kStageBatch * (int)blockDim.x) body(base);
}
__device__ __forceinline__ void stage_copy(const int32_t* __restrict__ src, int n, int* dst) {
  if (n <= 0) return;
  stage_batches(n, [&](int base) {
    int v[kStageBatch];
#pragma unroll
    for (int u = 0; u < kStageBatch; ++u)
      v[u] = src[min(base + u * (int)blockDim.x + (int)threadIdx.x, n - 1)];
#pragma unroll
    for (int u = 0; u < kStageBatch; ++u) {
      const int i = base + u * (int)blockDim.x + (int)threadIdx.x;
      if (i < n) dst[i] = v[u];
    }
  });
}

// Stages the index slice a workgroup (row, split) needs in LDS; returns the
// first staged entry.  No barrier: the caller syncs before reading s_idx.
template <int KIND, int CH>
__device__ __forceinline__ int stage_indices(const AttnArgs& a, int row, int split, int* s_idx) {
  if constexpr (KIND == 2) return 0;
  const Dims& d = a.d;
  const int nchunks = (a.ltot + CH - 1) / CH;
  const int c_begin = split * a.cps;
  const int c_end = min(c_begin + a.cps, nchunks);
  int e0, e1;
  const int32_t* src;
  if constexpr (KIND == 0) {
    e0 = (c_begin * CH) / d.Bs;
    e1 = min(a.count, (c_end * CH + d.Bs - 1) / d.Bs);
    src = a.idx + (int64_t)row * a.count;
  } else {
    const int b = row / d.Hkv;
    e0 = c_begin * CH;
    e1 = min(a.ltot, c_end * CH);
    // kind 1: the sequence's list; kind 4: the row's (query head's) own list
    src = a.idx + (int64_t)(KIND == 4 ? row : b) * a.count;
  }
  stage_copy(src + e0, e1 - e0, s_idx);
  return e0;
}

// Attention of one row (or one split of it) on VALU; the row's index slice is
// staged in s_idx (entries from e0 on).  `sync` waits for the staging.
// qraw, when given, holds the lane's 16 bytes of each of the group's G query
// rows (already loaded by the caller in this lane layout).
template <typename T, int D, int G, int KIND, int NWMAX = kMaxWaves>
__device__ __forceinline__ void attn_row_valu(const AttnArgs& a, int row, int split, const int* s_idx,
                                              const int* s_pg, int e0, bool sync,
                                              const uint4* qraw = nullptr) {
  constexpr int EPL = KV<T>::EPL;
  constexpr int LPT = D / EPL;
  constexpr int SPW = 64 / LPT;
  constexpr int NI = kLoadsPerChunk;
  constexpr int CH = SPW * NI;
  constexpr int P = kPrefetchChunks;
  __shared__ float s_m[NWMAX][G];
  __shared__ float s_l[NWMAX][G];
  __shared__ float s_acc[NWMAX][G][D];

  const Dims& d = a.d;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const int slot = lane / LPT, li = lane % LPT;
  const int b = row / d.Hkv, g = row - b * d.Hkv;
  const int64_t kvrow =
      ((KIND == 3 || KIND == 5) ? (int64_t)g * d.Bs * D
       : KIND == 6 ? (int64_t)(g / a.kv_div) * d.Bs * D
       : KIND == 4 ? ((int64_t)b * (d.Hkv / a.kv_div) + g / a.kv_div) * d.Tcap * D
                   : (int64_t)row * d.Tcap * D) +
      li * EPL;
  const T* kbase = (const T*)a.k + kvrow;
  const T* vbase = (const T*)a.v + kvrow;

  const int nchunks = (a.ltot + CH - 1) / CH;
  const int c_begin = split * a.cps;
  const int c_end = min(c_begin + a.cps, nchunks);

  float qv[G][EPL];
  uint4 qb[G];  // the raw query pieces (bf16 logits on dot2)
#pragma unroll
  for (int h = 0; h < G; ++h) {
    qb[h] = qraw ? qraw[h] : ld16((const T*)a.q + ((int64_t)b * d.Hq + g * G + h) * D + li * EPL);
    KV<T>::widen(qb[h], qv[h]);
#pragma unroll
    for (int e = 0; e < EPL; ++e) qv[h][e] *= a.qscale;
  }

  float m[G], l[G], acc[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -FLT_MAX;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }
  if (sync) __syncthreads();

  const int c0 = c_begin + wave;
  const int my_n = c0 < c_end ? (c_end - c0 + nw - 1) / nw : 0;
  uint4 kb[P][NI], vb[P][NI];
  bool okb[P][NI];
#pragma unroll
  for (int s = 0; s < P; ++s)
    if (s < my_n)
      load_chunk<T, D, KIND, CH, SPW, NI>(a, s_idx, s_pg, e0, slot, c0 + s * nw, kbase, vbase,
                                          kb[s], vb[s], okb[s]);
  for (int j0 = 0; j0 < my_n; j0 += P) {
#pragma unroll
    for (int s = 0; s < P; ++s) {
      const int j = j0 + s;
      if (j < my_n) {
        uint4 kc[NI], vc[NI];
        bool okc[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          kc[i] = kb[s][i];
          vc[i] = vb[s][i];
          okc[i] = okb[s][i];
        }
        if (j + P < my_n)
          load_chunk<T, D, KIND, CH, SPW, NI>(a, s_idx, s_pg, e0, slot, c0 + (j + P) * nw, kbase,
                                              vbase, kb[s], vb[s], okb[s]);
        compute_chunk<T, D, G, NI, LPT>(qv, qb, a.qscale, kc, vc, okc, m, l, acc);
      }
    }
  }

  // merge the wave's slots (lanes li, li+LPT, ... hold the same channels)
#pragma unroll
  for (int off = LPT; off < 64; off <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mo = __shfl_xor(m[h], off);
      const float lo = __shfl_xor(l[h], off);
      const float M = fmaxf(m[h], mo);
      const float sa = fast_exp2(m[h] - M), sb = fast_exp2(mo - M);
      l[h] = l[h] * sa + lo * sb;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] = acc[h][e] * sa + __shfl_xor(acc[h][e], off) * sb;
      m[h] = M;
    }
  }
  if (slot == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (li == 0) {
        s_m[wave][h] = m[h];
        s_l[wave][h] = l[h];
      }
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_acc[wave][h][li * EPL + e] = acc[h][e];
    }
  }
  __syncthreads();

  merge_waves<D, G, NWMAX>(a, row, b, g, split, nw, s_m, s_l, s_acc);
}

// ---------------------------------------------------------------------------
// MFMA variant for bf16, D = 128 and G in {4, 8}.  Per chunk of 16 tokens:
//  * QK^T on v_mfma_f32_16x16x32_bf16: A = 16 token rows x 32 dims of K (lane
//    l holds token l%16, dims 8*(l/16).. of the slice, loaded straight from
//    HBM into that layout), B = the same 32 dims of the group's G query heads
//    (zero columns past G), four MFMAs cover D = 128.  The bf16 products are
//    exact and accumulate in fp32; the fp32 logits are scaled afterwards.
//    (Loading K coalesced and transposing it through LDS was measured slower
//    here: the extra LDS round trip per chunk costs more than it saves at the
//    8-12 waves per CU these kernels run with.)
//  * Softmax in the MFMA output layout (lane l: head l%16, tokens 4*(l/16)..):
//    one running max and sum per head for the whole wave, cross-lane steps by
//    xor-16/32 shuffles.
//  * The weights P (fp32) and the rescale factors go through a wave-private
//    LDS tile to the V layout (16 lanes per token row, as in the VALU kernel),
//    where P.V accumulates on VALU in fp32.
// Softmax state is per wave rather than per slot, so the slots of a wave are
// merged by plain sums.
// Attention of one row (or one split of it) with MFMA QK^T (bf16, D = 128,
// G in {4, 8}); indices staged as for attn_row_valu.
// VK: the dense walk (kind 2, or kind 3 over every block) also writes the
// vote's keys (a.vkeys); dense walks without a vote compile without them.
template <int G, int KIND, bool VK = false, int NWMAX = kMaxWaves>
__device__ __forceinline__ void attn_row_mfma(const AttnArgs& a, int row, int split, const int* s_idx,
                                              const int* s_pg, int e0, bool sync) {
  static_assert(!VK || KIND == 2 || KIND == 3, "vote keys come from dense walks");
  constexpr int D = 128;
  constexpr int EPL = 8;
  constexpr int SPW = 4;
  constexpr int NI = 4;
  constexpr int CH = 16;
  static_assert(CH == SPW * NI, "chunk of the VALU kernel");
  __shared__ float s_m[NWMAX][G];
  __shared__ float s_l[NWMAX][G];
  __shared__ float s_acc[NWMAX][G][D];
  __shared__ float s_p[NWMAX][CH + 1][8];  // rows 0..15: P[token][head]; row 16: rescale

  const Dims& d = a.d;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const int r = lane & 15, kg = lane >> 4;  // MFMA: row/column and k-group / row quad
  const int slot = kg, li = r;             // V layout: token slot and 16-byte piece
  const int b = row / d.Hkv, g = row - b * d.Hkv;
  const int64_t kvrow =
      (KIND == 3 || KIND == 5) ? (int64_t)g * d.Bs * D : (int64_t)row * d.Tcap * D;
  const uint16_t* kbase = (const uint16_t*)a.k + kvrow + 8 * kg;
  const uint16_t* vbase = (const uint16_t*)a.v + kvrow + li * EPL;

  const int nchunks = (a.ltot + CH - 1) / CH;
  const int c_begin = split * a.cps;
  const int c_end = min(c_begin + a.cps, nchunks);

  // B operand: the group's queries, column n = head r (zero past G)
  bf16x8_t qop[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint4 u = make_uint4(0u, 0u, 0u, 0u);
    if (r < G) u = ld16((const uint16_t*)a.q + ((int64_t)b * d.Hq + g * G + r) * D + 32 * i + 8 * kg);
    qop[i] = as_bf16x8(u);
  }
  float m = -FLT_MAX, lsum = 0.f;  // softmax state of head r (MFMA layout)
  float acc[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  if (sync) __syncthreads();

  const int c0 = c_begin + wave;
  const int my_n = c0 < c_end ? (c_end - c0 + nw - 1) / nw : 0;
  float(*pt)[8] = s_p[wave];

  // loads of one chunk: K in the MFMA A layout, V in the row layout
  auto load = [&](int c, uint4* kr, uint4* vr, bool& okk) {
    int tk[1];
    bool ok1[1];
    resolve_chunk<KIND, CH, 1, 1>(a, s_idx, s_pg, e0, r, c, tk, ok1);  // position c*16 + r
    okk = ok1[0];
#pragma unroll
    for (int i = 0; i < NI; ++i) kr[i] = ld_kv(kbase + (int64_t)tk[0] * D + 32 * i);
    int tv[NI];
    bool okv[NI];
    resolve_chunk<KIND, CH, SPW, NI>(a, s_idx, s_pg, e0, slot, c, tv, okv);
#pragma unroll
    for (int i = 0; i < NI; ++i) vr[i] = ld_kv(vbase + (int64_t)tv[i] * D);
  };

  // VK: the key rows [G, vkstride] of the group's heads as one store range;
  // lanes without a key (heads past G, tokens past the history) are dropped
  const __amdgpu_buffer_rsrc_t krs =
      store_range(VK ? (void*)(a.vkeys + ((int64_t)b * d.Hq + g * G) * a.vkstride) : nullptr,
                  VK ? (uint32_t)(G * a.vkstride) * 4u : 0u);

  // one chunk's scores, softmax update and P.V (chunk j of the wave)
  auto consume = [&](const uint4* kc, const uint4* vc, bool okc, int j) {
    f32x4_t S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NI; ++i) S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kc[i]), qop[i], S, 0, 0, 0);
    if constexpr (VK) {
      // the selection layer: keys of head r's raw logits of tokens 4kg..4kg+3
      // (the vote scorer's arithmetic, so the same keys), 16 bytes at a time;
      // positions are token ids in a dense walk (kind 3: over every block in
      // order).  A group that straddles the end of the history is stored
      // whole: its slots past the history lie in the row's padding to a
      // multiple of 4, which nothing reads.
      const int t = (c0 + j * nw) * CH + 4 * kg;
      const uint32_t off =
          (r < G && t < a.vhist) ? (uint32_t)(r * a.vkstride + t) * 4u : kDropOffset;
      st16_range(krs, off,
                 make_uint4(order_key(S[0]), order_key(S[1]), order_key(S[2]), order_key(S[3])));
    }
    const uint64_t vm = __ballot(okc);  // bit t (t < 16): chunk token t is attended
    float sv[4];
    bool val[4];
    float mloc = -FLT_MAX;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      sv[jj] = S[jj] * a.qscale;
      val[jj] = (vm >> (4 * kg + jj)) & 1ull;
      if (val[jj]) mloc = fmaxf(mloc, sv[jj]);
    }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    const float mnew = fmaxf(m, mloc);
    const float alpha = fast_exp2(m - mnew);
    float ps = 0.f;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      sv[jj] = val[jj] ? fast_exp2(sv[jj] - mnew) : 0.f;
      ps += sv[jj];
    }
    ps += __shfl_xor(ps, 16);
    ps += __shfl_xor(ps, 32);
    lsum = fmaf(lsum, alpha, ps);
    m = mnew;
    if (r < G) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) pt[4 * kg + jj][r] = sv[jj];
      if (kg == 0) pt[CH][r] = alpha;
    }
    wave_lds_fence();
    // rescale only when some head's running max moved (see compute_chunk)
    if (__ballot(r < G && kg == 0 && alpha != 1.f)) {
      float al[G];
#pragma unroll
      for (int h = 0; h < G; ++h) al[h] = pt[CH][h];
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] *= al[h];
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float pv[G];
#pragma unroll
      for (int h = 0; h < G; ++h) pv[h] = pt[4 * i + slot][h];
      float f[EPL];
      KV<uint16_t>::widen(vc[i], f);
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(pv[h], f[e], acc[h][e]);
    }
    wave_lds_fence();
  };

  // a ring of kMfmaPrefetch register buffers: chunk j is consumed while the
  // loads of the wave's next kMfmaPrefetch chunks are in flight
  constexpr int PF = kMfmaPrefetch;
  uint4 kb[PF][NI], vb[PF][NI];
  bool okb[PF];
#pragma unroll
  for (int u = 0; u < PF; ++u) {
    okb[u] = false;
    if (u < my_n) load(c0 + u * nw, kb[u], vb[u], okb[u]);
  }
  // a store that writes nothing: the loop is entered with the same memory
  // operations outstanding as every iteration leaves behind, so the waits
  // for the next chunk's loads leave the previous chunk's key store in flight
  if constexpr (VK) st16_range(krs, kDropOffset, make_uint4(0u, 0u, 0u, 0u));
  for (int j0 = 0; j0 < my_n; j0 += PF) {
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const int j = j0 + u;
      if (j >= my_n) break;
      uint4 kc[NI], vc[NI];
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        kc[i] = kb[u][i];
        vc[i] = vb[u][i];
      }
      const bool okc = okb[u];
      if (j + PF < my_n) load(c0 + (j + PF) * nw, kb[u], vb[u], okb[u]);
      consume(kc, vc, okc, j);
    }
  }

  // slots share the wave's softmax state: their accumulators simply add up
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      acc[h][e] += __shfl_xor(acc[h][e], 16);
      acc[h][e] += __shfl_xor(acc[h][e], 32);
    }
  if (lane < G) {
    s_m[wave][lane] = m;
    s_l[wave][lane] = lsum;
  }
  if (slot == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_acc[wave][h][li * EPL + e] = acc[h][e];
  }
  __syncthreads();
  merge_waves<D, G, NWMAX>(a, row, b, g, split, nw, s_m, s_l, s_acc);
}

}  // namespace ksa

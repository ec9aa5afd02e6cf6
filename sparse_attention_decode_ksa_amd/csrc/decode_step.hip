// decode_step.hip -- a whole decode step of block top-k attention in one
// launch (Kinetics explainer, section 五: the newest token's block gets its
// mean key, every block's mean key is scored against the query, the K' most
// relevant blocks are kept and attention runs over their tokens only).
//
// One workgroup of 8 waves (4 when the rows outnumber the 8-wave workgroups
// the chip holds at once) owns one (sequence, KV head) row and runs the four
// steps back to back:
//  1. scoring: the row's summaries stream through double-buffered runs of
//     16-byte loads that the waves take from a shared counter; each block's
//     relevance (sum_h q_h) . S_j (fp32) becomes an order-preserving key in
//     LDS, and the keys' range is gathered with LDS atomics;
//  2. refresh (optional), by wave 0 before it joins the scoring (the other
//     waves start scoring at once, so the refresh is off the row's critical
//     path): the token rows of block (T-1)/Bs go through LDS, each lane sums
//     its channels in fp64 in token order, and the rounded mean is written
//     to the summaries and scored;
//  3. top-k: row_topk_list of ksa_topk.h on the LDS keys (over the gathered
//     range, so no separate min/max pass): one histogram round, the cut
//     bucket ranked from an LDS list, a selection mask; then every wave
//     writes the selected block ids, ascending, into the attention's LDS
//     index stage (wave 0 also to block_idx when asked) and goes on to its
//     attention at once;
//  4. attention: the per-row body of ksa_attention.h (VALU, or MFMA for bf16
//     D = 128 with G >= 4) over the selected blocks, one split.
// The keys never leave the chip and three kernel boundaries disappear.  Each
// step repeats the arithmetic of the separate calls (block_summaries_kernel,
// block_score_kernel, topk_rows_kernel, the attention bodies), so summaries
// and selections are bitwise those of ksa_block_summaries + ksa_select_topk;
// the attention equals ksa_sparse_decode's up to the fp32 order of the wave
// merge (bitwise when both run one 8-wave workgroup per row).
#include <atomic>
#include <type_traits>

#include "ksa_attention.h"
#include "ksa_topk.h"

namespace ksa {
namespace {

// Waves per SIMD the register budget is held to for groups of at most two
// heads (4 -> 128 VGPRs: sixteen waves per CU).  A tuning knob.
#ifndef KSA_STEP_OCC
#define KSA_STEP_OCC 4
#endif
// Summaries a lane loads per scoring unit (a unit is SPW * this many blocks).
// Small units end the scoring phase with the waves close together, since
// each wave takes its next unit from the shared counter: 4 measured 2-3 %
// faster than 8 for the Qwen3-8B-shaped step (32 x 8 rows, block 32) and
// ~1 % for the block-16 shapes, with 2 and 3 no better.  A tuning knob.
#ifndef KSA_STEP_UNROLL
#define KSA_STEP_UNROLL 4
#endif
constexpr int kStepUnroll = KSA_STEP_UNROLL;  // summaries in flight per lane per batch

struct StepArgs {
  AttnArgs a;          // attention over the selected blocks (ids come from LDS)
  void* summ;          // [B, Hkv, NBcap, D]; block (T-1)/Bs is rewritten on refresh
  int refresh;
  int keff;            // k_eff; paged: top_k (each row's k_eff is at most this)
  int32_t* block_idx;  // [B, Hkv, keff] or null
};

template <typename T, int D>
constexpr int ref_stage_slots() {
  // LDS 16-byte slots for the refresh block's rows; the same buffer later
  // holds the attention's index stage
  constexpr int ref = kStepMaxBs * (D / KV<T>::EPL);
  constexpr int idx = kIdxStage / 4;
  return ref > idx ? ref : idx;
}

// NW waves per workgroup (4 or 8).  PAGED: K and V are page pools (the
// attention's kind 3) and every row has its own length from seq_lens.  A
// contiguous cache may also carry seq_lens (lengths up to the call's T).
template <typename T, int D, int G, int NW, bool PAGED>
__global__ __launch_bounds__(NW * 64, (G <= 2 ? KSA_STEP_OCC : 1)) void block_topk_decode_kernel(
    StepArgs s) {
  constexpr int kStepThreads = NW * 64;
  constexpr int kStepKPT = (kStepMaxBlocks + kStepThreads - 1) / kStepThreads;  // keys per thread
  constexpr int EPL = KV<T>::EPL;
  constexpr int LPT = D / EPL;
  constexpr int U = kStepUnroll;
  constexpr bool kMfma = std::is_same<T, uint16_t>::value && D == 128 && G >= 4;
  __shared__ uint32_t s_keys[kStepMaxBlocks];
  __shared__ uint4 s_buf[ref_stage_slots<T, D>()];
  __shared__ uint4 s_mean[D / EPL];  // the refreshed block's rounded mean
  __shared__ TopkShared s_topk;
  __shared__ int s_next;           // next free scoring unit
  __shared__ uint32_t s_lo, s_hi;  // range of the row's keys
  __shared__ int s_pgbuf[PAGED ? kIdxStage : 1];  // pages of the selected blocks
  uint4* s_ref = s_buf;                        // step 2
  int* s_idx = reinterpret_cast<int*>(s_buf);  // steps 3-4
  int* s_pg = PAGED ? s_pgbuf : nullptr;

  const Dims& d = s.a.d;
  const int row = blockIdx.x;
  const int b = row / d.Hkv, g = row - b * d.Hkv;
  const int tid = threadIdx.x, li = tid % LPT;
  // the row's length, blocks and k_eff; for a paged cache the attention
  // sees this row's length
  AttnArgs a = s.a;
  int keff = s.keff;
  const int32_t* ptab = nullptr;
  if constexpr (PAGED) {
    a.d.T = seq_len_of(a.seq_lens, b, d.T);
    a.d.NB = (a.d.T + d.Bs - 1) / d.Bs;
    keff = min(s.keff, a.d.NB);
    a.ltot = keff * d.Bs;
    ptab = a.table + (int64_t)b * a.tstride;
  } else if (a.seq_lens) {  // contiguous cache, one length per sequence (at most T)
    a.d.T = seq_len_of(a.seq_lens, b, d.T);
    a.d.NB = (a.d.T + d.Bs - 1) / d.Bs;
    keff = min(s.keff, a.d.NB);
    a.ltot = keff * d.Bs;
  }
  const int Trow = a.d.T;
  const int NB = a.d.NB;
  T* srow = (T*)s.summ + (int64_t)row * d.NBcap * D + li * EPL;
  const int jref = s.refresh ? (Trow - 1) / d.Bs : -1;
  const int nref = s.refresh ? Trow - jref * d.Bs : 0;

  // the group's query rows (kept for the attention) and their fp32 sum, the
  // group query of block_score_kernel
  uint4 qraw[G];
  float qs[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) qs[e] = 0.f;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    qraw[h] = ld16((const T*)a.q + ((int64_t)b * d.Hq + g * G + h) * D + li * EPL);
    float f[EPL];
    KV<T>::widen(qraw[h], f);
#pragma unroll
    for (int e = 0; e < EPL; ++e) qs[e] += f[e];
  }

  // Scoring units: wave-sized runs of WU consecutive blocks (group s of a
  // wave takes blocks u*SPW + s of the run, so each load instruction reads
  // SPW whole summaries back to back).  A wave's first unit is its own; it
  // then takes the next free unit from an LDS counter, so waves that are
  // served faster by the memory system score more units and the workgroup's
  // scoring ends close to its average wave.  Keys do not depend on which
  // wave computed them.
  constexpr int SPW = 64 / LPT;
  constexpr int WU = SPW * U;
  const int lane = tid & 63, wave = tid >> 6, slot = lane / LPT;
  const int nw = NW;
  const int nu = (NB + WU - 1) / WU;
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;  // range of the keys this lane stored
  auto load_unit = [&](int k, uint4* r) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      r[u] = ld16_stream(srow + (int64_t)min(k * WU + u * SPW + slot, NB - 1) * D);
  };
  auto score_unit = [&](int k, const uint4* r) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = k * WU + u * SPW + slot;
      float f[EPL];
      KV<T>::widen(r[u], f);
      float p = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) p = fmaf(qs[e], f[e], p);
      p = group_sum<LPT>(p);
      if (li == 0 && j < NB && j != jref) {
        const uint32_t kk = order_key(p);
        s_keys[j] = kk;
        kmin = min(kmin, kk);
        kmax = max(kmax, kk);
      }
    }
  };
  auto grab = [&]() -> int {
    int v = 0;
    if (lane == 0) v = atomicAdd(&s_next, 1);
    return __builtin_amdgcn_readfirstlane(v);
  };

  // 1. scoring, two units in flight per wave (the refresh block is scored
  // by step 2).  Loads are unconditional (past the last unit they re-read the
  // last block), so each unit waits only for its own loads.
  uint4 bufA[U], bufB[U];
  int ua = wave;
  load_unit(ua, bufA);
  if (tid == 0) {
    s_next = nw;
    s_lo = 0xFFFFFFFFu;
    s_hi = 0u;
  }
  topk_clear(s_topk);
  __syncthreads();

  // 2. refresh, by wave 0 while the others score: the block's rows go to
  // LDS (SPW rows per load instruction), lane c sums channels c, c+64, ...
  // in fp64 in token order (as block_summaries_kernel), and group 0 stores
  // the rounded mean and scores it as score_unit does
  if (s.refresh && wave == 0) {
    const T* kp;
    if constexpr (PAGED)  // the block's page; its rows start the page's KV-head slab
      kp = (const T*)a.k + ((int64_t)ptab[jref] * d.Hkv + g) * d.Bs * D + li * EPL;
    else
      kp = (const T*)a.k + ((int64_t)row * d.Tcap + (int64_t)jref * d.Bs) * D + li * EPL;
    constexpr int RB = 4;  // load instructions in flight
    for (int t0 = 0; t0 < nref; t0 += RB * SPW) {
      uint4 r[RB];
#pragma unroll
      for (int i = 0; i < RB; ++i) r[i] = ld16(kp + (int64_t)min(t0 + i * SPW + slot, nref - 1) * D);
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const int t = t0 + i * SPW + slot;
        if (t < nref) s_ref[t * LPT + li] = r[i];
      }
    }
    wave_lds_fence();
    const T* sr = reinterpret_cast<const T*>(s_ref);
    T* sm = reinterpret_cast<T*>(s_mean);
    for (int c = lane; c < D; c += 64) {
      double acc = 0.0;
      for (int t = 0; t < nref; ++t) acc += (double)KV<T>::widen1(sr[t * D + c]);
      sm[c] = mean_elem<T>(acc, nref);
    }
    wave_lds_fence();
    if (lane < LPT) {
      const uint4 mb = s_mean[li];
      st16(srow + (int64_t)jref * D, mb);
      float f[EPL];
      KV<T>::widen(mb, f);
      float p = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) p = fmaf(qs[e], f[e], p);
      p = group_sum<LPT>(p);
      if (li == 0) {
        const uint32_t kk = order_key(p);
        s_keys[jref] = kk;
        kmin = min(kmin, kk);
        kmax = max(kmax, kk);
      }
    }
  }

  for (;;) {
    const int ub = grab();
    load_unit(ub, bufB);
    if (ua >= nu) break;
    score_unit(ua, bufA);
    ua = grab();
    load_unit(ua, bufA);
    if (ub >= nu) break;
    score_unit(ub, bufB);
  }

  if (li == 0) {
    atomicMin(&s_lo, kmin);
    atomicMax(&s_hi, kmax);
  }
  __syncthreads();

  // 3. top-k over the LDS keys; thread t takes positions [t*kpt, (t+1)*kpt).
  // The register array is sized for the row's kpt (2, 4 or the most), so
  // the unrolled passes of the top-k do no predicated-off iterations.
  const int kpt = (NB + kStepThreads - 1) / kStepThreads;
  const int j0 = tid * kpt;
  int32_t* gidx = s.block_idx ? s.block_idx + (int64_t)row * s.keff : nullptr;
  // every wave writes the whole ascending list into the LDS stage (the same
  // values), so it starts its attention without waiting for the others
  static_assert(kStepMaxBlocks <= kTopkListMax, "selection mask");
  auto topk = [&](auto kpt_max) {
    constexpr int K = decltype(kpt_max)::value;
    uint32_t key[K];
#pragma unroll
    for (int i = 0; i < K; ++i) key[i] = (i < kpt && j0 + i < NB) ? s_keys[j0 + i] : 0u;
    row_topk_list<K>(key, kpt, j0, NB, keff, s_lo, s_hi, s_topk,
                     [&](int rank, int j, bool primary) {
                       s_idx[rank] = j;
                       if constexpr (PAGED) s_pg[rank] = ptab[j];
                       if (primary && gidx) gidx[rank] = j;
                     });
  };
  if (kpt <= 2)
    topk(std::integral_constant<int, 2>{});
  else if (kpt <= 4)
    topk(std::integral_constant<int, 4>{});
  else
    topk(std::integral_constant<int, kStepKPT>{});
  if (PAGED || a.seq_lens) {  // ids past this row's k_eff
    if (gidx)
      for (int i = keff + tid; i < s.keff; i += kStepThreads) gidx[i] = -1;
  }
  wave_lds_fence();

  // 4. attention over the selected blocks
  constexpr int KIND = PAGED ? 3 : 0;
  if constexpr (kMfma)
    attn_row_mfma<G, KIND, false, NW>(a, row, 0, s_idx, s_pg, 0, false);
  else
    attn_row_valu<T, D, G, KIND, NW>(a, row, 0, s_idx, s_pg, 0, false, qraw);
}

// Eight-wave workgroups of the step kernel that the device holds at once
// (resident per CU times CUs), found once per kernel and device.
constexpr int kMaxDevices = 64;
template <typename T, int D, int G, bool PAGED>
int eight_wave_capacity(int dev) {
  static std::atomic<int> cache[kMaxDevices];  // 0: not yet known
  const bool cached = dev >= 0 && dev < kMaxDevices;
  int cap = cached ? cache[dev].load(std::memory_order_relaxed) : 0;
  if (cap > 0) return cap;
  int n = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, block_topk_decode_kernel<T, D, G, 8, PAGED>,
                                                   512, 0) != hipSuccess || n < 1)
    n = 1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1)
    cus = 256;
  cap = n * cus;
  if (cached) cache[dev].store(cap, std::memory_order_relaxed);
  return cap;
}

template <typename T, int D, int G, bool PAGED>
hipError_t launch_g(const StepArgs& s, int rows, hipStream_t stream) {
  // Eight waves per row unless the rows outnumber the workgroups of eight
  // waves that fit on the chip at once: then four, so that more rows are in
  // flight and one row's top-k is covered by the others' streaming.
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const dim3 grid(rows);
  if (rows > eight_wave_capacity<T, D, G, PAGED>(dev))
    hipLaunchKernelGGL((block_topk_decode_kernel<T, D, G, 4, PAGED>), grid, dim3(256), 0, stream, s);
  else
    hipLaunchKernelGGL((block_topk_decode_kernel<T, D, G, 8, PAGED>), grid, dim3(512), 0, stream, s);
  return hipGetLastError();
}

template <typename T, int D, bool PAGED>
hipError_t launch_typed(const StepArgs& s, hipStream_t stream) {
  const int rows = s.a.d.B * s.a.d.Hkv;
  switch (s.a.d.G) {
    case 1: return launch_g<T, D, 1, PAGED>(s, rows, stream);
    case 2: return launch_g<T, D, 2, PAGED>(s, rows, stream);
    case 4: return launch_g<T, D, 4, PAGED>(s, rows, stream);
    default: return launch_g<T, D, 8, PAGED>(s, rows, stream);
  }
}

template <bool PAGED>
hipError_t launch_dtype(const StepArgs& s, hipStream_t stream) {
  const Dims& d = s.a.d;
  if (d.dtype == KSA_BF16) {
    if (d.D == 64) return launch_typed<uint16_t, 64, PAGED>(s, stream);
    return launch_typed<uint16_t, 128, PAGED>(s, stream);
  }
  if (d.D == 64) return launch_typed<float, 64, PAGED>(s, stream);
  return launch_typed<float, 128, PAGED>(s, stream);
}

}  // namespace

hipError_t launch_block_topk_decode(const Dims& d, const void* q, const void* k, const void* v,
                                    void* summaries, int keff, int refresh, int32_t* block_idx,
                                    float* out, float* lse, hipStream_t stream,
                                    const PagedKv* paged, const int32_t* seq_lens) {
  // keff is the id stride; a paged call's rows select at most max_blocks
  const int kplan = keff < d.NBcap ? keff : d.NBcap;
  const int ch = chunk_tokens(d);
  const int nchunks = ceil_div((int64_t)kplan * d.Bs, ch);
  const AttnPlan plan{kMaxWaves, 1, nchunks, ch};
  StepArgs s;
  s.a = make_attn_args(d, 0, q, k, v, nullptr, kplan, out, lse, nullptr, plan);
  s.summ = summaries;
  s.refresh = refresh ? 1 : 0;
  s.keff = keff;
  s.block_idx = block_idx;
  if (paged) {
    s.a.table = paged->table;
    s.a.seq_lens = paged->seq_lens;
    s.a.tstride = paged->max_blocks;
    return launch_dtype<true>(s, stream);
  }
  s.a.seq_lens = seq_lens;
  return launch_dtype<false>(s, stream);
}

}  // namespace ksa

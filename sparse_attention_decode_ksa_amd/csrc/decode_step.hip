// decode_step.hip -- a whole decode step of block top-k attention in one
// launch (Kinetics explainer, section 五: the newest token's block gets its
// mean key, every block's mean key is scored against the query, the K' most
// relevant blocks are kept and attention runs over their tokens only).
//
// One workgroup of 512 threads owns one (sequence, KV head) row and runs the
// four steps back to back:
//  1. refresh (optional): the token rows of block (T-1)/Bs are loaded, one
//     per LPT-lane group, parked in LDS, and summed by one group in fp64 in
//     token order; the rounded mean is written to the summaries and scored
//     from registers;
//  2. scoring: the row's summaries stream through double-buffered batches of
//     16-byte loads; each block's relevance (sum_h q_h) . S_j (fp32) becomes
//     an order-preserving key in LDS;
//  3. top-k: the bucket search of ksa_topk.h on the LDS keys writes the
//     selected block ids, ascending, into the attention's LDS index stage
//     (and to block_idx when asked);
//  4. attention: the per-row body of ksa_attention.h (VALU, or MFMA for bf16
//     D = 128 with G >= 4) over the selected blocks, one split.
// The keys never leave the chip and three kernel boundaries disappear.  Each
// step repeats the arithmetic of the separate calls (block_summaries_kernel,
// block_score_kernel, topk_rows_kernel, the attention bodies), so summaries
// and selections are bitwise those of ksa_block_summaries + ksa_select_topk,
// and the attention equals ksa_sparse_decode's whenever that call plans one
// split of 8 waves per row.
#include <type_traits>

#include "ksa_attention.h"
#include "ksa_topk.h"

namespace ksa {
namespace {

constexpr int kStepThreads = kMaxWaves * 64;
constexpr int kStepKPT = kStepMaxBlocks / kStepThreads;  // keys per thread in the top-k
#ifndef KSA_STEP_UNROLL
#define KSA_STEP_UNROLL 8
#endif
constexpr int kStepUnroll = KSA_STEP_UNROLL;  // summaries in flight per lane per batch

struct StepArgs {
  AttnArgs a;          // attention over the selected blocks (ids come from LDS)
  void* summ;          // [B, Hkv, NBcap, D]; block (T-1)/Bs is rewritten on refresh
  int refresh;
  int keff;
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

template <typename T, int D, int G>
__global__ __launch_bounds__(kStepThreads, (G <= 2 ? 4 : 1)) void block_topk_decode_kernel(
    StepArgs s) {
  constexpr int EPL = KV<T>::EPL;
  constexpr int LPT = D / EPL;
  constexpr int NGRP = kStepThreads / LPT;
  constexpr int U = kStepUnroll;
  constexpr int RP = (kStepMaxBs + NGRP - 1) / NGRP;  // refresh rows per group
  constexpr bool kMfma = std::is_same<T, uint16_t>::value && D == 128 && G >= 4;
  __shared__ uint32_t s_keys[kStepMaxBlocks];
  __shared__ uint4 s_buf[ref_stage_slots<T, D>()];
  __shared__ TopkShared s_topk;
  uint4* s_ref = s_buf;                              // steps 1
  int* s_idx = reinterpret_cast<int*>(s_buf);        // steps 3-4

  const AttnArgs& a = s.a;
  const Dims& d = a.d;
  const int row = blockIdx.x;
  const int b = row / d.Hkv, g = row - b * d.Hkv;
  const int tid = threadIdx.x, li = tid % LPT, grp = tid / LPT;
  const int NB = d.NB;
  T* srow = (T*)s.summ + (int64_t)row * d.NBcap * D + li * EPL;
  const int jref = s.refresh ? (d.T - 1) / d.Bs : -1;
  const int nref = s.refresh ? d.T - jref * d.Bs : 0;

  // 1a. refresh rows first, so their loads return ahead of the summaries
  uint4 rr[RP];
  if (s.refresh) {
    const T* kp = (const T*)a.k + ((int64_t)row * d.Tcap + (int64_t)jref * d.Bs) * D + li * EPL;
#pragma unroll
    for (int r = 0; r < RP; ++r) {
      const int t = grp + r * NGRP;
      if (t < nref) rr[r] = ld16(kp + (int64_t)t * D);
    }
  }

  // group query: sum of the G heads, fp32 (as block_score_kernel)
  float qs[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) qs[e] = 0.f;
  for (int h = 0; h < G; ++h) {
    float f[EPL];
    KV<T>::widen(ld16((const T*)a.q + ((int64_t)b * d.Hq + g * G + h) * D + li * EPL), f);
#pragma unroll
    for (int e = 0; e < EPL; ++e) qs[e] += f[e];
  }

  constexpr int kBatch = NGRP * U;
  auto load_batch = [&](int base, uint4* r) {
#pragma unroll
    for (int u = 0; u < U; ++u) r[u] = ld16_stream(srow + (int64_t)min(base + u * NGRP + grp, NB - 1) * D);
  };
  auto score_batch = [&](int base, const uint4* r) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = base + u * NGRP + grp;
      float f[EPL];
      KV<T>::widen(r[u], f);
      float p = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) p = fmaf(qs[e], f[e], p);
      p = group_sum<LPT>(p);
      if (li == 0 && j < NB && j != jref) s_keys[j] = order_key(p);
    }
  };

  uint4 bufA[U], bufB[U];
  load_batch(0, bufA);

  // 1b. refresh: in-order fp64 sum by group 0 (as block_summaries_kernel)
  if (s.refresh) {
#pragma unroll
    for (int r = 0; r < RP; ++r) {
      const int t = grp + r * NGRP;
      if (t < nref) s_ref[t * LPT + li] = rr[r];
    }
    __syncthreads();
    if (tid < LPT) {
      double acc[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = 0.0;
      for (int t = 0; t < nref; ++t) {
        float f[EPL];
        KV<T>::widen(s_ref[t * LPT + li], f);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] += (double)f[e];
      }
      const uint4 mb = mean_bits<T>(acc, nref);
      st16(srow + (int64_t)jref * D, mb);
      float f[EPL];
      KV<T>::widen(mb, f);
      float p = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) p = fmaf(qs[e], f[e], p);
      p = group_sum<LPT>(p);
      if (li == 0) s_keys[jref] = order_key(p);
    }
  }

  // 2. scoring, two batches in flight
  for (int base = 0; base < NB; base += 2 * kBatch) {
    if (base + kBatch < NB) load_batch(base + kBatch, bufB);
    score_batch(base, bufA);
    if (base + 2 * kBatch < NB) load_batch(base + 2 * kBatch, bufA);
    if (base + kBatch < NB) score_batch(base + kBatch, bufB);
  }
  __syncthreads();

  // 3. top-k over the LDS keys; thread t takes positions [t*kpt, (t+1)*kpt)
  const int kpt = (NB + kStepThreads - 1) / kStepThreads;
  const int j0 = tid * kpt;
  uint32_t key[kStepKPT];
#pragma unroll
  for (int i = 0; i < kStepKPT; ++i) key[i] = (i < kpt && j0 + i < NB) ? s_keys[j0 + i] : 0u;
  int32_t* gidx = s.block_idx ? s.block_idx + (int64_t)row * s.keff : nullptr;
  row_topk<kStepKPT>(key, kpt, j0, NB, s.keff, s_topk, [&](int rank, int j) {
    s_idx[rank] = j;
    if (gidx) gidx[rank] = j;
  });
  __syncthreads();

  // 4. attention over the selected blocks
  if constexpr (kMfma)
    attn_row_mfma<G, 0>(a, row, 0, s_idx, 0, false);
  else
    attn_row_valu<T, D, G, 0>(a, row, 0, s_idx, 0, false);
}

template <typename T, int D>
hipError_t launch_typed(const StepArgs& s, hipStream_t stream) {
  const dim3 grid(s.a.d.B * s.a.d.Hkv), block(kStepThreads);
  switch (s.a.d.G) {
    case 1: hipLaunchKernelGGL((block_topk_decode_kernel<T, D, 1>), grid, block, 0, stream, s); break;
    case 2: hipLaunchKernelGGL((block_topk_decode_kernel<T, D, 2>), grid, block, 0, stream, s); break;
    case 4: hipLaunchKernelGGL((block_topk_decode_kernel<T, D, 4>), grid, block, 0, stream, s); break;
    default: hipLaunchKernelGGL((block_topk_decode_kernel<T, D, 8>), grid, block, 0, stream, s); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_block_topk_decode(const Dims& d, const void* q, const void* k, const void* v,
                                    void* summaries, int keff, int refresh, int32_t* block_idx,
                                    float* out, float* lse, hipStream_t stream) {
  const int ch = chunk_tokens(d);
  const int nchunks = ceil_div((int64_t)keff * d.Bs, ch);
  const AttnPlan plan{kMaxWaves, 1, nchunks, ch};
  StepArgs s;
  s.a = make_attn_args(d, 0, q, k, v, nullptr, keff, out, lse, nullptr, plan);
  s.summ = summaries;
  s.refresh = refresh ? 1 : 0;
  s.keff = keff;
  s.block_idx = block_idx;
  if (d.dtype == KSA_BF16) {
    if (d.D == 64) return launch_typed<uint16_t, 64>(s, stream);
    return launch_typed<uint16_t, 128>(s, stream);
  }
  if (d.D == 64) return launch_typed<float, 64>(s, stream);
  return launch_typed<float, 128>(s, stream);
}

}  // namespace ksa

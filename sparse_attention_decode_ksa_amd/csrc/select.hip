// select.hip -- choose the K' most relevant blocks per (sequence, KV head)
// (Kinetics explainer, section 五: blocks are ranked by the relevance of
// their mean key to the query and the top K' are attended).
//
// Two kernels:
//  1. block_score_kernel.  Grid = (tiles of blocks) x rows, so the summaries
//     stream through many workgroups with all of their loads in flight.  The
//     relevance of block j is sum_h q_h . S_j over the group's G query heads,
//     computed as (sum_h q_h) . S_j in fp32 (the group query is summed once;
//     bf16 x bf16 products are exact in fp32).  Groups of LPT lanes read a
//     summary with one 16-byte load per lane and reduce the dot product with
//     DPP; each score is stored as an order-preserving uint32 key in the
//     workspace [rows, NB].
//  2. topk_rows_kernel.  One workgroup per row with the row's keys in
//     registers runs the bucket search of ksa_topk.h: LDS histograms of at
//     most 256 buckets over the row's key range find the k-th largest key
//     and how many keys equal to it are taken; a per-thread count and one
//     workgroup scan place every selected id in ascending order, the lowest
//     ids winning among equal keys.
// Integer work after phase 1 is exact, so the selection is a fixed function
// of the fp32 scores.
#include <float.h>

#include "ksa_device.h"
#include "ksa_internal.h"
#include "ksa_topk.h"

namespace ksa {
namespace {

#ifndef KSA_SCORE_THREADS
#define KSA_SCORE_THREADS 256
#endif
#ifndef KSA_SCORE_UNROLL
#define KSA_SCORE_UNROLL 8
#endif
constexpr int kScoreThreads = KSA_SCORE_THREADS;  // per scoring workgroup
constexpr int kScoreUnroll = KSA_SCORE_UNROLL;    // summaries in flight per lane
constexpr int kTopkThreads = 256;  // one workgroup per row; also the histogram size

// Relevance of a tile of blocks of one row.  Every LPT-lane group issues all
// of its loads before consuming any.  MAXAGG: the selection variant that
// ranks a block by its largest single-head dot product (each head's q kept
// in registers) instead of the group's sum.  forced >= 0: that block's key
// is the largest possible, so it is always selected (its score is still
// reported as computed).
// Row block counts: uniform d.NB, or from seq_lens (rows of a paged cache;
// key rows keep the stride d.NB, the longest row's).
__device__ __forceinline__ int row_blocks(const Dims& d, const int32_t* seq_lens, int b) {
  if (!seq_lens) return d.NB;
  const int Tb = seq_len_of(seq_lens, b, d.T);
  return (Tb + d.Bs - 1) / d.Bs;
}

template <typename T, int D, bool MAXAGG>
__global__ __launch_bounds__(kScoreThreads) void block_score_kernel(
    const T* __restrict__ q, const T* __restrict__ summ, Dims d, uint32_t* __restrict__ keys,
    float* __restrict__ block_scores, float score_scale, int forced,
    const int32_t* __restrict__ seq_lens) {
  constexpr int EPL = KV<T>::EPL;
  constexpr int LPT = D / EPL;
  constexpr int NGRP = kScoreThreads / LPT;
  constexpr int TILE = NGRP * kScoreUnroll;
  const int row = blockIdx.y;
  const int b = row / d.Hkv, g = row % d.Hkv;
  const int li = threadIdx.x % LPT, grp = threadIdx.x / LPT;
  const int NB = row_blocks(d, seq_lens, b);
  const int kst = d.NB;  // key row stride
  if (seq_lens && forced >= 0) forced = NB - 1;  // each row's own newest block
  if ((int)blockIdx.x * TILE >= NB) return;  // uniform: a tile past this row's blocks
  const int j0 = blockIdx.x * TILE + grp;
  const T* sp = summ + (int64_t)row * d.NBcap * D + li * EPL;

  uint4 raw[kScoreUnroll];
#pragma unroll
  for (int u = 0; u < kScoreUnroll; ++u)
    raw[u] = ld16_stream(sp + (int64_t)min(j0 + u * NGRP, NB - 1) * D);

  if constexpr (MAXAGG) {
    constexpr int GM = 8;  // largest group
    float qv[GM][EPL];
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      if (h < d.G) KV<T>::widen(ld16(q + ((int64_t)b * d.Hq + g * d.G + h) * D + li * EPL), qv[h]);
    }
#pragma unroll
    for (int u = 0; u < kScoreUnroll; ++u) {
      const int j = j0 + u * NGRP;
      float f[EPL];
      KV<T>::widen(raw[u], f);
      float best = -FLT_MAX;
#pragma unroll
      for (int h = 0; h < GM; ++h) {
        if (h < d.G) {  // uniform
          float p = 0.f;
#pragma unroll
          for (int e = 0; e < EPL; ++e) p = fmaf(qv[h][e], f[e], p);
          best = fmaxf(best, group_sum<LPT>(p));
        }
      }
      if (li == 0 && j < NB) {
        keys[(int64_t)row * kst + j] = j == forced ? 0xFFFFFFFFu : order_key(best);
        if (block_scores) block_scores[(int64_t)row * kst + j] = best * score_scale;
      }
    }
    return;
  }
  // group query: sum of the G heads, fp32
  float qs[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) qs[e] = 0.f;
  for (int h = 0; h < d.G; ++h) {
    float f[EPL];
    KV<T>::widen(ld16(q + ((int64_t)b * d.Hq + g * d.G + h) * D + li * EPL), f);
#pragma unroll
    for (int e = 0; e < EPL; ++e) qs[e] += f[e];
  }
#pragma unroll
  for (int u = 0; u < kScoreUnroll; ++u) {
    const int j = j0 + u * NGRP;
    float f[EPL];
    KV<T>::widen(raw[u], f);
    float p = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) p = fmaf(qs[e], f[e], p);
    p = group_sum<LPT>(p);
    if (li == 0 && j < NB) {
      keys[(int64_t)row * kst + j] = j == forced ? 0xFFFFFFFFu : order_key(p);
      if (block_scores) block_scores[(int64_t)row * kst + j] = p * score_scale;
    }
  }
}

// Top-k of one row per workgroup of kTopkThreads threads, keys in registers
// (thread t holds positions [t*KPT, (t+1)*KPT)).
// With seq_lens every row has its own block count NB_b and selects
// min(keff, NB_b) ids into a row of id_stride entries, -1 after them.
template <int KPT>
__global__ __launch_bounds__(kTopkThreads) void topk_rows_kernel(
    const uint32_t* __restrict__ gkeys, Dims d, int keff, int32_t* __restrict__ block_idx,
    const int32_t* __restrict__ seq_lens, int id_stride) {
  __shared__ TopkShared sh;
  const int row = blockIdx.x;
  const uint32_t* rk = gkeys + (int64_t)row * d.NB;
  const int n = row_blocks(d, seq_lens, row / d.Hkv);
  const int ke = min(keff, n);
  const int j0 = threadIdx.x * KPT;
  uint32_t key[KPT];
#pragma unroll
  for (int i = 0; i < KPT; ++i) key[i] = j0 + i < n ? rk[j0 + i] : 0u;
  int32_t* out = block_idx + (int64_t)row * (seq_lens ? id_stride : keff);
  if (seq_lens)
    for (int i = ke + (int)threadIdx.x; i < id_stride; i += kTopkThreads) out[i] = -1;
  topk_clear(sh);
  row_topk<KPT>(key, KPT, j0, n, ke, sh, [&](int rank, int j) { out[rank] = j; });
}

template <typename T, int D>
hipError_t launch_typed(const Dims& d, const void* q, const void* summ, int keff, int32_t* idx,
                        float* scores, uint32_t* keys, const SelectVariant& var, hipStream_t s) {
  constexpr int LPT = D / KV<T>::EPL;
  constexpr int TILE = (kScoreThreads / LPT) * kScoreUnroll;
  const int rows = d.B * d.Hkv;
  const dim3 sgrid((d.NB + TILE - 1) / TILE, rows);
  if (var.agg_max)
    hipLaunchKernelGGL((block_score_kernel<T, D, true>), sgrid, dim3(kScoreThreads), 0, s,
                       (const T*)q, (const T*)summ, d, keys, scores, d.scale, var.forced_block,
                       var.seq_lens);
  else
    hipLaunchKernelGGL((block_score_kernel<T, D, false>), sgrid, dim3(kScoreThreads), 0, s,
                       (const T*)q, (const T*)summ, d, keys, scores, d.scale / (float)d.G,
                       var.forced_block, var.seq_lens);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid(rows), block(kTopkThreads);
  const int32_t* sl = var.seq_lens;
  const int ids = var.id_stride;
  if (d.NB <= 4 * kTopkThreads)
    hipLaunchKernelGGL((topk_rows_kernel<4>), grid, block, 0, s, keys, d, keff, idx, sl, ids);
  else if (d.NB <= 8 * kTopkThreads)
    hipLaunchKernelGGL((topk_rows_kernel<8>), grid, block, 0, s, keys, d, keff, idx, sl, ids);
  else if (d.NB <= 16 * kTopkThreads)
    hipLaunchKernelGGL((topk_rows_kernel<16>), grid, block, 0, s, keys, d, keff, idx, sl, ids);
  else
    hipLaunchKernelGGL((topk_rows_kernel<64>), grid, block, 0, s, keys, d, keff, idx, sl, ids);
  return hipGetLastError();
}

}  // namespace

size_t select_workspace_bytes(const Dims& d) {
  return (size_t)d.B * d.Hkv * d.NB * sizeof(uint32_t);
}

hipError_t launch_select_topk(const Dims& d, const void* q, const void* summaries, int keff,
                              int32_t* block_idx, float* block_scores, void* workspace,
                              hipStream_t stream, const SelectVariant& var) {
  uint32_t* k = (uint32_t*)workspace;
  if (d.dtype == KSA_BF16) {
    if (d.D == 64)
      return launch_typed<uint16_t, 64>(d, q, summaries, keff, block_idx, block_scores, k, var, stream);
    return launch_typed<uint16_t, 128>(d, q, summaries, keff, block_idx, block_scores, k, var, stream);
  }
  if (d.D == 64)
    return launch_typed<float, 64>(d, q, summaries, keff, block_idx, block_scores, k, var, stream);
  return launch_typed<float, 128>(d, q, summaries, keff, block_idx, block_scores, k, var, stream);
}

}  // namespace ksa

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
//     registers: a bucket search over the row's key range (LDS histograms of
//     at most 256 buckets, one wave scanning them) finds the k-th largest key
//     `thr` and how many keys equal to it are taken; a per-thread count and
//     one workgroup scan place every selected id in ascending order, the
//     lowest ids winning among keys equal to thr.
// Integer work after phase 1 is exact, so the selection is a fixed function
// of the fp32 scores.
#include "ksa_device.h"
#include "ksa_internal.h"

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
// of its loads before consuming any.
template <typename T, int D>
__global__ __launch_bounds__(kScoreThreads) void block_score_kernel(
    const T* __restrict__ q, const T* __restrict__ summ, Dims d, uint32_t* __restrict__ keys,
    float* __restrict__ block_scores, float score_scale) {
  constexpr int EPL = KV<T>::EPL;
  constexpr int LPT = D / EPL;
  constexpr int NGRP = kScoreThreads / LPT;
  constexpr int TILE = NGRP * kScoreUnroll;
  const int row = blockIdx.y;
  const int b = row / d.Hkv, g = row % d.Hkv;
  const int li = threadIdx.x % LPT, grp = threadIdx.x / LPT;
  const int NB = d.NB;
  const int j0 = blockIdx.x * TILE + grp;
  const T* sp = summ + (int64_t)row * d.NBcap * D + li * EPL;

  uint4 raw[kScoreUnroll];
#pragma unroll
  for (int u = 0; u < kScoreUnroll; ++u)
    raw[u] = ld16_stream(sp + (int64_t)min(j0 + u * NGRP, NB - 1) * D);

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
      keys[(int64_t)row * NB + j] = order_key(p);
      if (block_scores) block_scores[(int64_t)row * NB + j] = p * score_scale;
    }
  }
}

// Top-k of one row per workgroup of kTopkThreads threads.  Thread t holds
// keys [t*KPT, (t+1)*KPT) in registers, so a per-thread count and one
// workgroup scan give every selected id its place in ascending order.
//
// Bucket search on the row's key range: with all candidates in [lo, hi], a
// key's bucket is (key - lo) >> shift, shift chosen so that the range maps
// onto at most 256 buckets (a monotone map, so buckets are ordered like the
// keys).  One LDS histogram and one wave scan find the bucket holding the
// `remaining`-th largest candidate; the range shrinks to that bucket.  It
// stops when that bucket holds exactly the keys still needed (all of them
// are taken) or when it is a single key value (the lowest ids among equal
// keys are taken).  Buckets follow the data's own range rather than fixed
// bit fields, so fp32 scores spread over the histogram instead of piling
// onto the few bins a fixed top byte gives them.
template <int KPT>
__global__ __launch_bounds__(kTopkThreads) void topk_rows_kernel(
    const uint32_t* __restrict__ gkeys, int NB, int keff, int32_t* __restrict__ block_idx) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t red[2][kTopkThreads / 64];
  __shared__ uint32_t sh_bucket[3];
  __shared__ uint64_t scan_scratch[17];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = blockIdx.x;
  const uint32_t* rk = gkeys + (int64_t)row * NB;
  const int j0 = tid * KPT;
  uint32_t key[KPT];
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const bool in = j0 + i < NB;
    key[i] = in ? rk[j0 + i] : 0u;
    if (in) {
      kmin = min(kmin, key[i]);
      kmax = max(kmax, key[i]);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o));
  }
  if (lane == 0) {
    red[0][wave] = kmin;
    red[1][wave] = kmax;
  }
  __syncthreads();
  uint32_t lo = red[0][0], hi = red[1][0];
#pragma unroll
  for (int w = 1; w < kTopkThreads / 64; ++w) {
    lo = min(lo, red[0][w]);
    hi = max(hi, red[1][w]);
  }

  uint32_t remaining = (uint32_t)keff;
  uint32_t quota, thr;
#pragma unroll 1
  for (;;) {
    const uint32_t span = hi - lo;
    if (span == 0) {  // one value left: ties, lowest ids first
      thr = lo;
      quota = remaining;
      break;
    }
    const int bits = 32 - __clz(span);
    const int shift = bits > 8 ? bits - 8 : 0;
    hist[tid] = 0;  // kTopkThreads == 256 bins
    __syncthreads();
#pragma unroll
    for (int i = 0; i < KPT; ++i)
      if (j0 + i < NB && key[i] >= lo && key[i] <= hi) atomicAdd(&hist[(key[i] - lo) >> shift], 1u);
    __syncthreads();
    if (wave == 0) {
      // lane l holds buckets 255-4l .. 252-4l (highest in lane 0)
      const int top = 255 - 4 * lane;
      const uint32_t c0 = hist[top], c1 = hist[top - 1], c2 = hist[top - 2], c3 = hist[top - 3];
      const uint32_t s = c0 + c1 + c2 + c3;
      const uint32_t incl = wave_incl_scan(s);
      const uint32_t excl = incl - s;
      if (excl < remaining && remaining <= incl) {
        uint32_t c = excl, n;
        int bk;
        if (c + c0 >= remaining) {
          bk = top; n = c0;
        } else if ((c += c0) + c1 >= remaining) {
          bk = top - 1; n = c1;
        } else if ((c += c1) + c2 >= remaining) {
          bk = top - 2; n = c2;
        } else {
          c += c2;
          bk = top - 3; n = c3;
        }
        sh_bucket[0] = (uint32_t)bk;
        sh_bucket[1] = c;
        sh_bucket[2] = n;
      }
    }
    __syncthreads();
    const uint32_t bk = sh_bucket[0], above = sh_bucket[1], n = sh_bucket[2];
    remaining -= above;
    const uint64_t blo = (uint64_t)lo + ((uint64_t)bk << shift);
    const uint64_t bhi = (uint64_t)lo + (((uint64_t)bk + 1) << shift) - 1;
    lo = (uint32_t)blo;
    hi = bhi < (uint64_t)hi ? (uint32_t)bhi : hi;
    if (n == remaining) {  // the whole bucket is taken: everything >= lo
      thr = lo;
      quota = 0xFFFFFFFFu;
      break;
    }
  }

  // ascending compaction: keys > thr, then keys == thr up to the quota
  uint32_t n_gt = 0, n_eq = 0;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    n_gt += (j0 + i < NB) && key[i] > thr;
    n_eq += (j0 + i < NB) && key[i] == thr;
  }
  uint64_t total;
  const uint64_t before = block_excl_scan64(((uint64_t)n_gt << 32) | n_eq, scan_scratch, &total);
  uint32_t gt_before = (uint32_t)(before >> 32), eq_before = (uint32_t)before;
  int32_t* out = block_idx + (int64_t)row * keff;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    if (j0 + i >= NB) break;
    if (key[i] > thr) {
      out[gt_before + min(eq_before, quota)] = j0 + i;
      ++gt_before;
    } else if (key[i] == thr) {
      if (eq_before < quota) out[gt_before + eq_before] = j0 + i;
      ++eq_before;
    }
  }
}

template <typename T, int D>
hipError_t launch_typed(const Dims& d, const void* q, const void* summ, int keff, int32_t* idx,
                        float* scores, uint32_t* keys, hipStream_t s) {
  constexpr int LPT = D / KV<T>::EPL;
  constexpr int TILE = (kScoreThreads / LPT) * kScoreUnroll;
  const float score_scale = d.scale / (float)d.G;
  const int rows = d.B * d.Hkv;
  hipLaunchKernelGGL((block_score_kernel<T, D>), dim3((d.NB + TILE - 1) / TILE, rows),
                     dim3(kScoreThreads), 0, s, (const T*)q, (const T*)summ, d, keys, scores,
                     score_scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid(rows), block(kTopkThreads);
  if (d.NB <= 4 * kTopkThreads)
    hipLaunchKernelGGL((topk_rows_kernel<4>), grid, block, 0, s, keys, d.NB, keff, idx);
  else if (d.NB <= 8 * kTopkThreads)
    hipLaunchKernelGGL((topk_rows_kernel<8>), grid, block, 0, s, keys, d.NB, keff, idx);
  else if (d.NB <= 16 * kTopkThreads)
    hipLaunchKernelGGL((topk_rows_kernel<16>), grid, block, 0, s, keys, d.NB, keff, idx);
  else
    hipLaunchKernelGGL((topk_rows_kernel<64>), grid, block, 0, s, keys, d.NB, keff, idx);
  return hipGetLastError();
}

}  // namespace

size_t select_workspace_bytes(const Dims& d) {
  return (size_t)d.B * d.Hkv * d.NB * sizeof(uint32_t);
}

hipError_t launch_select_topk(const Dims& d, const void* q, const void* summaries, int keff,
                              int32_t* block_idx, float* block_scores, void* workspace,
                              hipStream_t stream) {
  uint32_t* keys = (uint32_t*)workspace;
  if (d.dtype == KSA_BF16) {
    if (d.D == 64)
      return launch_typed<uint16_t, 64>(d, q, summaries, keff, block_idx, block_scores, keys, stream);
    return launch_typed<uint16_t, 128>(d, q, summaries, keff, block_idx, block_scores, keys, stream);
  }
  if (d.D == 64)
    return launch_typed<float, 64>(d, q, summaries, keff, block_idx, block_scores, keys, stream);
  return launch_typed<float, 128>(d, q, summaries, keff, block_idx, block_scores, keys, stream);
}

}  // namespace ksa

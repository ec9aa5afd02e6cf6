// select.hip -- choose the K' most relevant blocks per (sequence, KV head)
// (Kinetics explainer, section 五: blocks are ranked by the relevance of
// their mean key to the query and the top K' are attended).
//
// One workgroup per (sequence b, KV head g) row, in three phases:
//  1. Scoring.  The relevance of block j is sum_h q_h . S_j over the group's
//     G query heads, computed as (sum_h q_h) . S_j in fp32 (the group query
//     is summed once; bf16 x bf16 products are exact in fp32).  Groups of
//     LPT lanes stream the row's summaries with 16-byte loads and reduce the
//     dot product with DPP; each score becomes an order-preserving uint32 key
//     kept in LDS.
//  2. Threshold.  An MSB-first radix select (four 8-bit digits, LDS
//     histograms, one wave scanning the 256 bins) finds the k-th largest key
//     `thr` and how many keys equal to it must be taken.
//  3. Compaction.  Each thread owns a contiguous run of block ids; one
//     workgroup scan of (#keys > thr, #keys == thr) gives every selected block
//     its output slot, so block_idx comes out in ascending order, and among
//     keys equal to thr the lowest ids win.
// Integer work after phase 1 is exact, so the selection is a fixed function
// of the fp32 scores.
#include "ksa_device.h"
#include "ksa_internal.h"

namespace ksa {
namespace {

constexpr int kSelThreads = 512;
constexpr int kSelUnroll = 8;

template <typename T, int D>
__global__ __launch_bounds__(kSelThreads) void select_topk_kernel(
    const T* __restrict__ q, const T* __restrict__ summ, Dims d, int keff,
    int32_t* __restrict__ block_idx, float* __restrict__ block_scores, float score_scale) {
  constexpr int EPL = KV<T>::EPL;
  constexpr int LPT = D / EPL;
  constexpr int NGRP = kSelThreads / LPT;
  extern __shared__ uint32_t keys[];  // NB keys
  __shared__ uint32_t hist[256];
  __shared__ uint64_t scan_scratch[17];
  __shared__ uint32_t sh_digit, sh_above;

  const int tid = threadIdx.x;
  const int row = blockIdx.x;
  const int b = row / d.Hkv, g = row % d.Hkv;
  const int li = tid % LPT, grp = tid / LPT;
  const int NB = d.NB;

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

  // 1. scoring
  const T* sp = summ + (int64_t)row * d.NBcap * D + li * EPL;
  for (int j0 = grp; j0 < NB; j0 += NGRP * kSelUnroll) {
    uint4 raw[kSelUnroll];
#pragma unroll
    for (int u = 0; u < kSelUnroll; ++u) {
      const int j = min(j0 + u * NGRP, NB - 1);
      raw[u] = ld16(sp + (int64_t)j * D);
    }
#pragma unroll
    for (int u = 0; u < kSelUnroll; ++u) {
      const int j = j0 + u * NGRP;
      float f[EPL];
      KV<T>::widen(raw[u], f);
      float p = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) p = fmaf(qs[e], f[e], p);
      p = group_sum<LPT>(p);
      if (li == 0 && j < NB) {
        keys[j] = order_key(p);
        if (block_scores) block_scores[(int64_t)row * NB + j] = p * score_scale;
      }
    }
  }
  __syncthreads();

  // 2. radix select of the keff-th largest key
  uint32_t prefix = 0, mask = 0;
  uint32_t remaining = (uint32_t)keff;
#pragma unroll 1
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < 256; i += kSelThreads) hist[i] = 0;
    __syncthreads();
    for (int j = tid; j < NB; j += kSelThreads) {
      const uint32_t key = keys[j];
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      // lane l holds bins 255-4l .. 252-4l (highest digits in lane 0)
      const int top = 255 - 4 * tid;
      const uint32_t c0 = hist[top], c1 = hist[top - 1], c2 = hist[top - 2], c3 = hist[top - 3];
      const uint32_t s = c0 + c1 + c2 + c3;
      const uint32_t incl = wave_incl_scan(s);
      const uint32_t excl = incl - s;
      if (excl < remaining && remaining <= incl) {
        uint32_t c = excl;
        int dig;
        if (c + c0 >= remaining) {
          dig = top;
        } else if ((c += c0) + c1 >= remaining) {
          dig = top - 1;
        } else if ((c += c1) + c2 >= remaining) {
          dig = top - 2;
        } else {
          c += c2;
          dig = top - 3;
        }
        sh_digit = (uint32_t)dig;
        sh_above = c;
      }
    }
    __syncthreads();
    prefix |= sh_digit << shift;
    mask |= 255u << shift;
    remaining -= sh_above;
    __syncthreads();
  }
  const uint32_t thr = prefix;  // remaining = keys equal to thr still to take (>= 1)

  // 3. ascending compaction
  const int per = (NB + kSelThreads - 1) / kSelThreads;
  const int ja = min(tid * per, NB), jb = min(ja + per, NB);
  uint32_t n_gt = 0, n_eq = 0;
  for (int j = ja; j < jb; ++j) {
    const uint32_t key = keys[j];
    n_gt += key > thr;
    n_eq += key == thr;
  }
  uint64_t total;
  const uint64_t before =
      block_excl_scan64(((uint64_t)n_gt << 32) | n_eq, scan_scratch, &total);
  uint32_t gt_before = (uint32_t)(before >> 32), eq_before = (uint32_t)before;
  int32_t* out = block_idx + (int64_t)row * keff;
  for (int j = ja; j < jb; ++j) {
    const uint32_t key = keys[j];
    if (key > thr) {
      out[gt_before + min(eq_before, remaining)] = j;
      ++gt_before;
    } else if (key == thr) {
      if (eq_before < remaining) out[gt_before + eq_before] = j;
      ++eq_before;
    }
  }
}

template <typename T, int D>
hipError_t launch_typed(const Dims& d, const void* q, const void* summ, int keff, int32_t* idx,
                        float* scores, hipStream_t s) {
  const size_t lds = (size_t)d.NB * sizeof(uint32_t);
  const float score_scale = d.scale / (float)d.G;
  hipLaunchKernelGGL((select_topk_kernel<T, D>), dim3(d.B * d.Hkv), dim3(kSelThreads), lds, s,
                     (const T*)q, (const T*)summ, d, keff, idx, scores, score_scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_select_topk(const Dims& d, const void* q, const void* summaries, int keff,
                              int32_t* block_idx, float* block_scores, hipStream_t stream) {
  if (d.dtype == KSA_BF16) {
    if (d.D == 64) return launch_typed<uint16_t, 64>(d, q, summaries, keff, block_idx, block_scores, stream);
    return launch_typed<uint16_t, 128>(d, q, summaries, keff, block_idx, block_scores, stream);
  }
  if (d.D == 64) return launch_typed<float, 64>(d, q, summaries, keff, block_idx, block_scores, stream);
  return launch_typed<float, 128>(d, q, summaries, keff, block_idx, block_scores, stream);
}

}  // namespace ksa

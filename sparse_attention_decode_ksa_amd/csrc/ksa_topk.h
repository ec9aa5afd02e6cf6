// ksa_topk.h -- exact top-k of one row of order-preserving uint32 keys by
// one workgroup (the "keep the K' most relevant blocks" step of the Kinetics
// explainer, section 五).
//
// Every thread holds a contiguous run of the row's keys in registers
// (positions j0 .. j0+kpt-1), so a per-thread count and one workgroup scan
// place every selected position in ascending order.
//
// Bucket search on the row's key range: with all candidates in [lo, hi], a
// key's bucket is (key - lo) >> shift, shift chosen so that the range maps
// onto at most 256 buckets (a monotone map, so buckets are ordered like the
// keys).  One LDS histogram and one wave scan find the bucket holding the
// `remaining`-th largest candidate; the range shrinks to that bucket.  It
// stops when that bucket holds exactly the keys still needed (all of them
// are taken) or when it is a single key value (the lowest positions among
// equal keys are taken).  Buckets follow the data's own range rather than
// fixed bit fields, so fp32 scores spread over the histogram instead of
// piling onto the few bins a fixed top byte gives them.
#pragma once

#include "ksa_device.h"

namespace ksa {

struct TopkShared {
  uint32_t hist[256];
  uint32_t red[2][16];
  uint32_t bucket[3];
  uint64_t scan[17];
};

// Selects the keff largest keys of the row (ties: lowest position first) and
// calls emit(rank, position) for each, rank 0..keff-1 in ascending position
// order.  Thread t's keys are key[0..kpt) at positions j0 + i; positions >= n
// are not candidates.  Requires 1 <= keff <= n, kpt <= KPT, a workgroup of
// 256..1024 threads (a multiple of 64), and every thread of it calling.
template <int KPT, typename Emit>
__device__ __forceinline__ void row_topk(const uint32_t (&key)[KPT], int kpt, int j0, int n,
                                         int keff, TopkShared& sh, Emit emit) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nwaves = blockDim.x >> 6;
  auto valid = [&](int i) { return i < kpt && j0 + i < n; };
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    if (valid(i)) {
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
    sh.red[0][wave] = kmin;
    sh.red[1][wave] = kmax;
  }
  __syncthreads();
  uint32_t lo = sh.red[0][0], hi = sh.red[1][0];
  for (int w = 1; w < nwaves; ++w) {
    lo = min(lo, sh.red[0][w]);
    hi = max(hi, sh.red[1][w]);
  }

  uint32_t remaining = (uint32_t)keff;
  uint32_t quota, thr;
#pragma unroll 1
  for (;;) {
    const uint32_t span = hi - lo;
    if (span == 0) {  // one value left: ties, lowest positions first
      thr = lo;
      quota = remaining;
      break;
    }
    const int bits = 32 - __clz(span);
    const int shift = bits > 8 ? bits - 8 : 0;
    if (tid < 256) sh.hist[tid] = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < KPT; ++i)
      if (valid(i) && key[i] >= lo && key[i] <= hi) atomicAdd(&sh.hist[(key[i] - lo) >> shift], 1u);
    __syncthreads();
    if (wave == 0) {
      // lane l holds buckets 255-4l .. 252-4l (highest in lane 0)
      const int top = 255 - 4 * lane;
      const uint32_t c0 = sh.hist[top], c1 = sh.hist[top - 1], c2 = sh.hist[top - 2],
                     c3 = sh.hist[top - 3];
      const uint32_t s = c0 + c1 + c2 + c3;
      const uint32_t incl = wave_incl_scan(s);
      const uint32_t excl = incl - s;
      if (excl < remaining && remaining <= incl) {
        uint32_t c = excl, cnt;
        int bk;
        if (c + c0 >= remaining) {
          bk = top; cnt = c0;
        } else if ((c += c0) + c1 >= remaining) {
          bk = top - 1; cnt = c1;
        } else if ((c += c1) + c2 >= remaining) {
          bk = top - 2; cnt = c2;
        } else {
          c += c2;
          bk = top - 3; cnt = c3;
        }
        sh.bucket[0] = (uint32_t)bk;
        sh.bucket[1] = c;
        sh.bucket[2] = cnt;
      }
    }
    __syncthreads();
    const uint32_t bk = sh.bucket[0], above = sh.bucket[1], cnt = sh.bucket[2];
    remaining -= above;
    const uint64_t blo = (uint64_t)lo + ((uint64_t)bk << shift);
    const uint64_t bhi = (uint64_t)lo + (((uint64_t)bk + 1) << shift) - 1;
    lo = (uint32_t)blo;
    hi = bhi < (uint64_t)hi ? (uint32_t)bhi : hi;
    if (cnt == remaining) {  // the whole bucket is taken: everything >= lo
      thr = lo;
      quota = 0xFFFFFFFFu;
      break;
    }
  }

  // ascending compaction: keys > thr, then keys == thr up to the quota
  uint32_t n_gt = 0, n_eq = 0;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    n_gt += valid(i) && key[i] > thr;
    n_eq += valid(i) && key[i] == thr;
  }
  uint64_t total;
  const uint64_t before = block_excl_scan64(((uint64_t)n_gt << 32) | n_eq, sh.scan, &total);
  uint32_t gt_before = (uint32_t)(before >> 32), eq_before = (uint32_t)before;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    if (!valid(i)) break;
    if (key[i] > thr) {
      emit((int)(gt_before + min(eq_before, quota)), j0 + i);
      ++gt_before;
    } else if (key[i] == thr) {
      if (eq_before < quota) emit((int)(gt_before + eq_before), j0 + i);
      ++eq_before;
    }
  }
}

}  // namespace ksa

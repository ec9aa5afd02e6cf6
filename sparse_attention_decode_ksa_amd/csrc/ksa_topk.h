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
// keys).  One LDS histogram and one DPP wave scan find the bucket holding the
// `remaining`-th largest candidate; the range shrinks to that bucket.  It
// stops when that bucket holds exactly the keys still needed (all of them
// are taken) or when it is a single key value (the lowest positions among
// equal keys are taken).  Buckets follow the data's own range rather than
// fixed bit fields, so fp32 scores spread over the histogram instead of
// piling onto the few bins a fixed top byte gives them.  Two histogram
// buffers alternate between rounds, so a round costs two barriers.
#pragma once

#include "ksa_device.h"

namespace ksa {

// Keys of the cut bucket that the list finish ranks directly (above this,
// the bucket search goes on).
constexpr int kTopkCand = 256;
// Positions a row_topk_list selection mask covers.
constexpr int kTopkMaskWords = 128;
constexpr int kTopkListMax = kTopkMaskWords * 32;

struct TopkShared {
  uint32_t hist[2][256];  // both zero on entry to topk_cut
  uint32_t red[2][16];
  uint32_t bucket[3];
  uint32_t scan[16];
  uint32_t ncand;              // zero on entry to topk_cut_fp32
  uint32_t cut[2];
  uint64_t cand[kTopkCand];    // (key << 32) | ~position of the cut bucket's keys
  uint32_t mask[kTopkMaskWords];  // selected positions (row_topk_list), zero on entry
};

// Zeroes both histogram buffers, the candidate count and the selection mask
// (every thread of the workgroup calls it; the caller's next barrier
// publishes it).
__device__ __forceinline__ void topk_clear(TopkShared& sh) {
  for (int i = threadIdx.x; i < 512; i += blockDim.x) (&sh.hist[0][0])[i] = 0u;
  for (int i = threadIdx.x; i < kTopkMaskWords; i += blockDim.x) sh.mask[i] = 0u;
  if (threadIdx.x == 0) sh.ncand = 0u;
}

// Where the keff largest keys of a row end: every key > thr is taken, and
// of the keys == thr the `quota` at the lowest positions (quota 0xFFFFFFFF:
// all of them, which is exactly what is still needed).
struct TopkCut {
  uint32_t thr, quota;
};

// The bucket search.  Thread t's candidates are key[i] with valid(i); every
// candidate lies in [lo, hi].  Requires 1 <= keff <= the number of
// candidates, both histogram buffers zero and visible, a workgroup of
// 256..1024 threads (a multiple of 64), and every thread of it calling.
// Leaves one histogram buffer dirty (row_topk_range does not reuse them).
template <int KPT, typename Valid>
__device__ __forceinline__ TopkCut topk_cut(const uint32_t (&key)[KPT], Valid valid, int keff,
                                            uint32_t lo, uint32_t hi, TopkShared& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t remaining = (uint32_t)keff;
  int buf = 0;
#pragma unroll 1
  for (;;) {
    const uint32_t span = hi - lo;
    if (span == 0) return TopkCut{lo, remaining};  // one value left: ties, lowest positions first
    const int bits = 32 - __clz(span);
    const int shift = bits > 8 ? bits - 8 : 0;
    uint32_t* hist = sh.hist[buf];
    // the other buffer is cleared for the next round (nobody reads it now)
    if (tid < 256) sh.hist[buf ^ 1][tid] = 0u;
#pragma unroll
    for (int i = 0; i < KPT; ++i)
      if (valid(i) && key[i] >= lo && key[i] <= hi) atomicAdd(&hist[(key[i] - lo) >> shift], 1u);
    __syncthreads();
    if (wave == 0) {
      // lane l holds buckets 255-4l .. 252-4l (highest in lane 0)
      const int top = 255 - 4 * lane;
      const uint32_t c0 = hist[top], c1 = hist[top - 1], c2 = hist[top - 2], c3 = hist[top - 3];
      const uint32_t s = c0 + c1 + c2 + c3;
      const uint32_t incl = wave_incl_scan_dpp(s);
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
    buf ^= 1;
    remaining -= above;
    const uint64_t blo = (uint64_t)lo + ((uint64_t)bk << shift);
    const uint64_t bhi = (uint64_t)lo + (((uint64_t)bk + 1) << shift) - 1;
    lo = (uint32_t)blo;
    hi = bhi < (uint64_t)hi ? (uint32_t)bhi : hi;
    if (cnt == remaining) return TopkCut{lo, 0xFFFFFFFFu};  // the whole bucket: everything >= lo
  }
}

// The fp32 score a key encodes (the inverse of order_key).
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Finishes the cut once the bucket holding it is known: the bucket's `cnt`
// keys (in_bucket(i); cnt <= kTopkCand) are listed in LDS with their
// positions, packed so that (key desc, position asc) is descending order of
// the packed value, and each is ranked by counting the list entries above
// it.  The entry ranked rem-1 gives the threshold key; the quota is rem less
// the entries whose key is above it.  Two barriers, where a bucket round
// costs two per round.  Requires sh.ncand == 0 and visible, and every thread
// of the workgroup calling.
template <int KPT, typename InBucket>
__device__ __forceinline__ TopkCut topk_finish_list(const uint32_t (&key)[KPT], InBucket in_bucket,
                                                    int j0, uint32_t cnt, uint32_t rem,
                                                    TopkShared& sh) {
#pragma unroll
  for (int i = 0; i < KPT; ++i)
    if (in_bucket(i))
      sh.cand[atomicAdd(&sh.ncand, 1u)] =
          ((uint64_t)key[i] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)(j0 + i));
  __syncthreads();
  for (uint32_t t = threadIdx.x; t < cnt; t += blockDim.x) {
    const uint64_t v = sh.cand[t];
    uint32_t above = 0;
    for (uint32_t j = 0; j < cnt; ++j) above += sh.cand[j] > v;
    if (above == rem - 1u) {  // exactly one entry: the packed values are distinct
      const uint32_t thr = (uint32_t)(v >> 32);
      uint32_t gt = 0;
      for (uint32_t j = 0; j < cnt; ++j) gt += (uint32_t)(sh.cand[j] >> 32) > thr;
      sh.cut[0] = thr;
      sh.cut[1] = rem - gt;
    }
  }
  __syncthreads();
  return TopkCut{sh.cut[0], sh.cut[1]};
}

// topk_cut for keys of fp32 scores, with a first round on the scores' own
// scale: bucket = floor((x - x_lo) * 256 / (x_hi - x_lo)) is monotone in x
// (each fp32 step rounds monotonically), and it spreads scores over the
// histogram where their bit patterns, whose leading bits are mostly the
// exponent, pile onto a few buckets (which serialises the LDS atomics).  A
// cut bucket of at most kTopkCand keys is finished by topk_finish_list
// (thread t's key i sits at position j0 + i); a larger one narrows the key
// range for topk_cut.  Same requirements as topk_cut, and sh.ncand zero.
template <int KPT, typename Valid>
__device__ __forceinline__ TopkCut topk_cut_fp32(const uint32_t (&key)[KPT], Valid valid, int keff,
                                                 uint32_t lo, uint32_t hi, int j0, TopkShared& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nwaves = blockDim.x >> 6;
  const float xlo = key_value(lo);
  const float scale = 256.0f / (key_value(hi) - xlo);
  // a range too wide for fp32 arithmetic, or too narrow to scale, skips the round
  if (!(hi > lo) || !(scale > 0.f && scale < 1.0e30f))
    return topk_cut<KPT>(key, valid, keff, lo, hi, sh);
  auto bucket = [&](uint32_t k) { return min(255, (int)((key_value(k) - xlo) * scale)); };
  uint32_t* hist = sh.hist[0];
#pragma unroll
  for (int i = 0; i < KPT; ++i)
    if (valid(i)) atomicAdd(&hist[bucket(key[i])], 1u);
  __syncthreads();
  if (wave == 0) {
    const int top = 255 - 4 * lane;
    const uint32_t c0 = hist[top], c1 = hist[top - 1], c2 = hist[top - 2], c3 = hist[top - 3];
    const uint32_t s = c0 + c1 + c2 + c3;
    const uint32_t incl = wave_incl_scan_dpp(s);
    const uint32_t excl = incl - s;
    const uint32_t need = (uint32_t)keff;
    if (excl < need && need <= incl) {
      uint32_t c = excl, cnt;
      int bk;
      if (c + c0 >= need) {
        bk = top; cnt = c0;
      } else if ((c += c0) + c1 >= need) {
        bk = top - 1; cnt = c1;
      } else if ((c += c1) + c2 >= need) {
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
  const int bk = (int)sh.bucket[0];
  const uint32_t rem = (uint32_t)keff - sh.bucket[1], cnt = sh.bucket[2];
  if (cnt <= (uint32_t)kTopkCand)
    return topk_finish_list<KPT>(key, [&](int i) { return valid(i) && bucket(key[i]) == bk; }, j0,
                                 cnt, rem, sh);
  // the bucket's key range (keys between two of its keys are in it too)
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    if (valid(i) && bucket(key[i]) == bk) {
      kmin = min(kmin, key[i]);
      kmax = max(kmax, key[i]);
    }
  }
  kmin = wave_min_dpp(kmin);
  kmax = wave_max_dpp(kmax);
  if (tid < 256) hist[tid] = 0u;  // read by wave 0 before the last barrier
  if (lane == 0) {
    sh.red[0][wave] = kmin;
    sh.red[1][wave] = kmax;
  }
  __syncthreads();
  lo = sh.red[0][0];
  hi = sh.red[1][0];
  for (int w = 1; w < nwaves; ++w) {
    lo = min(lo, sh.red[0][w]);
    hi = max(hi, sh.red[1][w]);
  }
  if (cnt == rem) return TopkCut{lo, 0xFFFFFFFFu};  // the whole bucket is taken
  return topk_cut<KPT>(key, valid, (int)rem, lo, hi, sh);
}

// Selects the keff largest keys of the row (ties: lowest position first) and
// calls emit(rank, position) for each, rank 0..keff-1 in ascending position
// order.  Thread t's keys are key[0..kpt) at positions j0 + i; positions >= n
// are not candidates; every candidate key lies in [lo, hi].  Requires
// 1 <= keff <= n, n <= 65535, kpt <= KPT, both histogram buffers zero and
// visible, a workgroup of 256..1024 threads (a multiple of 64), and every
// thread of it calling.
template <int KPT, typename Emit>
__device__ __forceinline__ void row_topk_range(const uint32_t (&key)[KPT], int kpt, int j0, int n,
                                               int keff, uint32_t lo, uint32_t hi, TopkShared& sh,
                                               Emit emit) {
  auto valid = [&](int i) { return i < kpt && j0 + i < n; };
  const TopkCut cut = topk_cut_fp32<KPT>(key, valid, keff, lo, hi, j0, sh);
  const uint32_t thr = cut.thr, quota = cut.quota;

  // ascending compaction: keys > thr, then keys == thr up to the quota.
  // Counts are packed (gt << 16 | eq); both totals stay below 2^16.
  uint32_t n_gt = 0, n_eq = 0;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    n_gt += valid(i) && key[i] > thr;
    n_eq += valid(i) && key[i] == thr;
  }
  const uint32_t before = block_excl_scan32((n_gt << 16) | n_eq, sh.scan);
  uint32_t gt_before = before >> 16, eq_before = before & 0xFFFFu;
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

// As row_topk_range, with the key range found here (one min/max reduction).
// Requires both histogram buffers zero; they need not be visible yet (the
// reduction's barrier publishes them).
template <int KPT, typename Emit>
__device__ __forceinline__ void row_topk(const uint32_t (&key)[KPT], int kpt, int j0, int n,
                                         int keff, TopkShared& sh, Emit emit) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    if (i < kpt && j0 + i < n) {
      kmin = min(kmin, key[i]);
      kmax = max(kmax, key[i]);
    }
  }
  kmin = wave_min_dpp(kmin);
  kmax = wave_max_dpp(kmax);
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
  row_topk_range<KPT>(key, kpt, j0, n, keff, lo, hi, sh, emit);
}

// The bucket of the histogram `hist` (256 counts, highest bucket 255)
// holding the need-th largest candidate, found by every wave on its own (the
// scan of topk_cut): returns the bucket, the candidates above it and those
// in it, wave-uniform.  Requires need <= the histogram's total.
__device__ __forceinline__ void wave_cut_bucket(const uint32_t* hist, uint32_t need, int* bk,
                                                uint32_t* above, uint32_t* cnt) {
  const int lane = threadIdx.x & 63;
  const int top = 255 - 4 * lane;  // lane l holds buckets 255-4l .. 252-4l
  const uint32_t c0 = hist[top], c1 = hist[top - 1], c2 = hist[top - 2], c3 = hist[top - 3];
  const uint32_t sum = c0 + c1 + c2 + c3;
  const uint32_t incl = wave_incl_scan_dpp(sum);
  const uint32_t excl = incl - sum;
  uint32_t c = excl, n;
  int b;
  if (c + c0 >= need) {
    b = top; n = c0;
  } else if ((c += c0) + c1 >= need) {
    b = top - 1; n = c1;
  } else if ((c += c1) + c2 >= need) {
    b = top - 2; n = c2;
  } else {
    c += c2;
    b = top - 3; n = c3;
  }
  const int src = __ffsll((unsigned long long)__ballot(excl < need && need <= incl)) - 1;
  *bk = __builtin_amdgcn_readlane(b, src);
  *above = __builtin_amdgcn_readlane(c, src);
  *cnt = __builtin_amdgcn_readlane(n, src);
}

// Selects the keff largest keys of a row as row_topk_range does (ties: lowest
// position first), with fewer barriers: one histogram round on the scores'
// own scale, which every wave then scans; the cut bucket's keys listed with
// their positions; each thread ranks its own keys of that bucket against the
// list and marks its selected positions in an LDS bit mask; and after one
// barrier every wave reads the mask and calls emit(rank, position, primary)
// for every selected position in ascending order (primary: the calling wave
// is wave 0, so that once-only side effects can be left to one wave).  Each
// wave returns as soon as its own pass is done: the calls of the other waves
// may still be running.  When the scores' range is unusable for the fp32
// round or the cut bucket holds more than kTopkCand keys, falls back to
// row_topk_range (emit then runs once per selected position, in the owning
// thread, with primary set) and returns after a barrier.  Requires
// row_topk_range's conditions, n <= kTopkListMax, and sh cleared by
// topk_clear before the caller's last barrier.
template <int KPT, typename Emit>
__device__ __forceinline__ void row_topk_list(const uint32_t (&key)[KPT], int kpt, int j0, int n,
                                              int keff, uint32_t lo, uint32_t hi, TopkShared& sh,
                                              Emit emit) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  auto valid = [&](int i) { return i < kpt && j0 + i < n; };
  auto fallback = [&]() {
    row_topk_range<KPT>(key, kpt, j0, n, keff, lo, hi, sh,
                        [&](int rank, int j) { emit(rank, j, true); });
    __syncthreads();
  };
  const float xlo = key_value(lo);
  const float scale = 256.0f / (key_value(hi) - xlo);
  if (!(hi > lo) || !(scale > 0.f && scale < 1.0e30f)) {
    fallback();
    return;
  }
  auto bucket = [&](uint32_t k) { return min(255, (int)((key_value(k) - xlo) * scale)); };
  uint32_t* hist = sh.hist[0];
#pragma unroll
  for (int i = 0; i < KPT; ++i)
    if (valid(i)) atomicAdd(&hist[bucket(key[i])], 1u);
  __syncthreads();
  int bk;
  uint32_t above, cnt;
  wave_cut_bucket(hist, (uint32_t)keff, &bk, &above, &cnt);
  if (cnt > (uint32_t)kTopkCand) {  // uniform: every wave found the same bucket
    __syncthreads();  // every wave has read the histogram
    if (threadIdx.x < 256) hist[threadIdx.x] = 0u;
    __syncthreads();
    fallback();
    return;
  }
  const uint32_t rem = (uint32_t)keff - above;
  auto packed = [&](int i) {
    return ((uint64_t)key[i] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)(j0 + i));
  };
#pragma unroll
  for (int i = 0; i < KPT; ++i)
    if (valid(i) && bucket(key[i]) == bk) sh.cand[atomicAdd(&sh.ncand, 1u)] = packed(i);
  __syncthreads();
  // a key above the cut bucket is taken; one in it is taken when fewer than
  // rem of the bucket's keys come before it in (key desc, position asc)
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    if (!valid(i)) continue;
    const int b = bucket(key[i]);
    bool take = b > bk;
    if (b == bk) {
      const uint64_t v = packed(i);
      uint32_t before = 0;
      for (uint32_t j = 0; j < cnt; ++j) before += sh.cand[j] > v;
      take = before < rem;
    }
    if (take) atomicOr(&sh.mask[(j0 + i) >> 5], 1u << ((j0 + i) & 31));
  }
  __syncthreads();
  // every wave: the selected positions in ascending order, from the mask
  const int words = (n + 31) >> 5;
  uint32_t base = 0;
  for (int w0 = 0; w0 < words; w0 += 64) {
    const int wi = w0 + lane;
    uint32_t m = wi < words ? sh.mask[wi] : 0u;
    const uint32_t pc = (uint32_t)__popc(m);
    const uint32_t incl = wave_incl_scan_dpp(pc);
    uint32_t r = base + incl - pc;
    while (m) {
      emit((int)r++, wi * 32 + __ffs(m) - 1, wave == 0);
      m &= m - 1u;
    }
    base += __builtin_amdgcn_readlane(incl, 63);
  }
}

}  // namespace ksa

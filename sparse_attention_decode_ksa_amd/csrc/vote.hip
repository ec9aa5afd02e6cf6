// vote.hip -- the shared token set of the vote-union variant (LessIsMore
// explainer, section 二: equal votes per head, tokens ranked by vote total,
// 75 % of the budget voted / 25 % most recent; section 五: the selection
// layer scores every token for every head, aggregates and sorts the heads'
// picks and appends the most recent tokens).
//
// Per sequence b with history C = [0, T-W) and Kv = N - W picks per head:
//  1. vote_scores: every (b, KV head g) row streams its keys once; the G
//     query heads of the group score each history token in fp32 (lanes and
//     loads as in the attention kernel) and store order-preserving uint32
//     keys [B, Hq, C] in the workspace.
//  2. vote_head_select: one workgroup per (b, h) finds, by MSB-first radix
//     select on the keys, the Kv-th largest key and how many keys equal to it
//     are taken (lowest token ids first), and writes the head's picks as a
//     bitmask [B, Hq, ceil(C/32)] words.
//  3. vote_set: one workgroup per b counts, for every history token, the
//     heads whose bitmask has it (its vote total), finds the vote threshold
//     with a histogram over 0..Hq, and compacts the first Kv tokens by
//     (votes desc, t asc) in ascending order with one workgroup scan; the W
//     recent tokens follow.  Votes are written out as uint8 when asked for.
// Everything after the fp32 scores is exact integer work.
#include <float.h>

#include "ksa_device.h"
#include "ksa_internal.h"

namespace ksa {
namespace {

constexpr int kScoreWaves = 4;
constexpr int kScoreChunksPerWave = 8;
constexpr int kHeadThreads = 512;
constexpr int kSetThreads = 1024;

// ------------------------------------------------------------------ 1
template <typename T, int D, int G>
__global__ __launch_bounds__(kScoreWaves * 64) void vote_scores_kernel(
    const T* __restrict__ q, const T* __restrict__ k, Dims d, int hist,
    uint32_t* __restrict__ keys) {
  constexpr int EPL = KV<T>::EPL;
  constexpr int LPT = D / EPL;
  constexpr int SPW = 64 / LPT;
  constexpr int NI = kLoadsPerChunk;
  constexpr int CH = SPW * NI;
  static_assert(G <= LPT, "one writer lane per head");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int slot = lane / LPT, li = lane % LPT;
  const int row = blockIdx.y;
  const int b = row / d.Hkv, g = row - b * d.Hkv;
  const T* kb = k + (int64_t)row * d.Tcap * D + li * EPL;

  float qv[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h)
    KV<T>::widen(ld16(q + ((int64_t)b * d.Hq + g * G + h) * D + li * EPL), qv[h]);

  const int nchunks = (hist + CH - 1) / CH;
  const int c0 = (blockIdx.x * kScoreWaves + wave) * kScoreChunksPerWave;
  const int c1 = min(c0 + kScoreChunksPerWave, nchunks);
  // head written by this lane (lanes li < G of each slot write)
  uint32_t* kout = keys + ((int64_t)b * d.Hq + g * G + (li < G ? li : 0)) * hist;
  if (c0 >= c1) return;

  uint4 kr[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i)
    kr[i] = ld16_stream(kb + (int64_t)min(c0 * CH + i * SPW + slot, hist - 1) * D);
  for (int c = c0; c < c1; ++c) {
    uint4 kc[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) kc[i] = kr[i];
    if (c + 1 < c1) {
#pragma unroll
      for (int i = 0; i < NI; ++i)
        kr[i] = ld16_stream(kb + (int64_t)min((c + 1) * CH + i * SPW + slot, hist - 1) * D);
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float f[EPL];
      KV<T>::widen(kc[i], f);
      float mine = 0.f;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float p = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) p = fmaf(qv[h][e], f[e], p);
        p = group_sum<LPT>(p);
        if (li == h) mine = p;
      }
      const int t = c * CH + i * SPW + slot;
      if (li < G && t < hist) kout[t] = order_key(mine);
    }
  }
}

// ------------------------------------------------------------------ 2
__global__ __launch_bounds__(kHeadThreads) void vote_head_select_kernel(
    const uint32_t* __restrict__ keys, int hist, int kv, int words, uint32_t* __restrict__ bits) {
  __shared__ uint32_t hbin[256];
  __shared__ uint64_t scan_scratch[17];
  __shared__ uint32_t sh_digit, sh_above, sh_bin;
  const int tid = threadIdx.x;
  const int64_t hr = blockIdx.x;  // b * Hq + h
  const uint32_t* kr = keys + hr * hist;
  uint32_t* br = bits + hr * words;
  if (kv == 0) {  // the whole budget is the recency window: no picks
    for (int w = tid; w < words; w += kHeadThreads) br[w] = 0u;
    return;
  }

  uint32_t prefix = 0, mask = 0, remaining = (uint32_t)kv, eq_total = 0;
#pragma unroll 1
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < 256; i += kHeadThreads) hbin[i] = 0;
    __syncthreads();
    for (int t = tid; t < hist; t += kHeadThreads) {
      const uint32_t key = kr[t];
      if ((key & mask) == prefix) atomicAdd(&hbin[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      const int top = 255 - 4 * tid;
      const uint32_t c0 = hbin[top], c1 = hbin[top - 1], c2 = hbin[top - 2], c3 = hbin[top - 3];
      const uint32_t s = c0 + c1 + c2 + c3;
      const uint32_t incl = wave_incl_scan(s);
      const uint32_t excl = incl - s;
      if (excl < remaining && remaining <= incl) {
        uint32_t c = excl;
        int dig;
        uint32_t bin;
        if (c + c0 >= remaining) {
          dig = top; bin = c0;
        } else if ((c += c0) + c1 >= remaining) {
          dig = top - 1; bin = c1;
        } else if ((c += c1) + c2 >= remaining) {
          dig = top - 2; bin = c2;
        } else {
          c += c2;
          dig = top - 3; bin = c3;
        }
        sh_digit = (uint32_t)dig;
        sh_above = c;
        sh_bin = bin;
      }
    }
    __syncthreads();
    prefix |= sh_digit << shift;
    mask |= 255u << shift;
    remaining -= sh_above;
    eq_total = sh_bin;  // after the last pass: number of keys equal to the threshold
    __syncthreads();
  }
  const uint32_t thr = prefix;
  const int lane = tid & 63;
  if (eq_total == remaining) {
    // every key equal to the threshold is taken: membership is key >= thr
    for (int t0 = 0; t0 < hist; t0 += kHeadThreads) {
      const int t = t0 + tid;
      const bool sel = t < hist && kr[min(t, hist - 1)] >= thr;
      const uint64_t bal = __ballot(sel);
      if (lane == 0 && (t >> 5) < words) br[t >> 5] = (uint32_t)bal;
      if (lane == 32 && (t >> 5) < words) br[t >> 5] = (uint32_t)(bal >> 32);
    }
  } else {
    // only the lowest-index `remaining` of the equal keys are taken
    uint32_t carry = 0;
    for (int t0 = 0; t0 < hist; t0 += kHeadThreads) {
      const int t = t0 + tid;
      const uint32_t key = t < hist ? kr[t] : 0u;
      const bool eq = t < hist && key == thr;
      uint64_t tot;
      const uint32_t before = carry + (uint32_t)block_excl_scan64(eq ? 1 : 0, scan_scratch, &tot);
      const bool sel = t < hist && (key > thr || (eq && before < remaining));
      const uint64_t bal = __ballot(sel);
      if (lane == 0 && (t >> 5) < words) br[t >> 5] = (uint32_t)bal;
      if (lane == 32 && (t >> 5) < words) br[t >> 5] = (uint32_t)(bal >> 32);
      carry += (uint32_t)tot;
    }
  }
}

// ------------------------------------------------------------------ 3
__device__ __forceinline__ void word_votes(const uint32_t* __restrict__ bits, int64_t stride,
                                           int Hq, int w, uint32_t* cnt) {
#pragma unroll
  for (int i = 0; i < 32; ++i) cnt[i] = 0;
  for (int h = 0; h < Hq; ++h) {
    const uint32_t x = bits[(int64_t)h * stride + w];
#pragma unroll
    for (int i = 0; i < 32; ++i) cnt[i] += (x >> i) & 1u;
  }
}

__global__ __launch_bounds__(kSetThreads) void vote_set_kernel(
    const uint32_t* __restrict__ bits, int Hq, int T, int hist, int words, int kv, int N, int W,
    int32_t* __restrict__ token_idx, uint8_t* __restrict__ votes) {
  __shared__ uint32_t vbin[256];
  __shared__ uint64_t scan_scratch[17];
  __shared__ uint32_t sh_v, sh_above;
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const uint32_t* bb = bits + (int64_t)b * Hq * words;

  for (int i = tid; i < 256; i += kSetThreads) vbin[i] = 0;
  __syncthreads();
  for (int w = tid; w < words; w += kSetThreads) {
    uint32_t cnt[32];
    word_votes(bb, words, Hq, w, cnt);
    const int nt = min(32, hist - w * 32);
    for (int i = 0; i < nt; ++i) atomicAdd(&vbin[cnt[i]], 1u);
  }
  __syncthreads();
  // vote threshold v*: count(votes > v*) < kv <= count(votes >= v*)
  if (tid < 64) {
    const int top = 255 - 4 * tid;
    const uint32_t c0 = vbin[top], c1 = vbin[top - 1], c2 = vbin[top - 2], c3 = vbin[top - 3];
    const uint32_t s = c0 + c1 + c2 + c3;
    const uint32_t incl = wave_incl_scan(s);
    const uint32_t excl = incl - s;
    const uint32_t need = (uint32_t)kv;
    if (excl < need && need <= incl) {
      uint32_t c = excl;
      int v;
      if (c + c0 >= need) {
        v = top;
      } else if ((c += c0) + c1 >= need) {
        v = top - 1;
      } else if ((c += c1) + c2 >= need) {
        v = top - 2;
      } else {
        c += c2;
        v = top - 3;
      }
      sh_v = (uint32_t)v;
      sh_above = c;
    }
  }
  if (tid == 0 && kv == 0) {  // nothing is voted in: no count exceeds 256
    sh_v = 256u;
    sh_above = 0u;
  }
  __syncthreads();
  const uint32_t vthr = sh_v;
  const uint32_t take_eq = (uint32_t)kv - sh_above;

  // ascending compaction over contiguous word runs
  const int per = (words + kSetThreads - 1) / kSetThreads;
  const int wa = min(tid * per, words), wb = min(wa + per, words);
  uint32_t n_gt = 0, n_eq = 0;
  for (int w = wa; w < wb; ++w) {
    uint32_t cnt[32];
    word_votes(bb, words, Hq, w, cnt);
    const int nt = min(32, hist - w * 32);
    for (int i = 0; i < nt; ++i) {
      n_gt += cnt[i] > vthr;
      n_eq += cnt[i] == vthr;
    }
  }
  uint64_t total;
  const uint64_t before = block_excl_scan64(((uint64_t)n_gt << 32) | n_eq, scan_scratch, &total);
  uint32_t gt_before = (uint32_t)(before >> 32), eq_before = (uint32_t)before;
  int32_t* out = token_idx + (int64_t)b * N;
  uint8_t* vout = votes ? votes + (int64_t)b * T : nullptr;
  for (int w = wa; w < wb; ++w) {
    uint32_t cnt[32];
    word_votes(bb, words, Hq, w, cnt);
    const int nt = min(32, hist - w * 32);
    for (int i = 0; i < nt; ++i) {
      const int t = w * 32 + i;
      if (vout) vout[t] = (uint8_t)cnt[i];
      if (cnt[i] > vthr) {
        out[gt_before + min(eq_before, take_eq)] = t;
        ++gt_before;
      } else if (cnt[i] == vthr) {
        if (eq_before < take_eq) out[gt_before + eq_before] = t;
        ++eq_before;
      }
    }
  }
  for (int i = tid; i < W; i += kSetThreads) {
    out[kv + i] = hist + i;
    if (vout) vout[hist + i] = 0;
  }
}

// T <= N: the whole context, no vote.
__global__ void vote_all_kernel(int T, int32_t* __restrict__ token_idx, uint8_t* __restrict__ votes) {
  const int b = blockIdx.y;
  for (int t = blockIdx.x * blockDim.x + threadIdx.x; t < T; t += gridDim.x * blockDim.x) {
    token_idx[(int64_t)b * T + t] = t;
    if (votes) votes[(int64_t)b * T + t] = 0;
  }
}

template <typename T, int D, int G>
hipError_t launch_scores(const Dims& d, const void* q, const void* k, int hist, uint32_t* keys,
                         hipStream_t s) {
  const int ch = chunk_tokens(d);
  const int nchunks = (hist + ch - 1) / ch;
  const int per_wg = kScoreWaves * kScoreChunksPerWave;
  const dim3 grid((nchunks + per_wg - 1) / per_wg, d.B * d.Hkv);
  hipLaunchKernelGGL((vote_scores_kernel<T, D, G>), grid, dim3(kScoreWaves * 64), 0, s,
                     (const T*)q, (const T*)k, d, hist, keys);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_scores_g(const Dims& d, const void* q, const void* k, int hist, uint32_t* keys,
                           hipStream_t s) {
  switch (d.G) {
    case 1: return launch_scores<T, D, 1>(d, q, k, hist, keys, s);
    case 2: return launch_scores<T, D, 2>(d, q, k, hist, keys, s);
    case 4: return launch_scores<T, D, 4>(d, q, k, hist, keys, s);
    default: return launch_scores<T, D, 8>(d, q, k, hist, keys, s);
  }
}

}  // namespace

VotePlan plan_vote(const Dims& d, int N, int W) {
  VotePlan p;
  p.hist = d.T - W;
  p.words = (p.hist + 31) / 32;
  p.kv = N - W;
  const size_t rows = (size_t)d.B * d.Hq;
  p.keys_off = 0;
  const size_t keys_bytes = rows * (size_t)p.hist * sizeof(uint32_t);
  p.bits_off = (p.keys_off + keys_bytes + 255) & ~(size_t)255;
  p.total = p.bits_off + rows * (size_t)p.words * sizeof(uint32_t);
  if (d.T <= N) p.total = 0;
  return p;
}

hipError_t launch_vote_select(const Dims& d, const void* q, const void* k, int N, int W,
                              int32_t* token_idx, uint8_t* votes, void* workspace,
                              const VotePlan& plan, hipStream_t stream) {
  if (d.T <= N) {
    hipLaunchKernelGGL(vote_all_kernel, dim3((d.T + 255) / 256, d.B), dim3(256), 0, stream, d.T,
                       token_idx, votes);
    return hipGetLastError();
  }
  uint32_t* keys = (uint32_t*)((char*)workspace + plan.keys_off);
  uint32_t* bits = (uint32_t*)((char*)workspace + plan.bits_off);
  hipError_t e;
  if (d.dtype == KSA_BF16)
    e = d.D == 64 ? launch_scores_g<uint16_t, 64>(d, q, k, plan.hist, keys, stream)
                  : launch_scores_g<uint16_t, 128>(d, q, k, plan.hist, keys, stream);
  else
    e = d.D == 64 ? launch_scores_g<float, 64>(d, q, k, plan.hist, keys, stream)
                  : launch_scores_g<float, 128>(d, q, k, plan.hist, keys, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(vote_head_select_kernel, dim3(d.B * d.Hq), dim3(kHeadThreads), 0, stream,
                     keys, plan.hist, plan.kv, plan.words, bits);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(vote_set_kernel, dim3(d.B), dim3(kSetThreads), 0, stream, bits, d.Hq, d.T,
                     plan.hist, plan.words, plan.kv, N, W, token_idx, votes);
  return hipGetLastError();
}

}  // namespace ksa

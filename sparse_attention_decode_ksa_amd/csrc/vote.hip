// vote.hip -- the shared token set of the vote-union variant (LessIsMore
// explainer, section 二: equal votes per head, tokens ranked by vote total,
// 75 % of the budget voted / 25 % most recent; section 五: the selection
// layer scores every token for every head, aggregates and sorts the heads'
// picks and appends the most recent tokens).
//
// Per sequence b with history C = [0, T-W) and Kv = N - W picks per head:
//  1. vote_scores: every (b, KV head g) row streams its history keys once;
//     the G query heads of the group score every token in fp32 (MFMA for
//     bf16 D=128 groups of 4 and 8, VALU otherwise) and store
//     order-preserving uint32 keys [B, Hq, C (padded to 4)] in the
//     workspace.
//  2. vote_head_topk: one workgroup per (b, h), the head's keys held in
//     registers (in LDS or re-read for very long histories), finds the
//     Kv-th largest key and how many keys equal to it are taken (lowest
//     token ids first) by radix rounds on the keys' bits and a bucket
//     search, and writes the head's picks as a bitmask [B, Hq, ceil(C/32)].
//  3. vote_tally_set (histories up to 32768 tokens): one workgroup per b
//     adds the heads' bitmasks into bit-sliced vote totals (a carry-save
//     tree, eight heads at a time), finds the vote
//     threshold by a binary search on popcounts, and compacts the first Kv
//     tokens by (votes desc, t asc) in ascending order with one workgroup
//     scan; the W recent tokens follow.  Longer histories take two kernels:
//     vote_count (one lane per token sums its bit over the heads, stores the
//     total and fills a per-sequence histogram of totals) and vote_set (the
//     threshold from the histogram, then the same compaction).
// Everything after the fp32 scores is exact integer work.
#include <float.h>

#include <algorithm>
#include <type_traits>

#include "ksa_device.h"
#include "ksa_internal.h"
#include "ksa_topk.h"

namespace ksa {
namespace {

constexpr int kScoreWaves = 4;
constexpr int kScoreChunksPerWave = 8;  // VALU scoring
// MFMA scoring: chunks of 16 tokens per wave, and how many are in flight
#ifndef KSA_VOTE_CHUNKS
#define KSA_VOTE_CHUNKS 8
#endif
#ifndef KSA_VOTE_PREFETCH
#define KSA_VOTE_PREFETCH 2
#endif
constexpr int kVoteChunks = KSA_VOTE_CHUNKS;
constexpr int kVotePrefetch = KSA_VOTE_PREFETCH;
static_assert(kVoteChunks % kVotePrefetch == 0, "whole prefetch rounds per wave");
constexpr int kHeadThreads = 1024;  // selection with the keys in LDS or re-read
// selection with the keys in registers: threads per workgroup and the most
// history tokens per thread
#ifndef KSA_HEAD_NT
#define KSA_HEAD_NT 512
#endif
constexpr int kHeadNT = KSA_HEAD_NT;
constexpr int kHeadMaxKPT = 64;
constexpr int kHeadLdsKeys = 36864;  // keys a head-select workgroup keeps in LDS (144 KB)
constexpr int kCountThreads = 256;
constexpr int kSetThreads = 1024;
constexpr int kSetStage = 8192;  // picks per sequence the vote set stages in LDS
#ifndef KSA_SET_STEPS
#define KSA_SET_STEPS 2
#endif
constexpr int kSetSteps = KSA_SET_STEPS;  // steps of four tokens per thread per piece of the vote set

// A paged cache for the vote (table == nullptr: contiguous): each sequence
// has its own length T_b and history T_b - W (none when T_b <= N).
struct VotePaging {
  const int32_t* table;     // [B, tstride] pages of logical blocks
  const int32_t* seq_lens;  // [B]
  int tstride;
  int N, W;
};

// The history length of sequence b (0: no vote for it).
__device__ __forceinline__ int vote_hist(const VotePaging& pg, const Dims& d, int b, int hist) {
  if (!pg.seq_lens) return hist;
  const int Tb = seq_len_of(pg.seq_lens, b, d.T);
  return Tb > pg.N ? Tb - pg.W : 0;
}

// Element offset of token t's K row of (b, g): contiguous [B, Hkv, T_cap, D]
// or a pool [num_pages, Hkv, Bs, D] through the block table.
template <bool PAGED>
__device__ __forceinline__ int64_t vote_row(const VotePaging& pg, const Dims& d, int b, int g,
                                            int t) {
  if constexpr (PAGED) {
    const int j = t / d.Bs;
    return (((int64_t)pg.table[(int64_t)b * pg.tstride + j] * d.Hkv + g) * d.Bs + (t - j * d.Bs)) *
           d.D;
  } else {
    return ((int64_t)(b * d.Hkv + g) * d.Tcap + t) * d.D;
  }
}

// ------------------------------------------------------------------ 1 (VALU)
template <typename T, int D, int G, bool PAGED>
__global__ __launch_bounds__(kScoreWaves * 64) void vote_scores_kernel(
    const T* __restrict__ q, const T* __restrict__ k, Dims d, int hist, int kstride,
    uint32_t* __restrict__ keys, VotePaging pg) {
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
  const T* kb = k + li * EPL;
  hist = vote_hist(pg, d, b, hist);

  float qv[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h)
    KV<T>::widen(ld16(q + ((int64_t)b * d.Hq + g * G + h) * D + li * EPL), qv[h]);

  const int nchunks = (hist + CH - 1) / CH;
  const int c0 = (blockIdx.x * kScoreWaves + wave) * kScoreChunksPerWave;
  const int c1 = min(c0 + kScoreChunksPerWave, nchunks);
  // head written by this lane (lanes li < G of each slot write)
  uint32_t* kout = keys + ((int64_t)b * d.Hq + g * G + (li < G ? li : 0)) * kstride;
  if (c0 >= c1) return;

  uint4 kr[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i)
    kr[i] = ld16_stream(kb + vote_row<PAGED>(pg, d, b, g, min(c0 * CH + i * SPW + slot, hist - 1)));
  for (int c = c0; c < c1; ++c) {
    uint4 kc[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) kc[i] = kr[i];
    if (c + 1 < c1) {
#pragma unroll
      for (int i = 0; i < NI; ++i)
        kr[i] = ld16_stream(
            kb + vote_row<PAGED>(pg, d, b, g, min((c + 1) * CH + i * SPW + slot, hist - 1)));
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

// ------------------------------------------------------------------ 1 (MFMA)
// bf16, D = 128, G in {4, 8}: per chunk of 16 tokens, K rows are loaded with
// coalesced row-layout loads, re-read in the MFMA A layout from a
// wave-private swizzled LDS tile, and S = K Q^T runs on four
// v_mfma_f32_16x16x32_bf16; lane l then holds head l%16's logits of tokens
// 4*(l/16) .. +3 and puts their four keys into the workgroup's LDS key
// stage with one 16-byte store; the stage goes to the workspace at the end.
// Each wave owns kVoteChunks consecutive chunks and keeps kVotePrefetch of
// them in flight; loads past its range re-read its last token (in cache), so
// every load is unconditional.
template <int G, bool PAGED>
__global__ __launch_bounds__(kScoreWaves * 64) void vote_scores_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, Dims d, int hist, int kstride,
    uint32_t* __restrict__ keys, VotePaging pg) {
  constexpr int D = 128;
  constexpr int CH = 16;
  constexpr int P = kVotePrefetch;
  constexpr int Q = kVoteChunks;
  constexpr int kWgTok = kScoreWaves * Q * CH;  // tokens of one workgroup
  __shared__ uint4 s_k[kScoreWaves][CH * 16];
  __shared__ uint4 s_key[G][kWgTok / 4];  // the workgroup's keys, written out at the end
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, kg = lane >> 4;  // MFMA row / k-group; also row layout piece / slot
  const int row = blockIdx.y;
  const int b = row / d.Hkv, g = row - b * d.Hkv;
  const uint16_t* kb = k + 8 * r;
  hist = vote_hist(pg, d, b, hist);

  const int c0 = (blockIdx.x * kScoreWaves + wave) * Q;
  const bool any = c0 * CH < hist;  // this wave has tokens (every wave reaches the barrier)
  const int tend = min((c0 + Q) * CH, hist) - 1;  // last token of this wave's range
  bf16x8_t qop[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint4 u = make_uint4(0u, 0u, 0u, 0u);
    if (r < G) u = ld16(q + ((int64_t)b * d.Hq + g * G + r) * D + 32 * i + 8 * kg);
    qop[i] = as_bf16x8(u);
  }
  uint4* kt = s_k[wave];

  // row layout: load i, lane (slot kg, piece r) reads token 4i + kg of the chunk
  uint4 kr[P][4];
  auto load = [&](int c, uint4(&dst)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      dst[i] = ld16_stream(kb + vote_row<PAGED>(pg, d, b, g, min(c * CH + 4 * i + kg, tend)));
  };
  if (any) {
#pragma unroll
    for (int s = 0; s < P; ++s) load(c0 + s, kr[s]);
#pragma unroll 1
    for (int j0 = 0; j0 < Q; j0 += P) {
#pragma unroll
      for (int s = 0; s < P; ++s) {
        const int c = c0 + j0 + s;
#pragma unroll
        for (int i = 0; i < 4; ++i) kt[ktile_slot(4 * i + kg, r)] = kr[s][i];
        load(c + P, kr[s]);
        wave_lds_fence();
        f32x4_t S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i)
          S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kt[ktile_slot(r, 4 * i + kg)]), qop[i],
                                                      S, 0, 0, 0);
        wave_lds_fence();
        // head r's keys of tokens 4kg..4kg+3 of the chunk, staged in LDS
        if (r < G)
          s_key[r][(wave * Q + j0 + s) * (CH / 4) + kg] =
              make_uint4(order_key(S[0]), order_key(S[1]), order_key(S[2]), order_key(S[3]));
      }
    }
  }
  // The workgroup's keys go out head by head as 16-byte pieces of one
  // contiguous run per head (the last workgroup of a row stops at the
  // history; keys staged past it are dropped).  Written as a burst at the
  // end rather than one 16-lane store per chunk: 115.6 against 117.3 us for
  // the c4 shape (16 sequences, 8 KV heads, 19488 history tokens).
  __syncthreads();
  const int t0 = blockIdx.x * kWgTok;
  for (int u = threadIdx.x; u < G * (kWgTok / 4); u += kScoreWaves * 64) {
    const int h = u / (kWgTok / 4), o4 = u - h * (kWgTok / 4);
    const int t = t0 + 4 * o4;
    if (t >= hist) continue;
    uint32_t* ko = keys + ((int64_t)b * d.Hq + g * G + h) * kstride;
    const uint4 v = s_key[h][o4];
    if (t + 3 < hist) {
      st16(ko + t, v);  // kstride and t are multiples of 4
    } else {
      ko[t] = v.x;
      if (t + 1 < hist) ko[t + 1] = v.y;
      if (t + 2 < hist) ko[t + 2] = v.z;
    }
  }
}

// ------------------------------------------------------------------ 2
// Per (b, h), history of at most NT * KPT tokens: the head's keys sit in
// registers, token t = i * NT + tid in key[i] (coalesced loads).  A first
// histogram on the keys' 12 leading bits picks the bucket where the Kv
// largest end, a second on the next 12 bits of the keys in that bucket
// narrows it to one bin, the bucket search of ksa_topk.h resolves the last 8
// bits when needed, and each wave's ballot of "taken" is two words of the
// bitmask as it stands.  Ties at the threshold (equal fp32 logits) take the
// lowest token ids: the equal keys are ranked in token order by a
// per-(slot, wave) count.  The first
// workgroup of each sequence also clears that sequence's vote histogram,
// which vote_count fills after this kernel.
template <int NT, int KPT>
__global__ __launch_bounds__(NT) void vote_head_topk_kernel(
    const uint32_t* __restrict__ keys, int hist, int kstride, int kv, int words, int Hq,
    uint32_t* __restrict__ bits, uint32_t* __restrict__ vhist, HeadMask voting, Dims d,
    VotePaging pg) {
  constexpr int NWV = NT / 64;
  static_assert(4096 % NT == 0, "radix buckets per thread");
  __shared__ TopkShared sh;
  __shared__ uint32_t s_rh[4097];  // first-round histogram (4096: tokens past the history)
  __shared__ uint32_t s_rh2[4096];  // second round, inside the first round's cut bucket
  __shared__ uint32_t s_eq[KPT][NWV];  // equal keys per (slot, wave), then their prefix
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t hr = blockIdx.x;  // b * Hq + h
  if (hr % Hq == 0)
    for (int i = tid; i < 256; i += NT) vhist[(hr / Hq) * 256 + i] = 0u;
  uint32_t* br = bits + hr * words;
  const int h = (int)(hr % Hq);
  hist = vote_hist(pg, d, (int)(hr / Hq), hist);
  // no picks: the whole budget is the recency window, the sequence is too
  // short to vote, or the head does not vote
  if (kv == 0 || hist == 0 || !((voting.w[h >> 5] >> (h & 31)) & 1u)) {
    for (int w = tid; w < words; w += NT) br[w] = 0u;
    return;
  }
  const uint32_t* kr = keys + hr * kstride;
  auto valid = [&](int i) { return i * NT + tid < hist; };
  uint32_t key[KPT];
#pragma unroll
  for (int i = 0; i < KPT; ++i) key[i] = kr[min(i * NT + tid, hist - 1)];  // unconditional loads
#pragma unroll
  for (int i = 0; i < KPT; ++i) key[i] = valid(i) ? key[i] : 0u;
  for (int j = tid; j < 4097; j += NT) s_rh[j] = 0u;
  for (int j = tid; j < 4096; j += NT) s_rh2[j] = 0u;
  topk_clear(sh);
  __syncthreads();
  // First round on the keys' 12 leading bits (sign, exponent and three
  // mantissa bits of the score): fp32 scores spread over these buckets
  // without a pass for their range, and each key costs one shift.
#pragma unroll
  for (int i = 0; i < KPT; ++i) atomicAdd(&s_rh[valid(i) ? key[i] >> 20 : 4096u], 1u);
  __syncthreads();
  // The bin of a 4096-bin histogram (highest first) that holds the
  // need-th largest entry: sh.bucket = {bin, entries above it, entries in it}.
  auto find_bin = [&](const uint32_t* hb, uint32_t need) {
    // thread t owns bins 4095 - BPT*t down to 4096 - BPT*(t+1)
    constexpr int BPT = 4096 / NT;
    uint32_t c[BPT], sum = 0;
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      c[j] = hb[4095 - BPT * tid - j];
      sum += c[j];
    }
    const uint32_t excl = block_excl_scan32(sum, sh.scan);
    if (excl < need && need <= excl + sum) {
      uint32_t acc = excl;
#pragma unroll
      for (int j = 0; j < BPT; ++j) {
        if (acc + c[j] >= need) {
          sh.bucket[0] = (uint32_t)(4095 - BPT * tid - j);
          sh.bucket[1] = acc;
          sh.bucket[2] = c[j];
          break;
        }
        acc += c[j];
      }
    }
    __syncthreads();
  };
  find_bin(s_rh, (uint32_t)kv);
  const uint32_t b1 = sh.bucket[0], rem1 = (uint32_t)kv - sh.bucket[1];
  TopkCut cut{b1 << 20, 0xFFFFFFFFu};  // when the whole bucket is taken
  if (sh.bucket[2] != rem1) {  // uniform
    // Second round on the next 12 bits of the keys in that bucket (a few
    // hundred keys of fp32 logits, which these bins spread to about one
    // each), so that at most a short bucket search over the last 8 bits
    // remains.
#pragma unroll
    for (int i = 0; i < KPT; ++i)
      if (valid(i) && (key[i] >> 20) == b1) atomicAdd(&s_rh2[(key[i] >> 8) & 0xFFFu], 1u);
    __syncthreads();
    find_bin(s_rh2, rem1);
    const uint32_t lo = (b1 << 20) | (sh.bucket[0] << 8), rem2 = rem1 - sh.bucket[1];
    cut = sh.bucket[2] == rem2 ? TopkCut{lo, 0xFFFFFFFFu}
                               : topk_cut<KPT>(key, valid, (int)rem2, lo, lo | 0xFFu, sh);
  }
  const bool ties = cut.quota != 0xFFFFFFFFu;  // uniform
  const uint64_t below = (1ull << lane) - 1ull;
  if (ties) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const uint64_t m = __ballot(valid(i) && key[i] == cut.thr);
      if (lane == 0) s_eq[i][wave] = (uint32_t)__popcll(m);
    }
    __syncthreads();
    if (tid == 0) {  // exclusive prefix in token order (slot-major, then wave)
      uint32_t run = 0;
      for (int i = 0; i < KPT; ++i)
        for (int w = 0; w < NWV; ++w) {
          const uint32_t c = s_eq[i][w];
          s_eq[i][w] = run;
          run += c;
        }
    }
    __syncthreads();
  }
  // the ballot of slot i goes to lane i (two words), stored after the loop
  uint32_t mlo = 0u, mhi = 0u;
  auto keep = [&](int i, uint64_t bal) {
    mlo = lane == i ? (uint32_t)bal : mlo;
    mhi = lane == i ? (uint32_t)(bal >> 32) : mhi;
  };
  if (ties) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const bool eq = valid(i) && key[i] == cut.thr;
      const uint64_t m = __ballot(eq);
      const bool take = (valid(i) && key[i] > cut.thr) ||
                        (eq && s_eq[i][wave] + (uint32_t)__popcll(m & below) < cut.quota);
      keep(i, __ballot(take));
    }
  } else {
#pragma unroll
    for (int i = 0; i < KPT; ++i) keep(i, __ballot(valid(i) && key[i] >= cut.thr));
  }
  const int w0 = (lane * NT + wave * 64) >> 5;
  if (lane < KPT && w0 < words) br[w0] = mlo;
  if (lane < KPT && w0 + 1 < words) br[w0 + 1] = mhi;
}

// Per (b, h), any history length: the same selection with the keys in LDS
// (kLdsKeys) or re-read from the workspace each pass.
template <bool kLdsKeys>
__global__ __launch_bounds__(kHeadThreads) void vote_head_select_kernel(
    const uint32_t* __restrict__ keys, int hist, int kstride, int kv, int words, int Hq,
    uint32_t* __restrict__ bits, uint32_t* __restrict__ vhist, HeadMask voting, Dims d,
    VotePaging pg) {
  extern __shared__ uint32_t lkeys[];  // the head's keys (kLdsKeys)
  __shared__ uint32_t hbin[256];
  __shared__ uint32_t red[2][kHeadThreads / 64];
  __shared__ uint32_t shv[3];
  __shared__ uint64_t scan_scratch[17];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t hr = blockIdx.x;  // b * Hq + h
  if (hr % Hq == 0)
    for (int i = tid; i < 256; i += kHeadThreads) vhist[(hr / Hq) * 256 + i] = 0u;
  uint32_t* br = bits + hr * words;
  const int h = (int)(hr % Hq);
  hist = vote_hist(pg, d, (int)(hr / Hq), hist);
  // no picks: the whole budget is the recency window, the sequence is too
  // short to vote, or the head does not vote
  if (kv == 0 || hist == 0 || !((voting.w[h >> 5] >> (h & 31)) & 1u)) {
    for (int w = tid; w < words; w += kHeadThreads) br[w] = 0u;
    return;
  }
  const uint32_t* kr = keys + hr * kstride;

  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  for (int t = tid; t < hist; t += kHeadThreads) {
    const uint32_t key = kr[t];
    if (kLdsKeys) lkeys[t] = key;
    kmin = min(kmin, key);
    kmax = max(kmax, key);
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
  for (int w = 1; w < kHeadThreads / 64; ++w) {
    lo = min(lo, red[0][w]);
    hi = max(hi, red[1][w]);
  }

  uint32_t remaining = (uint32_t)kv;
  uint32_t quota, thr;
#pragma unroll 1
  for (;;) {
    const uint32_t span = hi - lo;
    if (span == 0) {
      thr = lo;
      quota = remaining;
      break;
    }
    const int nbits = 32 - __clz(span);
    const int shift = nbits > 8 ? nbits - 8 : 0;
    if (tid < 256) hbin[tid] = 0;
    __syncthreads();
    for (int t = tid; t < hist; t += kHeadThreads) {
      const uint32_t key = kLdsKeys ? lkeys[t] : kr[t];
      if (key >= lo && key <= hi) atomicAdd(&hbin[(key - lo) >> shift], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      const int top = 255 - 4 * lane;
      const uint32_t c0 = hbin[top], c1 = hbin[top - 1], c2 = hbin[top - 2], c3 = hbin[top - 3];
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
        shv[0] = (uint32_t)bk;
        shv[1] = c;
        shv[2] = n;
      }
    }
    __syncthreads();
    const uint32_t bk = shv[0], above = shv[1], n = shv[2];
    remaining -= above;
    const uint64_t blo = (uint64_t)lo + ((uint64_t)bk << shift);
    const uint64_t bhi = (uint64_t)lo + (((uint64_t)bk + 1) << shift) - 1;
    lo = (uint32_t)blo;
    hi = bhi < (uint64_t)hi ? (uint32_t)bhi : hi;
    if (n == remaining) {
      thr = lo;
      quota = 0xFFFFFFFFu;
      break;
    }
  }

  // membership bitmask in token order (lanes 0 and 32 of each wave store a word)
  uint32_t carry = 0;
  for (int t0 = 0; t0 < hist; t0 += kHeadThreads) {
    const int t = t0 + tid;
    const uint32_t key = t < hist ? (kLdsKeys ? lkeys[t] : kr[t]) : 0u;
    bool sel;
    if (quota == 0xFFFFFFFFu) {
      sel = t < hist && key >= thr;
    } else {
      const bool eq = t < hist && key == thr;
      uint64_t tot;
      const uint32_t before = carry + (uint32_t)block_excl_scan64(eq ? 1 : 0, scan_scratch, &tot);
      sel = t < hist && (key > thr || (eq && before < quota));
      carry += (uint32_t)tot;
    }
    const uint64_t bal = __ballot(sel);
    if (lane == 0 && (t >> 5) < words) br[t >> 5] = (uint32_t)bal;
    if (lane == 32 && (t >> 5) < words) br[t >> 5] = (uint32_t)(bal >> 32);
  }
}

// ------------------------------------------------------------------ 3
__global__ __launch_bounds__(kCountThreads) void vote_count_kernel(
    const uint32_t* __restrict__ bits, int Hq, int hist, int words, int T,
    uint8_t* __restrict__ votes8, uint8_t* __restrict__ votes, uint32_t* __restrict__ vhist,
    Dims d, VotePaging pg) {
  __shared__ uint32_t lh[256];
  const int tid = threadIdx.x;
  const int b = blockIdx.y;
  const int t = blockIdx.x * kCountThreads + tid;
  hist = vote_hist(pg, d, b, hist);  // this sequence's history (0: it does not vote)
  lh[tid] = 0u;  // kCountThreads == 256 bins
  __syncthreads();
  if (t < hist) {
    const uint32_t* bb = bits + (int64_t)b * Hq * words + (t >> 5);
    const int bit = t & 31;
    uint32_t cnt = 0;
#pragma unroll 8
    for (int h = 0; h < Hq; ++h) cnt += (bb[(int64_t)h * words] >> bit) & 1u;
    votes8[(int64_t)b * words * 32 + t] = (uint8_t)cnt;
    if (votes) votes[(int64_t)b * T + t] = (uint8_t)cnt;
    atomicAdd(&lh[cnt], 1u);
  }
  __syncthreads();
  if (lh[tid]) atomicAdd(&vhist[b * 256 + tid], lh[tid]);
}

// ------------------------------------------------------------------ 4
__global__ __launch_bounds__(kSetThreads) void vote_set_kernel(
    const uint8_t* __restrict__ votes8, const uint32_t* __restrict__ vhist, int T, int hist, int kv,
    int N, int W, int n_out, int32_t* __restrict__ token_idx, uint8_t* __restrict__ votes, Dims d,
    VotePaging pg) {
  __shared__ uint32_t sh_v, sh_above;
  __shared__ int32_t s_pick[kSetStage];
  __shared__ uint32_t s_cnt[2][kSetSteps * (kSetThreads / 64)];  // per (step, wave): above, on
  __shared__ uint32_t s_tot[2];
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  int32_t* out = token_idx + (int64_t)b * n_out;
  const int64_t vstride = (int64_t)((hist + 31) / 32) * 32;  // votes8 row stride (longest history)
  if (pg.seq_lens) {  // this sequence's own length (T is then the longest)
    const int Tb = seq_len_of(pg.seq_lens, b, d.T);
    if (Tb <= N) {  // no vote: the whole sequence, then -1
      for (int i = tid; i < n_out; i += kSetThreads) out[i] = i < Tb ? i : -1;
      if (votes)
        for (int t = tid; t < T; t += kSetThreads) votes[(int64_t)b * T + t] = 0;
      return;
    }
    hist = Tb - W;
    if (votes)
      for (int t = Tb + tid; t < T; t += kSetThreads) votes[(int64_t)b * T + t] = 0;
  }
  for (int i = tid; i < W; i += kSetThreads) {
    out[kv + i] = hist + i;
    if (votes) votes[(int64_t)b * T + hist + i] = 0;
  }
  if (kv == 0) return;  // uniform: the whole workgroup leaves
  // vote threshold v*: count(votes > v*) < kv <= count(votes >= v*)
  if (tid < 64) {
    const int top = 255 - 4 * tid;
    const uint32_t* vh = vhist + b * 256;
    const uint32_t c0 = vh[top], c1 = vh[top - 1], c2 = vh[top - 2], c3 = vh[top - 3];
    const uint32_t s = c0 + c1 + c2 + c3;
    const uint32_t incl = wave_incl_scan_dpp(s);
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
  __syncthreads();
  const uint32_t vthr = sh_v;
  const uint32_t take_eq = (uint32_t)kv - sh_above;

  // Ascending compaction, four tokens per thread per step: thread tid of
  // step i holds the vote bytes of tokens 4u .. 4u+3, u = base + i *
  // kSetThreads + tid (one 32-bit load).  Pass 1 counts, per (step, wave),
  // the tokens above the threshold and those on it (ballots per byte); one
  // wave turns the counts into exclusive prefixes in token order; pass 2
  // places every pick from its prefix and its rank inside the wave.
  // Histories longer than kSetSteps steps run in pieces with a carry.  The
  // picks are staged in LDS when they fit, so the output is written
  // coalesced.
  constexpr int NWV = kSetThreads / 64;
  const int lane = tid & 63, wave = tid >> 6;
  const uint64_t below = (1ull << lane) - 1ull;
  const uint32_t* vb = reinterpret_cast<const uint32_t*>(votes8 + (int64_t)b * vstride);
  const int nq = (hist + 3) / 4;  // vote words of four tokens
  const bool stage = kv <= kSetStage;  // uniform
  uint32_t carry_gt = 0, carry_eq = 0;
  for (int base = 0; base < nq; base += kSetSteps * kSetThreads) {
    uint32_t vv[kSetSteps];
#pragma unroll
    for (int i = 0; i < kSetSteps; ++i) vv[i] = vb[min(base + i * kSetThreads + tid, nq - 1)];
    // ballots of step i: g[k] / e[k] = lanes whose token 4u+k is above / on the threshold
    auto ballots = [&](int i, uint64_t(&g)[4], uint64_t(&e)[4]) {
      const int t0 = 4 * (base + i * kSetThreads + tid);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t v = (vv[i] >> (8 * k)) & 0xFFu;
        const bool in = t0 + k < hist;
        g[k] = __ballot(in && v > vthr);
        e[k] = __ballot(in && v == vthr);
      }
    };
#pragma unroll
    for (int i = 0; i < kSetSteps; ++i) {
      uint64_t g[4], e[4];
      ballots(i, g, e);
      if (lane == 0) {
        s_cnt[0][i * NWV + wave] = (uint32_t)(__popcll(g[0]) + __popcll(g[1]) + __popcll(g[2]) + __popcll(g[3]));
        s_cnt[1][i * NWV + wave] = (uint32_t)(__popcll(e[0]) + __popcll(e[1]) + __popcll(e[2]) + __popcll(e[3]));
      }
    }
    __syncthreads();
    if (wave == 0) {  // lane l: the entries of step l, in wave order
      uint32_t sg = 0, se = 0;
      if (lane < kSetSteps) {
#pragma unroll
        for (int j = 0; j < NWV; ++j) {
          const uint32_t gc = s_cnt[0][lane * NWV + j], ec = s_cnt[1][lane * NWV + j];
          s_cnt[0][lane * NWV + j] = sg;
          s_cnt[1][lane * NWV + j] = se;
          sg += gc;
          se += ec;
        }
      }
      const uint32_t ig = wave_incl_scan_dpp(sg), ie = wave_incl_scan_dpp(se);
      if (lane < kSetSteps) {
#pragma unroll
        for (int j = 0; j < NWV; ++j) {
          s_cnt[0][lane * NWV + j] += ig - sg + carry_gt;
          s_cnt[1][lane * NWV + j] += ie - se + carry_eq;
        }
      }
      if (lane == 63) {
        s_tot[0] = ig;
        s_tot[1] = ie;
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kSetSteps; ++i) {
      uint64_t g[4], e[4];
      ballots(i, g, e);
      uint32_t rg = s_cnt[0][i * NWV + wave], re = s_cnt[1][i * NWV + wave];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        rg += (uint32_t)__popcll(g[k] & below);
        re += (uint32_t)__popcll(e[k] & below);
      }
      const int t0 = 4 * (base + i * kSetThreads + tid);
#pragma unroll
      for (int k = 0; k < 4; ++k) {  // the thread's own tokens, in order
        const bool gt = (g[k] >> lane) & 1ull, eq = (e[k] >> lane) & 1ull;
        int pos = -1;
        if (gt) pos = (int)(rg + min(re, take_eq));
        if (eq && re < take_eq) pos = (int)(rg + re);
        if (pos >= 0) {
          if (stage)
            s_pick[pos] = t0 + k;
          else
            out[pos] = t0 + k;
        }
        rg += gt;
        re += eq;
      }
    }
    carry_gt += s_tot[0];
    carry_eq += s_tot[1];
    __syncthreads();  // s_cnt and s_tot are rewritten by the next piece
  }
  if (stage) {
    for (int i = tid; i < kv; i += kSetThreads) out[i] = s_pick[i];
  }
}

// ------------------------------------------------------------------ 3+4 in one
// Histories of at most kSetThreads * 32 tokens: one workgroup per sequence
// tallies the votes and builds the set.  Thread w owns the 32 tokens of
// bitmask word w: it adds the Hq heads' words into NP bit planes (a
// bit-sliced counter, so plane k holds bit k of every token's vote total).
// The vote threshold v* (the largest v with at least Kv tokens voted >= v)
// comes from a binary search whose counts are popcounts of bit-sliced
// comparisons; the picks are the tokens above v* and the first ones on it,
// placed in token order by one workgroup scan and staged in LDS.
// Full adder on 32 lanes of bits: a + b + ci = s + 2 co.
__device__ __forceinline__ void full_add(uint32_t a, uint32_t b, uint32_t ci, uint32_t& s,
                                         uint32_t& co) {
  const uint32_t u = a ^ b;
  s = u ^ ci;
  co = (a & b) | (u & ci);
}

// Adds eight bit vectors x[0..7] (bit j: token j of the word picked by that
// head) into the bit-sliced counter c (plane k: bit k of each token's
// total).  A carry-save tree first reduces the eight to a 4-bit count per
// token (planes n0..n3), which a ripple adder then adds into c: about 53
// bit operations, where adding the eight one at a time costs 3 * NP each.
template <int NP>
__device__ __forceinline__ void add8_bitsliced(uint32_t (&c)[NP], const uint32_t* x) {
  static_assert(NP >= 4, "a count of eight needs four planes");
  uint32_t s, t0, t1, t2;
  full_add(x[0], x[1], x[2], s, t0);
  full_add(s, x[3], x[4], s, t1);
  full_add(s, x[5], x[6], s, t2);
  const uint32_t n0 = s ^ x[7], t3 = s & x[7];  // weight 1; t0..t3 weight 2
  uint32_t u, f0;
  full_add(t0, t1, t2, u, f0);
  const uint32_t n1 = u ^ t3, f1 = u & t3;      // weight 2; f0, f1 weight 4
  const uint32_t n2 = f0 ^ f1, n3 = f0 & f1;    // weights 4 and 8
  uint32_t cy = c[0] & n0;
  c[0] ^= n0;
  full_add(c[1], n1, cy, c[1], cy);
  full_add(c[2], n2, cy, c[2], cy);
  full_add(c[3], n3, cy, c[3], cy);
#pragma unroll
  for (int k = 4; k < NP; ++k) {
    const uint32_t t = c[k] & cy;
    c[k] ^= cy;
    cy = t;
  }
}

template <int NP>
__device__ __forceinline__ uint32_t votes_at_least(const uint32_t (&c)[NP], int v) {
  // tokens of the word whose vote total is >= v (0 <= v < 2^NP), MSB first
  uint32_t gt = 0u, eq = 0xFFFFFFFFu;
#pragma unroll
  for (int k = NP - 1; k >= 0; --k) {
    if ((v >> k) & 1) {
      eq &= c[k];
    } else {
      gt |= eq & c[k];
      eq &= ~c[k];
    }
  }
  return gt | eq;
}

template <int NP>
__global__ __launch_bounds__(kSetThreads) void vote_tally_set_kernel(
    const uint32_t* __restrict__ bits, int Hq, int T, int hist, int words, int kv, int N, int W,
    int n_out, int32_t* __restrict__ token_idx, uint8_t* __restrict__ votes, Dims d,
    VotePaging pg) {
  constexpr int NWV = kSetThreads / 64;
  __shared__ uint32_t s_red[2][NWV];
  __shared__ uint32_t s_scan[16];
  __shared__ int32_t s_pick[kSetStage];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.x;
  int32_t* out = token_idx + (int64_t)b * n_out;
  if (pg.seq_lens) {  // this sequence's own length (T is then the longest)
    const int Tb = seq_len_of(pg.seq_lens, b, d.T);
    if (Tb <= N) {  // no vote: the whole sequence, then -1
      for (int i = tid; i < n_out; i += kSetThreads) out[i] = i < Tb ? i : -1;
      if (votes)
        for (int t = tid; t < T; t += kSetThreads) votes[(int64_t)b * T + t] = 0;
      return;
    }
    hist = Tb - W;
    if (votes)
      for (int t = Tb + tid; t < T; t += kSetThreads) votes[(int64_t)b * T + t] = 0;
  }
  for (int i = tid; i < W; i += kSetThreads) {
    out[kv + i] = hist + i;
    if (votes) votes[(int64_t)b * T + hist + i] = 0;
  }

  // bit-sliced vote totals of the thread's word
  const int w = tid;
  const int words_b = (hist + 31) / 32;
  const uint32_t valid = w >= words_b ? 0u
                         : (w == words_b - 1 && (hist & 31)) ? (1u << (hist & 31)) - 1u
                                                              : 0xFFFFFFFFu;
  uint32_t c[NP];
#pragma unroll
  for (int k = 0; k < NP; ++k) c[k] = 0u;
  const uint32_t* bw = bits + (int64_t)b * Hq * words + min(w, words - 1);
  // the heads' words in batches of 32 loads in flight (one round trip for
  // up to 32 heads), added 8 at a time by a carry-save tree; waves whose
  // words all lie past the history skip it (their totals stay zero)
  if (__builtin_amdgcn_readfirstlane(tid & ~63) < words_b) {
    for (int h0 = 0; h0 < Hq; h0 += 32) {
      uint32_t x[32];
#pragma unroll
      for (int j = 0; j < 32; ++j) x[j] = bw[(int64_t)min(h0 + j, Hq - 1) * words];
      if (h0 + 32 > Hq) {  // uniform: heads past Hq add nothing
#pragma unroll
        for (int j = 0; j < 32; ++j) x[j] = h0 + j < Hq ? x[j] : 0u;
      }
#pragma unroll
      for (int j = 0; j < 32; j += 8) add8_bitsliced<NP>(c, x + j);
    }
#pragma unroll
    for (int k = 0; k < NP; ++k) c[k] &= valid;
  }
  if (votes && w < words) {
    for (int j = 0; j < 32 && w * 32 + j < hist; ++j) {
      uint32_t v = 0;
#pragma unroll
      for (int k = 0; k < NP; ++k) v |= ((c[k] >> j) & 1u) << k;
      votes[(int64_t)b * T + w * 32 + j] = (uint8_t)v;
    }
  }
  if (kv == 0) return;  // uniform: the whole workgroup leaves

  // v*: count(votes >= lo) >= Kv > count(votes >= hi), hi - lo shrinking to
  // 1 (a binary search: a handful of popcount rounds, where a histogram of
  // every total would cost a wave reduction per total)
  auto count_at_least = [&](int v, int parity) {
    uint32_t n = (uint32_t)__popc(votes_at_least<NP>(c, v) & valid);
    n = wave_incl_scan_dpp(n);
    if (lane == 63) s_red[parity][wave] = n;
    __syncthreads();
    uint32_t tot = 0;
#pragma unroll
    for (int i = 0; i < NWV; ++i) tot += s_red[parity][i];
    return tot;
  };
  int lo = 0, hi = Hq + 1, parity = 0;
  uint32_t above = 0;  // count(votes >= hi)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    const uint32_t n = count_at_least(mid, parity);
    parity ^= 1;
    if (n >= (uint32_t)kv) {
      lo = mid;
    } else {
      hi = mid;
      above = n;
    }
  }
  const uint32_t take_eq = (uint32_t)kv - above;
  const uint32_t ge = votes_at_least<NP>(c, lo) & valid;
  const uint32_t gtm = hi <= Hq ? votes_at_least<NP>(c, hi) & valid : 0u;
  const uint32_t eqm = ge & ~gtm;

  // ascending compaction over the words, one scan
  const uint32_t n_gt = (uint32_t)__popc(gtm), n_eq = (uint32_t)__popc(eqm);
  const uint32_t before = block_excl_scan32((n_gt << 16) | n_eq, s_scan);
  uint32_t gt_before = before >> 16, eq_before = before & 0xFFFFu;
  const bool stage = kv <= kSetStage;  // uniform
  uint32_t m = gtm | eqm;
  while (m) {
    const int j = __ffs(m) - 1;
    m &= m - 1u;
    const int t = w * 32 + j;
    int pos = -1;
    if ((gtm >> j) & 1u) {
      pos = (int)(gt_before + min(eq_before, take_eq));
      ++gt_before;
    } else {
      if (eq_before < take_eq) pos = (int)(gt_before + eq_before);
      ++eq_before;
    }
    if (pos >= 0) {
      if (stage)
        s_pick[pos] = t;
      else
        out[pos] = t;
    }
  }
  if (stage) {
    __syncthreads();
    for (int i = tid; i < kv; i += kSetThreads) out[i] = s_pick[i];
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

#ifndef KSA_MFMA
#define KSA_MFMA 1
#endif

template <typename T, int D, int G>
hipError_t launch_scores(const Dims& d, const void* q, const void* k, int hist, int kstride,
                         uint32_t* keys, hipStream_t s, const VotePaging& pg) {
  constexpr bool mfma = KSA_MFMA && std::is_same<T, uint16_t>::value && D == 128 && G >= 4;
  const bool paged = pg.table != nullptr;
  if constexpr (mfma) {
    const int nchunks = (hist + 15) / 16;
    const int per_wg = kScoreWaves * kVoteChunks;
    const dim3 grid((nchunks + per_wg - 1) / per_wg, d.B * d.Hkv);
    if (paged)
      hipLaunchKernelGGL((vote_scores_mfma_kernel<G, true>), grid, dim3(kScoreWaves * 64), 0, s,
                         (const uint16_t*)q, (const uint16_t*)k, d, hist, kstride, keys, pg);
    else
      hipLaunchKernelGGL((vote_scores_mfma_kernel<G, false>), grid, dim3(kScoreWaves * 64), 0, s,
                         (const uint16_t*)q, (const uint16_t*)k, d, hist, kstride, keys, pg);
  } else {
    const int nchunks = (hist + chunk_tokens(d) - 1) / chunk_tokens(d);
    const int per_wg = kScoreWaves * kScoreChunksPerWave;
    const dim3 grid((nchunks + per_wg - 1) / per_wg, d.B * d.Hkv);
    if (paged)
      hipLaunchKernelGGL((vote_scores_kernel<T, D, G, true>), grid, dim3(kScoreWaves * 64), 0, s,
                         (const T*)q, (const T*)k, d, hist, kstride, keys, pg);
    else
      hipLaunchKernelGGL((vote_scores_kernel<T, D, G, false>), grid, dim3(kScoreWaves * 64), 0, s,
                         (const T*)q, (const T*)k, d, hist, kstride, keys, pg);
  }
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_scores_g(const Dims& d, const void* q, const void* k, int hist, int kstride,
                           uint32_t* keys, hipStream_t s, const VotePaging& pg) {
  switch (d.G) {
    case 1: return launch_scores<T, D, 1>(d, q, k, hist, kstride, keys, s, pg);
    case 2: return launch_scores<T, D, 2>(d, q, k, hist, kstride, keys, s, pg);
    case 4: return launch_scores<T, D, 4>(d, q, k, hist, kstride, keys, s, pg);
    default: return launch_scores<T, D, 8>(d, q, k, hist, kstride, keys, s, pg);
  }
}

hipError_t launch_scores_any(const Dims& d, const void* q, const void* k, int hist, int kstride,
                             uint32_t* keys, hipStream_t s, const VotePaging& pg) {
  if (d.dtype == KSA_BF16)
    return d.D == 64 ? launch_scores_g<uint16_t, 64>(d, q, k, hist, kstride, keys, s, pg)
                     : launch_scores_g<uint16_t, 128>(d, q, k, hist, kstride, keys, s, pg);
  return d.D == 64 ? launch_scores_g<float, 64>(d, q, k, hist, kstride, keys, s, pg)
                   : launch_scores_g<float, 128>(d, q, k, hist, kstride, keys, s, pg);
}

hipError_t launch_head_select(const Dims& d, const VotePlan& p, const uint32_t* keys, uint32_t* bits,
                              uint32_t* vhist, const HeadMask& voting, hipStream_t stream,
                              const VotePaging& pg) {
  const dim3 grid(d.B * d.Hq), block(kHeadThreads);
  const int kpt = (p.hist + kHeadNT - 1) / kHeadNT;
#define KSA_HEAD_TOPK(K)                                                                      \
  hipLaunchKernelGGL((vote_head_topk_kernel<kHeadNT, K>), grid, dim3(kHeadNT), 0, stream, keys, \
                     p.hist, p.kstride, p.kv, p.words, d.Hq, bits, vhist, voting, d, pg)
  if (kpt <= 8) {
    KSA_HEAD_TOPK(8);
  } else if (kpt <= 16) {
    KSA_HEAD_TOPK(16);
  } else if (kpt <= 24) {
    KSA_HEAD_TOPK(24);
  } else if (kpt <= 32) {
    KSA_HEAD_TOPK(32);
  } else if (kpt <= 40) {
    KSA_HEAD_TOPK(40);
  } else if (kpt <= 48) {
    KSA_HEAD_TOPK(48);
  } else if (kpt <= kHeadMaxKPT) {
    KSA_HEAD_TOPK(kHeadMaxKPT);
  } else if (p.hist <= kHeadLdsKeys) {
#undef KSA_HEAD_TOPK
    const size_t lds = (size_t)p.hist * sizeof(uint32_t);
    if (lds > 65536) {
      const hipError_t e = hipFuncSetAttribute((const void*)vote_head_select_kernel<true>,
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(vote_head_select_kernel<true>, grid, block, lds, stream, keys, p.hist,
                       p.kstride, p.kv, p.words, d.Hq, bits, vhist, voting, d, pg);
  } else {
    hipLaunchKernelGGL(vote_head_select_kernel<false>, grid, block, 0, stream, keys, p.hist,
                       p.kstride, p.kv, p.words, d.Hq, bits, vhist, voting, d, pg);
  }
  return hipGetLastError();
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

VotePlan plan_vote(const Dims& d, int N, int W) {
  VotePlan p;
  p.hist = d.T - W;
  p.words = (p.hist + 31) / 32;
  p.kstride = (p.hist + 3) & ~3;  // key rows start 16-byte aligned
  p.kv = N - W;
  const size_t rows = (size_t)d.B * d.Hq;
  p.keys_off = 0;
  p.bits_off = align256(rows * (size_t)p.kstride * sizeof(uint32_t));
  p.votes_off = align256(p.bits_off + rows * (size_t)p.words * sizeof(uint32_t));
  p.vhist_off = align256(p.votes_off + (size_t)d.B * p.words * 32);
  p.total = p.vhist_off + (size_t)d.B * 256 * sizeof(uint32_t);
  if (d.T <= N) p.total = 0;
  return p;
}

namespace {
// Per (b, h), the per-head-sets ablation: the head's own picks (its bitmask,
// exactly Kv bits) in ascending order, then the W most recent tokens.
// Thread t owns words [t*R, (t+1)*R) of the bitmask; one workgroup scan.
constexpr int kHeadSetThreads = 256;
// With paging (pg.seq_lens) each sequence has its own history, and a
// sequence no longer than N takes all its tokens, then -1.
__global__ __launch_bounds__(kHeadSetThreads) void head_set_kernel(
    const uint32_t* __restrict__ bits, int words, int hist, int kv, int W, int n_out,
    int32_t* __restrict__ token_idx, Dims d, VotePaging pg) {
  __shared__ uint32_t s_scan[16];
  const int tid = threadIdx.x;
  const int64_t hr = blockIdx.x;
  const uint32_t* br = bits + hr * words;
  int32_t* out = token_idx + hr * n_out;
  if (pg.seq_lens) {
    const int Tb = seq_len_of(pg.seq_lens, (int)(hr / d.Hq), d.T);
    if (Tb <= pg.N) {
      for (int i = tid; i < n_out; i += kHeadSetThreads) out[i] = i < Tb ? i : -1;
      return;
    }
    hist = Tb - W;
  }
  for (int i = tid; i < W; i += kHeadSetThreads) out[kv + i] = hist + i;
  const int R = (words + kHeadSetThreads - 1) / kHeadSetThreads;
  uint32_t n = 0;
  for (int r = 0; r < R; ++r) {
    const int w = tid * R + r;
    if (w < words) n += (uint32_t)__popc(br[w]);
  }
  uint32_t pos = block_excl_scan32(n, s_scan);
  for (int r = 0; r < R; ++r) {
    const int w = tid * R + r;
    if (w >= words) break;
    uint32_t m = br[w];
    while (m) {
      const int j = __ffs(m) - 1;
      m &= m - 1u;
      if (pos < (uint32_t)kv) out[pos] = w * 32 + j;
      ++pos;
    }
  }
}

// T <= N: every head attends the whole context.
// Every row keeps all its tokens (T <= N): row r of T entries; with paging
// row (b, h) holds its sequence's T_b tokens, then -1.
__global__ void head_all_kernel(int T, int rows, int32_t* __restrict__ token_idx, Dims d,
                                VotePaging pg) {
  const int64_t n = (int64_t)rows * T;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int col = (int)(i % T);
    int lim = T;
    if (pg.seq_lens) lim = seq_len_of(pg.seq_lens, (int)((i / T) / d.Hq), d.T);
    token_idx[i] = col < lim ? col : -1;
  }
}
}  // namespace

hipError_t launch_vote_per_head(const Dims& d, const void* q, const void* k, int N, int W,
                                int32_t* token_idx, void* workspace, const VotePlan& plan,
                                hipStream_t stream, const PagedKv* paged) {
  const int rows = d.B * d.Hq;
  const VotePaging pg = paged ? VotePaging{paged->table, paged->seq_lens, paged->max_blocks, N, W}
                              : VotePaging{nullptr, nullptr, 0, N, W};
  if (d.T <= N) {
    hipLaunchKernelGGL(head_all_kernel, dim3(std::min<int64_t>(4096, ((int64_t)rows * d.T + 255) / 256)),
                       dim3(256), 0, stream, d.T, rows, token_idx, d, pg);
    return hipGetLastError();
  }
  char* ws = (char*)workspace;
  uint32_t* keys = (uint32_t*)(ws + plan.keys_off);
  uint32_t* bits = (uint32_t*)(ws + plan.bits_off);
  uint32_t* vhist = (uint32_t*)(ws + plan.vhist_off);
  hipError_t e = launch_scores_any(d, q, k, plan.hist, plan.kstride, keys, stream, pg);
  if (e != hipSuccess) return e;
  e = launch_head_select(d, plan, keys, bits, vhist, HeadMask(), stream, pg);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(head_set_kernel, dim3(rows), dim3(kHeadSetThreads), 0, stream, bits,
                     plan.words, plan.hist, plan.kv, W, N, token_idx, d, pg);
  return hipGetLastError();
}

namespace {
hipError_t vote_finish(const Dims& d, int N, int W, int n_out, int32_t* token_idx, uint8_t* votes,
                       void* workspace, const VotePlan& plan, hipStream_t stream,
                       const HeadMask& voting, const VotePaging& pg, bool scored) {
  char* ws = (char*)workspace;
  uint32_t* keys = (uint32_t*)(ws + plan.keys_off);
  uint32_t* bits = (uint32_t*)(ws + plan.bits_off);
  uint8_t* votes8 = (uint8_t*)(ws + plan.votes_off);
  uint32_t* vhist = (uint32_t*)(ws + plan.vhist_off);
  hipError_t e;
  if (scored) {
    e = launch_head_select(d, plan, keys, bits, vhist, voting, stream, pg);
    if (e != hipSuccess) return e;
  }
  if (plan.words <= kSetThreads) {
    if (d.Hq < 64)
      hipLaunchKernelGGL(vote_tally_set_kernel<6>, dim3(d.B), dim3(kSetThreads), 0, stream, bits,
                         d.Hq, d.T, plan.hist, plan.words, plan.kv, N, W, n_out, token_idx, votes,
                         d, pg);
    else
      hipLaunchKernelGGL(vote_tally_set_kernel<8>, dim3(d.B), dim3(kSetThreads), 0, stream, bits,
                         d.Hq, d.T, plan.hist, plan.words, plan.kv, N, W, n_out, token_idx, votes,
                         d, pg);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(vote_count_kernel, dim3((plan.hist + kCountThreads - 1) / kCountThreads, d.B),
                     dim3(kCountThreads), 0, stream, bits, d.Hq, plan.hist, plan.words, d.T, votes8,
                     votes, vhist, d, pg);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(vote_set_kernel, dim3(d.B), dim3(kSetThreads), 0, stream, votes8, vhist, d.T,
                     plan.hist, plan.kv, N, W, n_out, token_idx, votes, d, pg);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_vote_finish(const Dims& d, int N, int W, int32_t* token_idx, uint8_t* votes,
                              void* workspace, const VotePlan& plan, hipStream_t stream,
                              const HeadMask& voting) {
  const VotePaging none{nullptr, nullptr, 0, N, W};
  return vote_finish(d, N, W, N, token_idx, votes, workspace, plan, stream, voting, none, true);
}

hipError_t launch_vote_all(const Dims& d, int32_t* token_idx, uint8_t* votes, hipStream_t stream) {
  hipLaunchKernelGGL(vote_all_kernel, dim3((d.T + 255) / 256, d.B), dim3(256), 0, stream, d.T,
                     token_idx, votes);
  return hipGetLastError();
}

hipError_t launch_vote_select(const Dims& d, const void* q, const void* k, int N, int W,
                              int32_t* token_idx, uint8_t* votes, void* workspace,
                              const VotePlan& plan, hipStream_t stream, const HeadMask& voting) {
  if (d.T <= N) return launch_vote_all(d, token_idx, votes, stream);
  uint32_t* keys = (uint32_t*)((char*)workspace + plan.keys_off);
  const VotePaging none{nullptr, nullptr, 0, N, W};
  hipError_t e = launch_scores_any(d, q, k, plan.hist, plan.kstride, keys, stream, none);
  if (e != hipSuccess) return e;
  return vote_finish(d, N, W, N, token_idx, votes, workspace, plan, stream, voting, none, true);
}

hipError_t launch_paged_vote_finish(const Dims& d, const PagedKv& p, int N, int W,
                                    int32_t* token_idx, uint8_t* votes, void* workspace,
                                    const VotePlan& plan, hipStream_t stream) {
  const VotePaging pg{p.table, p.seq_lens, p.max_blocks, N, W};
  const int n_out = d.T < N ? d.T : N;
  return vote_finish(d, N, W, n_out, token_idx, votes, workspace, plan, stream, HeadMask(), pg,
                     d.T > N);
}

hipError_t launch_paged_vote_select(const Dims& d, const PagedKv& p, const void* q,
                                    const void* k_pool, int N, int W, int32_t* token_idx,
                                    uint8_t* votes, void* workspace, const VotePlan& plan,
                                    hipStream_t stream, const HeadMask& voting) {
  const VotePaging pg{p.table, p.seq_lens, p.max_blocks, N, W};
  const int n_out = d.T < N ? d.T : N;
  const bool any_vote = d.T > N;  // d.T is the longest sequence
  if (any_vote) {
    uint32_t* keys = (uint32_t*)((char*)workspace + plan.keys_off);
    hipError_t e = launch_scores_any(d, q, k_pool, plan.hist, plan.kstride, keys, stream, pg);
    if (e != hipSuccess) return e;
  }
  return vote_finish(d, N, W, n_out, token_idx, votes, workspace, plan, stream, voting, pg,
                     any_vote);
}

}  // namespace ksa

// attention.hip -- the decode attention kernels and their launch plans.
// The per-row bodies (numerics, lane layout, pipelining) are in
// ksa_attention.h; this file holds the kernels that give each workgroup one
// (row, split) pair, the fixed-order split merge, and plan_attention.
#include <atomic>
#include <chrono>
#include <type_traits>

#include "ksa_attention.h"

namespace ksa {
namespace {

// For G <= 2 the register budget is held at 128 per lane, so that two
// 512-thread workgroups (16 waves) fit on a CU.
template <typename T, int D, int G, int KIND>
__global__ __launch_bounds__(kMaxWaves * 64, (G <= 2 ? 4 : 1)) void attn_partial_kernel(AttnArgs a) {
  constexpr int CH = (64 / (D / KV<T>::EPL)) * kLoadsPerChunk;
  __shared__ int s_idx[kIdxStage];
  const int split = blockIdx.x % a.splits;
  const int row = blockIdx.x / a.splits;
  const int e0 = stage_indices<KIND, CH>(a, row, split, s_idx);
  attn_row_valu<T, D, G, KIND>(a, row, split, s_idx, nullptr, e0, KIND != 2);
}

template <int G, int KIND, bool VK = false>
__global__ __launch_bounds__(kMaxWaves * 64) void attn_mfma_kernel(AttnArgs a) {
  __shared__ int s_idx[kIdxStage];
  const int split = blockIdx.x % a.splits;
  const int row = blockIdx.x / a.splits;
  const int e0 = stage_indices<KIND, 16>(a, row, split, s_idx);
  attn_row_mfma<G, KIND, VK>(a, row, split, s_idx, nullptr, e0, KIND != 2);
}

#ifndef KSA_MFMA
#define KSA_MFMA 1
#endif

// Dense attention over a paged cache: the row's length comes from seq_lens,
// and the logical ids and pages of the blocks in this split's range are
// staged in LDS (splits past a short row's end write an empty partial
// state, which the merge weighs by zero).
template <typename T, int D, int G, bool VK = false>
__global__ __launch_bounds__(kMaxWaves * 64, (G <= 2 ? 4 : 1)) void attn_paged_dense_kernel(
    AttnArgs a0) {
  constexpr bool kMfma = KSA_MFMA && std::is_same<T, uint16_t>::value && D == 128 && G >= 4;
  constexpr int CH = kMfma ? 16 : (64 / (D / KV<T>::EPL)) * kLoadsPerChunk;
  __shared__ int s_idx[kIdxStage];
  __shared__ int s_pg[kIdxStage];
  const int split = blockIdx.x % a0.splits;
  const int row = blockIdx.x / a0.splits;
  const int b = row / a0.d.Hkv;
  const int Bs = a0.d.Bs;
  AttnArgs a = a0;
  const int Tb = seq_len_of(a0.seq_lens, b, a0.d.T);
  const int nb = (Tb + Bs - 1) / Bs;
  a.d.T = Tb;
  a.ltot = nb * Bs;
  a.count = nb;
  if constexpr (VK) a.vhist = Tb > a.vbudget ? Tb - a.vwindow : 0;  // this sequence's vote history
  const int nchunks = (a.ltot + CH - 1) / CH;
  const int c_begin = split * a.cps;
  const int c_end = min(c_begin + a.cps, nchunks);
  const int e0 = (c_begin * CH) / Bs;
  const int e1 = min(nb, (c_end * CH + Bs - 1) / Bs);
  const int32_t* tb = a.table + (int64_t)b * a.tstride;
  for (int i = threadIdx.x; i < e1 - e0; i += blockDim.x) s_idx[i] = e0 + i;
  stage_copy(tb + e0, e1 - e0, s_pg);
  if constexpr (kMfma)
    attn_row_mfma<G, 3, VK>(a, row, split, s_idx, s_pg, e0, true);
  else
    attn_row_valu<T, D, G, 3>(a, row, split, s_idx, s_pg, e0, true);
}

// Attention over a given list on a paged cache: kind 3 = block ids
// [B, Hkv, count] (logical, -1 = padding), kind 5 = token ids [B, count]
// shared by the sequence's heads (-1 = padding), kind 6 = token ids
// [B, Hq, count], one list per query head (rows are query heads, G = 1).  The row's length comes from
// seq_lens; the ids of this split's range and their pages (kind 3) or pool
// rows (kind 5) are staged in LDS.
template <typename T, int D, int G, int KIND>
__global__ __launch_bounds__(kMaxWaves * 64, (G <= 2 ? 4 : 1)) void attn_paged_list_kernel(
    AttnArgs a0) {
  constexpr bool kMfma = KSA_MFMA && std::is_same<T, uint16_t>::value && D == 128 && G >= 4;
  constexpr int CH = kMfma ? 16 : (64 / (D / KV<T>::EPL)) * kLoadsPerChunk;
  __shared__ int s_idx[kIdxStage];
  __shared__ int s_pg[kIdxStage];
  const int split = blockIdx.x % a0.splits;
  const int row = blockIdx.x / a0.splits;
  const int b = row / a0.d.Hkv;
  const int Bs = a0.d.Bs;
  AttnArgs a = a0;
  const int Tb = seq_len_of(a0.seq_lens, b, a0.d.T);
  a.d.T = Tb;
  const int nchunks = (a.ltot + CH - 1) / CH;
  const int c_begin = split * a.cps;
  const int c_end = min(c_begin + a.cps, nchunks);
  const int32_t* tb = a.table + (int64_t)b * a.tstride;
  int e0, e1;
  const int32_t* src;
  if constexpr (KIND == 3) {
    e0 = (c_begin * CH) / Bs;
    e1 = min(a.count, (c_end * CH + Bs - 1) / Bs);
    src = a.idx + (int64_t)row * a.count;
  } else {
    e0 = c_begin * CH;
    e1 = min(a.ltot, c_end * CH);
    src = a.idx + (int64_t)(KIND == 6 ? row : b) * a.count;
  }
  const int nbb = (Tb + Bs - 1) / Bs;
  // ids, then their pages, each a batch of loads in flight at once
  const int n = e1 - e0;
  if (n > 0) {
    stage_batches(n, [&](int base) {
      int x[kStageBatch], pg[kStageBatch];
#pragma unroll
      for (int u = 0; u < kStageBatch; ++u)
        x[u] = src[e0 + min(base + u * (int)blockDim.x + (int)threadIdx.x, n - 1)];
#pragma unroll
      for (int u = 0; u < kStageBatch; ++u) {
        const bool ok = KIND == 3 ? (x[u] >= 0 && x[u] < nbb) : (x[u] >= 0 && x[u] < Tb);
        const int j = ok ? (KIND == 3 ? x[u] : x[u] / Bs) : 0;
        pg[u] = tb[j];
      }
#pragma unroll
      for (int u = 0; u < kStageBatch; ++u) {
        const int i = base + u * (int)blockDim.x + (int)threadIdx.x;
        if (i < n) {
          const bool ok = KIND == 3 ? (x[u] >= 0 && x[u] < nbb) : (x[u] >= 0 && x[u] < Tb);
          s_idx[i] = x[u];
          if constexpr (KIND == 3)
            s_pg[i] = ok ? pg[u] : 0;
          else
            s_pg[i] = ok ? pg[u] * a.page_rows + x[u] % Bs : 0;
        }
      }
    });
  }
  if constexpr (kMfma)
    attn_row_mfma<G, KIND>(a, row, split, s_idx, s_pg, e0, true);
  else
    attn_row_valu<T, D, G, KIND>(a, row, split, s_idx, s_pg, e0, true);
}

template <typename T, int D, int G>
hipError_t launch_typed(const AttnArgs& a, int kind, const AttnPlan& p, hipStream_t s) {
  const int rows = a.d.B * a.d.Hkv;
  const dim3 grid(rows * p.splits), block(p.nw * 64);
  constexpr bool mfma = KSA_MFMA && std::is_same<T, uint16_t>::value && D == 128 && G >= 4;
  if (kind == 3 && a.idx == nullptr) {  // paged dense: every block of the row
    if constexpr (mfma) {
      if (a.vkeys)
        hipLaunchKernelGGL((attn_paged_dense_kernel<T, D, G, true>), grid, block, 0, s, a);
      else
        hipLaunchKernelGGL((attn_paged_dense_kernel<T, D, G>), grid, block, 0, s, a);
    } else {
      hipLaunchKernelGGL((attn_paged_dense_kernel<T, D, G>), grid, block, 0, s, a);
    }
  } else if (kind == 3) {
    hipLaunchKernelGGL((attn_paged_list_kernel<T, D, G, 3>), grid, block, 0, s, a);
  } else if (kind == 5) {
    hipLaunchKernelGGL((attn_paged_list_kernel<T, D, G, 5>), grid, block, 0, s, a);
  } else if (kind == 6) {  // rows are query heads: one head per row
    if constexpr (G == 1)
      hipLaunchKernelGGL((attn_paged_list_kernel<T, D, 1, 6>), grid, block, 0, s, a);
  } else if (kind == 4) {  // rows are query heads: one head per row
    if constexpr (G == 1)
      hipLaunchKernelGGL((attn_partial_kernel<T, D, 1, 4>), grid, block, 0, s, a);
  } else if constexpr (mfma) {
    switch (kind) {
      case 0: hipLaunchKernelGGL((attn_mfma_kernel<G, 0>), grid, block, 0, s, a); break;
      case 1: hipLaunchKernelGGL((attn_mfma_kernel<G, 1>), grid, block, 0, s, a); break;
      default:
        if (a.vkeys)
          hipLaunchKernelGGL((attn_mfma_kernel<G, 2, true>), grid, block, 0, s, a);
        else
          hipLaunchKernelGGL((attn_mfma_kernel<G, 2>), grid, block, 0, s, a);
        break;
    }
  } else {
    switch (kind) {
      case 0: hipLaunchKernelGGL((attn_partial_kernel<T, D, G, 0>), grid, block, 0, s, a); break;
      case 1: hipLaunchKernelGGL((attn_partial_kernel<T, D, G, 1>), grid, block, 0, s, a); break;
      default: hipLaunchKernelGGL((attn_partial_kernel<T, D, G, 2>), grid, block, 0, s, a); break;
    }
  }
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_g(const AttnArgs& a, int kind, const AttnPlan& p, hipStream_t s) {
  switch (a.d.G) {
    case 1: return launch_typed<T, D, 1>(a, kind, p, s);
    case 2: return launch_typed<T, D, 2>(a, kind, p, s);
    case 4: return launch_typed<T, D, 4>(a, kind, p, s);
    default: return launch_typed<T, D, 8>(a, kind, p, s);
  }
}

}  // namespace

AttnPlan plan_attention(const Dims& d, int kind, int64_t tokens_per_row) {
  const int ch = chunk_tokens(d);
  const int64_t chunks = (tokens_per_row + ch - 1) / ch;
  const int64_t rows = (int64_t)d.B * d.Hkv;
  // Planned for MI355X (256 CUs) whatever the device, so that the plan, the
  // workspace size and the fp32 merge order are functions of the shape alone.
  const int64_t kCUs = 256;
  const int64_t kMinChunksPerWave = KSA_PLAN_MIN_CHUNKS;  // keeps a wave's pipeline busy past its fill
  // Splits: the fewest that give every CU KSA_PLAN_WGS_PER_CU workgroups (a
  // split row is merged by its last workgroup to finish), as long as each
  // split keeps real work.
  int64_t splits = (kCUs * KSA_PLAN_WGS_PER_CU + rows - 1) / rows;
  const int64_t max_splits = chunks / kMinChunksPerWave > 1 ? chunks / kMinChunksPerWave : 1;
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  int64_t cps = (chunks + splits - 1) / splits;
  int nw = 1;
  while (nw < kMaxWaves && (int64_t)nw * 2 * kMinChunksPerWave <= cps) nw *= 2;
#if defined(KSA_PLAN_WAVES) && defined(KSA_PLAN_SPLITS)
  // a fixed launch shape, for variant builds that sweep shapes
  static_assert(KSA_PLAN_WAVES >= 1 && KSA_PLAN_WAVES <= kMaxWaves && KSA_PLAN_SPLITS >= 1, "plan");
  nw = KSA_PLAN_WAVES;
  splits = KSA_PLAN_SPLITS;
  cps = (chunks + splits - 1) / splits;
#endif
  // a workgroup's index slice must fit the LDS stage
  int64_t cap = INT64_MAX;
  if (kind == 1 || kind == 4 || kind == 5 || kind == 6) cap = kIdxStage / ch;
  if (kind == 0 || kind == 3) cap = ((int64_t)(kIdxStage - 2) * d.Bs) / ch;
  if (cps > cap) cps = cap;
  if (cps < 1) cps = 1;
  splits = (chunks + cps - 1) / cps;
  if (splits < 1) splits = 1;
  if (splits > kMaxSplits) {  // arrival counts are 16-bit
    splits = kMaxSplits;
    cps = (chunks + splits - 1) / splits;
  }
  return AttnPlan{nw, (int)splits, (int)cps, ch};
}

size_t attention_workspace_bytes(const Dims& d, const AttnPlan& p) {
  if (p.splits <= 1) return 0;
  const size_t rows = (size_t)d.B * d.Hkv;
  return arrival_bytes(rows) + rows * p.splits * d.G * (size_t)(d.D + 2) * sizeof(float);
}

namespace {
// A 47-bit tag per call (bit 47 clear), for the arrival words of split rows:
// splitmix64 (Steele, Lea and Flood, 2014) of a process-wide call counter
// started from the clock, so that tags differ between calls and processes.
unsigned long long next_call_tag() {
  static std::atomic<unsigned long long> counter{
      (unsigned long long)std::chrono::steady_clock::now().time_since_epoch().count()};
  unsigned long long x = counter.fetch_add(1, std::memory_order_relaxed) + 0x9E3779B97F4A7C15ull;
  x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
  x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
  x ^= x >> 31;
  return x & 0x7FFFFFFFFFFFull;
}
}  // namespace

hipError_t launch_attention(const Dims& d, int kind, const void* q, const void* k, const void* v,
                            const int32_t* idx, int count, float* out, float* lse, void* workspace,
                            const AttnPlan& plan, hipStream_t stream, const PagedKv* paged,
                            const VoteKeys* vote_keys, int kv_div) {
  AttnArgs a = make_attn_args(d, kind, q, k, v, idx, count, out, lse, workspace, plan);
  if (plan.splits > 1) a.tag = next_call_tag();
  if (paged) {
    a.table = paged->table;
    a.seq_lens = paged->seq_lens;
    a.tstride = paged->max_blocks;
  }
  if (vote_keys) {
    a.vkeys = vote_keys->keys;
    a.vkstride = vote_keys->kstride;
    a.vhist = vote_keys->hist;
    a.vbudget = vote_keys->budget;
    a.vwindow = vote_keys->window;
  }
  if (kind == 4 || kind == 6) a.kv_div = kv_div;
  if (kind == 6) a.page_rows = (d.Hkv / kv_div) * d.Bs;  // d has a row per query head
  if (d.dtype == KSA_BF16) {
    if (d.D == 64) return launch_g<uint16_t, 64>(a, kind, plan, stream);
    return launch_g<uint16_t, 128>(a, kind, plan, stream);
  }
  if (d.D == 64) return launch_g<float, 64>(a, kind, plan, stream);
  return launch_g<float, 128>(a, kind, plan, stream);
}

namespace {
__global__ __launch_bounds__(256) void recall_kernel(const float* __restrict__ lse_sel,
                                                     const float* __restrict__ lse_dense,
                                                     float* __restrict__ recall, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) recall[i] = expf(lse_sel[i] - lse_dense[i]);
}
}  // namespace

hipError_t launch_attention_recall(const float* lse_sel, const float* lse_dense, float* recall,
                                   int n, hipStream_t stream) {
  hipLaunchKernelGGL(recall_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, lse_sel,
                     lse_dense, recall, n);
  return hipGetLastError();
}

}  // namespace ksa

// summaries.hip -- mean key of each block (Kinetics explainer, section 五:
// every block of history tokens is represented by its average).
//
// One group of LPT lanes owns one (sequence, KV head, block) row; each lane
// owns 16 bytes of the D-wide key (8 bf16 or 4 fp32 channels).  The block's
// keys are summed in fp64 in token order, divided once in fp64 (IEEE,
// correctly rounded) and rounded once to the KV dtype with
// round-to-nearest-even, so the stored value is a fixed function of the
// input bytes: RNE(fl64(fl64-sum / n)).
#include "ksa_device.h"
#include "ksa_internal.h"

namespace ksa {
namespace {

constexpr int kBatch = 16;

template <typename T, int D>
__global__ __launch_bounds__(256) void block_summaries_kernel(const T* __restrict__ k,
                                                              T* __restrict__ summ, Dims d,
                                                              int first_block, int num_blocks) {
  constexpr int EPL = KV<T>::EPL;
  constexpr int LPT = D / EPL;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t rowid = gid / LPT;
  const int li = (int)(gid % LPT);
  const int64_t rows = (int64_t)d.B * d.Hkv * num_blocks;
  if (rowid >= rows) return;
  const int j = first_block + (int)(rowid % num_blocks);
  const int64_t bg = rowid / num_blocks;
  const int t0 = j * d.Bs;
  const int t1 = min(t0 + d.Bs, d.T);
  const int n = t1 - t0;
  const T* kp = k + (bg * d.Tcap + t0) * D + li * EPL;
  double acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.0;
  // all of a batch's loads are issued before the in-order fp64 sum consumes them
#pragma unroll 1
  for (int t0 = 0; t0 < n; t0 += kBatch) {
    uint4 r[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) r[u] = ld16(kp + (int64_t)min(t0 + u, n - 1) * D);
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (t0 + u < n) {
        float f[EPL];
        KV<T>::widen(r[u], f);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] += (double)f[e];
      }
    }
  }
  st16(summ + (bg * d.NBcap + j) * D + li * EPL, mean_bits<T>(acc, n));
}

// The same mean over a paged cache: block j of sequence b is a page of the
// pool [num_pages, Hkv, Bs, D]; blocks at or past the sequence's NB_b are
// skipped; first_block < 0 picks each sequence's newest block.
template <typename T, int D>
__global__ __launch_bounds__(256) void paged_block_summaries_kernel(
    const T* __restrict__ k, T* __restrict__ summ, Dims d, const int32_t* __restrict__ table,
    const int32_t* __restrict__ seq_lens, int tstride, int first_block, int num_blocks) {
  constexpr int EPL = KV<T>::EPL;
  constexpr int LPT = D / EPL;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t rowid = gid / LPT;
  const int li = (int)(gid % LPT);
  const int64_t rows = (int64_t)d.B * d.Hkv * num_blocks;
  if (rowid >= rows) return;
  const int64_t bg = rowid / num_blocks;
  const int b = (int)(bg / d.Hkv), g = (int)(bg - (int64_t)b * d.Hkv);
  const int Tb = seq_len_of(seq_lens, b, d.T);
  const int j = first_block < 0 ? (Tb - 1) / d.Bs : first_block + (int)(rowid % num_blocks);
  const int t0 = j * d.Bs;
  if (t0 >= Tb) return;
  const int n = min(d.Bs, Tb - t0);
  const int64_t page = table[(int64_t)b * tstride + j];
  const T* kp = k + ((page * d.Hkv + g) * d.Bs) * D + li * EPL;
  double acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.0;
#pragma unroll 1
  for (int u0 = 0; u0 < n; u0 += kBatch) {
    uint4 r[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) r[u] = ld16(kp + (int64_t)min(u0 + u, n - 1) * D);
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (u0 + u < n) {
        float f[EPL];
        KV<T>::widen(r[u], f);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] += (double)f[e];
      }
    }
  }
  st16(summ + (bg * d.NBcap + j) * D + li * EPL, mean_bits<T>(acc, n));
}

template <typename T, int D>
hipError_t launch_paged_typed(const Dims& d, const PagedKv& p, const void* k, void* summ, int first,
                              int num, hipStream_t s) {
  constexpr int LPT = D / KV<T>::EPL;
  const int64_t threads = (int64_t)d.B * d.Hkv * num * LPT;
  const int grid = (int)((threads + 255) / 256);
  hipLaunchKernelGGL((paged_block_summaries_kernel<T, D>), dim3(grid), dim3(256), 0, s,
                     (const T*)k, (T*)summ, d, p.table, p.seq_lens, p.max_blocks, first, num);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_typed(const Dims& d, const void* k, void* summ, int first, int num,
                        hipStream_t s) {
  constexpr int LPT = D / KV<T>::EPL;
  const int64_t threads = (int64_t)d.B * d.Hkv * num * LPT;
  const int grid = (int)((threads + 255) / 256);
  hipLaunchKernelGGL((block_summaries_kernel<T, D>), dim3(grid), dim3(256), 0, s,
                     (const T*)k, (T*)summ, d, first, num);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_block_summaries(const Dims& d, const void* k, void* summaries, int first_block,
                                  int num_blocks, hipStream_t stream) {
  if (d.dtype == KSA_BF16) {
    if (d.D == 64) return launch_typed<uint16_t, 64>(d, k, summaries, first_block, num_blocks, stream);
    return launch_typed<uint16_t, 128>(d, k, summaries, first_block, num_blocks, stream);
  }
  if (d.D == 64) return launch_typed<float, 64>(d, k, summaries, first_block, num_blocks, stream);
  return launch_typed<float, 128>(d, k, summaries, first_block, num_blocks, stream);
}

hipError_t launch_paged_block_summaries(const Dims& d, const PagedKv& p, const void* k_pool,
                                        void* summaries, int first_block, int num_blocks,
                                        hipStream_t stream) {
  if (d.dtype == KSA_BF16) {
    if (d.D == 64)
      return launch_paged_typed<uint16_t, 64>(d, p, k_pool, summaries, first_block, num_blocks, stream);
    return launch_paged_typed<uint16_t, 128>(d, p, k_pool, summaries, first_block, num_blocks, stream);
  }
  if (d.D == 64)
    return launch_paged_typed<float, 64>(d, p, k_pool, summaries, first_block, num_blocks, stream);
  return launch_paged_typed<float, 128>(d, p, k_pool, summaries, first_block, num_blocks, stream);
}

}  // namespace ksa

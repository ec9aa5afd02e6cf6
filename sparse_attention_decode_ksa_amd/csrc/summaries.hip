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

// fp64 -> bf16 bit pattern, round to nearest, ties to even.  Normal range:
// drop 45 of the 52 fraction bits with an RNE bias on the integer pattern
// (a carry into the exponent is the correct result).  Below 2^-126 the bf16
// grid is uniform with spacing 2^-133: scale (exactly) and round there.
__device__ __forceinline__ uint16_t bf16_rne_from_f64(double x) {
  unsigned long long u = (unsigned long long)__double_as_longlong(x);
  const unsigned long long sign = u & 0x8000000000000000ull;
  unsigned long long a = u ^ sign;
  uint32_t bits;
  if (a < 0x3810000000000000ull) {  // |x| < 2^-126 (also 0)
    double r = rint(__longlong_as_double((long long)a) * 0x1p133);
    bits = (uint32_t)r;  // 0..128; 128 is the smallest normal
  } else {
    const unsigned long long lsb = (a >> 45) & 1ull;
    a += 0xFFFFFFFFFFFull + lsb;  // 2^44 - 1 + lsb
    a >>= 45;                     // (exp64 << 7) | fraction7
    const unsigned long long e = (a >> 7) - 896;  // rebias 1023 -> 127
    bits = e >= 255 ? 0x7F80u : (uint32_t)((e << 7) | (a & 0x7Full));
  }
  return (uint16_t)((sign >> 48) | bits);
}

template <typename T>
__device__ __forceinline__ void store_mean(T* dst, const double* acc, int n);

template <>
__device__ __forceinline__ void store_mean<uint16_t>(uint16_t* dst, const double* acc, int n) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t lo = bf16_rne_from_f64(acc[2 * i] / (double)n);
    uint32_t hi = bf16_rne_from_f64(acc[2 * i + 1] / (double)n);
    w[i] = lo | (hi << 16);
  }
  st16(dst, make_uint4(w[0], w[1], w[2], w[3]));
}

template <>
__device__ __forceinline__ void store_mean<float>(float* dst, const double* acc, int n) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = __float_as_uint((float)(acc[i] / (double)n));
  st16(dst, make_uint4(w[0], w[1], w[2], w[3]));
}

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
  store_mean<T>(summ + (bg * d.NBcap + j) * D + li * EPL, acc, n);
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

}  // namespace ksa

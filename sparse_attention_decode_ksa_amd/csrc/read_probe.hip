// read_probe.hip -- measurement only, not part of the library's interface:
// the HBM read rate this chip gives for the access patterns of the decode
// kernels, with their arithmetic taken away.  The token rows of K and V
// (D = 128 bf16: 256 bytes a row) are read with the attention kernels' lane
// layout (a group of 16 lanes owns one row, 16 bytes a lane, so one wave load
// covers four whole rows) in chunks of 16 listed tokens, from per-row token
// lists: [0, T) for a dense walk, the tokens of the selected blocks (block
// top-k), or one token set shared by the KV heads of a sequence (vote
// union).  Loaded words are folded with XOR and one word per thread is
// written, so no load can be dropped.  The rates bound what a kernel that
// must move exactly these bytes can reach on the same launch shape.
//
// Built into its own libksa_probe.so; the benchmark's --read-probe mode
// drives it (ctypes, device pointers from torch).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kChunk = 16;        // tokens a wave reads per chunk
constexpr int kStageMax = 2048;   // list entries a workgroup stages in LDS
constexpr int kRowU4 = 16;        // 16-byte pieces in one 256-byte token row

__device__ __forceinline__ uint4 ld_nt(const uint4* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 r = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(r.x, r.y, r.z, r.w);
}

// Row r of the launch reads K (and V when TWO) rows t of list
// (r / rows_per_list) at 16-byte offset r * row_stride + t * 16, with t
// clamped into the row's capacity [0, cap) (row_stride >= cap * 16).  Workgroup
// (r, s) takes chunks [s * cps, (s + 1) * cps) of the list; its waves take
// them round-robin and keep INFLIGHT chunks of loads (four or eight 16-byte
// loads a lane each) in flight.
template <int INFLIGHT, bool TWO>
__global__ __launch_bounds__(512) void read_probe_kernel(const uint4* __restrict__ k,
                                                          const uint4* __restrict__ v,
                                                          long long row_stride,
                                                          const int32_t* __restrict__ lists,
                                                          int rows_per_list, int ntok, int cap,
                                                          int splits, int cps,
                                                          uint32_t* __restrict__ sink) {
  __shared__ int s_tok[kStageMax];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int slot = lane >> 4, li = lane & 15;
  const int row = blockIdx.x / splits, split = blockIdx.x - row * splits;
  const int nchunks = (ntok + kChunk - 1) / kChunk;
  const int c_begin = split * cps;
  const int c_end = min(c_begin + cps, nchunks);
  const int e0 = c_begin * kChunk, e1 = min(ntok, c_end * kChunk);
  const int32_t* list = lists + (long long)(row / rows_per_list) * ntok;
  for (int i = threadIdx.x; i < e1 - e0; i += blockDim.x)
    s_tok[i] = min(max(list[e0 + i], 0), cap - 1);
  __syncthreads();
  const uint4* kb = k + (long long)row * row_stride + li;
  const uint4* vb = TWO ? v + (long long)row * row_stride + li : nullptr;
  const int c0 = c_begin + wave;
  const int my_n = c0 < c_end ? (c_end - c0 + nw - 1) / nw : 0;
  // entry of load i of the wave's j-th chunk (past the slice: its last entry)
  auto at = [&](int j, int i) {
    const int p = (c0 + j * nw) * kChunk + 4 * i + slot;
    return s_tok[min(p, e1 - 1) - e0];
  };
  constexpr int NL = TWO ? 8 : 4;  // loads per lane per chunk
  uint4 buf[INFLIGHT][NL];
  uint32_t acc = 0u;
  auto load = [&](int j, uint4(&b)[NL]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const long long t = (long long)at(j, i) * kRowU4;
      b[i] = ld_nt(kb + t);
      if constexpr (TWO) b[4 + i] = ld_nt(vb + t);
    }
  };
  auto fold = [&](const uint4(&b)[NL]) {
#pragma unroll
    for (int i = 0; i < NL; ++i) acc ^= b[i].x ^ b[i].y ^ b[i].z ^ b[i].w;
  };
  // the first INFLIGHT chunks, then each chunk folded and its buffer refilled
  // with the chunk INFLIGHT further on (the loads inside the loop are
  // unconditional, so the wait before each fold is for that chunk alone);
  // the last fewer-than-INFLIGHT chunks go one at a time
  int j = 0;
  if (my_n >= INFLIGHT) {
#pragma unroll
    for (int u = 0; u < INFLIGHT; ++u) load(u, buf[u]);
    for (; j + 2 * INFLIGHT <= my_n; j += INFLIGHT) {
#pragma unroll
      for (int u = 0; u < INFLIGHT; ++u) {
        fold(buf[u]);
        load(j + INFLIGHT + u, buf[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < INFLIGHT; ++u) fold(buf[u]);
    j += INFLIGHT;
  }
  for (; j < my_n; ++j) {  // fewer than INFLIGHT chunks left: one at a time
    load(j, buf[0]);
    fold(buf[0]);
  }
  sink[(long long)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

}  // namespace

extern "C" {

// Reads, for each of `rows` rows, the K and V token rows listed in
// lists[(r / rows_per_list) * ntok ...] (int32 token ids, each < the rows'
// capacity; ntok <= splits * 2048), asynchronously on `stream`.  k, v:
// device pointers to bf16 rows of 256 bytes, row r starting row_stride_bytes
// * r bytes in (a multiple of 16, and at least cap * 256: cap token rows per
// row; listed ids are clamped into [0, cap)); v may be null (K alone, as the
// vote scorer and the summary scan read).  Launch: rows * splits workgroups of
// waves * 64 threads (1 <= waves <= 8), inflight in {1, 2, 4}.  sink: device
// buffer of rows * splits * waves * 64 uint32.  Returns 0, 1 for an argument
// out of range, or 2 when the launch failed.
int ksa_probe_read(const void* k, const void* v, long long row_stride_bytes, int cap,
                   const int32_t* lists, int rows_per_list, int rows, int ntok, int splits,
                   int waves, int inflight, uint32_t* sink, void* stream) {
  if (!k || !lists || !sink || rows < 1 || ntok < 1 || splits < 1 || waves < 1 ||
      waves > 8 || rows_per_list < 1 || cap < 1 || row_stride_bytes % 16 != 0 ||
      row_stride_bytes < (long long)cap * 256)
    return 1;
  const int nchunks = (ntok + kChunk - 1) / kChunk;
  const int cps = (nchunks + splits - 1) / splits;
  if ((long long)cps * kChunk > kStageMax) return 1;
  const dim3 grid((unsigned)(rows * splits)), block((unsigned)(waves * 64));
  const long long stride = row_stride_bytes / 16;
  hipStream_t s = (hipStream_t)stream;
#define KSA_PROBE_LAUNCH(F, TWO)                                                              \
  hipLaunchKernelGGL((read_probe_kernel<F, TWO>), grid, block, 0, s, (const uint4*)k,           \
                     (const uint4*)v, stride, lists, rows_per_list, ntok, cap, splits, cps, sink)
  const bool two = v != nullptr;
  switch (inflight) {
    case 1:
      if (two) KSA_PROBE_LAUNCH(1, true); else KSA_PROBE_LAUNCH(1, false);
      break;
    case 2:
      if (two) KSA_PROBE_LAUNCH(2, true); else KSA_PROBE_LAUNCH(2, false);
      break;
    case 4:
      if (two) KSA_PROBE_LAUNCH(4, true); else KSA_PROBE_LAUNCH(4, false);
      break;
    default:
      return 1;
  }
#undef KSA_PROBE_LAUNCH
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"

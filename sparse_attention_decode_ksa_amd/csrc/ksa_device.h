// ksa_device.h -- device-side helpers for the gfx950 kernels of libksa:
// 16-byte KV loads and widening, 64-wide wavefront reductions through DPP,
// exactly rounded block means, order-preserving 32-bit keys for fp32 scores,
// and wave/block scans.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ksa {

// ---------------------------------------------------------------- KV types
// A lane always moves 16 bytes: 8 bf16 (raw uint16 bit patterns) or 4 fp32.
template <typename T>
struct KV;

template <>
struct KV<uint16_t> {
  static constexpr int EPL = 8;
  // bf16 -> fp32 is exact: the bf16 bits are the fp32's upper half.
  __device__ __forceinline__ static void widen(const uint4& u, float* f) {
    f[0] = __uint_as_float(u.x << 16);
    f[1] = __uint_as_float(u.x & 0xffff0000u);
    f[2] = __uint_as_float(u.y << 16);
    f[3] = __uint_as_float(u.y & 0xffff0000u);
    f[4] = __uint_as_float(u.z << 16);
    f[5] = __uint_as_float(u.z & 0xffff0000u);
    f[6] = __uint_as_float(u.w << 16);
    f[7] = __uint_as_float(u.w & 0xffff0000u);
  }
  __device__ __forceinline__ static float widen1(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }
};

template <>
struct KV<float> {
  static constexpr int EPL = 4;
  __device__ __forceinline__ static void widen(const uint4& u, float* f) {
    f[0] = __uint_as_float(u.x);
    f[1] = __uint_as_float(u.y);
    f[2] = __uint_as_float(u.z);
    f[3] = __uint_as_float(u.w);
  }
  __device__ __forceinline__ static float widen1(float x) { return x; }
};

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
// 16-byte load with the nontemporal (streaming) cache hint, for data read
// once per call.
__device__ __forceinline__ uint4 ld16_stream(const void* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 r = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(r.x, r.y, r.z, r.w);
}
__device__ __forceinline__ void st16(void* p, const uint4& v) { *reinterpret_cast<uint4*>(p) = v; }

// Stores through a buffer resource of `bytes` bytes at `base`: the hardware
// drops every lane whose offset lies past the end, so a wave can issue one
// store instruction whatever subset of its lanes has data (no branch, and a
// fixed number of memory operations per loop iteration, which lets the
// compiler wait for later loads without waiting for the store).
constexpr uint32_t kDropOffset = 0x80000000u;  // past the end of any range made here
__device__ __forceinline__ __amdgpu_buffer_rsrc_t store_range(void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void st16_range(__amdgpu_buffer_rsrc_t rs, uint32_t off, const uint4& v) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 d = {v.x, v.y, v.z, v.w};
  __builtin_amdgcn_raw_buffer_store_b128(d, rs, (int)off, 0, 0);
}

// A sequence's own length read from a device length array, clamped into
// [1, T] with T the call's seq_len (the longest length: launches, workspaces
// and outputs are sized from it, so no length may exceed it).
__device__ __forceinline__ int seq_len_of(const int32_t* seq_lens, int b, int T) {
  return min(max(seq_lens[b], 1), T);
}

// ---------------------------------------------------------------- DPP
// Lane permutations inside a 16-lane row (gfx9 DPP controls).
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i within each 8 lanes
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i within each 16 lanes

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Sum over each aligned group of LPT lanes (LPT in {8, 16, 32}); every lane
// of the group receives the group's sum.
template <int LPT>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(LPT == 8 || LPT == 16 || LPT == 32, "lanes per token");
  x += dpp<kDppXor1>(x);
  x += dpp<kDppXor2>(x);
  x += dpp<kDppHalfMirror>(x);
  if constexpr (LPT >= 16) x += dpp<kDppMirror>(x);
  if constexpr (LPT >= 32) x += __shfl_xor(x, 16);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// ---------------------------------------------------------------- MFMA
// Operand types of v_mfma_f32_16x16x32_bf16.  Lane layout (checked on the
// GPU): A lane l holds row l%16, k-elements 8*(l/16)..+8; B lane l holds
// column l%16, the same k-elements; C lane l holds column l%16, rows
// 4*(l/16)..+4.
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

// a.bf16[0] * b.bf16[0] + a.bf16[1] * b.bf16[1] + c in fp32 (v_dot2c_f32_bf16;
// the bf16 products are exact in fp32)
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& u) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = {u.x, u.y, u.z, u.w};
  return __builtin_bit_cast(bf16x8_t, v);
}

// K tile transpose through LDS.  A 16-token x 256-byte K tile is loaded with
// coalesced row-layout loads (lane = 16 * token-slot + piece) and re-read in
// the MFMA A layout (lane = 16 * k-group + token).  Token t's 16-byte piece c
// lives at slot t*16 + (c ^ t): both the row-layout writes and the A-layout
// reads then touch 16 distinct 16-byte slots per 16 lanes (no bank conflict).
__device__ __forceinline__ int ktile_slot(int t, int c) { return t * 16 + (c ^ t); }

// Orders this wave's LDS accesses around the point for the compiler; the
// hardware executes a wave's LDS instructions in order.
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// ---------------------------------------------------------------- block means
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

// The 16 bytes of a block mean one lane stores: acc holds the lane's fp64
// channel sums (token order), n the block's token count; each channel is
// divided once in fp64 (IEEE) and rounded once, to nearest-even, to the KV
// dtype.
template <typename T>
__device__ __forceinline__ uint4 mean_bits(const double* acc, int n);

template <>
__device__ __forceinline__ uint4 mean_bits<uint16_t>(const double* acc, int n) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t lo = bf16_rne_from_f64(acc[2 * i] / (double)n);
    uint32_t hi = bf16_rne_from_f64(acc[2 * i + 1] / (double)n);
    w[i] = lo | (hi << 16);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

template <>
__device__ __forceinline__ uint4 mean_bits<float>(const double* acc, int n) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = __float_as_uint((float)(acc[i] / (double)n));
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// One channel of mean_bits: the same division and rounding, as a T.
template <typename T>
__device__ __forceinline__ T mean_elem(double acc, int n);

template <>
__device__ __forceinline__ uint16_t mean_elem<uint16_t>(double acc, int n) {
  return bf16_rne_from_f64(acc / (double)n);
}

template <>
__device__ __forceinline__ float mean_elem<float>(double acc, int n) {
  return (float)(acc / (double)n);
}

// ---------------------------------------------------------------- keys
// Order-preserving map of an fp32 score to uint32: larger score -> larger
// key; -0 is folded onto +0 so that equal scores give equal keys.
__device__ __forceinline__ uint32_t order_key(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------- scans
// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

__device__ __forceinline__ uint64_t wave_incl_scan64(uint64_t x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint64_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

// DPP forms (no LDS traffic): row shifts build 16-lane prefixes, the row
// broadcasts of lanes 15 and 31 carry them across the wave.
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  // lanes whose source is outside the row, or whose row is masked off, read 0
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROW_MASK, 0xF, true);
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_incl_scan_dpp(uint32_t x) {
  x += dpp_u32<kDppRowShr1>(x);
  x += dpp_u32<kDppRowShr2>(x);
  x += dpp_u32<kDppRowShr4>(x);
  x += dpp_u32<kDppRowShr8>(x);
  x += dpp_u32<kDppRowBcast15, 0xA>(x);  // rows 1 and 3 add the end of rows 0 and 2
  x += dpp_u32<kDppRowBcast31, 0xC>(x);  // rows 2 and 3 add the end of row 1
  return x;
}

// Minimum / maximum over the 64 lanes of a wave, returned to every lane.
__device__ __forceinline__ uint32_t wave_min_dpp(uint32_t x) {
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, kDppXor1, 0xF, 0xF, false));
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, kDppXor2, 0xF, 0xF, false));
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, kDppHalfMirror, 0xF, 0xF, false));
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, kDppMirror, 0xF, 0xF, false));
  const uint32_t a = __builtin_amdgcn_readlane(x, 0), b = __builtin_amdgcn_readlane(x, 16);
  const uint32_t c = __builtin_amdgcn_readlane(x, 32), e = __builtin_amdgcn_readlane(x, 48);
  return min(min(a, b), min(c, e));
}
__device__ __forceinline__ uint32_t wave_max_dpp(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, kDppXor1, 0xF, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, kDppXor2, 0xF, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, kDppHalfMirror, 0xF, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, kDppMirror, 0xF, 0xF, false));
  const uint32_t a = __builtin_amdgcn_readlane(x, 0), b = __builtin_amdgcn_readlane(x, 16);
  const uint32_t c = __builtin_amdgcn_readlane(x, 32), e = __builtin_amdgcn_readlane(x, 48);
  return max(max(a, b), max(c, e));
}

// Exclusive prefix sum of 32-bit values over the workgroup (blockDim.x a
// multiple of 64, at most 1024 threads); `scratch` holds 16 uint32 in LDS.
// One barrier; every thread of the workgroup must call it, and scratch must
// not be written again before the caller's next barrier.
__device__ __forceinline__ uint32_t block_excl_scan32(uint32_t x, uint32_t* scratch) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nwaves = blockDim.x >> 6;
  const uint32_t incl = wave_incl_scan_dpp(x);
  if (lane == 63) scratch[wave] = incl;
  __syncthreads();
  const uint32_t t = lane < nwaves ? scratch[lane] : 0u;
  const uint32_t ti = wave_incl_scan_dpp(t);
  const uint32_t wave_before = __builtin_amdgcn_readlane(ti - t, wave);
  return wave_before + incl - x;
}

// Exclusive prefix sum over the workgroup (blockDim.x a multiple of 64,
// at most 1024 threads).  `scratch` holds 17 uint64 in LDS.  Returns the
// exclusive prefix and writes the workgroup total to *total.  Contains
// barriers: every thread of the workgroup must call it.
__device__ __forceinline__ uint64_t block_excl_scan64(uint64_t x, uint64_t* scratch,
                                                      uint64_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  uint64_t incl = wave_incl_scan64(x);
  if (lane == 63) scratch[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    uint64_t w = lane < nwaves ? scratch[lane] : 0;
    uint64_t wi = wave_incl_scan64(w);
    if (lane < nwaves) scratch[lane] = wi - w;
    if (lane == 63) scratch[16] = wi;
  }
  __syncthreads();
  uint64_t r = scratch[wave] + incl - x;
  *total = scratch[16];
  __syncthreads();
  return r;
}

}  // namespace ksa

/* decode_step.c -- the C ABI of libksa used from plain C (no Python, no
 * torch): device buffers from hipMalloc, one decode step of block top-k
 * attention, checked by properties that hold for any input:
 *   - with every block selected (top_k >= NB) the one-launch step attends all
 *     tokens, so its output equals ksa_dense_decode's (fp32 rounding only);
 *   - with a real top-k the ids of every row are ascending, distinct and < NB,
 *     and the separate calls (summaries, select, sparse decode) pick the
 *     same blocks as the one-launch step;
 *   - an invalid argument returns a status, and ksa_status_string names it.
 * Prints "OK" and exits 0 when every check holds. */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ksa.h"

#define HIP_CHECK(x)                                                             \
  do {                                                                           \
    hipError_t e_ = (x);                                                         \
    if (e_ != hipSuccess) {                                                      \
      fprintf(stderr, "%s:%d %s\n", __FILE__, __LINE__, hipGetErrorString(e_)); \
      return 2;                                                                  \
    }                                                                            \
  } while (0)
#define KSA_CHECK(x)                                                             \
  do {                                                                           \
    ksa_status s_ = (x);                                                         \
    if (s_ != KSA_OK) {                                                          \
      fprintf(stderr, "%s:%d %s\n", __FILE__, __LINE__, ksa_status_string(s_));  \
      return 3;                                                                  \
    }                                                                            \
  } while (0)

static uint32_t lcg_state = 12345u;
static float uniform01(void) {
  lcg_state = lcg_state * 1664525u + 1013904223u;
  return (float)(lcg_state >> 8) * (1.0f / 16777216.0f);
}
/* roughly N(0,1): the sum of four uniforms, centred and scaled */
static float normalish(void) {
  return (uniform01() + uniform01() + uniform01() + uniform01() - 2.0f) * 1.7320508f;
}
/* fp32 -> bf16, round to nearest even */
static uint16_t to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

int main(void) {
  enum { B = 2, HQ = 8, HKV = 2, D = 128, T = 1000, BS = 16 };
  const int NB = (T + BS - 1) / BS;
  const size_t nq = (size_t)B * HQ * D, nkv = (size_t)B * HKV * T * D;
  uint16_t* hq = (uint16_t*)malloc(nq * 2);
  uint16_t* hk = (uint16_t*)malloc(nkv * 2);
  uint16_t* hv = (uint16_t*)malloc(nkv * 2);
  for (size_t i = 0; i < nq; ++i) hq[i] = to_bf16(normalish());
  for (size_t i = 0; i < nkv; ++i) hk[i] = to_bf16(normalish());
  for (size_t i = 0; i < nkv; ++i) hv[i] = to_bf16(normalish());

  void *dq, *dk, *dv, *ds, *dws;
  float *dout, *dlse, *dout2, *dlse2, *dout3, *dlse3;
  int32_t *didx, *didx2;
  HIP_CHECK(hipMalloc(&dq, nq * 2));
  HIP_CHECK(hipMalloc(&dk, nkv * 2));
  HIP_CHECK(hipMalloc(&dv, nkv * 2));
  HIP_CHECK(hipMalloc(&ds, (size_t)B * HKV * NB * D * 2));
  HIP_CHECK(hipMalloc((void**)&dout, nq * 4));
  HIP_CHECK(hipMalloc((void**)&dlse, (size_t)B * HQ * 4));
  HIP_CHECK(hipMalloc((void**)&dout2, nq * 4));
  HIP_CHECK(hipMalloc((void**)&dlse2, (size_t)B * HQ * 4));
  HIP_CHECK(hipMalloc((void**)&dout3, nq * 4));
  HIP_CHECK(hipMalloc((void**)&dlse3, (size_t)B * HQ * 4));
  HIP_CHECK(hipMalloc((void**)&didx, (size_t)B * HKV * NB * 4));
  HIP_CHECK(hipMalloc((void**)&didx2, (size_t)B * HKV * NB * 4));
  HIP_CHECK(hipMemcpy(dq, hq, nq * 2, hipMemcpyHostToDevice));
  HIP_CHECK(hipMemcpy(dk, hk, nkv * 2, hipMemcpyHostToDevice));
  HIP_CHECK(hipMemcpy(dv, hv, nkv * 2, hipMemcpyHostToDevice));

  const ksa_problem p = {B, HQ, HKV, D, T, T, BS, KSA_BF16, 0.0f};
  size_t ws_bytes = 0;
  const int ops[3] = {KSA_OP_DENSE, KSA_OP_SELECT_TOPK, KSA_OP_SPARSE_BLOCKS};
  const int params[3] = {0, 8, 8};
  for (int i = 0; i < 3; ++i) {
    const size_t w = ksa_workspace_bytes(&p, ops[i], params[i]);
    if (w == (size_t)-1) return 4;
    if (w > ws_bytes) ws_bytes = w;
  }
  HIP_CHECK(hipMalloc(&dws, ws_bytes ? ws_bytes : 16));

  /* every block selected: the one-launch step equals dense attention */
  KSA_CHECK(ksa_block_summaries(&p, dk, ds, 0, NB, NULL));
  KSA_CHECK(ksa_block_topk_decode(&p, dq, dk, dv, ds, NB, 1, didx, dout, dlse, NULL));
  KSA_CHECK(ksa_dense_decode(&p, dq, dk, dv, dout2, dlse2, dws, ws_bytes, NULL));
  HIP_CHECK(hipDeviceSynchronize());
  float* o1 = (float*)malloc(nq * 4);
  float* o2 = (float*)malloc(nq * 4);
  float* l1 = (float*)malloc((size_t)B * HQ * 4);
  float* l2 = (float*)malloc((size_t)B * HQ * 4);
  int32_t* ids = (int32_t*)malloc((size_t)B * HKV * NB * 4);
  int32_t* ids2 = (int32_t*)malloc((size_t)B * HKV * NB * 4);
  HIP_CHECK(hipMemcpy(o1, dout, nq * 4, hipMemcpyDeviceToHost));
  HIP_CHECK(hipMemcpy(o2, dout2, nq * 4, hipMemcpyDeviceToHost));
  HIP_CHECK(hipMemcpy(l1, dlse, (size_t)B * HQ * 4, hipMemcpyDeviceToHost));
  HIP_CHECK(hipMemcpy(l2, dlse2, (size_t)B * HQ * 4, hipMemcpyDeviceToHost));
  HIP_CHECK(hipMemcpy(ids, didx, (size_t)B * HKV * NB * 4, hipMemcpyDeviceToHost));
  double err = 0.0, lerr = 0.0;
  for (size_t i = 0; i < nq; ++i) err = fmax(err, fabs((double)o1[i] - o2[i]));
  for (int i = 0; i < B * HQ; ++i) lerr = fmax(lerr, fabs((double)l1[i] - l2[i]));
  for (int r = 0; r < B * HKV; ++r)
    for (int j = 0; j < NB; ++j)
      if (ids[r * NB + j] != j) {
        fprintf(stderr, "k = NB: row %d id %d is %d\n", r, j, ids[r * NB + j]);
        return 5;
      }
  if (!(err <= 1e-5 && lerr <= 1e-5)) {
    fprintf(stderr, "k = NB: step vs dense max |out| diff %.3g, |lse| diff %.3g\n", err, lerr);
    return 6;
  }

  /* a real top-8: ascending distinct ids, the same from both paths */
  const int K = 8;
  KSA_CHECK(ksa_block_summaries(&p, dk, ds, 0, NB, NULL));
  KSA_CHECK(ksa_select_topk(&p, dq, ds, K, didx2, NULL, dws, ws_bytes, NULL));
  ksa_selection sel = {KSA_SEL_BLOCKS, didx2, K};
  KSA_CHECK(ksa_sparse_decode(&p, dq, dk, dv, &sel, dout3, dlse3, dws, ws_bytes, NULL));
  KSA_CHECK(ksa_block_topk_decode(&p, dq, dk, dv, ds, K, 1, didx, dout, dlse, NULL));
  HIP_CHECK(hipDeviceSynchronize());
  HIP_CHECK(hipMemcpy(ids, didx, (size_t)B * HKV * K * 4, hipMemcpyDeviceToHost));
  HIP_CHECK(hipMemcpy(ids2, didx2, (size_t)B * HKV * K * 4, hipMemcpyDeviceToHost));
  HIP_CHECK(hipMemcpy(o1, dout, nq * 4, hipMemcpyDeviceToHost));
  HIP_CHECK(hipMemcpy(o2, dout3, nq * 4, hipMemcpyDeviceToHost));
  for (int r = 0; r < B * HKV; ++r)
    for (int j = 0; j < K; ++j) {
      const int32_t x = ids[r * K + j];
      if (x < 0 || x >= NB || (j > 0 && x <= ids[r * K + j - 1]) || x != ids2[r * K + j]) {
        fprintf(stderr, "top-%d: row %d position %d: %d / %d\n", K, r, j, x, ids2[r * K + j]);
        return 7;
      }
    }
  err = 0.0;
  for (size_t i = 0; i < nq; ++i) {
    if (!isfinite(o1[i])) return 8;
    err = fmax(err, fabs((double)o1[i] - o2[i]));
  }
  if (!(err <= 1e-5)) {
    fprintf(stderr, "top-%d: step vs separate calls max |out| diff %.3g\n", K, err);
    return 9;
  }

  /* an invalid argument launches nothing and says why */
  const ksa_problem bad = {B, HQ, 3, D, T, T, BS, KSA_BF16, 0.0f}; /* Hq % Hkv != 0 */
  const ksa_status st = ksa_block_topk_decode(&bad, dq, dk, dv, ds, K, 1, didx, dout, dlse, NULL);
  if (st != KSA_ERR_INVALID_ARGUMENT || strstr(ksa_status_string(st), "INVALID") == NULL) return 10;

  printf("OK libksa %s: k = NB step equals dense (max |diff| %.2g), top-%d ids agree\n",
         ksa_version(), lerr > err ? lerr : err, K);
  return 0;
}

/* abi_example.c -- the C ABI used from plain C: HIP runtime allocation and
 * streams, no Python, no torch.  Each check is a closed form of the step:
 *   x = residual = 0.5 and weight = 1 give residual_out = 1, rstd = 1/sqrt(1 + eps)
 *   and y = bf16(0.9999995) = 1, so the per-token scale is 1/448 and every FP8
 *   code is 0x7E (448 * 1/448 = 1 -> 448); the MXFP4 block maximum 1 gives the
 *   E8M0 byte 125 and every E2M1 code 6 (1 * 2^2 = 4), packed as 0x66;
 *   a QK head of constant 1024 with eps = 0 has rstd = 2^-10 exactly, so with
 *   w = 0 the normalized head is 1.0 and the gate is copied unchanged; its FP8
 *   variant gives codes 0x7E and scale 1/448 for every head.
 * Prints "abi example ok" and returns 0 on success. */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "rmsnorm_quant.h"

#define CHECK_HIP(call)                                                      \
  do {                                                                       \
    hipError_t e_ = (call);                                                  \
    if (e_ != hipSuccess) {                                                  \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));       \
      return 1;                                                              \
    }                                                                        \
  } while (0)

#define EXPECT(cond, what)                                                   \
  do {                                                                       \
    if (!(cond)) {                                                           \
      fprintf(stderr, "check failed: %s\n", what);                           \
      return 1;                                                              \
    }                                                                        \
  } while (0)

static int all_u16(const uint16_t* p, size_t n, uint16_t v) {
  for (size_t i = 0; i < n; ++i)
    if (p[i] != v) return 0;
  return 1;
}
static int all_u8(const uint8_t* p, size_t n, uint8_t v) {
  for (size_t i = 0; i < n; ++i)
    if (p[i] != v) return 0;
  return 1;
}

int main(void) {
  enum { M = 16, H = 4096 };
  const size_t n = (size_t)M * H;
  uint16_t* h16 = (uint16_t*)malloc(n * sizeof(uint16_t));
  uint8_t* h8 = (uint8_t*)malloc(n);
  float hs[M];
  uint16_t *x, *w, *ro, *y;
  uint8_t *q, *sb;
  float* s;
  hipStream_t stream;
  CHECK_HIP(hipStreamCreate(&stream));
  CHECK_HIP(hipMalloc((void**)&x, n * 2));
  CHECK_HIP(hipMalloc((void**)&w, H * 2));
  CHECK_HIP(hipMalloc((void**)&ro, n * 2));
  CHECK_HIP(hipMalloc((void**)&y, n * 2));
  CHECK_HIP(hipMalloc((void**)&q, n));
  CHECK_HIP(hipMalloc((void**)&sb, (size_t)M * (H / 32)));
  CHECK_HIP(hipMalloc((void**)&s, (size_t)M * sizeof(float)));

  for (size_t i = 0; i < n; ++i) h16[i] = 0x3F00; /* bf16 0.5 */
  CHECK_HIP(hipMemcpy(x, h16, n * 2, hipMemcpyHostToDevice));
  for (size_t i = 0; i < H; ++i) h16[i] = 0x3F80; /* bf16 1.0 */
  CHECK_HIP(hipMemcpy(w, h16, H * 2, hipMemcpyHostToDevice));

  /* fused per-token FP8; residual is x itself (inputs may alias each other) */
  EXPECT(rmsnorm_quant_fp8_per_token(x, H, x, H, w, M, H, 1e-6f, ro, q, s, y, stream) == RQ_OK, "per-token call");
  CHECK_HIP(hipStreamSynchronize(stream));
  CHECK_HIP(hipMemcpy(h16, ro, n * 2, hipMemcpyDeviceToHost));
  EXPECT(all_u16(h16, n, 0x3F80), "residual_out == 1");
  CHECK_HIP(hipMemcpy(h16, y, n * 2, hipMemcpyDeviceToHost));
  EXPECT(all_u16(h16, n, 0x3F80), "y == 1");
  CHECK_HIP(hipMemcpy(h8, q, n, hipMemcpyDeviceToHost));
  EXPECT(all_u8(h8, n, 0x7E), "FP8 codes == 0x7E");
  CHECK_HIP(hipMemcpy(hs, s, sizeof hs, hipMemcpyDeviceToHost));
  for (int m = 0; m < M; ++m) EXPECT(hs[m] == 1.0f / 448.0f, "scale == 1/448");

  /* fused MXFP4 */
  EXPECT(rmsnorm_quant_mxfp4(x, H, x, H, w, M, H, 1e-6f, ro, q, sb, NULL, stream) == RQ_OK, "mxfp4 call");
  CHECK_HIP(hipStreamSynchronize(stream));
  CHECK_HIP(hipMemcpy(h8, q, n / 2, hipMemcpyDeviceToHost));
  EXPECT(all_u8(h8, n / 2, 0x66), "E2M1 bytes == 0x66");
  CHECK_HIP(hipMemcpy(h8, sb, (size_t)M * (H / 32), hipMemcpyDeviceToHost));
  EXPECT(all_u8(h8, (size_t)M * (H / 32), 125), "E8M0 bytes == 125");

  /* the unfused sequence: quantize y alone */
  EXPECT(quantize_fp8_per_token(y, H, M, H, q, s, stream) == RQ_OK, "quantize call");
  CHECK_HIP(hipStreamSynchronize(stream));
  CHECK_HIP(hipMemcpy(h8, q, n, hipMemcpyDeviceToHost));
  EXPECT(all_u8(h8, n, 0x7E), "quantize(y) codes == 0x7E");

  /* QK: T = 4 tokens, 2 q heads, 1 k head, D = 256; every value 1024, w = 0 */
  {
    enum { T = 4, HQ = 2, HK = 1, D = 256 };
    uint16_t *qg, *k, *qw, *qo, *ko, *go;
    const size_t nqg = (size_t)T * 2 * HQ * D, nk = (size_t)T * HK * D, nq = (size_t)T * HQ * D;
    CHECK_HIP(hipMalloc((void**)&qg, nqg * 2));
    CHECK_HIP(hipMalloc((void**)&k, nk * 2));
    CHECK_HIP(hipMalloc((void**)&qw, D * 2));
    CHECK_HIP(hipMalloc((void**)&qo, nq * 2));
    CHECK_HIP(hipMalloc((void**)&ko, nk * 2));
    CHECK_HIP(hipMalloc((void**)&go, nq * 2));
    for (size_t i = 0; i < nqg; ++i) h16[i] = 0x4480; /* bf16 1024 */
    CHECK_HIP(hipMemcpy(qg, h16, nqg * 2, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(k, h16, nk * 2, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemset(qw, 0, D * 2));
    EXPECT(qk_gemma_rmsnorm_gate(qg, 2 * HQ * D, k, HK * D, qw, qw, T, HQ, HK, D, 0.0f, qo, ko, go, stream) == RQ_OK,
           "qk call");
    CHECK_HIP(hipStreamSynchronize(stream));
    CHECK_HIP(hipMemcpy(h16, qo, nq * 2, hipMemcpyDeviceToHost));
    EXPECT(all_u16(h16, nq, 0x3F80), "normalized q == 1");
    CHECK_HIP(hipMemcpy(h16, ko, nk * 2, hipMemcpyDeviceToHost));
    EXPECT(all_u16(h16, nk, 0x3F80), "normalized k == 1");
    CHECK_HIP(hipMemcpy(h16, go, nq * 2, hipMemcpyDeviceToHost));
    EXPECT(all_u16(h16, nq, 0x4480), "gate copied");
    /* the FP8 variant: every normalized head is 1, so codes 0x7E and scale 1/448 a head */
    {
      uint8_t *qc, *kc;
      float *qs, *ks;
      float hq[T * HQ], hk[T * HK];
      CHECK_HIP(hipMalloc((void**)&qc, nq));
      CHECK_HIP(hipMalloc((void**)&kc, nk));
      CHECK_HIP(hipMalloc((void**)&qs, sizeof hq));
      CHECK_HIP(hipMalloc((void**)&ks, sizeof hk));
      EXPECT(qk_gemma_rmsnorm_gate_fp8(qg, 2 * HQ * D, k, HK * D, qw, qw, T, HQ, HK, D, 0.0f, qc, qs, kc, ks, go,
                                       stream) == RQ_OK,
             "qk fp8 call");
      EXPECT(qk_gemma_rmsnorm_gate_fp8(qg, 2 * HQ * D, k, HK * D, qw, qw, T, HQ, HK, D, 0.0f, qc, NULL, kc, ks, go,
                                       stream) == RQ_ERR_INVALID,
             "qk fp8 without q scales is invalid");
      CHECK_HIP(hipStreamSynchronize(stream));
      CHECK_HIP(hipMemcpy(h8, qc, nq, hipMemcpyDeviceToHost));
      EXPECT(all_u8(h8, nq, 0x7E), "q FP8 codes == 0x7E");
      CHECK_HIP(hipMemcpy(h8, kc, nk, hipMemcpyDeviceToHost));
      EXPECT(all_u8(h8, nk, 0x7E), "k FP8 codes == 0x7E");
      CHECK_HIP(hipMemcpy(hq, qs, sizeof hq, hipMemcpyDeviceToHost));
      CHECK_HIP(hipMemcpy(hk, ks, sizeof hk, hipMemcpyDeviceToHost));
      for (int i = 0; i < T * HQ; ++i) EXPECT(hq[i] == 1.0f / 448.0f, "q scale == 1/448");
      for (int i = 0; i < T * HK; ++i) EXPECT(hk[i] == 1.0f / 448.0f, "k scale == 1/448");
      hipFree(qc); hipFree(kc); hipFree(qs); hipFree(ks);
    }
    hipFree(qg); hipFree(k); hipFree(qw); hipFree(qo); hipFree(ko); hipFree(go);
  }

  /* deterministic preflight: nothing is enqueued on error */
  EXPECT(rmsnorm_quant_fp8_per_token(NULL, H, x, H, w, M, H, 1e-6f, ro, q, s, NULL, stream) == RQ_ERR_INVALID,
         "null x is invalid");
  EXPECT(rmsnorm_quant_mxfp4(x, H, x, H, w, M, 48, 1e-6f, ro, q, sb, NULL, stream) == RQ_ERR_UNSUPPORTED,
         "H = 48 cannot fuse MXFP4");
  EXPECT(strncmp(rq_status_string(RQ_ERR_UNSUPPORTED), "RQ_ERR_UNSUPPORTED", 18) == 0, "status string");

  hipFree(x); hipFree(w); hipFree(ro); hipFree(y); hipFree(q); hipFree(sb); hipFree(s);
  CHECK_HIP(hipStreamDestroy(stream));
  free(h16);
  free(h8);
  printf("abi example ok\n");
  return 0;
}

// Host-only fuzz of the C ABI's preflight, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code (tests/test_abi_preflight_sanitized.py).
// Fake pointers: it runs only where no GPU is visible (checked first), so that
// every call that passes the preflight stops at the device check.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <limits>
#include <random>

#include "rmsnorm_quant.h"

static std::mt19937_64 rng(12345);
static const int64_t kVals[] = {-1, 0, 1, 2, 3, 7, 8, 16, 31, 32, 64, 100, 128, 256, 512, 1024, 2048, 4096, 7168,
                                8192, 16384, 16392, 65536, (int64_t(1) << 31) - 1, int64_t(1) << 31,
                                int64_t(1) << 40, int64_t(1) << 47, int64_t(1) << 48, int64_t(1) << 62,
                                std::numeric_limits<int64_t>::max(), std::numeric_limits<int64_t>::min(),
                                std::numeric_limits<int64_t>::max() / 2 + 1, -4096};
static int64_t iv() {
  if (rng() % 4 == 0) return (int64_t)(rng() % 20000) - 100;
  return kVals[rng() % (sizeof(kVals) / sizeof(kVals[0]))];
}
static float fv() {
  const float v[] = {1e-6f, 0.0f, -1.0f, NAN, INFINITY, 1e30f, -0.0f};
  return v[rng() % 7];
}
static int slot = 0;
template <typename T>
static T* pv() {
  const uint64_t r = rng() % 16;
  if (r == 0) return nullptr;
  if (r == 1) return reinterpret_cast<T*>(uintptr_t(1) << 44);  // a repeated base: overlaps
  uintptr_t p = (uintptr_t)(++slot % 64 + 1) << 50;             // far-apart bases
  if (r == 2) p += 2;                                           // misaligned
  if (r == 3) p = ~uintptr_t(0) - 4095;                         // top of the address space
  return reinterpret_cast<T*>(p);
}

static long counts[5];
static void seen(rq_status s) {
  if ((int)s < 0 || (int)s > 4) {
    std::fprintf(stderr, "bad status %d\n", (int)s);
    std::abort();
  }
  if (s == RQ_OK) {
    // M == 0 / T == 0 only: nothing may launch here
    counts[0]++;
    return;
  }
  counts[(int)s]++;
}

int main(int argc, char** argv) {
  int n = 0;
  if (hipGetDeviceCount(&n) == hipSuccess && n > 0) {
    std::fprintf(stderr, "a GPU is visible: this fuzz passes fake pointers and runs only without one\n");
    return 2;
  }
  const long iters = argc > 1 ? std::atol(argv[1]) : 200000;
  using u16 = uint16_t;
  using u8 = uint8_t;
  for (long i = 0; i < iters; ++i) {
    switch (i % 21) {
      case 0: seen(rmsnorm_quant_fp8_per_token(pv<const u16>(), iv(), pv<const u16>(), iv(), pv<const u16>(), iv(), iv(), fv(), pv<u16>(), pv<u8>(), pv<float>(), pv<u16>(), nullptr)); break;
      case 1: seen(rmsnorm_quant_fp8_per_group(pv<const u16>(), iv(), pv<const u16>(), iv(), pv<const u16>(), iv(), iv(), fv(), iv(), pv<u16>(), pv<u8>(), pv<float>(), pv<u16>(), nullptr)); break;
      case 2: seen(rmsnorm_quant_mxfp4(pv<const u16>(), iv(), pv<const u16>(), iv(), pv<const u16>(), iv(), iv(), fv(), pv<u16>(), pv<u8>(), pv<u8>(), pv<u16>(), nullptr)); break;
      case 3: seen(rmsnorm_residual_bf16(pv<const u16>(), iv(), pv<const u16>(), iv(), pv<const u16>(), iv(), iv(), fv(), pv<u16>(), pv<u16>(), nullptr)); break;
      case 4: seen(quantize_fp8_per_token(pv<const u16>(), iv(), iv(), iv(), pv<u8>(), pv<float>(), nullptr)); break;
      case 5: seen(quantize_fp8_per_group(pv<const u16>(), iv(), iv(), iv(), iv(), pv<u8>(), pv<float>(), nullptr)); break;
      case 6: seen(quantize_mxfp4(pv<const u16>(), iv(), iv(), iv(), pv<u8>(), pv<u8>(), nullptr)); break;
      case 7: seen(rmsnorm_quant_fp8_per_token_f16(pv<const u16>(), iv(), pv<const u16>(), iv(), pv<const u16>(), iv(), iv(), fv(), pv<u16>(), pv<u8>(), pv<float>(), pv<u16>(), nullptr)); break;
      case 8: seen(rmsnorm_quant_fp8_per_group_f16(pv<const u16>(), iv(), pv<const u16>(), iv(), pv<const u16>(), iv(), iv(), fv(), iv(), pv<u16>(), pv<u8>(), pv<float>(), pv<u16>(), nullptr)); break;
      case 9: seen(rmsnorm_quant_mxfp4_f16(pv<const u16>(), iv(), pv<const u16>(), iv(), pv<const u16>(), iv(), iv(), fv(), pv<u16>(), pv<u8>(), pv<u8>(), pv<u16>(), nullptr)); break;
      case 10: seen(rmsnorm_residual_f16(pv<const u16>(), iv(), pv<const u16>(), iv(), pv<const u16>(), iv(), iv(), fv(), pv<u16>(), pv<u16>(), nullptr)); break;
      case 11: seen(quantize_fp8_per_token_f16(pv<const u16>(), iv(), iv(), iv(), pv<u8>(), pv<float>(), nullptr)); break;
      case 12: seen(quantize_fp8_per_group_f16(pv<const u16>(), iv(), iv(), iv(), iv(), pv<u8>(), pv<float>(), nullptr)); break;
      case 13: seen(quantize_mxfp4_f16(pv<const u16>(), iv(), iv(), iv(), pv<u8>(), pv<u8>(), nullptr)); break;
      case 14: seen(rmsnorm_quant_fp8_per_group_tscale(pv<const u16>(), iv(), pv<const u16>(), iv(), pv<const u16>(), iv(), iv(), fv(), iv(), pv<u16>(), pv<u8>(), pv<float>(), iv(), pv<u16>(), nullptr)); break;
      case 15: seen(rmsnorm_quant_mxfp4_tscale(pv<const u16>(), iv(), pv<const u16>(), iv(), pv<const u16>(), iv(), iv(), fv(), pv<u16>(), pv<u8>(), pv<u8>(), iv(), pv<u16>(), nullptr)); break;
      case 16: seen(rmsnorm_quant_fp8_per_group_tscale_f16(pv<const u16>(), iv(), pv<const u16>(), iv(), pv<const u16>(), iv(), iv(), fv(), iv(), pv<u16>(), pv<u8>(), pv<float>(), iv(), pv<u16>(), nullptr)); break;
      case 17: seen(rmsnorm_quant_mxfp4_tscale_f16(pv<const u16>(), iv(), pv<const u16>(), iv(), pv<const u16>(), iv(), iv(), fv(), pv<u16>(), pv<u8>(), pv<u8>(), iv(), pv<u16>(), nullptr)); break;
      case 18: seen(qk_gemma_rmsnorm_gate(pv<const u16>(), iv(), pv<const u16>(), iv(), pv<const u16>(), pv<const u16>(), iv(), iv(), iv(), iv(), fv(), pv<u16>(), pv<u16>(), pv<u16>(), nullptr)); break;
      case 19: seen(qk_gemma_rmsnorm_gate_fp8(pv<const u16>(), iv(), pv<const u16>(), iv(), pv<const u16>(), pv<const u16>(), iv(), iv(), iv(), iv(), fv(), pv<u8>(), pv<float>(), pv<u8>(), pv<float>(), pv<u16>(), nullptr)); break;
      case 20: seen(qk_gemma_rmsnorm_gate_mxfp4(pv<const u16>(), iv(), pv<const u16>(), iv(), pv<const u16>(), pv<const u16>(), iv(), iv(), iv(), iv(), fv(), pv<u8>(), pv<u8>(), pv<u8>(), pv<u8>(), pv<u16>(), nullptr)); break;
    }
  }
  for (int s = -1; s < 100; ++s) (void)rq_status_string((rq_status)s);
  std::printf("calls %ld: ok %ld invalid %ld unsupported %ld hip %ld device %ld\n", iters, counts[0], counts[1],
              counts[2], counts[3], counts[4]);
  return 0;
}

// Every oracle entry point on heap buffers of exactly the extent its arguments
// describe (strided inputs, column-major scales, interleaved QK rows), with
// random shapes and random bit patterns (non-finite values included).  Built
// with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_oracle_sanitized.py: a read or write past any buffer ends the run.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "rq_oracle.h"

static std::mt19937_64 rng(2024);

// An exactly sized heap buffer (operator new[]: ASan guards both ends).
template <typename T>
struct Buf {
  T* p;
  explicit Buf(int64_t n) : p(new T[n > 0 ? n : 1]) {
    for (int64_t i = 0; i < n; ++i) p[i] = (T)rng();
  }
  ~Buf() { delete[] p; }
  Buf(const Buf&) = delete;
  Buf& operator=(const Buf&) = delete;
};

static int64_t pick(std::initializer_list<int64_t> v) { return *(v.begin() + rng() % v.size()); }
static int64_t range(int64_t lo, int64_t hi) { return lo + (int64_t)(rng() % (uint64_t)(hi - lo + 1)); }
static void ok(int status, const char* what) {
  if (status != 0) {
    std::fprintf(stderr, "%s returned %d\n", what, status);
    std::exit(1);
  }
}

typedef int (*RowFn)(const uint16_t*, int64_t, const uint16_t*, int64_t, const uint16_t*, int64_t, int64_t, float,
                     uint16_t*, uint8_t*, void*, uint16_t*);

int main(int argc, char** argv) {
  const int iters = argc > 1 ? std::atoi(argv[1]) : 300;
  // "short": the weight buffer one element short of H, a negative control
  // that the sanitizer must report
  const int64_t short_by = argc > 2 && argv[2][0] == 's' ? 1 : 0;
  long calls = 0;
  for (int it = 0; it < iters; ++it) {
    const int64_t M = range(1, 9), H = 32 * range(1, 24);
    const int64_t ldx = H + 8 * range(0, 3), ldr = H + 8 * range(0, 3);
    const int64_t group = H % 128 == 0 ? pick({32, 64, 128}) : 32;
    const int64_t G = H / group, B = H / 32;
    const float eps = (float)pick({0, 1}) * 1e-6f;
    const bool f16 = rng() & 1, emit_y = rng() & 1;
    Buf<uint16_t> x((M - 1) * ldx + H), r((M - 1) * ldr + H), w(H - short_by), ro(M * H), y(M * H);
    uint16_t* yp = emit_y ? y.p : nullptr;
    {
      Buf<uint8_t> q(M * H);
      Buf<float> s(M);
      ok((f16 ? rq_ref_rmsnorm_quant_fp8_per_token_f16 : rq_ref_rmsnorm_quant_fp8_per_token)(
             x.p, ldx, r.p, ldr, w.p, M, H, eps, ro.p, q.p, s.p, yp), "fp8 per token");
    }
    {
      Buf<uint8_t> q(M * H);
      Buf<float> s(M * G);
      ok((f16 ? rq_ref_rmsnorm_quant_fp8_per_group_f16 : rq_ref_rmsnorm_quant_fp8_per_group)(
             x.p, ldx, r.p, ldr, w.p, M, H, eps, group, ro.p, q.p, s.p, yp), "fp8 per group");
      ok((f16 ? rq_ref_quantize_fp8_f16 : rq_ref_quantize_fp8)(ro.p, M, H, group, q.p, s.p), "quantize fp8");
    }
    {
      Buf<uint8_t> q(M * H / 2), s(M * B);
      ok((f16 ? rq_ref_rmsnorm_quant_mxfp4_f16 : rq_ref_rmsnorm_quant_mxfp4)(
             x.p, ldx, r.p, ldr, w.p, M, H, eps, ro.p, q.p, s.p, yp), "mxfp4");
      ok((f16 ? rq_ref_quantize_mxfp4_f16 : rq_ref_quantize_mxfp4)(ro.p, M, H, q.p, s.p), "quantize mxfp4");
    }
    {
      const int64_t ld = M + range(0, 5);
      Buf<uint8_t> q(M * H);
      Buf<float> s((G - 1) * ld + M);
      ok((f16 ? rq_ref_rmsnorm_quant_fp8_per_group_tscale_f16 : rq_ref_rmsnorm_quant_fp8_per_group_tscale)(
             x.p, ldx, r.p, ldr, w.p, M, H, eps, group, ro.p, q.p, s.p, ld, yp), "fp8 per group, column-major");
      Buf<uint8_t> q4(M * H / 2), s4((B - 1) * ld + M);
      ok((f16 ? rq_ref_rmsnorm_quant_mxfp4_tscale_f16 : rq_ref_rmsnorm_quant_mxfp4_tscale)(
             x.p, ldx, r.p, ldr, w.p, M, H, eps, ro.p, q4.p, s4.p, ld, yp), "mxfp4, column-major");
    }
    {
      const int64_t T = range(1, 5), Hq = range(1, 4), Hk = range(1, 3), D = pick({32, 64, 128, 256});
      const int64_t ld_qg = 2 * Hq * D + 8 * range(0, 2), ld_k = Hk * D + 8 * range(0, 2);
      Buf<uint16_t> qg((T - 1) * ld_qg + 2 * Hq * D), k((T - 1) * ld_k + Hk * D), qw(D), kw(D);
      Buf<uint16_t> qo(T * Hq * D), ko(T * Hk * D), go(T * Hq * D);
      ok(rq_ref_qk_gemma_rmsnorm_gate(qg.p, ld_qg, k.p, ld_k, qw.p, kw.p, T, Hq, Hk, D, eps, qo.p, ko.p, go.p),
         "qk");
      Buf<uint8_t> qc(T * Hq * D), kc(T * Hk * D);
      Buf<float> qs(T * Hq), ks(T * Hk);
      ok(rq_ref_qk_gemma_rmsnorm_gate_fp8(qg.p, ld_qg, k.p, ld_k, qw.p, kw.p, T, Hq, Hk, D, eps, qc.p, qs.p, kc.p,
                                          ks.p, go.p), "qk fp8");
      Buf<uint8_t> qc4(T * Hq * D / 2), kc4(T * Hk * D / 2), qs4(T * Hq * D / 32), ks4(T * Hk * D / 32);
      ok(rq_ref_qk_gemma_rmsnorm_gate_mxfp4(qg.p, ld_qg, k.p, ld_k, qw.p, kw.p, T, Hq, Hk, D, eps, qc4.p, qs4.p,
                                            kc4.p, ks4.p, go.p), "qk mxfp4");
    }
    calls += 11;
  }
  for (int b = 0; b < 65536; ++b) {
    (void)rq_ref_f64_from_bf16((uint16_t)b);
    (void)rq_ref_f64_from_f16((uint16_t)b);
  }
  std::printf("oracle calls %ld clean\n", calls);
  return 0;
}

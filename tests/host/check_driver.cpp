#include <algorithm>
#include <cmath>
// Host-only driver for the C-ABI argument checks (built with g++ and the
// address/undefined-behaviour sanitizers by tests/test_abi_cpu.py; no HIP).
#include <cstdio>
#include <cstdint>
#include <string>

#include "check.h"
#include "fexp.h"

static int failures = 0;
#define EXPECT(cond)                                                  \
  do {                                                                \
    if (!(cond)) {                                                    \
      std::printf("FAILED line %d: %s\n", __LINE__, #cond);           \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

int main() {
  using namespace orthrus;
  // fake, 16-byte aligned, never dereferenced device addresses
  void* P = reinterpret_cast<void*>(uintptr_t(0x10000));
  const int32_t* I = reinterpret_cast<const int32_t*>(uintptr_t(0x20000));
  orthrus_kv kv{P, P, I, I, 4096, 16, 8, 128, 2600};
  std::string err;
  AttnPlan plan;

  // a valid 40K call: only the workspace size decides
  AttnPlan ok;
  EXPECT(plan_attention_shape(1, 32, 32, 8, 128, 40960, 0, &ok, nullptr));
  EXPECT(ok.split % 64 == 0 && ok.nsplit * ok.split >= 40960 + 32);
  EXPECT(check_attention(&kv, P, P, P, P, 1, 32, 32, 0.088f, 40960, 0, P, ok.ws_bytes, &plan, &err) == ORTHRUS_OK);
  EXPECT(check_attention(&kv, P, P, P, P, 1, 32, 32, 0.088f, 40960, 0, P, ok.ws_bytes - 1, &plan, &err) == ORTHRUS_ERR_WORKSPACE_TOO_SMALL);

  EXPECT(check_attention(nullptr, P, P, P, P, 1, 32, 32, 0.1f, 100, 0, P, 1 << 30, &plan, &err) == ORTHRUS_ERR_INVALID_ARG);
  EXPECT(check_attention(&kv, nullptr, P, P, P, 1, 32, 32, 0.1f, 100, 0, P, 1 << 30, &plan, &err) == ORTHRUS_ERR_INVALID_ARG);
  EXPECT(check_attention(&kv, P, P, P, P, 1, 0, 32, 0.1f, 100, 0, P, 1 << 30, &plan, &err) == ORTHRUS_ERR_UNSUPPORTED_SHAPE);
  EXPECT(check_attention(&kv, P, P, P, P, 1, 65, 32, 0.1f, 100, 0, P, 1 << 30, &plan, &err) == ORTHRUS_ERR_UNSUPPORTED_SHAPE);
  EXPECT(check_attention(&kv, P, P, P, P, 1, 32, 30, 0.1f, 100, 0, P, 1 << 30, &plan, &err) == ORTHRUS_ERR_UNSUPPORTED_SHAPE);
  EXPECT(check_attention(&kv, P, P, P, P, 1, 32, 32 * 17, 0.1f, 100, 0, P, 1 << 30, &plan, &err) == ORTHRUS_ERR_UNSUPPORTED_SHAPE);
  EXPECT(check_attention(&kv, P, P, P, P, 1, 32, 32, 0.0f, 100, 0, P, 1 << 30, &plan, &err) == ORTHRUS_ERR_INVALID_ARG);
  EXPECT(check_attention(&kv, P, P, P, P, 1, 32, 32, 0.1f, 100, 100, P, 1 << 30, &plan, &err) == ORTHRUS_ERR_INVALID_ARG);
  EXPECT(check_attention(&kv, P, P, P, P, -1, 32, 32, 0.1f, 100, 0, P, 1 << 30, &plan, &err) == ORTHRUS_ERR_INVALID_ARG);
  EXPECT(check_attention(&kv, P, P, P, P, 1, 32, 32, 0.1f, 2600 * 16 - 31, 0, P, 1u << 31, &plan, &err) == ORTHRUS_ERR_CAPACITY);
  void* mis = reinterpret_cast<void*>(uintptr_t(0x10008));
  EXPECT(check_attention(&kv, mis, P, P, P, 1, 32, 32, 0.1f, 100, 0, P, 1 << 30, &plan, &err) == ORTHRUS_ERR_INVALID_ARG);
  orthrus_kv bad = kv;
  bad.page_size = 32;
  EXPECT(check_attention(&bad, P, P, P, P, 1, 32, 32, 0.1f, 100, 0, P, 1 << 30, &plan, &err) == ORTHRUS_ERR_UNSUPPORTED_SHAPE);
  bad = kv;
  bad.head_dim = 96;
  EXPECT(check_attention(&bad, P, P, P, P, 1, 32, 32, 0.1f, 100, 0, P, 1 << 30, &plan, &err) == ORTHRUS_ERR_UNSUPPORTED_SHAPE);
  // batch 0 is a no-op even with null tensors
  EXPECT(check_attention(&kv, nullptr, nullptr, nullptr, nullptr, 0, 32, 32, 0.1f, 100, 0, nullptr, 0, &plan, &err) == ORTHRUS_OK);

  ArgmaxPlan ap;
  LmHeadPlan lp0;
  EXPECT(plan_argmax(32, 151936, &ap) && ap.chunk % 4 == 0 && int64_t(ap.chunk) * ap.nchunks >= 151936);
  EXPECT(check_argmax(reinterpret_cast<const float*>(P), 32, 151936, I, P, ap.ws_bytes, &ap, &err) == ORTHRUS_OK);
  EXPECT(check_argmax(reinterpret_cast<const float*>(P), 32, 151936, I, P, 8, &ap, &err) == ORTHRUS_ERR_WORKSPACE_TOO_SMALL);
  EXPECT(check_argmax(reinterpret_cast<const float*>(P), 32, 0, I, P, 1 << 20, &ap, &err) == ORTHRUS_ERR_INVALID_ARG);
  EXPECT(check_argmax(nullptr, 0, 10, nullptr, nullptr, 0, &ap, &err) == ORTHRUS_OK);
  // vocabularies up to 2^30 keep every chunk bound (start + chunk) below 2^31
  EXPECT(check_argmax(reinterpret_cast<const float*>(P), 1, kMaxVocab + 1, I, P, size_t(1) << 40, &ap, &err) == ORTHRUS_ERR_UNSUPPORTED_SHAPE);
  EXPECT(check_argmax(reinterpret_cast<const float*>(P), 1, kMaxVocab, I, P, size_t(1) << 40, &ap, &err) == ORTHRUS_OK);
  EXPECT(int64_t(ap.chunk) * (ap.nchunks - 1) + ap.chunk < (int64_t(1) << 31));
  EXPECT(!plan_lmhead(1, 4096, kMaxVocab + 1, &lp0, nullptr));
  EXPECT(check_accept(reinterpret_cast<const float*>(P), I, 1, 32, 1024, const_cast<int32_t*>(I), const_cast<int32_t*>(I), const_cast<int32_t*>(I), nullptr, P, 1 << 20, &ap, &err) == ORTHRUS_ERR_INVALID_ARG);
  EXPECT(check_accept(reinterpret_cast<const float*>(P), I, 1, 65, 1024, const_cast<int32_t*>(I), const_cast<int32_t*>(I), const_cast<int32_t*>(I), const_cast<int32_t*>(I), P, 1 << 20, &ap, &err) == ORTHRUS_ERR_UNSUPPORTED_SHAPE);

  // LM head: the 32-row streaming kernel up to 32 rows; one row tile (up to 128 rows): GEMM
  // over contiguous vocabulary ranges; above, the GEMM tile whose workgroups
  // fill rounds of 256 CUs better (wide tiles cost ~1.87x a narrow one)
  LmHeadPlan lp;
  EXPECT(plan_lmhead(32, 4096, 151936, &lp, nullptr) && lp.gemm == 0 && lp.nwg == 256 && lp.nrc == 1);
  EXPECT(plan_lmhead(33, 4096, 151936, &lp, nullptr) && lp.gemm == 3 && lp.nwg == 256 && lp.nrc == 1);
  EXPECT(plan_lmhead(64, 4096, 151936, &lp, nullptr) && lp.gemm == 3 && lp.nrc == 1);
  EXPECT(plan_lmhead(65, 4096, 151936, &lp, nullptr) && lp.gemm == 3 && lp.nwg == 256 && lp.nrc == 1);
  EXPECT(plan_lmhead(128, 4096, 151936, &lp, nullptr) && lp.gemm == 3);
  EXPECT(plan_lmhead(100, 192, 300, &lp, nullptr) && lp.gemm == 3 && lp.nwg == 256);
  EXPECT(plan_lmhead(100, 192, 77, &lp, nullptr) && lp.gemm == 3 && lp.nwg == 77);
  EXPECT(plan_lmhead(129, 4096, 151936, &lp, nullptr) && lp.gemm == 1 && lp.nwg == 594 && lp.nrc == 2);
  EXPECT(plan_lmhead(384, 4096, 151936, &lp, nullptr) && lp.gemm == 1 && lp.nrc == 3);
  EXPECT(plan_lmhead(512, 4096, 151936, &lp, nullptr) && lp.gemm == 2 && lp.nwg == 594 && lp.nrc == 2);
  EXPECT(lp.ws_bytes >= size_t(512) * 594 * 8);
  EXPECT(plan_lmhead(300, 1024, 25523, &lp, nullptr) && lp.gemm == 2 && lp.nwg == 100 && lp.nrc == 2);
  EXPECT(plan_lmhead(300, 1024, 20011, &lp, nullptr) && lp.gemm == 1);
  EXPECT(!plan_lmhead(32, 4000, 151936, &lp, nullptr));   // hidden not a multiple of 64

  // sampling statistics: chunks of 1024 entries while their wavefronts fit on
  // the GPU at once (152 per row of 151936: up to 47 rows), else 2048; groups
  // of 4 chunks; 4.2 M words make 4102 chunks (more than the 1024 whose
  // weights a draw keeps in LDS)
  SamplePlan sp;
  EXPECT(plan_sample(32, 0, 151936, &sp) && sp.chunk == 1024 && sp.nchunks == 149 && sp.ngroups == 38);
  EXPECT(plan_sample(47, 0, 151936, &sp) && sp.chunk == 1024);
  EXPECT(plan_sample(48, 0, 151936, &sp) && sp.chunk == 2048 && sp.nchunks == 75 && sp.ngroups == 19);
  EXPECT(plan_sample(2 * 16 * 32, 16, 151936, &sp) && sp.nchunks == 75 && sp.rchunks == 149);
  EXPECT(sp.rcpw == 10 && (sp.rchunks + sp.rcpw - 1) / sp.rcpw * 16 <= 256);   // one workgroup per CU at most
  {
    SamplePlan s1;
    EXPECT(plan_sample(2 * 32, 1, 151936, &s1) && s1.rchunks == 149 && s1.rcpw == 1);
    EXPECT(plan_sample(2 * 32, 0, 151936, &s1) && s1.rchunks == 0 && s1.rcpw == 1);
  }
  EXPECT(sp.cs_off >= size_t(1024) * 75 * 4 && sp.gs_off >= sp.gm_off + size_t(1024) * 19 * 4);
  EXPECT(sp.rs_off + size_t(16) * sp.rchunks * 8 <= sp.ws_bytes);
  EXPECT(plan_sample(1, 0, 4200000, &sp) && sp.nchunks == 4102 && sp.ngroups == 1026);
  EXPECT(plan_sample(7, 0, 1000, &sp) && sp.nchunks == 1 && sp.ngroups == 1);
  // at most 2^30 (row, chunk) cells per call
  EXPECT(check_sample(reinterpret_cast<const float*>(P), 65535, 1 << 26, 1.0f, reinterpret_cast<const float*>(P), I, P, size_t(1) << 50, &sp, &err) == ORTHRUS_ERR_UNSUPPORTED_SHAPE);
  EXPECT(check_sample(reinterpret_cast<const float*>(P), 1024, 1 << 20, 1.0f, reinterpret_cast<const float*>(P), I, P, size_t(1) << 50, &sp, &err) == ORTHRUS_OK);
  EXPECT(check_sample(reinterpret_cast<const float*>(P), 1, kMaxVocab + 1, 1.0f, reinterpret_cast<const float*>(P), I, P, size_t(1) << 40, &sp, &err) == ORTHRUS_ERR_UNSUPPORTED_SHAPE);
  EXPECT(check_accept_sampled(reinterpret_cast<const float*>(P), reinterpret_cast<const float*>(P), I, 1, 32, kMaxVocab + 1, 1.0f, reinterpret_cast<const float*>(P), reinterpret_cast<const float*>(P), I, I, I, I, P, size_t(1) << 40, &sp, &err) == ORTHRUS_ERR_UNSUPPORTED_SHAPE);

  int32_t* O = reinterpret_cast<int32_t*>(uintptr_t(0x30000));
  const int64_t pool = int64_t(4096) * 8 * 16 * 128;
  EXPECT(check_commit(&kv, 2, pool, P, P, 32 * 8 * 128, I, 1, 32, O, &err) == ORTHRUS_OK);
  EXPECT(check_commit(&kv, 2, pool - 1, P, P, 32 * 8 * 128, I, 1, 32, O, &err) == ORTHRUS_ERR_INVALID_ARG);
  EXPECT(check_commit(&kv, 1, 0, P, P, 0, I, 1, 32, const_cast<int32_t*>(I), &err) == ORTHRUS_ERR_INVALID_ARG);
  EXPECT(check_commit(&kv, 0, 0, P, P, 0, I, 1, 32, O, &err) == ORTHRUS_ERR_INVALID_ARG);

  for (int s : {0, -1, -2, -3, -4, -5, -99}) EXPECT(std::string(status_string(s)).rfind("ORTHRUS_", 0) == 0);

  // the sampling kernels' 2^(t/64) for t <= 0: within 2 ulp of the C
  // library's exp2 on a dense grid of [-69300, 0] plus landmarks (0, the
  // table and rounding boundaries n + 1/2, the underflow region), exactly 0
  // far below; the table is 2^(j/64) to within half an ulp of exp2; and
  // e^x through t = x * 64/ln2 stays within 2^-51 (1 + |x|) (relative) of exp
  {
    for (int j = 0; j < 64; ++j) {
      const double want = std::exp2(j / 64.0);
      EXPECT(std::fabs(kExp2Frac[j] - want) <= 0.5 * (std::nextafter(want, 4.0) - want));
    }
    double worst = 0.0;
    auto check = [&](double t) {
      const double got = exp2_64(t, kExp2Frac), want = std::exp2(t / 64.0);
      if (want < 0x1p-1022) { EXPECT(std::fabs(got - want) <= 0x1p-1070); return; }
      const double ulp = std::nextafter(want, 1e300) - want;
      worst = std::max(worst, std::fabs(got - want) / ulp);
    };
    for (int i = 0; i <= 4000000; ++i) check(-69300.0 * i / 4000000.0);
    for (int n = -70000; n <= 0; n += 7) {         // around the rounding boundaries n + 1/2
      check(n + 0.5);
      check(std::nextafter(n + 0.5, 0.0));
      check(std::nextafter(n + 0.5, -1e9));
      check(double(n));
    }
    for (double t : {0.0, -0.0, -1e-300, -1e-17, -65000.0, -65472.0, -68800.0, -69300.0})
      check(t);
    EXPECT(exp2_64(-1e30, kExp2Frac) == 0.0 && exp2_64(-80000.0, kExp2Frac) == 0.0);
    EXPECT(exp2_64(0.0, kExp2Frac) == 1.0);
    EXPECT(worst <= 2.0);
    double worst_x = 0.0;
    for (int i = 1; i <= 200000; ++i) {
      const double x = -700.0 * i / 200000.0, want = std::exp(x);
      worst_x = std::max(worst_x, std::fabs(exp2_64(x * kExp2Scale, kExp2Frac) - want) / (want * (1.0 - x)));
    }
    EXPECT(worst_x <= 0x1p-51);
    std::printf("exp2_64: worst %.2f ulp; e^x via t: %.3g (1 + |x|) relative\n", worst, worst_x);
  }
  std::printf("%s (%d failures)\n", failures ? "FAIL" : "OK", failures);
  return failures ? 1 : 0;
}

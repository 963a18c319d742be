// Host-only driver for the C-ABI argument checks (built with g++ and the
// address/undefined-behaviour sanitizers by tests/test_abi_cpu.py; no HIP).
#include <cstdio>
#include <cstdint>
#include <string>

#include "check.h"

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
  EXPECT(plan_argmax(32, 151936, &ap) && ap.chunk % 4 == 0 && int64_t(ap.chunk) * ap.nchunks >= 151936);
  EXPECT(check_argmax(reinterpret_cast<const float*>(P), 32, 151936, I, P, ap.ws_bytes, &ap, &err) == ORTHRUS_OK);
  EXPECT(check_argmax(reinterpret_cast<const float*>(P), 32, 151936, I, P, 8, &ap, &err) == ORTHRUS_ERR_WORKSPACE_TOO_SMALL);
  EXPECT(check_argmax(reinterpret_cast<const float*>(P), 32, 0, I, P, 1 << 20, &ap, &err) == ORTHRUS_ERR_INVALID_ARG);
  EXPECT(check_argmax(nullptr, 0, 10, nullptr, nullptr, 0, &ap, &err) == ORTHRUS_OK);
  EXPECT(check_accept(reinterpret_cast<const float*>(P), I, 1, 32, 1024, const_cast<int32_t*>(I), const_cast<int32_t*>(I), const_cast<int32_t*>(I), nullptr, P, 1 << 20, &ap, &err) == ORTHRUS_ERR_INVALID_ARG);
  EXPECT(check_accept(reinterpret_cast<const float*>(P), I, 1, 65, 1024, const_cast<int32_t*>(I), const_cast<int32_t*>(I), const_cast<int32_t*>(I), const_cast<int32_t*>(I), P, 1 << 20, &ap, &err) == ORTHRUS_ERR_UNSUPPORTED_SHAPE);

  // LM head: rows kernel up to 64 rows; one row tile (up to 128 rows): GEMM
  // over contiguous vocabulary ranges; above, the GEMM tile whose workgroups
  // fill rounds of 256 CUs better (wide tiles cost ~1.87x a narrow one)
  LmHeadPlan lp;
  EXPECT(plan_lmhead(32, 4096, 151936, &lp, nullptr) && lp.gemm == 0 && lp.nwg == 256 && lp.nrc == 1);
  EXPECT(plan_lmhead(64, 4096, 151936, &lp, nullptr) && lp.gemm == 0 && lp.nrc == 2);
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

  // sampling statistics: chunks of 4096..16384 entries; 1 x 4.2 M words makes
  // 1026 chunks (more than the fused draw's 1024)
  SamplePlan sp;
  EXPECT(plan_sample(32, 0, 151936, &sp) && sp.chunk == 4096 && sp.nchunks == 38);
  EXPECT(plan_sample(1, 0, 4200000, &sp) && sp.chunk == 4096 && sp.nchunks == 1026);
  EXPECT(plan_sample(2, 0, 4200000, &sp) && sp.chunk <= kSampleMaxChunk && sp.nchunks <= 1024);

  int32_t* O = reinterpret_cast<int32_t*>(uintptr_t(0x30000));
  const int64_t pool = int64_t(4096) * 8 * 16 * 128;
  EXPECT(check_commit(&kv, 2, pool, P, P, 32 * 8 * 128, I, 1, 32, O, &err) == ORTHRUS_OK);
  EXPECT(check_commit(&kv, 2, pool - 1, P, P, 32 * 8 * 128, I, 1, 32, O, &err) == ORTHRUS_ERR_INVALID_ARG);
  EXPECT(check_commit(&kv, 1, 0, P, P, 0, I, 1, 32, const_cast<int32_t*>(I), &err) == ORTHRUS_ERR_INVALID_ARG);
  EXPECT(check_commit(&kv, 0, 0, P, P, 0, I, 1, 32, O, &err) == ORTHRUS_ERR_INVALID_ARG);

  for (int s : {0, -1, -2, -3, -4, -5, -99}) EXPECT(std::string(status_string(s)).rfind("ORTHRUS_", 0) == 0);
  std::printf("%s (%d failures)\n", failures ? "FAIL" : "OK", failures);
  return failures ? 1 : 0;
}

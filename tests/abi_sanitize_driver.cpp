// Host-only driver for the sanitizer build of the C ABI (tests/test_abi_cpu.py):
// every entry point is called with arguments that its validation must reject
// before touching HIP, and every workspace-size query with ordinary and extreme
// shapes.  Built with AddressSanitizer and UndefinedBehaviorSanitizer on the
// host code (no GPU is used); a sanitizer report aborts the run.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "../include/lsi.h"

static int g_fail = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      std::printf("FAILED: %s (line %d): %s\n", #cond, __LINE__,        \
                  lsi_last_error_detail());                            \
      ++g_fail;                                                        \
    }                                                                  \
  } while (0)

static void* P(uintptr_t v) { return reinterpret_cast<void*>(v); }

int main() {
  lsi_batch b{1, 4, 256, 0, static_cast<const int32_t*>(P(0x1000)), static_cast<const int32_t*>(P(0x2000))};
  lsi_paged_cache k8{LSI_FP8_E4M3, 64, 8, 128, P(0x4000), static_cast<const float*>(P(0x3000))};
  lsi_paged_cache k4{LSI_INT4, 64, 8, 128, P(0x4000), static_cast<const float*>(P(0x3000))};
  lsi_paged_cache kv{LSI_BF16, 64, 8, 576, P(0x4000), nullptr};

  // indexer scan
  EXPECT(lsi_index_scores(nullptr, &b, P(0x5000), 64, 128, static_cast<const float*>(P(0x6000)),
                          static_cast<float*>(P(0x7000)), 256, nullptr) == LSI_ERR_INVALID_ARG);
  EXPECT(lsi_index_scores(&k8, nullptr, P(0x5000), 64, 128, static_cast<const float*>(P(0x6000)),
                          static_cast<float*>(P(0x7000)), 256, nullptr) == LSI_ERR_INVALID_ARG);
  EXPECT(lsi_index_scores(&k8, &b, P(0x5000), 32, 128, static_cast<const float*>(P(0x6000)),
                          static_cast<float*>(P(0x7000)), 256, nullptr) == LSI_ERR_UNSUPPORTED);
  EXPECT(lsi_index_scores(&k8, &b, P(0x5000), 64, 128, static_cast<const float*>(P(0x6000)),
                          static_cast<float*>(P(0x7000)), 100, nullptr) == LSI_ERR_INVALID_ARG);
  lsi_batch big = b;
  big.max_seq_len = INT32_MAX;
  EXPECT(lsi_index_scores(&k8, &big, P(0x5000), 64, 128, static_cast<const float*>(P(0x6000)),
                          static_cast<float*>(P(0x7000)), INT64_MAX, nullptr) == LSI_ERR_INVALID_ARG);
  lsi_paged_cache huge = k8;
  huge.num_pages = INT32_MAX;
  EXPECT(lsi_index_scores(&huge, &b, P(0x5000), 64, 128, static_cast<const float*>(P(0x6000)),
                          static_cast<float*>(P(0x7000)), 256, nullptr) == LSI_ERR_INVALID_ARG);

  // top-k
  const size_t tk = lsi_topk_workspace_bytes(2, 1000, 64);
  EXPECT(tk > 0 && tk % 256 == 0);
  EXPECT(lsi_topk(static_cast<const float*>(P(0x1000)), 1000, &b, 0, static_cast<int32_t*>(P(0x2000)),
                  static_cast<int32_t*>(P(0x3000)), P(0x100000), tk, nullptr) == LSI_ERR_INVALID_ARG);
  EXPECT(lsi_topk(static_cast<const float*>(P(0x1000)), 1000, &b, 64, static_cast<int32_t*>(P(0x2000)),
                  static_cast<int32_t*>(P(0x3000)), P(0x100010), tk, nullptr) == LSI_ERR_WORKSPACE);
  EXPECT(lsi_topk(static_cast<const float*>(P(0x1000)), 1000, &b, 70000, static_cast<int32_t*>(P(0x2000)),
                  static_cast<int32_t*>(P(0x3000)), P(0x100000), tk, nullptr) == LSI_ERR_INVALID_ARG);

  // attention
  EXPECT(lsi_sparse_mla_decode(&kv, nullptr, &b, P(0x5000), 72, 576, 512, static_cast<const int32_t*>(P(0x6000)),
                               2048, 0.04f, P(0x7000), static_cast<float*>(P(0x8000)), P(0x100000), 1u << 30,
                               nullptr) == LSI_ERR_UNSUPPORTED);
  EXPECT(lsi_sparse_mla_decode(&kv, nullptr, &b, P(0x5000), 128, 576, 512, static_cast<const int32_t*>(P(0x6000)),
                               2048, -1.0f, P(0x7000), static_cast<float*>(P(0x8000)), P(0x100000), 1u << 30,
                               nullptr) == LSI_ERR_INVALID_ARG);

  // decode step (workspace and no-allocation variants)
  EXPECT(lsi_decode_step(&k8, &kv, nullptr, &b, P(0x5000), 64, 128, static_cast<const float*>(P(0x6000)),
                         P(0x7000), 128, 576, 512, 0.04f, 2048, static_cast<int32_t*>(P(0x8000)),
                         static_cast<int32_t*>(P(0x9000)), P(0xA000), static_cast<float*>(P(0xB000)), nullptr,
                         0, nullptr) == LSI_ERR_WORKSPACE);
  lsi_batch wide{64, 4688, 300000, 0, static_cast<const int32_t*>(P(0x1000)), static_cast<const int32_t*>(P(0x2000))};
  EXPECT(lsi_decode_step_noalloc(&k8, &kv, nullptr, &wide, P(0x5000), 64, 128,
                                 static_cast<const float*>(P(0x6000)), P(0x7000), 128, 576, 512, 0.04f, 2048,
                                 static_cast<int32_t*>(P(0x8000)), static_cast<int32_t*>(P(0x9000)), P(0xA000),
                                 static_cast<float*>(P(0xB000)), nullptr) == LSI_ERR_WORKSPACE);

  // two-stage search and prefill chunk
  EXPECT(lsi_two_stage_topk(&k8, &k4, &b, P(0x5000), 64, 128, static_cast<const float*>(P(0x6000)), 200, 100,
                            static_cast<int32_t*>(P(0x7000)), static_cast<int32_t*>(P(0x8000)), nullptr,
                            P(0x100000), 1u << 30, nullptr) == LSI_ERR_INVALID_ARG);
  EXPECT(lsi_prefill_index_topk(nullptr, nullptr, 10, static_cast<const uint8_t*>(P(0x1000)),
                                static_cast<const float*>(P(0x2000)), 4, P(0x3000), 64, 128,
                                static_cast<const float*>(P(0x4000)), 16, 32, static_cast<int32_t*>(P(0x5000)),
                                static_cast<int32_t*>(P(0x6000)), nullptr, P(0x100000), 1u << 30, nullptr,
                                nullptr) == LSI_ERR_INVALID_ARG);
  EXPECT(lsi_prefill_index_topk(nullptr, nullptr, 0, static_cast<const uint8_t*>(P(0x1000)),
                                static_cast<const float*>(P(0x2000)), INT32_MAX, P(0x3000), 64, 128,
                                static_cast<const float*>(P(0x4000)), 16, 32, static_cast<int32_t*>(P(0x5000)),
                                static_cast<int32_t*>(P(0x6000)), nullptr, P(0x100000), 1u << 30, nullptr,
                                nullptr) != LSI_OK);

  // several layers
  const void* arr[4] = {P(0x10000), P(0x10100), P(0x10200), P(0x10300)};
  lsi_paged_cache ik4[4] = {k8, k8, k8, k8};
  lsi_paged_cache kv4[4] = {kv, kv, kv, kv};
  EXPECT(lsi_multilayer_decode(0, 1, LSI_SCHED_MLI, ik4, kv4, &b, arr, 64, 128,
                               reinterpret_cast<const float* const*>(arr), arr, 128, 576, 512, 0.04f, 64,
                               reinterpret_cast<int32_t* const*>(const_cast<void**>(arr)),
                               reinterpret_cast<int32_t* const*>(const_cast<void**>(arr)),
                               const_cast<void* const*>(arr), reinterpret_cast<float* const*>(const_cast<void**>(arr)),
                               P(0x100000), 1u << 30, nullptr, nullptr) == LSI_ERR_INVALID_ARG);

  // workspace sizes: ordinary, extreme and invalid shapes (no overflow, no UB)
  const int32_t lens[] = {0, 1, 63, 64, 4096, 131072, 524288, 1 << 24, INT32_MAX};
  for (int32_t L : lens) {
    for (int32_t R : {1, 2, 64, 1024}) {
      (void)lsi_topk_workspace_bytes(R, L, 2048);
      (void)lsi_decode_step_workspace_bytes(R, L, 2048, 128, 512);
      (void)lsi_multilayer_workspace_bytes(R, L, 2048, 128, 512);
      (void)lsi_two_stage_workspace_bytes(R, L, 8192, 2048);
      (void)lsi_sparse_mla_workspace_bytes(R, 128, 512, 2048);
      (void)lsi_decode_step_state_bytes(R);
    }
    (void)lsi_prefill_workspace_bytes(L, 4096, 128, 8192, 2048, 0);
  }
  EXPECT(lsi_topk_workspace_bytes(0, 100, 10) == 0);
  EXPECT(lsi_decode_step_workspace_bytes(1, -5, 2048, 128, 512) == 0);
  lsi_ws_query q;
  std::memset(&q, 0, sizeof(q));
  q.num_req = 1;
  q.max_seq_len = 131072;
  q.k = 2048;
  q.n_heads = 128;
  q.dv = 512;
  q.n_cand = 8192;
  q.dim = 128;
  q.block_tokens = 8192;
  for (int32_t op = -1; op <= 8; ++op) (void)lsi_workspace_bytes(op, &q);
  EXPECT(lsi_workspace_bytes(LSI_OP_DECODE_STEP, &q) == lsi_decode_step_workspace_bytes(1, 131072, 2048, 128, 512));
  EXPECT(lsi_workspace_bytes(LSI_OP_TOPK, nullptr) == 0);
  for (int32_t st = -3; st <= 8; ++st) EXPECT(lsi_status_string(st) != nullptr);
  EXPECT(lsi_last_error_detail() != nullptr);
  EXPECT(lsi_profile_events(nullptr, nullptr, 0) == 0);

  std::printf("%s (%d failures)\n", g_fail ? "FAILED" : "sanitized ABI checks passed", g_fail);
  return g_fail ? 1 : 0;
}

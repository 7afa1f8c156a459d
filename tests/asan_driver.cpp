// Host-side driver for the sanitizer test: exercises every entry point of
// the C ABI along its host-only paths (planning, argument validation, status
// strings, error messages, timing records) with no device work, so that an
// AddressSanitizer / UndefinedBehaviorSanitizer build of the host code can
// check them on a machine without a GPU.  Prints "ok" and returns 0 when every
// call returns the expected status.
#include <cmath>
#include <cstdio>
#include <cstring>

#include "kdloss.h"

static int g_fail = 0;

static void expect(int got, int want, const char* what) {
  if (got != want) {
    std::printf("FAIL %s: got %d want %d (%s)\n", what, got, want, kd_last_error_message());
    g_fail = 1;
  }
}

int main() {
  const size_t budget = size_t(64) << 30;
  kd_plan_t p;
  std::memset(&p, 0, sizeof(p));
  // planner: the 32K workload, every dtype, explicit and automatic chunks
  expect(kd_plan_query(KD_BF16, 32768, 2880, 201088, 100, 0, budget, &p), KD_OK, "plan bf16 32K");
  if (p.chunk != 8192 || p.n_chunks != 4 || p.workspace_bytes < p.fwd_workspace_bytes) {
    std::printf("FAIL plan fields: chunk %lld n_chunks %lld\n", (long long)p.chunk, (long long)p.n_chunks);
    g_fail = 1;
  }
  expect(kd_plan_query(KD_F32, 256, 256, 4096, 16, 64, budget, &p), KD_OK, "plan f32 tiny");
  expect(kd_plan_query(KD_BF16, 262144, 3072, 128256, 100, 0, budget, &p), KD_OK, "plan 256K");
  expect(kd_plan_query(KD_BF16, 1, 64, 100, 100, 0, budget, &p), KD_OK, "plan one row, K = V");
  // planner rejections
  expect(kd_plan_query(KD_BF16, 32768, 2880, 201088, 100, 0, 1 << 20, &p), KD_E_WORKSPACE, "tiny budget");
  if (std::strlen(kd_last_error_message()) == 0) {
    std::printf("FAIL empty message after KD_E_WORKSPACE\n");
    g_fail = 1;
  }
  expect(kd_plan_query(7, 256, 256, 4096, 16, 0, budget, &p), KD_E_INVAL, "bad dtype");
  expect(kd_plan_query(KD_BF16, 0, 256, 4096, 16, 0, budget, &p), KD_E_INVAL, "n = 0");
  expect(kd_plan_query(KD_BF16, 256, 0, 4096, 16, 0, budget, &p), KD_E_INVAL, "d = 0");
  expect(kd_plan_query(KD_BF16, 256, 256, 16, 17, 0, budget, &p), KD_E_INVAL, "K > V");
  expect(kd_plan_query(KD_BF16, 256, 256, 4096, 0, 0, budget, &p), KD_E_INVAL, "K = 0");
  expect(kd_plan_query(KD_BF16, 1000, 256, 4096, 16, 100, budget, &p), KD_E_INVAL, "ragged chunk");
  expect(kd_plan_query(KD_BF16, 256, 256, 4096, 16, 0, budget, nullptr), KD_E_INVAL, "null plan");
  expect(kd_plan_query(KD_BF16, 256, 256, 4096, 16, 0, budget, &p), KD_OK, "plan after failures");
  if (std::strlen(kd_last_error_message()) != 0) {
    std::printf("FAIL message not cleared by a successful call\n");
    g_fail = 1;
  }

  // loss calls (explicit chunk, so the plan itself succeeds): null pointers
  // and bad temperatures are rejected before any device work
  alignas(16) float dummy[4] = {0.f, 0.f, 0.f, 0.f};
  alignas(16) int idx[4] = {0, 1, 2, 3};
  alignas(16) char ws[256];
  expect(kd_fused_chunked_kl_fwd(KD_BF16, nullptr, dummy, idx, dummy, nullptr, 256, 256, 4096, 16, 256, 1.f,
                                 ws, sizeof(ws), dummy, dummy, nullptr, nullptr, nullptr),
         KD_E_INVAL, "fwd null H");
  expect(kd_fused_chunked_kl_fwd(KD_BF16, dummy, dummy, idx, dummy, nullptr, 256, 256, 4096, 16, 256, 1.f,
                                 ws, sizeof(ws), nullptr, dummy, nullptr, nullptr, nullptr),
         KD_E_INVAL, "fwd null loss");
  const float bad_tau[3] = {0.f, -1.f, std::nanf("")};
  for (float tau : bad_tau)
    expect(kd_fused_chunked_kl_fwd(KD_BF16, dummy, dummy, idx, dummy, nullptr, 256, 256, 4096, 16, 256, tau,
                                   ws, sizeof(ws), dummy, dummy, nullptr, nullptr, nullptr),
           KD_E_INVAL, "fwd bad temperature");
  expect(kd_fused_chunked_kl_bwd(KD_BF16, dummy, dummy, idx, dummy, nullptr, 256, 256, 4096, 16, 256, 1.f,
                                 nullptr, dummy, dummy, dummy, 0, ws, sizeof(ws), nullptr),
         KD_E_INVAL, "bwd null lse");
  expect(kd_fused_chunked_kl_bwd(KD_BF16, dummy, dummy, idx, dummy, nullptr, 256, 256, 4096, 16, 256,
                                 INFINITY, dummy, dummy, dummy, dummy, 0, ws, sizeof(ws), nullptr),
         KD_E_INVAL, "bwd infinite temperature");

  // cache builder
  kd_topk_plan_t tp;
  expect(kd_teacher_topk_plan(KD_BF16, 32768, 2880, 201088, 100, 0, 0, budget, &tp), KD_OK, "topk plan");
  expect(kd_teacher_topk_plan(KD_BF16, 32768, 2880, 201088, 100, 0, 50, budget, &tp), KD_E_INVAL, "cap < K");
  expect(kd_teacher_topk_plan(KD_BF16, 256, 256, 4096, 5000, 0, 0, budget, &tp), KD_E_INVAL, "K > V");
  expect(kd_teacher_topk(KD_BF16, nullptr, dummy, 256, 256, 4096, 16, 256, 0, ws, sizeof(ws), idx, dummy,
                         nullptr),
         KD_E_INVAL, "topk null Ht");

  // comparison variants: grid sizes, refusals before any device work
  if (kd_comparator_grid_bytes(KD_VARIANT_DENSE, 256, 4096) != 2 * kd_comparator_grid_bytes(KD_VARIANT_FORWARD_CHUNKED, 256, 4096) ||
      kd_comparator_grid_bytes(3, 256, 4096) != 0 || kd_comparator_grid_bytes(KD_VARIANT_DENSE, 0, 4096) != 0) {
    std::printf("FAIL comparator grid bytes\n");
    g_fail = 1;
  }
  expect(kd_dense_kl_fwd(KD_F32, dummy, dummy, idx, dummy, nullptr, 256, 256, 4096, 16, 64, ws, sizeof(ws), ws,
                         sizeof(ws), dummy, dummy, nullptr, nullptr),
         KD_E_INVAL, "dense fwd fp32");
  expect(kd_forward_chunked_kl_fwd(KD_BF16, dummy, dummy, idx, dummy, nullptr, 256, 256, 4096, 16, 64, ws,
                                   sizeof(ws), ws, sizeof(ws), dummy, dummy, nullptr, nullptr),
         KD_E_WORKSPACE, "forward-chunked fwd small workspace");
  expect(kd_dense_kl_bwd(KD_BF16, dummy, dummy, idx, dummy, nullptr, 256, 256, 4096, 16, 64, nullptr, 0, dummy,
                         dummy, dummy, dummy, 0, ws, sizeof(ws), nullptr),
         KD_E_WORKSPACE, "dense bwd small workspace");
  // the no-allocation forward: a problem beyond its scratch is refused before any device work
  expect(kd_fused_chunked_kl_fwd_noalloc(KD_BF16, dummy, dummy, idx, dummy, nullptr, 262144, 3072, 128256, 100, 0,
                                         1.f, dummy, dummy, nullptr, nullptr, nullptr),
         KD_E_WORKSPACE, "no-alloc fwd beyond scratch");
  expect(kd_fused_chunked_kl_fwd_noalloc(KD_BF16, dummy, dummy, idx, dummy, nullptr, 256, 256, 4096, 16, 64, 1.f,
                                         nullptr, dummy, nullptr, nullptr, nullptr),
         KD_E_INVAL, "no-alloc fwd null loss");

  // status strings, validation switch, timing records
  for (int s = -6; s <= 2; ++s)
    if (kd_status_string(s) == nullptr || std::strlen(kd_status_string(s)) == 0) {
      std::printf("FAIL status string %d\n", s);
      g_fail = 1;
    }
  expect(kd_set_validate(1), KD_OK, "validate on");
  expect(kd_set_validate(0), KD_OK, "validate off");
  expect(kd_profile_enable(1), KD_OK, "profile on");
  expect(kd_profile_reset(), KD_OK, "profile reset");
  expect(kd_profile_read(nullptr, 0), 0, "profile count");
  kd_kernel_stat_t st[2];
  expect(kd_profile_read(st, 2), 0, "profile read");
  expect(kd_profile_enable(0), KD_OK, "profile off");

  if (g_fail) return 1;
  std::printf("ok\n");
  return 0;
}

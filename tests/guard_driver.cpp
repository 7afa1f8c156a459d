// Host-only driver of the dH launch bounds check: every call below is refused
// before anything is launched, or is a pure check, so it runs on a machine
// without a GPU.  Prints "ok" and returns 0 when every case gives the
// expected answer.
#include <cstdio>

#include "kd_internal.h"

static int g_fail = 0;

static void expect_ok(const char* why, const char* what) {
  if (why != nullptr) {
    std::printf("FAIL %s: refused (%s)\n", what, why);
    g_fail = 1;
  }
}

static void expect_refused(const char* why, const char* what) {
  if (why == nullptr) {
    std::printf("FAIL %s: accepted\n", what);
    g_fail = 1;
  }
}

int main() {
  using kd::DType;
  // the 32K workload's dH launch: 8192 rows, V padded to 201088, d = 2880, 2 splits
  const int rows = 8192, v_pad = 201088, d = 2880;
  const long long stride = (long long)rows * d;
  const size_t part2 = size_t(2) * stride * 4;
  expect_ok(kd::dh_launch_error(DType::BF16, rows, v_pad, d, 2, stride, part2), "planned launch");
  expect_ok(kd::dh_launch_error(DType::BF16, 700, 1024, 320, 1, 700LL * 320, 700 * 320 * 4), "one split");
  // the record of a past harness fault: a grid of 768 splits against a
  // partials buffer sized for a few of them
  expect_refused(kd::dh_launch_error(DType::BF16, rows, v_pad, d, 768, stride, size_t(8) * stride * 4),
                 "768 splits, partials for 8");
  expect_refused(kd::dh_launch_error(DType::BF16, rows, v_pad, d, 3, stride, part2), "3 splits, partials for 2");
  // more splits than K blocks (64 bf16 / 32 fp32 per block)
  expect_refused(kd::dh_launch_error(DType::BF16, 64, 128, 64, 3, 64 * 64, size_t(1) << 20), "3 splits of 2 blocks");
  expect_ok(kd::dh_launch_error(DType::F32, 64, 128, 64, 4, 64 * 64, size_t(1) << 20), "4 splits of 4 fp32 blocks");
  // a split left empty by the rounding of the blocks per split (10 blocks, 4 splits of 3)
  expect_ok(kd::dh_launch_error(DType::BF16, 64, 640, 64, 4, 64 * 64, size_t(1) << 20), "10 blocks, 4 splits");
  expect_refused(kd::dh_launch_error(DType::BF16, 64, 640, 64, 6, 64 * 64, size_t(1) << 20), "10 blocks, 6 splits");
  expect_refused(kd::dh_launch_error(DType::BF16, 64, 640, 64, 0, 64 * 64, size_t(1) << 20), "0 splits");
  // a partial larger than its stride (splits would overlap)
  expect_refused(kd::dh_launch_error(DType::BF16, 128, 640, 64, 2, 64 * 64, size_t(1) << 20), "stride too small");
  // the launcher itself refuses and launches nothing (no device is touched)
  float* part = reinterpret_cast<float*>(4096);
  const void* g = reinterpret_cast<const void*>(4096);
  if (kd::launch_dh_gemm(DType::BF16, g, rows, v_pad, g, true, v_pad, d, 768, part, stride,
                         size_t(8) * stride * 4, nullptr)) {
    std::printf("FAIL launcher accepted 768 splits\n");
    g_fail = 1;
  }
  if (g_fail) return 1;
  std::printf("ok\n");
  return 0;
}

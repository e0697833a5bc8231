// CPU-only checks of the library's host layer, built with AddressSanitizer
// and UndefinedBehaviorSanitizer against the stand-in device side: a launch
// failure reaches the caller as MOE_ERR_HIP with the call named in the
// detail; an error left pending by an earlier device call of the caller is
// dropped before the launch, not reported as this call's; nothing is
// launched when validation fails; the error detail is per thread.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <thread>

#include "moe_qexpert.h"
#include "stub_device.h"

static int failures = 0;
#define CHECK(cond)                                                    \
  do {                                                                 \
    if (!(cond)) {                                                     \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

static void* fake(uintptr_t a) { return reinterpret_cast<void*>(a); }

static moe_status route() {
  return moe_route_topk(static_cast<const float*>(fake(0x1000)), 4, 8, 2, static_cast<int32_t*>(fake(0x2000)),
                        static_cast<float*>(fake(0x3000)), nullptr);
}

static moe_wdesc int4_desc() {
  moe_wdesc d;
  memset(&d, 0, sizeof(d));
  d.abi_version = MOE_ABI_VERSION;
  d.format = MOE_W_INT4_GROUP;
  d.layout = MOE_LAYOUT_TILED;
  d.E = 8;
  d.N = 256;
  d.K = 512;
  d.group_size = 128;
  d.zero_point = 8;
  d.codes = static_cast<const uint8_t*>(fake(0x10000));
  d.scales = static_cast<const uint16_t*>(fake(0x20000));
  return d;
}

static moe_status gemm(const moe_wdesc& d, int rows, int M, void* ws, size_t ws_bytes, int kernel) {
  return moe_grouped_qgemm(&d, static_cast<const uint16_t*>(fake(0x1000)), rows,
                           static_cast<const int32_t*>(fake(0x2000)), 2, static_cast<const int32_t*>(fake(0x3000)),
                           M, MOE_EPI_SWIGLU, kernel, fake(0x4000), ws, ws_bytes, nullptr);
}

int main() {
  // a launch that fails: MOE_ERR_HIP, the detail names the call and the device's message
  stub::launch_error = 98;
  CHECK(route() == MOE_ERR_HIP);
  CHECK(strstr(moe_last_error_detail(), "route_topk") != nullptr);
  CHECK(strstr(moe_last_error_detail(), "stub device error") != nullptr);
  stub::launch_error = 0;
  CHECK(route() == MOE_OK);
  CHECK(moe_last_error_detail()[0] == '\0');

  // an error left pending by the caller is dropped before the launch
  stub::pending_error = 700;
  const int taken0 = stub::taken, launches0 = stub::launches;
  CHECK(route() == MOE_OK);
  CHECK(stub::pending_error == 0 && stub::taken == taken0 + 1 && stub::launches == launches0 + 1);

  // validation failures launch nothing and do not touch the pending error
  stub::pending_error = 5;
  const int launches1 = stub::launches;
  CHECK(moe_route_topk(nullptr, 4, 8, 2, nullptr, nullptr, nullptr) == MOE_ERR_NULL_ARG);
  CHECK(moe_route_topk(static_cast<const float*>(fake(0x1000)), 4, 8, 9, static_cast<int32_t*>(fake(0x2000)),
                       static_cast<float*>(fake(0x3000)), nullptr) == MOE_ERR_BAD_SHAPE);
  moe_wdesc d = int4_desc();
  CHECK(gemm(d, 64, 128, nullptr, 0, 9) == MOE_ERR_BAD_FORMAT);
  CHECK(gemm(d, 64, 128, nullptr, 0, MOE_KERNEL_SMALL_PER_WIDTH) == MOE_ERR_UNSUPPORTED);
  CHECK(stub::launches == launches1 && stub::pending_error == 5);
  stub::pending_error = 0;

  // the grouped GEMM: workspace sized per kernel choice, a failing launch propagates
  const size_t need = moe_grouped_qgemm_workspace_size(&d, 4096, 8192, MOE_KERNEL_AUTO);
  CHECK(need == (size_t)4096 * (512 / 128) * 4);
  CHECK(moe_grouped_qgemm_workspace_size(&d, 4096, 8192, MOE_KERNEL_SMALL) == 0);
  CHECK(gemm(d, 4096, 8192, nullptr, 0, MOE_KERNEL_AUTO) == MOE_ERR_WORKSPACE_TOO_SMALL);
  CHECK(gemm(d, 4096, 8192, nullptr, 0, MOE_KERNEL_SMALL) == MOE_OK);
  stub::launch_error = 1;
  CHECK(gemm(d, 4096, 8192, fake(0x5000), need, MOE_KERNEL_AUTO) == MOE_ERR_HIP);
  CHECK(strstr(moe_last_error_detail(), "grouped_qgemm") != nullptr);
  stub::launch_error = 0;

  // the no-allocation variant: the static scratch stands in for the workspace;
  // a call needing more than it holds is refused before anything is launched
  CHECK(moe_grouped_qgemm_noalloc_scratch_bytes() == ((size_t)8 << 20));
  CHECK(moe_grouped_qgemm_noalloc(&d, static_cast<const uint16_t*>(fake(0x1000)), 4096,
                                  static_cast<const int32_t*>(fake(0x2000)), 2, static_cast<const int32_t*>(fake(0x3000)),
                                  8192, MOE_EPI_SWIGLU, MOE_KERNEL_AUTO, fake(0x4000), nullptr) == MOE_OK);
  CHECK(stub::last_ws == fake(0x7000000));
  const int launches3 = stub::launches;
  CHECK(moe_grouped_qgemm_noalloc(&d, static_cast<const uint16_t*>(fake(0x1000)), 1 << 20,
                                  static_cast<const int32_t*>(fake(0x2000)), 2, static_cast<const int32_t*>(fake(0x3000)),
                                  1 << 21, MOE_EPI_SWIGLU, MOE_KERNEL_AUTO, fake(0x4000), nullptr) == MOE_ERR_UNSUPPORTED);
  CHECK(strstr(moe_last_error_detail(), "static scratch") != nullptr);
  CHECK(stub::launches == launches3);

  // per-expert width tables are read (under the sanitizers) and checked
  int32_t bits[4] = {4, 2, 3, 2}, zero[4] = {8, 1, 3, 2};
  moe_wdesc m = int4_desc();
  m.format = MOE_W_INT_PER_EXPERT;
  m.E = 4;
  m.expert_bits = bits;
  m.expert_zero = zero;
  CHECK(gemm(m, 64, 128, nullptr, 0, MOE_KERNEL_AUTO) == MOE_OK);
  zero[1] = 4;
  CHECK(gemm(m, 64, 128, nullptr, 0, MOE_KERNEL_AUTO) == MOE_ERR_BAD_SHAPE);

  // the combine with its valid-row count
  CHECK(moe_unpermute_combine(fake(0x1000), MOE_DTYPE_F32, static_cast<const int32_t*>(fake(0x2000)),
                              static_cast<const int32_t*>(fake(0x3000)), nullptr, 4, 2, 16,
                              static_cast<uint16_t*>(fake(0x4000)), nullptr) == MOE_OK);

  // strided plane copies: argument checks before anything is queued, failures reported
  CHECK(moe_copy_rows_async(fake(0x1000), fake(0x2000), 0, 1024, 512, nullptr) == MOE_OK);  // nothing to do
  CHECK(stub::copies == 0);
  CHECK(moe_copy_rows_async(nullptr, fake(0x2000), 4, 1024, 512, nullptr) == MOE_ERR_NULL_ARG);
  CHECK(moe_copy_rows_async(fake(0x1000), fake(0x2000), 4, 256, 512, nullptr) == MOE_ERR_BAD_SHAPE);
  CHECK(stub::copies == 0);
  CHECK(moe_copy_rows_async(fake(0x1000), fake(0x2000), 4, 1024, 512, nullptr) == MOE_OK);
  CHECK(stub::copies == 1);
  stub::launch_error = 1;
  CHECK(moe_copy_rows_async(fake(0x1000), fake(0x2000), 4, 1024, 512, nullptr) == MOE_ERR_HIP);
  CHECK(strstr(moe_last_error_detail(), "copy_rows") != nullptr);
  stub::launch_error = 0;

  // the current-device query fails: MOE_ERR_HIP before any launch
  stub::device_error = 100;
  const int launches2 = stub::launches;
  CHECK(route() == MOE_ERR_HIP);
  CHECK(stub::launches == launches2);
  stub::device_error = 0;

  // another architecture: MOE_ERR_UNSUPPORTED (checked once per device and thread: a new thread)
  std::thread([] {
    stub::arch = "gfx942";
    CHECK(route() == MOE_ERR_UNSUPPORTED);
    CHECK(strstr(moe_last_error_detail(), "gfx942") != nullptr);
    stub::arch = "gfx950:sramecc+:xnack-";
  }).join();

  // the error detail is per thread
  CHECK(moe_route_topk(nullptr, 4, 8, 2, nullptr, nullptr, nullptr) == MOE_ERR_NULL_ARG);
  std::thread([] {
    CHECK(moe_last_error_detail()[0] == '\0');
    CHECK(route() == MOE_OK);
  }).join();
  CHECK(strstr(moe_last_error_detail(), "required") != nullptr);

  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("host layer checks passed\n");
  return 0;
}

// Stand-in device side for a CPU-only build of the library's host layer
// (abi.cpp + plan.cpp): the launchers and runtime queries of launch.h touch
// no device, count the launches, and return the errors a test sets.
#include <stdio.h>

#include "launch.h"
#include "stub_device.h"

namespace stub {
int launch_error = 0;
int pending_error = 0;
int device_error = 0;
int launches = 0;
int taken = 0;
const char* arch = "gfx950:sramecc+:xnack-";
void* last_ws = nullptr;
int copies = 0;
}  // namespace stub

namespace {
int launched() {
  ++stub::launches;
  return stub::launch_error;
}
}  // namespace

namespace moe {
int rt_current_device(int* dev) {
  if (stub::device_error) return stub::device_error;
  *dev = 0;
  return 0;
}
int rt_device_arch(int, char* name, size_t n) {
  snprintf(name, n, "%s", stub::arch);
  return 0;
}
int rt_take_error() {
  const int e = stub::pending_error;
  stub::pending_error = 0;
  ++stub::taken;
  return e;
}
const char* rt_error_string(int err) { return err ? "stub device error" : "no error"; }
int rt_copy_rows_h2d(void*, const void*, size_t, size_t, size_t, void*) {
  ++stub::copies;
  return stub::launch_error;
}

int launch_route_topk(const float*, int, int, int, int32_t*, float*, void*) { return launched(); }
int launch_permute(const PermuteArgs&, void*) { return launched(); }
int launch_route_permute(const float*, int, int, int, const uint8_t*, int32_t*, float*, int32_t*, int32_t*, int32_t*,
                         int32_t*, void*, void*) {
  return launched();
}
int launch_combine(const void*, int, const int32_t*, const int32_t*, const float*, int, int, int, uint16_t*, void*) {
  return launched();
}
int launch_qgemm(const QGemmArgs& a, void*) {
  stub::last_ws = a.ws;
  return launched();
}
int qgemm_static_scratch(void** ptr) {
  *ptr = reinterpret_cast<void*>(0x7000000);
  return 0;
}
int launch_repack(const QWeights&, const QWeights&, void*) { return launched(); }
}  // namespace moe

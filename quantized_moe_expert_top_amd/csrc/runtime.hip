// Device runtime queries of the host layer (abi.cpp), which itself builds
// without the HIP headers.
#include <string.h>

#include "common.h"

namespace moe {

int rt_current_device(int* dev) { return (int)hipGetDevice(dev); }

int rt_device_arch(int dev, char* name, size_t n) {
  hipDeviceProp_t prop;
  const hipError_t e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return (int)e;
  strncpy(name, prop.gcnArchName, n - 1);
  name[n - 1] = '\0';
  return 0;
}

int rt_take_error() { return (int)hipGetLastError(); }

const char* rt_error_string(int err) { return hipGetErrorString(static_cast<hipError_t>(err)); }

int rt_copy_rows_h2d(void* dst, const void* src, size_t rows, size_t pitch, size_t width, void* stream) {
  return (int)hipMemcpy2DAsync(dst, pitch, src, pitch, width, rows, hipMemcpyHostToDevice,
                               static_cast<hipStream_t>(stream));
}

}  // namespace moe

// Ceiling probes for the roofline figures: how fast this part streams HBM and
// issues bf16 MFMA when nothing else is asked of it.  They measure the
// machine, not the method; the benchmark reports every kernel's roofline
// fraction against these measured ceilings beside the vendor peaks.
//
//   moe_probe_stream_read  reads `bytes` once with 16-byte loads spread over
//                          the whole chip (grid-stride, 4 loads in flight per
//                          lane) and writes one word per workgroup so the
//                          loads cannot be dropped
//   moe_probe_mfma_loop    every wavefront runs `iters` rounds of 8
//                          independent v_mfma_f32_16x16x32_bf16 chains on
//                          register operands (no memory traffic)
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                          uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    const u32x4 b = __builtin_nontemporal_load(src + i + stride);
    const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3] ^ b[0] ^ b[1] ^ b[2] ^ b[3] ^ c[0] ^ c[1] ^ c[2] ^ c[3] ^ d[0] ^ d[1] ^ d[2] ^ d[3];
  }
  for (; i < n16; i += stride) {
    const u32x4 a = src[i];
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
  }
  __shared__ uint32_t red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t v = 0;
    for (int j = 0; j < 256; ++j) v ^= red[j];
    sink[blockIdx.x] = v;
  }
}

__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  u32x4 ar = {0x3F803F80u ^ (uint32_t)lane, 0x3F80BF80u, 0xBF803F80u, 0x3F803F80u};
  u32x4 br = {0x3F003F00u, 0x3F00BF00u ^ (uint32_t)lane, 0xBF003F00u, 0x3F003F00u};
  const bf16x8 a = __builtin_bit_cast(bf16x8, ar);
  const bf16x8 b = __builtin_bit_cast(bf16x8, br);
  f32x4 c[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) c[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c[j], 0, 0, 0);
  }
  f32x4 s = c[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) s += c[j];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s[0] + s[1] + s[2] + s[3];
}
}  // namespace

extern "C" {

// Streams `bytes` (a multiple of 16) from `src` once; `sink` holds one u32 per
// workgroup (`blocks` of them).  Returns a hipError_t.
int moe_probe_stream_read(const void* src, size_t bytes, uint32_t* sink, int blocks, void* stream) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(src), bytes / 16, sink);
  return (int)hipGetLastError();
}

// `blocks` workgroups of 4 wavefronts, each wavefront 8 * iters MFMAs of
// 16x16x32 (16384 flops each); `out` holds blocks * 256 floats.
int moe_probe_mfma_loop(int iters, int blocks, float* out, void* stream) {
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), iters, out);
  return (int)hipGetLastError();
}

}  // extern "C"

// Gate-weighted combine of each token's k expert outputs:
//   out[t] = sum_{j<k} w[t][j] * y_perm[pair_pos[t*k+j]]
// accumulated in fp32 in slot order and rounded once to bf16.  No atomics, so
// the result is bitwise reproducible.  One workgroup per token; each lane
// moves 8 outputs per row and slot (16 bytes of a 16-bit y, 32 of an fp32 one).  With `n_valid`, a pair whose
// grouped row lies at or past *n_valid (a pair the grouping flagged as
// invalid, whose row no GEMM wrote) adds nothing and its row is not read.
#include "common.h"

namespace moe {

namespace {
constexpr int kThreads = 256;

// YT: expert outputs in bf16 (0), fp32 (1, not rounded before the combine)
// or fp16 (2).  Slots are taken in batches of 8: all row loads of a batch are
// issued before the first multiply-add, in slot order.
__device__ __forceinline__ float f16_lo(uint32_t v) { return f16_to_f32((uint16_t)(v & 0xFFFFu)); }
__device__ __forceinline__ float f16_hi(uint32_t v) { return f16_to_f32((uint16_t)(v >> 16)); }
template <int YT>
__global__ __launch_bounds__(kThreads) void combine_kernel(const void* __restrict__ yv,
                                                           const int32_t* __restrict__ pos,
                                                           const int32_t* __restrict__ n_valid,
                                                           const float* __restrict__ w, int k, int H,
                                                           uint16_t* __restrict__ out) {
  constexpr int B = 8;
  const int t = blockIdx.x;
  const int nvec = H >> 3;
  const int nv = n_valid ? *n_valid : 0x7FFFFFFF;
  for (int c = threadIdx.x; c < nvec; c += kThreads) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < k; j0 += B) {
      f32x4 v[B][2];
      float g[B];
#pragma unroll
      for (int i = 0; i < B; ++i) {
        const int j = j0 + i;
        g[i] = 0.f;
        v[i][0] = v[i][1] = f32x4{};
        const int p = j < k ? pos[(size_t)t * k + j] : nv;
        if (p < nv) {
          g[i] = w ? w[(size_t)t * k + j] : 1.0f;
          if (YT == 1) {
            const f32x4* row = reinterpret_cast<const f32x4*>(static_cast<const float*>(yv) + (size_t)p * H);
            v[i][0] = row[2 * c];
            v[i][1] = row[2 * c + 1];
          } else {
            const u32x4 b = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(yv) + (size_t)p * H)[c];
#pragma unroll
            for (int q = 0; q < 2; ++q)
              v[i][q] = YT == 2 ? f32x4{f16_lo(b[2 * q]), f16_hi(b[2 * q]), f16_lo(b[2 * q + 1]), f16_hi(b[2 * q + 1])}
                                : f32x4{bf16_lo(b[2 * q]), bf16_hi(b[2 * q]), bf16_lo(b[2 * q + 1]), bf16_hi(b[2 * q + 1])};
          }
        }
      }
#pragma unroll
      for (int i = 0; i < B; ++i) {
        if (j0 + i < k) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc[q] = __builtin_fmaf(g[i], v[i][0][q], acc[q]);
            acc[4 + q] = __builtin_fmaf(g[i], v[i][1][q], acc[4 + q]);
          }
        }
      }
    }
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
    reinterpret_cast<u32x4*>(out + (size_t)t * H)[c] = o;
  }
}
}  // namespace

int launch_combine(const void* y, int y_dtype, const int32_t* pos, const int32_t* n_valid, const float* w, int T,
                   int k, int H, uint16_t* out, void* stream) {
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (T == 0) return 0;
  if (y_dtype == 1) hipLaunchKernelGGL(combine_kernel<1>, dim3(T), dim3(kThreads), 0, s, y, pos, n_valid, w, k, H, out);
  else if (y_dtype == 2) hipLaunchKernelGGL(combine_kernel<2>, dim3(T), dim3(kThreads), 0, s, y, pos, n_valid, w, k, H, out);
  else hipLaunchKernelGGL(combine_kernel<0>, dim3(T), dim3(kThreads), 0, s, y, pos, n_valid, w, k, H, out);
  return (int)hipGetLastError();
}

}  // namespace moe

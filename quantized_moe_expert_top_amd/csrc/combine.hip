// Gate-weighted combine of each token's k expert outputs:
//   out[t] = sum_{j<k} w[t][j] * y_perm[pair_pos[t*k+j]]
// accumulated in fp32 in slot order and rounded once to bf16.  No atomics, so
// the result is bitwise reproducible.  One workgroup per token; each lane
// moves 8 bf16 (16 bytes) per row and slot.
#include "common.h"

namespace moe {

namespace {
constexpr int kThreads = 256;

// Y_F32: expert outputs in fp32 (not rounded before the combine) or bf16.
// Slots are taken in batches of 8: all row loads of a batch are issued before
// the first multiply-add, in slot order.
template <bool Y_F32>
__global__ __launch_bounds__(kThreads) void combine_kernel(const void* __restrict__ yv,
                                                           const int32_t* __restrict__ pos,
                                                           const float* __restrict__ w, int k, int H,
                                                           uint16_t* __restrict__ out) {
  constexpr int B = 8;
  const int t = blockIdx.x;
  const int nvec = H >> 3;
  for (int c = threadIdx.x; c < nvec; c += kThreads) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < k; j0 += B) {
      f32x4 v[B][2];
      float g[B];
#pragma unroll
      for (int i = 0; i < B; ++i) {
        const int j = j0 + i;
        if (j < k) {
          const int p = pos[(size_t)t * k + j];
          g[i] = w ? w[(size_t)t * k + j] : 1.0f;
          if (Y_F32) {
            const f32x4* row = reinterpret_cast<const f32x4*>(static_cast<const float*>(yv) + (size_t)p * H);
            v[i][0] = row[2 * c];
            v[i][1] = row[2 * c + 1];
          } else {
            const u32x4 b = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(yv) + (size_t)p * H)[c];
#pragma unroll
            for (int q = 0; q < 2; ++q)
              v[i][q] = f32x4{bf16_lo(b[2 * q]), bf16_hi(b[2 * q]), bf16_lo(b[2 * q + 1]), bf16_hi(b[2 * q + 1])};
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

hipError_t launch_combine(const void* y, bool y_f32, const int32_t* pos, const float* w, int T, int k, int H,
                          uint16_t* out, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (y_f32) hipLaunchKernelGGL(combine_kernel<true>, dim3(T), dim3(kThreads), 0, s, y, pos, w, k, H, out);
  else hipLaunchKernelGGL(combine_kernel<false>, dim3(T), dim3(kThreads), 0, s, y, pos, w, k, H, out);
  return hipGetLastError();
}

}  // namespace moe

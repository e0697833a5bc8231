// Internal helpers shared by the HIP kernels of the routed-expert MoE library.
// gfx950 (CDNA4) only: 64-lane wavefronts, bf16 MFMA, v_cvt_pk_bf16_f32.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// float -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __builtin_bit_cast(float, v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __builtin_bit_cast(float, v & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __builtin_bit_cast(float, (uint32_t)v << 16); }
__device__ __forceinline__ float f16_to_f32(uint16_t v) { return (float)__builtin_bit_cast(_Float16, v); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// D = A * B + C for a 32x32 tile with K = 16 (v_mfma_f32_32x32x16_bf16).
// Operand lane layout: lane l holds row (l % 32), k = 8*(l / 32) .. +7 of A
// (and column (l % 32), same k range, of B).  Accumulator: lane l, register r
// holds row 8*(r/4) + 4*(l/32) + (r%4), column l % 32.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// Kernel-side launch helpers return hipGetLastError() after the launch.
hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                             hipStream_t s);

struct PermuteArgs {
  const int32_t* ids;
  const uint8_t* bits;
  int P, k, E, S;
  int32_t* counts;
  int32_t* seg_offsets;
  int32_t* sorted_pair;
  int32_t* pair_pos;
  const uint16_t* x;
  int H;
  uint16_t* x_perm;
  void* ws;
};
size_t permute_workspace_bytes(int P, int E, int S);
hipError_t launch_permute(const PermuteArgs& a, hipStream_t s);

hipError_t launch_combine(const void* y, bool y_f32, const int32_t* pos, const float* w, int T, int k, int H,
                          uint16_t* out, hipStream_t s);

// Weight descriptor as the kernels see it (tiled layout only).
struct QWeights {
  int fmt;  // 1 INT4, 2 MWQ, 3 DELTA2
  int E, N, K, G, z, n_sal;
  const uint8_t* codes;
  const uint8_t* p3;
  const uint8_t* p4;
  const uint16_t* scales;
  const int32_t* sal_idx;
  const uint16_t* sal_val;
  const uint16_t* base;
};
struct QGemmArgs {
  QWeights w;
  const uint16_t* A;
  const int32_t* gather;
  int k;
  const int32_t* seg_offsets;
  int nseg;
  int M_total;
  int epilogue;  // 0 bf16, 1 SwiGLU bf16, 2 fp32
  void* out;
  void* ws;
};
size_t qgemm_workspace_bytes(const QWeights& w, int A_rows, int M_total);
hipError_t launch_qgemm(const QGemmArgs& a, hipStream_t s);

hipError_t launch_repack(const QWeights& src, const QWeights& dst, hipStream_t s);
size_t tiled_salient_bytes(int E, int N, int n_sal);

}  // namespace moe

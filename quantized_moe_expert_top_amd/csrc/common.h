// Internal helpers shared by the HIP kernels of the routed-expert MoE library.
// gfx950 (CDNA4) only: 64-lane wavefronts, bf16 MFMA, v_cvt_pk_bf16_f32.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

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
// fp16, round to nearest even (|f| past the fp16 range becomes +-inf)
__device__ __forceinline__ uint16_t f32_to_f16(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __builtin_bit_cast(float, v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __builtin_bit_cast(float, v & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __builtin_bit_cast(float, (uint32_t)v << 16); }
__device__ __forceinline__ float f16_to_f32(uint16_t v) { return (float)__builtin_bit_cast(_Float16, v); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
// acc + lo(v) + hi(v) for a bf16 pair, one v_dot2 with (1, 1).  Takes the
// dword by value: a bit_cast applied directly to an ext_vector element
// expression (v[h]) is miscompiled to always read element 0.
__device__ __forceinline__ float add_bf16_pair(uint32_t v, float acc) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, v), __builtin_bit_cast(bf16x2_t, 0x3F803F80u),
                                         acc, false);
}

// Raw buffer loads: wave-uniform resource + per-lane byte offset + uniform
// byte offset.  Reads at or past `bytes` return zero instead of faulting.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_x4(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ u32x2 buf_x2(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}
__device__ __forceinline__ uint32_t buf_x1(rsrc_t r, uint32_t voff, uint32_t soff) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}
__device__ __forceinline__ uint16_t buf_u16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
}

// D = A * B + C for a 32x32 tile with K = 16 (v_mfma_f32_32x32x16_bf16).
// Operand lane layout: lane l holds row (l % 32), k = 8*(l / 32) .. +7 of A
// (and column (l % 32), same k range, of B).  Accumulator: lane l, register r
// holds row 8*(r/4) + 4*(l/32) + (r%4), column l % 32.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// Top-k of one token by one wavefront, E <= 64 (expert gate of the Dual
// Routing equations, D2MoE page): lane e holds logit e and counts the experts
// that beat it (larger logit, or equal logit and lower index); a count below k
// is the lane's slot.  Gates = softmax over the k selected logits in float64,
// rounded once to float32.  sel_val / sel_exp: 64-entry LDS scratch of this
// wavefront; slot_ids (optional) receives the k ids as well.
// v: this lane's logit (lane < E), -inf for lanes >= E.
__device__ __forceinline__ void route_token_rank(float v, int E, int k, int32_t* __restrict__ ids,
                                                 float* __restrict__ w, float* sel_val, double* sel_exp,
                                                 int* slot_ids) {
  const int lane = threadIdx.x & 63;
  int rank = 0;
#pragma unroll
  for (int j = 0; j < 64; ++j) {
    const float vj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), j));
    rank += (vj > v || (vj == v && j < lane)) ? 1 : 0;
  }
  if (lane < E && rank < k) {
    ids[rank] = lane;
    sel_val[rank] = v;
    if (slot_ids) slot_ids[rank] = lane;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const double l0 = (double)sel_val[0];
  if (lane < k) sel_exp[lane] = exp((double)sel_val[lane] - l0);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (lane < k) {
    double sum = 0.0;
    for (int j = 0; j < k; ++j) sum += sel_exp[j];
    w[lane] = (float)(sel_exp[lane] / sum);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Static per-expert widths (format 4): the kernels get each expert's width,
// zero point and first tile block (in units of 256 bytes; a tile block of a
// b-bit expert is 256 * b bytes) by value, in the launch arguments.
struct XTab {
  uint8_t bits[kMaxMixedExperts];
  uint8_t zero[kMaxMixedExperts];
  uint32_t off[kMaxMixedExperts];
};

}  // namespace moe

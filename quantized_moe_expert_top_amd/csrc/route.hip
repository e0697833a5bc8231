// Top-k expert gate (expert gate of the Dual Routing equations, D2MoE page,
// Design): per token, the k largest logits in descending order, ties to the
// lower expert index, and gate weights = softmax over the k selected logits.
//
// One 64-lane wavefront per token.  For E <= 64 every lane holds one logit and
// computes its rank against the other 63 (scalar broadcasts, no shuffles).
// For larger E lane l owns experts l, l+64, ... (up to 16 per lane,
// E <= 1024) and each of the k rounds is a wave-wide arg-max over
// (logit, -index) with butterfly shuffles; the winner is marked taken.  The
// softmax runs in float64 on the selected values (k exp calls per token) and
// is rounded once to float32, so the gates differ from the exact value by at
// most half an fp32 ulp plus the fp64 rounding of the sum.
#include "common.h"

namespace moe {

namespace {
constexpr int kMaxSlots = 16;  // 16 * 64 = 1024 experts
constexpr int kWavesPerBlock = 4;
constexpr int kMaxK = 1024;

__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                          int32_t* __restrict__ ids, float* __restrict__ w) {
  __shared__ float sel_val[kWavesPerBlock][kMaxK];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int t = blockIdx.x * kWavesPerBlock + wv;
  if (t >= T) return;
  const float* row = logits + (size_t)t * E;
  const int nslots = (E + 63) >> 6;

  float v[kMaxSlots];
#pragma unroll
  for (int s = 0; s < kMaxSlots; ++s) {
    const int e = lane + 64 * s;
    v[s] = (s < nslots && e < E) ? row[e] : -__builtin_inff();
  }
  uint32_t taken = 0;  // bit s: slot s already selected (or absent)
#pragma unroll
  for (int s = 0; s < kMaxSlots; ++s)
    if (!(s < nslots && lane + 64 * s < E)) taken |= 1u << s;

  float l0 = 0.f;
  double sum = 0.0;
  for (int j = 0; j < k; ++j) {
    // lane-local best among untaken slots
    float bv = -__builtin_inff();
    int bi = 0x7fffffff;
#pragma unroll
    for (int s = 0; s < kMaxSlots; ++s) {
      const int e = lane + 64 * s;
      if (!((taken >> s) & 1u) && better(v[s], e, bv, bi)) {
        bv = v[s];
        bi = e;
      }
    }
    // wave-wide arg-max, ties to the lower index
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const float ov = __shfl_xor(bv, off, 64);
      const int oi = __shfl_xor(bi, off, 64);
      if (better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (j == 0) l0 = bv;
    sum += exp((double)bv - (double)l0);
    if (lane == 0) {
      ids[(size_t)t * k + j] = bi;
      sel_val[wv][j] = bv;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  for (int j = lane; j < k; j += 64) {
    const double e = exp((double)sel_val[wv][j] - (double)l0);
    w[(size_t)t * k + j] = (float)(e / sum);
  }
}
// E <= 64: lane e holds logit e and counts the experts that beat it (larger
// logit, or equal logit and lower index); that count is its slot if < k.
__global__ __launch_bounds__(256) void route_rank_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                         int32_t* __restrict__ ids, float* __restrict__ w) {
  __shared__ float sel_val[kWavesPerBlock][64];
  __shared__ double sel_exp[kWavesPerBlock][64];
  const int wv = threadIdx.x >> 6;
  const int t = blockIdx.x * kWavesPerBlock + wv;
  if (t >= T) return;
  const int lane = threadIdx.x & 63;
  const float v = lane < E ? logits[(size_t)t * E + lane] : -__builtin_inff();
  route_token_rank(v, E, k, ids + (size_t)t * k, w + (size_t)t * k, sel_val[wv], sel_exp[wv], nullptr);
}
}  // namespace

int launch_route_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w, void* stream) {
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (T == 0) return 0;
  const int blocks = (T + kWavesPerBlock - 1) / kWavesPerBlock;
  if (E <= 64)
    hipLaunchKernelGGL(route_rank_kernel, dim3(blocks), dim3(64 * kWavesPerBlock), 0, s, logits, T, E, k, ids, w);
  else
    hipLaunchKernelGGL(route_topk_kernel, dim3(blocks), dim3(64 * kWavesPerBlock), 0, s, logits, T, E, k, ids, w);
  return (int)hipGetLastError();
}

}  // namespace moe

// Grouped low-bit GEMM over expert segments (grouped batched expert execution,
// ExactMoE page; "dequantise -> 16-bit GEMM" pipeline equation, D2MoE page).
//
// Work split: one workgroup (4 wavefronts) per (32-row tile of one segment,
// output-channel tile).  The output-channel tile is 32 SwiGLU channels (a gate
// tile and the matching up tile) or 64 plain channels (two tiles).  The four
// wavefronts split K and reduce through LDS in a fixed order.  Row tiles are
// assigned on the device from seg_offsets, so the host never reads counts.
//
// Dequantisation is exact and costs one shift + one and-or per pair of
// weights: a code c is dropped into the low mantissa bits of the bf16 number
// 128 (bits 0x4300), giving exactly 128 + c.  The MFMA then accumulates
// sum_k a_k * (128 + c_k) in fp32, and a second MFMA chain with the constant
// -(128 + z) adds sum_k a_k * (-(128 + z)), so the sum of the two is exactly
// sum_k a_k * (c_k - z) up to fp32 accumulation rounding.  The group scale (or
// the per-channel step) multiplies that in fp32 once per group.
//   INT4 (ExactMoE W4A16):       w = s[n][k/G] * (c - z)
//   MWQ  (D2MoE MWQ equations):  c_b = 4*q2 + 2*d3*[b>=3] + d4*[b==4]; the
//                                planes a segment's bit-width does not need are
//                                never loaded
//   DELTA2 (ME-Switch):          d = step[n] * (c - z) off the salient
//                                channels (their codes were zeroed by the
//                                repack); salient channels are one more MFMA
//                                K-chunk with bf16 values; the shared base is a
//                                plain bf16 MFMA on the same A operand
#include "common.h"

namespace moe {

namespace {
constexpr int kThreads = 256;
constexpr int kRows = 32;

struct KArgs {
  const uint8_t* codes;
  const uint8_t* p3;
  const uint8_t* p4;
  const uint16_t* scales;
  const int32_t* sal_idx;
  const uint16_t* sal_val;
  const uint16_t* base;
  const uint16_t* A;
  const int32_t* gather;
  const int32_t* seg_offsets;
  void* out;
  int k, nseg, S, N, K, G, z, n_sal, n_out, ntiles_n;
};

// Locate the row tile `y` (in segment order) -> segment and first row.
__device__ __forceinline__ bool find_tile(const int32_t* seg_offsets, int nseg, int y, int& seg, int& m0) {
  const int lane = threadIdx.x & 63;
  int carry = 0;
  for (int s0 = 0; s0 < nseg; s0 += 64) {
    const int s = s0 + lane;
    int tiles = 0;
    if (s < nseg) tiles = (seg_offsets[s + 1] - seg_offsets[s] + kRows - 1) / kRows;
    int incl = tiles;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off, 64);
      if (lane >= off) incl += o;
    }
    const int excl = carry + incl - tiles;
    const bool hit = s < nseg && y >= excl && y < excl + tiles;
    const uint64_t b = __ballot(hit);
    if (b) {
      const int src = __ffsll((unsigned long long)b) - 1;
      seg = s0 + src;
      m0 = (y - __shfl(excl, src, 64)) * kRows;
      return true;
    }
    carry += __shfl(incl, 63, 64);
  }
  return false;
}

__device__ __forceinline__ uint32_t shr(uint32_t v, int sh) { return sh >= 0 ? (v >> sh) : (v << (-sh)); }

// 8 bf16 values (128 + code) for MFMA step s of one lane.
__device__ __forceinline__ bf16x8 deq_u4(const u32x4& lo, const u32x4& hi, int s) {
  const uint32_t d = s < 4 ? lo[s & 3] : hi[s & 3];
  u32x4 r;
  r[0] = (d & 0x000F000Fu) | 0x43004300u;
  r[1] = ((d >> 4) & 0x000F000Fu) | 0x43004300u;
  r[2] = ((d >> 8) & 0x000F000Fu) | 0x43004300u;
  r[3] = ((d >> 12) & 0x000F000Fu) | 0x43004300u;
  return as_bf16x8(r);
}

__device__ __forceinline__ bf16x8 deq_mwq(const u32x4& q2, const u32x2& d3, const u32x2& d4, int s, int b) {
  const uint32_t Q = q2[s >> 1];
  const uint32_t D3 = d3[s >> 2];
  const uint32_t D4 = d4[s >> 2];
  u32x4 r;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int P = 4 * (s & 1) + p;
    const int P3 = 4 * (s & 3) + p;
    uint32_t v = (shr(Q, 2 * P - 2) & 0x000C000Cu) | 0x43004300u;
    if (b >= 3) v |= shr(D3, P3 - 1) & 0x00020002u;
    if (b == 4) v |= shr(D4, P3) & 0x00010001u;
    r[p] = v;
  }
  return as_bf16x8(r);
}

__device__ __forceinline__ bf16x8 deq_u2(const u32x4& c, int s) {
  const uint32_t C = c[s >> 1];
  u32x4 r;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int P = 4 * (s & 1) + p;
    r[p] = (shr(C, 2 * P) & 0x00030003u) | 0x43004300u;
  }
  return as_bf16x8(r);
}

// EPI: 0 = bf16 out, 1 = SwiGLU bf16 out, 2 = fp32 out
template <int FMT, int EPI>
__global__ __launch_bounds__(kThreads) void qgemm_kernel(KArgs p) {
  constexpr bool SWIGLU = EPI == 1;
  __shared__ float red[4][2][16][64];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;

  int seg, m0;
  if (!find_tile(p.seg_offsets, p.nseg, blockIdx.y, seg, m0)) return;
  const int row0 = p.seg_offsets[seg] + m0;
  const int rows = min(kRows, p.seg_offsets[seg + 1] - row0);
  const int e = seg / p.S;
  const int bits = 4 - (seg % p.S);  // MWQ only

  const int NT = p.N / 32;
  const int KB = p.K / 128;
  // channel tiles handled by this workgroup
  int ct[2];
  bool tv[2];
  if (SWIGLU) {
    ct[0] = blockIdx.x;
    ct[1] = NT / 2 + blockIdx.x;
    tv[0] = tv[1] = true;
  } else {
    ct[0] = 2 * blockIdx.x;
    tv[0] = true;
    tv[1] = 2 * (int)blockIdx.x + 1 < NT;
    ct[1] = tv[1] ? ct[0] + 1 : ct[0];  // an odd last tile recomputes tile 0 and skips its store
  }

  // A operand rows: lane -> row (lane % 32) of the tile, K half (lane / 32)
  const int mrow = min(lane & 31, rows - 1);
  const int q = lane >> 5;
  const int gi = row0 + mrow;
  const size_t arow = p.gather ? (size_t)(p.gather[gi] / p.k) : (size_t)gi;
  const uint16_t* Ap = p.A + arow * p.K + 8 * q;

  const uint32_t negc = (0xC300u | (uint32_t)p.z) * 0x00010001u;
  const bf16x8 neg = as_bf16x8(u32x4{negc, negc, negc, negc});

  f32x16 acc[2], accb[2], tmp[2], corr;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    acc[t] = f32x16{};
    accb[t] = f32x16{};
    tmp[t] = f32x16{};
  }
  corr = f32x16{};

  const int kb0 = (wv * KB) / 4, kb1 = ((wv + 1) * KB) / 4;
  const int spg = (FMT == 3) ? 8 : p.G / 16;  // MFMA steps per scale group
  for (int kb = kb0; kb < kb1; ++kb) {
    u32x4 a[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) a[s] = *reinterpret_cast<const u32x4*>(Ap + kb * 128 + 16 * s);

    u32x4 blo[2], bhi[2], bq[2];
    u32x2 b3[2], b4[2];
    u32x4 bb[2][8];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const size_t blk = ((size_t)e * NT + ct[t]) * KB + kb;
      if (FMT == 1) {
        const uint8_t* bp = p.codes + blk * 2048 + 16 * lane;
        blo[t] = *reinterpret_cast<const u32x4*>(bp);
        bhi[t] = *reinterpret_cast<const u32x4*>(bp + 1024);
      } else {
        bq[t] = *reinterpret_cast<const u32x4*>(p.codes + blk * 1024 + 16 * lane);
        if (FMT == 2) {
          b3[t] = bits >= 3 ? *reinterpret_cast<const u32x2*>(p.p3 + blk * 512 + 8 * lane) : u32x2{0u, 0u};
          b4[t] = bits == 4 ? *reinterpret_cast<const u32x2*>(p.p4 + blk * 512 + 8 * lane) : u32x2{0u, 0u};
        }
        if (FMT == 3 && p.base) {
          const uint16_t* bp = p.base + ((size_t)ct[t] * KB + kb) * 4096 + 8 * lane;
#pragma unroll
          for (int s = 0; s < 8; ++s) bb[t][s] = *reinterpret_cast<const u32x4*>(bp + 512 * s);
        }
      }
    }

#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const bf16x8 av = as_bf16x8(a[s]);
      corr = mfma32(av, neg, corr);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        bf16x8 bv;
        if (FMT == 1) bv = deq_u4(blo[t], bhi[t], s);
        else if (FMT == 2) bv = deq_mwq(bq[t], b3[t], b4[t], s, bits);
        else bv = deq_u2(bq[t], s);
        tmp[t] = mfma32(av, bv, tmp[t]);
        if (FMT == 3 && p.base) accb[t] = mfma32(av, as_bf16x8(bb[t][s]), accb[t]);
      }
      if (FMT != 3 && ((s + 1) % spg) == 0) {
        // end of a scale group: acc += s[n][g] * (tmp + corr)
        const int g = (kb * 128 + 16 * s) / p.G;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int ch = ct[t] * 32 + (lane & 31);
          const float sc = f16_to_f32(p.scales[((size_t)e * p.N + ch) * (p.K / p.G) + g]);
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[t][r] = __builtin_fmaf(sc, tmp[t][r] + corr[r], acc[t][r]);
          tmp[t] = f32x16{};
        }
        corr = f32x16{};
      }
    }
  }

  if (FMT == 3) {
    // salient input channels: one more K chunk of exact bf16 values (wave 0)
    if (wv == 0 && p.n_sal > 0) {
      const int nsteps = (p.n_sal + 15) / 16;
      const uint16_t* Arow = p.A + arow * p.K;
      for (int st = 0; st < nsteps; ++st) {
        u32x4 av;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          uint32_t v = 0;
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int j = 16 * st + 8 * q + 2 * h + u;
            const int idx = j < p.n_sal ? min(max(p.sal_idx[(size_t)e * p.n_sal + j], 0), p.K - 1) : 0;
            v |= (uint32_t)Arow[idx] << (16 * u);
          }
          av[h] = v;
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const u32x4 sv = *reinterpret_cast<const u32x4*>(
              p.sal_val + (((size_t)e * NT + ct[t]) * nsteps + st) * 512 + 8 * lane);
          accb[t] = mfma32(as_bf16x8(av), as_bf16x8(sv), accb[t]);
        }
      }
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int ch = ct[t] * 32 + (lane & 31);
      const float st = f16_to_f32(p.scales[(size_t)e * p.N + ch]);
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[t][r] = __builtin_fmaf(st, tmp[t][r] + corr[r], accb[t][r]);
    }
  }

  // split-K reduction in wave order 0..3, then the epilogue
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) red[wv][t][r][lane] = acc[t][r];
  __syncthreads();
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int r = 4 * wv + rr;
    const int row = acc_row(r, lane);
    float v0 = red[0][0][r][lane] + red[1][0][r][lane] + red[2][0][r][lane] + red[3][0][r][lane];
    float v1 = red[0][1][r][lane] + red[1][1][r][lane] + red[2][1][r][lane] + red[3][1][r][lane];
    if (row < rows) {
      if (EPI == 2) {
        float* orow = static_cast<float*>(p.out) + (size_t)(row0 + row) * p.n_out;
        orow[ct[0] * 32 + (lane & 31)] = v0;
        if (tv[1]) orow[ct[1] * 32 + (lane & 31)] = v1;
      } else {
        uint16_t* orow = static_cast<uint16_t*>(p.out) + (size_t)(row0 + row) * p.n_out;
        if (SWIGLU) {
          const float h = v0 / (1.0f + __expf(-v0)) * v1;
          orow[blockIdx.x * 32 + (lane & 31)] = f32_to_bf16(h);
        } else {
          orow[ct[0] * 32 + (lane & 31)] = f32_to_bf16(v0);
          if (tv[1]) orow[ct[1] * 32 + (lane & 31)] = f32_to_bf16(v1);
        }
      }
    }
  }
}

template <int FMT>
hipError_t launch_fmt(const KArgs& ka, int epi, dim3 grid, hipStream_t s) {
  if (epi == 1) hipLaunchKernelGGL((qgemm_kernel<FMT, 1>), grid, dim3(kThreads), 0, s, ka);
  else if (epi == 2) hipLaunchKernelGGL((qgemm_kernel<FMT, 2>), grid, dim3(kThreads), 0, s, ka);
  else hipLaunchKernelGGL((qgemm_kernel<FMT, 0>), grid, dim3(kThreads), 0, s, ka);
  return hipGetLastError();
}
}  // namespace

size_t qgemm_workspace_bytes(const QWeights&, int, int) { return 0; }

hipError_t launch_qgemm(const QGemmArgs& a, hipStream_t s) {
  if (a.M_total == 0) return hipSuccess;
  const QWeights& w = a.w;
  KArgs ka;
  ka.codes = w.codes;
  ka.p3 = w.p3;
  ka.p4 = w.p4;
  ka.scales = w.scales;
  ka.sal_idx = w.sal_idx;
  ka.sal_val = w.sal_val;
  ka.base = w.base;
  ka.A = a.A;
  ka.gather = a.gather;
  ka.seg_offsets = a.seg_offsets;
  ka.out = a.out;
  ka.k = a.k;
  ka.nseg = a.nseg;
  ka.S = (w.fmt == 2) ? 3 : 1;
  ka.N = w.N;
  ka.K = w.K;
  ka.G = w.G;
  ka.z = w.z;
  ka.n_sal = w.n_sal;
  const bool swiglu = a.epilogue == 1;
  ka.n_out = swiglu ? w.N / 2 : w.N;
  const int NT = w.N / 32;
  ka.ntiles_n = swiglu ? NT / 2 : (NT + 1) / 2;
  const int ytiles = (a.M_total + kRows - 1) / kRows + a.nseg;
  dim3 grid(ka.ntiles_n, ytiles);
  switch (w.fmt) {
    case 1: return launch_fmt<1>(ka, a.epilogue, grid, s);
    case 2: return launch_fmt<2>(ka, a.epilogue, grid, s);
    default: return launch_fmt<3>(ka, a.epilogue, grid, s);
  }
}

}  // namespace moe

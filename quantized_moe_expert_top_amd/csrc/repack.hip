// Offline conversion of canonical weight storage to the tiled layout that the
// grouped GEMM streams.  Codes are moved, never changed (except the salient
// input channels of a 2-bit delta, whose codes become the zero code because
// their value travels separately in bf16).
//
// Tiled layout, one "tile block" per (expert e, 16 output channels ct, 128
// input channels kb), tile blocks ordered (e, ct, kb) so that a wavefront
// streams one channel tile along K contiguously.  Inside a tile block, lane l
// of a wavefront owns channel ct*16 + (l % 16) and, for each 32-wide K step
// t = 0..3, the 8 inputs k = kb*128 + 32*t + 8*(l/16) + i, i = 0..7 (the
// operand layout of v_mfma_f32_16x16x32_bf16).  The bits of one lane and step
// are placed so that pairs (i = 2p, 2p+1) land in the low / high halfword of a
// dword after one shift and mask.  Nibble j of a dword (bits 4j .. 4j+3)
// stands for element i = 2 (j % 4) + j / 4 (j = 4 (i&1) + (i>>1)):
//   4-bit  (1 KB / tile block): dword at 16*l + 4*t; element i's code in its
//          nibble (bit 16*(i&1) + 4*(i>>1)).
//   2-bit delta (512 B): dword at 8*l + 4*(t/2); with P = 4*(t%2) + (i>>1),
//          element i at bit 16*(i&1) + 2*P.
//   nested MWQ (1 KB, all in `codes`): planes at bytes 0 (q2), 512 (d3) and
//          768 (d4), so one tile block is one contiguous kilobyte (read whole
//          by the prefill kernels, plane by plane by the decode kernel, which
//          skips the planes it needs not).  q2: dword at 8*l + 4*(t/2), in
//          element i's nibble at bits 2-3 for even t, 0-1 for odd t; d3 and
//          d4: dword at 4*l, element i's bit of step t at bit 3 - t of its
//          nibble.  Masking and shifting each plane by t then ORs the three
//          into the 4-bit codes of step t in the INT4 order: about five
//          operations per step and lane, then the INT4 conversion.
//   bf16 base (4 KB, no expert index): 16 bytes at 1024*t + 16*l hold the 8
//          inputs in order.
//   salient values: per (e, ct) ceil(S/32) blocks of 1 KB; lane l holds slots
//          32*step + 8*(l/16) + i of channel ct*16 + l%16 (zero past S).
#include "common.h"

namespace moe {

namespace {
constexpr int kThreads = 256;

struct TileIdx {
  size_t e;
  int ct, kb;
};
__device__ __forceinline__ TileIdx tile_of(size_t blk, int N, int K) {
  const int KB = K / 128, NT = N / 16;
  TileIdx r;
  r.kb = (int)(blk % KB);
  const size_t ect = blk / KB;
  r.ct = (int)(ect % NT);
  r.e = ect / NT;
  return r;
}

__global__ __launch_bounds__(kThreads) void repack_u4_kernel(const uint8_t* __restrict__ src, int N, int K,
                                                             uint32_t* __restrict__ dst, size_t ndw) {
  const size_t d = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (d >= ndw) return;
  const TileIdx ti = tile_of(d / 256, N, K);
  const int within = (int)(d % 256);
  const int l = within / 4, t = within % 4;
  const int ch = ti.ct * 16 + (l & 15);
  const int k0 = ti.kb * 128 + 32 * t + 8 * (l >> 4);
  const uint32_t v = *reinterpret_cast<const uint32_t*>(src + (ti.e * N + ch) * (size_t)(K / 2) + k0 / 2);
  uint32_t o = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) o |= ((v >> (4 * i)) & 0xFu) << (16 * (i & 1) + 4 * (i >> 1));
  dst[d] = o;
}

// nibble position of element i (0..7) of an MFMA step
__device__ __forceinline__ int nib_of(int i) { return 4 * (i & 1) + (i >> 1); }

// 2-bit plane, one 128-thread workgroup per 512-byte tile block; zero_code >= 0
// replaces the codes of salient channels (2-bit delta).  q2: the nested
// planes' layout (nibbles) instead of the delta's.
__global__ __launch_bounds__(128) void repack_u2_kernel(const uint8_t* __restrict__ src, int N, int K,
                                                        uint32_t* __restrict__ dst, int blk_dw, const int32_t* sal_idx,
                                                        int n_sal, int zero_code, bool q2) {
  __shared__ uint32_t salmask[4];
  const TileIdx ti = tile_of(blockIdx.x, N, K);
  if (threadIdx.x < 4) salmask[threadIdx.x] = 0;
  __syncthreads();
  if (sal_idx && (int)threadIdx.x < n_sal) {
    const int kk = sal_idx[ti.e * n_sal + threadIdx.x] - ti.kb * 128;
    if (kk >= 0 && kk < 128) atomicOr(&salmask[kk >> 5], 1u << (kk & 31));
  }
  __syncthreads();
  const int l = threadIdx.x / 2, w = threadIdx.x % 2;
  const int ch = ti.ct * 16 + (l & 15);
  uint32_t o = 0;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int t = 2 * w + tt;
    const int koff = 32 * t + 8 * (l >> 4);
    const int k0 = ti.kb * 128 + koff;
    const uint32_t v = *reinterpret_cast<const uint16_t*>(src + (ti.e * N + ch) * (size_t)(K / 4) + k0 / 4);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t f = (v >> (2 * i)) & 3u;
      const int kk = koff + i;
      if (zero_code >= 0 && ((salmask[kk >> 5] >> (kk & 31)) & 1u)) f = (uint32_t)zero_code;
      const int P = 4 * tt + (i >> 1);
      o |= f << (q2 ? 4 * nib_of(i) + 2 - 2 * tt : 16 * (i & 1) + 2 * P);
    }
  }
  dst[(size_t)blockIdx.x * blk_dw + threadIdx.x] = o;  // tile blocks blk_dw dwords apart
}

// d3 / d4 plane of the nested layout.  d = dword index of the plane; written
// at dword off_dw of a tile block of blk_dw dwords
__global__ __launch_bounds__(kThreads) void repack_u1_kernel(const uint8_t* __restrict__ src, int N, int K,
                                                             uint32_t* __restrict__ dst, int blk_dw, int off_dw,
                                                             size_t ndw) {
  const size_t d = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (d >= ndw) return;
  const TileIdx ti = tile_of(d / 64, N, K);
  const int l = (int)(d % 64);
  const int ch = ti.ct * 16 + (l & 15);
  uint32_t o = 0;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int k0 = ti.kb * 128 + 32 * t + 8 * (l >> 4);
    const uint32_t v = src[(ti.e * N + ch) * (size_t)(K / 8) + k0 / 8];
#pragma unroll
    for (int i = 0; i < 8; ++i) o |= ((v >> i) & 1u) << (4 * nib_of(i) + 3 - t);
  }
  dst[(d / 64) * blk_dw + off_dw + d % 64] = o;
}

__global__ __launch_bounds__(kThreads) void repack_base_kernel(const uint16_t* __restrict__ src, int N, int K,
                                                               u32x4* __restrict__ dst, size_t nvec) {
  const size_t d = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (d >= nvec) return;
  const int KB = K / 128;
  const size_t blk = d / 256;
  const int within = (int)(d % 256);
  const int t = within / 64, l = within % 64;
  const int kb = (int)(blk % KB);
  const int ct = (int)(blk / KB);
  const int ch = ct * 16 + (l & 15);
  const int k0 = kb * 128 + 32 * t + 8 * (l >> 4);
  dst[d] = *reinterpret_cast<const u32x4*>(src + (size_t)ch * K + k0);
}

__global__ __launch_bounds__(kThreads) void repack_salient_kernel(const uint16_t* __restrict__ src, int N,
                                                                  int n_sal, int nsteps,
                                                                  uint32_t* __restrict__ dst, size_t ndw) {
  const size_t d = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (d >= ndw) return;
  const int NT = N / 16;
  const size_t blk = d / 256;  // (e, ct, step)
  const int within = (int)(d % 256);
  const int l = within / 4, w = within % 4;
  const int step = (int)(blk % nsteps);
  const size_t ect = blk / nsteps;
  const int ct = (int)(ect % NT);
  const size_t e = ect / NT;
  const int ch = ct * 16 + (l & 15);
  uint32_t o = 0;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int j = 32 * step + 8 * (l >> 4) + 2 * w + h;
    const uint32_t v = j < n_sal ? src[(e * n_sal + j) * (size_t)N + ch] : 0u;
    o |= v << (16 * h);
  }
  dst[d] = o;
}

// Per-expert width b: one expert's N x K codes (little-endian b-bit stream per
// row) -> its tiled blocks of 256 * b bytes: each code shifted to 4 bits,
// c4 = c << (4 - b), as the nested planes q2 = c4 >> 2 (2-bit layout), d3 =
// bit 1 and d4 = bit 0 (1-bit layouts), of which only the first b are stored.
__global__ __launch_bounds__(kThreads) void repack_mixed_kernel(const uint8_t* __restrict__ src, int N, int K,
                                                                int b, uint32_t* __restrict__ dst, size_t ndw) {
  const size_t d = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (d >= ndw) return;
  const int bdw = 64 * b;  // dwords per tile block
  const size_t blk = d / bdw;
  const int w = (int)(d % bdw);
  const int KB = K / 128;
  const int kb = (int)(blk % KB), ct = (int)(blk / KB);
  const size_t row_bits = (size_t)K * b;
  auto code4 = [&](int ch, int k) -> uint32_t {
    const size_t pos = (size_t)ch * row_bits + (size_t)k * b;  // bit position in the expert's stream
    uint32_t v = src[pos >> 3];
    if ((int)(pos & 7) + b > 8) v |= (uint32_t)src[(pos >> 3) + 1] << 8;
    return ((v >> (pos & 7)) & ((1u << b) - 1)) << (4 - b);
  };
  uint32_t o = 0;
  if (b == 8) {  // 8-bit codes as bytes: lane l = w / 8 holds 32 bytes, step t = (w % 8) / 2 at bytes 8t .. 8t + 7
    const int l = w >> 3, j = w & 7, t = j >> 1, ch = ct * 16 + (l & 15);
    const uint8_t* row = src + (size_t)ch * K + kb * 128 + 32 * t + 8 * (l >> 4) + 4 * (j & 1);
#pragma unroll
    for (int q = 0; q < 4; ++q) o |= (uint32_t)row[q] << (8 * q);
  } else if (w < 128) {  // q2: lane l = w / 2, steps 2 (w & 1) and 2 (w & 1) + 1
    const int l = w >> 1, ch = ct * 16 + (l & 15);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int t = 2 * (w & 1) + tt;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        o |= (code4(ch, kb * 128 + 32 * t + 8 * (l >> 4) + i) >> 2) << (4 * nib_of(i) + 2 - 2 * tt);
    }
  } else {  // d3 (w < 192) or d4: lane l = w % 64, all four steps
    const int l = (w - 128) & 63, ch = ct * 16 + (l & 15);
    const int sh = w < 192 ? 1 : 0;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        o |= ((code4(ch, kb * 128 + 32 * t + 8 * (l >> 4) + i) >> sh) & 1u) << (4 * nib_of(i) + 3 - t);
  }
  dst[d] = o;
}

inline unsigned grid_for(size_t n) { return (unsigned)((n + kThreads - 1) / kThreads); }
}  // namespace


int launch_repack(const QWeights& src, const QWeights& dst, void* stream) {
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t ENK = (size_t)src.E * src.N * src.K;
  if (ENK == 0) return 0;
  uint32_t* codes = reinterpret_cast<uint32_t*>(const_cast<uint8_t*>(dst.codes));
  if (src.fmt == 4) {  // per expert: canonical and tiled bytes and offsets agree
    size_t off = 0;
    for (int e = 0; e < src.E; ++e) {
      const int b = src.xbits[e];
      const size_t nbytes = (size_t)src.N * src.K * b / 8;
      const size_t ndw = nbytes / 4;
      hipLaunchKernelGGL(repack_mixed_kernel, dim3(grid_for(ndw)), dim3(kThreads), 0, s, src.codes + off, src.N,
                         src.K, b, reinterpret_cast<uint32_t*>(const_cast<uint8_t*>(dst.codes) + off), ndw);
      off += nbytes;
    }
    return (int)hipGetLastError();
  }
  if (src.fmt == 1) {
    const size_t ndw = ENK / 8;
    hipLaunchKernelGGL(repack_u4_kernel, dim3(grid_for(ndw)), dim3(kThreads), 0, s, src.codes, src.N, src.K, codes,
                       ndw);
  } else {
    const size_t nblk = ENK / (16 * 128);
    const bool delta = src.fmt == 3;
    // DELTA2: 512-byte blocks of 2-bit codes; MWQ: 1 KB blocks, q2 at dword 0, d3 at 128, d4 at 192
    const int blk_dw = delta ? 128 : 256;
    hipLaunchKernelGGL(repack_u2_kernel, dim3((unsigned)nblk), dim3(128), 0, s, src.codes, src.N, src.K, codes,
                       blk_dw, delta ? src.sal_idx : nullptr, delta ? src.n_sal : 0, delta ? src.z : -1, !delta);
    if (src.fmt == 2) {
      const size_t ndw = ENK / 32;
      hipLaunchKernelGGL(repack_u1_kernel, dim3(grid_for(ndw)), dim3(kThreads), 0, s, src.p3, src.N, src.K, codes,
                         blk_dw, 128, ndw);
      hipLaunchKernelGGL(repack_u1_kernel, dim3(grid_for(ndw)), dim3(kThreads), 0, s, src.p4, src.N, src.K, codes,
                         blk_dw, 192, ndw);
    }
    if (delta) {
      if (src.n_sal > 0) {
        const int nsteps = (src.n_sal + 31) / 32;
        const size_t ndw = tiled_salient_bytes(src.E, src.N, src.n_sal) / 4;
        hipLaunchKernelGGL(repack_salient_kernel, dim3(grid_for(ndw)), dim3(kThreads), 0, s, src.sal_val, src.N,
                           src.n_sal, nsteps, reinterpret_cast<uint32_t*>(const_cast<uint16_t*>(dst.sal_val)), ndw);
      }
      if (src.base) {
        const size_t nvec = (size_t)src.N * src.K / 8;
        hipLaunchKernelGGL(repack_base_kernel, dim3(grid_for(nvec)), dim3(kThreads), 0, s, src.base, src.N, src.K,
                           reinterpret_cast<u32x4*>(const_cast<uint16_t*>(dst.base)), nvec);
      }
    }
  }
  return (int)hipGetLastError();
}

}  // namespace moe

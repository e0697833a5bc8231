// Grouped low-bit GEMM over expert segments (grouped batched expert execution,
// ExactMoE page; "dequantise -> 16-bit GEMM" pipeline equation, D2MoE page).
//
// Work split: one workgroup (4 wavefronts) per (tile of up to 32 rows of one
// segment, channel group).  Each wavefront owns two 16-channel tiles (a gate
// tile and the matching up tile for SwiGLU, else two neighbouring tiles) and
// streams all of K for them with v_mfma_f32_16x16x32_bf16; a 32-row tile is
// two 16-row MFMA tiles, the second skipped when the tile has <= 16 rows.  Row
// tiles are assigned on the device from seg_offsets, so the host never reads
// counts back.  The activation rows of a K block are staged once per
// workgroup through a 3-slot LDS ring; the weight stream of every wavefront
// runs 3 K blocks ahead in a 4-slot register ring.
//
// Dequantisation is exact and costs one shift + one and-or per pair of
// weights: a code c is dropped into the low mantissa bits of the bf16 number
// 128 (bits 0x4300), giving exactly 128 + c.  The MFMA accumulates
// sum_k a_k * (128 + c_k) in fp32, a second MFMA chain with the constant
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
//                                K chunk with bf16 values; the shared base is a
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
  int k, nseg, S, N, K, G, z, n_sal, n_out;
  uint32_t A_bytes;
};

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

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

// 8 bf16 values (128 + code) of MFMA step t (0..3) for one lane.
__device__ __forceinline__ bf16x8 deq_u4(const u32x4& cd, int t) {
  const uint32_t d = cd[t];
  const uint32_t m = 0x000F000Fu, o = 0x43004300u;
  u32x4 r;
  r[0] = and_or(d, m, o);
  r[1] = and_or(d >> 4, m, o);
  r[2] = and_or(d >> 8, m, o);
  r[3] = and_or(d >> 12, m, o);
  return as_bf16x8(r);
}

__device__ __forceinline__ bf16x8 deq_mwq(const u32x2& q2, uint32_t d3, uint32_t d4, int t, int b) {
  const uint32_t Q = q2[t >> 1];
  u32x4 r;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int P = 4 * (t & 1) + p;
    const int P3 = 4 * t + p;
    uint32_t v = and_or(shr(Q, 2 * P - 2), 0x000C000Cu, 0x43004300u);
    if (b >= 3) v = and_or(shr(d3, P3 - 1), 0x00020002u, v);
    if (b == 4) v = and_or(shr(d4, P3), 0x00010001u, v);
    r[p] = v;
  }
  return as_bf16x8(r);
}

__device__ __forceinline__ bf16x8 deq_u2(const u32x2& c, int t) {
  const uint32_t C = c[t >> 1];
  u32x4 r;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int P = 4 * (t & 1) + p;
    r[p] = and_or(shr(C, 2 * P), 0x00030003u, 0x43004300u);
  }
  return as_bf16x8(r);
}

struct Ctx {
  int row0, rows, e, bits;
};

__device__ __forceinline__ bool setup(const KArgs& p, Ctx& c) {
  int seg, m0;
  if (!find_tile(p.seg_offsets, p.nseg, blockIdx.y, seg, m0)) return false;
  c.row0 = p.seg_offsets[seg] + m0;
  c.rows = min(kRows, p.seg_offsets[seg + 1] - c.row0);
  c.e = seg / p.S;
  c.bits = 4 - (seg % p.S);  // nested planes only
  return true;
}

// Source row of the grouped row `r` of this tile (clamped into the tile).
__device__ __forceinline__ size_t src_row(const KArgs& p, const Ctx& c, int r) {
  const int gi = c.row0 + min(r, c.rows - 1);
  return p.gather ? (size_t)(p.gather[gi] / p.k) : (size_t)gi;
}

// This wavefront's two 16-channel tiles; false if the wavefront has no tile.
template <bool SWIGLU>
__device__ __forceinline__ bool wave_tiles(const KArgs& p, int wv, int& ct0, int& ct1, bool& v1, int& hch) {
  if (SWIGLU) {
    hch = blockIdx.x * 64 + 16 * wv;  // first h channel
    ct0 = hch / 16;
    ct1 = p.N / 32 + hch / 16;
    v1 = true;
    return hch < p.N / 2;
  }
  const int ch = blockIdx.x * 128 + 32 * wv;
  hch = ch;
  ct0 = ch / 16;
  v1 = ch + 16 < p.N;
  ct1 = v1 ? ct0 + 1 : ct0;
  return ch < p.N;
}

// EPI: 0 = bf16 out, 1 = SwiGLU bf16 out, 2 = fp32 out.  acc[rt][tile].
template <int EPI>
__device__ __forceinline__ void store_tiles(const KArgs& p, const Ctx& c, const f32x4 (&acc)[2][2], int ct0,
                                            int ct1, bool v1, int hch, bool two) {
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    if (rt == 1 && !two) break;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = rt * 16 + 4 * (lane >> 4) + r;
      if (row >= c.rows) continue;
      const float v0 = acc[rt][0][r], vv1 = acc[rt][1][r];
      if (EPI == 2) {
        float* orow = static_cast<float*>(p.out) + (size_t)(c.row0 + row) * p.n_out;
        orow[ct0 * 16 + col] = v0;
        if (v1) orow[ct1 * 16 + col] = vv1;
      } else {
        uint16_t* orow = static_cast<uint16_t*>(p.out) + (size_t)(c.row0 + row) * p.n_out;
        if (EPI == 1) {
          orow[hch + col] = f32_to_bf16(v0 * __builtin_amdgcn_rcpf(1.0f + __expf(-v0)) * vv1);
        } else {
          orow[ct0 * 16 + col] = f32_to_bf16(v0);
          if (v1) orow[ct1 * 16 + col] = f32_to_bf16(vv1);
        }
      }
    }
  }
}

// ---------------------------------------------------------------- INT4 / MWQ
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Load from a wave-uniform base plus a 32-bit per-lane byte offset (global
// loads in "scalar base + vector offset" form: no 64-bit address arithmetic).
template <class T>
__device__ __forceinline__ T ldg(const void* ubase, uint32_t voff) {
  return *reinterpret_cast<const T*>(static_cast<const char*>(ubase) + voff);
}

// Weight registers of one K block for one wavefront: INT4 = one 16-byte
// fragment per tile; MWQ = q2 (8 bytes) + d3 + d4 (4 bytes each) per tile.
struct BRegs {
  u32x4 c[2];
  u32x2 q[2];
  uint32_t d3[2], d4[2];
};

template <int FMT, int EPI, int GPB>
__global__ __launch_bounds__(kThreads) void qgemm_q_kernel(KArgs p) {
  constexpr int SPG = 4 / GPB;  // MFMA steps per scale group
  __shared__ u32x4 lds_a[3][2][4][64];  // [slot][row tile][step][lane], 24 KB
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = uniform(tid >> 6);
  Ctx c;
  if (!setup(p, c)) return;  // uniform over the workgroup
  c.row0 = uniform(c.row0);
  c.rows = uniform(c.rows);
  c.e = uniform(c.e);
  c.bits = uniform(c.bits);
  const bool two = c.rows > 16;
  int ct0, ct1, hch;
  bool v1;
  const bool wvalid = wave_tiles<EPI == 1>(p, wv, ct0, ct1, v1, hch);
  const int KB = p.K / 128, NT = p.N / 16;

  // activation staging: this thread carries (row tile rt, step wv, lane) of each K block
  const rsrc_t ar = make_rsrc(p.A, p.A_bytes);
  uint32_t aoff[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
    aoff[rt] = (uint32_t)((src_row(p, c, rt * 16 + (lane & 15)) * p.K + 32 * wv + 8 * (lane >> 4)) * 2);
  // weight and scale streams of this wavefront's two tiles
  constexpr uint32_t CB = FMT == 1 ? 1024 : 512;  // code bytes per tile block
  rsrc_t br[2], r3[2], r4[2], sr[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const size_t tile = (size_t)c.e * NT + (u ? ct1 : ct0);
    br[u] = make_rsrc(p.codes + tile * KB * CB, KB * CB);
    r3[u] = make_rsrc(FMT == 2 ? p.p3 + tile * KB * 256 : nullptr, FMT == 2 ? KB * 256 : 0);
    r4[u] = make_rsrc(FMT == 2 ? p.p4 + tile * KB * 256 : nullptr, FMT == 2 ? KB * 256 : 0);
    sr[u] = make_rsrc(p.scales + (tile * 16) * (size_t)(KB * GPB), 16 * KB * GPB * 2);
  }
  const uint32_t soff = (uint32_t)((lane & 15) * KB * GPB * 2);

  const uint32_t negc = (0xC300u | (uint32_t)p.z) * 0x00010001u;
  const bf16x8 neg = as_bf16x8(u32x4{negc, negc, negc, negc});
  f32x4 acc[2][2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int u = 0; u < 2; ++u) acc[rt][u] = f32x4{};

  // Register rings: weights (and scales) run PFB K blocks ahead in a ring of
  // RB = PFB + 1 slots, activations PFA = 3 ahead in a ring of RA = 4 slots;
  // the loop is unrolled by 8 so every ring index is a compile-time constant.
  constexpr int PFB = 3, RB = PFB + 1, RA = 4;
  static_assert(8 % RB == 0 && 8 % RA == 0, "ring sizes must divide the unroll factor");
  u32x4 ra[RA][2];
  BRegs rb[RB];
  uint16_t rs[RB][2][GPB];

#define QG_ISSUE_A(SLOT, KBI)                                                                        \
  {                                                                                                  \
    ra[SLOT][0] = buf_x4(ar, aoff[0], (KBI) * 256);                                                  \
    if (two) ra[SLOT][1] = buf_x4(ar, aoff[1], (KBI) * 256);                                         \
  }
#define QG_ISSUE_B(SLOT, KBI)                                                                        \
  if (wvalid) {                                                                                      \
    _Pragma("unroll") for (int u = 0; u < 2; ++u) {                                                  \
      if (FMT == 1) {                                                                                \
        rb[SLOT].c[u] = buf_x4(br[u], 16 * lane, (KBI) * CB);                                        \
      } else {                                                                                       \
        rb[SLOT].q[u] = buf_x2(br[u], 8 * lane, (KBI) * CB);                                         \
        rb[SLOT].d3[u] = c.bits >= 3 ? buf_x1(r3[u], 4 * lane, (KBI) * 256) : 0u;                    \
        rb[SLOT].d4[u] = c.bits == 4 ? buf_x1(r4[u], 4 * lane, (KBI) * 256) : 0u;                    \
      }                                                                                              \
      _Pragma("unroll") for (int g = 0; g < GPB; ++g)                                                \
        rs[SLOT][u][g] = buf_u16(sr[u], soff, ((KBI) * GPB + g) * 2);                                \
    }                                                                                                \
  }
#define QG_STAGE(SLOT, KBI)                                                                          \
  {                                                                                                  \
    lds_a[(KBI) % 3][0][wv][lane] = ra[SLOT][0];                                                     \
    if (two) lds_a[(KBI) % 3][1][wv][lane] = ra[SLOT][1];                                            \
  }
  // one scale group (SPG steps starting at T0) for row tile RT: the correction
  // chain first, then each tile's chain starts from it; acc += scale * chain
#define QG_GROUP(J, RT, T0, SLOT3)                                                                   \
  {                                                                                                  \
    f32x4 cr = f32x4{};                                                                              \
    _Pragma("unroll") for (int t = T0; t < T0 + SPG; ++t)                                            \
      cr = mfma16(as_bf16x8(lds_a[SLOT3][RT][t][lane]), neg, cr);                                    \
    _Pragma("unroll") for (int u = 0; u < 2; ++u) {                                                  \
      f32x4 tm = cr;                                                                                 \
      _Pragma("unroll") for (int t = T0; t < T0 + SPG; ++t) {                                        \
        const bf16x8 bv = (FMT == 1) ? deq_u4(rb[(J) % RB].c[u], t)                                  \
                                     : deq_mwq(rb[(J) % RB].q[u], rb[(J) % RB].d3[u], rb[(J) % RB].d4[u], t, c.bits); \
        tm = mfma16(as_bf16x8(lds_a[SLOT3][RT][t][lane]), bv, tm);                                   \
      }                                                                                              \
      const float sv = f16_to_f32(rs[(J) % RB][u][T0 / SPG]);                                               \
      _Pragma("unroll") for (int r = 0; r < 4; ++r) acc[RT][u][r] = __builtin_fmaf(sv, tm[r], acc[RT][u][r]); \
    }                                                                                                \
  }
#define QG_STEP(J)                                                                                   \
  if (kb + J < KB) {                                                                                 \
    const int i = kb + J;                                                                            \
    if (i + PFB < KB) QG_ISSUE_B(((J) + PFB) % RB, i + PFB);                                           \
    if (i + 3 < KB) QG_ISSUE_A((J + 3) % RA, i + 3);                                                 \
    if (i + 1 < KB) QG_STAGE((J + 1) % RA, i + 1);                                                   \
    __syncthreads();                                                                                 \
    if (wvalid) {                                                                                    \
      const int sl = i % 3;                                                                          \
      _Pragma("unroll") for (int t0 = 0; t0 < 4; t0 += SPG) {                                        \
        QG_GROUP(J, 0, t0, sl);                                                                      \
        if (two) QG_GROUP(J, 1, t0, sl);                                                             \
      }                                                                                              \
    }                                                                                                \
  }

  // prologue: weights of K blocks 0..PFB-1 and activations of 0..2 in flight, block 0 staged
#pragma unroll
  for (int j = 0; j < PFB; ++j)
    if (j < KB) QG_ISSUE_B(j % RB, j);
#pragma unroll
  for (int j = 0; j < 3; ++j)
    if (j < KB) QG_ISSUE_A(j, j);
  QG_STAGE(0, 0);
  for (int kb = 0; kb < KB; kb += 8) {
    QG_STEP(0)
    QG_STEP(1)
    QG_STEP(2)
    QG_STEP(3)
    QG_STEP(4)
    QG_STEP(5)
    QG_STEP(6)
    QG_STEP(7)
  }
#undef QG_ISSUE_A
#undef QG_ISSUE_B
#undef QG_STAGE
#undef QG_GROUP
#undef QG_STEP
  if (wvalid) store_tiles<EPI>(p, c, acc, ct0, ct1, v1, hch, two);
}

// -------------------------------------------------------------------- DELTA2
// y = x W_base^T + x D_e^T per wavefront (two 16-channel tiles, up to 32 rows):
// a bf16 MFMA on the base fragments, the biased 2-bit codes with the
// -(128+z) correction chain, the per-channel step applied once at the end,
// and the salient channels as one more exact bf16 K chunk.
template <int EPI>
__global__ __launch_bounds__(kThreads) void qgemm_delta_kernel(KArgs p) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  Ctx c;
  if (!setup(p, c)) return;
  const bool two = c.rows > 16;
  int ct0, ct1, hch;
  bool v1;
  if (!wave_tiles<EPI == 1>(p, wv, ct0, ct1, v1, hch)) return;
  const int NT = p.N / 16, KB = p.K / 128;
  const size_t arow[2] = {src_row(p, c, lane & 15), src_row(p, c, 16 + (lane & 15))};
  const uint16_t* Ap[2] = {p.A + arow[0] * p.K + 8 * (lane >> 4), p.A + arow[1] * p.K + 8 * (lane >> 4)};
  const uint32_t negc = (0xC300u | (uint32_t)p.z) * 0x00010001u;
  const bf16x8 neg = as_bf16x8(u32x4{negc, negc, negc, negc});
  f32x4 accb[2][2], tmp[2][2], corr[2], acc[2][2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    corr[rt] = f32x4{};
#pragma unroll
    for (int u = 0; u < 2; ++u) accb[rt][u] = tmp[rt][u] = f32x4{};
  }
  for (int kb = 0; kb < KB; ++kb) {
    u32x4 a[2][4], bb[2][4];
    u32x2 cd[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int ct = u ? ct1 : ct0;
      cd[u] = *reinterpret_cast<const u32x2*>(p.codes + (((size_t)c.e * NT + ct) * KB + kb) * 512 + 8 * lane);
      if (p.base) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
          bb[u][t] = *reinterpret_cast<const u32x4*>(p.base + ((size_t)ct * KB + kb) * 2048 + 512 * t + 8 * lane);
      }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      a[0][t] = *reinterpret_cast<const u32x4*>(Ap[0] + kb * 128 + 32 * t);
      a[1][t] = two ? *reinterpret_cast<const u32x4*>(Ap[1] + kb * 128 + 32 * t) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        if (rt == 1 && !two) break;
        const bf16x8 av = as_bf16x8(a[rt][t]);
        corr[rt] = mfma16(av, neg, corr[rt]);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          tmp[rt][u] = mfma16(av, deq_u2(cd[u], t), tmp[rt][u]);
          if (p.base) accb[rt][u] = mfma16(av, as_bf16x8(bb[u][t]), accb[rt][u]);
        }
      }
    }
  }
  // salient input channels: one more K chunk of exact bf16 values
  if (p.n_sal > 0) {
    const int nsteps = (p.n_sal + 31) / 32;
    for (int st = 0; st < nsteps; ++st) {
      u32x4 sv[2];
#pragma unroll
      for (int u = 0; u < 2; ++u)
        sv[u] = *reinterpret_cast<const u32x4*>(p.sal_val + (((size_t)c.e * NT + (u ? ct1 : ct0)) * nsteps + st) * 512 +
                                                8 * lane);
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        if (rt == 1 && !two) break;
        const uint16_t* Arow = p.A + arow[rt] * p.K;
        u32x4 av;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          uint32_t v = 0;
#pragma unroll
          for (int w = 0; w < 2; ++w) {
            const int j = 32 * st + 8 * (lane >> 4) + 2 * h + w;
            const int idx = j < p.n_sal ? min(max(p.sal_idx[(size_t)c.e * p.n_sal + j], 0), p.K - 1) : 0;
            v |= (uint32_t)Arow[idx] << (16 * w);
          }
          av[h] = v;
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) accb[rt][u] = mfma16(as_bf16x8(av), as_bf16x8(sv[u]), accb[rt][u]);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const float step = f16_to_f32(p.scales[(size_t)c.e * p.N + (u ? ct1 : ct0) * 16 + (lane & 15)]);
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[rt][u][r] = __builtin_fmaf(step, tmp[rt][u][r] + corr[rt][r], accb[rt][u][r]);
  }
  store_tiles<EPI>(p, c, acc, ct0, ct1, v1, hch, two);
}

template <int FMT, int EPI>
void launch_q(const KArgs& ka, dim3 grid, hipStream_t s) {
  switch (ka.G) {
    case 128: hipLaunchKernelGGL((qgemm_q_kernel<FMT, EPI, 1>), grid, dim3(kThreads), 0, s, ka); break;
    case 64: hipLaunchKernelGGL((qgemm_q_kernel<FMT, EPI, 2>), grid, dim3(kThreads), 0, s, ka); break;
    default: hipLaunchKernelGGL((qgemm_q_kernel<FMT, EPI, 4>), grid, dim3(kThreads), 0, s, ka); break;
  }
}

template <int EPI>
void launch_epi(const KArgs& ka, int fmt, dim3 grid, hipStream_t s) {
  if (fmt == 1) launch_q<1, EPI>(ka, grid, s);
  else if (fmt == 2) launch_q<2, EPI>(ka, grid, s);
  else hipLaunchKernelGGL((qgemm_delta_kernel<EPI>), grid, dim3(kThreads), 0, s, ka);
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
  ka.A_bytes = (uint32_t)((size_t)a.A_rows * w.K * 2);
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
  // a workgroup covers 64 SwiGLU channels or 128 plain channels
  const int gx = swiglu ? (w.N / 2 + 63) / 64 : (w.N + 127) / 128;
  const int gy = (a.M_total + kRows - 1) / kRows + a.nseg;
  dim3 grid(gx, gy);
  if (a.epilogue == 1) launch_epi<1>(ka, w.fmt, grid, s);
  else if (a.epilogue == 2) launch_epi<2>(ka, w.fmt, grid, s);
  else launch_epi<0>(ka, w.fmt, grid, s);
  return hipGetLastError();
}

}  // namespace moe

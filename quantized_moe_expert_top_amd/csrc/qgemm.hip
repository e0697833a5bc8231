// Grouped low-bit GEMM over expert segments (grouped batched expert execution,
// ExactMoE page; "dequantise -> 16-bit GEMM" pipeline equation, D2MoE page).
//
// Row tiles of a segment are located on the device from seg_offsets (the host
// never reads counts back), and every kernel streams the tiled weight layout
// (16 channels x 128 inputs per tile block, see repack.hip) with
// v_mfma_f32_16x16x32_bf16.  The kernels:
//   qgemm_d_kernel  few rows per segment (decode): 16-row tiles, 4 wavefronts
//                   x 2 channel tiles each, activations shared through LDS,
//                   weights and activations prefetched in register rings;
//                   nested MWQ takes all widths of an expert per tile; long K
//                   with few work items splits K (splitk_reduce_kernel).
//   qgemm_p_kernel  many rows per segment: 64-row tiles, each dequantised
//                   weight fragment reused for 64 rows.
//   qgemm_p2_kernel INT4 (and nested MWQ at large batches) with many rows:
//                   128-row x 256-channel tiles fed by LDS-DMA only.
//   qgemm_delta_kernel / qgemm_p2d_kernel  2-bit delta + salient channels +
//                   shared bf16 base (32-row tiles / 128-row LDS-DMA tiles).
//
// Dequantisation is exact and cheap (INT4: seven VALU operations per eight
// weights): a code c is dropped into the low mantissa bits of the bf16 number
// 128 (bits 0x4300), giving exactly 128 + c.  The MFMA accumulates
// sum_k a_k * (128 + c_k) in fp32, a second MFMA chain with the constant
// -(128 + z) adds sum_k a_k * (-(128 + z)), so the sum of the two is exactly
// sum_k a_k * (c_k - z) up to fp32 accumulation rounding.  The group scale (or
// the per-channel step) multiplies that in fp32 once per group.
//   INT4 (ExactMoE W4A16):       w = s[n][k/G] * (c - z)
//   MWQ  (D2MoE MWQ equations):  c_b = 4*q2 + 2*d3*[b>=3] + d4*[b==4]; the
//                                decode kernel never loads the planes its
//                                tile's widths do not need
//   DELTA2 (ME-Switch):          d = step[n] * (c - z) off the salient
//                                channels (their codes were zeroed by the
//                                repack); salient channels are one more MFMA
//                                K chunk with bf16 values; the shared base is a
//                                plain bf16 MFMA on the same A operand
#include <mutex>
#include <type_traits>

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
  float* part;  // split-K partial sums [n_ks][M_total][N] (decode kernel, plain epilogues)
  int k, nseg, S, N, K, G, z, n_sal, n_out, M_total;
  uint32_t A_bytes;
};

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Plain epilogues: EPI 0 bf16, 2 fp32, 3 fp16 (EPI 1, SwiGLU, stores bf16 h).
// A 16-bit output is the fp32 result rounded once.  For fp16 the value passes
// an empty register barrier first (no instruction is emitted): otherwise the
// compiler may contract the conversion into the producing fma as a
// mixed-precision fma that rounds the exact sum straight to fp16, and the fp16
// output would no longer be the fp32 output rounded.
template <int EPI>
__device__ __forceinline__ void store_plain(void* out, size_t i, float v) {
  if (EPI == 2) {
    static_cast<float*>(out)[i] = v;
  } else if (EPI == 3) {
    asm volatile("" : "+v"(v));
    static_cast<uint16_t*>(out)[i] = f32_to_f16(v);
  } else {
    static_cast<uint16_t*>(out)[i] = f32_to_bf16(v);
  }
}

// Locate the row tile `y` (in segment order; tiles of `rows_per_tile` rows)
// -> segment and first row.
// With `stride` > 1, segment s spans seg_offsets[s*stride] .. seg_offsets[(s+1)*stride]
// (all bit-width sub-segments of one expert).
__device__ __forceinline__ bool find_tile(const int32_t* seg_offsets, int nseg, int y, int& seg, int& m0,
                                          int rows_per_tile = kRows, int stride = 1) {
  const int kRows = rows_per_tile;
  const int lane = threadIdx.x & 63;
  int carry = 0;
  for (int s0 = 0; s0 < nseg; s0 += 64) {
    const int s = s0 + lane;
    int tiles = 0;
    if (s < nseg) tiles = (seg_offsets[(s + 1) * stride] - seg_offsets[s * stride] + kRows - 1) / kRows;
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

// 8 bf16 values (128 + code) of MFMA step t (0..3) for one lane.  A code c
// in the low mantissa bits of the bf16 number 128 (bits 0x4300) is exactly
// 128 + c.  INT4: the dword of step t holds element i at bit 16*(i&1) +
// 4*(i>>1); masking the low / high nibble of every byte leaves one code per
// byte, and a byte permute with the constant 0x43 builds each pair
// (elements 2p, 2p+1) as two bf16 values: 7 VALU operations per 8 weights.
__device__ __forceinline__ u32x4 deq_nib(uint32_t d) {
  const uint32_t lo = d & 0x0F0F0F0Fu;         // bytes: e0 e4 e1 e5
  const uint32_t hi = (d >> 4) & 0x0F0F0F0Fu;  // bytes: e2 e6 e3 e7
  const uint32_t K = 0x43434343u;
  u32x4 r;
  r[0] = __builtin_amdgcn_perm(K, lo, 0x04020400u);  // (e0, e1)
  r[1] = __builtin_amdgcn_perm(K, hi, 0x04020400u);  // (e2, e3)
  r[2] = __builtin_amdgcn_perm(K, lo, 0x04030401u);  // (e4, e5)
  r[3] = __builtin_amdgcn_perm(K, hi, 0x04030401u);  // (e6, e7)
  return r;
}
__device__ __forceinline__ bf16x8 deq_u4(const u32x4& cd, int t) { return as_bf16x8(deq_nib(cd[t])); }

// MWQ: c_b = 4*q2 + 2*d3*[b>=3] + d4*[b==4] as 4-bit nibbles in the INT4
// order, from the nested planes' tiled layout (each plane masked and shifted
// by the step: q2 at bits 2-3 of each nibble for even steps, 0-1 for odd ones;
// d3 / d4 at bit 3 - t), then the INT4 conversion.
__device__ __forceinline__ uint32_t mwq_nib(const u32x2& q2, uint32_t d3, uint32_t d4, int t, int b) {
  const uint32_t Q = q2[t >> 1];
  uint32_t n = ((t & 1) ? (Q << 2) : Q) & 0xCCCCCCCCu;
  if (b >= 3) n |= shr(d3, 2 - t) & 0x22222222u;
  if (b == 4) n |= shr(d4, 3 - t) & 0x11111111u;
  return n;
}
__device__ __forceinline__ u32x4 deq_mwq_bits(const u32x2& q2, uint32_t d3, uint32_t d4, int t, int b) {
  return deq_nib(mwq_nib(q2, d3, d4, t, b));
}
__device__ __forceinline__ bf16x8 deq_mwq(const u32x2& q2, uint32_t d3, uint32_t d4, int t, int b) {
  return as_bf16x8(deq_mwq_bits(q2, d3, d4, t, b));
}
__device__ __forceinline__ u32x4 and4(const u32x4& v, uint32_t m) { return u32x4{v[0] & m, v[1] & m, v[2] & m, v[3] & m}; }

__device__ __forceinline__ bf16x8 deq_u2(const u32x2& c, int t) {
  const uint32_t C = c[t >> 1];
  u32x4 r;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int P = 4 * (t & 1) + p;
    r[p] = (shr(C, 2 * P) & 0x00030003u) | 0x43004300u;
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
__device__ __forceinline__ bool wave_tiles(const KArgs& p, int wv, int& ct0, int& ct1, bool& v1, int& hch,
                                           int cg = blockIdx.x) {
  if (SWIGLU) {
    hch = cg * 64 + 16 * wv;  // first h channel
    ct0 = hch / 16;
    ct1 = p.N / 32 + hch / 16;
    v1 = true;
    return hch < p.N / 2;
  }
  const int ch = cg * 128 + 32 * wv;
  hch = ch;
  ct0 = ch / 16;
  v1 = ch + 16 < p.N;
  ct1 = v1 ? ct0 + 1 : ct0;
  return ch < p.N;
}

// EPI: 0 = bf16 out, 1 = SwiGLU bf16 out, 2 = fp32 out, 3 = fp16 out.  acc[rt][tile].
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
      const size_t o = (size_t)(c.row0 + row) * p.n_out;
      if (EPI == 1) {
        static_cast<uint16_t*>(p.out)[o + hch + col] = f32_to_bf16(v0 * __builtin_amdgcn_rcpf(1.0f + __expf(-v0)) * vv1);
      } else {
        store_plain<EPI>(p.out, o + ct0 * 16 + col, v0);
        if (v1) store_plain<EPI>(p.out, o + ct1 * 16 + col, vv1);
      }
    }
  }
}

// ---------------------------------------------------------------- INT4 / MWQ
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Weight registers of one K block for one wavefront: INT4 = one 16-byte
// fragment per tile; MWQ = q2 (8 bytes) + d3 + d4 (4 bytes each) per tile.
struct BRegs {
  u32x4 c[2];
  u32x4 c8[2];  // 8-bit codes: MFMA steps 2 and 3 (steps 0 and 1 in c)
  u32x2 q[2];
  uint32_t d3[2], d4[2];
};

// Two floats that are exact in bf16 (here integers of at most 8 significant
// bits) as a bf16 pair, the first in the low half: their high halves.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, hi), __builtin_bit_cast(uint32_t, lo), 0x07060302u);
}

// 8-bit codes: the 8 codes of MFMA step t (bytes 8t .. 8t + 7 of the lane's 32)
// become the exact bf16 values c - z (|c - z| <= 255 needs 8 significant bits).
__device__ __forceinline__ bf16x8 deq_u8(const u32x4& lo, const u32x4& hi, int t, float z) {
  const u32x4& v = t < 2 ? lo : hi;
  u32x4 r;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t d = v[2 * (t & 1) + h];
    r[2 * h] = pack_bf16x2((float)(d & 0xFFu) - z, (float)((d >> 8) & 0xFFu) - z);
    r[2 * h + 1] = pack_bf16x2((float)((d >> 16) & 0xFFu) - z, (float)(d >> 24) - z);
  }
  return as_bf16x8(r);
}

// ------------------------------------------------------------ decode, deep
// One workgroup per (16-row tile of one segment, channel group of 64 SwiGLU /
// 128 plain channels); each wavefront owns two 16-channel tiles and streams
// all of K.  Weights, scales and activations run PF = 3 K blocks ahead in
// register rings (the memory counter retires loads in issue order, so the
// activations, issued first, never make a wavefront wait for weights it does
// not need yet).  Per scale group, one bias-correction chain (the activation
// fragments times -(128 + z)) seeds the chains of both tiles on the
// dequantised codes.  Workgroups are numbered so that the row tiles of one
// segment and channel group run on one XCD, back to back: a segment of more
// than 16 rows reads its weights from HBM once and from that XCD's L2 after.
//
// The steady-state loop has no branch: every load is issued unconditionally
// (a wavefront without a tile, and a bit plane the segment's width does not
// use, read through a zero-size buffer resource, which returns zeros without
// touching memory), so the compiler can count the loads in flight and wait
// only for the one a step needs; a branch in the loop makes it wait for all
// of them.  The last blocks run in a guarded tail.
//
// FMT 4 (nested MWQ, all widths of an expert in one tile): a tile takes 16
// rows of the expert's three sub-segments (b = 4, 3, 2, adjacent in the
// grouped order), loads each bit plane once for all of them, and runs one
// MFMA per width present in the wavefront's rows: the activation rows of width
// b (the others masked to zero) times the codes truncated to b bits.  Every
// width has the same scale and zero point, so the one correction chain over
// all rows still applies, and each row's sum is the one it would get in its
// own sub-segment (the other widths add exact zeros).
//
// Split K (n_ks > 1, plain epilogues only): work item ks covers K blocks
// [ks * kb_per, ...) and stores its fp32 sums in p.part[ks]; splitk_reduce_kernel
// adds the n_ks partials in order.  It gives a long-K GEMM with few channel
// groups and row tiles (the down projection of a decode batch) enough
// wavefronts to keep loads in flight.
//
// FMT 5 (static width per expert, from `tab`): the codes, shifted to 4 bits,
// are stored as the nested planes, only the first b of them per tile block
// (256 * b bytes); the correction uses z << (4 - b) and the group scale is
// multiplied by 2^(b - 4), both exact.  An 8-bit expert keeps plain bytes (32
// per lane and tile block, 2 KB per block) that convert straight to the exact
// bf16 values c - z: no correction chain.
// The per-expert table travels only with FMT 5: 1.5 KB of launch arguments
// would slow every launch of the other formats.
struct NoTab {};
template <int FMT>
using TabOf = typename std::conditional<FMT == 5 || FMT == 6, XTab, NoTab>::type;
__device__ __forceinline__ int tab_bits(const XTab& t, int e) { return t.bits[e]; }
__device__ __forceinline__ int tab_zero(const XTab& t, int e) { return t.zero[e]; }
__device__ __forceinline__ size_t tab_off(const XTab& t, int e) { return t.off[e]; }
__device__ __forceinline__ int tab_bits(const NoTab&, int) { return 4; }
__device__ __forceinline__ int tab_zero(const NoTab&, int) { return 0; }
__device__ __forceinline__ size_t tab_off(const NoTab&, int) { return 0; }

#ifndef QD_PF
#define QD_PF 3  // K blocks of weights in flight per wavefront
#endif
template <int FMT, int EPI, int GPB>
__global__ __launch_bounds__(kThreads) void qgemm_d_kernel(KArgs p, int n_cg, int n_rt, int n_ks, int kb_per,
                                                           TabOf<FMT> tab) {
  constexpr bool MW = FMT != 1;                // nested bit planes
  constexpr bool FU = FMT == 4;                // all widths of an expert per tile
  constexpr bool FX = FMT == 5 || FMT == 6;    // one width per expert (6: the 8-bit experts, 5: the others)
  constexpr int SPG = 4 / GPB;                 // MFMA steps per scale group
  constexpr int PF = QD_PF, R = QD_PF + 1;     // prefetch distance, ring size
  __shared__ u32x4 lds_a[3][4][64];            // [slot][step][lane], 12 KB
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = uniform(tid >> 6);

  const int per_xcd = gridDim.x / 8;
  const int item = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  const int cgk = item / n_rt, rtile = item % n_rt;  // (channel group, K split) major, row tile minor
  const int cg = n_ks == 1 ? cgk : cgk / n_ks, ks = n_ks == 1 ? 0 : cgk % n_ks;
  if (cg >= n_cg) return;
  int seg, m0;
  const int SS = FU ? p.S : 1;  // sub-segments per tile segment
  if (!find_tile(p.seg_offsets, p.nseg / SS, rtile, seg, m0, 16, SS)) return;
  Ctx c;
  c.row0 = uniform(p.seg_offsets[seg * SS] + m0);
  c.rows = uniform(min(16, p.seg_offsets[(seg + 1) * SS] - c.row0));
  c.e = uniform(FU ? seg : seg / p.S);
  c.bits = uniform(4 - (seg % p.S));
  // FMT 4: rows [.., o1) have b = 4, [o1, o2) b = 3, [o2, ..) b = 2
  const int o1 = FU ? uniform(p.seg_offsets[seg * SS + 1]) : 0;
  const int o2 = FU ? uniform(p.seg_offsets[seg * SS + 2]) : 0;
  if (FX) c.bits = uniform(tab_bits(tab, c.e));
  // the 8-bit experts' larger register ring runs in a launch of its own
  if (FX && ((c.bits == 8) != (FMT == 6))) return;
  const bool need3 = FU ? c.row0 < o2 : c.bits >= 3;
  const bool need4 = FU ? c.row0 < o1 : c.bits == 4;
  const int lrow = c.row0 + (lane & 15);
  const uint32_t m4 = lrow < o1 ? ~0u : 0u, m3 = (lrow >= o1 && lrow < o2) ? ~0u : 0u, m2 = lrow >= o2 ? ~0u : 0u;
  int ct0, ct1, hch;
  bool v1;
  const bool wvalid = wave_tiles<EPI == 1>(p, wv, ct0, ct1, v1, hch, cg);
  const int KBt = p.K / 128, NT = p.N / 16;
  const int kb_lo = ks * kb_per;               // this split's first K block
  const int KB = min(kb_per, KBt - kb_lo);     // and its number of K blocks (>= 1)

  // activations: this thread carries (step wv, lane) of each K block
  const rsrc_t ar = make_rsrc(p.A, p.A_bytes);
  const uint32_t aoff = (uint32_t)((src_row(p, c, lane & 15) * p.K + 32 * wv + 8 * (lane >> 4)) * 2 + kb_lo * 256);
  // tile block: INT4 codes, or the q2 / d3 / d4 planes at 0 / 512 / 768 (FMT 5: 256 * b bytes)
  const uint32_t CB = FX ? uniform(256 * c.bits) : 1024u;
  const uint8_t* codes_e = FX ? p.codes + tab_off(tab, c.e) * 256 : p.codes;  // FMT 5: this expert's blocks
  rsrc_t br[2], r3[2], r4[2], sr[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const size_t tile = (size_t)c.e * NT + (wvalid ? (u ? ct1 : ct0) : 0);
    const size_t tb = (FX ? tile - (size_t)c.e * NT : tile) * KBt + kb_lo;  // first tile block of the split
    br[u] = make_rsrc(codes_e + tb * CB, wvalid ? KB * CB : 0);
    r3[u] = make_rsrc(MW ? codes_e + tb * CB + 512 : nullptr, MW && wvalid && need3 ? KB * CB - 512 : 0);
    r4[u] = make_rsrc(MW ? codes_e + tb * CB + 768 : nullptr, MW && wvalid && need4 ? KB * CB - 768 : 0);
    // scales [channel][group]: rows of KBt * GPB entries, this split's columns from kb_lo * GPB
    sr[u] = make_rsrc(p.scales + (tile * 16) * (size_t)(KBt * GPB) + (size_t)kb_lo * GPB,
                      wvalid ? (16 * KBt * GPB - kb_lo * GPB) * 2 : 0);
  }
  const uint32_t soff = (uint32_t)((lane & 15) * KBt * GPB * 2);
  const uint32_t zl = FX ? (c.bits < 8 ? uniform(tab_zero(tab, c.e) << (4 - c.bits)) : 0u) : (uint32_t)p.z;
  const uint32_t negc = (0xC300u | zl) * 0x00010001u;
  const bf16x8 neg = as_bf16x8(u32x4{negc, negc, negc, negc});
  const float smul = (FX && c.bits < 8) ? __builtin_ldexpf(1.0f, c.bits - 4) : 1.0f;  // 4-bit-shifted codes: exact
  const float zf = FX ? (float)tab_zero(tab, c.e) : 0.f;  // 8-bit experts

  f32x4 acc[2] = {f32x4{}, f32x4{}};
  u32x4 ra[R];
  BRegs rb[R];
  uint32_t rsc[R][2][GPB];  // one register per scale: packing two would wait for both loads

#define QD_ISSUE(SLOT, KBI)                                                              \
  {                                                                                      \
    const int kbi = (KBI);                                                               \
    ra[SLOT] = buf_x4(ar, aoff, kbi * 256);                                              \
    _Pragma("unroll") for (int u = 0; u < 2; ++u) {                                      \
      if (FMT == 1) {                                                                    \
        rb[SLOT].c[u] = buf_x4(br[u], 16 * lane, kbi * CB);                              \
      } else if (B8) {                                                                   \
        rb[SLOT].c[u] = buf_x4(br[u], 32 * lane, kbi * CB);                              \
        rb[SLOT].c8[u] = buf_x4(br[u], 32 * lane + 16, kbi * CB);                        \
      } else {                                                                           \
        rb[SLOT].q[u] = buf_x2(br[u], 8 * lane, kbi * CB);                               \
        rb[SLOT].d3[u] = L3 ? buf_x1(r3[u], 4 * lane, kbi * CB) : 0u;                    \
        rb[SLOT].d4[u] = L4 ? buf_x1(r4[u], 4 * lane, kbi * CB) : 0u;                    \
      }                                                                                  \
      _Pragma("unroll") for (int g = 0; g < GPB; ++g)                                    \
          rsc[SLOT][u][g] = buf_u16(sr[u], soff, (kbi * GPB + g) * 2);                   \
    }                                                                                    \
  }
  // block I (ring slot J) from LDS stage I % 3
#define QD_COMPUTE(J, I)                                                                                 \
  {                                                                                                      \
    const int sl = (I) % 3;                                                                              \
    _Pragma("unroll") for (int t0 = 0; t0 < 4; t0 += SPG) {                                              \
      f32x4 cr = f32x4{};                                                                                \
      _Pragma("unroll") for (int t = t0; t < t0 + SPG; ++t) if (!B8) cr = mfma16(as_bf16x8(lds_a[sl][t][lane]), neg, cr); \
      f32x4 tm[2] = {cr, cr};                                                                            \
      _Pragma("unroll") for (int t = t0; t < t0 + SPG; ++t) {                                            \
        const u32x4 araw = lds_a[sl][t][lane];                                                           \
        const bf16x8 av = as_bf16x8(araw);                                                               \
        _Pragma("unroll") for (int u = 0; u < 2; ++u) {                                                  \
          if (FU) {                                                                                      \
            const u32x4 b4 = deq_mwq_bits(rb[J].q[u], rb[J].d3[u], rb[J].d4[u], t, 4);                   \
            tm[u] = mfma16(as_bf16x8(and4(araw, m4)), as_bf16x8(b4), tm[u]);                             \
            tm[u] = mfma16(as_bf16x8(and4(araw, m3)), as_bf16x8(and4(b4, 0xFFFEFFFEu)), tm[u]);          \
            tm[u] = mfma16(as_bf16x8(and4(araw, m2)), as_bf16x8(and4(b4, 0xFFFCFFFCu)), tm[u]);          \
          } else {                                                                                       \
            const bf16x8 bv = (FMT == 1) ? deq_u4(rb[J].c[u], t)                                         \
                              : B8       ? deq_u8(rb[J].c[u], rb[J].c8[u], t, zf)                        \
                                         : deq_mwq(rb[J].q[u], rb[J].d3[u], rb[J].d4[u], t, BW ? BW : 4); \
            tm[u] = mfma16(av, bv, tm[u]);                                                               \
          }                                                                                              \
        }                                                                                                \
      }                                                                                                  \
      const int g = t0 / SPG;                                                                            \
      _Pragma("unroll") for (int u = 0; u < 2; ++u) {                                                    \
        const float sv = f16_to_f32((uint16_t)rsc[J][u][g]) * smul;                                      \
        _Pragma("unroll") for (int r = 0; r < 4; ++r) acc[u][r] = __builtin_fmaf(sv, tm[u][r], acc[u][r]); \
      }                                                                                                  \
    }                                                                                                    \
  }
  // steady state: blocks i + PF and i + 1 exist
#define QD_STEP_U(J)                                                   \
  {                                                                    \
    const int i = kb0 + (J);                                           \
    QD_ISSUE(((J) + PF) % R, i + PF);                                  \
    lds_a[(i + 1) % 3][wv][lane] = ra[((J) + 1) % R];                  \
    __syncthreads();                                                   \
    QD_COMPUTE(J, i);                                                  \
  }
#define QD_STEP(J)                                                     \
  if (kb0 + (J) < KB) {                                                \
    const int i = kb0 + (J);                                           \
    if (i + PF < KB) QD_ISSUE(((J) + PF) % R, i + PF);                 \
    if (i + 1 < KB) lds_a[(i + 1) % 3][wv][lane] = ra[((J) + 1) % R];  \
    __syncthreads();                                                   \
    QD_COMPUTE(J, i);                                                  \
  }

  // The K loop, once per code width known at compile time (BW = 2, 3, 4: a
  // width per tile, FMT 2 and 5; 0 otherwise): a narrower tile neither loads
  // nor decodes the planes it does not have.
  auto k_loop = [&](auto bw_tag) {
    constexpr int BW = decltype(bw_tag)::value;
    constexpr bool B8 = BW == 8;                            // plain 8-bit codes
    constexpr bool L3 = BW != 2 && !B8, L4 = BW == 0 || BW == 4;  // d3 / d4 planes loaded
    // prologue: activations and weights of K blocks 0..PF-1 in flight, block 0 staged
#pragma unroll
    for (int j = 0; j < PF; ++j)
      if (j < KB) QD_ISSUE(j, j);
    lds_a[0][wv][lane] = ra[0];
    int kb0 = 0;
    for (; kb0 + R + PF <= KB; kb0 += R) {
#pragma unroll
      for (int j_ = 0; j_ < R; ++j_) QD_STEP_U(j_)
    }
    for (; kb0 < KB; kb0 += R) {
#pragma unroll
      for (int j_ = 0; j_ < R; ++j_) QD_STEP(j_)
    }
  };
  if constexpr (FMT == 6) {
    k_loop(std::integral_constant<int, 8>{});
  } else if constexpr (FX) {
    if (c.bits == 2) k_loop(std::integral_constant<int, 2>{});
    else if (c.bits == 3) k_loop(std::integral_constant<int, 3>{});
    else k_loop(std::integral_constant<int, 4>{});
  } else if constexpr (FMT == 2) {
    if (c.bits == 2) k_loop(std::integral_constant<int, 2>{});
    else if (c.bits == 3) k_loop(std::integral_constant<int, 3>{});
    else k_loop(std::integral_constant<int, 4>{});
  } else {
    k_loop(std::integral_constant<int, 0>{});
  }
#undef QD_ISSUE
#undef QD_COMPUTE
#undef QD_STEP_U
#undef QD_STEP
  if (!wvalid) return;
  const int col = lane & 15;
  if (EPI != 1 && n_ks > 1) {
    float* part = p.part + (size_t)ks * p.M_total * p.N;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 4 * (lane >> 4) + r;
      if (row >= c.rows) continue;
      float* orow = part + (size_t)(c.row0 + row) * p.N;
      orow[ct0 * 16 + col] = acc[0][r];
      if (v1) orow[ct1 * 16 + col] = acc[1][r];
    }
    return;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = 4 * (lane >> 4) + r;
    if (row >= c.rows) continue;
    const size_t o = (size_t)(c.row0 + row) * p.n_out;
    if (EPI == 1) {
      const float g = acc[0][r];
      static_cast<uint16_t*>(p.out)[o + hch + col] = f32_to_bf16(g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * acc[1][r]);
    } else {
      store_plain<EPI>(p.out, o + ct0 * 16 + col, acc[0][r]);
      if (v1) store_plain<EPI>(p.out, o + ct1 * 16 + col, acc[1][r]);
    }
  }
}

// -------------------------------------------------------------------- DELTA2
// y = x W_base^T + x D_e^T per wavefront (two 16-channel tiles, up to 32 rows):
// a bf16 MFMA on the base fragments, the biased 2-bit codes with the
// -(128+z) correction chain, the per-channel step applied once at the end,
// and the salient channels as one more exact bf16 K chunk.
template <int EPI, bool BASE>
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
  // Operands of one K block; block kb + 1 is loaded while block kb is
  // multiplied.  No branch in the loop (a branch makes the compiler wait for
  // every load in flight): buffer loads with per-lane offsets fixed and the
  // K block in the scalar offset; the second row tile is always loaded (its
  // rows are clamped into the segment and never stored).
  struct DBlk {
    u32x4 a[2][4], bb[2][4];
    u32x2 cd[2];
  };
  const rsrc_t ar = make_rsrc(p.A, p.A_bytes);
  const uint32_t aoff[2] = {(uint32_t)(arow[0] * p.K * 2 + 16 * (lane >> 4)),
                            (uint32_t)(arow[1] * p.K * 2 + 16 * (lane >> 4))};
  rsrc_t crs[2], brs[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int ct = u ? ct1 : ct0;
    crs[u] = make_rsrc(p.codes + ((size_t)c.e * NT + ct) * KB * 512, KB * 512);
    brs[u] = make_rsrc(BASE ? p.base + (size_t)ct * KB * 2048 : nullptr, BASE ? KB * 4096 : 0);
  }
  auto load_blk = [&](DBlk& d, int kb) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      d.a[0][t] = buf_x4(ar, aoff[0], kb * 256 + 64 * t);
      d.a[1][t] = buf_x4(ar, aoff[1], kb * 256 + 64 * t);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      d.cd[u] = buf_x2(crs[u], 8 * lane, kb * 512);
      if (BASE)
#pragma unroll
        for (int t = 0; t < 4; ++t) d.bb[u][t] = buf_x4(brs[u], 16 * lane, kb * 4096 + 1024 * t);
    }
  };
  auto mul_blk = [&](const DBlk& d) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const bf16x8 av = as_bf16x8(d.a[rt][t]);
        corr[rt] = mfma16(av, neg, corr[rt]);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          tmp[rt][u] = mfma16(av, deq_u2(d.cd[u], t), tmp[rt][u]);
          if (BASE) accb[rt][u] = mfma16(av, as_bf16x8(d.bb[u][t]), accb[rt][u]);
        }
      }
    }
  };
  DBlk d0, d1;
  load_blk(d0, 0);
  int kb = 0;
  for (; kb + 3 <= KB; kb += 2) {  // steady state: blocks kb + 1, kb + 2 exist
    load_blk(d1, kb + 1);
    mul_blk(d0);
    load_blk(d0, kb + 2);
    mul_blk(d1);
  }
  if (kb + 1 < KB) {
    load_blk(d1, kb + 1);
    mul_blk(d0);
    mul_blk(d1);
  } else {
    mul_blk(d0);
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

// ------------------------------------------------------------------ prefill
// Large row tiles for segments with many rows.  A workgroup of WR x WC
// wavefronts covers MT = 64 * WR rows x 16 * WC SwiGLU channels (32 * WC
// plain channels); wavefront (wm, wn) owns 64 rows (4 MFMA row tiles) and two
// 16-channel tiles (the gate tile and its up tile for SwiGLU, else two
// neighbouring tiles), so each dequantised weight fragment feeds 4 MFMAs.
// The activation rows of a K block are gathered once per workgroup into a
// double-buffered LDS tile; while staging them the loader threads also sum
// each row over every scale group (v_dot2 with (1, 1)), and that row sum
// times -(128 + z) starts each group's MFMA chain, which removes the +128 bias
// of the dequantised codes without a separate correction chain.  Workgroups
// are numbered in groups of row tiles per XCD (L2 reuse of both operands).
//
// LDS slot of (row r of a 16-row tile, MFMA step t, 8-wide k group g4) in a
// staged activation block: the MFMA operand layout (slot = r + 16 * g4) with
// the row rotated by 4 * t, so that the loader's stores (four rows x four
// steps per 16 lanes) fall in distinct banks; readers apply the same map.
__device__ __forceinline__ int a_slot(int r, int t, int g4) { return ((r + 4 * t) & 15) + 16 * g4; }

template <int FMT, int EPI, int GPB, int WR, int WC>
__global__ __launch_bounds__(64 * WR * WC, 8 / (WR * WC)) void qgemm_p_kernel(KArgs p, int n_nblk, int n_mt, int GM) {
  constexpr int NT_ = 64 * WR * WC;    // threads
  constexpr int RT = 4, UT = 2;        // MFMA row tiles, channel tiles per wavefront
  constexpr int MT = 64 * WR;          // rows per workgroup
  constexpr int SPG = 4 / GPB;         // MFMA steps per scale group
  constexpr int NCH = MT * 16 / NT_;   // 16-byte chunks per loader thread per K block
  constexpr int TPR = 16 / NCH;        // loader threads per row (4 or 8)
  static_assert(TPR == 4 || TPR == 8, "row sums reduce over 4 or 8 lanes");
  static_assert(NT_ == MT * TPR, "one loader thread per (row, chunk group)");
  __shared__ u32x4 lds_a[2][MT / 16][4][64];
  __shared__ __attribute__((aligned(16))) float lds_r[2][GPB][MT];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = uniform(tid >> 6), wm = wv / WC, wn = wv % WC;

  // XCD-aware numbering: workgroup L runs on XCD L % 8; each XCD gets a
  // contiguous range of items, ordered (group of GM row tiles, channel block,
  // row tile): the GM row tiles of a group share each channel block's weights
  // and keep their activation rows in that XCD's L2 across channel blocks
  // (GM = all row tiles when the weights outweigh the activations).
  const int per_xcd = gridDim.x / 8;
  const int item = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  const int grp = item / (GM * n_nblk), rem = item % (GM * n_nblk);
  const int nb = rem / GM, mt = grp * GM + rem % GM;
  if (mt >= n_mt) return;
  int seg, m0;
  if (!find_tile(p.seg_offsets, p.nseg, mt, seg, m0, MT)) return;
  const int row0 = uniform(p.seg_offsets[seg] + m0);
  const int rows = uniform(min(MT, p.seg_offsets[seg + 1] - row0));
  const int e = uniform(seg / p.S);
  const int bits = uniform(4 - (seg % p.S));
  const int KB = p.K / 128, NT = p.N / 16;

  // this wavefront's 2 channel tiles
  int ct[UT];
  bool cv;
  int hch0 = 0;
  if (EPI == 1) {
    hch0 = nb * 16 * WC + 16 * wn;
    ct[0] = hch0 / 16;
    ct[1] = NT / 2 + hch0 / 16;
    cv = hch0 < p.N / 2;
  } else {
    ct[0] = nb * 2 * WC + 2 * wn;
    ct[1] = ct[0] + 1;
    cv = ct[0] < NT;
  }
  const bool cv1 = EPI == 1 ? cv : ct[1] < NT;
  if (!cv) ct[0] = 0;  // never stored; keeps the loads in bounds
  if (!cv1) ct[1] = 0;

  // activation loader: thread -> row lr, chunks [part*NCH, part*NCH + NCH) of each K block
  const int lr = tid / TPR, part = tid % TPR;
  const rsrc_t ar = make_rsrc(p.A, p.A_bytes);
  const uint32_t aoff = (uint32_t)((src_row(p, Ctx{row0, rows, e, bits}, lr) * p.K + 8 * part * NCH) * 2);

  constexpr uint32_t CB = 1024;  // tile block: INT4 codes, or the q2 / d3 / d4 planes at 0 / 512 / 768
  rsrc_t br[UT], r3[UT], r4[UT], sr[UT];
#pragma unroll
  for (int u = 0; u < UT; ++u) {
    const size_t tile = (size_t)e * NT + ct[u];
    br[u] = make_rsrc(p.codes + tile * KB * CB, KB * CB);
    r3[u] = make_rsrc(FMT == 2 ? p.codes + tile * KB * CB + 512 : nullptr, FMT == 2 ? KB * CB - 512 : 0);
    r4[u] = make_rsrc(FMT == 2 ? p.codes + tile * KB * CB + 768 : nullptr, FMT == 2 ? KB * CB - 768 : 0);
    sr[u] = make_rsrc(p.scales + (tile * 16) * (size_t)(KB * GPB), 16 * KB * GPB * 2);
  }
  const uint32_t soff = (uint32_t)((lane & 15) * KB * GPB * 2);
  const float negz = -(128.0f + (float)p.z);

  f32x4 acc[RT][UT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int u = 0; u < UT; ++u) acc[rt][u] = f32x4{};

  // Register rings: activations and weights run PF K blocks ahead (the
  // activations issued first: the memory counter retires loads in issue
  // order); the loop is unrolled by R so that ring slots are constants.
  constexpr int PF = 3, R = 4;
  u32x4 ra[R][NCH];
  BRegs rb[R];          // per slot: tiles 0, 1 in c[0], c[1] (or q / d3 / d4)
  uint16_t rs[R][UT][GPB];

  auto issue_a = [&](int slot, int kb) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) ra[slot][c] = buf_x4(ar, aoff + 16 * c, kb * 256);
  };
  auto stage_a = [&](int slot, int buf) {
    float part_sum[GPB];
#pragma unroll
    for (int g = 0; g < GPB; ++g) part_sum[g] = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int ch = part * NCH + c;        // 16-byte chunk of the 128-wide K block
      const int t = ch / 4, g4 = ch % 4;
      lds_a[buf][lr / 16][t][a_slot(lr % 16, t, g4)] = ra[slot][c];
      const int grp = (8 * ch) / (128 / GPB);
      float sacc = part_sum[grp];
#pragma unroll
      for (int h = 0; h < 4; ++h) sacc = add_bf16_pair(ra[slot][c][h], sacc);
      part_sum[grp] = sacc;
    }
    // the TPR threads of a row are lanes TPR*j .. TPR*j + TPR-1: after two
    // quad permutes every lane holds its quad's total; for TPR = 8 a
    // half-row mirror (lane i <- lane 7 - i within each 8 lanes) adds the
    // other quad, so lane 0 of the 8 holds the row's total
#pragma unroll
    for (int g = 0; g < GPB; ++g) {
      float v = part_sum[g];
      v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));  // [1,0,3,2]
      v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));  // [2,3,0,1]
      if (TPR == 8)
        v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, true));  // row_half_mirror
      if (part == 0) lds_r[buf][g][lr] = v * negz;
    }
  };
  auto issue_b = [&](int slot, int kb) {
#pragma unroll
    for (int u = 0; u < UT; ++u) {
      if (FMT == 1) {
        rb[slot].c[u] = buf_x4(br[u], 16 * lane, kb * CB);
      } else {
        rb[slot].q[u] = buf_x2(br[u], 8 * lane, kb * CB);
        rb[slot].d3[u] = bits >= 3 ? buf_x1(r3[u], 4 * lane, kb * CB) : 0u;
        rb[slot].d4[u] = bits == 4 ? buf_x1(r4[u], 4 * lane, kb * CB) : 0u;
      }
#pragma unroll
      for (int g = 0; g < GPB; ++g) rs[slot][u][g] = buf_u16(sr[u], soff, (kb * GPB + g) * 2);
    }
  };
  auto compute = [&](int slot, int buf) {
#pragma unroll
    for (int g = 0; g < GPB; ++g) {
      // bias correction of this group (row sum * -(128 + z)) seeds both tiles' chains
      f32x4 tmp[RT][UT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const f32x4 rv = *reinterpret_cast<const f32x4*>(&lds_r[buf][g][wm * 64 + 16 * rt + 4 * (lane >> 4)]);
#pragma unroll
        for (int u = 0; u < UT; ++u) tmp[rt][u] = rv;
      }
      // per step: both tiles' fragments dequantised once, each used by 4 MFMAs
#pragma unroll
      for (int tt = 0; tt < SPG; ++tt) {
        const int t = g * SPG + tt;
        bf16x8 bv[UT];
#pragma unroll
        for (int u = 0; u < UT; ++u)
          bv[u] = (FMT == 1) ? deq_u4(rb[slot].c[u], t)
                             : deq_mwq(rb[slot].q[u], rb[slot].d3[u], rb[slot].d4[u], t, bits);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const bf16x8 av = as_bf16x8(lds_a[buf][wm * RT + rt][t][a_slot(lane & 15, t, lane >> 4)]);
#pragma unroll
          for (int u = 0; u < UT; ++u) tmp[rt][u] = mfma16(av, bv[u], tmp[rt][u]);
        }
      }
#pragma unroll
      for (int u = 0; u < UT; ++u) {
        const float sv = f16_to_f32(rs[slot][u][g]);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[rt][u][r] = __builtin_fmaf(sv, tmp[rt][u][r], acc[rt][u][r]);
      }
    }
  };


  // prologue: activations and weights of blocks 0..PF-1 in flight, block 0 staged
#pragma unroll
  for (int j = 0; j < PF; ++j)
    if (j < KB) {
      issue_a(j, j);
      issue_b(j, j);
    }
  stage_a(0, 0);
  __syncthreads();
#define QP_STEP(J)                                      \
  if (kb + (J) < KB) {                                  \
    const int i = kb + (J);                             \
    if (i + PF < KB) {                                  \
      issue_a(((J) + PF) % R, i + PF);                  \
      issue_b(((J) + PF) % R, i + PF);                  \
    }                                                   \
    compute((J) % R, i & 1);                            \
    if (i + 1 < KB) stage_a(((J) + 1) % R, (i + 1) & 1); \
    __syncthreads();                                    \
  }
  for (int kb = 0; kb < KB; kb += R) {
    static_assert(R == 4, "the loop below is unrolled by 4");
    QP_STEP(0)
    QP_STEP(1)
    QP_STEP(2)
    QP_STEP(3)
  }
#undef QP_STEP

  // epilogue
  const int col = lane & 15;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = wm * 64 + 16 * rt + 4 * (lane >> 4) + r;
      if (row >= rows) continue;
      if (EPI == 1) {
        if (!cv) continue;
        uint16_t* orow = static_cast<uint16_t*>(p.out) + (size_t)(row0 + row) * p.n_out;
        const float g = acc[rt][0][r], up = acc[rt][1][r];
        orow[hch0 + col] = f32_to_bf16(g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * up);
      } else {
#pragma unroll
        for (int u = 0; u < UT; ++u) {
          if (!(u ? cv1 : cv)) continue;
          const size_t o = (size_t)(row0 + row) * p.n_out + ct[u] * 16 + col;
          store_plain<EPI>(p.out, o, acc[rt][u][r]);
        }
      }
    }
  }
}

// ------------------------------------------------------- prefill, LDS-DMA
// INT4 and nested MWQ with many rows per segment.  One workgroup per (64-row
// tile, 256-channel block) of 4 wavefronts, two workgroups per CU (or, with 4
// scale groups per K block, per 128-row tile of 8 wavefronts); wavefront
// (wm, wn) owns 64 rows x 4 channel tiles, so every activation fragment read
// from LDS feeds 4 MFMAs and every dequantised weight fragment 4.
// Activations, weight codes and the activation row sums of each K block go
// straight from memory into an LDS stage (global_load_lds, no register
// staging), one block ahead of the block being multiplied (two with three
// stages): each wavefront waits for its own loads with an explicit vmcnt, and
// one barrier per K block publishes the stage to the others and retires the
// stage the next loads overwrite.  Two 64-row workgroups with two stages each
// (70 KB of LDS apiece) beat one 128-row workgroup with three: while one
// waits at its barrier the other issues MFMAs.  The group scales
// (two bytes per channel and group) come through registers.  The row sums are
// those of the bias correction, -(128 + z) * sum_k a_k per scale group,
// written by rowsum_kernel into the workspace.
constexpr int kP2Threads = 512, kP2Rows = 128;
#ifndef P2_WM
#define P2_WM 1  // 64-row workgroups
#endif
#ifndef P2_NS
#define P2_NS 2  // two LDS stages
#endif

template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));  // expcnt, lgkmcnt: no wait
}

// out[row][g] = -(128 + z) * (sum of the bf16 values of group g of A's row);
// one wavefront per row, lane l sums 16-byte chunks l, l + 64, ...
__global__ __launch_bounds__(256) void rowsum_kernel(const uint16_t* __restrict__ A, int rows, int K, int G,
                                                     float negz, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const u32x4* src = reinterpret_cast<const u32x4*>(A + (size_t)row * K);
  const int nch = K / 8, cpg = G / 8, ng = K / G;
  for (int c0 = 0; c0 < nch; c0 += 64) {
    const int c = c0 + lane;
    float s = 0.f;
    if (c < nch) {
      const u32x4 v = src[c];
      const uint32_t w0 = v[0], w1 = v[1], w2 = v[2], w3 = v[3];
      s = add_bf16_pair(w3, add_bf16_pair(w2, add_bf16_pair(w1, add_bf16_pair(w0, s))));
    }
    for (int o = 1; o < cpg; o <<= 1) s += __shfl_xor(s, o, 64);
    if (c < nch && (lane & (cpg - 1)) == 0) out[(size_t)row * ng + c / cpg] = s * negz;
  }
}

// One LDS stage of a K block for a workgroup of 4 * WM wavefronts (64 * WM
// rows); LB: the code tiles go through LDS too.
template <int WM, bool LB>
struct __attribute__((aligned(16))) P2Stage {
  u32x4 a[4 * WM][4][64];  // activations [row tile][MFMA step][lane], 16 KB per 64 rows
  u32x4 b[LB ? 16 : 1][64];  // codes [workgroup tile][lane], 16 KB
  float r[256 * WM];       // row sums [group][row] (+ padding)
  uint32_t s[256 * WM];    // group scales, one dword (two fp16) per channel and group pair
};

// SL: the group scales of each K block travel by LDS-DMA with the block, one
// aligned dword per channel (and pair of groups), so that the loop issues
// nothing but LDS-DMA loads.  It needs an even number of groups per channel
// (K/G); otherwise every K block loads its scales into registers.

// Nested MWQ in the 64- and 128-row kernels: the rows of an expert are cut
// into 16-row chunks inside each width's sub-segment (b = 4, 3, 2 in grouped
// order), so that every MFMA row tile has one width, and a workgroup takes 4
// or 8 chunks of one expert.  All planes of a tile block are loaded once for all
// of them; each row tile multiplies the codes truncated to its width.
__device__ __forceinline__ int mwq_chunks(const int32_t* so, int e) {
  const int o0 = so[3 * e], o1 = so[3 * e + 1], o2 = so[3 * e + 2], o3 = so[3 * e + 3];
  return (o1 - o0 + 15) / 16 + (o2 - o1 + 15) / 16 + (o3 - o2 + 15) / 16;
}
// Work item y (in expert order, ceil(chunks / cpg) per expert) -> expert e and
// its chunk group g.
__device__ __forceinline__ bool find_mwq_group(const int32_t* so, int E, int y, int& e, int& g, int cpg) {
  const int lane = threadIdx.x & 63;
  int carry = 0;
  for (int s0 = 0; s0 < E; s0 += 64) {
    const int s = s0 + lane;
    const int tiles = s < E ? (mwq_chunks(so, s) + cpg - 1) / cpg : 0;
    int incl = tiles;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off, 64);
      if (lane >= off) incl += o;
    }
    const int excl = carry + incl - tiles;
    const uint64_t b = __ballot(s < E && y >= excl && y < excl + tiles);
    if (b) {
      const int src = __ffsll((unsigned long long)b) - 1;
      e = s0 + src;
      g = y - __shfl(excl, src, 64);
      return true;
    }
    carry += __shfl(incl, 63, 64);
  }
  return false;
}

// MW: 0 INT4; 1 nested MWQ, workgroups of 16-row chunks of every width of an
// expert (above); 2 nested MWQ, row tiles inside one width sub-segment (a
// segment per expert and width, like INT4's per expert): the workgroup's width
// is then known, so the K loop is compiled once per width, loads no plane
// it does not use (those lanes read past the buffer's end: no traffic) and
// decodes its codes at that width with no per-row-tile mask.
// WM: wavefront rows of the workgroup (1: 4 wavefronts on 64 rows, 2: 8 on
// 128 rows); NS: LDS stages (K blocks in flight: NS - 1).  A 64-row workgroup
// with two stages takes 70 KB of LDS, so two run on one CU and fill each
// other's barrier and load waits.  The kernels below declare their LDS stages
// (one object per stage) and run this body.
template <int EPI, int GPB, bool SL, int MW, int WM, int NS, class Stage>
__device__ __forceinline__ void qgemm_p2_body(const KArgs& p, const float* __restrict__ rowsum, int n_nblk, int n_mt,
                                              int GM, Stage& st0, Stage& st1, Stage& st2) {
  static_assert(WM == 1 || WM == 2, "64 or 128 rows per workgroup");
  static_assert(NS == 2 || NS == 3, "two or three LDS stages");
  static_assert(WM == 2 || GPB <= 2, "64-row workgroups keep one scale dword per channel");
  static_assert(MW >= 0 && MW <= 2, "INT4, nested chunks or nested per width");
  constexpr int RT = 4, UT = 4, SPG = 4 / GPB;
  constexpr int MT = 64 * WM;          // rows per workgroup
  constexpr int CPW = 4 / WM;          // code tiles loaded per wavefront
  // 64-row workgroups: each wavefront multiplies the 4 code tiles it loads, so
  // they go straight into its registers (a ring of NS blocks), not through LDS
  constexpr bool RB = WM == 1 && MW != 1;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = uniform(tid >> 6), wm = wv >> 2, wn = wv & 3;

  const int per_xcd = gridDim.x / 8;
  const int item = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  const int grp = item / (GM * n_nblk), rem = item % (GM * n_nblk);
  const int nb = rem / GM, mt = grp * GM + rem % GM;
  if (mt >= n_mt) return;
  int seg = 0, m0 = 0;
  if (MW == 1) {
    if (!find_mwq_group(p.seg_offsets, p.nseg / 3, mt, seg, m0, 4 * WM)) return;  // seg = expert, m0 = chunk group
  } else if (!find_tile(p.seg_offsets, p.nseg, mt, seg, m0, MT)) {
    return;
  }
  const Ctx c = MW == 1 ? Ctx{0, 0, uniform(seg), 4}
                        : Ctx{uniform(p.seg_offsets[seg] + m0),
                              uniform(min(MT, p.seg_offsets[seg + 1] - p.seg_offsets[seg] - m0)),
                              uniform(MW == 2 ? seg / 3 : seg), 4};
  const int tile_bits = MW == 2 ? 4 - seg % 3 : 4;  // sub-segments in grouped order: 4, 3, 2 bits
  const int KB = p.K / 128, NT = p.N / 16;

  // MW: chunk j (0 .. 4 WM - 1) of the workgroup -> first grouped row, rows (0 past the
  // expert's last chunk, whose loads then repeat the expert's first row), width
  int o[4] = {0, 0, 0, 0}, nc[3] = {0, 0, 0};
  if (MW == 1) {
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = uniform(p.seg_offsets[3 * c.e + q]);
#pragma unroll
    for (int q = 0; q < 3; ++q) nc[q] = (o[q + 1] - o[q] + 15) / 16;
  }
  auto chunk = [&](int j, int& start, int& rows, int& bits) {
    int ci = 4 * WM * m0 + j;
    start = o[0];
    rows = 0;
    bits = 2;
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      if (rows == 0 && ci >= 0 && ci < nc[q]) {
        start = o[q] + 16 * ci;
        rows = min(16, o[q + 1] - start);
        bits = 4 - q;
      }
      ci -= nc[q];
    }
  };
  // grouped row -> source row of A
  auto a_row = [&](int gi) -> size_t { return p.gather ? (size_t)(p.gather[gi] / p.k) : (size_t)gi; };
  // MW: source row of row r (0 .. MT - 1) of the workgroup tile
  auto mw_src_row = [&](int r) -> size_t {
    int st, rw, bt;
    chunk(r >> 4, st, rw, bt);
    return a_row(st + min(r & 15, max(rw, 1) - 1));
  };

  // workgroup tile j = 4 * (consumer wavefront wn) + u; SwiGLU: u = 0, 1 gate, 2, 3 up
  auto wg_tile = [&](int j, bool& valid) -> int {
    const int w4 = j >> 2, u = j & 3;
    int t;
    if (EPI == 1) {
      const int hch = nb * 128 + 32 * w4 + 16 * (u & 1);
      t = (u < 2 ? 0 : NT / 2) + hch / 16;
      valid = hch < p.N / 2;
    } else {
      t = nb * 16 + j;
      valid = t < NT;
    }
    return valid ? t : 0;  // invalid tiles load tile 0 and are never stored
  };

  // loads issued by this wavefront: activation row tile wv (4 steps), workgroup
  // tiles CPW wv .. CPW wv + CPW - 1, row-sum entries 64wv .. 64wv + 63.  Buffer
  // loads: the per-lane offset stays fixed and each K block only moves the
  // scalar offset.
  const rsrc_t ar = make_rsrc(p.A, p.A_bytes);
  const uint32_t a_off = (uint32_t)((MW == 1 ? mw_src_row(16 * wv + (lane & 15)) : src_row(p, c, 16 * wv + (lane & 15))) *
                                         (size_t)p.K * 2 + 16 * (lane >> 4));
  rsrc_t br[4];  // CPW used
#pragma unroll
  for (int q = 0; q < CPW; ++q) {
    bool v;
    const int t = wg_tile(CPW * wv + q, v);
    br[q] = make_rsrc(p.codes + ((size_t)c.e * NT + t) * (size_t)KB * 1024, KB * 1024);
  }
  // MW: the four dword loads j = 0..3 of a code tile build, in LDS, lane L's
  // 16-byte record (q2 dwords 2L and 2L + 1, d3 dword L, d4 dword L) for
  // L = 16 j .. 16 j + 15: load lane m writes dword m % 4 of record 16 j + m / 4
  // (MW 2: the lanes of a plane the tile's width does not use read past the end)
  uint32_t bo[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int L = 16 * j + (lane >> 2), w = lane & 3;
    const bool unused = (w == 2 && tile_bits < 3) || (w == 3 && tile_bits < 4);
    bo[j] = unused ? 0x80000000u : (uint32_t)(w < 2 ? 8 * L + 4 * w : 512 + 256 * (w - 2) + 4 * L);
  }
  const int ng = KB * GPB;
  const int en = 64 * wv + lane;
  const bool ren = en < MT * GPB;
  const rsrc_t rr = make_rsrc(rowsum, (p.A_bytes / (2u * p.K)) * ng * 4);
  const uint32_t r_off =
      (uint32_t)(((MW == 1 ? mw_src_row(ren ? (en % MT) : 0) : src_row(p, c, ren ? (en % MT) : 0)) * (size_t)ng +
                  (ren ? (en / MT) : 0)) * 4);
  // MW: this wavefront's row tiles (chunks 4wm + rt): codes truncated to their width
  uint32_t mrt[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    int st, rw, bt;
    chunk(4 * wm + rt, st, rw, bt);
    mrt[rt] = MW == 1 ? uniform(bt == 4 ? 0xFFFFFFFFu : bt == 3 ? 0xFFFEFFFEu : 0xFFFCFFFCu) : 0xFFFFFFFFu;
  }

  // scale entries: dword 64wv + lane of the stage holds, for GPB <= 2,
  // channel (j, c) = (entry / 16, entry % 16) (with 8 wavefronts, entries 256..
  // are padding, they reload entry 0), for GPB = 4 the group pair entry % 2 of
  // channel entry / 2
  const rsrc_t scr = make_rsrc(p.scales, (uint32_t)((size_t)(p.nseg / p.S) * p.N * ng * 2));
  uint32_t s_off;
  {
    const int se = 64 * wv + lane;
    const int ch = GPB == 4 ? se >> 1 : (se < 256 ? se : 0);
    bool v;
    const int t = wg_tile(ch >> 4, v);
    s_off = (uint32_t)((((size_t)c.e * p.N + t * 16 + (ch & 15)) * ng + (GPB == 4 ? 2 * (se & 1) : 0)) * 2);
  }

  // this wavefront's own tiles (consumer side): scales and stores
  int ct[UT];
  bool cval[UT];
#pragma unroll
  for (int u = 0; u < UT; ++u) ct[u] = wg_tile(4 * wn + u, cval[u]);
  rsrc_t sr[UT];
#pragma unroll
  for (int u = 0; u < UT; ++u) sr[u] = make_rsrc(p.scales + ((size_t)c.e * NT + ct[u]) * 16 * (size_t)ng, 16 * ng * 2);
  const uint32_t soff = (uint32_t)((lane & 15) * ng * 2);

  f32x4 acc[RT][UT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int u = 0; u < UT; ++u) acc[rt][u] = f32x4{};
  uint32_t rsc[NS][UT][GPB];  // one register per scale: packing two would wait for both loads

#define P2_ISSUE(S, ST, KBI) \
  _Pragma("unroll") for (int q_ = 0; q_ < 6 + NB; ++q_) P2_PART(S, ST, KBI, q_)
// Part Q (0 .. 5 + NB) of the loads of block KBI into stage ST: activations
// step 0..3, the CPW code tiles (MW 1: four parts each; RB: into the register
// ring slot S, nested planes one part per plane the width uses), row sums,
// scales; with register scales (!SL) the last part loads them into slot S.
// Offsets go in the scalar operand: the immediate one would move the LDS
// address too.
#define P2_PART(S, ST, KBI, Q)                                                                         \
  {                                                                                                    \
    const int kbi = (KBI);                                                                             \
    if ((Q) < 4)                                                                                       \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, &ST.a[wv][(Q) & 3][0], 16, a_off, kbi * 256 + 64 * ((Q) & 3), 0, 0); \
    else if ((Q) < 4 + NB) {                                                                           \
      if constexpr (RB && MW == 2) {                                                                   \
        const int pt = ((Q) - 4) / NPT, pl = ((Q) - 4) % NPT;                                          \
        if (pl == 0) {                                                                                 \
          const u32x2 q2v = buf_x2(br[pt], 8 * lane, kbi * 1024);                                      \
          rcb[S][pt][0] = q2v[0];                                                                      \
          rcb[S][pt][1] = q2v[1];                                                                      \
        } else {                                                                                       \
          rcb[S][pt][1 + pl] = buf_x1(br[pt], 256 + 256 * pl + 4 * lane, kbi * 1024);                  \
        }                                                                                              \
      } else if constexpr (RB)                                                                         \
        rcb[S][(Q) - 4] = buf_x4(br[(Q) - 4], 16 * lane, kbi * 1024);                                  \
      else if (MW)                                                                                     \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(br[((Q) - 4) >> 2], &ST.b[CPW * wv + (((Q) - 4) >> 2)][16 * (((Q) - 4) & 3)], \
                                                 4, bo[((Q) - 4) & 3], kbi * 1024, 0, 0);              \
      else                                                                                             \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(br[(Q) - 4], &ST.b[CPW * wv + (Q) - 4][0], 16, 16 * lane, \
                                                 kbi * 1024, 0, 0);                                    \
    } else if ((Q) == 4 + NB)                                                                          \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, &ST.r[64 * wv], 4, r_off, kbi * GPB * 4, 0, 0);     \
    else if (SL)                                                                                       \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(scr, &ST.s[64 * wv], 4, s_off,                          \
                                               GPB == 1 ? 4 * (kbi >> 1) : 4 * kbi * (GPB / 2), 0, 0); \
    else                                                                                               \
      _Pragma("unroll") for (int u = 0; u < UT; ++u) _Pragma("unroll") for (int g = 0; g < GPB; ++g)   \
          rsc[S][u][g] = buf_u16(sr[u], soff, (kbi * GPB + g) * 2);                                    \
  }
// With one scale group per K block the load instructions of block i + 2
// are spread over the four MFMA steps of block i (a burst of them right after
// the barrier kept every wavefront waiting at issue); with more groups they
// are issued together before the block (spreading them costs registers).
// Per scale group: the correction (row sums) is the C input of the first
// MFMA of each chain; the activation fragments of the next MFMA step are read
// from LDS while the current step's MFMAs run.
#define P2_COMPUTE(S, ST, KBI, DO_ISSUE, IS_, IS, IKB)                                                     \
  {                                                                                                        \
    _Pragma("unroll") for (int g = 0; g < GPB; ++g) {                                                      \
      f32x4 rv[RT];                                                                                        \
      _Pragma("unroll") for (int rt = 0; rt < RT; ++rt)                                                    \
          rv[rt] = *reinterpret_cast<const f32x4*>(&ST.r[g * MT + 64 * wm + 16 * rt + 4 * (lane >> 4)]); \
      u32x4 av[2][RT];                                                                                     \
      _Pragma("unroll") for (int rt = 0; rt < RT; ++rt) av[0][rt] = ST.a[4 * wm + rt][g * SPG][lane];      \
      f32x4 tmp[RT][UT];                                                                                   \
      _Pragma("unroll") for (int tt = 0; tt < SPG; ++tt) {                                                 \
        const int t = g * SPG + tt;                                                                        \
        if (tt + 1 < SPG) {                                                                                \
          _Pragma("unroll") for (int rt = 0; rt < RT; ++rt) av[(tt + 1) & 1][rt] = ST.a[4 * wm + rt][t + 1][lane]; \
          __builtin_amdgcn_sched_barrier(0); /* keep these reads ahead of this step's MFMAs */              \
        }                                                                                                  \
        if (DO_ISSUE) {                                                                                    \
          _Pragma("unroll") for (int qp = 0; qp < PPS; ++qp)                                               \
              if (PPS * t + qp < 6 + NB) P2_PART(IS_, IS, IKB, PPS * t + qp)                               \
          __builtin_amdgcn_sched_barrier(0); /* spread the loads over the block's MFMA steps */            \
        }                                                                                                  \
        u32x4 bv[UT];                                                                                      \
        _Pragma("unroll") for (int u = 0; u < UT; ++u)                                                     \
            bv[u] = MW ? deq_mwq_bits(u32x2{cb[u][0], cb[u][1]}, cb[u][2], cb[u][3], t, BW)                \
                       : __builtin_bit_cast(u32x4, deq_u4(cb[u], t));                                      \
        _Pragma("unroll") for (int rt = 0; rt < RT; ++rt) {                                                \
          const bf16x8 a = as_bf16x8(av[tt & 1][rt]);                                                      \
          _Pragma("unroll") for (int u = 0; u < UT; ++u)                                                   \
              tmp[rt][u] = mfma16(a, as_bf16x8(MW == 1 ? and4(bv[u], mrt[rt]) : bv[u]), tt == 0 ? rv[rt] : tmp[rt][u]); \
        }                                                                                                  \
      }                                                                                                    \
      _Pragma("unroll") for (int u = 0; u < UT; ++u) {                                                     \
        const float sv = f16_to_f32(SL ? sc16[u][g] : (uint16_t)rsc[S][u][g]);                             \
        _Pragma("unroll") for (int rt = 0; rt < RT; ++rt)                                                  \
            _Pragma("unroll") for (int r = 0; r < 4; ++r) acc[rt][u][r] = __builtin_fmaf(sv, tmp[rt][u][r], acc[rt][u][r]); \
      }                                                                                                    \
    }                                                                                                      \
  }
  // Block i sits in stage i % 3.  Before block i this wavefront waits for its
  // own loads of block i, and the barrier makes every wavefront's loads
  // visible and retires stage (i - 1) % 3, into which block i + 2 is then
  // issued.  Each step reads its codes before issuing: at the loop header the
  // compiler loses track of which stage the loads in flight write and waits
  // for all of them before the first LDS read, which is then only block i + 1.
#define P2_READY(I)                  \
  {                                  \
    __builtin_amdgcn_sched_barrier(0); \
    if ((I) + 1 < KB) vm_wait<VW>(); \
    else vm_wait<0>();               \
    __builtin_amdgcn_s_barrier();    \
  }
#define P2_READY_U                     \
  {                                    \
    __builtin_amdgcn_sched_barrier(0); \
    vm_wait<VW>();                     \
    __builtin_amdgcn_s_barrier();      \
  }
#define P2_STEP_U(J, CS, IS, I)                                                     \
  {                                                                                 \
    u32x4 cb[UT];                                                                   \
    _Pragma("unroll") for (int u = 0; u < UT; ++u) cb[u] = RB ? rcb[J][u] : CS.b[RB ? 0 : 4 * wn + u][lane]; \
    uint16_t sc16[UT][GPB];                                                         \
    if (SL)                                                                         \
      _Pragma("unroll") for (int u = 0; u < UT; ++u) _Pragma("unroll") for (int g = 0; g < GPB; ++g) { \
        const int chn = (4 * wn + u) * 16 + (lane & 15);                            \
        const uint32_t d = CS.s[GPB == 4 ? 2 * chn + (g >> 1) : chn];              \
        const int half = GPB == 1 ? ((I) & 1) : (g & 1);                            \
        sc16[u][g] = (uint16_t)(d >> (16 * half));                                   \
      }                                                                             \
    if (GPB != 1) P2_ISSUE(((J) + NS - 1) % NS, IS, (I) + NS - 1);                  \
    P2_COMPUTE(J, CS, I, GPB == 1, ((J) + NS - 1) % NS, IS, (I) + NS - 1);          \
  }
#define P2_STEP(J, CS, IS, I)                                                       \
  {                                                                                 \
    u32x4 cb[UT];                                                                   \
    _Pragma("unroll") for (int u = 0; u < UT; ++u) cb[u] = RB ? rcb[J][u] : CS.b[RB ? 0 : 4 * wn + u][lane]; \
    uint16_t sc16[UT][GPB];                                                         \
    if (SL)                                                                         \
      _Pragma("unroll") for (int u = 0; u < UT; ++u) _Pragma("unroll") for (int g = 0; g < GPB; ++g) { \
        const int chn = (4 * wn + u) * 16 + (lane & 15);                            \
        const uint32_t d = CS.s[GPB == 4 ? 2 * chn + (g >> 1) : chn];              \
        const int half = GPB == 1 ? ((I) & 1) : (g & 1);                            \
        sc16[u][g] = (uint16_t)(d >> (16 * half));                                   \
      }                                                                             \
    if (GPB != 1 && (I) + NS - 1 < KB) P2_ISSUE(((J) + NS - 1) % NS, IS, (I) + NS - 1); \
    P2_COMPUTE(J, CS, I, GPB == 1 && (I) + NS - 1 < KB, ((J) + NS - 1) % NS, IS, (I) + NS - 1); \
  }

  // The K loop, once per code width known at compile time (BW: 4 unless MW 2).
  auto k_loop = [&](auto bw_tag) {
  constexpr int BW = decltype(bw_tag)::value;
  constexpr int NPT = MW == 2 ? 1 + (BW >= 3) + (BW == 4) : 1;  // RB, nested: plane loads per code tile
  // vector-memory instructions per K block and wavefront for the code tiles
  // (through LDS, MW: four dword loads per code tile)
  constexpr int NB = RB ? CPW * NPT : MW ? 4 * CPW : CPW;
  constexpr int V = SL ? 6 + NB : 5 + NB + UT * GPB;
  constexpr int VW = NS == 3 ? V : 0;  // loads that may stay in flight before a block is read
  constexpr int PPS = (6 + NB + 3) / 4;  // load parts issued per MFMA step (one scale group per block)
  u32x4 rcb[NS][UT];  // RB: code tiles of the blocks in flight
  P2_ISSUE(0, st0, 0);
  if (NS == 3 && 1 < KB) P2_ISSUE(1, st1, 1);
  P2_READY(0)
  // Steady state: NS blocks per iteration with no branch inside (every load
  // it issues is in range): the compiler then keeps track of which stage each
  // load in flight writes and waits only for the stage read next (a merge of
  // control-flow paths, or more load instructions per loop body, makes it
  // wait for every load in flight); then the tail.
  int kb0 = 0;
  if constexpr (NS == 3) {
    for (; kb0 + 5 <= KB; kb0 += 3) {
      P2_STEP_U(0, st0, st2, kb0)
      P2_READY_U
      P2_STEP_U(1, st1, st0, kb0 + 1)
      P2_READY_U
      P2_STEP_U(2, st2, st1, kb0 + 2)
      P2_READY_U
    }
    for (; kb0 < KB; kb0 += 3) {
      P2_STEP(0, st0, st2, kb0)
      if (kb0 + 1 < KB) {
        P2_READY(kb0 + 1)
        P2_STEP(1, st1, st0, kb0 + 1)
      }
      if (kb0 + 2 < KB) {
        P2_READY(kb0 + 2)
        P2_STEP(2, st2, st1, kb0 + 2)
      }
      if (kb0 + 3 < KB) P2_READY(kb0 + 3)
    }
  } else {
    for (; kb0 + 3 <= KB; kb0 += 2) {
      P2_STEP_U(0, st0, st1, kb0)
      P2_READY_U
      P2_STEP_U(1, st1, st0, kb0 + 1)
      P2_READY_U
    }
    for (; kb0 < KB; kb0 += 2) {
      P2_STEP(0, st0, st1, kb0)
      if (kb0 + 1 < KB) {
        P2_READY(kb0 + 1)
        P2_STEP(1, st1, st0, kb0 + 1)
      }
      if (kb0 + 2 < KB) P2_READY(kb0 + 2)
    }
  }
  };
  if constexpr (MW == 2) {
    if (tile_bits == 2) k_loop(std::integral_constant<int, 2>{});
    else if (tile_bits == 3) k_loop(std::integral_constant<int, 3>{});
    else k_loop(std::integral_constant<int, 4>{});
  } else {
    k_loop(std::integral_constant<int, 4>{});
  }
#undef P2_STEP_U
#undef P2_READY_U
#undef P2_STEP
#undef P2_READY
#undef P2_COMPUTE
#undef P2_ISSUE
#undef P2_PART

  const int col = lane & 15;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    // grouped rows of row tile rt: row0 + 16 rt + .. (a 16-row chunk for MW)
    int row0 = c.row0 + 64 * wm + 16 * rt, rows = c.rows - 64 * wm - 16 * rt;
    if (MW == 1) {
      int bt;
      chunk(4 * wm + rt, row0, rows, bt);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 4 * (lane >> 4) + r;
      if (row >= rows) continue;
      if (EPI == 1) {
        uint16_t* orow = static_cast<uint16_t*>(p.out) + (size_t)(row0 + row) * p.n_out;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          if (!cval[h]) continue;
          const float g = acc[rt][h][r], up = acc[rt][h + 2][r];
          orow[nb * 128 + 32 * wn + 16 * h + col] = f32_to_bf16(g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * up);
        }
      } else {
#pragma unroll
        for (int u = 0; u < UT; ++u) {
          if (!cval[u]) continue;
          const size_t oi = (size_t)(row0 + row) * p.n_out + ct[u] * 16 + col;
          store_plain<EPI>(p.out, oi, acc[rt][u][r]);
        }
      }
    }
  }
}

// ------------------------------------------------- delta with base, LDS-DMA
// y = x W_base^T + x D_e^T for many rows per expert (ME-Switch delta layer).
// One workgroup of 8 wavefronts per (128-row tile, 128-channel block);
// wavefront (wm, wn) owns 64 rows x 2 channel tiles, and each activation
// fragment read from LDS feeds 4 MFMAs: the bf16 base product and the 2-bit
// delta product of both tiles.  The K loop runs over half K blocks (64
// channels): four LDS stages of 34 KB each hold a half block's 128 activation
// rows, the bf16 base fragments and the 2-bit codes of the 8 tiles, loaded by
// LDS-DMA three half blocks ahead (two full-block stages, one block ahead,
// left the wavefronts waiting on memory about half the time).  The delta has one step
// per output channel, so its chain runs over all of K: it starts from the
// row's -(128 + z) * sum_k a_k (one row sum over all of K, from
// rowsum_full_kernel) and the step multiplies once at the end.  The salient
// channels are one more exact bf16 K chunk: their activation values are
// gathered into LDS after the loop.
__global__ __launch_bounds__(256) void rowsum_full_kernel(const uint16_t* __restrict__ A, int rows, int K, float negz,
                                                          float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const u32x4* src = reinterpret_cast<const u32x4*>(A + (size_t)row * K);
  float s = 0.f;
  for (int c = lane; c < K / 8; c += 64) {
    const u32x4 v = src[c];
    const uint32_t w0 = v[0], w1 = v[1], w2 = v[2], w3 = v[3];
    s = add_bf16_pair(w3, add_bf16_pair(w2, add_bf16_pair(w1, add_bf16_pair(w0, s))));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
  if (lane == 0) out[row] = s * negz;
}

struct __attribute__((aligned(16))) P2DStage {
  u32x4 a[8][2][64];  // activations of half a K block [row tile][MFMA step][lane], 16 KB
  u32x4 b[8][2][64];  // base [tile][MFMA step][lane], 16 KB
  uint32_t d[8][64];  // 2-bit codes [tile][lane] (one dword: two MFMA steps), 2 KB
};

template <int EPI>
__global__ __launch_bounds__(kP2Threads) void qgemm_p2d_kernel(KArgs p, const float* __restrict__ rowsum, int n_nblk,
                                                               int n_mt, int GM) {
  constexpr int RT = 4, UT = 2, V = 5;  // V: vector-memory instructions per half K block and wavefront
  __shared__ P2DStage st0, st1, st2, st3;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = uniform(tid >> 6), wm = wv >> 2, wn = wv & 3;

  const int per_xcd = gridDim.x / 8;
  const int item = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  const int grp = item / (GM * n_nblk), rem = item % (GM * n_nblk);
  const int nb = rem / GM, mt = grp * GM + rem % GM;
  if (mt >= n_mt) return;
  int seg, m0;
  if (!find_tile(p.seg_offsets, p.nseg, mt, seg, m0, kP2Rows)) return;
  const Ctx c{uniform(p.seg_offsets[seg] + m0), uniform(min(kP2Rows, p.seg_offsets[seg + 1] - p.seg_offsets[seg] - m0)),
              uniform(seg), 2};
  const int KB = p.K / 128, NT = p.N / 16;
  auto tile_of = [&](int j, bool& valid) -> int {  // workgroup tile j = 2 * wn + u
    const int t = nb * 8 + j;
    valid = t < NT;
    return valid ? t : 0;
  };

  // loads issued by this wavefront: activation row tile wv, base and codes of workgroup tile wv
  const rsrc_t ar = make_rsrc(p.A, p.A_bytes);
  const uint32_t a_off = (uint32_t)(src_row(p, c, 16 * wv + (lane & 15)) * (size_t)p.K * 2 + 16 * (lane >> 4));
  bool tv;
  const int tw = tile_of(wv, tv);
  const rsrc_t bsr = make_rsrc(p.base + (size_t)tw * KB * 2048, KB * 4096);
  const rsrc_t csr = make_rsrc(p.codes + ((size_t)c.e * NT + tw) * KB * 512, KB * 512);

  // consumer side: this wavefront's tiles, steps, row sums
  int ct[UT];
  bool cval[UT];
  float step[UT];
#pragma unroll
  for (int u = 0; u < UT; ++u) {
    ct[u] = tile_of(2 * wn + u, cval[u]);
    step[u] = f16_to_f32(p.scales[(size_t)c.e * p.N + ct[u] * 16 + (lane & 15)]);
  }
  // the row sums of this lane's 16 accumulator rows: all source rows first, then all sums
  // (one branch for the whole batch: a branch per lookup serialises the loads)
  size_t srow[RT][4];
  if (p.gather) {
    int g[RT][4];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) g[rt][r] = p.gather[c.row0 + min(64 * wm + 16 * rt + 4 * (lane >> 4) + r, c.rows - 1)];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) srow[rt][r] = (size_t)(g[rt][r] / p.k);
  } else {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) srow[rt][r] = (size_t)(c.row0 + min(64 * wm + 16 * rt + 4 * (lane >> 4) + r, c.rows - 1));
  }
  f32x4 accb[RT][UT], accd[RT][UT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    f32x4 rv;
#pragma unroll
    for (int r = 0; r < 4; ++r) rv[r] = rowsum[srow[rt][r]];
#pragma unroll
    for (int u = 0; u < UT; ++u) {
      accb[rt][u] = f32x4{};
      accd[rt][u] = rv;
    }
  }

// half block J: K block J / 2, MFMA steps 2 (J % 2) and 2 (J % 2) + 1
#define PD_ISSUE(ST, J)                                                                                    \
  {                                                                                                        \
    const int kbi = (J) >> 1, hh = (J) & 1;                                                                \
    _Pragma("unroll") for (int q = 0; q < 2; ++q)                                                          \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, &ST.a[wv][q][0], 16, a_off, kbi * 256 + 64 * (2 * hh + q), 0, 0); \
    _Pragma("unroll") for (int q = 0; q < 2; ++q)                                                          \
        __builtin_amdgcn_raw_ptr_buffer_load_lds(bsr, &ST.b[wv][q][0], 16, 16 * lane, kbi * 4096 + 1024 * (2 * hh + q), 0, 0); \
    __builtin_amdgcn_raw_ptr_buffer_load_lds(csr, &ST.d[wv][0], 4, 8 * lane, kbi * 512 + 4 * hh, 0, 0);     \
  }
#define PD_COMPUTE(ST, J)                                                                                  \
  {                                                                                                        \
    u32x2 cd[UT];                                                                                          \
    _Pragma("unroll") for (int u = 0; u < UT; ++u) { const uint32_t w_ = ST.d[2 * wn + u][lane]; cd[u] = u32x2{w_, w_}; } \
    _Pragma("unroll") for (int tt = 0; tt < 2; ++tt) {                                                     \
      const int t = 2 * ((J) & 1) + tt;                                                                    \
      bf16x8 bb[UT], bd[UT];                                                                               \
      _Pragma("unroll") for (int u = 0; u < UT; ++u) {                                                     \
        bb[u] = as_bf16x8(ST.b[2 * wn + u][tt][lane]);                                                     \
        bd[u] = deq_u2(cd[u], t);                                                                          \
      }                                                                                                    \
      _Pragma("unroll") for (int rt = 0; rt < RT; ++rt) {                                                  \
        const bf16x8 av = as_bf16x8(ST.a[4 * wm + rt][tt][lane]);                                          \
        _Pragma("unroll") for (int u = 0; u < UT; ++u) {                                                   \
          accb[rt][u] = mfma16(av, bb[u], accb[rt][u]);                                                    \
          accd[rt][u] = mfma16(av, bd[u], accd[rt][u]);                                                    \
        }                                                                                                  \
      }                                                                                                    \
    }                                                                                                      \
  }
  // block i in stage i % 2: wait for this wavefront's loads of block i, the
  // barrier publishes them and retires the other stage, then block i + 1 is
  // issued into it and block i multiplied; the steady state has no branch
  // half block j in stage j % 4, three in flight: before j, wait for this
  // wavefront's loads of j (those of j + 1 and j + 2 may stay in flight); the
  // barrier publishes them and retires stage (j - 1) % 4, into which j + 3 goes
#define PD_STEP_U(CS, IS, J)            \
  {                                     \
    __builtin_amdgcn_sched_barrier(0);  \
    vm_wait<2 * V>();                   \
    __builtin_amdgcn_s_barrier();       \
    PD_ISSUE(IS, (J) + 3);              \
    PD_COMPUTE(CS, J);                  \
  }
#define PD_STEP(CS, IS, J)                                   \
  if ((J) < NH) {                                            \
    __builtin_amdgcn_sched_barrier(0);                       \
    if ((J) + 2 < NH) vm_wait<2 * V>();                      \
    else if ((J) + 1 < NH) vm_wait<V>();                     \
    else vm_wait<0>();                                       \
    __builtin_amdgcn_s_barrier();                            \
    if ((J) + 3 < NH) PD_ISSUE(IS, (J) + 3);                 \
    PD_COMPUTE(CS, J);                                       \
  }
  const int NH = 2 * KB;  // half blocks
  PD_ISSUE(st0, 0);
  PD_ISSUE(st1, 1);
  // unconditional, so the loop's wait counts hold from its first step; with one K
  // block this half block lies past the end: the buffer resources bound its loads
  // and no step reads that stage
  PD_ISSUE(st2, 2);
  int j0 = 0;
  for (; j0 + 7 <= NH; j0 += 4) {
    PD_STEP_U(st0, st3, j0)
    PD_STEP_U(st1, st0, j0 + 1)
    PD_STEP_U(st2, st1, j0 + 2)
    PD_STEP_U(st3, st2, j0 + 3)
  }
  for (; j0 < NH; j0 += 4) {
    PD_STEP(st0, st3, j0)
    PD_STEP(st1, st0, j0 + 1)
    PD_STEP(st2, st1, j0 + 2)
    PD_STEP(st3, st2, j0 + 3)
  }
#undef PD_STEP
#undef PD_STEP_U
#undef PD_COMPUTE
#undef PD_ISSUE

  // salient input channels: gather their activation values into stage 0 in
  // the MFMA operand layout (2 steps of 32 slots), then one more bf16 K chunk
  const int nsteps = (p.n_sal + 31) / 32;
  if (nsteps > 0) {
    __syncthreads();  // every wavefront is done with stage 0
    for (int slot = tid; slot < 8 * 2 * 64; slot += kP2Threads) {
      const int rt8 = slot >> 7, sstep = (slot >> 6) & 1, l = slot & 63;
      const uint16_t* Arow = p.A + src_row(p, c, 16 * rt8 + (l & 15)) * (size_t)p.K;
      u32x4 v;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        uint32_t w = 0;
#pragma unroll
        for (int e2 = 0; e2 < 2; ++e2) {
          const int j = 32 * sstep + 8 * (l >> 4) + 2 * h + e2;
          const int idx = j < p.n_sal ? min(max(p.sal_idx[(size_t)c.e * p.n_sal + j], 0), p.K - 1) : -1;
          w |= (uint32_t)(idx >= 0 ? Arow[idx] : 0) << (16 * e2);
        }
        v[h] = w;
      }
      st0.a[rt8][sstep][l] = v;
    }
    __syncthreads();
    for (int ss = 0; ss < nsteps; ++ss) {
      u32x4 sv[UT];
#pragma unroll
      for (int u = 0; u < UT; ++u)
        sv[u] = *reinterpret_cast<const u32x4*>(p.sal_val + (((size_t)c.e * NT + ct[u]) * nsteps + ss) * 512 + 8 * lane);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const bf16x8 av = as_bf16x8(st0.a[4 * wm + rt][ss][lane]);
#pragma unroll
        for (int u = 0; u < UT; ++u) accb[rt][u] = mfma16(av, as_bf16x8(sv[u]), accb[rt][u]);
      }
    }
  }

  const int col = lane & 15;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 64 * wm + 16 * rt + 4 * (lane >> 4) + r;
      if (row >= c.rows) continue;
#pragma unroll
      for (int u = 0; u < UT; ++u) {
        if (!cval[u]) continue;
        const float y = __builtin_fmaf(step[u], accd[rt][u][r], accb[rt][u][r]);
        const size_t o = (size_t)(c.row0 + row) * p.n_out + ct[u] * 16 + col;
        store_plain<EPI>(p.out, o, y);
      }
    }
  }
}

// out[row] = sum over ks = 0..n_ks-1 of part[ks][row], in that order, for the
// rows the segments hold, [seg_offsets[0], seg_offsets[nseg]) (a caller may
// pass a slice of a longer offset table whose first entry is not zero); fp32,
// bf16 or fp16 out.  One thread per 4 outputs; the grid covers M_total rows.
template <int EPI>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part, int n_ks, int M_total,
                                                            int N, const int32_t* __restrict__ seg_offsets, int nseg,
                                                            void* __restrict__ out) {
  const size_t first = (size_t)seg_offsets[0] * N / 4, last = (size_t)seg_offsets[nseg] * N / 4;
  const size_t i4 = first + (size_t)blockIdx.x * 256 + threadIdx.x;  // N % 32 == 0: rows hold whole vectors
  if (i4 >= last) return;
  const size_t plane = (size_t)M_total * N;
  f32x4 v = reinterpret_cast<const f32x4*>(part)[i4];
  for (int ks = 1; ks < n_ks; ++ks) v += reinterpret_cast<const f32x4*>(part + ks * plane)[i4];
  if (EPI == 2) {
    reinterpret_cast<f32x4*>(out)[i4] = v;
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) store_plain<EPI>(out, i4 * 4 + q, v[q]);
  }
}

template <int FMT, int EPI>
void launch_d_one(const KArgs& ka, int n_cg, int n_rt, int n_ks, int kb_per, const TabOf<FMT>& targ, hipStream_t s) {
  const int items = n_cg * n_ks * n_rt;
  const dim3 grid((unsigned)(((items + 7) / 8) * 8));  // multiple of 8: one equal share per XCD
  switch (ka.G) {
    case 128:
      hipLaunchKernelGGL((qgemm_d_kernel<FMT, EPI, 1>), grid, dim3(kThreads), 0, s, ka, n_cg, n_rt, n_ks, kb_per,
                         targ);
      break;
    case 64:
      hipLaunchKernelGGL((qgemm_d_kernel<FMT, EPI, 2>), grid, dim3(kThreads), 0, s, ka, n_cg, n_rt, n_ks, kb_per,
                         targ);
      break;
    default:
      hipLaunchKernelGGL((qgemm_d_kernel<FMT, EPI, 4>), grid, dim3(kThreads), 0, s, ka, n_cg, n_rt, n_ks, kb_per,
                         targ);
      break;
  }
}

// FMT 5 (a width per expert): one launch for the experts of 2, 3 and 4 bits
// and one for those of 8 bits, each only if there are such experts.
template <int FMT, int EPI>
void launch_d(const KArgs& ka, int n_cg, int n_rt, const XTab& tab, hipStream_t s) {
  const int KBt = ka.K / 128;
  const int n_ks = (EPI == 1 || !ka.part) ? 1 : decode_splits(n_cg * n_rt, ka.K);
  const int kb_per = (KBt + n_ks - 1) / n_ks;
  if constexpr (FMT == 5) {
    bool narrow = false, wide = false;
    for (int e = 0; e < ka.nseg; ++e) (tab.bits[e] == 8 ? wide : narrow) = true;
    if (narrow) launch_d_one<5, EPI>(ka, n_cg, n_rt, n_ks, kb_per, tab, s);
    if (wide) launch_d_one<6, EPI>(ka, n_cg, n_rt, n_ks, kb_per, tab, s);
  } else {
    launch_d_one<FMT, EPI>(ka, n_cg, n_rt, n_ks, kb_per, NoTab{}, s);
  }
  if (n_ks > 1) {
    const size_t n4 = (size_t)ka.M_total * ka.N / 4;
    hipLaunchKernelGGL((splitk_reduce_kernel<EPI>), dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, ka.part,
                       n_ks, ka.M_total, ka.N, ka.seg_offsets, ka.nseg, ka.out);
  }
}

// Row tiles per ordering group: all of them (channel-block major) when the
// weights are the larger operand, else as many as hold about `a_target` bytes
// of activation rows (2 MB for the 64-row kernel, 4 MB for the 128-row one).
int group_rows(const KArgs& ka, int M_total, int n_mt, int MT, int fmt, size_t a_target = 2u << 20) {
  const double a_bytes = (double)M_total * ka.K * 2.0;
  const double w_bytes = (double)(ka.nseg / ka.S) * ka.N * ka.K * (fmt == 1 ? 0.5 : 0.25);
  if (a_bytes < w_bytes) return n_mt;
  const int gm = (int)(a_target / ((size_t)MT * ka.K * 2));
  return gm < 1 ? 1 : (gm > n_mt ? n_mt : gm);
}

template <int FMT, int EPI, int WR, int WC>
void launch_p(const KArgs& ka, int M_total, hipStream_t s) {
  const int n_nblk = EPI == 1 ? (ka.N / 2 + 16 * WC - 1) / (16 * WC) : (ka.N + 32 * WC - 1) / (32 * WC);
  const int n_mt = (M_total + 64 * WR - 1) / (64 * WR) + ka.nseg;
  const int GM = group_rows(ka, M_total, n_mt, 64 * WR, FMT);
  const int items = n_nblk * ((n_mt + GM - 1) / GM) * GM;  // whole groups
  const dim3 grid((unsigned)(((items + 7) / 8) * 8));        // multiple of 8: one equal share per XCD
  const dim3 block(64 * WR * WC);
  switch (ka.G) {
    case 128: hipLaunchKernelGGL((qgemm_p_kernel<FMT, EPI, 1, WR, WC>), grid, block, 0, s, ka, n_nblk, n_mt, GM); break;
    case 64: hipLaunchKernelGGL((qgemm_p_kernel<FMT, EPI, 2, WR, WC>), grid, block, 0, s, ka, n_nblk, n_mt, GM); break;
    default: hipLaunchKernelGGL((qgemm_p_kernel<FMT, EPI, 4, WR, WC>), grid, block, 0, s, ka, n_nblk, n_mt, GM); break;
  }
}

// One LDS object per stage: the compiler tracks outstanding LDS-DMA writes per
// LDS object, and only a few objects at a time.
template <int EPI, int GPB, bool SL, int MW, int NS>
__global__ __launch_bounds__(512, 1) void qgemm_p2_kernel(KArgs p, const float* __restrict__ rowsum, int n_nblk,
                                                          int n_mt, int GM) {
  __shared__ P2Stage<2, true> st0, st1, st2;
  qgemm_p2_body<EPI, GPB, SL, MW, 2, NS>(p, rowsum, n_nblk, n_mt, GM, st0, st1, st2);
}
template <int EPI, int GPB, bool SL, int MW, int NS>
__global__ __launch_bounds__(256, 2) void qgemm_p2h_kernel(KArgs p, const float* __restrict__ rowsum, int n_nblk,
                                                           int n_mt, int GM) {
  __shared__ P2Stage<1, MW == 1> st0, st1, st2;
  qgemm_p2_body<EPI, GPB, SL, MW, 1, NS>(p, rowsum, n_nblk, n_mt, GM, st0, st1, NS == 3 ? st2 : st0);
}

template <int EPI, int MW, int WM, int NS>
void launch_p2(const KArgs& ka, const float* rowsum, int M_total, hipStream_t s) {
  constexpr int MT = 64 * WM;
  const int n_nblk = EPI == 1 ? (ka.N / 2 + 127) / 128 : (ka.N + 255) / 256;
  // nested MWQ in chunks: at most one partial 16-row chunk per width sub-segment, 4 WM chunks per
  // workgroup; otherwise at most one partial row tile per segment
  const int n_mt = MW == 1 ? (M_total / 16 + ka.nseg + 4 * WM - 1) / (4 * WM) + ka.nseg / 3
                           : (M_total + MT - 1) / MT + ka.nseg;
  const int GM = group_rows(ka, M_total, n_mt, MT, 1, 4u << 20);  // measured best: about 4 MB
  const int items = n_nblk * ((n_mt + GM - 1) / GM) * GM;
  const dim3 grid((unsigned)(((items + 7) / 8) * 8));
  const dim3 block(256 * WM);
#define P2_LAUNCH(GPB, SL)                                                                                   \
  do {                                                                                                       \
    if constexpr (WM == 2)                                                                                   \
      hipLaunchKernelGGL((qgemm_p2_kernel<EPI, GPB, SL, MW, NS>), grid, block, 0, s, ka, rowsum, n_nblk, n_mt, GM); \
    else                                                                                                     \
      hipLaunchKernelGGL((qgemm_p2h_kernel<EPI, GPB, SL, MW, NS>), grid, block, 0, s, ka, rowsum, n_nblk, n_mt, GM); \
  } while (0)
  const bool sl = ((ka.K / ka.G) & 1) == 0;
  switch (ka.G) {
    case 128: if (sl) P2_LAUNCH(1, true); else P2_LAUNCH(1, false); break;
    case 64: if (sl) P2_LAUNCH(2, true); else P2_LAUNCH(2, false); break;
    default:  // G = 32: 128-row workgroups only (one scale dword per channel and group pair)
      if constexpr (WM == 2) {
        if (sl) P2_LAUNCH(4, true);
        else P2_LAUNCH(4, false);
      }
      break;
  }
#undef P2_LAUNCH
}

// path: 0 = small-row-tile kernel, 64 / 128 = large-row-tile kernel with that
// tile height, 2 = 128-row LDS-DMA kernel (INT4; row sums in `ws`)
template <int EPI>
void launch_p2d(const KArgs& ka, const float* rowsum, int M_total, hipStream_t s) {
  const int n_nblk = (ka.N + 127) / 128;
  const int n_mt = (M_total + kP2Rows - 1) / kP2Rows + ka.nseg;
  const int GM = group_rows(ka, M_total, n_mt, kP2Rows, 3, 4u << 20);
  const int items = n_nblk * ((n_mt + GM - 1) / GM) * GM;
  const dim3 grid((unsigned)(((items + 7) / 8) * 8));
  hipLaunchKernelGGL((qgemm_p2d_kernel<EPI>), grid, dim3(kP2Threads), 0, s, ka, rowsum, n_nblk, n_mt, GM);
}

template <int EPI>
void launch_epi(const KArgs& ka, int fmt, int path, int M_total, int A_rows, void* ws, const XTab& tab,
                hipStream_t s) {
  if (path == 3 && EPI != 1) {
    float* rs = static_cast<float*>(ws);
    hipLaunchKernelGGL(rowsum_full_kernel, dim3((unsigned)((A_rows + 3) / 4)), dim3(256), 0, s, ka.A, A_rows, ka.K,
                       -(128.0f + (float)ka.z), rs);
    launch_p2d<EPI>(ka, rs, M_total, s);
    return;
  }
  if (path == 2 || path == 5) {
    float* rs = static_cast<float*>(ws);
    const int rows = A_rows;
    hipLaunchKernelGGL(rowsum_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, ka.A, rows, ka.K, ka.G,
                       -(128.0f + (float)ka.z), rs);
    // 64-row workgroups (two per CU) unless G = 32 (four groups per K block)
    const int mw = fmt == 2 ? (path == 5 ? 2 : 1) : 0;
    if (ka.G == 32) {
      if (mw == 1) launch_p2<EPI, 1, 2, 3>(ka, rs, M_total, s);
      else if (mw == 2) launch_p2<EPI, 2, 2, 3>(ka, rs, M_total, s);
      else launch_p2<EPI, 0, 2, 3>(ka, rs, M_total, s);
    } else {
      if (mw == 1) launch_p2<EPI, 1, P2_WM, P2_NS>(ka, rs, M_total, s);
      else if (mw == 2) launch_p2<EPI, 2, P2_WM, P2_NS>(ka, rs, M_total, s);
      else launch_p2<EPI, 0, P2_WM, P2_NS>(ka, rs, M_total, s);
    }
    return;
  }
  if (fmt != 3 && path != 0 && path != 1) {
    // 64 rows per workgroup with 8 (path 64) or 4 (65) wavefront columns, or
    // 128 rows as two rows of 4 (128)
    if (fmt == 1) {
      if (path == 64) launch_p<1, EPI, 1, 8>(ka, M_total, s);
      else if (path == 65) launch_p<1, EPI, 1, 4>(ka, M_total, s);
      else launch_p<1, EPI, 2, 4>(ka, M_total, s);
    } else {
      if (path == 64) launch_p<2, EPI, 1, 8>(ka, M_total, s);
      else if (path == 65) launch_p<2, EPI, 1, 4>(ka, M_total, s);
      else launch_p<2, EPI, 2, 4>(ka, M_total, s);
    }
    return;
  }
  // a workgroup covers 64 SwiGLU channels or 128 plain channels
  const int gx = EPI == 1 ? (ka.N / 2 + 63) / 64 : (ka.N + 127) / 128;
  if (fmt == 3) {
    const int gy = (M_total + kRows - 1) / kRows + ka.nseg;
    if (ka.base) hipLaunchKernelGGL((qgemm_delta_kernel<EPI, true>), dim3(gx, gy), dim3(kThreads), 0, s, ka);
    else hipLaunchKernelGGL((qgemm_delta_kernel<EPI, false>), dim3(gx, gy), dim3(kThreads), 0, s, ka);
    return;
  }
  // row tiles: at most one partial tile per (tile) segment; the plain
  // epilogues may split K into the workspace
  KArgs kd = ka;
  if (EPI != 1) kd.part = static_cast<float*>(ws);
  const int n_rt = decode_row_tiles(fmt, path, M_total, ka.nseg / ka.S);
  if (fmt == 1) launch_d<1, EPI>(kd, gx, n_rt, tab, s);
  else if (fmt == 4) launch_d<5, EPI>(kd, gx, n_rt, tab, s);  // a width per expert
  else if (path == 1) launch_d<2, EPI>(kd, gx, n_rt, tab, s);  // one width per tile
  else launch_d<4, EPI>(kd, gx, n_rt, tab, s);                 // all widths per tile
}

}  // namespace


int launch_qgemm(const QGemmArgs& a, void* stream) {
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (a.M_total == 0) return 0;
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
  ka.part = nullptr;
  ka.M_total = a.M_total;
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
  (void)swiglu;
  const int path = pick_path(w, a.M_total, a.nseg, a.epilogue, a.kernel);
  // per-expert widths: width, zero point and first 256-byte unit of each expert's tile blocks
  static const XTab kNoTab{};
  XTab tab{};
  if (w.fmt == 4) {
    uint32_t off = 0;
    for (int e = 0; e < w.E; ++e) {
      tab.bits[e] = (uint8_t)w.xbits[e];
      tab.zero[e] = (uint8_t)w.xzero[e];
      tab.off[e] = off;
      off += (uint32_t)((w.N / 16) * (w.K / 128) * w.xbits[e]);
    }
  }
  const XTab& t = w.fmt == 4 ? tab : kNoTab;
  if (a.epilogue == 1) launch_epi<1>(ka, w.fmt, path, a.M_total, a.A_rows, a.ws, t, s);
  else if (a.epilogue == 2) launch_epi<2>(ka, w.fmt, path, a.M_total, a.A_rows, a.ws, t, s);
  else if (a.epilogue == 3) launch_epi<3>(ka, w.fmt, path, a.M_total, a.A_rows, a.ws, t, s);
  else launch_epi<0>(ka, w.fmt, path, a.M_total, a.A_rows, a.ws, t, s);
  return (int)hipGetLastError();
}

// ------------------------------------------------ static scratch (no allocation)
// Device scratch of the no-allocation grouped GEMM: the same workspace the
// kernels take from the caller elsewhere (activation row sums, split-K
// partial sums), held in a device array that each GPU keeps until the process
// ends.  In host code `scratch` is only a stand-in for the symbol: its device
// address, one per GPU, comes from hipGetSymbolAddress with that GPU current
// and is what the kernels receive.
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

int qgemm_static_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return 0;
}

}  // namespace moe

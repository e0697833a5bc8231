// Grouping of (token, slot) pairs by expert (expert-aware batching, Read-ME
// summary; grouped expert execution, ExactMoE page), optionally sub-keyed by
// the pair's bit-width (Bit Gate of the Dual Routing equations, D2MoE page).
//
// A stable counting sort over keys 0..NK-1 (NK = E*S) plus one overflow key
// NK for invalid pairs:
//   count   per-chunk key histograms (LDS atomics: counts are order-free)
//   scan    per key, exclusive scan over chunks, then over keys
//   scatter each chunk walks its pairs in order, 256 at a time; a pair's rank
//           among equal keys inside a wavefront comes from bit-sliced ballots,
//           across the chunk's 4 wavefronts from tagged LDS counters.  The
//           result is the unique stable order: ascending (key, pair index).
// Small problems run all three phases in one workgroup (one launch).
#include "common.h"

namespace moe {

namespace {
constexpr int kThreads = 256;
constexpr int kChunk = kPermuteChunk;        // pairs per workgroup in the multi-block path
constexpr int kSmallMax = kPermuteSmallMax;  // up to this many pairs: single workgroup
constexpr int kMaxKeys = 3 * 1024 + 1;

struct Keyer {
  const int32_t* ids;
  const uint8_t* bits;
  int E, S, NK;
  __device__ __forceinline__ int key(int p, uint32_t& bad) const {
    const int id = ids[p];
    bool ok = (unsigned)id < (unsigned)E;
    int k = id;
    if (S == 3) {
      const int b = bits[p];
      ok = ok && b >= 2 && b <= 4;
      k = id * 3 + (4 - b);
    }
    if (!ok) {
      bad = 1;
      return NK;
    }
    return k;
  }
};

__device__ __forceinline__ int nbits_for(int n) {  // bits to tell keys 0..n apart
  int b = 0;
  while ((1 << b) <= n) ++b;
  return b;
}

// Exclusive scan in place over data[0..n) (LDS), all NT threads of the block.
// Returns the total.
template <int NT>
__device__ int block_exclusive_scan(int* data, int n, int* scratch /* >= NT/64 + 1 ints */) {
  constexpr int kThreads = NT;
  const int tid = threadIdx.x;
  const int per = (n + kThreads - 1) / kThreads;
  const int lo = min(n, tid * per), hi = min(n, lo + per);
  int local = 0;
  for (int i = lo; i < hi; ++i) local += data[i];
  // inclusive scan across the wave
  const int lane = tid & 63;
  int v = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(v, off, 64);
    if (lane >= off) v += o;
  }
  if (lane == 63) scratch[tid >> 6] = v;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int w = 0; w < kThreads / 64; ++w) {
      const int t = scratch[w];
      scratch[w] = run;
      run += t;
    }
    scratch[kThreads / 64] = run;
  }
  __syncthreads();
  int run = scratch[tid >> 6] + v - local;
  for (int i = lo; i < hi; ++i) {
    const int t = data[i];
    data[i] = run;
    run += t;
  }
  const int total = scratch[kThreads / 64];
  __syncthreads();
  return total;
}

// Stable scatter of pairs [p0, p1) whose key bases are in base[] (LDS; base[key]
// = output position of the next pair with that key).  tagbuf: NT/64 * (NK+1)
// ints.  NT threads take NT pairs per step.
template <int NT>
__device__ void scatter_chunk(const Keyer& kr, int p0, int p1, int* base, int* tagbuf, int32_t* sorted_pair,
                              int32_t* pair_pos) {
  constexpr int kThreads = NT;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nk1 = kr.NK + 1;
  const int nbits = nbits_for(kr.NK);
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int step = 0;
  for (int s0 = p0; s0 < p1; s0 += kThreads, ++step) {
    const int p = s0 + tid;
    const bool act = p < p1;
    uint32_t bad = 0;
    const int key = act ? kr.key(p, bad) : 0;
    uint64_t m = __ballot(act);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (key >> b) & 1;
      const uint64_t bb = __ballot(bit);
      m &= bit ? bb : ~bb;
    }
    const int rank = __popcll(m & lt);
    const int cnt = __popcll(m);
    const int tag = (step & 0xffff) << 16;
    if (act && rank == 0) tagbuf[wv * nk1 + key] = tag | cnt;
    __syncthreads();
    if (act) {
      int off = base[key];
      for (int w = 0; w < wv; ++w) {
        const int t = tagbuf[w * nk1 + key];
        if ((t & 0xffff0000) == tag) off += t & 0xffff;
      }
      const int pos = off + rank;
      sorted_pair[pos] = p;
      pair_pos[p] = pos;
    }
    __syncthreads();
    if (act && rank == 0) atomicAdd(&base[key], cnt);
    __syncthreads();
  }
}

// All three phases in one workgroup of NT threads.  hist: NK+1 ints,
// tagbuf: NT/64 * (NK+1) ints, scratch: NT/64 + 1 ints (all LDS).
template <int NT>
__device__ void permute_block(const Keyer& kr, int P, int32_t* counts, int32_t* seg_offsets, int32_t* sorted_pair,
                              int32_t* pair_pos, uint32_t* flag, int* hist, int* tagbuf, int* scratch,
                              uint32_t* sbad) {
  const int tid = threadIdx.x;
  const int nk1 = kr.NK + 1;
  for (int i = tid; i < nk1; i += NT) hist[i] = 0;
  for (int i = tid; i < (NT / 64) * nk1; i += NT) tagbuf[i] = -1;  // tag 0xffff never matches step 0..
  if (tid == 0) *sbad = 0;
  __syncthreads();
  uint32_t bad = 0;
  for (int p = tid; p < P; p += NT) atomicAdd(&hist[kr.key(p, bad)], 1);
  if (bad) atomicOr(sbad, 1u);
  __syncthreads();
  for (int e = tid; e < kr.E; e += NT) {
    int c = 0;
    for (int s = 0; s < kr.S; ++s) c += hist[e * kr.S + s];
    counts[e] = c;
  }
  __syncthreads();
  block_exclusive_scan<NT>(hist, nk1, scratch);
  for (int i = tid; i < nk1; i += NT) seg_offsets[i] = hist[i];
  if (tid == 0) flag[0] = *sbad;
  __syncthreads();
  scatter_chunk<NT>(kr, 0, P, hist, tagbuf, sorted_pair, pair_pos);
}

__global__ __launch_bounds__(kThreads) void permute_small_kernel(Keyer kr, int P, int32_t* counts,
                                                                 int32_t* seg_offsets, int32_t* sorted_pair,
                                                                 int32_t* pair_pos, uint32_t* flag) {
  __shared__ int hist[kMaxKeys];
  __shared__ int tagbuf[4 * kMaxKeys];
  __shared__ int scratch[8];
  __shared__ uint32_t sbad;
  permute_block<kThreads>(kr, P, counts, seg_offsets, sorted_pair, pair_pos, flag, hist, tagbuf, scratch, &sbad);
}

// Routing and grouping of a small batch in one launch: every workgroup routes
// 4 tokens (one wavefront each, the rank method of the routing kernel), makes
// its ids visible device-wide and counts itself in; the last workgroup to
// arrive groups all pairs and resets the counter.  Outputs are identical to
// moe_route_topk followed by moe_permute.
constexpr int kRPMaxE = kRoutePermuteMaxE, kRPMaxKeys = 3 * kRPMaxE + 1;
__global__ __launch_bounds__(kThreads) void route_permute_kernel(const float* __restrict__ logits, int T, int E,
                                                                 int k, const uint8_t* bits, int32_t* ids, float* w,
                                                                 int32_t* counts, int32_t* seg_offsets,
                                                                 int32_t* sorted_pair, int32_t* pair_pos,
                                                                 uint32_t* ws) {
  __shared__ float sel_val[4][64];
  __shared__ double sel_exp[4][64];
  __shared__ int hist[kRPMaxKeys];
  __shared__ int tagbuf[4 * kRPMaxKeys];
  __shared__ int scratch[8];
  __shared__ uint32_t sbad;
  __shared__ int last;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wv;
  if (t < T) {
    const float v = lane < E ? logits[(size_t)t * E + lane] : -__builtin_inff();
    route_token_rank(v, E, k, ids + (size_t)t * k, w + (size_t)t * k, sel_val[wv], sel_exp[wv], nullptr);
  }
  __threadfence();  // release this workgroup's ids and gates device-wide
  __syncthreads();
  uint32_t* counter = ws + 1;  // ws[0] is the invalid-id flag
  if (threadIdx.x == 0) last = atomicAdd(counter, 1u) == gridDim.x - 1;
  __syncthreads();
  if (!last) return;
  __threadfence();  // acquire every workgroup's ids
  const int S = bits ? 3 : 1;
  const Keyer kr{ids, bits, E, S, E * S};
  permute_block<kThreads>(kr, T * k, counts, seg_offsets, sorted_pair, pair_pos, ws, hist, tagbuf, scratch, &sbad);
  if (threadIdx.x == 0) *counter = 0u;  // ready for the next call
}

// ---- multi-block path -------------------------------------------------------
// workspace: [0] flag word, [16 B ..] nb flags, then nb * (NK+1) ints
__global__ __launch_bounds__(kThreads) void permute_count_kernel(Keyer kr, int P, int* chunk_hist,
                                                                 uint32_t* chunk_flag) {
  __shared__ int hist[kMaxKeys];
  __shared__ uint32_t sbad;
  const int tid = threadIdx.x;
  const int nk1 = kr.NK + 1;
  for (int i = tid; i < nk1; i += kThreads) hist[i] = 0;
  if (tid == 0) sbad = 0;
  __syncthreads();
  const int p0 = blockIdx.x * kChunk, p1 = min(P, p0 + kChunk);
  uint32_t bad = 0;
  for (int p = p0 + tid; p < p1; p += kThreads) atomicAdd(&hist[kr.key(p, bad)], 1);
  if (bad) atomicOr(&sbad, 1u);
  __syncthreads();
  int* out = chunk_hist + (size_t)blockIdx.x * nk1;
  for (int i = tid; i < nk1; i += kThreads) out[i] = hist[i];
  if (tid == 0) chunk_flag[blockIdx.x] = sbad;
}

// Per key, the exclusive scan over chunks, then over keys; chunk_hist[b][key]
// becomes the output position of chunk b's first pair with that key.  When
// the chunk histograms fit (kScanLds ints) they are read once, coalesced, into
// LDS, scanned there and written back once; otherwise each key walks its
// chunks in global memory (a chain of dependent round trips).
constexpr int kScanLds = 8192;
__global__ __launch_bounds__(kThreads) void permute_scan_kernel(Keyer kr, int nb, int* chunk_hist,
                                                                const uint32_t* chunk_flag, int32_t* counts,
                                                                int32_t* seg_offsets, uint32_t* flag) {
  __shared__ int total[kMaxKeys];
  __shared__ int sh[kScanLds];
  __shared__ int scratch[8];
  __shared__ uint32_t sbad;
  const int tid = threadIdx.x;
  const int nk1 = kr.NK + 1;
  const int n = nb * nk1;
  const bool in_lds = n <= kScanLds;
  if (tid == 0) sbad = 0;
  if (in_lds)
    for (int i = tid; i < n; i += kThreads) sh[i] = chunk_hist[i];
  __syncthreads();
  for (int key = tid; key < nk1; key += kThreads) {
    int run = 0;
    for (int b = 0; b < nb; ++b) {
      int* h = in_lds ? sh + b * nk1 + key : chunk_hist + (size_t)b * nk1 + key;
      const int t = *h;
      *h = run;
      run += t;
    }
    total[key] = run;
  }
  uint32_t bad = 0;
  for (int b = tid; b < nb; b += kThreads) bad |= chunk_flag[b];
  if (bad) atomicOr(&sbad, 1u);
  __syncthreads();
  for (int e = tid; e < kr.E; e += kThreads) {
    int c = 0;
    for (int s = 0; s < kr.S; ++s) c += total[e * kr.S + s];
    counts[e] = c;
  }
  __syncthreads();
  block_exclusive_scan<kThreads>(total, nk1, scratch);
  for (int i = tid; i < nk1; i += kThreads) seg_offsets[i] = total[i];
  if (in_lds) {
    for (int i = tid; i < n; i += kThreads) chunk_hist[i] = sh[i] + total[i % nk1];
  } else {
    for (int key = tid; key < nk1; key += kThreads) {
      const int base = total[key];
      for (int b = 0; b < nb; ++b) chunk_hist[(size_t)b * nk1 + key] += base;
    }
  }
  if (tid == 0) flag[0] = sbad;
}

__global__ __launch_bounds__(kThreads) void permute_scatter_kernel(Keyer kr, int P, const int* chunk_base,
                                                                   int32_t* sorted_pair, int32_t* pair_pos) {
  __shared__ int base[kMaxKeys];
  __shared__ int tagbuf[4 * kMaxKeys];
  const int tid = threadIdx.x;
  const int nk1 = kr.NK + 1;
  for (int i = tid; i < nk1; i += kThreads) base[i] = chunk_base[(size_t)blockIdx.x * nk1 + i];
  for (int i = tid; i < 4 * nk1; i += kThreads) tagbuf[i] = -1;
  __syncthreads();
  const int p0 = blockIdx.x * kChunk, p1 = min(P, p0 + kChunk);
  scatter_chunk<kThreads>(kr, p0, p1, base, tagbuf, sorted_pair, pair_pos);
}

__global__ __launch_bounds__(kThreads) void gather_rows_kernel(const uint16_t* __restrict__ x, int H, int k,
                                                               const int32_t* __restrict__ sorted_pair, int P,
                                                               uint16_t* __restrict__ x_perm) {
  const int i = blockIdx.x;
  if (i >= P) return;
  const int t = sorted_pair[i] / k;
  const u32x4* src = reinterpret_cast<const u32x4*>(x + (size_t)t * H);
  u32x4* dst = reinterpret_cast<u32x4*>(x_perm + (size_t)i * H);
  for (int c = threadIdx.x; c < H / 8; c += kThreads) dst[c] = src[c];
}

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }
}  // namespace


int launch_route_permute(const float* logits, int T, int E, int k, const uint8_t* bits, int32_t* ids, float* w,
                         int32_t* counts, int32_t* seg_offsets, int32_t* sorted_pair, int32_t* pair_pos, void* ws,
                         void* stream) {
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(route_permute_kernel, dim3((unsigned)((T + 3) / 4)), dim3(kThreads), 0, s, logits, T, E, k, bits,
                     ids, w, counts, seg_offsets, sorted_pair, pair_pos, static_cast<uint32_t*>(ws));
  return (int)hipGetLastError();
}


int launch_permute(const PermuteArgs& a, void* stream) {
  const hipStream_t s = static_cast<hipStream_t>(stream);
  Keyer kr{a.ids, a.bits, a.E, a.S, a.E * a.S};
  uint8_t* ws = static_cast<uint8_t*>(a.ws);
  uint32_t* flag = reinterpret_cast<uint32_t*>(ws);
  if (a.P <= kSmallMax) {
    hipLaunchKernelGGL(permute_small_kernel, dim3(1), dim3(kThreads), 0, s, kr, a.P, a.counts, a.seg_offsets,
                       a.sorted_pair, a.pair_pos, flag);
  } else {
    const int nb = (a.P + kChunk - 1) / kChunk;
    uint32_t* chunk_flag = reinterpret_cast<uint32_t*>(ws + 256);
    int* chunk_hist = reinterpret_cast<int*>(ws + 256 + align256((size_t)nb * 4));
    hipLaunchKernelGGL(permute_count_kernel, dim3(nb), dim3(kThreads), 0, s, kr, a.P, chunk_hist, chunk_flag);
    hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(kThreads), 0, s, kr, nb, chunk_hist, chunk_flag,
                       a.counts, a.seg_offsets, flag);
    hipLaunchKernelGGL(permute_scatter_kernel, dim3(nb), dim3(kThreads), 0, s, kr, a.P, chunk_hist,
                       a.sorted_pair, a.pair_pos);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return (int)e;
  if (a.x_perm && a.P > 0) {
    hipLaunchKernelGGL(gather_rows_kernel, dim3(a.P), dim3(kThreads), 0, s, a.x, a.H, a.k, a.sorted_pair, a.P,
                       a.x_perm);
    e = hipGetLastError();
  }
  return (int)e;
}

}  // namespace moe

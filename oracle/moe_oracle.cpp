// CPU oracle of the routed-expert quantized MoE path, plain C++17 in float64.
// TEST INFRASTRUCTURE ONLY: built for the test suite, the smoke check and the
// benchmark's CPU baseline; the GPU library never links or calls it, and it
// shares no code, header, table or helper with the GPU library.  It reads the
// generator's canonical storage (bit patterns of bf16 / fp16 values, packed
// codes) and decodes every format with its own code.
//
// What is computed is the plain definition of the layer.  The method changes
// only how expert weights are stored and moved ("Every Expert Counts: ExactMoE
// for Memory-Efficient W4A16 Inference": the router's decisions are unchanged
// and every selected expert runs), so:
//   route    per token, the k largest logits, descending, ties to the lower
//            expert index (expert gate of the Dual Routing equations, D2MoE
//            page, Design); gate = softmax over the k selected logits
//   group    pairs p = t*k + j keyed by expert (and by 4 - b for nested
//            weights), stable in p (expert-aware batching, Read-ME summary)
//   dequant  INT4 (ExactMoE W4A16): w = s[n][k/G] * (c - z);
//            nested planes (D2MoE, MWQ equations W(2)=Q2, W(3)=Q2+D3,
//            W(4)=Q2+D3+D4): c_b = 4 q2 + 2 d3 [b>=3] + d4 [b=4];
//            a b-bit expert (EdgeMoE, expert-wise bit-width adaptation):
//            w = s * (c - z_e) with c the expert's own b-bit code;
//            delta (ME-Switch): d = salient value on a salient input channel,
//            else step[n] * (c - z)
//   expert   g = x Wg^T, u = x Wu^T, h = silu(g) * u, y = h Wd^T
//   combine  out[t] = sum_j w[t][j] * y[t*k + j]
// Every sum runs in ascending index order in float64 (so results do not
// depend on the thread count); a second output evaluates the layer with h
// rounded once to bf16 before the down product (the 16-bit activation that
// W4A16 and the D2MoE pipeline equation feed to the next expert GEMM), as a
// diagnostic beside the definition.
//
// Parallelism: std::thread over (segment, tile of pairs) work items, the
// weights of one (expert, bit-width) dequantised at a time.  Dense products
// run over blocks of 32 output channels with the dequantised weights laid out
// [channel block][k][32]: each output still sums its k terms in ascending
// order, one multiply-add at a time.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <functional>
#include <thread>
#include <vector>

namespace {

constexpr int kNB = 32;  // output channels per block of the dense products
constexpr int kTB = 8;   // rows per tile of the dense products

double bf16_value(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

// IEEE binary16 bit pattern -> exact value.
double f16_value(uint16_t h) {
  const int sign = (h >> 15) & 1, exp = (h >> 10) & 31, man = h & 1023;
  double v;
  if (exp == 0) v = ldexp((double)man, -24);
  else if (exp == 31) v = man ? NAN : INFINITY;
  else v = ldexp((double)(1024 + man), exp - 25);
  return sign ? -v : v;
}

// Nearest value with 8 significant bits (bf16), ties to even, from a double.
double round_bf16(double v) {
  if (v == 0.0 || !isfinite(v)) return v;
  int e;
  const double m = frexp(v, &e);  // v = m 2^e, 0.5 <= |m| < 1
  return ldexp(nearbyint(ldexp(m, 8)), e - 8);
}

double silu(double g) { return g / (1.0 + exp(-g)); }

int n_threads(int want) {
  if (want > 0) return want;
  const unsigned h = std::thread::hardware_concurrency();
  return h ? (int)h : 1;
}

// Runs body(i) for i in [0, n) on `threads` threads (work handed out in order).
void parallel_for(int n, int threads, const std::function<void(int)>& body) {
  threads = std::min(threads, n);
  if (threads <= 1) {
    for (int i = 0; i < n; ++i) body(i);
    return;
  }
  std::atomic<int> next{0};
  std::vector<std::thread> pool;
  for (int w = 0; w < threads; ++w)
    pool.emplace_back([&] {
      for (int i = next.fetch_add(1); i < n; i = next.fetch_add(1)) body(i);
    });
  for (auto& t : pool) t.join();
}

// A dequantised matrix W [N][K] (row n = output channel n), stored as
// blocks[N/32][K][32]: element (n, k) at ((n / 32) * K + k) * 32 + n % 32.
struct Dense {
  int N = 0, K = 0;
  std::vector<double> v;
  void resize(int n, int k) {
    N = n;
    K = k;
    v.assign((size_t)((n + kNB - 1) / kNB) * k * kNB, 0.0);
  }
  double& at(int n, int k) { return v[((size_t)(n / kNB) * K + k) * kNB + n % kNB]; }
};

// out[t][n] = sum_{k ascending} a[t][k] * W[n][k] for rows t < rows (a: rows
// of lda doubles), channels [n0, n1) of W, into out rows of ldo doubles.
// Built without floating-point contraction: every term is a rounded product
// added to the running sum.  Compiled for AVX2 and for the baseline, chosen
// at load time (same arithmetic either way).
__attribute__((target_clones("avx2", "default"))) void dense_product(const double* a, int rows, int lda, const Dense& W,
                                                                    int n0, int n1, double* out, int ldo) {
  for (int t0 = 0; t0 < rows; t0 += kTB) {
    const int tb = std::min(kTB, rows - t0);
    for (int nb = n0 / kNB; nb * kNB < n1; ++nb) {
      double acc[kTB][kNB];
      for (int t = 0; t < kTB; ++t)
        for (int j = 0; j < kNB; ++j) acc[t][j] = 0.0;
      const double* wb = W.v.data() + (size_t)nb * W.K * kNB;
      for (int k = 0; k < W.K; ++k) {
        const double* w = wb + (size_t)k * kNB;
        for (int t = 0; t < tb; ++t) {
          const double xk = a[(size_t)(t0 + t) * lda + k];
          for (int j = 0; j < kNB; ++j) acc[t][j] += xk * w[j];
        }
      }
      for (int t = 0; t < tb; ++t)
        for (int j = 0; j < kNB; ++j) {
          const int n = nb * kNB + j;
          if (n >= n0 && n < n1 && n < W.N) out[(size_t)(t0 + t) * ldo + (n - n0)] = acc[t][j];
        }
    }
  }
}

// ------------------------------------------------------------ decoding
// 4-bit code k of a row: byte k/2, even k in the low nibble.
int code_u4(const uint8_t* row, int k) { return (row[k >> 1] >> ((k & 1) * 4)) & 15; }
// 2-bit field k of a row: byte k/4, bits 2 (k & 3) .. 2 (k & 3) + 1.
int code_u2(const uint8_t* row, int k) { return (row[k >> 2] >> (2 * (k & 3))) & 3; }
// 1-bit field k of a row: bit k & 7 of byte k/8.
int code_u1(const uint8_t* row, int k) { return (row[k >> 3] >> (k & 7)) & 1; }
// b-bit code number i of a little-endian bit stream (bits i*b .. i*b + b - 1).
int code_stream(const uint8_t* s, size_t i, int b) {
  int c = 0;
  for (int j = 0; j < b; ++j) {
    const size_t bit = i * (size_t)b + j;
    c |= ((s[bit >> 3] >> (bit & 7)) & 1) << j;
  }
  return c;
}

// Which format a matrix is stored in, and its storage (canonical layouts).
struct Store {
  int fmt;            // 1 INT4, 2 nested planes, 4 own width per expert
  int N, K, G;
  const uint8_t* codes;  // INT4 [E][N][K/2]; planes: q2 [E][N][K/4]; per expert: flat stream
  const uint8_t* d3;     // planes: [E][N][K/8]
  const uint8_t* d4;
  const uint16_t* scales;  // fp16 [E][N][K/G]
  const int32_t* bits;     // per expert (format 4)
  const int32_t* zero;     // per expert (format 4)
  int z;                   // zero point (formats 1, 2)
};

// W of expert e at bit-width b (b only matters for nested planes).
void dequant(const Store& st, int e, int b, Dense& W, int threads) {
  W.resize(st.N, st.K);
  const int N = st.N, K = st.K, G = st.G;
  size_t stream_off = 0;  // format 4: byte offset of expert e's codes
  if (st.fmt == 4)
    for (int j = 0; j < e; ++j) stream_off += (size_t)N * K * st.bits[j] / 8;
  parallel_for(N, threads, [&](int n) {
    const uint16_t* srow = st.scales + ((size_t)e * N + n) * (K / G);
    double s = 0.0;
    for (int k = 0; k < K; ++k) {
      if (k % G == 0) s = f16_value(srow[k / G]);
      int c, z = st.z;
      if (st.fmt == 1) {
        c = code_u4(st.codes + ((size_t)e * N + n) * (K / 2), k);
      } else if (st.fmt == 2) {
        const size_t r = (size_t)e * N + n;
        c = 4 * code_u2(st.codes + r * (K / 4), k);
        if (b >= 3) c += 2 * code_u1(st.d3 + r * (K / 8), k);
        if (b == 4) c += code_u1(st.d4 + r * (K / 8), k);
      } else {
        c = code_stream(st.codes + stream_off, (size_t)n * K + k, st.bits[e]);
        z = st.zero[e];
      }
      W.at(n, k) = s * (double)(c - z);
    }
  });
}

// ------------------------------------------------------------ routing
void route(const float* logits, int T, int E, int k, int32_t* ids, double* w) {
  std::vector<int> order(E);
  for (int t = 0; t < T; ++t) {
    const float* l = logits + (size_t)t * E;
    for (int e = 0; e < E; ++e) order[e] = e;
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return l[a] > l[b]; });
    const double l0 = l[order[0]];
    double sum = 0.0;
    for (int j = 0; j < k; ++j) sum += exp((double)l[order[j]] - l0);
    for (int j = 0; j < k; ++j) {
      ids[(size_t)t * k + j] = order[j];
      w[(size_t)t * k + j] = exp((double)l[order[j]] - l0) / sum;
    }
  }
}

// key of pair p: e (S = 1) or 3 e + (4 - b) (nested planes, S = 3).  Returns
// false on an id or bit-width out of range.
bool group(const int32_t* ids, const uint8_t* bits, int P, int E, int32_t* counts, int32_t* seg_offsets,
           int32_t* sorted_pair, int32_t* pair_pos) {
  const int S = bits ? 3 : 1;
  std::vector<int> key(P);
  for (int e = 0; e < E; ++e) counts[e] = 0;
  std::vector<int> per_key((size_t)E * S, 0);
  for (int p = 0; p < P; ++p) {
    if (ids[p] < 0 || ids[p] >= E) return false;
    if (bits && (bits[p] < 2 || bits[p] > 4)) return false;
    key[p] = bits ? 3 * ids[p] + (4 - bits[p]) : ids[p];
    ++counts[ids[p]];
    ++per_key[key[p]];
  }
  seg_offsets[0] = 0;
  for (int q = 0; q < E * S; ++q) seg_offsets[q + 1] = seg_offsets[q] + per_key[q];
  std::vector<int> fill(seg_offsets, seg_offsets + E * S);
  for (int p = 0; p < P; ++p) {  // ascending p inside each key: a stable counting sort
    const int i = fill[key[p]]++;
    sorted_pair[i] = p;
    pair_pos[p] = i;
  }
  return true;
}

}  // namespace

// ====================================================================== C API
extern "C" {

int oracle_hardware_threads(void) { return n_threads(0); }

int oracle_route_topk(const float* logits, int T, int E, int k, int32_t* ids, double* w) {
  if (T < 0 || E < 1 || k < 1 || k > E) return 1;
  for (size_t i = 0; i < (size_t)T * E; ++i)
    if (!isfinite(logits[i])) return 2;
  route(logits, T, E, k, ids, w);
  return 0;
}

int oracle_permute(const int32_t* ids, const uint8_t* bits, int P, int E, int32_t* counts, int32_t* seg_offsets,
                   int32_t* sorted_pair, int32_t* pair_pos) {
  return group(ids, bits, P, E, counts, seg_offsets, sorted_pair, pair_pos) ? 0 : 1;
}

// One routed-expert SwiGLU layer.  Storage as the generator writes it:
//   x bf16 [T][H]; logits f32 [T][E]; pair_bits u8 [T*k] (nested planes) or NULL
//   gate_up: N = 2I, K = H (rows [0, I) gate, [I, 2I) up); down: N = H, K = I
// want: token mask [T] (1 = compute its pairs), or NULL for every token.
// Outputs (any of the float64 ones may be NULL): ids, w [T*k]; counts [E];
// seg_offsets [E*S + 1]; sorted_pair, pair_pos [T*k]; h_perm [T*k][I];
// y_perm, y_perm16 [T*k][H]; out, out16 [T][H].  Rows of pairs not computed
// are left untouched.  Returns 0, or non-zero on bad input.
int oracle_moe_forward(int fmt, int T, int H, int I, int E, int k, int G, int zero_point, const uint16_t* x,
                       const float* logits, const uint8_t* pair_bits, const uint8_t* gu_codes, const uint8_t* gu_d3,
                       const uint8_t* gu_d4, const uint16_t* gu_scales, const uint8_t* dn_codes,
                       const uint8_t* dn_d3, const uint8_t* dn_d4, const uint16_t* dn_scales,
                       const int32_t* expert_bits, const int32_t* expert_zero, const uint8_t* want, int threads,
                       int32_t* ids, double* w, int32_t* counts, int32_t* seg_offsets, int32_t* sorted_pair,
                       int32_t* pair_pos, double* h_perm, double* y_perm, double* y_perm16, double* out,
                       double* out16) {
  if (!(fmt == 1 || fmt == 2 || fmt == 4) || T < 0 || E < 1 || k < 1 || k > E || H % G || I % G) return 1;
  threads = n_threads(threads);
  const int P = T * k, S = fmt == 2 ? 3 : 1;
  if (oracle_route_topk(logits, T, E, k, ids, w) != 0) return 2;
  if (!group(ids, fmt == 2 ? pair_bits : nullptr, P, E, counts, seg_offsets, sorted_pair, pair_pos)) return 3;
  const Store gu{fmt, 2 * I, H, G, gu_codes, gu_d3, gu_d4, gu_scales, expert_bits, expert_zero, zero_point};
  const Store dn{fmt, H, I, G, dn_codes, dn_d3, dn_d4, dn_scales, expert_bits, expert_zero, zero_point};
  std::vector<double> y((size_t)P * H, 0.0), y16((size_t)P * H, 0.0);
  Dense Wgu, Wd;
  for (int seg = 0; seg < E * S; ++seg) {
    // the segment's pairs to compute, in grouped order
    std::vector<int> rows;
    for (int i = seg_offsets[seg]; i < seg_offsets[seg + 1]; ++i)
      if (!want || want[sorted_pair[i] / k]) rows.push_back(i);
    if (rows.empty()) continue;
    const int e = seg / S, b = 4 - seg % S;
    dequant(gu, e, b, Wgu, threads);
    dequant(dn, e, b, Wd, threads);
    const int ntile = ((int)rows.size() + kTB - 1) / kTB;
    parallel_for(ntile, threads, [&](int tile) {
      const int r0 = tile * kTB, nr = std::min(kTB, (int)rows.size() - r0);
      std::vector<double> a((size_t)kTB * H), gu_out((size_t)kTB * 2 * I), h((size_t)kTB * I),
          h16((size_t)kTB * I), yo((size_t)kTB * H);
      for (int r = 0; r < nr; ++r) {
        const uint16_t* xr = x + (size_t)(sorted_pair[rows[r0 + r]] / k) * H;
        for (int c = 0; c < H; ++c) a[(size_t)r * H + c] = bf16_value(xr[c]);
      }
      dense_product(a.data(), nr, H, Wgu, 0, 2 * I, gu_out.data(), 2 * I);
      for (int r = 0; r < nr; ++r)
        for (int n = 0; n < I; ++n) {
          const double v = silu(gu_out[(size_t)r * 2 * I + n]) * gu_out[(size_t)r * 2 * I + I + n];
          h[(size_t)r * I + n] = v;
          h16[(size_t)r * I + n] = round_bf16(v);
        }
      dense_product(h.data(), nr, I, Wd, 0, H, yo.data(), H);
      for (int r = 0; r < nr; ++r) {
        const size_t i = rows[r0 + r];
        memcpy(&y[i * H], &yo[(size_t)r * H], sizeof(double) * H);
        if (h_perm) memcpy(&h_perm[i * I], &h[(size_t)r * I], sizeof(double) * I);
      }
      dense_product(h16.data(), nr, I, Wd, 0, H, yo.data(), H);
      for (int r = 0; r < nr; ++r) memcpy(&y16[(size_t)rows[r0 + r] * H], &yo[(size_t)r * H], sizeof(double) * H);
    });
  }
  for (int t = 0; t < T; ++t) {
    if (want && !want[t]) continue;
    for (int c = 0; c < H; ++c) {
      double acc = 0.0, acc16 = 0.0;
      for (int j = 0; j < k; ++j) {
        const size_t i = pair_pos[(size_t)t * k + j];
        acc += w[(size_t)t * k + j] * y[i * H + c];
        acc16 += w[(size_t)t * k + j] * y16[i * H + c];
      }
      if (out) out[(size_t)t * H + c] = acc;
      if (out16) out16[(size_t)t * H + c] = acc16;
    }
  }
  if (y_perm || y_perm16)
    for (int p = 0; p < P; ++p)
      if (!want || want[sorted_pair[p] / k]) {
        if (y_perm) memcpy(&y_perm[(size_t)p * H], &y[(size_t)p * H], sizeof(double) * H);
        if (y_perm16) memcpy(&y_perm16[(size_t)p * H], &y16[(size_t)p * H], sizeof(double) * H);
      }
  return 0;
}

// The ME-Switch delta layer: y[t] = x[t] W_base^T + x[t] D_{e(t)}^T, tokens
// grouped by expert.  x bf16 [T][K]; ids i32 [T]; base bf16 [N][K]; codes u8
// [E][N][K/4] (2-bit, packed as above); step fp16 [E][N]; salient_idx i32
// [E][n_sal] (distinct); salient_val bf16 [E][n_sal][N]; z: the 2-bit zero
// point.  want: token mask or NULL.  out [T][N] (rows of other tokens untouched).
int oracle_delta_linear(int T, int K, int N, int E, int n_sal, int z, const uint16_t* x, const int32_t* ids,
                        const uint16_t* base, const uint8_t* codes, const uint16_t* step,
                        const int32_t* salient_idx, const uint16_t* salient_val, const uint8_t* want, int threads,
                        int32_t* counts, int32_t* seg_offsets, int32_t* sorted_pair, int32_t* pair_pos,
                        double* out) {
  if (T < 0 || K < 1 || N < 1 || E < 1 || n_sal < 0) return 1;
  threads = n_threads(threads);
  if (!group(ids, nullptr, T, E, counts, seg_offsets, sorted_pair, pair_pos)) return 3;
  Dense Wb, D;
  Wb.resize(N, K);
  parallel_for(N, threads, [&](int n) {
    for (int kk = 0; kk < K; ++kk) Wb.at(n, kk) = bf16_value(base[(size_t)n * K + kk]);
  });
  for (int e = 0; e < E; ++e) {
    std::vector<int> rows;
    for (int i = seg_offsets[e]; i < seg_offsets[e + 1]; ++i)
      if (!want || want[sorted_pair[i]]) rows.push_back(i);
    if (rows.empty()) continue;
    D.resize(N, K);
    parallel_for(N, threads, [&](int n) {
      const double st = f16_value(step[(size_t)e * N + n]);
      const uint8_t* crow = codes + ((size_t)e * N + n) * (K / 4);
      for (int kk = 0; kk < K; ++kk) D.at(n, kk) = st * (double)(code_u2(crow, kk) - z);
      for (int j = 0; j < n_sal; ++j)
        D.at(n, salient_idx[(size_t)e * n_sal + j]) = bf16_value(salient_val[((size_t)e * n_sal + j) * N + n]);
    });
    const int ntile = ((int)rows.size() + kTB - 1) / kTB;
    parallel_for(ntile, threads, [&](int tile) {
      const int r0 = tile * kTB, nr = std::min(kTB, (int)rows.size() - r0);
      std::vector<double> a((size_t)kTB * K), yb((size_t)kTB * N), yd((size_t)kTB * N);
      for (int r = 0; r < nr; ++r) {
        const uint16_t* xr = x + (size_t)sorted_pair[rows[r0 + r]] * K;
        for (int c = 0; c < K; ++c) a[(size_t)r * K + c] = bf16_value(xr[c]);
      }
      dense_product(a.data(), nr, K, Wb, 0, N, yb.data(), N);
      dense_product(a.data(), nr, K, D, 0, N, yd.data(), N);
      for (int r = 0; r < nr; ++r) {
        const int t = sorted_pair[rows[r0 + r]];
        for (int n = 0; n < N; ++n) out[(size_t)t * N + n] = yb[(size_t)r * N + n] + yd[(size_t)r * N + n];
      }
    });
  }
  return 0;
}

}  // extern "C"

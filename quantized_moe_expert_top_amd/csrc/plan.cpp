// Host-side planning of the launches: which grouped-GEMM kernel runs a call,
// how decode-sized GEMMs split K, and how much workspace each entry point
// needs.  Plain C++: shared by the library and the CPU-only build of the host
// layer, and a pure function of the shapes and the caller's kernel choice
// (the host never reads device counts back).
#include "launch.h"

namespace moe {

// ------------------------------------------------------------- grouping
bool route_permute_fusable(int T, int k, int E) {
  return E <= kRoutePermuteMaxE && (int64_t)T * k <= kPermuteSmallMax;
}

namespace {
inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }
}  // namespace

// Word 0: invalid-id flag; word 1: arrival counter of the fused routing and
// grouping; then, for the multi-workgroup path, a flag word per chunk and
// the per-chunk key histograms.
size_t permute_workspace_bytes(int P, int E, int S) {
  const size_t nk1 = (size_t)E * S + 1;
  const size_t nb = P <= kPermuteSmallMax ? 0 : (size_t)(P + kPermuteChunk - 1) / kPermuteChunk;
  return 256 + align256(nb * 4) + align256(nb * nk1 * 4);
}

// --------------------------------------------------------------- repack
size_t tiled_salient_bytes(int E, int N, int n_sal) {
  const size_t nsteps = (size_t)(n_sal + 31) / 32;
  return (size_t)E * (N / 16) * nsteps * 1024;
}

// --------------------------------------------------------- grouped GEMM
// K splits of the decode kernel: one unless the (channel group, row tile)
// items leave the chip short of workgroups (fewer than 3 per CU), then enough
// to bring them to about 4 per CU, each split keeping at least 8 K blocks.
int decode_splits(int n_items, int K) {
  const int KBt = K / 128;
  if (n_items >= 768 || KBt < 16) return 1;
  int n = (1024 + n_items - 1) / n_items;
  n = n < KBt / 8 ? n : KBt / 8;
  const int kb_per = (KBt + n - 1) / n;
  return (KBt + kb_per - 1) / kb_per;  // every split non-empty
}

// Upper bound of the decode kernel's row tiles: one partial tile per tile
// segment (an expert, or for MWQ on path 1 each width of an expert).
int decode_row_tiles(int fmt, int path, int M_total, int E) {
  return (M_total + 15) / 16 + ((fmt == 2 && path == 1) ? 3 * E : E);
}

// path: 0 = 16-row tiles (decode kernel; DELTA2: the 32-row delta kernel),
// 1 = 16-row tiles of one width each (nested MWQ), 64 / 65 = 64-row tiles with
// 8 / 4 wavefront columns, 128 = 128-row register-fed tiles, 2 = the 128-row
// LDS-DMA kernel (INT4, nested MWQ; row sums in the workspace), 3 = the
// 128-row LDS-DMA delta kernel (with a shared base, plain epilogues), 5 = the
// LDS-DMA kernel on row tiles of one width each (nested MWQ).
//
// MOE_KERNEL_AUTO chooses from the mean rows per segment (the host never sees
// the device counts): few rows -> 16-row tiles (decode kernel); many -> the
// 128-row LDS-DMA kernel for INT4, 64-row tiles otherwise (and for INT4
// segments of under ~96 rows, where 128-row tiles would be mostly padding),
// with 8 wavefront columns (activations re-read half as often) when the
// activations outweigh the weights, else 4.  Nested MWQ -> from about 24 rows
// per width sub-segment the LDS-DMA kernel on row tiles of one width each
// (measured on the Mixtral-shaped layer at 512 tokens, ~43 rows per
// sub-segment: 447 us for gate/up against 595 us for 16-row chunks of all
// widths per workgroup, whose per-row-tile width masks cost 4 VALU operations
// per MFMA); fewer rows -> 16-row tiles that take all widths of an expert
// together (one read of each bit plane).  Any other MOE_KERNEL_* value is
// taken as given.
int pick_path(const QWeights& w, int M_total, int nseg, int epi, int kernel) {
  const int fmt = w.fmt;
  switch (kernel) {
    case 1: return 0;
    case 2: return 1;
    case 3: return 64;
    case 4: return 65;
    case 5: return 128;
    case 6: return fmt == 3 ? 3 : 2;
    case 7: return 5;
    default: break;
  }
  if (fmt == 4) return 0;  // a width per expert: 16-row tiles at every batch size
  const double avg = (double)M_total / (double)(nseg > 0 ? nseg : 1);
  if (fmt == 3) return (avg >= 96.0 && w.base && epi != 1) ? 3 : 0;
  if (avg < 24.0) return 0;
  if (fmt == 2) return 5;
  if (fmt == 1 && avg >= 96.0) return 2;
  const int E = fmt == 2 ? nseg / 3 : nseg;
  const double a_bytes = (double)M_total * w.K * 2.0;
  const double w_bytes = (double)E * w.N * w.K * (fmt == 1 ? 0.5 : 0.25);
  return a_bytes < w_bytes ? 65 : 64;
}

bool qgemm_kernel_supported(int fmt, int kernel) {
  switch (kernel) {
    case 0: case 1: return true;
    case 2: return fmt == 2;
    case 3: case 4: case 5: return fmt == 1 || fmt == 2;
    case 6: return fmt == 1 || fmt == 2 || fmt == 3;
    case 7: return fmt == 2;
    default: return false;
  }
}

namespace {
size_t ws_need(const QWeights& w, int path, int epi, int A_rows, int M_total) {
  if (path == 2 || path == 5) return ((size_t)A_rows * (w.K / w.G) * 4 + 255) & ~(size_t)255;  // row sums per group
  if (path == 3) return ((size_t)A_rows * 4 + 255) & ~(size_t)255;                 // row sums over all of K
  if (w.fmt != 3 && epi != 1 && (path == 0 || path == 1)) {
    // split-K partial sums of the plain epilogues (the SwiGLU one never splits)
    const int n_ks = decode_splits(((w.N + 127) / 128) * decode_row_tiles(w.fmt, path, M_total, w.E), w.K);
    if (n_ks > 1) return ((size_t)n_ks * M_total * w.N * 4 + 255) & ~(size_t)255;
  }
  return 0;
}
}  // namespace

size_t qgemm_workspace_bytes(const QWeights& w, int A_rows, int M_total, int kernel) {
  const int nseg = w.E * (w.fmt == 2 ? 3 : 1);
  size_t need = 0;
  for (int epi = 0; epi < 4; ++epi) {
    const size_t n = ws_need(w, pick_path(w, M_total, nseg, epi, kernel), epi, A_rows, M_total);
    need = n > need ? n : need;
  }
  return need;
}

}  // namespace moe

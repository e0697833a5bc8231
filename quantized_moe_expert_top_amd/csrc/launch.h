// Interface between the host layer (abi.cpp: argument validation, status
// codes, error details) and the device side (the .hip sources: kernels and
// the launches that issue them).  Plain C++ types only: the host layer
// builds without the HIP headers, so it can also be linked against stand-in
// launchers in a CPU-only test build.
//
// Every launch returns the HIP status of what it issued (0 = success) and
// never synchronises with the device.  Streams travel as void* (hipStream_t).
#pragma once
#include <stddef.h>
#include <stdint.h>

namespace moe {

// --------------------------------------------------------- device runtime
// 0 on success, else a HIP error code.
int rt_current_device(int* dev);
// Architecture name of device `dev` (e.g. "gfx950:sramecc+:xnack-") into name[n].
int rt_device_arch(int dev, char* name, size_t n);
// Returns and clears the calling thread's last HIP error (0 if none).
int rt_take_error();
const char* rt_error_string(int err);
// rows pieces of width bytes, pitch bytes apart in both buffers, host (pinned) to device, on stream
int rt_copy_rows_h2d(void* dst, const void* src, size_t rows, size_t pitch, size_t width, void* stream);

// ---------------------------------------------------------------- routing
int launch_route_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w, void* stream);

// --------------------------------------------------------------- grouping
constexpr int kPermuteChunk = 2048;     // pairs per workgroup in the multi-workgroup grouping
constexpr int kPermuteSmallMax = 4096;  // up to this many pairs: one workgroup
constexpr int kRoutePermuteMaxE = 64;   // fused routing + grouping: at most this many experts
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
int launch_permute(const PermuteArgs& a, void* stream);
// Routing + grouping in one launch (E <= 64 experts, T*k <= 4096 pairs).
bool route_permute_fusable(int T, int k, int E);
int launch_route_permute(const float* logits, int T, int E, int k, const uint8_t* bits, int32_t* ids, float* w,
                         int32_t* counts, int32_t* seg_offsets, int32_t* sorted_pair, int32_t* pair_pos, void* ws,
                         void* stream);

// ---------------------------------------------------------------- combine
// y_dtype: MOE_DTYPE_BF16, MOE_DTYPE_F32 or MOE_DTYPE_F16 (validated by the caller)
int launch_combine(const void* y, int y_dtype, const int32_t* pos, const int32_t* n_valid, const float* w, int T,
                   int k, int H, uint16_t* out, void* stream);

// ---------------------------------------------------------- grouped GEMM
// Weight descriptor as the kernels see it (tiled layout only).
struct QWeights {
  int fmt;  // 1 INT4, 2 MWQ, 3 DELTA2, 4 per-expert widths
  int E, N, K, G, z, n_sal;
  const int32_t* xbits;  // per-expert widths / zero points (host arrays, format 4)
  const int32_t* xzero;
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
  int A_rows;
  const int32_t* gather;
  int k;
  const int32_t* seg_offsets;
  int nseg;
  int M_total;
  int epilogue;  // 0 bf16, 1 SwiGLU bf16, 2 fp32
  int kernel;    // MOE_KERNEL_* (0 = chosen from the shapes)
  void* out;
  void* ws;
};
// Whether `kernel` (MOE_KERNEL_*) can run format `fmt`.
bool qgemm_kernel_supported(int fmt, int kernel);
// Workspace bytes for either epilogue (the larger need) with that kernel choice.
size_t qgemm_workspace_bytes(const QWeights& w, int A_rows, int M_total, int kernel);
int launch_qgemm(const QGemmArgs& a, void* stream);
// The no-allocation grouped GEMM's device scratch: its size, and its address
// on the current device (looked up once per device).
constexpr size_t kStaticScratchBytes = (size_t)8 << 20;
int qgemm_static_scratch(void** ptr);
// Planning (plan.cpp).  path: 0 = 16-row tiles (DELTA2: 32-row tiles), 1 = 16-row
// tiles of one width (MWQ), 64 / 65 = 64-row tiles with 8 / 4 wavefront
// columns, 128 = 128-row register-fed tiles, 2 = 128-row LDS-DMA (INT4, MWQ),
// 3 = 128-row LDS-DMA delta kernel.
int pick_path(const QWeights& w, int M_total, int nseg, int epi, int kernel);
int decode_splits(int n_items, int K);
int decode_row_tiles(int fmt, int path, int M_total, int E);

// ----------------------------------------------------------------- repack
constexpr int kMaxMixedExperts = 256;
int launch_repack(const QWeights& src, const QWeights& dst, void* stream);
size_t tiled_salient_bytes(int E, int N, int n_sal);

}  // namespace moe

// C ABI entry points: host-side validation, then stream-ordered launches.
// Every check happens before anything is launched; a failing call launches
// nothing and leaves a one-sentence reason in a thread-local buffer.
//
// Plain C++ (no HIP headers): the device side is reached only through the
// launchers and runtime queries of launch.h.  Before a launch, any error an
// earlier HIP call of the caller left pending is taken and dropped, so that
// MOE_ERR_HIP reports what this call's own launches returned.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "moe_qexpert.h"
#include "launch.h"

namespace {
thread_local char g_detail[512] = "";

moe_status fail(moe_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_detail, sizeof(g_detail), fmt, ap);
  va_end(ap);
  return s;
}
moe_status ok() {
  g_detail[0] = '\0';
  return MOE_OK;
}
moe_status hip_status(int e, const char* what) {
  if (e == 0) return ok();
  return fail(MOE_ERR_HIP, "%s: %s", what, moe::rt_error_string(e));
}
// Drops an error left pending by an earlier HIP call of the caller.
void clear_pending() { (void)moe::rt_take_error(); }
bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Validates a weight descriptor; `tiled` selects which layout is expected.
moe_status check_desc(const moe_wdesc* w, int layout, bool need_buffers) {
  if (!w) return fail(MOE_ERR_NULL_ARG, "weight descriptor is NULL");
  if (w->abi_version != MOE_ABI_VERSION)
    return fail(MOE_ERR_BAD_FORMAT, "descriptor abi_version %d, library %d", w->abi_version, MOE_ABI_VERSION);
  if (w->format < MOE_W_INT4_GROUP || w->format > MOE_W_INT_PER_EXPERT)
    return fail(MOE_ERR_BAD_FORMAT, "unknown weight format %d", w->format);
  if (w->layout != layout)
    return fail(MOE_ERR_BAD_FORMAT, "layout %d where %d is required%s", w->layout, layout,
                layout == MOE_LAYOUT_TILED ? " (run moe_repack_weights first)" : "");
  if (w->E < 1 || w->E > 1024 || w->N < 1 || w->K < 1)
    return fail(MOE_ERR_BAD_SHAPE, "E=%d N=%d K=%d out of range", w->E, w->N, w->K);
  if (w->N % 32 != 0 || w->K % 128 != 0)
    return fail(MOE_ERR_UNSUPPORTED, "N=%d must be a multiple of 32 and K=%d of 128", w->N, w->K);
  if ((int64_t)w->E * w->N * (int64_t)w->K / 2 > ((int64_t)1 << 40))
    return fail(MOE_ERR_BAD_SHAPE, "weights too large");
  if (w->format == MOE_W_DELTA2_SALIENT) {
    if (w->zero_point < 0 || w->zero_point > 3) return fail(MOE_ERR_BAD_SHAPE, "DELTA2 zero_point %d", w->zero_point);
    if (w->n_salient < 0 || w->n_salient > 64 || w->n_salient > w->K)
      return fail(MOE_ERR_UNSUPPORTED, "n_salient=%d (0..64 supported)", w->n_salient);
  } else {
    const int G = w->group_size;
    if (!(G == 32 || G == 64 || G == 128))
      return fail(MOE_ERR_UNSUPPORTED, "group_size %d (32, 64 or 128 supported)", G);
    if (w->format != MOE_W_INT_PER_EXPERT && (w->zero_point < 0 || w->zero_point > 15))
      return fail(MOE_ERR_BAD_SHAPE, "zero_point %d", w->zero_point);
  }
  if (w->format == MOE_W_INT_PER_EXPERT) {  // the tables are needed for sizes as well
    if (w->E > moe::kMaxMixedExperts)
      return fail(MOE_ERR_UNSUPPORTED, "E=%d with per-expert widths (at most %d)", w->E, moe::kMaxMixedExperts);
    if (!w->expert_bits || !w->expert_zero) return fail(MOE_ERR_NULL_ARG, "expert_bits / expert_zero is NULL");
    for (int e = 0; e < w->E; ++e) {
      const int b = w->expert_bits[e], z = w->expert_zero[e];
      if (!(b == 2 || b == 3 || b == 4 || b == 8))
        return fail(MOE_ERR_UNSUPPORTED, "expert %d: %d bits (2, 3, 4 or 8 supported)", e, b);
      if (z < 0 || z >= (1 << b)) return fail(MOE_ERR_BAD_SHAPE, "expert %d: zero point %d for %d bits", e, z, b);
    }
  }
  if (!need_buffers) return MOE_OK;
  if (!w->codes || !w->scales) return fail(MOE_ERR_NULL_ARG, "codes or scales is NULL");
  if (!aligned(w->codes, 16)) return fail(MOE_ERR_MISALIGNED, "codes must be 16-byte aligned");
  if (!aligned(w->scales, 2)) return fail(MOE_ERR_MISALIGNED, "scales must be 2-byte aligned");
  if (w->format == MOE_W_MWQ_2_3_4 && layout == MOE_LAYOUT_CANONICAL) {  // tiled: all planes in codes
    if (!w->plane3 || !w->plane4) return fail(MOE_ERR_NULL_ARG, "MWQ needs plane3 and plane4");
    if (!aligned(w->plane3, 16) || !aligned(w->plane4, 16))
      return fail(MOE_ERR_MISALIGNED, "planes must be 16-byte aligned");
  }
  if (w->format == MOE_W_DELTA2_SALIENT && w->n_salient > 0) {
    if (!w->salient_idx || !w->salient_val) return fail(MOE_ERR_NULL_ARG, "salient_idx / salient_val is NULL");
    if (!aligned(w->salient_val, 16) || !aligned(w->salient_idx, 4))
      return fail(MOE_ERR_MISALIGNED, "salient buffers misaligned");
  }
  if (w->format == MOE_W_DELTA2_SALIENT && w->base && !aligned(w->base, 16))
    return fail(MOE_ERR_MISALIGNED, "base must be 16-byte aligned");
  return MOE_OK;
}

moe::QWeights to_q(const moe_wdesc* w) {
  moe::QWeights q;
  q.fmt = w->format;
  q.E = w->E;
  q.N = w->N;
  q.K = w->K;
  q.G = w->format == MOE_W_DELTA2_SALIENT ? w->K : w->group_size;
  q.z = w->zero_point;
  q.n_sal = w->format == MOE_W_DELTA2_SALIENT ? w->n_salient : 0;
  q.xbits = w->format == MOE_W_INT_PER_EXPERT ? w->expert_bits : nullptr;
  q.xzero = w->format == MOE_W_INT_PER_EXPERT ? w->expert_zero : nullptr;
  q.codes = w->codes;
  q.p3 = w->plane3;
  q.p4 = w->plane4;
  q.scales = w->scales;
  q.sal_idx = w->salient_idx;
  q.sal_val = w->salient_val;
  q.base = w->base;
  return q;
}

// gfx950 check, once per device and thread, on the first launching call;
// then any error left pending by the caller's earlier HIP calls is dropped.
moe_status check_device() {
  int dev = 0;
  int e = moe::rt_current_device(&dev);
  if (e != 0) return fail(MOE_ERR_HIP, "current device: %s", moe::rt_error_string(e));
  static thread_local int checked_dev = -1;
  if (checked_dev != dev) {
    char arch[64] = "";
    e = moe::rt_device_arch(dev, arch, sizeof(arch));
    if (e != 0) return fail(MOE_ERR_HIP, "device properties: %s", moe::rt_error_string(e));
    if (strncmp(arch, "gfx950", 6) != 0)
      return fail(MOE_ERR_UNSUPPORTED, "device arch %s; this library is built for gfx950", arch);
    checked_dev = dev;
  }
  clear_pending();
  return MOE_OK;
}
}  // namespace

extern "C" {

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL_ARG: return "null argument";
    case MOE_ERR_BAD_SHAPE: return "bad shape";
    case MOE_ERR_BAD_FORMAT: return "bad format";
    case MOE_ERR_MISALIGNED: return "misaligned pointer";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MOE_ERR_UNSUPPORTED: return "unsupported";
    case MOE_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* moe_last_error_detail(void) { return g_detail; }

int32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

moe_status moe_route_topk(const float* logits, int32_t T, int32_t E, int32_t k, int32_t* topk_ids, float* topk_w,
                          void* stream) {
  if (T < 0) return fail(MOE_ERR_BAD_SHAPE, "T=%d < 0", T);
  if (E < 1 || E > 1024) return fail(MOE_ERR_BAD_SHAPE, "E=%d outside 1..1024", E);
  if (k < 1 || k > E) return fail(MOE_ERR_BAD_SHAPE, "k=%d outside 1..E (E=%d)", k, E);
  if ((int64_t)T * k >= ((int64_t)1 << 31)) return fail(MOE_ERR_BAD_SHAPE, "T*k too large");
  if (T == 0) return ok();
  if (!logits || !topk_ids || !topk_w) return fail(MOE_ERR_NULL_ARG, "logits, topk_ids and topk_w are required");
  if (!aligned(logits, 4) || !aligned(topk_ids, 4) || !aligned(topk_w, 4))
    return fail(MOE_ERR_MISALIGNED, "route buffers must be 4-byte aligned");
  moe_status st = check_device();
  if (st != MOE_OK) return st;
  return hip_status(moe::launch_route_topk(logits, T, E, k, topk_ids, topk_w, stream),
                    "route_topk launch");
}

size_t moe_permute_workspace_size(int32_t T, int32_t k, int32_t E, int32_t S) {
  if (T < 0 || k < 1 || E < 1 || E > 1024 || !(S == 1 || S == 3)) return 0;
  if ((int64_t)T * k >= ((int64_t)1 << 31)) return 0;
  return moe::permute_workspace_bytes(T * k, E, S);
}

moe_status moe_permute(const int32_t* topk_ids, const uint8_t* pair_bits, int32_t T, int32_t k, int32_t E,
                       int32_t* expert_counts, int32_t* seg_offsets, int32_t* sorted_pair, int32_t* pair_pos,
                       const uint16_t* x, int32_t H, uint16_t* x_perm, void* workspace, size_t workspace_bytes,
                       void* stream) {
  if (T < 0) return fail(MOE_ERR_BAD_SHAPE, "T=%d < 0", T);
  if (E < 1 || E > 1024) return fail(MOE_ERR_BAD_SHAPE, "E=%d outside 1..1024", E);
  if (k < 1 || k > E) return fail(MOE_ERR_BAD_SHAPE, "k=%d outside 1..E (E=%d)", k, E);
  if ((int64_t)T * k >= ((int64_t)1 << 31)) return fail(MOE_ERR_BAD_SHAPE, "T*k too large");
  const int S = pair_bits ? 3 : 1;
  if (!expert_counts || !seg_offsets || !workspace) return fail(MOE_ERR_NULL_ARG, "counts, offsets and workspace are required");
  if (T > 0 && (!topk_ids || !sorted_pair || !pair_pos)) return fail(MOE_ERR_NULL_ARG, "ids, sorted_pair and pair_pos are required");
  const size_t need = moe::permute_workspace_bytes(T * k, E, S);
  if (workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes, %zu needed", workspace_bytes, need);
  if (!aligned(workspace, 16)) return fail(MOE_ERR_MISALIGNED, "workspace must be 16-byte aligned");
  if (x_perm) {
    if (!x) return fail(MOE_ERR_NULL_ARG, "x_perm requested without x");
    if (H < 8 || H % 8 != 0) return fail(MOE_ERR_BAD_SHAPE, "H=%d must be a positive multiple of 8", H);
    if (!aligned(x, 16) || !aligned(x_perm, 16)) return fail(MOE_ERR_MISALIGNED, "x / x_perm must be 16-byte aligned");
  }
  moe_status st = check_device();
  if (st != MOE_OK) return st;
  moe::PermuteArgs a{topk_ids, pair_bits, T * k, k, E, S, expert_counts, seg_offsets, sorted_pair, pair_pos,
                     x, H, x_perm, workspace};
  return hip_status(moe::launch_permute(a, stream), "permute launch");
}

moe_status moe_route_permute(const float* logits, int32_t T, int32_t E, int32_t k, const uint8_t* pair_bits,
                             int32_t* topk_ids, float* topk_w, int32_t* expert_counts, int32_t* seg_offsets,
                             int32_t* sorted_pair, int32_t* pair_pos, void* workspace, size_t workspace_bytes,
                             void* stream) {
  if (T < 0) return fail(MOE_ERR_BAD_SHAPE, "T=%d < 0", T);
  if (E < 1 || E > 1024) return fail(MOE_ERR_BAD_SHAPE, "E=%d outside 1..1024", E);
  if (k < 1 || k > E) return fail(MOE_ERR_BAD_SHAPE, "k=%d outside 1..E (E=%d)", k, E);
  if ((int64_t)T * k >= ((int64_t)1 << 31)) return fail(MOE_ERR_BAD_SHAPE, "T*k too large");
  const int S = pair_bits ? 3 : 1;
  if (!expert_counts || !seg_offsets || !workspace) return fail(MOE_ERR_NULL_ARG, "counts, offsets and workspace are required");
  if (T > 0 && (!logits || !topk_ids || !topk_w || !sorted_pair || !pair_pos))
    return fail(MOE_ERR_NULL_ARG, "logits, ids, gates, sorted_pair and pair_pos are required");
  const size_t need = moe::permute_workspace_bytes(T * k, E, S);
  if (workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes, %zu needed", workspace_bytes, need);
  if (!aligned(workspace, 16)) return fail(MOE_ERR_MISALIGNED, "workspace must be 16-byte aligned");
  if (T > 0 && (!aligned(logits, 4) || !aligned(topk_ids, 4) || !aligned(topk_w, 4)))
    return fail(MOE_ERR_MISALIGNED, "route buffers must be 4-byte aligned");
  moe_status st = check_device();
  if (st != MOE_OK) return st;
  void* const s = stream;
  if (T > 0 && moe::route_permute_fusable(T, k, E))
    return hip_status(moe::launch_route_permute(logits, T, E, k, pair_bits, topk_ids, topk_w, expert_counts,
                                                seg_offsets, sorted_pair, pair_pos, workspace, s),
                      "route_permute launch");
  if (T > 0) {
    st = hip_status(moe::launch_route_topk(logits, T, E, k, topk_ids, topk_w, s), "route_topk launch");
    if (st != MOE_OK) return st;
  }
  moe::PermuteArgs a{topk_ids, pair_bits, T * k, k, E, S, expert_counts, seg_offsets, sorted_pair, pair_pos,
                     nullptr, 0, nullptr, workspace};
  return hip_status(moe::launch_permute(a, s), "permute launch");
}

size_t moe_weight_field_bytes(const moe_wdesc* w, int32_t field) {
  if (check_desc(w, w ? w->layout : 0, false) != MOE_OK) return 0;
  const size_t ENK = (size_t)w->E * w->N * w->K;
  const bool tiled = w->layout == MOE_LAYOUT_TILED;
  switch (field) {
    case MOE_FIELD_CODES:  // tiled MWQ: the three planes of a tile block side by side
      if (w->format == MOE_W_INT_PER_EXPERT) {
        size_t n = 0;
        for (int e = 0; e < w->E; ++e) n += (size_t)w->N * w->K * w->expert_bits[e] / 8;
        return n;
      }
      return (w->format == MOE_W_INT4_GROUP || (tiled && w->format == MOE_W_MWQ_2_3_4)) ? ENK / 2 : ENK / 4;
    case MOE_FIELD_PLANE3:
    case MOE_FIELD_PLANE4:
      return (w->format == MOE_W_MWQ_2_3_4 && !tiled) ? ENK / 8 : 0;
    case MOE_FIELD_SCALES:
      return w->format == MOE_W_DELTA2_SALIENT ? (size_t)w->E * w->N * 2
                                               : (size_t)w->E * w->N * (w->K / w->group_size) * 2;
    case MOE_FIELD_SALIENT_IDX:
      return w->format == MOE_W_DELTA2_SALIENT ? (size_t)w->E * w->n_salient * 4 : 0;
    case MOE_FIELD_SALIENT_VAL:
      if (w->format != MOE_W_DELTA2_SALIENT) return 0;
      return tiled ? moe::tiled_salient_bytes(w->E, w->N, w->n_salient) : (size_t)w->E * w->n_salient * w->N * 2;
    case MOE_FIELD_BASE:
      return w->format == MOE_W_DELTA2_SALIENT ? (size_t)w->N * w->K * 2 : 0;
    default:
      return 0;
  }
}

moe_status moe_repack_weights(const moe_wdesc* src, const moe_wdesc* dst, void* stream) {
  moe_status st = check_desc(src, MOE_LAYOUT_CANONICAL, true);
  if (st != MOE_OK) return st;
  st = check_desc(dst, MOE_LAYOUT_TILED, true);
  if (st != MOE_OK) return st;
  if (src->format != dst->format || src->E != dst->E || src->N != dst->N || src->K != dst->K ||
      src->group_size != dst->group_size || src->zero_point != dst->zero_point || src->n_salient != dst->n_salient)
    return fail(MOE_ERR_BAD_SHAPE, "source and destination descriptors disagree");
  if (src->format == MOE_W_INT_PER_EXPERT)
    for (int e = 0; e < src->E; ++e)
      if (src->expert_bits[e] != dst->expert_bits[e] || src->expert_zero[e] != dst->expert_zero[e])
        return fail(MOE_ERR_BAD_SHAPE, "expert %d: source and destination widths or zero points disagree", e);
  if (src->format == MOE_W_DELTA2_SALIENT && ((src->base == nullptr) != (dst->base == nullptr)))
    return fail(MOE_ERR_NULL_ARG, "base given on one side only");
  if (src->codes == dst->codes) return fail(MOE_ERR_BAD_SHAPE, "repack cannot run in place");
  st = check_device();
  if (st != MOE_OK) return st;
  return hip_status(moe::launch_repack(to_q(src), to_q(dst), stream), "repack launch");
}

moe_status moe_copy_rows_async(void* dst, const void* src, size_t rows, size_t pitch, size_t width, void* stream) {
  if (rows == 0 || width == 0) return ok();
  if (!dst || !src) return fail(MOE_ERR_NULL_ARG, "dst and src are required");
  if (width > pitch) return fail(MOE_ERR_BAD_SHAPE, "width %zu > pitch %zu", width, pitch);
  return hip_status(moe::rt_copy_rows_h2d(dst, src, rows, pitch, width, stream), "copy_rows");
}

size_t moe_grouped_qgemm_workspace_size(const moe_wdesc* w, int32_t A_rows, int32_t M_total, int32_t kernel) {
  if (check_desc(w, MOE_LAYOUT_TILED, false) != MOE_OK) return 0;
  if (A_rows < 0 || M_total < 0 || !moe::qgemm_kernel_supported(w->format, kernel)) return 0;
  return moe::qgemm_workspace_bytes(to_q(w), A_rows, M_total, kernel);
}

}  // extern "C"

namespace {
// Everything moe_grouped_qgemm checks before its workspace.  Sets *empty for
// a problem with no rows (a success with nothing to launch).
moe_status check_qgemm(const moe_wdesc* w, const uint16_t* A, int32_t A_rows, const int32_t* gather_pair, int32_t k,
                       const int32_t* seg_offsets, int32_t M_total, int32_t epilogue, int32_t kernel, void* out,
                       bool* empty) {
  *empty = false;
  moe_status st = check_desc(w, MOE_LAYOUT_TILED, true);
  if (st != MOE_OK) return st;
  if (M_total < 0 || A_rows < 0) return fail(MOE_ERR_BAD_SHAPE, "M_total=%d A_rows=%d", M_total, A_rows);
  if (epilogue != MOE_EPI_NONE && epilogue != MOE_EPI_SWIGLU && epilogue != MOE_EPI_NONE_F32 &&
      epilogue != MOE_EPI_NONE_F16)
    return fail(MOE_ERR_BAD_FORMAT, "unknown epilogue %d", epilogue);
  if (kernel < MOE_KERNEL_AUTO || kernel > MOE_KERNEL_LDS_DMA_PER_WIDTH)
    return fail(MOE_ERR_BAD_FORMAT, "unknown kernel choice %d", kernel);
  if (!moe::qgemm_kernel_supported(w->format, kernel))
    return fail(MOE_ERR_UNSUPPORTED, "kernel choice %d does not run weight format %d", kernel, w->format);
  if (w->format == MOE_W_DELTA2_SALIENT && kernel == MOE_KERNEL_LDS_DMA && (!w->base || epilogue == MOE_EPI_SWIGLU))
    return fail(MOE_ERR_UNSUPPORTED, "the LDS-DMA delta kernel needs a shared base and a plain epilogue");
  if (gather_pair) {
    if (k < 1) return fail(MOE_ERR_BAD_SHAPE, "k=%d with gather_pair", k);
    if ((int64_t)A_rows * k < M_total) return fail(MOE_ERR_BAD_SHAPE, "A_rows*k < M_total");
  } else if (A_rows < M_total) {
    return fail(MOE_ERR_BAD_SHAPE, "A_rows=%d < M_total=%d", A_rows, M_total);
  }
  if (M_total == 0) {
    *empty = true;
    return ok();
  }
  if (!A || !seg_offsets || !out) return fail(MOE_ERR_NULL_ARG, "A, seg_offsets and out are required");
  if (!aligned(A, 16) || !aligned(out, 16)) return fail(MOE_ERR_MISALIGNED, "A and out must be 16-byte aligned");
  if ((int64_t)A_rows * w->K * 2 >= ((int64_t)1 << 32))
    return fail(MOE_ERR_UNSUPPORTED, "activation matrix of %lld bytes (4 GiB or more)", (long long)A_rows * w->K * 2);
  return MOE_OK;
}

moe_status run_qgemm(const moe_wdesc* w, const uint16_t* A, int32_t A_rows, const int32_t* gather_pair, int32_t k,
                     const int32_t* seg_offsets, int32_t M_total, int32_t epilogue, int32_t kernel, void* out,
                     void* workspace, void* stream) {
  moe::QGemmArgs a{to_q(w), A, A_rows, gather_pair, k, seg_offsets, w->E * (w->format == MOE_W_MWQ_2_3_4 ? 3 : 1),
                   M_total, epilogue, kernel, out, workspace};
  return hip_status(moe::launch_qgemm(a, stream), "grouped_qgemm launch");
}
}  // namespace

extern "C" {

moe_status moe_grouped_qgemm(const moe_wdesc* w, const uint16_t* A, int32_t A_rows, const int32_t* gather_pair,
                             int32_t k, const int32_t* seg_offsets, int32_t M_total, int32_t epilogue,
                             int32_t kernel, void* out, void* workspace, size_t workspace_bytes, void* stream) {
  bool empty = false;
  moe_status st = check_qgemm(w, A, A_rows, gather_pair, k, seg_offsets, M_total, epilogue, kernel, out, &empty);
  if (st != MOE_OK || empty) return st;
  const size_t need = moe::qgemm_workspace_bytes(to_q(w), A_rows, M_total, kernel);
  if (workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes, %zu needed", workspace_bytes, need);
  if (need && !workspace) return fail(MOE_ERR_NULL_ARG, "workspace is NULL");
  if (need && !aligned(workspace, 16)) return fail(MOE_ERR_MISALIGNED, "workspace must be 16-byte aligned");
  st = check_device();
  if (st != MOE_OK) return st;
  return run_qgemm(w, A, A_rows, gather_pair, k, seg_offsets, M_total, epilogue, kernel, out, workspace, stream);
}

moe_status moe_grouped_qgemm_noalloc(const moe_wdesc* w, const uint16_t* A, int32_t A_rows,
                                     const int32_t* gather_pair, int32_t k, const int32_t* seg_offsets,
                                     int32_t M_total, int32_t epilogue, int32_t kernel, void* out, void* stream) {
  bool empty = false;
  moe_status st = check_qgemm(w, A, A_rows, gather_pair, k, seg_offsets, M_total, epilogue, kernel, out, &empty);
  if (st != MOE_OK || empty) return st;
  const size_t need = moe::qgemm_workspace_bytes(to_q(w), A_rows, M_total, kernel);
  if (need > moe::kStaticScratchBytes)
    return fail(MOE_ERR_UNSUPPORTED, "this call needs %zu bytes of scratch; the static scratch holds %zu "
                "(use moe_grouped_qgemm with a workspace)", need, moe::kStaticScratchBytes);
  st = check_device();
  if (st != MOE_OK) return st;
  void* scratch = nullptr;
  if (need) {
    const int e = moe::qgemm_static_scratch(&scratch);
    if (e != 0) return fail(MOE_ERR_HIP, "static scratch address: %s", moe::rt_error_string(e));
  }
  return run_qgemm(w, A, A_rows, gather_pair, k, seg_offsets, M_total, epilogue, kernel, out, scratch, stream);
}

size_t moe_grouped_qgemm_noalloc_scratch_bytes(void) { return moe::kStaticScratchBytes; }

moe_status moe_unpermute_combine(const void* y_perm, int32_t y_dtype, const int32_t* pair_pos,
                                 const int32_t* n_valid, const float* topk_w, int32_t T, int32_t k, int32_t H,
                                 uint16_t* out, void* stream) {
  if (y_dtype != MOE_DTYPE_BF16 && y_dtype != MOE_DTYPE_F32 && y_dtype != MOE_DTYPE_F16)
    return fail(MOE_ERR_BAD_FORMAT, "y_dtype %d", y_dtype);
  if (T < 0 || k < 1 || H < 8 || H % 8 != 0)
    return fail(MOE_ERR_BAD_SHAPE, "T=%d k=%d H=%d (H must be a positive multiple of 8)", T, k, H);
  if ((int64_t)T * k >= ((int64_t)1 << 31)) return fail(MOE_ERR_BAD_SHAPE, "T*k too large");
  if (T == 0) return ok();
  if (!y_perm || !pair_pos || !out) return fail(MOE_ERR_NULL_ARG, "y_perm, pair_pos and out are required");
  if (!aligned(y_perm, 16) || !aligned(out, 16)) return fail(MOE_ERR_MISALIGNED, "y_perm and out must be 16-byte aligned");
  if (n_valid && !aligned(n_valid, 4)) return fail(MOE_ERR_MISALIGNED, "n_valid must be 4-byte aligned");
  moe_status st = check_device();
  if (st != MOE_OK) return st;
  return hip_status(moe::launch_combine(y_perm, y_dtype, pair_pos, n_valid, topk_w, T, k, H, out,
                                        stream),
                    "combine launch");
}

}  // extern "C"

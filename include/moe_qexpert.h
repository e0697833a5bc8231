/*
 * moe_qexpert.h -- C ABI of the routed-expert quantized MoE library (MI355X / gfx950).
 *
 * One MoE layer runs as four stream-ordered calls:
 *
 *   moe_route_topk         logits -> top-k expert ids + gate weights
 *   moe_permute            (token, slot) pairs -> grouped per expert (and bit-width)
 *   moe_grouped_qgemm      grouped low-bit GEMM over the expert segments
 *                          (gate_up with a SwiGLU epilogue, then down; or the
 *                          delta linear layer with its shared base)
 *   moe_unpermute_combine  gate-weighted sum of each token's k expert outputs
 *
 * What is computed follows these pages:
 *   - "Every Expert Counts: ExactMoE for Memory-Efficient W4A16 Inference":
 *     only the routed experts are 4-bit (W4A16); the router's decisions are
 *     unchanged and every selected expert runs; experts run as grouped batches
 *     rather than one after another.
 *   - "D2MoE: Dual Routing and Dynamic Scheduling for Efficient On-Device
 *     MoE-based LLM Serving", Design: the Dual Routing equations (an expert
 *     gate and a per-pair bit-width), the MWQ equations W(2)=Q2, W(3)=Q2+D3,
 *     W(4)=Q2+D3+D4 (INT2 c INT3 c INT4), and the pipeline equation
 *     (dequantise to 16 bit, then GEMM).
 *   - "ME-Switch: A Memory-Efficient Expert Switching Framework for Large
 *     Language Models": expert weight = shared base + delta; the delta uses one
 *     quantisation step per output channel, salient input channels stay
 *     unquantised.
 *   - Read-ME summary ("Innovativer Ansatz zur Optimierung der Inferenz von
 *     Mixture-of-Experts-Modellen"): requests that need the same expert are
 *     batched together (the grouping step).
 *
 * Conventions (no page fixes them): top-k in descending logit order with ties
 * to the lower expert index; gate weights = softmax over the k selected
 * logits; SwiGLU experts h = bf16(silu(x Wg^T) * (x Wu^T)), y = h Wd^T (h is the
 * 16-bit activation entering the down GEMM).
 *
 * General rules for every call:
 *   - Buffer pointers are DEVICE pointers (hipMalloc / torch CUDA tensors)
 *     unless stated otherwise.  bf16 and fp16 values travel as uint16_t bit
 *     patterns.  The caller owns every buffer; the library allocates nothing
 *     and keeps no pointer after a call returns.  Buffers must stay valid
 *     until the stream has executed the call.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream).  Nothing synchronises with the host and nothing is copied back.
 *   - Arguments are validated on the host before anything is launched; on any
 *     error nothing is launched and the status says why
 *     (moe_last_error_detail() adds a sentence, per calling thread).
 *     A launch failure returns MOE_ERR_HIP.  An error that an earlier HIP call
 *     of the caller left pending is cleared before the launch (it is not this
 *     call's error).  Faults inside kernels surface at the caller's next
 *     synchronisation.
 *   - Identical inputs give bitwise identical outputs (no floating-point
 *     atomics; every reduction has a fixed order).
 *   - No exception or process exit crosses this interface.  The only library
 *     state is the thread-local error detail, so calls are thread-safe.
 */
#ifndef MOE_QEXPERT_H
#define MOE_QEXPERT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 3

typedef int32_t moe_status;
#define MOE_OK 0
#define MOE_ERR_NULL_ARG 1            /* a required pointer is NULL */
#define MOE_ERR_BAD_SHAPE 2           /* a size is out of range or inconsistent */
#define MOE_ERR_BAD_FORMAT 3          /* unknown format / layout / descriptor version */
#define MOE_ERR_MISALIGNED 4          /* a pointer breaks its alignment rule */
#define MOE_ERR_WORKSPACE_TOO_SMALL 5 /* workspace_bytes below the *_workspace_size() value */
#define MOE_ERR_UNSUPPORTED 6         /* valid but not implemented (e.g. group size, device arch) */
#define MOE_ERR_HIP 7                 /* a HIP runtime call or launch failed */

/* Static, never NULL. */
const char* moe_status_string(moe_status s);
/* Detail of the last failing call on this thread ("" after a success).
   Valid until the next library call on the same thread. */
const char* moe_last_error_detail(void);
/* Returns MOE_ABI_VERSION of the built library. */
int32_t moe_abi_version(void);

/* ------------------------------------------------------------------ routing
 * Expert gate of the Dual Routing equations (D2MoE page, Design).
 *   logits   f32 [T][E], finite
 *   topk_ids i32 [T][k]  out: slot j = the j-th largest logit (ties -> lower index)
 *   topk_w   f32 [T][k]  out: softmax over the k selected logits, evaluated in
 *                        float64 and rounded once to float32
 * 0 <= T, 1 <= k <= E <= 1024, T*k < 2^31.  4-byte aligned pointers.
 */
moe_status moe_route_topk(const float* logits, int32_t T, int32_t E, int32_t k,
                          int32_t* topk_ids, float* topk_w, void* stream);

/* ----------------------------------------------------------------- grouping
 * Groups the P = T*k (token, slot) pairs, pair p = t*k + j, by expert
 * (expert-aware batching, Read-ME summary; grouped execution, ExactMoE page).
 *
 *   topk_ids      i32 [P] in [0, E)
 *   pair_bits     u8  [P] bit-width of each pair in {2, 3, 4} for nested MWQ
 *                 weights (Bit Gate of the Dual Routing equations), or NULL.
 *                 NULL: S = 1 segment per expert, key = e.
 *                 non-NULL: S = 3 segments per expert, key = 3*e + (4 - b),
 *                 i.e. segments b = 4, 3, 2 in that order.
 *   expert_counts i32 [E]       out: pairs per expert
 *   seg_offsets   i32 [E*S + 1] out: exclusive prefix sum of pairs per key;
 *                               seg_offsets[E*S] = number of valid pairs
 *   sorted_pair   i32 [P]       out: pairs in ascending (key, p) order
 *   pair_pos      i32 [P]       out: inverse of sorted_pair
 *   x, H, x_perm  optional: if x_perm != NULL, x_perm[i] = x[sorted_pair[i] / k]
 *                 (bf16 rows of H values; H % 8 == 0, 16-byte aligned).  The
 *                 GEMM does not need it (it gathers rows itself).
 *   workspace     device scratch of moe_permute_workspace_size(T, k, E, S)
 *                 bytes (16-byte aligned).  Word 0 (u32) reads non-zero after
 *                 the call if some id was outside [0, E) or some bit-width was
 *                 outside {2,3,4}; such pairs are placed after every valid
 *                 segment and are not counted in expert_counts.
 * All index outputs are bit-exact and deterministic.
 */
size_t moe_permute_workspace_size(int32_t T, int32_t k, int32_t E, int32_t S);
moe_status moe_permute(const int32_t* topk_ids, const uint8_t* pair_bits,
                       int32_t T, int32_t k, int32_t E,
                       int32_t* expert_counts, int32_t* seg_offsets,
                       int32_t* sorted_pair, int32_t* pair_pos,
                       const uint16_t* x, int32_t H, uint16_t* x_perm,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Routing and grouping in one call: the same outputs as moe_route_topk
 * followed by moe_permute (without the x gather), bit for bit.  With
 * E <= 64 and T*k <= 4096 it is a single launch: each workgroup routes 4
 * tokens and the last workgroup to finish groups all pairs; otherwise it
 * issues the two separate launches.  Arguments and errors as for those two
 * calls.  workspace: moe_permute_workspace_size(T, k, E, pair_bits ? 3 : 1)
 * bytes, 16-byte aligned, whose second 32-bit word (an arrival counter) must
 * be zero before the first call; every call leaves it zero.  Calls that
 * share one workspace must not overlap on the device.
 */
moe_status moe_route_permute(const float* logits, int32_t T, int32_t E, int32_t k, const uint8_t* pair_bits,
                             int32_t* topk_ids, float* topk_w, int32_t* expert_counts, int32_t* seg_offsets,
                             int32_t* sorted_pair, int32_t* pair_pos, void* workspace, size_t workspace_bytes,
                             void* stream);

/* ----------------------------------------------------------- weight formats
 * MOE_W_INT4_GROUP   W4A16 (ExactMoE page): w[n][k] = s[n][k/G] * (c - z),
 *                    c in [0,15].  codes u8 [E][N][K/2] (canonical: even k in
 *                    the low nibble), scales fp16 [E][N][K/G].
 * MOE_W_MWQ_2_3_4    nested planes (D2MoE page, MWQ equations): q2 = top two
 *                    bits of the 4-bit code, d3 = bit 1, d4 = bit 0;
 *                    c_b = 4*q2 + 2*d3*[b>=3] + d4*[b==4];
 *                    w = s[n][k/G] * (c_b - z).  codes = q2 plane u8
 *                    [E][N][K/4] (canonical: field k&3 at bits 2*(k&3)),
 *                    plane3 = d3, plane4 = d4, u8 [E][N][K/8] (bit k&7);
 *                    scales fp16 [E][N][K/G].
 * MOE_W_INT_PER_EXPERT  static bit-width per expert (EdgeMoE page, expert-wise
 *                    bit-width adaptation): expert e stores b_e-bit codes,
 *                    b_e in {2, 3, 4, 8}, with its own zero point z_e in
 *                    [0, 2^b_e - 1]: w = s[n][k/G] * (c - z_e).  expert_bits
 *                    and expert_zero (host int32 [E], read on every call)
 *                    give b_e and z_e; zero_point is ignored; E <= 256.
 *                    codes u8, experts back to back, expert e's [N][K] codes
 *                    as one little-endian bit stream per row (code k at bits
 *                    k*b_e .. k*b_e + b_e - 1): N*K*b_e/8 bytes per expert;
 *                    scales fp16 [E][N][K/G].  Other widths (1, 5, 6, 7, ...)
 *                    are MOE_ERR_UNSUPPORTED.
 * MOE_W_DELTA2_SALIENT  ME-Switch delta: d[n][k] = salient value if k is a
 *                    salient input channel of expert e, else
 *                    step[n] * (c - z) with c in [0,3] (z = 2 normally).
 *                    codes u8 [E][N][K/4] (packed like q2), scales = step
 *                    fp16 [E][N], salient_idx i32 [E][n_salient] (distinct),
 *                    salient_val bf16 [E][n_salient][N]; optional shared
 *                    base bf16 [N][K] (y = x W_base^T + x D_e^T).
 *
 * Layouts: MOE_LAYOUT_CANONICAL is the storage layout above.  The GEMM reads
 * MOE_LAYOUT_TILED, produced once, offline, by moe_repack_weights: codes,
 * planes, salient_val and base are re-ordered into tiles of 16 output
 * channels x 128 inputs laid out as 64-lane MFMA operand fragments (same byte
 * counts for codes / planes / base); scales, step and salient_idx keep their
 * canonical layout and may be shared between the two descriptors.  Tiled
 * MWQ keeps all three planes in `codes` (ENK/2 bytes: per tile block 512 B of
 * q2, then 256 B of d3, then 256 B of d4, so a block is one contiguous
 * kilobyte); its plane3 / plane4 are unused (NULL).  Tiled per-expert widths
 * hold each code shifted to 4 bits (c << (4 - b_e)) as the same three planes,
 * only the first b_e of them stored: a tile block is 256 * b_e bytes, and each
 * expert keeps its canonical byte count and offset.
 */
#define MOE_W_INT4_GROUP 1
#define MOE_W_MWQ_2_3_4 2
#define MOE_W_DELTA2_SALIENT 3
#define MOE_W_INT_PER_EXPERT 4

#define MOE_LAYOUT_CANONICAL 0
#define MOE_LAYOUT_TILED 1

/* Kernel choice of moe_grouped_qgemm (tuning and tests; AUTO everywhere else).
   Every choice computes the same result; the LDS-DMA and 128-row kernels add
   row sums in a different order, so their bits may differ from the others'. */
#define MOE_KERNEL_AUTO 0            /* chosen from the mean rows per segment */
#define MOE_KERNEL_SMALL 1           /* 16-row tiles (decode batches); nested MWQ: all widths of an
                                        expert in one tile; DELTA2: 32-row tiles */
#define MOE_KERNEL_SMALL_PER_WIDTH 2 /* nested MWQ only: 16-row tiles of one width each */
#define MOE_KERNEL_TILE64_WIDE 3     /* INT4, MWQ: 64-row tiles, 128 SwiGLU / 256 plain channels */
#define MOE_KERNEL_TILE64 4          /* INT4, MWQ: 64-row tiles, 64 SwiGLU / 128 plain channels */
#define MOE_KERNEL_TILE128 5         /* INT4, MWQ: 128-row tiles fed through registers */
#define MOE_KERNEL_LDS_DMA 6         /* INT4, MWQ, DELTA2 with a base and a plain epilogue: 64- or
                                        128-row tiles fed by LDS-DMA (activation row sums in the
                                        workspace); nested MWQ: 16-row chunks of all widths */
#define MOE_KERNEL_LDS_DMA_PER_WIDTH 7 /* nested MWQ only: the LDS-DMA kernel on row tiles of one
                                          width each, loading only that width's planes */

#define MOE_EPI_NONE 0      /* out bf16 [M_total][N] */
#define MOE_EPI_SWIGLU 1    /* N = 2*I; rows [0,I) gate, [I,2I) up; out = bf16(silu(gate) * up), width I */
#define MOE_EPI_NONE_F32 2  /* out fp32 [M_total][N], not rounded (expert outputs feeding the combine) */
#define MOE_EPI_NONE_F16 3  /* out fp16 [M_total][N], rounded to nearest even: expert outputs for the combine
                               as 16-bit values (the FP16 pipeline of the D2MoE page), half the bytes of
                               fp32 with 11 significant bits; magnitudes past 65504 become +-inf */

#define MOE_DTYPE_BF16 0
#define MOE_DTYPE_F32 1
#define MOE_DTYPE_F16 2

typedef struct moe_wdesc {
  int32_t abi_version;   /* MOE_ABI_VERSION */
  int32_t format;        /* MOE_W_* */
  int32_t layout;        /* MOE_LAYOUT_* */
  int32_t E, N, K;       /* experts; output channels; input channels */
  int32_t group_size;    /* G along K (INT4, MWQ); ignored for DELTA2 */
  int32_t zero_point;    /* z: 0..15 (INT4, MWQ), 0..3 (DELTA2) */
  int32_t n_salient;     /* DELTA2: salient channels per expert, 0..64 */
  int32_t reserved;
  const uint8_t* codes;        /* INT4 nibbles | MWQ q2 plane (tiled: all planes) | DELTA2 2-bit codes */
  const uint8_t* plane3;       /* MWQ d3 plane (canonical layout), else NULL */
  const uint8_t* plane4;       /* MWQ d4 plane (canonical layout), else NULL */
  const uint16_t* scales;      /* fp16: [E][N][K/G] (INT4, MWQ) or [E][N] step (DELTA2) */
  const int32_t* salient_idx;  /* DELTA2 [E][n_salient] */
  const uint16_t* salient_val; /* DELTA2 bf16 */
  const uint16_t* base;        /* DELTA2 shared bf16 base [N][K], or NULL */
  const int32_t* expert_bits;  /* INT_PER_EXPERT: host int32 [E], each 2, 3, 4 or 8; else NULL */
  const int32_t* expert_zero;  /* INT_PER_EXPERT: host int32 [E], zero point of each expert; else NULL */
} moe_wdesc;

#define MOE_FIELD_CODES 0
#define MOE_FIELD_PLANE3 1
#define MOE_FIELD_PLANE4 2
#define MOE_FIELD_SCALES 3
#define MOE_FIELD_SALIENT_IDX 4
#define MOE_FIELD_SALIENT_VAL 5
#define MOE_FIELD_BASE 6

/* Bytes of one field of `w` in w->layout (0 if the format has no such field).
   Returns 0 as well for an invalid descriptor. */
size_t moe_weight_field_bytes(const moe_wdesc* w, int32_t field);

/* Offline conversion canonical -> tiled.  `src` (layout CANONICAL) and `dst`
 * (layout TILED) must describe the same format and sizes; dst's codes /
 * plane3 / plane4 / salient_val / base point to caller buffers of
 * moe_weight_field_bytes(dst, field) bytes, which are overwritten.  For
 * DELTA2 the tiled codes of salient channels are set to the zero code, so
 * they contribute only through salient_val.  dst->scales and
 * dst->salient_idx are not written (point them at src's buffers).
 * Requirements: N % 32 == 0, K % 128 == 0, 16-byte aligned buffers.
 */
moe_status moe_repack_weights(const moe_wdesc* src, const moe_wdesc* dst, void* stream);

/* --------------------------------------------------------- expert offload
 * Plane-by-plane loading of host-resident experts (D2MoE page, Design,
 * bit-width-aware I/O-compute pipeline and its HEBF order): in the tiled
 * nested-MWQ layout the planes of an expert are interleaved per 1 KB tile
 * block (q2 at bytes 0..511, d3 at 512..767, d4 at 768..1023), so one plane
 * of one expert is `rows` pieces of `width` bytes, `pitch` bytes apart.
 * Copies those pieces from `src` (pinned host memory) to `dst` (device
 * memory), both laid out with the same pitch (pass pointers already offset
 * to the plane), ordered on `stream` and asynchronous to the host.
 * Errors, before anything is queued: MOE_ERR_NULL_ARG (NULL buffer with
 * rows > 0), MOE_ERR_BAD_SHAPE (width > pitch).  MOE_ERR_HIP if the copy
 * cannot be queued.  rows == 0 or width == 0: nothing to do.
 */
moe_status moe_copy_rows_async(void* dst, const void* src, size_t rows, size_t pitch, size_t width, void* stream);

/* ---------------------------------------------------------- grouped GEMM
 * For every segment s of seg_offsets (E*S segments; S = 3 for MWQ, else 1)
 * and every row i in [seg_offsets[s], seg_offsets[s+1]):
 *     a_i = A[gather_pair[i] / k]  (gather_pair != NULL; A has A_rows = T rows)
 *     a_i = A[i]                   (gather_pair == NULL; A has A_rows >= M_total rows)
 *     y_i = a_i W_e^T  with W_e dequantised from the format, e = s / S
 *           (MWQ: bit-width b = 4 - s % 3 for all of W_e)
 *           (DELTA2: y_i = a_i W_base^T + a_i D_e^T if base != NULL)
 *     out[i] = y_i                       (MOE_EPI_NONE: bf16, MOE_EPI_NONE_F32: fp32,
 *                                         MOE_EPI_NONE_F16: fp16, width N)
 *     out[i] = silu(y_i[:I]) * y_i[I:]   (MOE_EPI_SWIGLU: bf16, width I = N/2)
 * Dequantisation is exact: codes become exact 16-bit values, products are
 * accumulated in fp32 and the group / channel scales are applied in fp32;
 * a 16-bit out is rounded once (pipeline equation of the D2MoE page:
 * dequantise, then a 16-bit GEMM; the SwiGLU output is the 16-bit
 * activation of the next GEMM).
 *
 *   w           tiled descriptor (host pointer; its buffers are device memory)
 *   A           bf16 [A_rows][K], 16-byte aligned, K % 128 == 0
 *   seg_offsets i32 [E*S + 1] from moe_permute (device), or any slice of
 *               E*S + 1 consecutive entries of a longer ascending table (a
 *               subset of segments); only rows in [seg_offsets[0],
 *               seg_offsets[E*S]) are written
 *   M_total     host upper bound of rows (T*k); grid sizing never reads the
 *               device counts back
 *   kernel      MOE_KERNEL_AUTO, or a MOE_KERNEL_* choice; a choice that does
 *               not run the format -> MOE_ERR_UNSUPPORTED
 *   out         bf16 or fp32 (see epilogue) [M_total][N or N/2], 16-byte aligned
 *   workspace   moe_grouped_qgemm_workspace_size(...) bytes, device memory,
 *               16-byte aligned; the 128-row prefill kernels keep per-row
 *               sums of A there (INT4: A_rows x K/G fp32; DELTA2 with base:
 *               A_rows fp32), rewritten on every call; size 0 (NULL allowed)
 *               for every other launch.  Decode-sized plain-epilogue calls
 *               with long K split K and keep fp32 partial sums there
 *               (n_splits x M_total x N).  Nothing in it needs to start at
 *               zero.  The size depends on the kernel choice.  Calls that
 *               share one workspace must be ordered on one stream.  Too small -> MOE_ERR_WORKSPACE_TOO_SMALL,
 *               misaligned -> MOE_ERR_MISALIGNED
 * Supported: N % 32 == 0, K % 128 == 0, G in {32, 64, 128} for INT4 and MWQ.
 */
size_t moe_grouped_qgemm_workspace_size(const moe_wdesc* w, int32_t A_rows, int32_t M_total, int32_t kernel);
moe_status moe_grouped_qgemm(const moe_wdesc* w, const uint16_t* A, int32_t A_rows,
                             const int32_t* gather_pair, int32_t k,
                             const int32_t* seg_offsets, int32_t M_total, int32_t epilogue,
                             int32_t kernel, void* out, void* workspace, size_t workspace_bytes,
                             void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * computation as moe_grouped_qgemm, with the same arguments except the
 * workspace.  The kernels' scratch (activation row sums, split-K partial
 * sums) lives in a static device array of moe_grouped_qgemm_noalloc_scratch_bytes()
 * bytes (8 MiB) that each GPU the library runs on holds until the process
 * ends; a call needing more (moe_grouped_qgemm_workspace_size() above that)
 * returns MOE_ERR_UNSUPPORTED and launches nothing.  Nothing is allocated,
 * freed or copied by the call.  Every call on one GPU shares that GPU's array:
 * calls that overlap on the device (other streams, or concurrent host
 * threads issuing to different streams) race on it and must be ordered by the
 * caller.  Nothing in the array needs to start at zero, and each call
 * rewrites what it reads.  Results are bit for bit those of moe_grouped_qgemm
 * with the same kernel choice.
 */
size_t moe_grouped_qgemm_noalloc_scratch_bytes(void);
moe_status moe_grouped_qgemm_noalloc(const moe_wdesc* w, const uint16_t* A, int32_t A_rows,
                                     const int32_t* gather_pair, int32_t k,
                                     const int32_t* seg_offsets, int32_t M_total, int32_t epilogue,
                                     int32_t kernel, void* out, void* stream);

/* ----------------------------------------------------------------- combine
 * out[t] = sum_{j<k} w[t][j] * y_perm[pair_pos[t*k + j]], accumulated in fp32
 * in slot order j = 0..k-1 and rounded once to bf16 (gate-weighted combine of
 * the selected experts' outputs).
 *   y_perm   [T*k][H] (grouped order) of y_dtype (MOE_DTYPE_BF16,
 *            MOE_DTYPE_F32 or MOE_DTYPE_F16), 16-byte aligned, H % 8 == 0
 *   pair_pos i32 [T*k]
 *   n_valid  device i32 [1], or NULL: the number of rows the GEMMs wrote
 *            (seg_offsets[E*S] of the grouping).  A pair whose pair_pos is at
 *            or past it (an id or bit-width the grouping flagged as invalid)
 *            adds nothing and its row is not read.  NULL: every row is valid.
 *   topk_w   f32 [T*k], or NULL for weight 1 (k = 1 delta layer)
 *   out      bf16 [T][H], 16-byte aligned
 */
moe_status moe_unpermute_combine(const void* y_perm, int32_t y_dtype, const int32_t* pair_pos,
                                 const int32_t* n_valid, const float* topk_w, int32_t T, int32_t k, int32_t H,
                                 uint16_t* out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_QEXPERT_H */

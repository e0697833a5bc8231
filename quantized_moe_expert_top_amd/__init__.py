"""Python binding of libmoe_qexpert.so (the routed-expert quantized MoE library).

Argument marshalling only: every step runs in the library's HIP kernels.
PyTorch supplies device memory and the current stream.  The functions carry
the C ABI's names; outputs are allocated here unless passed in.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_qexpert.so")

MOE_ABI_VERSION = 3
MOE_W_INT4_GROUP, MOE_W_MWQ_2_3_4, MOE_W_DELTA2_SALIENT, MOE_W_INT_PER_EXPERT = 1, 2, 3, 4
MOE_LAYOUT_CANONICAL, MOE_LAYOUT_TILED = 0, 1
MOE_EPI_NONE, MOE_EPI_SWIGLU, MOE_EPI_NONE_F32, MOE_EPI_NONE_F16 = 0, 1, 2, 3
MOE_DTYPE_BF16, MOE_DTYPE_F32, MOE_DTYPE_F16 = 0, 1, 2
# plain-epilogue output dtype of each epilogue, and the epilogue that writes a dtype
_EPI_DTYPE = {MOE_EPI_NONE_F32: torch.float32, MOE_EPI_NONE_F16: torch.float16}
_DTYPE_EPI = {torch.float32: MOE_EPI_NONE_F32, torch.float16: MOE_EPI_NONE_F16, torch.bfloat16: MOE_EPI_NONE}
(MOE_KERNEL_AUTO, MOE_KERNEL_SMALL, MOE_KERNEL_SMALL_PER_WIDTH, MOE_KERNEL_TILE64_WIDE, MOE_KERNEL_TILE64,
 MOE_KERNEL_TILE128, MOE_KERNEL_LDS_DMA, MOE_KERNEL_LDS_DMA_PER_WIDTH) = range(8)
(MOE_FIELD_CODES, MOE_FIELD_PLANE3, MOE_FIELD_PLANE4, MOE_FIELD_SCALES,
 MOE_FIELD_SALIENT_IDX, MOE_FIELD_SALIENT_VAL, MOE_FIELD_BASE) = range(7)

EXPORTED = [
    "moe_status_string", "moe_last_error_detail", "moe_abi_version", "moe_route_topk",
    "moe_permute_workspace_size", "moe_permute", "moe_route_permute", "moe_weight_field_bytes", "moe_repack_weights",
    "moe_grouped_qgemm_workspace_size", "moe_grouped_qgemm", "moe_unpermute_combine",
    "moe_grouped_qgemm_noalloc", "moe_grouped_qgemm_noalloc_scratch_bytes", "moe_copy_rows_async",
]


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status}: {detail}")
        self.status = status


class WDesc(ctypes.Structure):
    _fields_ = [
        ("abi_version", ctypes.c_int32), ("format", ctypes.c_int32), ("layout", ctypes.c_int32),
        ("E", ctypes.c_int32), ("N", ctypes.c_int32), ("K", ctypes.c_int32),
        ("group_size", ctypes.c_int32), ("zero_point", ctypes.c_int32), ("n_salient", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("codes", ctypes.c_void_p), ("plane3", ctypes.c_void_p), ("plane4", ctypes.c_void_p),
        ("scales", ctypes.c_void_p), ("salient_idx", ctypes.c_void_p), ("salient_val", ctypes.c_void_p),
        ("base", ctypes.c_void_p),
        ("expert_bits", ctypes.POINTER(ctypes.c_int32)), ("expert_zero", ctypes.POINTER(ctypes.c_int32)),
    ]


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run quantized_moe_expert_top_amd/build.py "
                          "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(path)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    sig = {
        "moe_status_string": (ctypes.c_char_p, [i32]),
        "moe_last_error_detail": (ctypes.c_char_p, []),
        "moe_abi_version": (i32, []),
        "moe_route_topk": (i32, [vp, i32, i32, i32, vp, vp, vp]),
        "moe_permute_workspace_size": (sz, [i32, i32, i32, i32]),
        "moe_permute": (i32, [vp, vp, i32, i32, i32, vp, vp, vp, vp, vp, i32, vp, vp, sz, vp]),
        "moe_route_permute": (i32, [vp, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "moe_weight_field_bytes": (sz, [ctypes.POINTER(WDesc), i32]),
        "moe_repack_weights": (i32, [ctypes.POINTER(WDesc), ctypes.POINTER(WDesc), vp]),
        "moe_grouped_qgemm_workspace_size": (sz, [ctypes.POINTER(WDesc), i32, i32, i32]),
        "moe_grouped_qgemm": (i32, [ctypes.POINTER(WDesc), vp, i32, vp, i32, vp, i32, i32, i32, vp, vp, sz, vp]),
        "moe_unpermute_combine": (i32, [vp, i32, vp, vp, vp, i32, i32, i32, vp, vp]),
        "moe_grouped_qgemm_noalloc": (i32, [ctypes.POINTER(WDesc), vp, i32, vp, i32, vp, i32, i32, i32, vp, vp]),
        "moe_grouped_qgemm_noalloc_scratch_bytes": (sz, []),
        "moe_copy_rows_async": (i32, [vp, vp, sz, sz, sz, vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        _lib = load_library()
        if _lib.moe_abi_version() != MOE_ABI_VERSION:
            raise ImportError("libmoe_qexpert.so ABI version mismatch")
    return _lib


def _check(status: int, where: str) -> None:
    if status != 0:
        raise MoeError(status, where, lib().moe_last_error_detail().decode())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream=None) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _bf16(t: torch.Tensor) -> torch.Tensor:
    if t.element_size() != 2:
        raise ValueError("expected 16-bit (bf16 bit pattern) tensor")
    return t


# ------------------------------------------------------------------ entry points
def moe_route_topk(logits: torch.Tensor, k: int, ids: torch.Tensor = None, w: torch.Tensor = None, stream=None):
    assert logits.dtype == torch.float32 and logits.dim() == 2
    T, E = logits.shape
    ids = torch.empty((T, k), dtype=torch.int32, device=logits.device) if ids is None else ids
    w = torch.empty((T, k), dtype=torch.float32, device=logits.device) if w is None else w
    _check(lib().moe_route_topk(_ptr(logits), T, E, k, _ptr(ids), _ptr(w), _stream(stream)), "moe_route_topk")
    return ids, w


@dataclass
class Permutation:
    counts: torch.Tensor
    seg_offsets: torch.Tensor
    sorted_pair: torch.Tensor
    pair_pos: torch.Tensor
    workspace: torch.Tensor
    x_perm: Optional[torch.Tensor] = None


def moe_permute(ids: torch.Tensor, E: int, pair_bits: torch.Tensor = None, x: torch.Tensor = None,
                want_x_perm: bool = False, out: Permutation = None, stream=None) -> Permutation:
    T, k = ids.shape
    S = 3 if pair_bits is not None else 1
    dev = ids.device
    if out is None:
        ws_bytes = lib().moe_permute_workspace_size(T, k, E, S)
        out = Permutation(
            counts=torch.empty(E, dtype=torch.int32, device=dev),
            seg_offsets=torch.empty(E * S + 1, dtype=torch.int32, device=dev),
            sorted_pair=torch.empty(T * k, dtype=torch.int32, device=dev),
            pair_pos=torch.empty(T * k, dtype=torch.int32, device=dev),
            workspace=torch.zeros(max(ws_bytes, 16), dtype=torch.uint8, device=dev),
            x_perm=(torch.empty((T * k, x.shape[1]), dtype=x.dtype, device=dev) if want_x_perm else None),
        )
    H = x.shape[1] if x is not None else 0
    _check(lib().moe_permute(_ptr(ids), _ptr(pair_bits), T, k, E, _ptr(out.counts), _ptr(out.seg_offsets),
                             _ptr(out.sorted_pair), _ptr(out.pair_pos), _ptr(x), H, _ptr(out.x_perm),
                             _ptr(out.workspace), out.workspace.numel(), _stream(stream)), "moe_permute")
    return out


def moe_route_permute(logits: torch.Tensor, k: int, pair_bits: torch.Tensor = None, ids: torch.Tensor = None,
                      w: torch.Tensor = None, out: Permutation = None, stream=None):
    """Routing + grouping in one call (one launch for small batches); returns (ids, w, Permutation).
    The Permutation's workspace must start zero-filled (as allocated here and by moe_permute)."""
    assert logits.dtype == torch.float32 and logits.dim() == 2
    T, E = logits.shape
    dev = logits.device
    S = 3 if pair_bits is not None else 1
    ids = torch.empty((T, k), dtype=torch.int32, device=dev) if ids is None else ids
    w = torch.empty((T, k), dtype=torch.float32, device=dev) if w is None else w
    if out is None:
        ws_bytes = lib().moe_permute_workspace_size(T, k, E, S)
        out = Permutation(
            counts=torch.empty(E, dtype=torch.int32, device=dev),
            seg_offsets=torch.empty(E * S + 1, dtype=torch.int32, device=dev),
            sorted_pair=torch.empty(T * k, dtype=torch.int32, device=dev),
            pair_pos=torch.empty(T * k, dtype=torch.int32, device=dev),
            workspace=torch.zeros(max(ws_bytes, 16), dtype=torch.uint8, device=dev))
    _check(lib().moe_route_permute(_ptr(logits), T, E, k, _ptr(pair_bits), _ptr(ids), _ptr(w), _ptr(out.counts),
                                   _ptr(out.seg_offsets), _ptr(out.sorted_pair), _ptr(out.pair_pos),
                                   _ptr(out.workspace), out.workspace.numel(), _stream(stream)), "moe_route_permute")
    return ids, w, out


@dataclass
class QuantizedExperts:
    """A weight set in one layout; keeps its tensors (and host tables) alive with the descriptor."""
    desc: WDesc
    tensors: dict = field(default_factory=dict)
    host: dict = field(default_factory=dict)

    @property
    def N(self):
        return self.desc.N

    @property
    def K(self):
        return self.desc.K


def make_desc(fmt: int, layout: int, E: int, N: int, K: int, group_size: int, zero_point: int,
              n_salient: int = 0, expert_bits=None, expert_zero=None, **tensors) -> QuantizedExperts:
    """expert_bits / expert_zero: per-expert widths and zero points (host sequences of E ints)."""
    d = WDesc()
    d.abi_version, d.format, d.layout = MOE_ABI_VERSION, fmt, layout
    d.E, d.N, d.K, d.group_size, d.zero_point, d.n_salient = E, N, K, group_size, zero_point, n_salient
    for name in ("codes", "plane3", "plane4", "scales", "salient_idx", "salient_val", "base"):
        t = tensors.get(name)
        setattr(d, name, _ptr(t) if t is not None else None)
    host = {}
    if expert_bits is not None:
        host["expert_bits"] = (ctypes.c_int32 * E)(*[int(v) for v in expert_bits])
        host["expert_zero"] = (ctypes.c_int32 * E)(*[int(v) for v in expert_zero])
        d.expert_bits = ctypes.cast(host["expert_bits"], ctypes.POINTER(ctypes.c_int32))
        d.expert_zero = ctypes.cast(host["expert_zero"], ctypes.POINTER(ctypes.c_int32))
    return QuantizedExperts(d, {k: v for k, v in tensors.items() if v is not None}, host)


def moe_weight_field_bytes(q: QuantizedExperts, fld: int) -> int:
    return lib().moe_weight_field_bytes(ctypes.byref(q.desc), fld)


def moe_repack_weights(src: QuantizedExperts, stream=None) -> QuantizedExperts:
    """Canonical -> tiled copy of a weight set (offline; allocates the tiled buffers)."""
    s = src.desc
    dev = next(iter(src.tensors.values())).device
    tables = {}
    if src.host:
        tables = {"expert_bits": list(src.host["expert_bits"]), "expert_zero": list(src.host["expert_zero"])}
    probe = make_desc(s.format, MOE_LAYOUT_TILED, s.E, s.N, s.K, s.group_size, s.zero_point, s.n_salient, **tables)
    t = {}
    for name, fld in (("codes", MOE_FIELD_CODES), ("plane3", MOE_FIELD_PLANE3), ("plane4", MOE_FIELD_PLANE4),
                      ("salient_val", MOE_FIELD_SALIENT_VAL)):
        nb = moe_weight_field_bytes(probe, fld)
        if nb and name in src.tensors:
            t[name] = torch.empty(nb, dtype=torch.uint8, device=dev)
    if "base" in src.tensors:
        t["base"] = torch.empty_like(src.tensors["base"])
    for name in ("scales", "salient_idx"):
        if name in src.tensors:
            t[name] = src.tensors[name]
    dst = make_desc(s.format, MOE_LAYOUT_TILED, s.E, s.N, s.K, s.group_size, s.zero_point, s.n_salient, **tables, **t)
    _check(lib().moe_repack_weights(ctypes.byref(s), ctypes.byref(dst.desc), _stream(stream)), "moe_repack_weights")
    return dst


def _check_segments(w: QuantizedExperts, seg_offsets: torch.Tensor) -> None:
    """The GEMM reads E*S + 1 offsets (S = 3 for nested planes, else 1): a shorter
    table would send its kernels to rows past the buffers."""
    need = w.desc.E * (3 if w.desc.format == MOE_W_MWQ_2_3_4 else 1) + 1
    if seg_offsets.dtype != torch.int32 or seg_offsets.dim() != 1 or seg_offsets.numel() < need:
        raise ValueError(f"seg_offsets must be int32 with at least {need} entries for this weight set "
                         f"(got {seg_offsets.dtype}, {tuple(seg_offsets.shape)})")


def moe_grouped_qgemm_workspace_size(w: QuantizedExperts, A_rows: int, M_total: int,
                                     kernel: int = MOE_KERNEL_AUTO) -> int:
    return lib().moe_grouped_qgemm_workspace_size(ctypes.byref(w.desc), A_rows, M_total, kernel)


def moe_grouped_qgemm(w: QuantizedExperts, A: torch.Tensor, seg_offsets: torch.Tensor, M_total: int,
                      epilogue: int = MOE_EPI_NONE, gather_pair: torch.Tensor = None, k: int = 1,
                      out: torch.Tensor = None, workspace: torch.Tensor = None, stream=None,
                      kernel: int = MOE_KERNEL_AUTO) -> torch.Tensor:
    _bf16(A)
    _check_segments(w, seg_offsets)
    A_rows = A.shape[0]
    n_out = w.N // 2 if epilogue == MOE_EPI_SWIGLU else w.N
    if out is None:
        dt = _EPI_DTYPE.get(epilogue, torch.bfloat16)
        out = torch.empty((M_total, n_out), dtype=dt, device=A.device)
    ws_need = moe_grouped_qgemm_workspace_size(w, A_rows, M_total, kernel)
    if workspace is None and ws_need:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=A.device)
    ws_bytes = workspace.numel() if workspace is not None else 0
    _check(lib().moe_grouped_qgemm(ctypes.byref(w.desc), _ptr(A), A_rows, _ptr(gather_pair), k, _ptr(seg_offsets),
                                   M_total, epilogue, kernel, _ptr(out), _ptr(workspace), ws_bytes,
                                   _stream(stream)),
           "moe_grouped_qgemm")
    return out


def moe_grouped_qgemm_noalloc(w: QuantizedExperts, A: torch.Tensor, seg_offsets: torch.Tensor, M_total: int,
                              epilogue: int = MOE_EPI_NONE, gather_pair: torch.Tensor = None, k: int = 1,
                              out: torch.Tensor = None, stream=None, kernel: int = MOE_KERNEL_AUTO) -> torch.Tensor:
    """moe_grouped_qgemm without a workspace: the library's static device scratch
    (moe_grouped_qgemm_noalloc_scratch_bytes()) serves instead.  Pass `out` to
    allocate nothing at all."""
    _bf16(A)
    _check_segments(w, seg_offsets)
    n_out = w.N // 2 if epilogue == MOE_EPI_SWIGLU else w.N
    if out is None:
        dt = _EPI_DTYPE.get(epilogue, torch.bfloat16)
        out = torch.empty((M_total, n_out), dtype=dt, device=A.device)
    _check(lib().moe_grouped_qgemm_noalloc(ctypes.byref(w.desc), _ptr(A), A.shape[0], _ptr(gather_pair), k,
                                           _ptr(seg_offsets), M_total, epilogue, kernel, _ptr(out),
                                           _stream(stream)), "moe_grouped_qgemm_noalloc")
    return out


def moe_copy_rows_async(dst: torch.Tensor, dst_offset: int, src: torch.Tensor, src_offset: int, rows: int,
                        pitch: int, width: int, stream=None) -> None:
    """Queues `rows` pieces of `width` bytes, `pitch` bytes apart, from pinned
    host tensor `src` (from byte src_offset) to device tensor `dst` (from byte
    dst_offset) on `stream` (one plane of a tiled nested-MWQ expert)."""
    if not src.is_pinned() or not dst.is_cuda:
        raise ValueError("moe_copy_rows_async copies pinned host memory to device memory")
    span = (rows - 1) * pitch + width if rows and width else 0
    for t, off in ((src, src_offset), (dst, dst_offset)):
        if off < 0 or off + span > t.numel() * t.element_size():
            raise ValueError("copy range outside the tensor")
    _check(lib().moe_copy_rows_async(dst.data_ptr() + dst_offset, src.data_ptr() + src_offset, rows, pitch, width,
                                     _stream(stream)), "moe_copy_rows_async")


def moe_unpermute_combine(y_perm: torch.Tensor, pair_pos: torch.Tensor, topk_w: Optional[torch.Tensor],
                          T: int, k: int, out: torch.Tensor = None, stream=None,
                          n_valid: torch.Tensor = None) -> torch.Tensor:
    """y_perm: fp32 or 16-bit (bf16 bit pattern) rows in grouped order.  n_valid: optional
    one-element int32 device tensor (e.g. seg_offsets[-1:]); pairs at or past it add nothing."""
    y_dtype = {torch.float32: MOE_DTYPE_F32, torch.float16: MOE_DTYPE_F16}.get(y_perm.dtype, MOE_DTYPE_BF16)
    if y_dtype == MOE_DTYPE_BF16:
        _bf16(y_perm)
    H = y_perm.shape[1]
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=y_perm.device)
    nv = None
    if n_valid is not None:
        if n_valid.dtype != torch.int32 or n_valid.numel() < 1 or not n_valid.is_cuda:
            raise ValueError("n_valid must be an int32 device tensor")
        nv = n_valid.data_ptr()  # a one-element view of a longer table is fine
    _check(lib().moe_unpermute_combine(_ptr(y_perm), y_dtype, _ptr(pair_pos), nv, _ptr(topk_w), T, k, H,
                                       _ptr(out), _stream(stream)), "moe_unpermute_combine")
    return out


# --------------------------------------------------------------- conveniences
def int4_experts(codes: torch.Tensor, scales: torch.Tensor, group_size: int, zero_point: int = 8) -> QuantizedExperts:
    """Canonical INT4 weights: codes u8 [E][N][K/2], scales fp16 [E][N][K/G]."""
    E, N, Kh = codes.shape
    return make_desc(MOE_W_INT4_GROUP, MOE_LAYOUT_CANONICAL, E, N, 2 * Kh, group_size, zero_point,
                     codes=codes, scales=scales)


def mwq_experts(q2, d3, d4, scales, group_size: int, zero_point: int = 8) -> QuantizedExperts:
    E, N, Kq = q2.shape
    return make_desc(MOE_W_MWQ_2_3_4, MOE_LAYOUT_CANONICAL, E, N, 4 * Kq, group_size, zero_point,
                     codes=q2, plane3=d3, plane4=d4, scales=scales)


def per_expert_experts(codes, scales, expert_bits, expert_zero, group_size: int) -> QuantizedExperts:
    """Static width per expert: codes u8 flat (expert e's N x K codes of
    expert_bits[e] bits, a little-endian bit stream per row, experts back to
    back), scales fp16 [E][N][K/G], expert_bits / expert_zero host sequences."""
    E, N, KG = scales.shape
    return make_desc(MOE_W_INT_PER_EXPERT, MOE_LAYOUT_CANONICAL, E, N, KG * group_size, group_size, 0,
                     expert_bits=expert_bits, expert_zero=expert_zero, codes=codes, scales=scales)


def delta2_experts(codes, step, salient_idx, salient_val, base=None, zero_point: int = 2) -> QuantizedExperts:
    E, N, Kq = codes.shape
    return make_desc(MOE_W_DELTA2_SALIENT, MOE_LAYOUT_CANONICAL, E, N, 4 * Kq, 4 * Kq, zero_point,
                     n_salient=salient_idx.shape[1], codes=codes, scales=step, salient_idx=salient_idx,
                     salient_val=salient_val, base=base)


@dataclass
class LayerBuffers:
    """Preallocated intermediates of one MoE layer forward."""
    ids: torch.Tensor
    w: torch.Tensor
    perm: Permutation
    h: torch.Tensor
    y_perm: torch.Tensor
    out: torch.Tensor


def alloc_layer(T: int, E: int, k: int, H: int, I: int, mwq: bool, device,
                y_dtype: torch.dtype = torch.float16) -> LayerBuffers:
    """y_dtype: the experts' outputs before the combine: float16 (default),
    float32 or bfloat16."""
    if y_dtype not in _DTYPE_EPI:
        raise ValueError(f"expert outputs in {y_dtype}: float16, float32 or bfloat16")
    S = 3 if mwq else 1
    ws = lib().moe_permute_workspace_size(T, k, E, S)
    perm = Permutation(
        counts=torch.empty(E, dtype=torch.int32, device=device),
        seg_offsets=torch.empty(E * S + 1, dtype=torch.int32, device=device),
        sorted_pair=torch.empty(T * k, dtype=torch.int32, device=device),
        pair_pos=torch.empty(T * k, dtype=torch.int32, device=device),
        workspace=torch.zeros(max(ws, 16), dtype=torch.uint8, device=device))
    return LayerBuffers(
        ids=torch.empty((T, k), dtype=torch.int32, device=device),
        w=torch.empty((T, k), dtype=torch.float32, device=device),
        perm=perm,
        h=torch.empty((T * k, I), dtype=torch.bfloat16, device=device),
        y_perm=torch.empty((T * k, H), dtype=y_dtype, device=device),
        out=torch.empty((T, H), dtype=torch.bfloat16, device=device))


def moe_layer_forward(x: torch.Tensor, logits: torch.Tensor, k: int, gate_up: QuantizedExperts,
                      down: QuantizedExperts, pair_bits: torch.Tensor = None,
                      buf: LayerBuffers = None, stream=None, kernel: int = MOE_KERNEL_AUTO) -> LayerBuffers:
    """Route -> group -> gate_up (+SwiGLU, bf16 h) -> down (expert outputs in buf.y_perm's dtype: fp16
    unless the buffers were allocated otherwise) -> combine, one stream.
    kernel: the grouped GEMMs' kernel choice (MOE_KERNEL_*; AUTO chooses from the shapes)."""
    T, H = x.shape
    E = logits.shape[1]
    I = gate_up.N // 2
    if (gate_up.desc.format == MOE_W_MWQ_2_3_4) != (pair_bits is not None):
        raise ValueError("nested-plane weights need pair_bits (a width per pair); other formats take none")
    if buf is None:
        buf = alloc_layer(T, E, k, H, I, pair_bits is not None, x.device)
    moe_route_permute(logits, k, pair_bits=pair_bits, ids=buf.ids, w=buf.w, out=buf.perm, stream=stream)
    moe_grouped_qgemm(gate_up, x, buf.perm.seg_offsets, T * k, MOE_EPI_SWIGLU, gather_pair=buf.perm.sorted_pair,
                      k=k, out=buf.h, stream=stream, kernel=kernel)
    moe_grouped_qgemm(down, buf.h, buf.perm.seg_offsets, T * k, _DTYPE_EPI[buf.y_perm.dtype], out=buf.y_perm, stream=stream,
                      kernel=kernel)
    moe_unpermute_combine(buf.y_perm, buf.perm.pair_pos, buf.w, T, k, out=buf.out, stream=stream,
                          n_valid=buf.perm.seg_offsets[-1:])
    return buf

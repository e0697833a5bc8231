"""Host-side checks of the C ABI library (no GPU needed): the built library
loads, exports every function the header declares, and rejects bad arguments
with the documented status codes before touching the device."""
import ctypes
import os
import re

import pytest

import quantized_moe_expert_top_amd as q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_qexpert.h")

OK, NULL_ARG, BAD_SHAPE, BAD_FORMAT, MISALIGNED, WS_SMALL, UNSUPPORTED, HIP = range(8)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(q.LIB_PATH):
        pytest.fail("library not built: run __graft_entry__.build()")
    return q.lib()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\*?\s+\*?(moe_[a-z_]+)\(", text, re.M)))


def test_header_declares_expected_entry_points():
    names = declared_functions()
    for n in ("moe_route_topk", "moe_permute", "moe_route_permute", "moe_grouped_qgemm", "moe_unpermute_combine",
              "moe_repack_weights", "moe_permute_workspace_size"):
        assert n in names
    assert set(names) == set(q.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(q.LIB_PATH)
    for name in declared_functions():
        assert hasattr(raw, name), name
    assert lib.moe_abi_version() == q.MOE_ABI_VERSION


def test_status_strings(lib):
    for s in range(8):
        assert lib.moe_status_string(s)
    assert lib.moe_status_string(99) == b"unknown status"


def fake(addr):
    return ctypes.c_void_p(addr)


def test_route_validation(lib):
    A = fake(0x1000)
    assert lib.moe_route_topk(A, 4, 0, 1, A, A, None) == BAD_SHAPE
    assert lib.moe_route_topk(A, 4, 8, 9, A, A, None) == BAD_SHAPE
    assert lib.moe_route_topk(A, 4, 2000, 2, A, A, None) == BAD_SHAPE
    assert lib.moe_route_topk(A, -1, 8, 2, A, A, None) == BAD_SHAPE
    assert lib.moe_route_topk(None, 4, 8, 2, A, A, None) == NULL_ARG
    assert b"required" in lib.moe_last_error_detail()
    assert lib.moe_route_topk(fake(0x1002), 4, 8, 2, A, A, None) == MISALIGNED
    assert lib.moe_route_topk(None, 0, 8, 2, None, None, None) == OK  # nothing to do
    assert lib.moe_last_error_detail() == b""
    assert lib.moe_route_topk(A, 1 << 28, 1024, 16, A, A, None) == BAD_SHAPE  # T*k >= 2^31


def test_permute_validation(lib):
    A = fake(0x1000)
    need = lib.moe_permute_workspace_size(8192, 8, 64, 1)
    assert need > 256
    assert lib.moe_permute_workspace_size(32, 8, 64, 1) == 256   # one-workgroup path: the flag and counter words only
    assert lib.moe_permute_workspace_size(4, 1, 8, 2) == 0  # S must be 1 or 3
    args = lambda ws_bytes, ws=A: (A, None, 8192, 8, 64, A, A, A, A, None, 0, None, ws, ws_bytes, None)  # noqa: E731
    assert lib.moe_permute(*args(need - 1)) == WS_SMALL
    assert lib.moe_permute(*args(need, None)) == NULL_ARG
    assert lib.moe_permute(*args(need, fake(0x1004))) == MISALIGNED
    assert lib.moe_permute(A, None, 16, 9, 8, A, A, A, A, None, 0, None, A, 1 << 20, None) == BAD_SHAPE
    # x_perm requested without x / with bad H
    assert lib.moe_permute(A, None, 16, 2, 8, A, A, A, A, None, 64, A, A, 1 << 20, None) == NULL_ARG
    assert lib.moe_permute(A, None, 16, 2, 8, A, A, A, A, A, 12, A, A, 1 << 20, None) == BAD_SHAPE


def test_route_permute_validation(lib):
    A = fake(0x1000)
    need = lib.moe_permute_workspace_size(32, 8, 64, 1)
    args = lambda T=32, E=64, k=8, ws=A, ws_bytes=need: (A, T, E, k, None, A, A, A, A, A, A, ws, ws_bytes, None)  # noqa: E731
    assert lib.moe_route_permute(*args(T=-1)) == BAD_SHAPE
    assert lib.moe_route_permute(*args(E=2000)) == BAD_SHAPE
    assert lib.moe_route_permute(*args(k=65)) == BAD_SHAPE
    assert lib.moe_route_permute(*args(ws_bytes=need - 1)) == WS_SMALL
    assert lib.moe_route_permute(*args(ws=None)) == NULL_ARG
    assert lib.moe_route_permute(*args(ws=fake(0x1004))) == MISALIGNED
    assert lib.moe_route_permute(None, 32, 64, 8, None, A, A, A, A, A, A, A, need, None) == NULL_ARG
    assert lib.moe_route_permute(fake(0x1002), 32, 64, 8, None, A, A, A, A, A, A, A, need, None) == MISALIGNED


def desc(fmt=q.MOE_W_INT4_GROUP, layout=q.MOE_LAYOUT_TILED, E=8, N=256, K=512, G=128, z=8, ns=0, **ptrs):
    d = q.WDesc()
    d.abi_version, d.format, d.layout = q.MOE_ABI_VERSION, fmt, layout
    d.E, d.N, d.K, d.group_size, d.zero_point, d.n_salient = E, N, K, G, z, ns
    d.codes = ptrs.get("codes", 0x10000)
    d.scales = ptrs.get("scales", 0x20000)
    d.plane3 = ptrs.get("plane3", 0x30000)
    d.plane4 = ptrs.get("plane4", 0x40000)
    d.salient_idx = ptrs.get("salient_idx", 0x50000)
    d.salient_val = ptrs.get("salient_val", 0x60000)
    d.base = ptrs.get("base", None)
    if "bits" in ptrs:  # per-expert widths: host tables, kept alive on the descriptor object
        d._tables = ((ctypes.c_int32 * E)(*ptrs["bits"]), (ctypes.c_int32 * E)(*ptrs["zero"]))
        d.expert_bits = ctypes.cast(d._tables[0], ctypes.POINTER(ctypes.c_int32))
        d.expert_zero = ctypes.cast(d._tables[1], ctypes.POINTER(ctypes.c_int32))
    return d


def gemm(lib, d, A=0x1000, rows=64, gather=0x2000, k=2, seg=0x3000, M=128, epi=q.MOE_EPI_SWIGLU, out=0x4000,
         kernel=q.MOE_KERNEL_AUTO):
    return lib.moe_grouped_qgemm(ctypes.byref(d), fake(A) if A else None, rows, fake(gather) if gather else None, k,
                                 fake(seg) if seg else None, M, epi, kernel, fake(out) if out else None, None, 0, None)


def test_grouped_qgemm_validation(lib):
    assert gemm(lib, desc(layout=q.MOE_LAYOUT_CANONICAL)) == BAD_FORMAT
    d = desc()
    d.abi_version = 7
    assert gemm(lib, d) == BAD_FORMAT
    assert gemm(lib, desc(fmt=9)) == BAD_FORMAT
    assert gemm(lib, desc(G=48)) == UNSUPPORTED
    assert gemm(lib, desc(N=48)) == UNSUPPORTED
    assert gemm(lib, desc(K=200)) == UNSUPPORTED
    assert gemm(lib, desc(z=16)) == BAD_SHAPE
    assert gemm(lib, desc(codes=0)) == NULL_ARG
    assert gemm(lib, desc(codes=0x10008)) == MISALIGNED
    # canonical nested planes need plane3 / plane4; the tiled layout keeps them in codes
    mwq_src = desc(fmt=q.MOE_W_MWQ_2_3_4, layout=q.MOE_LAYOUT_CANONICAL, plane3=0)
    mwq_dst = desc(fmt=q.MOE_W_MWQ_2_3_4, codes=0x70000)
    assert lib.moe_repack_weights(ctypes.byref(mwq_src), ctypes.byref(mwq_dst), None) == NULL_ARG
    assert gemm(lib, desc(fmt=q.MOE_W_DELTA2_SALIENT, z=2, ns=65)) == UNSUPPORTED
    assert gemm(lib, desc(), epi=5) == BAD_FORMAT
    assert gemm(lib, desc(G=16)) == UNSUPPORTED
    assert gemm(lib, desc(), rows=10, k=2, M=128) == BAD_SHAPE        # A_rows * k < M_total
    assert gemm(lib, desc(), gather=0, rows=10, M=128) == BAD_SHAPE   # A_rows < M_total
    assert gemm(lib, desc(), A=0) == NULL_ARG
    assert gemm(lib, desc(), out=0x4004) == MISALIGNED
    assert gemm(lib, desc(), M=0, A=0, seg=0, out=0) == OK           # empty problem
    # kernel choices: unknown, or not for this format
    assert gemm(lib, desc(), kernel=8) == BAD_FORMAT
    assert gemm(lib, desc(), kernel=q.MOE_KERNEL_LDS_DMA_PER_WIDTH) == UNSUPPORTED          # nested MWQ only
    assert gemm(lib, desc(), kernel=-1) == BAD_FORMAT
    assert gemm(lib, desc(), kernel=q.MOE_KERNEL_SMALL_PER_WIDTH) == UNSUPPORTED            # nested MWQ only
    delta = dict(fmt=q.MOE_W_DELTA2_SALIENT, z=2, ns=4)
    assert gemm(lib, desc(**delta), kernel=q.MOE_KERNEL_TILE64) == UNSUPPORTED
    assert gemm(lib, desc(**delta), kernel=q.MOE_KERNEL_LDS_DMA, epi=q.MOE_EPI_NONE) == UNSUPPORTED  # no base
    assert gemm(lib, desc(**delta, base=0x80000), kernel=q.MOE_KERNEL_LDS_DMA) == UNSUPPORTED  # SwiGLU epilogue
    mixed = desc(fmt=q.MOE_W_INT_PER_EXPERT, E=4, bits=[4, 2, 3, 2], zero=[8, 1, 3, 2])
    assert gemm(lib, mixed, kernel=q.MOE_KERNEL_LDS_DMA) == UNSUPPORTED
    assert lib.moe_grouped_qgemm_workspace_size(ctypes.byref(desc()), 64, 128, 9) == 0


def test_grouped_qgemm_workspace(lib):
    # many rows per expert (INT4): the 128-row kernel keeps activation row sums in the workspace
    d = desc(E=8, N=256, K=512, G=128)
    need = lib.moe_grouped_qgemm_workspace_size(ctypes.byref(d), 4096, 8192, 0)
    assert need == 4096 * (512 // 128) * 4
    assert lib.moe_grouped_qgemm_workspace_size(ctypes.byref(d), 32, 64, 0) == 0          # decode-sized: none
    mwq = desc(fmt=q.MOE_W_MWQ_2_3_4, E=8, N=256, K=512, G=128)
    # nested MWQ: 1024 rows per expert take the 128-row kernel; 64 do not
    assert lib.moe_grouped_qgemm_workspace_size(ctypes.byref(mwq), 4096, 8192, 0) == 4096 * (512 // 128) * 4
    assert lib.moe_grouped_qgemm_workspace_size(ctypes.byref(mwq), 256, 512, 0) == 0
    # long K, few channel groups and row tiles (a decode batch's down projection,
    # 32 rows, N 4096, K 14336): 32 x (2 + 8) work items -> 4 K splits of 28 blocks,
    # fp32 partial sums [4][32][4096]
    for fmt in (q.MOE_W_INT4_GROUP, q.MOE_W_MWQ_2_3_4):
        dn = desc(fmt=fmt, E=8, N=4096, K=14336, G=128)
        assert lib.moe_grouped_qgemm_workspace_size(ctypes.byref(dn), 32, 32, 0) == 4 * 32 * 4096 * 4
    # enough work items without a split (64 experts, N 2048, K 1024)
    assert lib.moe_grouped_qgemm_workspace_size(ctypes.byref(desc(E=64, N=2048, K=1024, G=128)), 256, 256, 0) == 0
    call = lambda ws, nbytes: lib.moe_grouped_qgemm(ctypes.byref(d), fake(0x1000), 4096, fake(0x2000), 2,  # noqa
                                                    fake(0x3000), 8192, q.MOE_EPI_SWIGLU, q.MOE_KERNEL_AUTO,
                                                    fake(0x4000), ws, nbytes, None)
    assert call(None, 0) == WS_SMALL
    assert call(fake(0x5000), need - 1) == WS_SMALL
    assert call(None, need) == NULL_ARG
    assert call(fake(0x5008), need) == MISALIGNED


def test_weight_field_bytes_and_nested_storage(lib):
    H, I, E, G = 4096, 14336, 8, 128
    mwq = desc(fmt=q.MOE_W_MWQ_2_3_4, layout=q.MOE_LAYOUT_CANONICAL, E=E, N=2 * I, K=H, G=G)
    int4 = desc(fmt=q.MOE_W_INT4_GROUP, layout=q.MOE_LAYOUT_CANONICAL, E=E, N=2 * I, K=H, G=G)
    fb = lambda d, f: lib.moe_weight_field_bytes(ctypes.byref(d), f)  # noqa: E731
    planes = fb(mwq, q.MOE_FIELD_CODES) + fb(mwq, q.MOE_FIELD_PLANE3) + fb(mwq, q.MOE_FIELD_PLANE4)
    assert planes == fb(int4, q.MOE_FIELD_CODES) == E * 2 * I * H // 2
    assert fb(int4, q.MOE_FIELD_PLANE3) == 0
    mwq_t = desc(fmt=q.MOE_W_MWQ_2_3_4, layout=q.MOE_LAYOUT_TILED, E=E, N=2 * I, K=H, G=G)
    assert fb(mwq_t, q.MOE_FIELD_CODES) == planes          # tiled: the three planes of a tile block together
    assert fb(mwq_t, q.MOE_FIELD_PLANE3) == fb(mwq_t, q.MOE_FIELD_PLANE4) == 0
    assert fb(int4, q.MOE_FIELD_SCALES) == E * 2 * I * (H // G) * 2
    tiled = desc(fmt=q.MOE_W_DELTA2_SALIENT, E=16, N=14336, K=4096, z=2, ns=41)
    assert fb(tiled, q.MOE_FIELD_SALIENT_VAL) == 16 * (14336 // 16) * 2 * 1024
    assert fb(tiled, q.MOE_FIELD_BASE) == 14336 * 4096 * 2
    assert fb(desc(G=48), q.MOE_FIELD_CODES) == 0   # invalid descriptor


def test_repack_validation(lib):
    src = desc(layout=q.MOE_LAYOUT_CANONICAL)
    dst = desc(layout=q.MOE_LAYOUT_TILED, codes=0x70000)
    assert lib.moe_repack_weights(ctypes.byref(dst), ctypes.byref(dst), None) == BAD_FORMAT
    bad = desc(layout=q.MOE_LAYOUT_TILED, codes=0x70000, N=512)
    assert lib.moe_repack_weights(ctypes.byref(src), ctypes.byref(bad), None) == BAD_SHAPE
    same = desc(layout=q.MOE_LAYOUT_TILED)
    assert lib.moe_repack_weights(ctypes.byref(src), ctypes.byref(same), None) == BAD_SHAPE


def test_combine_validation(lib):
    A = fake(0x1000)
    assert lib.moe_unpermute_combine(A, 0, A, None, A, 4, 2, 12, A, None) == BAD_SHAPE
    assert lib.moe_unpermute_combine(A, 3, A, None, A, 4, 2, 16, A, None) == BAD_FORMAT
    assert lib.moe_unpermute_combine(None, 1, A, None, A, 4, 2, 16, A, None) == NULL_ARG
    assert lib.moe_unpermute_combine(fake(0x1008), 0, A, None, A, 4, 2, 16, A, None) == MISALIGNED
    assert lib.moe_unpermute_combine(A, 0, A, fake(0x2002), A, 4, 2, 16, A, None) == MISALIGNED   # n_valid
    assert lib.moe_unpermute_combine(None, 0, None, None, None, 0, 2, 16, None, None) == OK


def test_binding_refuses_missing_library(tmp_path):
    with pytest.raises(ImportError):
        q.load_library(str(tmp_path / "missing.so"))



def test_per_expert_width_validation_and_sizes(lib):
    """Static bit-width per expert: tables required and checked; codes hold
    N*K*b_e/8 bytes per expert in either layout; no planes."""
    P = q.MOE_W_INT_PER_EXPERT
    fb = lambda d, f: lib.moe_weight_field_bytes(ctypes.byref(d), f)  # noqa: E731
    bits, zero = [4, 2, 3, 2], [8, 1, 3, 2]
    for layout in (q.MOE_LAYOUT_CANONICAL, q.MOE_LAYOUT_TILED):
        d = desc(fmt=P, layout=layout, E=4, N=256, K=512, bits=bits, zero=zero)
        assert fb(d, q.MOE_FIELD_CODES) == 256 * 512 * sum(bits) // 8
        assert fb(d, q.MOE_FIELD_PLANE3) == fb(d, q.MOE_FIELD_PLANE4) == 0
        assert fb(d, q.MOE_FIELD_SCALES) == 4 * 256 * (512 // 128) * 2
    assert fb(desc(fmt=P, E=4), q.MOE_FIELD_CODES) == 0                     # tables missing
    assert gemm(lib, desc(fmt=P, E=4)) == NULL_ARG
    for w in (1, 5, 6, 7, 9, 16):                                                             # 2, 3, 4, 8 only
        assert gemm(lib, desc(fmt=P, E=4, bits=[4, w, 2, 2], zero=[0, 0, 0, 0])) == UNSUPPORTED
    d8 = desc(fmt=P, E=4, N=256, K=512, bits=[4, 8, 2, 2], zero=[0, 255, 0, 0])                # an INT8 expert
    assert gemm(lib, d8, M=0, A=0, seg=0, out=0) == OK
    assert fb(d8, q.MOE_FIELD_CODES) == 256 * 512 * 16 // 8
    assert gemm(lib, desc(fmt=P, E=4, bits=[4, 8, 2, 2], zero=[0, 256, 0, 0])) == BAD_SHAPE
    assert gemm(lib, desc(fmt=P, E=4, bits=[4, 2, 2, 2], zero=[0, 4, 0, 0])) == BAD_SHAPE     # z >= 2^b
    assert gemm(lib, desc(fmt=P, E=300, bits=[2] * 300, zero=[1] * 300)) == UNSUPPORTED       # E > 256
    src = desc(fmt=P, layout=q.MOE_LAYOUT_CANONICAL, E=4, bits=bits, zero=zero)
    dst = desc(fmt=P, E=4, codes=0x70000, bits=bits, zero=[8, 1, 3, 1])
    assert lib.moe_repack_weights(ctypes.byref(src), ctypes.byref(dst), None) == BAD_SHAPE   # tables disagree


def test_binding_checks_segment_table_and_widths():
    """The binding refuses a segment table shorter than the weight set's E*S + 1
    offsets (the kernels would read offsets past it) and a layer call whose
    nested-plane weights come without per-pair widths (or widths without them),
    before any library call that launches."""
    import torch
    E, N, K = 4, 64, 128

    def weights(fmt):  # a descriptor only: nothing is launched
        d = q.WDesc()
        d.abi_version, d.format, d.layout, d.E, d.N, d.K, d.group_size = q.MOE_ABI_VERSION, fmt, q.MOE_LAYOUT_TILED, E, N, K, 128
        return q.QuantizedExperts(desc=d)
    mwq, int4 = weights(q.MOE_W_MWQ_2_3_4), weights(q.MOE_W_INT4_GROUP)
    A = torch.zeros((8, K), dtype=torch.int16)
    for w, short in ((mwq, E + 1), (int4, E)):
        with pytest.raises(ValueError, match="seg_offsets"):
            q.moe_grouped_qgemm(w, A, torch.zeros(short, dtype=torch.int32), 8)
        with pytest.raises(ValueError, match="seg_offsets"):
            q.moe_grouped_qgemm_noalloc(w, A, torch.zeros(short, dtype=torch.int32), 8)
    with pytest.raises(ValueError, match="seg_offsets"):
        q.moe_grouped_qgemm(int4, A, torch.zeros(E + 1, dtype=torch.int64), 8)
    x = torch.zeros((8, K), dtype=torch.int16)
    logits = torch.zeros((8, E), dtype=torch.float32)
    with pytest.raises(ValueError, match="pair_bits"):
        q.moe_layer_forward(x, logits, 2, mwq, mwq)
    with pytest.raises(ValueError, match="pair_bits"):
        q.moe_layer_forward(x, logits, 2, int4, int4, pair_bits=torch.full((8, 2), 4, dtype=torch.uint8))

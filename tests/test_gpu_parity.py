"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Bars: expert ids, counts, offsets and permutation indices bit-exact; gate
weights within 1e-6 relative; bf16 outputs within relative L2 5e-3 and
max-abs 2e-2 x RMS of the oracle output, against the oracle's float64 layer
(no intermediate rounding).  Several tests add an element-wise check against
the oracle's bf16-activation variant (check_ulp).
"""
import numpy as np
import pytest
import torch

import gen
import oracle
from oracle import cpp as REF  # the C++17 float64 oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def G():
    from tests import gpu_helpers  # imports torch and the binding
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return gpu_helpers


# ------------------------------------------------------------------ routing
@pytest.mark.parametrize("name,k", [("tiny", 2), ("olmoe_decode", 8), ("olmoe_prefill", 8),
                                    ("olmoe_prefill_zipf", 8), ("mixtral_mwq", 2)])
def test_route_topk_parity(G, name, k):
    cfg = gen.config(name)
    logits = gen._logits(cfg)
    ids, w = G.q.moe_route_topk(G.t(logits), k)
    ref_ids, ref_w = REF.route_topk(logits, k)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    np.testing.assert_allclose(w.cpu().numpy().astype(np.float64), ref_w, rtol=G.GATE_RTOL, atol=0)


@pytest.mark.parametrize("T,E,k", [(1, 8, 1), (37, 8, 8), (100, 1024, 16), (5, 130, 7), (64, 64, 64)])
def test_route_topk_edges_and_ties(G, T, E, k):
    rng = np.random.default_rng(T * 1000 + E)
    logits = rng.integers(-2, 3, size=(T, E)).astype(np.float32)  # heavy ties
    logits[0, :] = 0.0
    ids, w = G.q.moe_route_topk(G.t(logits), k)
    ref_ids, ref_w = REF.route_topk(logits, k)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    np.testing.assert_allclose(w.cpu().numpy().astype(np.float64), ref_w, rtol=G.GATE_RTOL, atol=0)


# ----------------------------------------------------------------- grouping
def _perm_check(G, ids_np, E, bits_np=None):
    ids = G.t(ids_np.astype(np.int32))
    bits = G.t(bits_np.astype(np.uint8)) if bits_np is not None else None
    p = G.q.moe_permute(ids, E, pair_bits=bits)
    torch.cuda.synchronize()
    c, s, sp, pp = REF.permute(ids_np, E, bits_np)
    assert np.array_equal(p.counts.cpu().numpy(), c)
    assert np.array_equal(p.seg_offsets.cpu().numpy(), s)
    assert np.array_equal(p.sorted_pair.cpu().numpy(), sp)
    assert np.array_equal(p.pair_pos.cpu().numpy(), pp)
    assert int(p.workspace[:4].view(torch.int32).item()) == 0


@pytest.mark.parametrize("T,E,k", [(64, 8, 2), (32, 64, 8), (8192, 64, 8), (1, 4, 1), (300, 5, 5), (5000, 1024, 3)])
def test_permute_parity(G, T, E, k):
    rng = np.random.default_rng(T + E + k)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]) if T else np.zeros((0, k))
    _perm_check(G, ids, E)


def test_permute_skew_and_bits(G):
    rng = np.random.default_rng(9)
    ids = np.zeros((3000, 1), np.int64)                       # every pair on expert 0
    _perm_check(G, ids, 16)
    ids = np.stack([rng.permutation(8)[:2] for _ in range(9000)])
    bits = rng.integers(2, 5, size=18000)
    _perm_check(G, ids, 8, bits)                              # MWQ sub-keys, multi-block path
    _perm_check(G, ids[:512], 8, bits[:1024])                 # MWQ sub-keys, single workgroup


def test_permute_flags_invalid_ids(G):
    ids = np.array([[0, 1], [2, 7], [1, 3]], np.int32)
    p = G.q.moe_permute(G.t(ids), 4)
    torch.cuda.synchronize()
    assert int(p.workspace[:4].view(torch.int32).item()) != 0
    assert p.seg_offsets.cpu().numpy()[-1] == 5
    assert p.counts.cpu().numpy().sum() == 5


@pytest.mark.parametrize("ydt", [torch.float32, torch.float16, torch.bfloat16])
def test_combine_skips_invalid_pairs(G, ydt):
    """A pair whose id the grouping flagged (placed after every valid segment,
    where no GEMM writes) adds nothing to its token's output when the combine
    gets the number of valid rows; its row is never read (NaN there stays out).
    Expert outputs in fp32, fp16 or bf16."""
    ids = np.array([[0, 1], [2, 7], [1, 3]], np.int32)   # E = 4: pair 3 is invalid
    p = G.q.moe_permute(G.t(ids), 4)
    torch.cuda.synchronize()
    nv = int(p.seg_offsets.cpu().numpy()[-1])
    assert nv == 5
    rng = np.random.default_rng(3)
    y = rng.standard_normal((6, 16)).astype(np.float32)
    y[nv:] = np.nan
    w = np.array([[0.5, 0.5], [0.25, 0.75], [0.6, 0.4]], np.float32)
    yd = G.t(y).to(ydt)  # the values the combine sees: y rounded to the storage type
    out = G.q.moe_unpermute_combine(yd, p.pair_pos, G.t(w), 3, 2, n_valid=p.seg_offsets[-1:])
    torch.cuda.synchronize()
    got = G.bf16_to_np(out)
    pos = p.pair_pos.cpu().numpy()
    ys = yd.float().cpu().numpy().astype(np.float64)
    y0 = np.where(np.arange(6)[:, None] < nv, ys, 0.0)
    ref = oracle.unpermute_combine(y0, pos, w.astype(np.float64), 3, 2)
    assert np.isfinite(got).all()
    assert np.all(np.abs(got - ref) <= G.bf16_ulp(ref))   # fp32 sums, one bf16 rounding


@pytest.mark.parametrize("T,E,k,mwq", [(1, 8, 2, False), (16, 8, 2, True), (32, 64, 8, False), (64, 64, 8, True),
                                        (64, 64, 64, False),
                                        (65, 64, 4, True), (512, 8, 8, False), (513, 8, 8, False),
                                        (300, 128, 4, True)])
def test_route_permute_matches_oracle(G, T, E, k, mwq):
    """One-call routing + grouping: a single launch when E <= 64 and T*k <= 4096
    (the last workgroup groups), two launches otherwise; called twice on one
    workspace, so the arrival counter must come back to zero."""
    rng = np.random.default_rng(T * 31 + E + k)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[:, 3 % E] = logits[:, 1 % E]                      # exact ties
    bits = rng.integers(2, 5, size=T * k).astype(np.uint8) if mwq else None
    rid, rw = REF.route_topk(logits.astype(np.float64), k)
    counts, offsets, sorted_pair, pair_pos = REF.permute(rid, E, pair_bits=bits)
    p = None
    for _ in range(2):
        ids, w, p = G.q.moe_route_permute(G.t(logits), k, pair_bits=None if bits is None else G.t(bits), out=p)
        torch.cuda.synchronize()
        assert np.array_equal(ids.cpu().numpy(), rid)
        np.testing.assert_allclose(w.cpu().numpy().astype(np.float64), rw, rtol=G.GATE_RTOL, atol=0)
        assert np.array_equal(p.counts.cpu().numpy(), counts)
        assert np.array_equal(p.seg_offsets.cpu().numpy(), offsets)
        assert np.array_equal(p.sorted_pair.cpu().numpy(), sorted_pair)
        assert np.array_equal(p.pair_pos.cpu().numpy(), pair_pos)
        flag_and_counter = p.workspace[:8].view(torch.int32).cpu().numpy()
        assert flag_and_counter[0] == 0 and flag_and_counter[1] == 0


# --------------------------------------------------------------- full layers
def _layer_parity(G, cfg, tokens=None, kernel=0, d=None):
    d = gen.generate(cfg) if d is None else d
    buf = G.run_layer(d, cfg, kernel=kernel)
    ref = REF.moe_forward(d, cfg, tokens=tokens)
    assert np.array_equal(buf.ids.cpu().numpy(), ref["ids"])
    np.testing.assert_allclose(buf.w.cpu().numpy().astype(np.float64), ref["w"], rtol=G.GATE_RTOL, atol=0)
    assert np.array_equal(buf.perm.counts.cpu().numpy(), ref["counts"])
    assert np.array_equal(buf.perm.seg_offsets.cpu().numpy(), ref["seg_offsets"])
    assert np.array_equal(buf.perm.sorted_pair.cpu().numpy(), ref["sorted_pair"])
    assert np.array_equal(buf.perm.pair_pos.cpu().numpy(), ref["pair_pos"])
    sel = ref["tokens"]
    rows = ref["pair_pos"].reshape(cfg.T, cfg.k)[sel].ravel()
    # intermediates: diagnostics with a looser bar (the kernels round h to bf16)
    hm = oracle.compare(G.bf16_to_np(buf.h)[rows], ref["h_perm"][rows])
    ym = oracle.compare(G.bf16_to_np(buf.y_perm)[rows], ref["y_perm_h16"][rows])
    assert hm["rel_l2"] < 1e-2 and ym["rel_l2"] < 1e-2, (hm, ym)
    m = G.check_close(G.bf16_to_np(buf.out)[sel], ref["out"][sel], cfg.name)
    print(cfg.name, "h", hm, "y", ym, "out", m)
    return buf, ref


def test_layer_tiny_full(G):
    _layer_parity(G, gen.config("tiny"))


def test_layer_decode_full(G):
    _layer_parity(G, gen.config("olmoe_decode"))


def test_layer_empty_batch(G):
    """No tokens: every call takes the empty problem, and the grouping still writes
    zero counts and offsets."""
    cfg = gen.config("tiny")
    d = gen.generate(cfg)
    gu, dn = G.tiled_layer(d, cfg)
    x = torch.empty((0, cfg.H), dtype=torch.bfloat16, device="cuda:0")
    logits = torch.empty((0, cfg.E), dtype=torch.float32, device="cuda:0")
    buf = G.q.moe_layer_forward(x, logits, cfg.k, gu, dn)
    torch.cuda.synchronize()
    assert tuple(buf.out.shape) == (0, cfg.H)
    assert not buf.perm.counts.cpu().numpy().any()
    assert not buf.perm.seg_offsets.cpu().numpy().any()


@pytest.mark.parametrize("T", [1, 33, 97])
def test_layer_ragged_small(G, T):
    _layer_parity(G, gen.config("tiny", T=T, seed=7 + T))


def test_layer_g128_one_hot_expert(G):
    # every token routed to expert 3 (all other experts empty), G = 128
    cfg = gen.config("tiny", T=70, H=256, I=256, E=6, k=1, G=128, seed=77)
    d = gen.generate(cfg)
    d["logits"][:, 3] = 50.0
    buf = G.run_layer(d, cfg)
    ref = REF.moe_forward(d, cfg)
    G.check_close(G.bf16_to_np(buf.out), ref["out"], "one expert")
    G.check_ulp(G.bf16_to_np(buf.out), ref["out_h16"], "one expert")


def test_layer_k_equals_E(G):
    _layer_parity(G, gen.config("tiny", T=40, E=4, k=4, seed=5))


@pytest.mark.parametrize("name", ["olmoe_prefill", "olmoe_prefill_zipf"])
def test_layer_prefill_full(G, name):
    """The prefill-shaped layer (8192 tokens, 64 experts, top-8), uniform and
    Zipf-skewed routing, in the launch configuration the benchmark times:
    every token against the oracle."""
    _layer_parity(G, gen.config(name))


@pytest.mark.parametrize("over", [
    dict(T=300, E=4, k=2, H=256, I=512, G=64, seed=61),     # 2 scale groups per K block
    dict(T=200, E=6, k=2, H=384, I=384, G=32, seed=62),     # 4 groups; 3 K blocks; half-empty channel block
    dict(T=97, E=8, k=3, H=256, I=256, G=128, seed=63),     # ragged: about 36 rows per expert
    dict(T=64, E=2, k=1, H=128, I=128, G=128, seed=64),     # a single K block
    dict(T=150, E=5, k=2, H=1024, I=640, G=128, seed=65),   # 8 / 5 K blocks
])
def test_layer_prefill_dma_kernel(G, over):
    """The 128-row LDS-DMA kernel forced on small layers (it is chosen by
    itself for INT4 segments of about 96 rows and more)."""
    _layer_parity(G, gen.config("tiny", **over), kernel=G.q.MOE_KERNEL_LDS_DMA)


@pytest.mark.parametrize("kernel", ["SMALL", "TILE64_WIDE", "TILE64", "TILE128"])
def test_layer_int4_every_kernel(G, kernel):
    """Every INT4 kernel choice on one ragged layer (about 75 rows per expert:
    several row tiles of each size, a partial last tile per expert)."""
    cfg = gen.config("tiny", T=150, E=8, k=4, H=512, I=384, G=64, seed=66)
    _layer_parity(G, cfg, kernel=getattr(G.q, "MOE_KERNEL_" + kernel))


def test_layer_mwq_small_full(G):
    _layer_parity(G, gen.config("mixtral_mwq", T=96, H=512, I=1024, E=4, k=2, seed=41))


def test_layer_mwq_all_b4_equals_int4(G):
    """Nested planes at b = 4 everywhere give the INT4 path on the same codes."""
    cfg = gen.config("mixtral_mwq", T=64, H=256, I=512, E=4, k=2, seed=43)
    d = gen.generate(cfg)
    d["pair_bits"][:] = 4
    buf = G.run_layer(d, cfg)
    ref = REF.moe_forward(d, cfg)
    G.check_close(G.bf16_to_np(buf.out), ref["out"], "mwq b=4")


def test_layer_mwq_full_size(G):
    """The Mixtral-shaped nested-plane layer (512 tokens, 8 experts, top-2, H
    4096, I 14336) in the benchmark's launch configuration: every token."""
    _layer_parity(G, gen.config("mixtral_mwq"))


def test_layer_mwq_decode_full(G):
    """Nested planes at a decode batch (16 tokens): most bit-width segments hold
    one or two rows, and a segment loads only the planes its width needs."""
    _layer_parity(G, gen.config("mixtral_mwq_decode", H=1024, I=2048))   # a smaller layer
    _layer_parity(G, gen.config("mixtral_mwq_decode"))                    # full size, every token


@pytest.mark.parametrize("over", [
    dict(T=300, E=4, k=2, H=512, I=512, G=64, seed=81),    # ~150 rows per expert: two chunk groups each
    dict(T=200, E=3, k=2, H=512, I=384, G=32, seed=82),    # 4 scale groups per K block
    dict(T=150, E=8, k=4, H=512, I=256, G=128, seed=83),   # ~75 rows per expert, ragged chunks
    dict(T=64, E=2, k=2, H=128, I=128, G=128, seed=84),    # one K block: odd groups per channel, register scales
])
@pytest.mark.parametrize("kernel", ["LDS_DMA", "LDS_DMA_PER_WIDTH"])
def test_layer_mwq_prefill_dma_kernel(G, over, kernel):
    """Nested planes in the LDS-DMA kernel: 16-row chunks of every width, one
    expert per workgroup; or row tiles of one width each."""
    cfg = gen.config("mixtral_mwq", **over)
    buf, ref = _layer_parity(G, cfg, kernel=getattr(G.q, "MOE_KERNEL_" + kernel))
    G.check_ulp(G.bf16_to_np(buf.out), ref["out_h16"], str(over))


@pytest.mark.parametrize("bits", [2, 3, 4, "cycle"])
@pytest.mark.parametrize("kernel", ["LDS_DMA", "LDS_DMA_PER_WIDTH"])
def test_layer_mwq_prefill_widths(G, bits, kernel):
    """The LDS-DMA kernels with one width everywhere, or widths cycling per pair
    (chunks of every width in each workgroup, partial chunks at each end)."""
    cfg = gen.config("mixtral_mwq", T=150, E=3, k=2, H=512, I=1024, seed=85)
    d = gen.generate(cfg)
    if bits == "cycle":
        d["pair_bits"][:] = (4 - np.arange(d["pair_bits"].size) % 3).reshape(d["pair_bits"].shape)
    else:
        d["pair_bits"][:] = bits
    ref = REF.moe_forward(d, cfg)
    buf = G.run_layer(d, cfg, kernel=getattr(G.q, "MOE_KERNEL_" + kernel))
    assert np.array_equal(buf.perm.seg_offsets.cpu().numpy(), ref["seg_offsets"])
    out = G.bf16_to_np(buf.out)
    G.check_close(out, ref["out"], f"mwq prefill widths {bits}")
    G.check_ulp(out, ref["out_h16"], f"mwq prefill widths {bits}")


@pytest.mark.parametrize("bits", ["drawn", 2, 3, 4, "cycle"])
def test_layer_mwq_decode_widths(G, bits):
    """16-row tiles that take all widths of an expert at once: about 23 rows
    per expert, so tiles cross the b = 4 / 3 / 2 sub-segment boundaries; some
    widths absent; the one-width-per-tile kernel gives the same bits.  Besides
    the layer bar, every output is within one bf16 ulp of the exact value (plus
    5e-3 RMS, see check_ulp)."""
    cfg = gen.config("mixtral_mwq_decode", T=35, H=256, I=512, E=3, k=2, seed=47)
    d = gen.generate(cfg)
    if bits == "cycle":
        d["pair_bits"][:] = (4 - np.arange(d["pair_bits"].size) % 3).reshape(d["pair_bits"].shape)
    elif bits != "drawn":
        d["pair_bits"][:] = bits
    ref = REF.moe_forward(d, cfg)
    buf = G.run_layer(d, cfg)
    assert np.array_equal(buf.perm.seg_offsets.cpu().numpy(), ref["seg_offsets"])
    out_fused = G.bf16_to_np(buf.out)
    G.check_close(out_fused, ref["out"], f"mwq widths {bits}")
    G.check_ulp(out_fused, ref["out_h16"], f"mwq widths {bits}")
    out_split = G.bf16_to_np(G.run_layer(d, cfg, kernel=G.q.MOE_KERNEL_SMALL_PER_WIDTH).out)
    assert np.array_equal(out_fused, out_split)


@pytest.mark.parametrize("name,over", [
    ("tiny", dict(T=8, E=2, k=1, H=256, I=2048, G=128, seed=71)),          # INT4: down K 2048 -> 2 K splits
    ("mixtral_mwq_decode", dict(T=6, E=2, k=1, H=256, I=2048, seed=72)),  # nested planes, all widths per tile
])
def test_decode_split_k(G, name, over):
    """A decode batch's down projection with long K and few work items runs as
    K splits whose fp32 partial sums are added in order; the 16-bit plain
    epilogues through the same split are the fp32 result rounded once."""
    cfg = gen.config(name, **over)
    d = gen.generate(cfg)
    gu, dn = G.tiled_layer(d, cfg)
    buf = G.run_layer(d, cfg, gu, dn)
    ref = REF.moe_forward(d, cfg)
    assert np.array_equal(buf.perm.seg_offsets.cpu().numpy(), ref["seg_offsets"])
    assert oracle.compare(G.bf16_to_np(buf.y_perm), ref["y_perm_h16"])["rel_l2"] < 1e-2
    G.check_close(G.bf16_to_np(buf.out), ref["out"], name)
    M = cfg.T * cfg.k
    y32 = G.q.moe_grouped_qgemm(dn, buf.h, buf.perm.seg_offsets, M, G.q.MOE_EPI_NONE_F32)
    y16 = G.q.moe_grouped_qgemm(dn, buf.h, buf.perm.seg_offsets, M, G.q.MOE_EPI_NONE)
    torch.cuda.synchronize()
    assert torch.equal(y16, y32.to(torch.bfloat16))
    assert torch.equal(buf.y_perm, y32.to(torch.float16))


def _plain_epilogues(G, w, A, seg, M, kernel, **kw):
    """The same GEMM with fp32, fp16 and bf16 plain epilogues: each 16-bit
    output is the fp32 one rounded once (to nearest even)."""
    y32 = G.q.moe_grouped_qgemm(w, A, seg, M, G.q.MOE_EPI_NONE_F32, kernel=kernel, **kw)
    yh = G.q.moe_grouped_qgemm(w, A, seg, M, G.q.MOE_EPI_NONE_F16, kernel=kernel, **kw)
    yb = G.q.moe_grouped_qgemm(w, A, seg, M, G.q.MOE_EPI_NONE, kernel=kernel, **kw)
    torch.cuda.synchronize()
    assert yh.dtype == torch.float16 and torch.equal(yh, y32.to(torch.float16)), kernel
    assert torch.equal(yb.view(torch.bfloat16), y32.to(torch.bfloat16)), kernel


@pytest.mark.parametrize("fmt,kernels", [
    ("int4", ["SMALL", "TILE64_WIDE", "TILE64", "TILE128", "LDS_DMA"]),
    ("mwq", ["SMALL", "SMALL_PER_WIDTH", "TILE64", "LDS_DMA", "LDS_DMA_PER_WIDTH"]),
    ("mixed", ["SMALL"]),
    ("edge", ["SMALL"]),  # 8-bit experts: a decode launch of their own
])
def test_plain_epilogue_dtypes(G, fmt, kernels):
    """fp16 expert outputs (the layer's default) on every kernel of every
    format: bit for bit the fp32 outputs rounded once, like bf16."""
    name = {"int4": "tiny", "mwq": "mixtral_mwq", "mixed": "olmoe_mixed_decode", "edge": "olmoe_edge_decode"}[fmt]
    cfg = gen.config(name, T=150, E=4, k=2, H=256, I=512, seed=91)
    d = gen.generate(cfg)
    gu, dn = G.tiled_layer(d, cfg)
    buf = G.run_layer(d, cfg, gu, dn)
    M = cfg.T * cfg.k
    for kn in kernels:
        _plain_epilogues(G, dn, buf.h, buf.perm.seg_offsets, M, getattr(G.q, "MOE_KERNEL_" + kn))
        _plain_epilogues(G, gu, G.t(d["x"]), buf.perm.seg_offsets, M, getattr(G.q, "MOE_KERNEL_" + kn),
                         gather_pair=buf.perm.sorted_pair, k=cfg.k)


@pytest.mark.parametrize("kernel", ["SMALL", "LDS_DMA"])
def test_plain_epilogue_dtypes_delta(G, kernel):
    cfg = gen.config("meswitch_delta", requests=20, tokens_per_request=16, K=512, N=256, E=3, n_salient=5, seed=92)
    d = gen.generate(cfg)
    w = G.delta_layer(d, cfg)
    perm = G.q.moe_permute(G.t(d["ids"]).view(cfg.T, 1), cfg.E)
    _plain_epilogues(G, w, G.t(d["x"]), perm.seg_offsets, cfg.T, getattr(G.q, "MOE_KERNEL_" + kernel),
                     gather_pair=perm.sorted_pair, k=1)


# ------------------------------------------- static bit-width per expert
def test_layer_mixed_decode_full(G):
    """OLMoE decode batch with 4 / 3 / 2 bits by expert popularity (EdgeMoE
    expert-wise bit-width adaptation), every token."""
    _layer_parity(G, gen.config("olmoe_mixed_decode"))


def test_layer_edge_decode_full(G):
    """OLMoE decode batch with INT8 / INT4 / INT2 experts by popularity (the
    widths EdgeMoE names), every token."""
    buf, ref = _layer_parity(G, gen.config("olmoe_edge_decode"))
    G.check_ulp(G.bf16_to_np(buf.out), ref["out_h16"], "olmoe_edge_decode")


@pytest.mark.parametrize("over", [
    dict(T=50, E=5, k=2, H=256, I=512, G=128, bit_probs=(0, 0, 1), seed=98),   # every expert 8 bits
    dict(T=33, E=6, k=3, H=384, I=256, G=32, zipf=None, seed=99),             # 4 groups per K block, ragged
    dict(T=8, E=3, k=1, H=256, I=2048, G=64, bit_probs=(0, 0, 1), seed=100),  # down K 2048: split K
])
def test_layer_edge_widths(G, over):
    cfg = gen.config("olmoe_edge_decode", **over)
    buf, ref = _layer_parity(G, cfg)
    G.check_ulp(G.bf16_to_np(buf.out), ref["out_h16"], str(over))


@pytest.mark.parametrize("over", [
    dict(T=64, E=8, k=2, H=256, I=512, G=64, zipf=None, seed=91),        # widths in a seeded order
    dict(T=33, E=6, k=3, H=384, I=256, G=32, zipf=None, seed=92),        # 4 groups per K block, ragged
    dict(T=40, E=4, k=4, H=256, I=256, G=128, zipf=None, seed=93),       # k = E
    dict(T=8, E=3, k=1, H=256, I=2048, G=128, zipf=None, seed=94),       # down K 2048: split K
    dict(T=50, E=5, k=2, H=256, I=512, G=128, bit_probs=(1, 0, 0), seed=95),  # every expert 2 bits
    dict(T=50, E=5, k=2, H=256, I=512, G=128, bit_probs=(0, 1, 0), seed=96),  # every expert 3 bits
    dict(T=50, E=5, k=2, H=256, I=512, G=128, bit_probs=(0, 0, 1), seed=97),  # every expert 4 bits
])
def test_layer_mixed_widths(G, over):
    cfg = gen.config("olmoe_mixed_decode", **over)
    buf, ref = _layer_parity(G, cfg)
    G.check_ulp(G.bf16_to_np(buf.out), ref["out_h16"], str(over))


# ------------------------------------------------------------------- delta
def _delta_parity(G, cfg, tokens=None, kernel=0):
    d = gen.generate(cfg)
    perm, y_perm, out = G.run_delta(d, cfg, kernel=kernel)
    ref = REF.delta_linear(d, cfg, tokens=tokens)
    assert np.array_equal(perm.counts.cpu().numpy(), ref["counts"])
    assert np.array_equal(perm.sorted_pair.cpu().numpy(), ref["sorted_pair"])
    sel = np.arange(cfg.T) if tokens is None else np.asarray(tokens)
    m = G.check_close(G.bf16_to_np(out)[sel], ref["out"][sel], cfg.name)
    print(cfg.name, m)


def test_delta_small_full(G):
    _delta_parity(G, gen.config("meswitch_delta", requests=12, tokens_per_request=5, K=512, N=256, E=4,
                                n_salient=7, seed=9))


@pytest.mark.parametrize("over", [
    dict(requests=12, tokens_per_request=5, K=512, N=256, E=4, n_salient=7, seed=9),
    dict(requests=40, tokens_per_request=7, K=384, N=160, E=3, n_salient=40, seed=19),  # 3 K blocks, partial block, 2 salient steps
    dict(requests=20, tokens_per_request=16, K=256, N=128, E=2, n_salient=1, seed=29),
    dict(requests=10, tokens_per_request=13, K=128, N=128, E=2, n_salient=3, seed=39),  # one K block: prologue past the end
    dict(requests=9, tokens_per_request=16, K=1152, N=128, E=2, n_salient=5, seed=49),  # three steady passes, then two tail passes
])
def test_delta_dma_kernel(G, over):
    """The 128-row LDS-DMA delta kernel forced on small layers (it is chosen by
    itself for about 96 rows per expert and more)."""
    _delta_parity(G, gen.config("meswitch_delta", **over), kernel=G.q.MOE_KERNEL_LDS_DMA)


def test_delta_full_size(G):
    """The ME-Switch-shaped delta layer (4096 tokens, 16 experts, 4096 -> 14336)
    in the benchmark's launch configuration: every token."""
    _delta_parity(G, gen.config("meswitch_delta"))


# ---------------------------------------------------------- combine, determinism
def test_combine_round_trip(G):
    cfg = gen.config("tiny")
    d = gen.generate(cfg)
    x = G.t(d["x"])
    ids, w = G.q.moe_route_topk(G.t(d["logits"]), cfg.k)
    p = G.q.moe_permute(ids, cfg.E)
    x_perm = G.q.moe_permute(ids, cfg.E, x=x, want_x_perm=True).x_perm
    back = G.q.moe_unpermute_combine(x_perm, p.pair_pos, w, cfg.T, cfg.k)
    torch.cuda.synchronize()
    G.check_close(G.bf16_to_np(back), oracle.bf16_to_f64(d["x"]), "round trip")


def test_bitwise_deterministic(G):
    cfg = gen.config("olmoe_decode")
    d = gen.generate(cfg)
    gu, dn = G.tiled_layer(d, cfg)
    a = G.run_layer(d, cfg, gu, dn).out.clone()
    b = G.run_layer(d, cfg, gu, dn).out.clone()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))

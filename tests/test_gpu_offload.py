"""Host-resident experts with a GPU slot cache: every step equals the
all-resident layer bit for bit (same kernels, same rows) and meets the bar
against the oracle, through hits, misses and evictions."""
import numpy as np
import pytest
import torch

import gen
import oracle
from oracle import cpp as REF  # the C++17 float64 oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def G():
    from tests import gpu_helpers
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return gpu_helpers


@pytest.mark.parametrize("overlap", [True, False])
def test_offload_steps_match_resident_layer(G, overlap):
    from quantized_moe_expert_top_amd.offload import OffloadedMoeLayer
    cfg = gen.config("tiny", T=4, E=16, k=2, H=256, I=256, G=64, seed=121)
    d = gen.generate(cfg)
    gu, dn = G.tiled_layer(d, cfg)
    layer = OffloadedMoeLayer(gu, dn, n_slots=8)
    x = G.t(d["x"])
    seen = set()
    total_hits = 0
    for step, seed in enumerate([1, 2, 1, 3, 4, 4, 5]):
        logits = gen.config("tiny", T=4, E=16, k=2, H=256, I=256, G=64, seed=seed)
        dl = gen.generate(logits)["logits"]
        out, st = layer.forward(x, G.t(dl), cfg.k, overlap=overlap)
        torch.cuda.synchronize()
        ref_buf = G.q.moe_layer_forward(x, G.t(dl), cfg.k, gu, dn)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_buf.out), f"step {step}"
        d2 = dict(d)
        d2["logits"] = dl
        ref = REF.moe_forward(d2, cfg)
        G.check_close(G.bf16_to_np(out), ref["out"], f"offload step {step}")
        touched = set(int(e) for e in np.unique(ref["ids"]))
        assert st.experts == len(touched)
        assert st.hits <= len(touched & seen)
        seen |= touched
        total_hits += st.hits
    assert total_hits > 0                       # repeated routings find their experts resident
    assert len(seen) > layer.S                  # and the cache had to evict


def test_offload_rejects_more_experts_than_slots(G):
    from quantized_moe_expert_top_amd.offload import OffloadedMoeLayer
    cfg = gen.config("tiny", T=16, E=16, k=4, H=256, I=256, G=64, seed=122)
    d = gen.generate(cfg)
    gu, dn = G.tiled_layer(d, cfg)
    layer = OffloadedMoeLayer(gu, dn, n_slots=4)
    with pytest.raises(ValueError):
        layer.forward(G.t(d["x"]), G.t(d["logits"]), cfg.k)


def test_offload_lookahead_prefetch(G):
    """Routing known one batch ahead: the next batch's missing experts are copied
    during the current step, so later steps find them resident; outputs unchanged."""
    from quantized_moe_expert_top_amd.offload import OffloadedMoeLayer
    cfg = gen.config("tiny", T=4, E=16, k=2, H=256, I=256, G=64, seed=123)
    d = gen.generate(cfg)
    gu, dn = G.tiled_layer(d, cfg)
    layer = OffloadedMoeLayer(gu, dn, n_slots=12)
    x = G.t(d["x"])
    seeds = [1, 2, 3, 4, 5, 6]
    logits = [gen.generate(gen.config("tiny", T=4, E=16, k=2, H=256, I=256, G=64, seed=s))["logits"] for s in seeds]
    nxt = [REF.route_topk(lg, cfg.k)[0] for lg in logits]  # the pre-gate's ids, known ahead
    queued = 0
    for i, lg in enumerate(logits):
        out, st = layer.forward(x, G.t(lg), cfg.k)
        if i > 0:
            assert st.hits == st.experts, f"step {i}: the lookahead left {st.experts - st.hits} misses"
        if i + 1 < len(logits):
            queued += layer.prefetch(nxt[i + 1])
        torch.cuda.synchronize()
        ref_buf = G.q.moe_layer_forward(x, G.t(lg), cfg.k, gu, dn)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_buf.out), f"step {i}"
        ref = REF.moe_forward(dict(d, logits=lg), cfg)
        G.check_close(G.bf16_to_np(out), ref["out"], f"lookahead step {i}")
    assert queued > 0


def _steps_logits(T, E, sets, seed):
    """One logit batch per step: token t goes to expert sets[i][t % len(sets[i])]
    (logit 10 against N(0,1) elsewhere), so each step touches a chosen set."""
    rng = np.random.default_rng(seed)
    out = []
    for s in sets:
        lg = rng.standard_normal((T, E)).astype(np.float32)
        for t in range(T):
            lg[t, s[t % len(s)]] = 10.0
        out.append(lg)
    return out


def test_offload_split_k_down_keeps_earlier_rows(G):
    """A down projection long enough in K to split (I = 2048) on a decode batch,
    with hits and misses in the same step: the copied experts' GEMMs run on a
    slice of the offset table whose first entry is not zero, and must leave the
    resident experts' rows alone.  Every step equals the in-HBM layer bit for
    bit and meets the bar against the oracle."""
    from quantized_moe_expert_top_amd.offload import OffloadedMoeLayer
    cfg = gen.config("tiny", T=8, E=6, k=1, H=256, I=2048, G=128, seed=124)
    d = gen.generate(cfg)
    gu, dn = G.tiled_layer(d, cfg)
    ws = G.q.moe_grouped_qgemm_workspace_size(dn, cfg.T, cfg.T)
    assert ws > 0, "this shape must split K"
    layer = OffloadedMoeLayer(gu, dn, n_slots=4)
    x = G.t(d["x"])
    sets = [[0, 1, 2], [0, 1, 3], [2, 4, 5], [0, 3, 4], [1, 4]]
    for i, lg in enumerate(_steps_logits(cfg.T, cfg.E, sets, 7)):
        out, st = layer.forward(x, G.t(lg), cfg.k)
        torch.cuda.synchronize()
        if i > 0:
            assert 0 < st.hits < st.experts, f"step {i}: want hits and misses"
        ref_buf = G.q.moe_layer_forward(x, G.t(lg), cfg.k, gu, dn)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_buf.out), f"step {i}"
        d2 = dict(d, logits=lg)
        G.check_close(G.bf16_to_np(out), REF.moe_forward(d2, cfg)["out"], f"split-K offload step {i}")


def test_grouped_gemm_on_offset_slices(G):
    """The grouped GEMM on two slices of one offset table (keys e and E + e):
    each call writes only its own rows, including through split K, and the two
    together give the one-call result bit for bit."""
    cfg = gen.config("tiny", T=12, E=3, k=1, H=256, I=2048, G=128, seed=125)
    d = gen.generate(cfg)
    gu, dn = G.tiled_layer(d, cfg)
    ids_np = REF.route_topk(d["logits"], 1)[0].astype(np.int32)
    half = (np.arange(cfg.T) % 2).reshape(-1, 1).astype(np.int32)
    keys = G.t(ids_np + cfg.E * half)
    perm2 = G.q.moe_permute(keys, 2 * cfg.E)
    h = torch.randn((cfg.T, cfg.I), device="cuda:0").to(torch.bfloat16)
    y = torch.full((cfg.T, cfg.H), float("nan"), device="cuda:0")
    for part in (0, 1):
        seg = perm2.seg_offsets[part * cfg.E:part * cfg.E + cfg.E + 1]
        hp = h[perm2.sorted_pair.long()].contiguous()
        G.q.moe_grouped_qgemm(dn, hp, seg, cfg.T, G.q.MOE_EPI_NONE_F32, out=y)
    torch.cuda.synchronize()
    assert not torch.isnan(y).any()
    # one call over expert-only keys on the same rows
    perm1 = G.q.moe_permute(G.t(ids_np), cfg.E)
    y1 = G.q.moe_grouped_qgemm(dn, h[perm1.sorted_pair.long()].contiguous(), perm1.seg_offsets, cfg.T,
                               G.q.MOE_EPI_NONE_F32)
    torch.cuda.synchronize()
    assert torch.equal(y[perm2.pair_pos.long()], y1[perm1.pair_pos.long()])


# ------------------------------------------------------ nested MWQ planes, HEBF
def _mwq_step_data(seed, bits=None):
    c = gen.config("mixtral_mwq_decode", T=4, E=16, k=2, H=512, I=1024, seed=seed)
    dd = gen.generate(c)
    if bits is not None:
        dd["pair_bits"][:] = bits
    return dd


@pytest.mark.parametrize("overlap", [True, False])
def test_mwq_offload_hebf_steps_match_oracle(G, overlap):
    """Plane-wise loading in HEBF order: every step meets the bar against the
    oracle and agrees with the all-resident layer; hits, misses, evictions and
    slots that only gain planes (a width-2 expert later asked for 4 bits)."""
    from quantized_moe_expert_top_amd.offload import OffloadedMwqLayer
    cfg = gen.config("mixtral_mwq_decode", T=4, E=16, k=2, H=512, I=1024, seed=131)
    d = gen.generate(cfg)
    gu, dn = G.tiled_layer(d, cfg)
    layer = OffloadedMwqLayer(gu, dn, n_slots=8)
    x = G.t(d["x"])
    plane = {b: layer.gu.plane_bytes(b) + layer.dn.plane_bytes(b) for b in (2, 3, 4)}
    plan = [(132, 2), (132, 4), (132, 3), (133, None), (134, None), (132, None), (135, 4)]
    seen = set()
    for step, (seed, bits) in enumerate(plan):
        dd = _mwq_step_data(seed, bits)
        print(f"[gpu] mwq offload step {step} seed {seed} bits {bits} overlap {overlap}", flush=True)
        out, st = layer.forward(x, G.t(dd["logits"]), cfg.k, G.t(dd["pair_bits"]), overlap=overlap)
        torch.cuda.synchronize()
        d2 = dict(d)
        d2["logits"], d2["pair_bits"] = dd["logits"], dd["pair_bits"]
        ref = REF.moe_forward(d2, cfg)
        got = G.bf16_to_np(out)
        G.check_close(got, ref["out"], f"mwq offload step {step}")
        res = G.q.moe_layer_forward(x, G.t(dd["logits"]), cfg.k, gu, dn, pair_bits=G.t(dd["pair_bits"]))
        torch.cuda.synchronize()
        assert oracle.compare(got, G.bf16_to_np(res.out))["rel_l2"] < 2e-3
        touched = set(int(e) for e in np.unique(ref["ids"]))
        assert st.experts == len(touched)
        if step == 1:   # same routing, all pairs now 4 bits: every expert resident, d3 and d4 copied
            assert st.hits == len(touched) and st.bytes_copied == len(touched) * (plane[3] + plane[4])
        if step == 2:   # 3 bits: everything already there
            assert st.hits == len(touched) and st.bytes_copied == 0
        if step == 0:   # cold: q2 only
            assert st.hits == 0 and st.bytes_copied == len(touched) * plane[2]
        seen |= touched
    assert len(seen) > layer.S   # the cache had to evict

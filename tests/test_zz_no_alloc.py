"""The no-allocation grouped GEMM (static device scratch instead of a
workspace) against the workspace entry point: bit for bit on every kernel
that uses scratch (activation row sums of the 128-row LDS-DMA kernels,
split-K partial sums of decode-sized down projections), over two calls in a
row on the shared scratch, the second with a smaller input."""
import numpy as np
import pytest
import torch

import gen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def G():
    from tests import gpu_helpers
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return gpu_helpers


def _both(G, w, A, seg, M, epi, **kw):
    ref = G.q.moe_grouped_qgemm(w, A, seg, M, epi, **kw)
    got = G.q.moe_grouped_qgemm_noalloc(w, A, seg, M, epi, **kw)
    torch.cuda.synchronize()
    return ref, got


def _layer_calls(G, cfg, kernel):
    d = gen.generate(cfg)
    gu, dn = G.tiled_layer(d, cfg)
    x = G.t(d["x"])
    ids, w = G.q.moe_route_topk(G.t(d["logits"]), cfg.k)
    perm = G.q.moe_permute(ids, cfg.E)
    M = cfg.T * cfg.k
    assert G.q.moe_grouped_qgemm_workspace_size(dn, M, M, kernel) > 0, "the down call must use scratch"
    print(f"[gpu] no-alloc {cfg.name} T={cfg.T} E={cfg.E} k={cfg.k} kernel={kernel}", flush=True)
    h_ref, h = _both(G, gu, x, perm.seg_offsets, M, G.q.MOE_EPI_SWIGLU, gather_pair=perm.sorted_pair, k=cfg.k,
                     kernel=kernel)
    assert torch.equal(h_ref.view(torch.int16), h.view(torch.int16))
    for epi in (G.q.MOE_EPI_NONE_F32, G.q.MOE_EPI_NONE_F16):  # fp32 and fp16 expert outputs
        y_ref, y = _both(G, dn, h_ref, perm.seg_offsets, M, epi, kernel=kernel)
        assert torch.equal(y_ref, y)


@pytest.mark.parametrize("kernel_name,big,small", [
    # 128-row LDS-DMA kernel: row sums of the activations in the scratch
    ("LDS_DMA", dict(T=512, E=4, k=2, H=512, I=512, G=64, seed=131), dict(T=300, E=4, k=2, H=512, I=512, G=64, seed=132)),
    # decode-sized down projection with K = 2048: split-K partial sums in the scratch
    ("AUTO", dict(T=8, E=2, k=1, H=256, I=2048, G=128, seed=133), dict(T=4, E=2, k=1, H=256, I=2048, G=128, seed=134)),
])
def test_noalloc_matches_workspace_entry_point(G, kernel_name, big, small):
    kernel = getattr(G.q, "MOE_KERNEL_" + kernel_name)
    _layer_calls(G, gen.config("tiny", **big), kernel)
    _layer_calls(G, gen.config("tiny", **small), kernel)


def test_noalloc_delta_rowsums(G):
    """The delta layer's 128-row kernel keeps whole-K row sums in the scratch."""
    for over in (dict(requests=20, tokens_per_request=16, K=512, N=256, E=2, n_salient=5, seed=135),
                 dict(requests=9, tokens_per_request=16, K=384, N=128, E=2, n_salient=3, seed=136)):
        cfg = gen.config("meswitch_delta", **over)
        d = gen.generate(cfg)
        w = G.delta_layer(d, cfg)
        x = G.t(d["x"])
        perm = G.q.moe_permute(G.t(d["ids"]).view(cfg.T, 1), cfg.E)
        print(f"[gpu] no-alloc delta T={cfg.T}", flush=True)
        ref, got = _both(G, w, x, perm.seg_offsets, cfg.T, G.q.MOE_EPI_NONE, gather_pair=perm.sorted_pair, k=1,
                         kernel=G.q.MOE_KERNEL_LDS_DMA)
        assert torch.equal(ref.view(torch.int16), got.view(torch.int16))


def test_noalloc_refuses_more_than_its_scratch(G):
    """A call whose scratch need exceeds the static array is refused before launch."""
    cfg = gen.config("tiny", T=64, E=4, k=2, H=512, I=512, G=32, seed=137)
    d = gen.generate(cfg)
    gu, _ = G.tiled_layer(d, cfg)
    limit = G.q.lib().moe_grouped_qgemm_noalloc_scratch_bytes()
    rows = 1 << 18                     # row sums: rows x K/G x 4 bytes = 16 MiB
    assert G.q.moe_grouped_qgemm_workspace_size(gu, rows, rows, G.q.MOE_KERNEL_LDS_DMA) > limit
    A = torch.zeros((rows, cfg.H), dtype=torch.bfloat16, device="cuda:0")
    seg = torch.zeros(cfg.E + 1, dtype=torch.int32, device="cuda:0")
    out = torch.empty((rows, cfg.I), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(G.q.MoeError) as ei:
        G.q.moe_grouped_qgemm_noalloc(gu, A, seg, rows, G.q.MOE_EPI_SWIGLU, out=out, kernel=G.q.MOE_KERNEL_LDS_DMA)
    assert ei.value.status == 6
    assert np.isfinite(float(limit))

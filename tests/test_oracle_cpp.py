"""The two CPU oracles against each other: the C++17 one (oracle/moe_oracle.cpp,
std::thread, fixed summation order) and the numpy one are independent
implementations of the same float64 definition; on every format they agree to
rounding (1e-12 relative), and the C++ one gives the same bits at any thread
count."""
import numpy as np
import pytest

import gen
import oracle
from oracle import cpp

CASES = [
    ("tiny", {}),
    ("tiny", dict(T=37, E=6, k=3, H=384, I=256, G=32, seed=3)),
    ("mixtral_mwq", dict(T=96, H=512, I=1024, E=4, k=2, seed=41)),
    ("mixtral_mwq_decode", dict(T=9, H=256, I=512, E=3, k=2, seed=47)),
    ("olmoe_mixed_decode", dict(T=33, E=6, k=3, H=384, I=256, G=32, zipf=None, seed=92)),
    ("olmoe_mixed_decode", dict(T=20, E=8, k=2, H=256, I=512, G=64, seed=93)),
]


def _rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


@pytest.mark.parametrize("name,over", CASES)
def test_cpp_oracle_matches_numpy_oracle(name, over):
    cfg = gen.config(name, **over)
    d = gen.generate(cfg)
    a = oracle.moe_forward(d, cfg)
    b = cpp.moe_forward(d, cfg)
    for key in ("ids", "counts", "seg_offsets", "sorted_pair", "pair_pos"):
        assert np.array_equal(a[key], b[key]), key
    np.testing.assert_allclose(b["w"], a["w"], rtol=1e-14, atol=0)
    for key in ("h_perm", "y_perm", "y_perm_h16", "out", "out_h16"):
        assert _rel(b[key], a[key]) < 1e-12, key


def test_cpp_oracle_token_subset_and_threads():
    cfg = gen.config("mixtral_mwq", T=64, H=256, I=512, E=4, k=2, seed=44)
    d = gen.generate(cfg)
    one = cpp.moe_forward(d, cfg, threads=1)
    many = cpp.moe_forward(d, cfg, threads=7)
    assert np.array_equal(one["out"], many["out"]) and np.array_equal(one["out_h16"], many["out_h16"])
    sub = cpp.moe_forward(d, cfg, tokens=[0, 17, 63], threads=3)
    assert np.array_equal(sub["out"][[0, 17, 63]], one["out"][[0, 17, 63]])
    assert np.isnan(sub["out"][1]).all()


def test_cpp_delta_matches_numpy_delta():
    for over in (dict(requests=12, tokens_per_request=5, K=512, N=256, E=4, n_salient=7, seed=9),
                 dict(requests=30, tokens_per_request=3, K=384, N=160, E=3, n_salient=40, seed=19)):
        cfg = gen.config("meswitch_delta", **over)
        d = gen.generate(cfg)
        a = oracle.delta_linear(d, cfg)
        b = cpp.delta_linear(d, cfg, threads=5)
        assert np.array_equal(a["sorted_pair"], b["sorted_pair"])
        assert _rel(b["out"], a["out"]) < 1e-12


def test_cpp_oracle_rejects_bad_input():
    with pytest.raises(ValueError):
        cpp.route_topk(np.zeros((2, 4), np.float32), 5)
    with pytest.raises(ValueError):
        cpp.route_topk(np.array([[0, np.nan]], np.float32), 1)
    with pytest.raises(ValueError):
        cpp.permute(np.array([[0, 9]]), 8)
    with pytest.raises(ValueError):
        cpp.permute(np.array([[0, 1]]), 8, pair_bits=np.array([4, 5], np.uint8))

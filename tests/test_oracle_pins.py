"""Pins for the CPU oracles (numpy, and C++17 in oracle/moe_oracle.cpp): checks
against facts the pages and plain mathematics fix, written independently of
the oracles' own code (brute force over subsets, pure-Python packing and dense
evaluation, closed forms, invariants).  Layer-level pins run on both."""
import itertools
import json
import math
import os
import random

import numpy as np
import pytest

import gen
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(params=["numpy", "cpp"])
def impl(request):
    """Each pin runs on both oracle implementations: the numpy one and the C++17 one."""
    if request.param == "numpy":
        return oracle
    from oracle import cpp
    return cpp


# ----------------------------------------------------------- pure-Python helpers
def pack_nibbles(codes_row):
    """list of 4-bit ints -> bytes, even index in the low nibble."""
    return [codes_row[i] | (codes_row[i + 1] << 4) for i in range(0, len(codes_row), 2)]


def pack_2bit(fields):
    out = []
    for i in range(0, len(fields), 4):
        out.append(fields[i] | (fields[i + 1] << 2) | (fields[i + 2] << 4) | (fields[i + 3] << 6))
    return out


def pack_1bit(bits):
    out = []
    for i in range(0, len(bits), 8):
        v = 0
        for j in range(8):
            v |= bits[i + j] << j
        out.append(v)
    return out


def f16(v):
    return int(np.array(v, dtype=np.float16).view(np.uint16))


def f16_val(bits):
    return float(np.array(bits, dtype=np.uint16).view(np.float16))


def bf16_val(bits):
    return float(np.array([bits << 16], dtype=np.uint32).view(np.float32)[0])


def py_silu(g):
    return g / (1.0 + math.exp(-g))


def py_bf16(v):
    """Nearest number with 8 significant bits (ties to even), pure Python."""
    if v == 0.0:
        return 0.0
    m, e = math.frexp(v)
    return math.ldexp(round(m * 256.0), e - 8)   # round(): half to even


def py_ffn(x, wgu, wd, I, h16=False):
    """Textbook SwiGLU on Python lists: wgu[n][k] (2I x H), wd[m][n] (H x I).
    With h16 the activation h entering the down projection is first rounded to
    bf16 (the oracle's diagnostic 16-bit-activation variant)."""
    H = len(x)
    g = [sum(x[kk] * wgu[n][kk] for kk in range(H)) for n in range(I)]
    u = [sum(x[kk] * wgu[I + n][kk] for kk in range(H)) for n in range(I)]
    h = [py_silu(g[n]) * u[n] for n in range(I)]
    if h16:
        h = [py_bf16(v) for v in h]
    return [sum(h[n] * wd[m][n] for n in range(I)) for m in range(H)]


def rel_err(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


# --------------------------------------------------------------------- routing
def _brute_topk_set(row, k):
    """The unique k-subset whose every member beats every non-member
    (larger logit, or equal logit and lower index)."""
    E = len(row)
    found = []
    for S in itertools.combinations(range(E), k):
        rest = [j for j in range(E) if j not in S]
        if all(row[i] > row[j] or (row[i] == row[j] and i < j) for i in S for j in rest):
            found.append(set(S))
    assert len(found) == 1
    return found[0]


@pytest.mark.parametrize("k", [1, 2, 3, 8])
@pytest.mark.parametrize("ties", [False, True])
def test_route_matches_bruteforce_subsets(k, ties, impl):
    rng = np.random.default_rng(7 + k)
    if ties:
        logits = rng.integers(0, 3, size=(40, 8)).astype(np.float32)
    else:
        logits = gen.gen_moe_int4(gen.config("tiny"))["logits"][:40]
    ids, w = impl.route_topk(logits, k)
    for t in range(logits.shape[0]):
        row = [float(v) for v in logits[t]]
        assert set(ids[t].tolist()) == _brute_topk_set(row, k)
        for j in range(k - 1):  # slot order: descending, ties -> lower index
            a, b = ids[t][j], ids[t][j + 1]
            assert row[a] > row[b] or (row[a] == row[b] and a < b)


def test_gates_closed_form(impl):
    logits = gen.gen_moe_int4(gen.config("olmoe_decode"))["logits"]
    ids, w = impl.route_topk(logits, 8)
    for t in range(logits.shape[0]):
        sel = [float(logits[t][e]) for e in ids[t]]
        assert abs(sum(w[t]) - 1.0) < 1e-14
        for i in range(8):
            for j in range(8):
                assert abs(w[t][i] / w[t][j] - math.exp(sel[i] - sel[j])) < 1e-12 * math.exp(sel[i] - sel[j])
    _, w1 = impl.route_topk(logits, 1)
    assert np.all(w1 == 1.0)


def test_route_rejects_bad_k_and_nonfinite(impl):
    with pytest.raises(ValueError):
        impl.route_topk(np.zeros((2, 4), np.float32), 5)
    with pytest.raises(ValueError):
        impl.route_topk(np.array([[0, np.nan]], np.float32), 1)


def test_golden_route_permute_hand_example(impl):
    """Hand-worked routing + grouping example (derivation in the fixture)."""
    with open(os.path.join(GOLDEN, "route_permute_hand.json")) as f:
        g = json.load(f)
    logits = np.array(g["logits"], dtype=np.float32)
    ids, w = impl.route_topk(logits, g["k"])
    assert ids.tolist() == g["ids"]
    np.testing.assert_allclose(w, np.array(g["w"]), rtol=1e-15, atol=0)
    counts, seg, sp, pp = impl.permute(ids, g["E"])
    assert counts.tolist() == g["counts"]
    assert seg.tolist() == g["seg_offsets"]
    assert sp.tolist() == g["sorted_pair"]
    assert pp.tolist() == g["pair_pos"]
    counts, seg, sp, pp = impl.permute(ids, g["E"], np.array(g["mwq_bits"], np.uint8))
    assert seg.tolist() == g["mwq_seg_offsets"]
    assert sp.tolist() == g["mwq_sorted_pair"]


# --------------------------------------------------------------------- grouping
def _check_permutation(ids, E, bits=None, impl=oracle):
    P = ids.size
    counts, seg, sp, pp = impl.permute(ids, E, bits)
    S = 1 if bits is None else 3
    flat = [int(v) for v in ids.ravel()]
    keys = [flat[p] * S + (0 if bits is None else 4 - int(bits.ravel()[p])) for p in range(P)]
    # counts and offsets by explicit counting
    for e in range(E):
        assert counts[e] == sum(1 for v in flat if v == e)
    assert int(counts.sum()) == P
    acc = 0
    for key in range(E * S):
        assert seg[key] == acc
        acc += sum(1 for v in keys if v == key)
    assert seg[E * S] == P
    # bijection + ascending (key, pair) order
    assert sorted(sp.tolist()) == list(range(P))
    for i in range(P):
        assert pp[sp[i]] == i
    for i in range(P - 1):
        assert (keys[sp[i]], sp[i]) < (keys[sp[i + 1]], sp[i + 1])
    for key in range(E * S):
        for i in range(seg[key], seg[key + 1]):
            assert keys[sp[i]] == key
    return counts, seg, sp, pp


def test_permute_invariants_random_and_edges(impl):
    rng = np.random.default_rng(3)
    _check_permutation(rng.integers(0, 8, size=(50, 2)), 8, impl=impl)
    _check_permutation(np.zeros((17, 1), np.int64), 5, impl=impl)            # all on one expert, others empty
    _check_permutation(np.tile(np.arange(6), (9, 1)), 6, impl=impl)           # k = E
    _check_permutation(np.zeros((0, 2), np.int64), 4, impl=impl)              # no tokens
    bits = rng.integers(2, 5, size=60).astype(np.uint8)
    _check_permutation(rng.integers(0, 8, size=(30, 2)), 8, bits, impl=impl)  # MWQ sub-keys
    with pytest.raises(ValueError):
        impl.permute(np.array([[0, 9]]), 8)


def test_permute_unpermute_round_trip():
    """Gathering x rows into grouped order and combining them back with gates
    that sum to one returns x (the combine undoes the grouping)."""
    cfg = gen.config("tiny")
    d = gen.gen_moe_int4(cfg)
    x = oracle.bf16_to_f64(d["x"])
    ids, w = oracle.route_topk(d["logits"], cfg.k)
    _, _, sp, pp = oracle.permute(ids, cfg.E)
    x_perm = x[sp // cfg.k]
    back = oracle.unpermute_combine(x_perm, pp, w, cfg.T, cfg.k)
    assert np.max(np.abs(back - x)) < 1e-14 * np.max(np.abs(x)) * 4


# ---------------------------------------------------------------------- formats
def test_int4_unpack_and_dequant_against_python_packing():
    rnd = random.Random(11)
    N, K, G = 6, 16, 4
    codes = [[rnd.randrange(16) for _ in range(K)] for _ in range(N)]
    scales = [[f16(0.001 * (1 + n) * (1 + 7 * g)) for g in range(K // G)] for n in range(N)]
    packed = np.array([pack_nibbles(r) for r in codes], np.uint8)
    W = oracle.dequant_int4(packed, np.array(scales, np.uint16), G)
    for n in range(N):
        for kk in range(K):
            assert W[n][kk] == f16_val(scales[n][kk // G]) * (codes[n][kk] - 8)
    # all-8 codes are zero weights
    assert np.all(oracle.dequant_int4(np.full((3, 8), 0x88, np.uint8), np.full((3, 4), f16(0.5), np.uint16), 4) == 0)


def test_int4_one_hot_probe_returns_weight_row():
    """x = e_i through x W^T returns column i of the dequantised matrix."""
    rnd = random.Random(5)
    N, K, G = 4, 8, 2
    codes = [[rnd.randrange(16) for _ in range(K)] for _ in range(N)]
    scales = np.array([[f16(0.25 * (g + 1) + n) for g in range(K // G)] for n in range(N)], np.uint16)
    W = oracle.dequant_int4(np.array([pack_nibbles(r) for r in codes], np.uint8), scales, G)
    for i in range(K):
        x = np.zeros(K)
        x[i] = 1.0
        y = x @ W.T
        assert y.tolist() == [f16_val(scales[n][i // G]) * (codes[n][i] - 8) for n in range(N)]


def _mwq_planes_from_codes(codes):
    q2 = [[c >> 2 for c in row] for row in codes]
    d3 = [[(c >> 1) & 1 for c in row] for row in codes]
    d4 = [[c & 1 for c in row] for row in codes]
    return (np.array([pack_2bit(r) for r in q2], np.uint8),
            np.array([pack_1bit(r) for r in d3], np.uint8),
            np.array([pack_1bit(r) for r in d4], np.uint8))


def test_mwq_nested_identity_and_subset_chain():
    """W(4) = Q2 + D3 + D4 reproduces the stored 4-bit code exactly; W(3), W(2)
    are its top 3 / 2 bits (INT2 c INT3 c INT4)."""
    rnd = random.Random(23)
    N, K, G = 5, 32, 8
    codes = [[rnd.randrange(16) for _ in range(K)] for _ in range(N)]
    q2, d3, d4 = _mwq_planes_from_codes(codes)
    scales = np.array([[f16(0.01 * (n + 1) + 0.003 * g) for g in range(K // G)] for n in range(N)], np.uint16)
    w_int4 = oracle.dequant_int4(np.array([pack_nibbles(r) for r in codes], np.uint8), scales, G)
    assert np.array_equal(oracle.dequant_mwq(q2, d3, d4, scales, G, 4), w_int4)
    u2, u1a, u1b = oracle.unpack_u2(q2), oracle.unpack_u1(d3), oracle.unpack_u1(d4)
    for b, mask in ((4, 0b1111), (3, 0b1110), (2, 0b1100)):
        cb = oracle.mwq_code(u2, u1a, u1b, b)
        W = oracle.dequant_mwq(q2, d3, d4, scales, G, b)
        for n in range(N):
            for kk in range(K):
                c = codes[n][kk]
                assert cb[n][kk] == c & mask
                assert 0 <= c - cb[n][kk] < 2 ** (4 - b)
                assert W[n][kk] == f16_val(scales[n][kk // G]) * ((c & mask) - 8)


def test_mwq_storage_equals_int4_storage():
    """The nested form stores no extra copy: q2 + d3 + d4 bytes == INT4 bytes
    (D2MoE, MWQ: higher precisions add residual bits, not copies)."""
    cfg = gen.config("mixtral_mwq")
    H, I, G = cfg.H, cfg.I, cfg.G
    per_matrix = lambda n, k: n * k // 4 + 2 * (n * k // 8)  # noqa: E731
    int4 = lambda n, k: n * k // 2  # noqa: E731
    mwq_b = per_matrix(2 * I, H) + per_matrix(H, I)
    int4_b = int4(2 * I, H) + int4(H, I)
    assert mwq_b == int4_b
    scales = (2 * I * H // G + H * I // G) * 2
    assert mwq_b + scales == 90_832_896
    d = gen.gen_moe_mwq(gen.config("mixtral_mwq", T=4, H=256, I=512))
    assert d["gu_q2"][0].nbytes + d["gu_d3"][0].nbytes + d["gu_d4"][0].nbytes == 2 * 512 * 256 // 2


def test_delta2_special_cases():
    rnd = random.Random(31)
    N, K, S = 4, 16, 3
    codes = [[rnd.randrange(4) for _ in range(K)] for _ in range(N)]
    step = np.array([f16(0.001 * (n + 1)) for n in range(N)], np.uint16)
    sal = np.array([2, 7, 11], np.int32)
    sval = np.array([[(0x3F80 + 0x10 * s + n) for n in range(N)] for s in range(S)], np.uint16)
    D = oracle.dequant_delta2(np.array([pack_2bit(r) for r in codes], np.uint8), step, sal, sval)
    for n in range(N):
        for kk in range(K):
            if kk in sal.tolist():
                assert D[n][kk] == bf16_val(int(sval[sal.tolist().index(kk)][n]))
            else:
                assert D[n][kk] == f16_val(int(step[n])) * (codes[n][kk] - 2)
    # codes under salient channels are ignored
    codes2 = [list(r) for r in codes]
    for r in codes2:
        for kk in sal.tolist():
            r[kk] = 3 - r[kk]
    D2 = oracle.dequant_delta2(np.array([pack_2bit(r) for r in codes2], np.uint8), step, sal, sval)
    assert np.array_equal(D, D2)


def test_delta_linear_reductions(impl):
    """codes all 2 and salient values 0 => y = x W_base^T; zero base with a
    one-hot x on a salient channel returns that salient row, on another
    channel step * (c - 2)."""
    cfg = gen.config("meswitch_delta", requests=3, tokens_per_request=2, K=32, N=8, E=2, n_salient=2)
    d = gen.gen_delta_linear(cfg)
    x = oracle.bf16_to_f64(d["x"])
    base = oracle.bf16_to_f64(d["base"])
    d0 = dict(d, codes=np.full_like(d["codes"], 0xAA), salient_val=np.zeros_like(d["salient_val"]))
    y = impl.delta_linear(d0, cfg)["out"]
    ref = [[sum(x[t][kk] * base[n][kk] for kk in range(cfg.K)) for n in range(cfg.N)] for t in range(cfg.T)]
    assert rel_err(y, ref) < 1e-13
    e = int(d["ids"][0])
    for ch in (int(d["salient_idx"][e][0]), next(c for c in range(cfg.K) if c not in d["salient_idx"][e])):
        xb = np.zeros_like(d["x"])
        xb[0, ch] = 0x3F80  # 1.0
        d1 = dict(d, x=xb, base=np.zeros_like(d["base"]))
        y = impl.delta_linear(d1, cfg, tokens=[0])["out"][0]
        if ch in d["salient_idx"][e]:
            s = list(d["salient_idx"][e]).index(ch)
            expect = [bf16_val(int(v)) for v in d["salient_val"][e][s]]
        else:
            c = [(int(d["codes"][e][n][ch // 4]) >> (2 * (ch % 4))) & 3 for n in range(cfg.N)]
            expect = [f16_val(int(d["step"][e][n])) * (c[n] - 2) for n in range(cfg.N)]
        assert y.tolist() == expect


def test_delta_linear_matches_dense_bruteforce_several_experts(impl):
    """y[t] = x[t] (W_base + D_{e(t)})^T evaluated densely in pure Python, per
    token with its own expert (ME-Switch: expert weight = shared base + its
    delta), against the grouped oracle: three experts, tokens on each, base
    and deltas non-zero."""
    cfg = gen.config("meswitch_delta", requests=6, tokens_per_request=2, K=32, N=8, E=3, n_salient=2, seed=13)
    d = gen.gen_delta_linear(cfg)
    d["ids"] = np.array([0, 2, 1, 1, 2, 0, 0, 1, 2, 2, 1, 0], np.int32)
    res = impl.delta_linear(d, cfg)
    x = [[bf16_val(int(v)) for v in row] for row in d["x"]]
    base = [[bf16_val(int(v)) for v in row] for row in d["base"]]

    def delta(e, n, kk):
        sal = [int(v) for v in d["salient_idx"][e]]
        if kk in sal:
            return bf16_val(int(d["salient_val"][e][sal.index(kk)][n]))
        c = (int(d["codes"][e][n][kk // 4]) >> (2 * (kk % 4))) & 3
        return f16_val(int(d["step"][e][n])) * (c - 2)

    for t in range(cfg.T):
        e = int(d["ids"][t])
        want = [sum(x[t][kk] * (base[n][kk] + delta(e, n, kk)) for kk in range(cfg.K)) for n in range(cfg.N)]
        assert rel_err(res["out"][t], want) < 1e-12
        # another expert's delta gives a visibly different row (the check can tell experts apart)
        other = (e + 1) % cfg.E
        alt = [sum(x[t][kk] * (base[n][kk] + delta(other, n, kk)) for kk in range(cfg.K)) for n in range(cfg.N)]
        assert rel_err(alt, want) > 1e-4
    assert sorted(set(d["ids"].tolist())) == [0, 1, 2]


def test_unpack_2bit_against_python_packing():
    rnd = random.Random(2)
    fields = [rnd.randrange(4) for _ in range(64)]
    assert oracle.unpack_u2(np.array(pack_2bit(fields), np.uint8)).tolist() == fields
    bits = [rnd.randrange(2) for _ in range(64)]
    assert oracle.unpack_u1(np.array(pack_1bit(bits), np.uint8)).tolist() == bits
    nib = [rnd.randrange(16) for _ in range(64)]
    assert oracle.unpack_u4(np.array(pack_nibbles(nib), np.uint8)).tolist() == nib


# ---------------------------------------------------------- expert FFN + combine
def _py_dequant_int4(packed_row_bytes, scale_bits, G):
    codes = []
    for byte in packed_row_bytes:
        codes += [int(byte) & 15, int(byte) >> 4]
    return [f16_val(int(scale_bits[kk // G])) * (codes[kk] - 8) for kk in range(len(codes))]


def test_moe_forward_matches_dense_bruteforce_int4(impl):
    """Per token: sum_j w_j * FFN_{e_j}(x_t), evaluated densely in pure Python
    (no grouping), equals the grouped oracle path."""
    cfg = gen.config("tiny", T=6, H=8, I=4, E=3, k=2, G=4)
    d = gen.gen_moe_int4(cfg)
    res = impl.moe_forward(d, cfg)
    x = [[bf16_val(int(v)) for v in row] for row in d["x"]]
    for t in range(cfg.T):
        row = [float(v) for v in d["logits"][t]]
        order = sorted(range(cfg.E), key=lambda e: (-row[e], e))[:cfg.k]
        ex = [math.exp(row[e] - row[order[0]]) for e in order]
        gates = [v / sum(ex) for v in ex]
        acc, acc16 = [0.0] * cfg.H, [0.0] * cfg.H
        for j, e in enumerate(order):
            wgu = [_py_dequant_int4(d["gu_codes"][e][n], d["gu_scales"][e][n], cfg.G) for n in range(2 * cfg.I)]
            wd = [_py_dequant_int4(d["dn_codes"][e][m], d["dn_scales"][e][m], cfg.G) for m in range(cfg.H)]
            y = py_ffn(x[t], wgu, wd, cfg.I)
            y16 = py_ffn(x[t], wgu, wd, cfg.I, h16=True)
            acc = [a + gates[j] * v for a, v in zip(acc, y)]
            acc16 = [a + gates[j] * v for a, v in zip(acc16, y16)]
        assert rel_err(res["out"][t], acc) < 1e-12
        assert rel_err(res["out_h16"][t], acc16) < 1e-12
        assert rel_err(res["out_h16"][t], acc) > 1e-6   # the bf16 rounding of h is visible


def test_moe_forward_k1_identical_experts_is_dense_ffn(impl):
    """k = 1 with every expert identical and gate 1: the layer is one plain
    dense SwiGLU FFN on every token."""
    cfg = gen.config("tiny", T=5, H=8, I=4, E=4, k=1, G=4)
    d = gen.gen_moe_int4(cfg)
    for key in ("gu_codes", "gu_scales", "dn_codes", "dn_scales"):
        d[key] = np.repeat(d[key][:1], cfg.E, axis=0)
    res = impl.moe_forward(d, cfg)
    wgu = [_py_dequant_int4(d["gu_codes"][0][n], d["gu_scales"][0][n], cfg.G) for n in range(2 * cfg.I)]
    wd = [_py_dequant_int4(d["dn_codes"][0][m], d["dn_scales"][0][m], cfg.G) for m in range(cfg.H)]
    for t in range(cfg.T):
        xt = [bf16_val(int(v)) for v in d["x"][t]]
        assert rel_err(res["out"][t], py_ffn(xt, wgu, wd, cfg.I)) < 1e-12
        assert rel_err(res["out_h16"][t], py_ffn(xt, wgu, wd, cfg.I, h16=True)) < 1e-12


def test_moe_forward_matches_dense_bruteforce_mwq(impl):
    cfg = gen.config("mixtral_mwq", T=6, H=16, I=8, E=3, k=2, G=8)
    d = gen.gen_moe_mwq(cfg)
    res = impl.moe_forward(d, cfg)
    for t in range(cfg.T):
        xt = [bf16_val(int(v)) for v in d["x"][t]]
        row = [float(v) for v in d["logits"][t]]
        order = sorted(range(cfg.E), key=lambda e: (-row[e], e))[:cfg.k]
        ex = [math.exp(row[e] - row[order[0]]) for e in order]
        acc, acc16 = [0.0] * cfg.H, [0.0] * cfg.H
        for j, e in enumerate(order):
            b = int(d["pair_bits"][t * cfg.k + j])
            mask = {4: 15, 3: 14, 2: 12}[b]

            def mat(prefix, n_rows, kdim):
                rows = []
                for n in range(n_rows):
                    q2 = oracle.unpack_u2(d[prefix + "q2"][e][n])
                    d3 = oracle.unpack_u1(d[prefix + "d3"][e][n])
                    d4 = oracle.unpack_u1(d[prefix + "d4"][e][n])
                    full = [int(4 * q2[i] + 2 * d3[i] + d4[i]) for i in range(kdim)]
                    rows.append([f16_val(int(d[prefix + "scales"][e][n][i // cfg.G])) * ((full[i] & mask) - 8)
                                 for i in range(kdim)])
                return rows
            wgu, wd = mat("gu_", 2 * cfg.I, cfg.H), mat("dn_", cfg.H, cfg.I)
            y = py_ffn(xt, wgu, wd, cfg.I)
            y16 = py_ffn(xt, wgu, wd, cfg.I, h16=True)
            acc = [a + ex[j] / sum(ex) * v for a, v in zip(acc, y)]
            acc16 = [a + ex[j] / sum(ex) * v for a, v in zip(acc16, y16)]
        assert rel_err(res["out"][t], acc) < 1e-12
        assert rel_err(res["out_h16"][t], acc16) < 1e-12


def test_moe_forward_token_subset_matches_full(impl):
    cfg = gen.config("tiny")
    d = gen.gen_moe_int4(cfg)
    full = impl.moe_forward(d, cfg)
    sub = impl.moe_forward(d, cfg, tokens=[0, 5, 63])
    assert rel_err(sub["out"][[0, 5, 63]], full["out"][[0, 5, 63]]) < 1e-14
    assert np.isnan(sub["out"][1]).all()


def test_compare_metric():
    r = np.array([3.0, 4.0])
    m = oracle.compare(r + np.array([0.03, 0.0]), r)
    assert abs(m["rel_l2"] - 0.03 / 5.0) < 1e-15
    assert abs(m["max_abs_over_rms"] - 0.03 / math.sqrt(12.5)) < 1e-15


def test_round_bf16_pins():
    """bf16 keeps 8 significant bits; ties go to the even neighbour."""
    one = 1.0
    assert oracle.round_bf16(one + 2.0 ** -8) == one                   # tie -> even (1.0)
    assert oracle.round_bf16(one + 3 * 2.0 ** -8) == one + 2.0 ** -6   # tie -> even (1 + 2^-6)
    assert oracle.round_bf16(one + 2.0 ** -8 + 2.0 ** -30) == one + 2.0 ** -7
    assert oracle.round_bf16(-3.0) == -3.0 and oracle.round_bf16(0.0) == 0.0
    assert oracle.round_bf16(255.0) == 255.0 and oracle.round_bf16(257.0) == 256.0
    # float32 inputs: agrees with the bit-level float32 -> bf16 conversion of the generator
    v = np.random.default_rng(4).standard_normal(20000).astype(np.float32) * 7
    bits = gen.f32_to_bf16_bits(v)
    assert np.array_equal(oracle.round_bf16(v.astype(np.float64)), gen.bf16_bits_to_f32(bits).astype(np.float64))
    for x in v[:200]:
        assert oracle.round_bf16(float(x)) == py_bf16(float(x))


# ------------------------------------------------- static bit-width per expert
def _py_bitstream(codes, b):
    """Pure-Python little-endian packing of b-bit codes (code k at bits k*b ..)."""
    acc, nbits, out = 0, 0, []
    for c in codes:
        acc |= int(c) << nbits
        nbits += b
        while nbits >= 8:
            out.append(acc & 0xFF)
            acc >>= 8
            nbits -= 8
    assert nbits == 0
    return np.array(out, dtype=np.uint8)


@pytest.mark.parametrize("b", [2, 3, 4, 8])
def test_unpack_bits_against_python_packing(b):
    rng = random.Random(30 + b)
    codes = [rng.randrange(1 << b) for _ in range(8 * 24)]
    got = oracle.unpack_bits(_py_bitstream(codes, b), len(codes), b)
    assert got.tolist() == codes


def test_per_expert_width_reduces_to_int4_and_2bit_layouts():
    """At 4 bits the little-endian stream is the INT4 nibble layout (even k in
    the low nibble), at 2 bits the q2 layout: the per-expert dequantisation
    then equals those formats' (independent decoders)."""
    rng = np.random.default_rng(12)
    N, K, G = 6, 32, 8
    s = gen._f16_bits(rng.uniform(0.01, 0.05, size=(N, K // G)))
    st4 = rng.integers(0, 256, size=N * K // 2, dtype=np.uint8)
    w4 = oracle.dequant_per_expert(st4, s, N, K, G, 4, 8)
    assert np.array_equal(w4, oracle.dequant_int4(st4.reshape(N, K // 2), s, G, 8))
    st2 = rng.integers(0, 256, size=N * K // 4, dtype=np.uint8)
    w2 = oracle.dequant_per_expert(st2, s, N, K, G, 2, 1)
    ref2 = np.repeat(oracle.f16_to_f64(s), G, axis=-1) * (oracle.unpack_u2(st2.reshape(N, K // 4)).astype(np.int64) - 1)
    assert np.array_equal(w2, ref2)
    st8 = rng.integers(0, 256, size=N * K, dtype=np.uint8)  # at 8 bits the stream is the codes, one a byte
    w8 = oracle.dequant_per_expert(st8, s, N, K, G, 8, 128)
    ref8 = np.repeat(oracle.f16_to_f64(s), G, axis=-1) * (st8.reshape(N, K).astype(np.int64) - 128)
    assert np.array_equal(w8, ref8)


def test_per_expert_3bit_one_hot_probe():
    """A 3-bit stream with one nonzero code: only that weight moves off -z * scale."""
    N, K, G, z = 2, 16, 8, 4
    codes = [0] * (N * K)
    codes[K + 11] = 6
    st = _py_bitstream(codes, 3)
    s = gen._f16_bits(np.array([[0.5, 0.25], [0.125, 2.0]]))
    w = oracle.dequant_per_expert(st, s, N, K, G, 3, z)
    want = np.repeat(oracle.f16_to_f64(s), G, axis=-1) * -z
    want[1, 11] = 2.0 * (6 - z)
    assert np.array_equal(w, want)


def test_mixed_expert_widths_recipe():
    cfg = gen.config("olmoe_mixed_decode")
    d = gen.generate(cfg)
    bits, zero = d["expert_bits"], d["expert_zero"]
    assert np.bincount(bits, minlength=5)[2:].tolist() == [26, 22, 16]
    assert (bits[:16] == 4).all() and (bits[-26:] == 2).all()  # popular experts keep more bits
    assert ((zero == 2 ** (bits - 1)) | (zero == 2 ** (bits - 1) - 1)).all()
    assert d["gu_codes"].size == oracle.expert_stream_offsets(bits, 2 * cfg.I, cfg.H)[-1]
    assert d["dn_codes"].size == oracle.expert_stream_offsets(bits, cfg.H, cfg.I)[-1]


def test_edge_expert_widths_recipe():
    """INT2 / INT4 / INT8 experts: the widest width goes to the most popular experts."""
    cfg = gen.config("olmoe_edge_decode")
    d = gen.generate(cfg)
    bits, zero = d["expert_bits"], d["expert_zero"]
    assert np.bincount(bits, minlength=9)[[2, 4, 8]].tolist() == [26, 22, 16]
    assert (bits[:16] == 8).all() and (bits[16:38] == 4).all() and (bits[-26:] == 2).all()
    assert ((zero == 2 ** (bits - 1)) | (zero == 2 ** (bits - 1) - 1)).all()
    assert d["gu_codes"].size == oracle.expert_stream_offsets(bits, 2 * cfg.I, cfg.H)[-1]


@pytest.mark.parametrize("name", ["olmoe_mixed_decode", "olmoe_edge_decode"])
def test_moe_forward_matches_dense_bruteforce_mixed(impl, name):
    """Per-expert widths: the grouped oracle equals a pure-Python dense evaluation
    that decodes each expert's bit stream itself."""
    cfg = gen.config(name, T=5, H=16, I=8, E=4, k=2, G=8, zipf=None)
    d = gen.generate(cfg)
    res = impl.moe_forward(d, cfg)

    def mat(prefix, e, n_rows, kdim):
        b, z = int(d["expert_bits"][e]), int(d["expert_zero"][e])
        start = sum(int(d["expert_bits"][j]) * n_rows * kdim // 8 for j in range(e))
        raw = d[prefix + "codes"][start:start + b * n_rows * kdim // 8]
        bitl = [(int(raw[i // 8]) >> (i % 8)) & 1 for i in range(8 * raw.size)]
        rows = []
        for n in range(n_rows):
            row = []
            for kk in range(kdim):
                pos = (n * kdim + kk) * b
                c = sum(bitl[pos + j] << j for j in range(b))
                row.append(f16_val(int(d[prefix + "scales"][e][n][kk // cfg.G])) * (c - z))
            rows.append(row)
        return rows
    assert set(d["expert_bits"].tolist()) == set(cfg.widths)  # every width of the recipe is exercised
    for t in range(cfg.T):
        xt = [bf16_val(int(v)) for v in d["x"][t]]
        row = [float(v) for v in d["logits"][t]]
        order = sorted(range(cfg.E), key=lambda e: (-row[e], e))[:cfg.k]
        ex = [math.exp(row[e] - row[order[0]]) for e in order]
        acc, acc16 = [0.0] * cfg.H, [0.0] * cfg.H
        for j, e in enumerate(order):
            wgu, wd = mat("gu_", e, 2 * cfg.I, cfg.H), mat("dn_", e, cfg.H, cfg.I)
            y = py_ffn(xt, wgu, wd, cfg.I)
            y16 = py_ffn(xt, wgu, wd, cfg.I, h16=True)
            acc = [a + ex[j] / sum(ex) * v for a, v in zip(acc, y)]
            acc16 = [a + ex[j] / sum(ex) * v for a, v in zip(acc16, y16)]
        assert rel_err(res["out"][t], acc) < 1e-12
        assert rel_err(res["out_h16"][t], acc16) < 1e-12

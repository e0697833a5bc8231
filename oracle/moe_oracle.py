"""CPU oracle for the routed-expert quantized MoE path.  TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module.  The GPU library never calls it, and it shares no code,
tables or helpers with the GPU library: it unpacks every storage format with
its own code and works in float64 throughout (one diagnostic variant rounds
the SwiGLU activation to bf16; see below).

What is computed (the plain definition; the method changes only how expert
weights are stored and moved, not what the layer computes):

* "Every Expert Counts: ExactMoE for Memory-Efficient W4A16 Inference" --
  the router makes the same decisions and every selected expert runs its own
  computation; only routed-expert weights are 4-bit (W4A16).  So the oracle is
  the dense MoE definition applied to exactly dequantised weights, with no
  capacity limit and no dropped (token, expert) pairs.
* "D2MoE: Dual Routing and Dynamic Scheduling ..." -- Design, Dual Routing
  equations: x -> Expert Gate -> E_i and x -> Bit Gate -> b_i (one bit-width
  per (token, expert) pair); MWQ equations W(2)=Q2, W(3)=Q2+D3, W(4)=Q2+D3+D4
  with INT2 c INT3 c INT4; pipeline equation: dequantise, then a 16-bit GEMM.
* "ME-Switch: A Memory-Efficient Expert Switching Framework ..." -- expert
  weight = shared base weight + delta; the delta is quantised with one step per
  output channel, except salient input channels, which are kept unquantised.
* Expert-aware batching (Read-ME summary) and grouped execution (ExactMoE):
  the (token, expert) pairs are grouped per expert before the expert runs.

Conventions no page fixes (the plainest reading, shared with the GPU path by
specification, not by code):
* top-k: descending logit, ties to the lower expert index; gate weights are a
  softmax over the k selected logits.
* INT4: w = scale[n][k // G] * (c - 8), c in [0, 15]; canonical layout
  [E][N][K/2], even k in the low nibble of its byte.
* MWQ: q2 = bits 3..2 of the 4-bit code, d3 = bit 1, d4 = bit 0, so
  c_b = 4*q2 + 2*d3*[b>=3] + d4*[b==4] and w = scale * (c_b - 8), no
  re-centring.  q2 packs four 2-bit fields per byte (k & 3 selects bits
  2*(k&3)+1 .. 2*(k&3)); d3 / d4 pack eight 1-bit fields (bit k & 7).
* DELTA2: d = salient_val if k is salient else step[n] * (c - 2), c in [0, 3],
  packed like q2.
* Static bit-width per expert (EdgeMoE, expert-wise bit-width adaptation):
  expert e stores b_e-bit codes, b_e in {2, 3, 4, 8} (the page names INT2,
  INT4 and INT8 experts), with its own zero point:
  w = scale[n][k // G] * (c - z_e).  Each row of an expert is a little-endian
  bit stream (code k in bits k*b .. k*b + b - 1); experts are back to back.
* SwiGLU expert: h = silu(x Wg^T) * (x Wu^T), y = h Wd^T, with gate rows
  0..I-1 and up rows I..2I-1 of the gate_up matrix.  Everything is float64:
  the gate/up products, SiLU, h, the expert output y and the combine.  As a
  second, diagnostic result (`out_h16`) the same layer is also evaluated with
  h rounded once to bf16 before the down product: the 16-bit activation that
  W4A16 (ExactMoE) and the D2MoE pipeline equation (dequantise, then a 16-bit
  GEMM) feed into the next expert GEMM.  The parity bar applies to `out`.
* MWQ segment order inside an expert: b = 4, 3, 2 (sub-key 4 - b).
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


# ------------------------------------------------------------ storage decoding
def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(F64)


def f16_to_f64(bits) -> np.ndarray:
    """IEEE binary16 bit patterns (uint16) -> exact float64 values."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(F64)


def unpack_u4(packed) -> np.ndarray:
    """[..., K/2] bytes -> [..., K] codes in [0, 15]; even k is the low nibble."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1], 2), dtype=np.uint8)
    out[..., 0] = p & 0xF
    out[..., 1] = p >> 4
    return out.reshape(p.shape[:-1] + (p.shape[-1] * 2,))


def unpack_u2(packed) -> np.ndarray:
    """[..., K/4] bytes -> [..., K] 2-bit fields; field k&3 sits at bits 2*(k&3)."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1], 4), dtype=np.uint8)
    for j in range(4):
        out[..., j] = (p >> (2 * j)) & 3
    return out.reshape(p.shape[:-1] + (p.shape[-1] * 4,))


def unpack_u1(packed) -> np.ndarray:
    """[..., K/8] bytes -> [..., K] bits; bit k&7 of byte k>>3."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1], 8), dtype=np.uint8)
    for j in range(8):
        out[..., j] = (p >> j) & 1
    return out.reshape(p.shape[:-1] + (p.shape[-1] * 8,))


# --------------------------------------------------------------- dequantisation
def dequant_int4(codes, scales, G: int, zero_point: int = 8) -> np.ndarray:
    """W4A16 expert matrix [N][K] (row n = output channel), exact in float64.

    w[n][k] = scale[n][k // G] * (c[n][k] - zero_point)   (ExactMoE: 4-bit
    routed-expert weights with 16-bit activations; group scales along K).
    """
    c = unpack_u4(codes)
    K = c.shape[-1]
    s = f16_to_f64(scales)
    assert s.shape[-1] * G == K
    return np.repeat(s, G, axis=-1) * (c.astype(F64) - zero_point)


def mwq_code(q2, d3, d4, b: int) -> np.ndarray:
    """Effective code of the nested planes at bit-width b (D2MoE, MWQ equations).

    W(2) = Q2, W(3) = Q2 + D3, W(4) = Q2 + D3 + D4 where Q2 holds the top two
    bits of the 4-bit code and D3, D4 the next two: the b-bit weight is the
    4-bit code truncated to its top b bits.
    """
    if b not in (2, 3, 4):
        raise ValueError("bit-width must be 2, 3 or 4")
    c = 4 * q2
    if b >= 3:
        c = c + 2 * d3
    if b == 4:
        c = c + d4
    return c


def dequant_mwq(q2p, d3p, d4p, scales, G: int, b: int, zero_point: int = 8) -> np.ndarray:
    """Nested-plane expert matrix [N][K] at bit-width b, exact in float64."""
    return dequant_mwq_planes(unpack_u2(q2p), unpack_u1(d3p), unpack_u1(d4p), scales, G, b, zero_point)


def dequant_mwq_planes(q2, d3, d4, scales, G: int, b: int, zero_point: int = 8) -> np.ndarray:
    """As dequant_mwq, from planes already unpacked to one field per weight."""
    c = mwq_code(q2, d3, d4, b)
    s = f16_to_f64(scales)
    assert s.shape[-1] * G == c.shape[-1]
    return np.repeat(s, G, axis=-1) * (c.astype(F64) - zero_point)


def unpack_bits(stream, n_codes: int, b: int) -> np.ndarray:
    """A little-endian bit stream -> n_codes unsigned codes of b bits each
    (code k is bits k*b .. k*b + b - 1, bit j of byte i being stream bit 8i + j)."""
    bitv = np.unpackbits(np.asarray(stream, dtype=np.uint8), bitorder="little")[: n_codes * b].astype(np.int64)
    return (bitv.reshape(n_codes, b) << np.arange(b, dtype=np.int64)).sum(axis=1)


def dequant_per_expert(stream, scales, N: int, K: int, G: int, b: int, zero_point: int) -> np.ndarray:
    """Expert matrix [N][K] stored at its own bit-width b (EdgeMoE expert-wise
    bit-width adaptation), exact in float64: w = scale[n][k // G] * (c - z)."""
    if b not in (2, 3, 4, 8):
        raise ValueError("bit-width must be 2, 3, 4 or 8")
    c = unpack_bits(stream, N * K, b).reshape(N, K)
    s = f16_to_f64(scales)
    assert s.shape == (N, K // G)
    return np.repeat(s, G, axis=-1) * (c.astype(F64) - zero_point)


def expert_stream_offsets(bits, N: int, K: int) -> np.ndarray:
    """Byte offset of each expert's codes in the flat per-expert stream (E + 1 entries)."""
    sizes = np.asarray(bits, dtype=np.int64) * N * K // 8
    return np.concatenate([[0], np.cumsum(sizes)])


def dequant_delta2(codes, step, salient_idx, salient_val) -> np.ndarray:
    """ME-Switch delta [N][K]: salient input channels keep their bf16 value,
    every other channel is step[n] * (c - 2) with a 2-bit code c."""
    c = unpack_u2(codes)
    d = f16_to_f64(step)[:, None] * (c.astype(F64) - 2.0)
    idx = np.asarray(salient_idx, dtype=np.int64)
    d[:, idx] = bf16_to_f64(salient_val).T
    return d


# ---------------------------------------------------------------------- routing
def route_topk(logits, k: int):
    """Expert gate (D2MoE Dual Routing: x -> Expert Gate -> E_i).

    ids[t][j]: the j-th largest logit of token t, ties to the lower expert
    index; w[t][j] = softmax over the k selected logits (float64).
    """
    lg = np.asarray(logits, dtype=np.float32).astype(F64)
    T, E = lg.shape
    if not (1 <= k <= E):
        raise ValueError("need 1 <= k <= E")
    if not np.all(np.isfinite(lg)):
        raise ValueError("logits must be finite")
    order = np.argsort(-lg, axis=1, kind="stable")[:, :k]
    sel = np.take_along_axis(lg, order, axis=1)
    e = np.exp(sel - sel[:, :1])
    w = e / e.sum(axis=1, keepdims=True)
    return order.astype(np.int32), w


# --------------------------------------------------------------------- grouping
def permute(ids, E: int, pair_bits=None):
    """Group (token, slot) pairs per expert (and per bit-width for MWQ).

    Pair p = t*k + j.  key = e            (S = 1)
                       = 3*e + (4 - b)    (MWQ, S = 3: segments b = 4, 3, 2)
    Returns counts[E] (pairs per expert), seg_offsets[E*S + 1] (exclusive
    prefix sum of pairs per key), sorted_pair (pairs in ascending (key, p)
    order) and pair_pos (its inverse: pair -> position in sorted order).
    """
    ids = np.asarray(ids, dtype=np.int64).ravel()
    P = ids.size
    if P and (ids.min() < 0 or ids.max() >= E):
        raise ValueError("expert id out of range")
    if pair_bits is None:
        S, key = 1, ids
    else:
        b = np.asarray(pair_bits, dtype=np.int64).ravel()
        if b.size != P or (P and (b.min() < 2 or b.max() > 4)):
            raise ValueError("bad bit-widths")
        S, key = 3, ids * 3 + (4 - b)
    counts = np.bincount(ids, minlength=E).astype(np.int32)
    per_key = np.bincount(key, minlength=E * S)
    seg_offsets = np.concatenate([[0], np.cumsum(per_key)]).astype(np.int32)
    sorted_pair = np.argsort(key, kind="stable").astype(np.int32)
    pair_pos = np.empty(P, dtype=np.int32)
    pair_pos[sorted_pair] = np.arange(P, dtype=np.int32)
    return counts, seg_offsets, sorted_pair, pair_pos


# ----------------------------------------------------------------------- experts
def round_bf16(a) -> np.ndarray:
    """Nearest bf16 value (8 significant bits, ties to even) of float64 values,
    rounded once from the float64 value; returned as float64."""
    a = np.asarray(a, dtype=F64)
    m, e = np.frexp(a)                    # a = m * 2**e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


def silu(g):
    return g / (1.0 + np.exp(-g))


def swiglu_expert(xrows, w_gate_up, w_down, h_bf16: bool = False):
    """SwiGLU FFN of one expert on rows of activations, in float64.

    w_gate_up [2I][H]: rows 0..I-1 gate, I..2I-1 up; w_down [H][I].
    h = silu(x Wg^T) * (x Wu^T), y = h Wd^T.  With h_bf16 the activation h
    is rounded once to bf16 before the down product (the 16-bit activation of
    W4A16; a diagnostic model, not the definition).
    Returns (h [m][I], y [m][H]).
    """
    I = w_gate_up.shape[0] // 2
    g = xrows @ w_gate_up[:I].T
    u = xrows @ w_gate_up[I:].T
    h = silu(g) * u
    if h_bf16:
        h = round_bf16(h)
    return h, h @ w_down.T


def unpermute_combine(y_perm, pair_pos, w, T: int, k: int):
    """Gate-weighted combine: out[t] = sum_j w[t][j] * y_perm[pair_pos[t*k+j]]."""
    y = np.asarray(y_perm, dtype=F64)
    pos = np.asarray(pair_pos, dtype=np.int64).reshape(T, k)
    w = np.ones((T, k)) if w is None else np.asarray(w, dtype=F64).reshape(T, k)
    out = np.zeros((T, y.shape[1]), dtype=F64)
    for j in range(k):
        out += w[:, j:j + 1] * y[pos[:, j]]
    return out


def _expert_weights_int4(data, e, G):
    wgu = dequant_int4(data["gu_codes"][e], data["gu_scales"][e], G)
    wd = dequant_int4(data["dn_codes"][e], data["dn_scales"][e], G)
    return wgu, wd


def _expert_planes_mwq(data, e):
    """The nested planes of expert e, unpacked once for all of its bit-widths."""
    return {m: (unpack_u2(data[m + "q2"][e]), unpack_u1(data[m + "d3"][e]), unpack_u1(data[m + "d4"][e]))
            for m in ("gu_", "dn_")}


def _expert_weights_mwq(data, planes, e, G, b):
    wgu = dequant_mwq_planes(*planes["gu_"], data["gu_scales"][e], G, b)
    wd = dequant_mwq_planes(*planes["dn_"], data["dn_scales"][e], G, b)
    return wgu, wd


def _expert_weights_mixed(data, e, cfg):
    b, z = int(data["expert_bits"][e]), int(data["expert_zero"][e])
    I, H, G = cfg.I, cfg.H, cfg.G
    og = expert_stream_offsets(data["expert_bits"], 2 * I, H)
    od = expert_stream_offsets(data["expert_bits"], H, I)
    wgu = dequant_per_expert(data["gu_codes"][og[e]:og[e + 1]], data["gu_scales"][e], 2 * I, H, G, b, z)
    wd = dequant_per_expert(data["dn_codes"][od[e]:od[e + 1]], data["dn_scales"][e], H, I, G, b, z)
    return wgu, wd


def moe_forward(data: dict, cfg, tokens=None) -> dict:
    """Full routed-expert layer: route -> group -> per-segment expert FFN -> combine.

    data: a generated workload (INT4, MWQ or per-expert widths).  tokens: optional subset of
    token indices; routing and grouping always cover all tokens, the expert
    FFN and the combine only the pairs of the chosen tokens (rows of h_perm /
    y_perm for other pairs stay NaN).
    Returns the float64 layer (`h_perm`, `y_perm`, `out`) and, as a
    diagnostic, `out_h16` / `y_perm_h16`: the same layer with the SwiGLU
    activation rounded once to bf16 before the down product.
    """
    T, E, k, G = cfg.T, cfg.E, cfg.k, cfg.G
    x = bf16_to_f64(data["x"])
    ids, w = route_topk(data["logits"], k)
    mwq = cfg.fmt == "mwq"
    bits = np.asarray(data["pair_bits"]) if mwq else None
    counts, seg_offsets, sorted_pair, pair_pos = permute(ids, E, bits)
    S = 3 if mwq else 1
    P = T * k
    want = np.ones(P, dtype=bool) if tokens is None else np.isin(np.arange(P) // k, np.asarray(tokens))
    I, H = cfg.I, cfg.H
    h_perm = np.full((P, I), np.nan)
    y_perm = np.full((P, H), np.nan)
    y_perm16 = np.full((P, H), np.nan)
    for e in range(E):
        planes = None
        for seg in range(e * S, (e + 1) * S):
            lo, hi = seg_offsets[seg], seg_offsets[seg + 1]
            rows = np.arange(lo, hi)
            rows = rows[want[sorted_pair[lo:hi]]]
            if rows.size == 0:
                continue
            if mwq:
                planes = planes or _expert_planes_mwq(data, e)
                wgu, wd = _expert_weights_mwq(data, planes, e, G, 4 - seg % S)
            elif cfg.fmt == "mixed":
                wgu, wd = _expert_weights_mixed(data, e, cfg)
            else:
                wgu, wd = _expert_weights_int4(data, e, G)
            toks = sorted_pair[rows] // k
            h, y = swiglu_expert(x[toks], wgu, wd)
            h_perm[rows] = h
            y_perm[rows] = y
            y_perm16[rows] = round_bf16(h) @ wd.T
    sel = np.arange(T) if tokens is None else np.asarray(tokens)
    out = unpermute_combine(np.nan_to_num(y_perm), pair_pos, w, T, k)
    out16 = unpermute_combine(np.nan_to_num(y_perm16), pair_pos, w, T, k)
    if tokens is not None:
        keep = np.zeros(T, dtype=bool)
        keep[sel] = True
        out[~keep] = np.nan
        out16[~keep] = np.nan
    return {
        "ids": ids, "w": w, "counts": counts, "seg_offsets": seg_offsets,
        "sorted_pair": sorted_pair, "pair_pos": pair_pos,
        "h_perm": h_perm, "y_perm": y_perm, "out": out, "tokens": sel,
        "y_perm_h16": y_perm16, "out_h16": out16,
    }


def delta_linear(data: dict, cfg, tokens=None) -> dict:
    """ME-Switch multi-expert linear: y[t] = x[t] W_base^T + x[t] D_{e(t)}^T.

    Tokens are grouped per expert (k = 1, gate weight 1).  tokens: optional
    subset of token indices for which y is computed (others stay NaN).
    """
    T, E = cfg.T, cfg.E
    x = bf16_to_f64(data["x"])
    ids = np.asarray(data["ids"], dtype=np.int32).reshape(T, 1)
    counts, seg_offsets, sorted_pair, pair_pos = permute(ids, E)
    base = bf16_to_f64(data["base"])
    want = np.zeros(T, dtype=bool)
    want[np.arange(T) if tokens is None else np.asarray(tokens)] = True
    y = np.full((T, cfg.N), np.nan)
    for e in range(E):
        toks = sorted_pair[seg_offsets[e]:seg_offsets[e + 1]]
        toks = toks[want[toks]]
        if toks.size == 0:
            continue
        d = dequant_delta2(data["codes"][e], data["step"][e], data["salient_idx"][e], data["salient_val"][e])
        y[toks] = x[toks] @ base.T + x[toks] @ d.T
    return {"ids": ids, "counts": counts, "seg_offsets": seg_offsets,
            "sorted_pair": sorted_pair, "pair_pos": pair_pos, "out": y}


# ------------------------------------------------------------------ comparison
def compare(gpu, ref) -> dict:
    """Relative L2 error and max-abs error relative to the reference RMS."""
    g = np.asarray(gpu, dtype=F64)
    r = np.asarray(ref, dtype=F64)
    diff = g - r
    nr = np.sqrt(np.sum(r * r))
    rms = np.sqrt(np.mean(r * r)) if r.size else 0.0
    return {
        "rel_l2": float(np.sqrt(np.sum(diff * diff)) / nr) if nr > 0 else float(np.sqrt(np.sum(diff * diff))),
        "max_abs_over_rms": float(np.max(np.abs(diff)) / rms) if rms > 0 else float(np.max(np.abs(diff), initial=0.0)),
    }

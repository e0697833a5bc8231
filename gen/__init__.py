"""Seeded synthetic inputs for the routed-expert quantized MoE path.

This module only draws random data in the storage formats the path consumes
(bf16 / fp16 bit patterns, packed integer codes, index arrays).  It holds no
routing, grouping, dequantisation or GEMM arithmetic: both the CPU oracle and
the GPU path read what it produces, and neither imports the other.

Every tensor comes from its own numpy PCG64 stream keyed by (seed, tag), so a
tensor does not change when another one is added or resized.

Workloads (shapes and distributions follow the workload descriptions of the
five summarised systems; no page fixes a seed, so the seeds are ours):

  tiny            64 tok, H 256, I 512, 8 experts, top-2, INT4 g64, scales U(0.005,0.02)
  olmoe_decode    32 tok, H 2048, I 1024, 64 experts, top-8, INT4 g128,
                  scales U(0.002,0.01), Zipf(1.1) popularity bias on the logits
  olmoe_prefill   8192 tok, same layer, i.i.d. N(0,1) logits
  olmoe_prefill_zipf  same with the Zipf(1.1) bias
  mixtral_mwq     512 tok, H 4096, I 14336, 8 experts, top-2, nested INT2+d3+d4
                  planes g128, per-pair bit-width from {2:0.40, 3:0.35, 4:0.25}
  mixtral_mwq_decode  the same layer at a decode batch of 16 tokens
  olmoe_mixed_decode  the olmoe_decode layer with a static bit-width per expert
                  (EdgeMoE expert-wise bit-width adaptation): the experts most
                  often routed to (Zipf rank) keep 4 bits, the next 3, the rest 2,
                  in the proportions 0.25 / 0.35 / 0.40; codes packed at their
                  own width, zero point per expert, group scales U(lo,hi) x 2^(4-b)
  olmoe_edge_decode  the same with the INT2 / INT4 / INT8 widths EdgeMoE names:
                  8 bits for the most routed-to quarter, 4 for the next 0.35, 2
                  for the rest
  meswitch_delta  256 requests x 16 tok, linear 4096 -> 14336, 16 experts,
                  shared bf16 base N(0,0.02), 2-bit delta codes with per-output
                  channel fp16 step U(0.0005,0.002), 41 salient input channels
                  per expert kept as bf16 N(0,0.002), Zipf(1.0) request->expert
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = [
    "MoeConfig", "DeltaConfig", "CONFIGS", "config", "rng_for",
    "f32_to_bf16_bits", "bf16_bits_to_f32", "zipf_probs",
    "gen_moe_int4", "gen_moe_mwq", "gen_moe_mixed", "gen_delta_linear",
]

# tensor tags: one independent stream per (seed, tag)
_TAG = {
    "x": 1, "logits": 2, "gu_codes": 3, "gu_scales": 4, "dn_codes": 5,
    "dn_scales": 6, "bits": 7, "base": 8, "d2_codes": 9, "d2_step": 10,
    "sal_idx": 11, "sal_val": 12, "requests": 13, "gu_q2": 14, "gu_d3": 15,
    "gu_d4": 16, "dn_q2": 17, "dn_d3": 18, "dn_d4": 19, "expert_bits": 20, "expert_zero": 21,
}


def rng_for(seed: int, tag: str) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), _TAG[tag]])))


@dataclasses.dataclass(frozen=True)
class MoeConfig:
    name: str
    T: int                 # tokens
    H: int                 # hidden size (K of gate/up, N of down)
    I: int                 # SwiGLU intermediate size
    E: int                 # experts
    k: int                 # experts per token
    G: int                 # quantisation group size along K
    fmt: str               # "int4" | "mwq" | "mixed"
    scale_lo: float
    scale_hi: float
    zipf: Optional[float]  # popularity exponent added to the logits, or None
    seed: int
    bit_probs: tuple = ()  # mwq: probabilities of bit-widths (2, 3, 4); mixed: shares of experts at each width
    widths: tuple = (2, 3, 4)  # mixed: the widths bit_probs refers to, ascending

    @property
    def pairs(self) -> int:
        return self.T * self.k


@dataclasses.dataclass(frozen=True)
class DeltaConfig:
    name: str
    requests: int
    tokens_per_request: int
    K: int                 # input channels
    N: int                 # output channels
    E: int                 # experts (fine-tuned deltas)
    n_salient: int
    base_std: float
    delta_std: float
    step_lo: float
    step_hi: float
    zipf: float
    seed: int

    @property
    def T(self) -> int:
        return self.requests * self.tokens_per_request

    k = 1
    fmt = "delta2"


CONFIGS = {
    "tiny": MoeConfig("tiny", 64, 256, 512, 8, 2, 64, "int4", 0.005, 0.02, None, 101),
    "olmoe_decode": MoeConfig("olmoe_decode", 32, 2048, 1024, 64, 8, 128, "int4", 0.002, 0.01, 1.1, 202),
    "olmoe_prefill": MoeConfig("olmoe_prefill", 8192, 2048, 1024, 64, 8, 128, "int4", 0.002, 0.01, None, 303),
    "olmoe_prefill_zipf": MoeConfig("olmoe_prefill_zipf", 8192, 2048, 1024, 64, 8, 128, "int4", 0.002, 0.01, 1.1, 304),
    "mixtral_mwq": MoeConfig("mixtral_mwq", 512, 4096, 14336, 8, 2, 128, "mwq", 0.002, 0.01, None, 404,
                             bit_probs=(0.40, 0.35, 0.25)),
    "mixtral_mwq_decode": MoeConfig("mixtral_mwq_decode", 16, 4096, 14336, 8, 2, 128, "mwq", 0.002, 0.01, None,
                                    406, bit_probs=(0.40, 0.35, 0.25)),
    "olmoe_mixed_decode": MoeConfig("olmoe_mixed_decode", 32, 2048, 1024, 64, 8, 128, "mixed", 0.002, 0.01, 1.1,
                                    707, bit_probs=(0.40, 0.35, 0.25)),
    "olmoe_edge_decode": MoeConfig("olmoe_edge_decode", 32, 2048, 1024, 64, 8, 128, "mixed", 0.002, 0.01, 1.1,
                                   708, bit_probs=(0.40, 0.35, 0.25), widths=(2, 4, 8)),
    "meswitch_delta": DeltaConfig("meswitch_delta", 256, 16, 4096, 14336, 16, 41, 0.02, 0.002,
                                  0.0005, 0.002, 1.0, 505),
}


def config(name: str, **overrides):
    """A named workload, optionally with some fields replaced (smaller test cases)."""
    base = CONFIGS[name]
    return dataclasses.replace(base, **overrides) if overrides else base


# ---------------------------------------------------------------- dtype helpers
def f32_to_bf16_bits(a) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even. Finite inputs."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _f16_bits(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64).astype(np.float16).view(np.uint16)


def zipf_probs(E: int, s: float) -> np.ndarray:
    """p_e proportional to (e+1)^-s over E items; item 0 is the most popular."""
    w = np.arange(1, E + 1, dtype=np.float64) ** (-float(s))
    return w / w.sum()


def _bytes(rng, shape) -> np.ndarray:
    # uniform bytes: every packed 4-, 2- or 1-bit field inside is uniform as well
    return rng.integers(0, 256, size=shape, dtype=np.uint8)


def _normal_bf16(rng, shape, std=1.0) -> np.ndarray:
    return f32_to_bf16_bits((rng.standard_normal(size=shape, dtype=np.float64) * std).astype(np.float32))


def _uniform_f16(rng, shape, lo, hi) -> np.ndarray:
    return _f16_bits(rng.uniform(lo, hi, size=shape))


def _logits(cfg) -> np.ndarray:
    z = rng_for(cfg.seed, "logits").standard_normal(size=(cfg.T, cfg.E), dtype=np.float64)
    if cfg.zipf is not None:
        z = z + np.log(zipf_probs(cfg.E, cfg.zipf))[None, :]
    return z.astype(np.float32)


# ------------------------------------------------------------------ generators
def gen_moe_int4(cfg: MoeConfig) -> dict:
    """INT4 W4A16 MoE layer in canonical layout.

    x        bf16 bits  [T][H]
    logits   float32    [T][E]
    gu_codes uint8      [E][2I][H/2]   two 4-bit codes per byte, rows 0..I-1 gate, I..2I-1 up
    gu_scales fp16 bits [E][2I][H/G]
    dn_codes uint8      [E][H][I/2]
    dn_scales fp16 bits [E][H][I/G]
    """
    assert cfg.fmt == "int4"
    T, H, I, E, G = cfg.T, cfg.H, cfg.I, cfg.E, cfg.G
    return {
        "x": _normal_bf16(rng_for(cfg.seed, "x"), (T, H)),
        "logits": _logits(cfg),
        "gu_codes": _bytes(rng_for(cfg.seed, "gu_codes"), (E, 2 * I, H // 2)),
        "gu_scales": _uniform_f16(rng_for(cfg.seed, "gu_scales"), (E, 2 * I, H // G), cfg.scale_lo, cfg.scale_hi),
        "dn_codes": _bytes(rng_for(cfg.seed, "dn_codes"), (E, H, I // 2)),
        "dn_scales": _uniform_f16(rng_for(cfg.seed, "dn_scales"), (E, H, I // G), cfg.scale_lo, cfg.scale_hi),
    }


def gen_moe_mwq(cfg: MoeConfig) -> dict:
    """Nested-plane MoE layer in canonical layout.

    Planes are drawn as uniform bits, which is the same distribution as
    splitting uniform 4-bit codes into a 2-bit base and two 1-bit residuals.
    q2 uint8 [E][N][K/4] (four 2-bit fields per byte), d3 / d4 uint8 [E][N][K/8]
    (eight 1-bit fields per byte); scales fp16 bits [E][N][K/G].
    pair_bits uint8 [T*k] in {2,3,4}, drawn per (token, slot) pair.
    """
    assert cfg.fmt == "mwq"
    T, H, I, E, G = cfg.T, cfg.H, cfg.I, cfg.E, cfg.G
    s = cfg.seed
    p = np.asarray(cfg.bit_probs, dtype=np.float64)
    u = rng_for(s, "bits").random(size=cfg.T * cfg.k)
    pair_bits = (2 + np.searchsorted(np.cumsum(p / p.sum()), u, side="right")).clip(2, 4).astype(np.uint8)
    return {
        "x": _normal_bf16(rng_for(s, "x"), (T, H)),
        "logits": _logits(cfg),
        "pair_bits": pair_bits,
        "gu_q2": _bytes(rng_for(s, "gu_q2"), (E, 2 * I, H // 4)),
        "gu_d3": _bytes(rng_for(s, "gu_d3"), (E, 2 * I, H // 8)),
        "gu_d4": _bytes(rng_for(s, "gu_d4"), (E, 2 * I, H // 8)),
        "gu_scales": _uniform_f16(rng_for(s, "gu_scales"), (E, 2 * I, H // G), cfg.scale_lo, cfg.scale_hi),
        "dn_q2": _bytes(rng_for(s, "dn_q2"), (E, H, I // 4)),
        "dn_d3": _bytes(rng_for(s, "dn_d3"), (E, H, I // 8)),
        "dn_d4": _bytes(rng_for(s, "dn_d4"), (E, H, I // 8)),
        "dn_scales": _uniform_f16(rng_for(s, "dn_scales"), (E, H, I // G), cfg.scale_lo, cfg.scale_hi),
    }


def expert_widths(cfg: MoeConfig) -> np.ndarray:
    """Static bit-width per expert (int32 [E], values from cfg.widths).

    With a popularity bias the experts are ranked by it (expert 0 is the most
    popular): the top share bit_probs[-1] keeps the widest width, the next
    bit_probs[-2] the next, and so on down to the narrowest for the rest.
    Without one the widths are a seeded permutation of the same counts.
    """
    E = cfg.E
    p = np.asarray(cfg.bit_probs, dtype=np.float64)
    p = p / p.sum()
    w = list(cfg.widths)
    counts, left = [], E
    for i in range(len(w) - 1, 0, -1):   # widest first
        n = min(int(round(p[i] * E)), left)
        counts.append((w[i], n))
        left -= n
    counts.append((w[0], left))
    ranked = np.array([b for b, n in counts for _ in range(n)], dtype=np.int32)
    if cfg.zipf is None:
        ranked = ranked[rng_for(cfg.seed, "expert_bits").permutation(E)]
    return ranked


def _bitstream(rng, E, N, K, bits) -> np.ndarray:
    # expert e: N rows of K codes of bits[e] bits, LSB first; uniform bits give uniform codes
    return np.concatenate([_bytes(rng, (N * K * int(b) // 8,)) for b in bits]) if E else np.zeros(0, np.uint8)


def gen_moe_mixed(cfg: MoeConfig) -> dict:
    """MoE layer with a static bit-width b_e per expert (cfg.widths: {2, 3, 4}
    or the INT2 / INT4 / INT8 mix {2, 4, 8}), canonical layout.

    expert_bits int32 [E]; expert_zero int32 [E], z_e in {2^(b_e-1) - 1, 2^(b_e-1)}
    gu_codes uint8 flat: expert e's [2I][H] codes of b_e bits, each row a
             little-endian bit stream (code k at bits k*b_e .. k*b_e + b_e - 1),
             experts back to back
    gu_scales fp16 bits [E][2I][H/G], drawn U(lo, hi) * 2^(4 - b_e)
    dn_codes / dn_scales likewise for [E][H][I]
    """
    assert cfg.fmt == "mixed"
    T, H, I, E, G = cfg.T, cfg.H, cfg.I, cfg.E, cfg.G
    s = cfg.seed
    bits = expert_widths(cfg)
    zero = (2 ** (bits - 1) - rng_for(s, "expert_zero").integers(0, 2, size=E)).astype(np.int32)
    mult = (2.0 ** (4 - bits)).astype(np.float64)[:, None, None]
    return {
        "x": _normal_bf16(rng_for(s, "x"), (T, H)),
        "logits": _logits(cfg),
        "expert_bits": bits,
        "expert_zero": zero,
        "gu_codes": _bitstream(rng_for(s, "gu_codes"), E, 2 * I, H, bits),
        "gu_scales": _f16_bits(rng_for(s, "gu_scales").uniform(cfg.scale_lo, cfg.scale_hi, size=(E, 2 * I, H // G))
                               * mult),
        "dn_codes": _bitstream(rng_for(s, "dn_codes"), E, H, I, bits),
        "dn_scales": _f16_bits(rng_for(s, "dn_scales").uniform(cfg.scale_lo, cfg.scale_hi, size=(E, H, I // G))
                               * mult),
    }


def gen_delta_linear(cfg: DeltaConfig) -> dict:
    """Shared-base + per-expert 2-bit delta linear layer, canonical layout.

    x           bf16 bits [T][K], T = requests * tokens_per_request
    ids         int32     [T]     expert of each token (all tokens of a request share it)
    base        bf16 bits [N][K]
    codes       uint8     [E][N][K/4]  2-bit codes, uniform over {0..3}
    step        fp16 bits [E][N]
    salient_idx int32     [E][S] distinct input channels, ascending
    salient_val bf16 bits [E][S][N]
    """
    T, K, N, E, S = cfg.T, cfg.K, cfg.N, cfg.E, cfg.n_salient
    s = cfg.seed
    u = rng_for(s, "requests").random(size=cfg.requests)
    req_expert = np.searchsorted(np.cumsum(zipf_probs(E, cfg.zipf)), u, side="right").clip(0, E - 1)
    ids = np.repeat(req_expert, cfg.tokens_per_request).astype(np.int32)
    r = rng_for(s, "sal_idx")
    sal_idx = np.stack([np.sort(r.choice(K, size=S, replace=False)) for _ in range(E)]).astype(np.int32)
    return {
        "x": _normal_bf16(rng_for(s, "x"), (T, K)),
        "ids": ids,
        "base": _normal_bf16(rng_for(s, "base"), (N, K), cfg.base_std),
        "codes": _bytes(rng_for(s, "d2_codes"), (E, N, K // 4)),
        "step": _uniform_f16(rng_for(s, "d2_step"), (E, N), cfg.step_lo, cfg.step_hi),
        "salient_idx": sal_idx,
        "salient_val": _normal_bf16(rng_for(s, "sal_val"), (E, S, N), cfg.delta_std),
    }


def generate(cfg) -> dict:
    if isinstance(cfg, DeltaConfig):
        return gen_delta_linear(cfg)
    if cfg.fmt == "mixed":
        return gen_moe_mixed(cfg)
    return gen_moe_int4(cfg) if cfg.fmt == "int4" else gen_moe_mwq(cfg)


def workload_bytes(cfg) -> float:
    """Total bytes of a generated workload (for sizing decisions in tests)."""
    if isinstance(cfg, DeltaConfig):
        return cfg.T * cfg.K * 2 + cfg.N * cfg.K * 2 + cfg.E * cfg.N * (cfg.K / 4 + 2 + 2 * cfg.n_salient)
    per_w = 0.5 + 2.0 / cfg.G
    return cfg.T * cfg.H * 2 + cfg.E * 3 * cfg.H * cfg.I * per_w


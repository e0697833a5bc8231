"""Shared helpers of the GPU tests: move generated workloads to the device and
run the library's C ABI calls on them (through the Python binding)."""
import numpy as np
import torch

import gen
import quantized_moe_expert_top_amd as q

DEV = "cuda:0"

# parity bar for bf16 outputs
REL_L2 = 5e-3
MAX_ABS_OVER_RMS = 2e-2
GATE_RTOL = 1e-6


def t(a, dtype=None):
    """numpy -> device tensor; uint16 bit patterns travel as int16."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    x = torch.from_numpy(a).to(DEV)
    return x if dtype is None else x.view(dtype)


def bf16_to_np(x: torch.Tensor) -> np.ndarray:
    """bf16 (or fp32 / fp16) device tensor -> float64 numpy."""
    if x.dtype in (torch.float32, torch.float16):
        return x.cpu().numpy().astype(np.float64)
    return x.view(torch.bfloat16).float().cpu().numpy().astype(np.float64)


def experts_int4(d, prefix, G):
    return q.int4_experts(t(d[prefix + "codes"]), t(d[prefix + "scales"]), G)


def experts_mwq(d, prefix, G):
    return q.mwq_experts(t(d[prefix + "q2"]), t(d[prefix + "d3"]), t(d[prefix + "d4"]), t(d[prefix + "scales"]), G)


def experts_mixed(d, prefix, G):
    return q.per_expert_experts(t(d[prefix + "codes"]), t(d[prefix + "scales"]), d["expert_bits"],
                                d["expert_zero"], G)


def tiled_layer(d, cfg):
    """Repacked (tiled) gate_up and down weight sets of a generated MoE layer."""
    mk = {"int4": experts_int4, "mwq": experts_mwq, "mixed": experts_mixed}[cfg.fmt]
    gu = q.moe_repack_weights(mk(d, "gu_", cfg.G))
    dn = q.moe_repack_weights(mk(d, "dn_", cfg.G))
    return gu, dn


def run_layer(d, cfg, gu=None, dn=None, kernel=q.MOE_KERNEL_AUTO):
    """Full layer on the GPU; returns the LayerBuffers (synchronised)."""
    if gu is None:
        gu, dn = tiled_layer(d, cfg)
    x = t(d["x"])
    logits = t(d["logits"])
    bits = t(d["pair_bits"]) if cfg.fmt == "mwq" else None
    print(f"[gpu] layer {cfg.name} T={cfg.T} E={cfg.E} k={cfg.k} kernel={kernel}", flush=True)
    buf = q.moe_layer_forward(x, logits, cfg.k, gu, dn, pair_bits=bits, kernel=kernel)
    torch.cuda.synchronize()
    return buf


def delta_layer(d, cfg):
    """Tiled DELTA2 weight set (with the shared base) of a generated delta layer."""
    src = q.delta2_experts(t(d["codes"]), t(d["step"]), t(d["salient_idx"]), t(d["salient_val"]), base=t(d["base"]))
    return q.moe_repack_weights(src)


def run_delta(d, cfg, w=None, kernel=q.MOE_KERNEL_AUTO):
    if w is None:
        w = delta_layer(d, cfg)
    x = t(d["x"])
    ids = t(d["ids"]).view(cfg.T, 1)
    print(f"[gpu] delta {cfg.name} T={cfg.T} E={cfg.E} kernel={kernel}", flush=True)
    perm = q.moe_permute(ids, cfg.E)
    y_perm = q.moe_grouped_qgemm(w, x, perm.seg_offsets, cfg.T, q.MOE_EPI_NONE, gather_pair=perm.sorted_pair, k=1,
                                 kernel=kernel)
    out = q.moe_unpermute_combine(y_perm, perm.pair_pos, None, cfg.T, 1)
    torch.cuda.synchronize()
    return perm, y_perm, out


def bf16_ulp(ref):
    """One bf16 ulp of each value of ref (0 for 0)."""
    mag = np.abs(np.asarray(ref, dtype=np.float64))
    return np.exp2(np.floor(np.log2(np.where(mag > 0, mag, 1.0))) - 7.0) * (mag > 0)


# Floor of check_ulp, in units of the output RMS: about three times the
# largest deviation that evaluating the gate/up products in fp32 (instead of
# fp64) causes through bf16 SwiGLU activations that round to the other
# neighbour (1.6e-3 RMS on these layers; derived in tests/test_bar.py).
ULP_FLOOR = 5e-3


def check_ulp(gpu, ref_h16, what="", floor=ULP_FLOOR):
    """Element by element against the oracle's bf16-activation variant
    (`out_h16`: the SwiGLU activation rounded once to bf16 before the down
    product, as the kernels do): |gpu - ref| <= one bf16 ulp of ref (the
    output's own rounding) + floor * RMS(ref) (activations whose fp32 value
    rounds to the other bf16 neighbour than the exact one)."""
    ref = ref_h16
    ref = np.asarray(ref, dtype=np.float64)
    gpu = np.asarray(gpu, dtype=np.float64)
    tol = bf16_ulp(ref) + floor * np.sqrt(np.mean(ref * ref))
    bad = np.abs(gpu - ref) > tol
    assert not bad.any(), f"{what}: {int(bad.sum())} outputs beyond one bf16 ulp, first at {np.argwhere(bad)[0]}"


def check_close(gpu, ref, what=""):
    """The layer bar for bf16 outputs against the exact (fp64) result: relative
    L2 <= 5e-3, and max-abs <= 2e-2 x RMS counted beyond half a bf16 ulp of
    each exact value.  That half ulp is the output's own rounding, which no
    bf16 result avoids: where an output peaks at 9.5 RMS it alone reaches
    2.2e-2 RMS (layers with one expert per token, or nested widths whose
    truncated codes are biased)."""
    from oracle import compare
    m = compare(gpu, ref)
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(r * r)) if r.size else 0.0
    excess = np.maximum(np.abs(g - r) - 0.5 * bf16_ulp(r), 0.0)
    m["max_excess_over_rms"] = float(np.max(excess, initial=0.0) / rms) if rms > 0 else float(np.max(excess, initial=0.0))
    assert m["rel_l2"] <= REL_L2 and m["max_excess_over_rms"] <= MAX_ABS_OVER_RMS, f"{what}: {m}"
    return m

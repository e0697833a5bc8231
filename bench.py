"""Benchmark of the routed-expert quantized MoE hot path on one MI355X.

A step is one whole layer on one batch of synthetic input, inputs already
resident in HBM: route (top-k) -> group (permute) -> grouped qGEMM gate_up with
SwiGLU -> grouped qGEMM down -> gate-weighted combine (the delta workload:
group -> grouped delta linear with the shared base -> scatter back).  Each step
is one HIP-graph replay.  Several copies of the expert weights are rotated so
that a step never finds its weights in the 256 MB Infinity Cache (a real model
has many layers, each with its own experts).

Default workload: the prefill-shaped OLMoE-like layer (8192 tokens, 64
experts, top-8, hidden 2048, SwiGLU 1024, INT4 g128, uniform routing), the
largest configuration, measured against bf16 MFMA peak.  The same line
carries the decode batch of that layer (32 tokens, Zipf(1.1) popularity,
measured against HBM) and the Zipf-skewed prefill as objects of their own,
and the ceilings this GPU reaches in plain streaming and MFMA probes.

Prints one JSON line.  The dominant kernel's duration comes from HIP events
around batches of its own launches on the stream it runs on (the queue is
kept busy first so the events time the kernels, not the host).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import gen  # noqa: E402

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
METRIC = "routed-expert qGEMM tokens/s, HBM GB/s & MFMA TFLOP/s as % of roofline"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="olmoe_prefill", choices=sorted(gen.CONFIGS))
    ap.add_argument("--no-sub", action="store_true",
                    help="skip the decode and Zipf-prefill objects of the default line")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the HBM / MFMA ceiling probes")
    ap.add_argument("--copies", type=int, default=0, help="weight copies rotated (0: enough to exceed 1 GB)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target length of the CPU oracle sample")
    ap.add_argument("--offload-slots", type=int, default=0,
                    help="INT4 or nested-MWQ layers: keep the experts in pinned host memory with this many GPU slots "
                         "(a separate measurement; routing changes every step)")
    ap.add_argument("--offload-tokens", type=int, default=0,
                    help="with --offload-slots: tokens per step (0: the workload's batch)")
    ap.add_argument("--hbm-probe", action="store_true",
                    help="only time a plain 512 MiB device copy (achievable HBM rate; counter calibration)")
    return ap.parse_args()


def hbm_probe():
    """Achievable HBM rate of a plain device-to-device copy of known size."""
    import torch
    n = 512 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    reps = 20
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record()
        dst.copy_(src)
        b.record()
    torch.cuda.synchronize()
    ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
    gbs = 2 * n / (ms * 1e-3) / 1e9
    print(json.dumps({"probe": "device copy", "bytes_read": n, "bytes_written": n, "ms": round(ms, 4),
                      "gbs_read_plus_write": round(gbs, 1)}), flush=True)


def to_dev(a):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to("cuda:0")


def weight_bytes_per_expert(cfg, matrix):
    """Algorithmic bytes one expert's matrix moves (codes + scales)."""
    H, I, G = cfg.H, cfg.I, cfg.G
    N, K = (2 * I, H) if matrix == "gate_up" else (H, I)
    return N * K // 2 + N * (K // G) * 2


def offload_bench_mwq(args, cfg):
    """Nested-MWQ experts host-resident, loaded plane by plane in HEBF order
    (hottest expert first, q2 -> d3 -> d4, up to the widest width its pairs
    need); 16 seeded routings and width draws in turn.  Against the same with
    every copy finished before any GEMM, and with every expert resident."""
    import torch
    import quantized_moe_expert_top_amd as q
    from quantized_moe_expert_top_amd.offload import OffloadedMwqLayer
    if args.offload_tokens:
        cfg = gen.config(args.config, T=args.offload_tokens)
    data = gen.generate(cfg)
    gu, dn = tiled_weights(q, cfg, data)
    x = to_dev(data["x"])
    draws = [gen.generate(gen.config(args.config, T=cfg.T, seed=cfg.seed + 1000 + i)) for i in range(16)]
    batches = [(to_dev(dd["logits"]), to_dev(dd["pair_bits"])) for dd in draws]
    res = {}
    for mode in ("overlap", "serial"):
        layer = OffloadedMwqLayer(gu, dn, args.offload_slots)
        hits = experts = copied = 0
        t0 = 0.0
        for i in range(args.warmup + args.steps):
            if i == args.warmup:
                torch.cuda.synchronize()
                hits = experts = copied = 0
                t0 = time.perf_counter()
            lg, bits = batches[i % 16]
            _, st = layer.forward(x, lg, cfg.k, bits, overlap=mode != "serial")
            hits, experts, copied = hits + st.hits, experts + st.experts, copied + st.bytes_copied
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        res[mode] = dict(ms=dt / args.steps * 1e3, tps=cfg.T * args.steps / dt, hit=hits / max(experts, 1),
                         mb=copied / args.steps / 1e6, gbs=copied / dt / 1e9)
    for i in range(3):
        q.moe_layer_forward(x, batches[i][0], cfg.k, gu, dn, pair_bits=batches[i][1])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        q.moe_layer_forward(x, batches[i % 16][0], cfg.k, gu, dn, pair_bits=batches[i % 16][1])
    torch.cuda.synchronize()
    resident_ms = (time.perf_counter() - t0) / args.steps * 1e3
    o, n = res["overlap"], res["serial"]
    print(json.dumps({
        "metric": "routed-expert nested-MWQ layer tokens/s with experts in host memory (HEBF plane loading)",
        "value": round(o["tps"], 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(o["ms"], 4), "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{cfg.name}_offload", "slots": args.offload_slots, "experts": cfg.E,
                   "tokens": cfg.T, "top_k": cfg.k, "routings": 16},
        "hit_rate": round(o["hit"], 3), "copied_mb_per_step": round(o["mb"], 2), "h2d_gbs": round(o["gbs"], 2),
        "no_overlap": {"ms_per_step": round(n["ms"], 4), "tokens_s": round(n["tps"], 1), "h2d_gbs": round(n["gbs"], 2)},
        "all_resident_ms_per_step": round(resident_ms, 4),
    }))


def offload_bench(args):
    """Experts host-resident, `--offload-slots` GPU slots, a new routing every step
    (16 seeded logit batches of the workload's distribution, in turn): tokens/s with the
    copies overlapped in hottest-first order and without overlap, hit rate, host-to-device
    bytes per step.  Its own JSON line; not the layer's headline metric."""
    import torch
    import quantized_moe_expert_top_amd as q
    from quantized_moe_expert_top_amd.offload import OffloadedMoeLayer
    cfg = gen.config(args.config)
    if cfg.fmt == "mwq":
        return offload_bench_mwq(args, cfg)
    if cfg.fmt != "int4":
        print(json.dumps({"error": "--offload-slots takes an INT4 or nested-MWQ workload"}))
        sys.exit(2)
    data = gen.generate(cfg)
    gu = q.moe_repack_weights(q.int4_experts(to_dev(data["gu_codes"]), to_dev(data["gu_scales"]), cfg.G))
    dn = q.moe_repack_weights(q.int4_experts(to_dev(data["dn_codes"]), to_dev(data["dn_scales"]), cfg.G))
    x = to_dev(data["x"])
    batches = [to_dev(gen.generate(gen.config(args.config, seed=cfg.seed + 1000 + i))["logits"]) for i in range(16)]
    # the routing of every batch, known ahead (a pre-gating router), for the lookahead variant
    ahead = [q.moe_route_topk(lg, cfg.k)[0].cpu().numpy() for lg in batches]
    res = {}
    for mode in ("overlap", "serial", "lookahead"):
        layer = OffloadedMoeLayer(gu, dn, args.offload_slots)
        hits = experts = copied = 0
        t0 = 0.0
        for i in range(args.warmup + args.steps):
            if i == args.warmup:
                torch.cuda.synchronize()
                hits = experts = copied = 0
                t0 = time.perf_counter()
            _, st = layer.forward(x, batches[i % 16], cfg.k, overlap=mode != "serial")
            hits, experts, copied = hits + st.hits, experts + st.experts, copied + st.bytes_copied
            if mode == "lookahead":
                copied += layer.prefetch(ahead[(i + 1) % 16])
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        res[mode] = dict(ms=dt / args.steps * 1e3, tps=cfg.T * args.steps / dt, hit=hits / max(experts, 1),
                         mb=copied / args.steps / 1e6, gbs=copied / dt / 1e9)
    # the same routings with every expert resident, for context
    for i in range(3):
        q.moe_layer_forward(x, batches[i], cfg.k, gu, dn)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        q.moe_layer_forward(x, batches[i % 16], cfg.k, gu, dn)
    torch.cuda.synchronize()
    resident_ms = (time.perf_counter() - t0) / args.steps * 1e3
    o, n, la = res["overlap"], res["serial"], res["lookahead"]
    print(json.dumps({
        "metric": "routed-expert layer tokens/s with experts in host memory", "value": round(o["tps"], 1),
        "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(o["ms"], 4), "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{cfg.name}_offload", "slots": args.offload_slots, "experts": cfg.E,
                   "tokens": cfg.T, "top_k": cfg.k, "routings": 16},
        "hit_rate": round(o["hit"], 3), "copied_mb_per_step": round(o["mb"], 2),
        "h2d_gbs": round(o["gbs"], 2),
        "no_overlap": {"ms_per_step": round(n["ms"], 4), "tokens_s": round(n["tps"], 1)},
        "lookahead": {"ms_per_step": round(la["ms"], 4), "tokens_s": round(la["tps"], 1),
                      "hit_rate": round(la["hit"], 3), "copied_mb_per_step": round(la["mb"], 2)},
        "all_resident_ms_per_step": round(resident_ms, 4),
    }))


def tiled_weights(q, cfg, data):
    """One tiled copy of a workload's expert weights: (gate_up, down) or (delta,)."""
    if isinstance(cfg, gen.DeltaConfig):
        src = q.delta2_experts(to_dev(data["codes"]), to_dev(data["step"]), to_dev(data["salient_idx"]),
                               to_dev(data["salient_val"]), base=to_dev(data["base"]))
        return (q.moe_repack_weights(src),)
    if cfg.fmt == "int4":
        mk = lambda p: q.int4_experts(to_dev(data[p + "codes"]), to_dev(data[p + "scales"]), cfg.G)  # noqa
    elif cfg.fmt == "mixed":
        mk = lambda p: q.per_expert_experts(to_dev(data[p + "codes"]), to_dev(data[p + "scales"]),  # noqa
                                            data["expert_bits"], data["expert_zero"], cfg.G)
    else:
        mk = lambda p: q.mwq_experts(to_dev(data[p + "q2"]), to_dev(data[p + "d3"]),  # noqa
                                     to_dev(data[p + "d4"]), to_dev(data[p + "scales"]), cfg.G)
    return q.moe_repack_weights(mk("gu_")), q.moe_repack_weights(mk("dn_"))


def touched_weight_bytes(cfg, data, counts, seg_offsets, matrix):
    """Algorithmic weight bytes of one GEMM of the layer: codes + scales of the
    experts that received rows (nested planes: only the planes their widths need)."""
    H, I, G = cfg.H, cfg.I, cfg.G
    N, K = (2 * I, H) if matrix == "gate_up" else (H, I)
    scales = N * (K // G) * 2
    wb = 0
    if cfg.fmt == "mixed":
        for e in range(cfg.E):
            if counts[e] > 0:
                wb += N * K * int(data["expert_bits"][e]) // 8 + scales
    elif cfg.fmt == "mwq":
        segs = np.diff(seg_offsets).reshape(cfg.E, 3)  # b = 4, 3, 2
        for e in range(cfg.E):
            if segs[e].sum() == 0:
                continue
            wb += N * K // 4 + scales
            wb += N * K // 8 if segs[e][0] + segs[e][1] > 0 else 0
            wb += N * K // 8 if segs[e][0] > 0 else 0
    else:
        wb = int((counts > 0).sum()) * (N * K // 2 + scales)
    return wb


def kernel_ms(fn, ncopies, steps):
    """Mean duration of one launch of fn(copy): HIP events on the current stream
    around batches of back-to-back launches (weight copies rotated), the queue
    kept busy first so that the events time the kernels and not the host."""
    import torch
    stream = torch.cuda.current_stream()
    batch, nbatch = 20, max(5, min(steps // 20, 20))
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nbatch)]
    for i in range(nbatch):
        torch.cuda._sleep(1_000_000)
        evs[i][0].record(stream)
        for j in range(batch):
            fn((i * batch + j) % ncopies)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in evs]) / batch)


def run_workload(q, name, steps, warmup, copies_arg=0):
    """Times `steps` graph replays of one layer step (after `warmup`), then the
    dominant kernel on its own.  Returns the measurements and what they rest on."""
    import torch
    cfg = gen.config(name)
    data = gen.generate(cfg)
    delta = isinstance(cfg, gen.DeltaConfig)
    dev = torch.device("cuda:0")
    first = tiled_weights(q, cfg, data)
    per_copy = sum(sum(t.numel() * t.element_size() for t in w.tensors.values()) for w in first)
    ncopies = copies_arg or max(2, int(np.ceil(1.0e9 / per_copy)))
    copies = [first] + [tiled_weights(q, cfg, data) for _ in range(ncopies - 1)]
    torch.cuda.synchronize()

    T, k = cfg.T, cfg.k
    x = to_dev(data["x"])
    if delta:
        ids = to_dev(data["ids"]).view(T, 1)
        perm = q.moe_permute(ids, cfg.E)
        y_perm = torch.empty((T, cfg.N), dtype=torch.bfloat16, device=dev)
        out = torch.empty((T, cfg.N), dtype=torch.bfloat16, device=dev)

        def step(c):
            q.moe_permute(ids, cfg.E, out=perm)
            q.moe_grouped_qgemm(copies[c][0], x, perm.seg_offsets, T, q.MOE_EPI_NONE,
                                gather_pair=perm.sorted_pair, k=1, out=y_perm)
            q.moe_unpermute_combine(y_perm, perm.pair_pos, None, T, 1, out=out)

        def dominant(c):
            q.moe_grouped_qgemm(copies[c][0], x, perm.seg_offsets, T, q.MOE_EPI_NONE,
                                gather_pair=perm.sorted_pair, k=1, out=y_perm)
    else:
        logits = to_dev(data["logits"])
        bits = to_dev(data["pair_bits"]) if cfg.fmt == "mwq" else None
        buf = q.alloc_layer(T, cfg.E, k, cfg.H, cfg.I, bits is not None, dev)

        def step(c):
            q.moe_layer_forward(x, logits, k, copies[c][0], copies[c][1], pair_bits=bits, buf=buf)

        def dominant(c):
            q.moe_grouped_qgemm(copies[c][0], x, buf.perm.seg_offsets, T * k, q.MOE_EPI_SWIGLU,
                                gather_pair=buf.perm.sorted_pair, k=k, out=buf.h)

    # eager run (first-call device checks happen outside capture), then one graph per weight copy
    for c in range(ncopies):
        step(c)
    torch.cuda.synchronize()
    graphs = []
    for c in range(ncopies):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(c)
        graphs.append(g)
    torch.cuda.synchronize()
    for i in range(warmup):
        graphs[i % ncopies].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        graphs[i % ncopies].replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    dom_ms = kernel_ms(dominant, ncopies, steps)

    # algorithmic bytes / flops of one dominant launch and of the whole step
    if delta:
        wbytes = cfg.N * cfg.K * 2 + cfg.E * cfg.N * (cfg.K // 4 + 2 + 2 * cfg.n_salient)
        dom_bytes = wbytes + T * cfg.K * 2 + T * cfg.N * 2
        dom_flops = 2.0 * T * cfg.K * cfg.N * 2
        layer_bytes, layer_flops = dom_bytes, dom_flops
        dom_name = "qgemm delta2 (base + 2-bit delta + salient)"
        touched = cfg.E
    else:
        counts = buf.perm.counts.cpu().numpy()
        seg = buf.perm.seg_offsets.cpu().numpy()
        touched = int((counts > 0).sum())
        rows = T * k
        wb_gu = touched_weight_bytes(cfg, data, counts, seg, "gate_up")
        wb_dn = touched_weight_bytes(cfg, data, counts, seg, "down")
        dom_bytes = wb_gu + T * cfg.H * 2 + rows * cfg.I * 2 + rows * 4 + (cfg.E + 1) * 4
        dom_flops = 2.0 * rows * cfg.H * 2 * cfg.I
        layer_bytes = wb_gu + wb_dn + T * cfg.H * 2 * 2 + T * cfg.E * 4   # weights, x, out, logits
        layer_flops = 6.0 * rows * cfg.H * cfg.I
        dom_name = "qgemm gate_up + SwiGLU"
    return dict(cfg=cfg, data=data, delta=delta, touched=touched, ncopies=ncopies, steps=steps, warmup=warmup,
                ms_per_step=elapsed * 1e3 / max(steps, 1), tokens_per_s=T * steps / elapsed, dom_ms=dom_ms,
                dom_bytes=dom_bytes, dom_flops=dom_flops, dom_name=dom_name, layer_bytes=layer_bytes,
                layer_flops=layer_flops)


HBM_BOUND = ("olmoe_decode", "mixtral_mwq_decode", "olmoe_mixed_decode", "olmoe_edge_decode", "tiny")


def roofline_of(r, ceilings):
    """The dominant kernel against its roofline (vendor peak, and the ceiling
    measured on this GPU by the probes)."""
    cfg = r["cfg"]
    gbs = r["dom_bytes"] / (r["dom_ms"] * 1e-3) / 1e9
    tflops = r["dom_flops"] / (r["dom_ms"] * 1e-3) / 1e12
    hbm = cfg.name in HBM_BOUND
    out = ({"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4)} if hbm else
           {"bound": "mfma", "achieved": round(tflops, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tflops / BF16_PEAK_TFLOPS, 4)})
    out["traffic"] = measured_traffic(cfg.name)
    meas = (ceilings or {}).get("hbm_stream_gbs" if hbm else "mfma_bf16_tflops")
    out.update({"measured_peak": meas, "frac_measured": round(out["achieved"] / meas, 4) if meas else None,
                "kernel": r["dom_name"], "kernel_ms": round(r["dom_ms"], 5),
                "algorithmic_bytes": int(r["dom_bytes"]), "algorithmic_flops": r["dom_flops"],
                "gbs": round(gbs, 1), "tflops": round(tflops, 2)})
    return out


def layer_summary(r, ceilings):
    """A whole step of one workload: throughput, and the step against the roofline
    of everything the layer must move (decode) or compute (prefill)."""
    cfg = r["cfg"]
    s = r["ms_per_step"] * 1e-3
    hbm = cfg.name in HBM_BOUND
    gbs = r["layer_bytes"] / s / 1e9
    tflops = r["layer_flops"] / s / 1e12
    d = {"workload": cfg.name, "tokens": cfg.T, "steps": r["steps"], "ms_per_step": round(r["ms_per_step"], 5),
         "tokens_s": round(r["tokens_per_s"], 1), "touched_experts": r["touched"],
         "layer_algorithmic_bytes": int(r["layer_bytes"]), "layer_algorithmic_flops": r["layer_flops"]}
    if hbm:
        meas = (ceilings or {}).get("hbm_stream_gbs")
        d.update({"layer_gbs": round(gbs, 1), "layer_frac": round(gbs / HBM_PEAK_GBS, 4),
                  "layer_frac_measured": round(gbs / meas, 4) if meas else None})
    else:
        meas = (ceilings or {}).get("mfma_bf16_tflops")
        d.update({"layer_tflops": round(tflops, 1), "layer_frac": round(tflops / BF16_PEAK_TFLOPS, 4),
                  "layer_frac_measured": round(tflops / meas, 4) if meas else None})
    d["roofline"] = roofline_of(r, ceilings)
    return d


def measure_ceilings():
    """Achievable HBM read rate and bf16 MFMA rate of this GPU, from the probe
    kernels (libmoe_probe.so): a cold streaming read of the decode gate_up
    working set (83 MB, buffers rotated through 1.3 GB so none is cached) and
    of 1 GB, and a register-only MFMA loop on every CU."""
    import ctypes
    import torch
    from quantized_moe_expert_top_amd import build as b
    if not os.path.exists(b.PROBE_LIB):
        return None
    lib = ctypes.CDLL(b.PROBE_LIB)
    lib.moe_probe_stream_read.restype = ctypes.c_int
    lib.moe_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                          ctypes.c_void_p]
    lib.moe_probe_mfma_loop.restype = ctypes.c_int
    lib.moe_probe_mfma_loop.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream
    blocks = 256 * 8
    sink = torch.empty(blocks, dtype=torch.int32, device="cuda:0")

    def stream_gbs(nbytes, nbuf):
        bufs = [torch.ones(nbytes // 4, dtype=torch.int32, device="cuda:0") for _ in range(nbuf)]
        fn = lambda c: lib.moe_probe_stream_read(bufs[c].data_ptr(), nbytes, sink.data_ptr(), blocks, sptr)  # noqa
        for c in range(nbuf):
            fn(c)
        ms = kernel_ms(fn, nbuf, 200)
        del bufs
        return nbytes / (ms * 1e-3) / 1e9

    res = {"hbm_stream_gbs": round(stream_gbs(83 << 20, 16), 1), "hbm_stream_1gb_gbs": round(stream_gbs(1 << 30, 3), 1)}
    iters, mblocks = 4096, 256 * 8
    out = torch.empty(mblocks * 256, dtype=torch.float32, device="cuda:0")
    fn = lambda c: lib.moe_probe_mfma_loop(iters, mblocks, out.data_ptr(), sptr)  # noqa
    fn(0)
    ms = kernel_ms(fn, 1, 100)
    flops = mblocks * 4 * 8 * iters * 16384.0
    res["mfma_bf16_tflops"] = round(flops / (ms * 1e-3) / 1e12, 1)
    torch.cuda.synchronize()
    return res


def main():
    args = parse()
    if args.hbm_probe:
        hbm_probe()
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the library and this benchmark run on one GPU; --gpus must be 1 "
                                   "(no collective or multi-GPU path exists)"}), flush=True)
        sys.exit(2)
    if args.offload_slots:
        offload_bench(args)
        return
    import torch  # noqa: F401
    import quantized_moe_expert_top_amd as q

    ceilings = None if args.no_ceilings else measure_ceilings()
    r = run_workload(q, args.config, args.steps, args.warmup, args.copies)
    cfg = r["cfg"]
    head = layer_summary(r, ceilings)
    extra = {}
    if not args.no_sub and args.config == "olmoe_prefill":
        # the two other halves of the target on the same layer: the decode batch (HBM) and Zipf-skewed prefill
        extra["decode"] = layer_summary(run_workload(q, "olmoe_decode", 200, 20), ceilings)
        extra["zipf"] = layer_summary(run_workload(q, "olmoe_prefill_zipf", max(args.steps, 20), 5), ceilings)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, r["data"], args.cpu_seconds)
    delta = r["delta"]
    line = {
        "metric": METRIC, "value": round(r["tokens_per_s"], 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; random-init quantized experts)",
        "config": {"workload": cfg.name, "tokens": cfg.T,
                   **({"in": cfg.K, "out": cfg.N, "experts": cfg.E, "format": "delta2+salient+base"} if delta else
                      {"hidden": cfg.H, "intermediate": cfg.I, "experts": cfg.E, "top_k": cfg.k,
                       "format": f"{cfg.fmt}_g{cfg.G}", "zipf": cfg.zipf, "touched_experts": r["touched"]}),
                   "weight_copies": r["ncopies"], "parallelism": "single GPU"},
        "roofline": head["roofline"],
        "layer": {k_: v for k_, v in head.items() if k_.startswith("layer_")},
        **extra,
        "ceilings": ceilings,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def measured_traffic(workload):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3
    counters (profiles/traffic.json: FETCH_SIZE and WRITE_SIZE per dispatch,
    scaled by a plain copy's readings), or None when that file has no entry
    for the workload or was taken on a different qgemm.hip."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    src = os.path.join(ROOT, "quantized_moe_expert_top_amd", "csrc", "qgemm.hip")
    try:
        t = json.load(open(path))
        if hashlib.sha256(open(src, "rb").read()).hexdigest() != t["qgemm_hip_sha256"]:
            return None
        w = t["workloads"][workload]
    except (OSError, KeyError, ValueError):
        return None
    return int((w["fetch_kib"] * t["fetch_scale"] + w["write_kib"] * t["write_scale"]) * 1024)


def cpu_baseline(cfg, data, target_s):
    """Times the C++17 float64 oracle as it stands (oracle/moe_oracle.cpp:
    std::thread over work items, hardware_concurrency() threads capped by this
    process's CPU share (OMP_NUM_THREADS), every sum in a fixed order) on this
    host's cores, on a bounded sample of the same
    workload: whole batches, repeated until about target_s seconds (one batch
    of the largest workloads takes about that long on its own)."""
    from oracle import cpp
    threads = cpp.default_threads()
    delta = isinstance(cfg, gen.DeltaConfig)
    T = cfg.T

    def run(tokens):
        t0 = time.perf_counter()
        if delta:
            cpp.delta_linear(data, cfg, tokens=tokens, threads=threads)
        else:
            cpp.moe_forward(data, cfg, tokens=tokens, threads=threads, intermediates=False)
        return time.perf_counter() - t0

    reps, el = 0, 0.0
    while el < target_s and reps < 200:
        el += run(None)
        reps += 1
    done, what = reps * T, f"{reps} x full batch"
    return {"value": round(done / el, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{what} of {cfg.name}, C++17 float64 oracle on {threads} threads "
                      f"(hardware_concurrency {cpp.hardware_threads()}), {el:.1f} s"}


if __name__ == "__main__":
    main()

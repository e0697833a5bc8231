"""Benchmark of the routed-expert quantized MoE hot path on one MI355X.

A step is one whole layer on one batch of synthetic input, inputs already
resident in HBM: route (top-k) -> group (permute) -> grouped qGEMM gate_up with
SwiGLU -> grouped qGEMM down -> gate-weighted combine (the delta workload:
group -> grouped delta linear with the shared base -> scatter back).  Each step
is one HIP-graph replay.  Several copies of the expert weights are rotated so
that a step never finds its weights in the 256 MB Infinity Cache (a real model
has many layers, each with its own experts).

Default workload: the decode-shaped OLMoE-like layer (32 tokens, 64 experts,
top-8, hidden 2048, SwiGLU 1024, INT4 g128, Zipf(1.1) popularity).

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
    ap.add_argument("--config", default="olmoe_decode", choices=sorted(gen.CONFIGS))
    ap.add_argument("--copies", type=int, default=0, help="weight copies rotated (0: enough to exceed 1 GB)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target length of the CPU oracle sample")
    ap.add_argument("--offload-slots", type=int, default=0,
                    help="INT4 layers: keep the experts in pinned host memory with this many GPU slots "
                         "(a separate measurement; routing changes every step)")
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


def offload_bench(args):
    """Experts host-resident, `--offload-slots` GPU slots, a new routing every step
    (16 seeded logit batches of the workload's distribution, in turn): tokens/s with the
    copies overlapped in hottest-first order and without overlap, hit rate, host-to-device
    bytes per step.  Its own JSON line; not the layer's headline metric."""
    import torch
    import quantized_moe_expert_top_amd as q
    from quantized_moe_expert_top_amd.offload import OffloadedMoeLayer
    cfg = gen.config(args.config)
    if cfg.fmt != "int4":
        print(json.dumps({"error": "--offload-slots takes an INT4 workload"}))
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


def main():
    args = parse()
    if args.hbm_probe:
        hbm_probe()
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    if args.offload_slots:
        offload_bench(args)
        return
    import torch
    import quantized_moe_expert_top_amd as q

    cfg = gen.config(args.config)
    data = gen.generate(cfg)
    delta = isinstance(cfg, gen.DeltaConfig)
    dev = torch.device("cuda:0")

    # ---- weights: canonical upload, repack, several copies
    def tiled_copy():
        if delta:
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

    first = tiled_copy()
    per_copy = sum(sum(t.numel() * t.element_size() for t in w.tensors.values()) for w in first)
    ncopies = args.copies or max(2, int(np.ceil(1.0e9 / per_copy)))
    copies = [first] + [tiled_copy() for _ in range(ncopies - 1)]
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

    for i in range(args.warmup):
        graphs[i % ncopies].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        graphs[i % ncopies].replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0
    ms_per_step = elapsed * 1e3 / max(args.steps, 1)
    tokens_per_s = T * args.steps / elapsed

    # ---- dominant kernel: HIP events on its own stream around batches of
    # back-to-back launches (weight copies rotated); the queue is kept busy
    # first, so the events time the kernels and not the host.  Per launch =
    # batch time / batch size (one event pair per launch would add the
    # dispatch latency of every launch to a ~20 us kernel).
    stream = torch.cuda.current_stream()
    batch, nbatch = 20, max(5, min(args.steps // 20, 20))
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nbatch)]
    for i in range(nbatch):
        torch.cuda._sleep(1_000_000)
        evs[i][0].record(stream)
        for j in range(batch):
            dominant((i * batch + j) % ncopies)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    durs_ms = np.array([a.elapsed_time(b) for a, b in evs]) / batch
    dom_ms = float(np.mean(durs_ms))

    # algorithmic bytes / flops of one dominant launch
    if delta:
        rows = T
        wbytes = cfg.N * cfg.K * 2 + cfg.E * cfg.N * (cfg.K // 4 + 2 + 2 * cfg.n_salient)
        dom_bytes = wbytes + T * cfg.K * 2 + T * cfg.N * 2
        dom_flops = 2.0 * T * cfg.K * cfg.N * 2
        dom_name = "qgemm delta2 (base + 2-bit delta + salient)"
        touched = cfg.E
    else:
        counts = (buf.perm.counts.cpu().numpy())
        touched = int((counts > 0).sum())
        rows = T * k
        per_e = weight_bytes_per_expert(cfg, "gate_up")
        if cfg.fmt in ("mwq", "mixed"):
            per_e = None
        if cfg.fmt == "mixed":
            # each touched expert's codes at its own width + scales
            N, K = 2 * cfg.I, cfg.H
            wb = sum(N * K * int(data["expert_bits"][e]) // 8 + N * (K // cfg.G) * 2
                     for e in range(cfg.E) if counts[e] > 0)
        elif per_e is None:
            # nested planes: q2 + scales always, d3 / d4 only for experts with b >= 3 / b == 4 rows
            segs = np.diff(buf.perm.seg_offsets.cpu().numpy()).reshape(cfg.E, 3)  # b = 4, 3, 2
            N, K = 2 * cfg.I, cfg.H
            wb = 0
            for e in range(cfg.E):
                if segs[e].sum() == 0:
                    continue
                wb += N * K // 4 + N * (K // cfg.G) * 2
                wb += N * K // 8 if segs[e][0] + segs[e][1] > 0 else 0
                wb += N * K // 8 if segs[e][0] > 0 else 0
        else:
            wb = touched * per_e
        dom_bytes = wb + T * cfg.H * 2 + rows * cfg.I * 2 + rows * 4 + (cfg.E + 1) * 4
        dom_flops = 2.0 * rows * cfg.H * 2 * cfg.I
        dom_name = "qgemm gate_up + SwiGLU"
    gbs = dom_bytes / (dom_ms * 1e-3) / 1e9
    tflops = dom_flops / (dom_ms * 1e-3) / 1e12
    hbm_bound = cfg.name in ("olmoe_decode", "mixtral_mwq_decode", "olmoe_mixed_decode", "tiny")
    roofline = ({"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                 "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None}
                if hbm_bound else
                {"bound": "mfma", "achieved": round(tflops, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                 "frac": round(tflops / BF16_PEAK_TFLOPS, 4), "traffic": None})
    roofline["traffic"] = measured_traffic(cfg.name)
    roofline.update({"kernel": dom_name, "kernel_ms": round(dom_ms, 5), "algorithmic_bytes": int(dom_bytes),
                     "algorithmic_flops": dom_flops, "gbs": round(gbs, 1), "tflops": round(tflops, 2)})

    # ---- CPU baseline: the float64 oracle on a bounded sample of the same workload
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, data, args.cpu_seconds)

    line = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; random-init quantized experts)",
        "config": {"workload": cfg.name, "tokens": T,
                   **({"in": cfg.K, "out": cfg.N, "experts": cfg.E, "format": "delta2+salient+base"} if delta else
                      {"hidden": cfg.H, "intermediate": cfg.I, "experts": cfg.E, "top_k": k,
                       "format": f"{cfg.fmt}_g{cfg.G}", "zipf": cfg.zipf, "touched_experts": touched}),
                   "weight_copies": ncopies, "parallelism": "single GPU"},
        "roofline": roofline,
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
    """Times the oracle as it stands on this host's cores."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        threads = 1
    delta = isinstance(cfg, gen.DeltaConfig)
    T = cfg.T
    # sample: whole batches for small workloads, else a token subset
    sample_tokens = None
    if cfg.name not in ("olmoe_decode", "mixtral_mwq_decode", "olmoe_mixed_decode", "tiny"):
        sample_tokens = np.arange(0, T, max(1, T // 16))[:16]
    done = 0
    t0 = time.perf_counter()
    reps = 0
    while True:
        if delta:
            oracle.delta_linear(data, cfg, tokens=sample_tokens)
        else:
            oracle.moe_forward(data, cfg, tokens=sample_tokens)
        reps += 1
        done += T if sample_tokens is None else len(sample_tokens)
        if time.perf_counter() - t0 >= target_s or reps >= 50:
            break
    el = time.perf_counter() - t0
    what = "full batch" if sample_tokens is None else f"{len(sample_tokens)} of {T} tokens (routing of all)"
    return {"value": round(done / el, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{reps} x {what} of {cfg.name}, float64 numpy oracle, {el:.1f} s"}


if __name__ == "__main__":
    main()

"""Host-resident experts with a GPU slot cache (expert offload on one GPU).

The routed experts' tiled INT4 weights live in pinned host memory; the GPU
holds `n_slots` expert slots.  Each layer step routes and groups on the GPU,
reads the per-expert counts back, and then walks the touched experts hottest
first: an expert already in a slot is computed at once, a missing one is
copied into a free or least recently used slot on a copy stream while the
experts before it are computed, and its GEMMs wait only for its own copy.

Pages: D2MoE (bit-width-aware I/O-compute pipeline: Load E2 in parallel with
Compute E1; HEBF, the hottest expert first), ExactMoE (GPU-resident slot cache
with host-resident experts), EdgeMoE (expert buffer for experts kept in
external storage).  With INT4 weights there is no bit order to follow inside
an expert.

Host logic only: every arithmetic step runs in the library's kernels (the
grouped GEMM on a one-expert view of a slot, then the combine over all
pairs); copies are stream-ordered host-to-device copies from pinned memory.
"""
from __future__ import annotations

import dataclasses

import torch

from . import (MOE_EPI_NONE_F32, MOE_EPI_SWIGLU, MOE_LAYOUT_TILED, MOE_W_INT4_GROUP, QuantizedExperts,
               make_desc, moe_grouped_qgemm, moe_route_permute, moe_unpermute_combine)


@dataclasses.dataclass
class OffloadStats:
    experts: int = 0       # distinct experts touched
    hits: int = 0          # of them already in a slot
    bytes_copied: int = 0  # host-to-device bytes of this step


class _HostExperts:
    """One tiled INT4 weight set split per expert: pinned host copies and S device slots."""

    def __init__(self, tiled: QuantizedExperts, n_slots: int, device):
        d = tiled.desc
        if d.format != MOE_W_INT4_GROUP or d.layout != MOE_LAYOUT_TILED:
            raise ValueError("expert offload takes tiled INT4 weights")
        self.E, self.N, self.K, self.G, self.z = d.E, d.N, d.K, d.group_size, d.zero_point
        codes = tiled.tensors["codes"].view(self.E, -1)
        scales = tiled.tensors["scales"].reshape(self.E, -1)
        self.host_codes = torch.empty(codes.shape, dtype=codes.dtype, pin_memory=True)
        self.host_scales = torch.empty(scales.shape, dtype=scales.dtype, pin_memory=True)
        self.host_codes.copy_(codes)
        self.host_scales.copy_(scales)
        self.slot_codes = torch.empty((n_slots, codes.shape[1]), dtype=codes.dtype, device=device)
        self.slot_scales = torch.empty((n_slots, scales.shape[1]), dtype=scales.dtype, device=device)
        # a one-expert descriptor per slot: the grouped GEMM runs on it unchanged
        self.views = [make_desc(MOE_W_INT4_GROUP, MOE_LAYOUT_TILED, 1, self.N, self.K, self.G, self.z,
                                codes=self.slot_codes[s], scales=self.slot_scales[s]) for s in range(n_slots)]
        self.expert_bytes = codes.shape[1] * codes.element_size() + scales.shape[1] * scales.element_size()

    def copy_in(self, e: int, s: int):
        self.slot_codes[s].copy_(self.host_codes[e], non_blocking=True)
        self.slot_scales[s].copy_(self.host_scales[e], non_blocking=True)


class OffloadedMoeLayer:
    """A routed-expert INT4 layer whose experts stay in host memory between uses."""

    def __init__(self, gate_up: QuantizedExperts, down: QuantizedExperts, n_slots: int, device=None):
        device = device or torch.device("cuda", torch.cuda.current_device())
        self.gu = _HostExperts(gate_up, n_slots, device)
        self.dn = _HostExperts(down, n_slots, device)
        if self.gu.E != self.dn.E:
            raise ValueError("gate_up and down have different expert counts")
        self.E, self.S = self.gu.E, n_slots
        self.I, self.H = self.gu.N // 2, self.dn.N
        self.slot_of: dict[int, int] = {}
        self.expert_in = [-1] * n_slots
        self.last_use = [0] * n_slots
        self.step = 0
        self.copy_stream = torch.cuda.Stream(device=device)  # default priority

    def _assign(self, hot):
        """Slots for this step's experts (hottest first): hits keep theirs; misses take
        a free slot, else the least recently used one not needed in this step."""
        needed = set(hot)
        misses = []
        for e in hot:
            s = self.slot_of.get(e)
            if s is None:
                free = [j for j in range(self.S) if self.expert_in[j] < 0]
                if free:
                    s = free[0]
                else:
                    cand = [j for j in range(self.S) if self.expert_in[j] not in needed]
                    s = min(cand, key=lambda j: self.last_use[j])
                    del self.slot_of[self.expert_in[s]]
                self.slot_of[e] = s
                self.expert_in[s] = e
                misses.append(e)
            self.last_use[s] = self.step
        return misses

    def forward(self, x: torch.Tensor, logits: torch.Tensor, k: int, overlap: bool = True):
        """Returns (out bf16 [T][H], OffloadStats).  overlap=False copies every missing
        expert before computing any (the load-then-compute baseline)."""
        T = x.shape[0]
        P = T * k
        ids, w, perm = moe_route_permute(logits, k)
        counts = perm.counts.cpu()  # the host schedules the copies from the counts
        hot = sorted((e for e in range(self.E) if counts[e] > 0), key=lambda e: (-int(counts[e]), e))
        if len(hot) > self.S:
            raise ValueError(f"{len(hot)} experts touched, {self.S} slots")
        self.step += 1
        misses = self._assign(hot)
        stats = OffloadStats(len(hot), len(hot) - len(misses), len(misses) * (self.gu.expert_bytes +
                                                                             self.dn.expert_bytes))
        compute = torch.cuda.current_stream()
        # the copies may overwrite slots that earlier work still reads
        self.copy_stream.wait_stream(compute)
        ready = {}
        with torch.cuda.stream(self.copy_stream):
            for e in misses:
                s = self.slot_of[e]
                self.gu.copy_in(e, s)
                self.dn.copy_in(e, s)
                ev = torch.cuda.Event()
                ev.record(self.copy_stream)
                ready[e] = ev
        if not overlap and misses:
            compute.wait_event(ready[misses[-1]])
        # expert e's rows are [first[e], first[e] + counts[e]) of the grouped order; each
        # expert's GEMMs run on views that start at its first row, with its own segment [0, c)
        first = [0] * (self.E + 1)
        for e in range(self.E):
            first[e + 1] = first[e] + int(counts[e])
        segs = torch.tensor([[0, int(counts[e])] for e in hot], dtype=torch.int32).to(x.device, non_blocking=True)
        h = torch.empty((P, self.I), dtype=torch.bfloat16, device=x.device)
        y = torch.empty((P, self.H), dtype=torch.float32, device=x.device)
        for j, e in enumerate(hot):
            if overlap and e in ready:
                compute.wait_event(ready[e])
            s, r0, c = self.slot_of[e], first[e], int(counts[e])
            moe_grouped_qgemm(self.gu.views[s], x, segs[j], c, MOE_EPI_SWIGLU, gather_pair=perm.sorted_pair[r0:],
                              k=k, out=h[r0:])
            moe_grouped_qgemm(self.dn.views[s], h[r0:r0 + c], segs[j], c, MOE_EPI_NONE_F32, out=y[r0:])
        out = moe_unpermute_combine(y, perm.pair_pos, w, T, k)
        return out, stats

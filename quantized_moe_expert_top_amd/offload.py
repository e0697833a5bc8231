"""Host-resident experts with a GPU slot cache (expert offload on one GPU).

The routed experts' tiled INT4 weights live in pinned host memory; the GPU
holds `n_slots` expert slots.  Each layer step routes on the GPU and reads the
expert ids back; the host gives every touched expert a slot (hits keep
theirs, misses take a free or the least recently used slot) and queues the
misses' copies hottest first on a copy stream.  The pairs are grouped by
(phase, slot): phase 0 holds the experts already resident, phase 1 the ones
being copied, so one grouped GEMM over the slots computes every resident
expert while the copies run, and a second one the copied experts after them.

Pages: D2MoE (bit-width-aware I/O-compute pipeline: Load E2 in parallel with
Compute E1; HEBF, the hottest expert first), ExactMoE (GPU-resident slot cache
with host-resident experts), EdgeMoE (expert buffer for experts kept in
external storage).  With INT4 weights there is no bit order to follow inside
an expert.  Nested-MWQ experts (OffloadedMwqLayer) follow it: an expert's q2
plane is copied before its d3 plane, d3 before d4, and only up to the widest
width its pairs ask for; the rows of width b start once the planes up to b
have landed.

Host logic only: every arithmetic step runs in the library's kernels
(routing, grouping, the grouped GEMMs on the slot buffer, the combine); the
host remaps expert ids to grouping keys and issues stream-ordered copies from
pinned memory.
"""
from __future__ import annotations

import dataclasses

import torch

import numpy as np

from . import (MOE_EPI_NONE_F16, MOE_EPI_SWIGLU, MOE_LAYOUT_TILED, MOE_W_INT4_GROUP, MOE_W_MWQ_2_3_4,
               QuantizedExperts, make_desc, moe_copy_rows_async, moe_grouped_qgemm, moe_permute, moe_route_topk,
               moe_unpermute_combine)


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
        # the slots as an S-expert weight set: the grouped GEMM runs on it unchanged
        self.view = make_desc(MOE_W_INT4_GROUP, MOE_LAYOUT_TILED, n_slots, self.N, self.K, self.G, self.z,
                              codes=self.slot_codes, scales=self.slot_scales)
        self.expert_bytes = codes.shape[1] * codes.element_size() + scales.shape[1] * scales.element_size()

    def copy_in(self, e: int, s: int):
        self.slot_codes[s].copy_(self.host_codes[e], non_blocking=True)
        self.slot_scales[s].copy_(self.host_scales[e], non_blocking=True)


class _SlotCache:
    """Which expert each GPU slot holds, least recently used first out."""

    def _init_slots(self, n_slots: int, device):
        self.S = n_slots
        self.slot_of: dict[int, int] = {}
        self.expert_in = [-1] * n_slots
        self.last_use = [0] * n_slots
        self.step = 0
        self.copy_stream = torch.cuda.Stream(device=device)  # default priority

    def _intermediates(self, P: int, device):
        """The step's h (bf16 [P][I]) and expert outputs y (fp16 [P][H]), kept from
        one step to the next of the same size (every use is ordered on the compute
        stream)."""
        hy = getattr(self, "_hy", None)
        if hy is None or hy[0].shape[0] != P or hy[0].device != device:
            hy = (torch.empty((P, self.I), dtype=torch.bfloat16, device=device),
                  torch.empty((P, self.H), dtype=torch.float16, device=device))
            self._hy = hy
        return hy

    def _assign(self, hot, keep=()):
        """Slots for this step's experts (hottest first): hits keep theirs; misses take
        a free slot, else the least recently used one holding none of `hot` or `keep`."""
        needed = set(hot) | set(keep)
        misses = []
        for e in hot:
            s = self.slot_of.get(e)
            if s is None:
                free = [j for j in range(self.S) if self.expert_in[j] < 0]
                if free:
                    s = free[0]
                else:
                    cand = [j for j in range(self.S) if self.expert_in[j] not in needed]
                    if not cand:
                        return None
                    s = min(cand, key=lambda j: self.last_use[j])
                    del self.slot_of[self.expert_in[s]]
                self.slot_of[e] = s
                self.expert_in[s] = e
                misses.append(e)
            self.last_use[s] = self.step
        return misses


class OffloadedMoeLayer(_SlotCache):
    """A routed-expert INT4 layer whose experts stay in host memory between uses."""

    def __init__(self, gate_up: QuantizedExperts, down: QuantizedExperts, n_slots: int, device=None):
        device = device or torch.device("cuda", torch.cuda.current_device())
        self.gu = _HostExperts(gate_up, n_slots, device)
        self.dn = _HostExperts(down, n_slots, device)
        if self.gu.E != self.dn.E:
            raise ValueError("gate_up and down have different expert counts")
        self.E = self.gu.E
        self.I, self.H = self.gu.N // 2, self.dn.N
        self._init_slots(n_slots, device)
        self.pending: dict[int, torch.cuda.Event] = {}  # slot -> copy issued ahead of its step

    def forward(self, x: torch.Tensor, logits: torch.Tensor, k: int, overlap: bool = True):
        """Returns (out bf16 [T][H], OffloadStats).  overlap=False copies every missing
        expert before computing any (the load-then-compute baseline)."""
        T = x.shape[0]
        P = T * k
        S = self.S
        ids, w = moe_route_topk(logits, k)
        ids_h = ids.cpu().numpy()  # the host schedules the copies from the routing
        counts = np.bincount(ids_h.ravel(), minlength=self.E)
        hot = sorted((e for e in range(self.E) if counts[e] > 0), key=lambda e: (-int(counts[e]), e))
        if len(hot) > S:
            raise ValueError(f"{len(hot)} experts touched, {S} slots")
        self.step += 1
        misses = self._assign(hot)
        if misses is None:
            raise ValueError("no slot left")
        stats = OffloadStats(len(hot), len(hot) - len(misses), len(misses) * (self.gu.expert_bytes +
                                                                             self.dn.expert_bytes))
        # grouping key of a pair: its expert's slot, plus S if that expert is being copied
        key_of = np.zeros(self.E, dtype=np.int32)
        for e in hot:
            key_of[e] = self.slot_of[e]
        for e in misses:
            key_of[e] += S
        keys = torch.from_numpy(key_of[ids_h]).to(x.device)
        perm = moe_permute(keys, 2 * S)
        compute = torch.cuda.current_stream()
        # the copies may overwrite slots that earlier work still reads
        self.copy_stream.wait_stream(compute)
        done = None
        if misses:
            with torch.cuda.stream(self.copy_stream):
                for e in misses:  # hottest first
                    s = self.slot_of[e]
                    self.gu.copy_in(e, s)
                    self.dn.copy_in(e, s)
                done = torch.cuda.Event()
                done.record(self.copy_stream)
            if not overlap:
                compute.wait_event(done)
        for e in hot:  # resident experts whose copy was issued ahead
            ev = self.pending.pop(self.slot_of[e], None)
            if ev is not None and e not in misses:
                compute.wait_event(ev)
        self._current = set(hot)
        h, y = self._intermediates(P, x.device)
        for phase in (0, 1):
            if phase == 1:
                if not misses:
                    break
                compute.wait_event(done)
            seg = perm.seg_offsets[phase * S:phase * S + S + 1]  # rows of this phase's slots
            moe_grouped_qgemm(self.gu.view, x, seg, P, MOE_EPI_SWIGLU, gather_pair=perm.sorted_pair, k=k, out=h)
            moe_grouped_qgemm(self.dn.view, h, seg, P, MOE_EPI_NONE_F16, out=y)
        out = moe_unpermute_combine(y, perm.pair_pos, w, T, k)
        return out, stats

    def prefetch(self, next_ids) -> int:
        """Lookahead with routing known ahead (Read-ME page: a pre-gating router
        routes before the layer runs): copy the experts of the next batch
        (expert ids, host array [T][k]) that are not resident, hottest first, into
        slots the current step does not use, on the copy stream, so that they
        overlap this step's GEMMs.  Call after forward().  Returns bytes queued."""
        ids_h = np.asarray(next_ids)
        counts = np.bincount(ids_h.ravel(), minlength=self.E)
        hot = sorted((e for e in range(self.E) if counts[e] > 0), key=lambda e: (-int(counts[e]), e))
        current = getattr(self, "_current", set())
        todo = [e for e in hot if e not in self.slot_of]
        queued = 0
        # the copy stream already waited for every step before this one; the
        # current step's slots are never chosen
        with torch.cuda.stream(self.copy_stream):
            for e in todo:
                got = self._assign([e], keep=current | set(hot))
                if got is None:
                    break
                s = self.slot_of[e]
                self.last_use[s] = self.step  # the next step uses it
                self.gu.copy_in(e, s)
                self.dn.copy_in(e, s)
                ev = torch.cuda.Event()
                ev.record(self.copy_stream)
                self.pending[s] = ev
                queued += self.gu.expert_bytes + self.dn.expert_bytes
        return queued


# ------------------------------------------------------- nested MWQ planes
_PLANE = {2: (0, 512), 3: (512, 256), 4: (768, 256)}  # width -> (offset, bytes) in a 1 KB tile block


class _HostPlanes:
    """One tiled nested-MWQ weight set split per expert: pinned host copies of
    its tile blocks and scales, S device slots, planes copied one at a time."""

    def __init__(self, tiled: QuantizedExperts, n_slots: int, device):
        d = tiled.desc
        if d.format != MOE_W_MWQ_2_3_4 or d.layout != MOE_LAYOUT_TILED:
            raise ValueError("plane-wise offload takes tiled nested-MWQ weights")
        self.E, self.N, self.K, self.G, self.z = d.E, d.N, d.K, d.group_size, d.zero_point
        codes = tiled.tensors["codes"].view(torch.uint8).view(self.E, -1)
        scales = tiled.tensors["scales"].reshape(self.E, -1)
        self.row_bytes = codes.shape[1]          # one expert's tile blocks
        self.nblk = self.row_bytes // 1024
        self.host_codes = torch.empty(codes.shape, dtype=codes.dtype, pin_memory=True)
        self.host_scales = torch.empty(scales.shape, dtype=scales.dtype, pin_memory=True)
        self.host_codes.copy_(codes)
        self.host_scales.copy_(scales)
        self.slot_codes = torch.empty((n_slots, self.row_bytes), dtype=codes.dtype, device=device)
        self.slot_scales = torch.empty((n_slots, scales.shape[1]), dtype=scales.dtype, device=device)
        self.view = make_desc(MOE_W_MWQ_2_3_4, MOE_LAYOUT_TILED, n_slots, self.N, self.K, self.G, self.z,
                              codes=self.slot_codes, scales=self.slot_scales)
        self.scale_bytes = scales.shape[1] * scales.element_size()

    def plane_bytes(self, b: int) -> int:
        return self.nblk * _PLANE[b][1] + (self.scale_bytes if b == 2 else 0)

    def copy_plane(self, e: int, s: int, b: int, stream):
        """Plane b (2: q2 with the scales, 3: d3, 4: d4) of expert e into slot s, on `stream`."""
        off, width = _PLANE[b]
        moe_copy_rows_async(self.slot_codes, s * self.row_bytes + off, self.host_codes, e * self.row_bytes + off,
                            self.nblk, 1024, width, stream)
        if b == 2:
            with torch.cuda.stream(stream):
                self.slot_scales[s].copy_(self.host_scales[e], non_blocking=True)


class OffloadedMwqLayer(_SlotCache):
    """A routed-expert nested-MWQ layer (per-pair widths 2 / 3 / 4 bits) whose
    experts stay in host memory between uses, loaded plane by plane in HEBF
    order (D2MoE page, Design, bit-width-aware I/O-compute pipeline).

    Each step: the touched experts hottest first (most pairs, then lowest id);
    for each, the planes its widest pair needs that its slot lacks, q2 -> d3 ->
    d4, one copy after the other on the copy stream.  A pair of width b of
    expert e is computed in phase 0 if e's slot already holds the planes up to
    b, else in the phase that follows the copy of e's plane b.  Grouping key of
    a pair: 3 (phase S + slot) + 4 - b, so each phase is one contiguous slice of
    the grouped GEMM's segments (slot s, widths 4, 3, 2), run after the
    phase's copy has landed while the next copies proceed."""

    def __init__(self, gate_up: QuantizedExperts, down: QuantizedExperts, n_slots: int, device=None):
        device = device or torch.device("cuda", torch.cuda.current_device())
        self.gu = _HostPlanes(gate_up, n_slots, device)
        self.dn = _HostPlanes(down, n_slots, device)
        if self.gu.E != self.dn.E:
            raise ValueError("gate_up and down have different expert counts")
        self.E = self.gu.E
        self.I, self.H = self.gu.N // 2, self.dn.N
        self._init_slots(n_slots, device)
        self.planes_in = [0] * n_slots  # widest width whose planes the slot holds (0: none)

    def forward(self, x: torch.Tensor, logits: torch.Tensor, k: int, pair_bits: torch.Tensor,
                overlap: bool = True):
        """pair_bits: u8 [T][k] width of each pair (2, 3, 4).  Returns (out bf16 [T][H],
        OffloadStats).  overlap=False copies everything before computing anything."""
        T = x.shape[0]
        P = T * k
        S = self.S
        ids, w = moe_route_topk(logits, k)
        ids_h = ids.cpu().numpy().ravel()  # the host schedules the copies from the routing
        bits_h = pair_bits.cpu().numpy().astype(np.int64).ravel()
        if ((bits_h < 2) | (bits_h > 4)).any():
            raise ValueError("pair widths must be 2, 3 or 4")
        counts = np.bincount(ids_h, minlength=self.E)
        hot = sorted((e for e in range(self.E) if counts[e] > 0), key=lambda e: (-int(counts[e]), e))
        if len(hot) > S:
            raise ValueError(f"{len(hot)} experts touched, {S} slots")
        need = np.zeros(self.E, dtype=np.int64)
        np.maximum.at(need, ids_h, bits_h)
        self.step += 1
        misses = self._assign(hot)
        if misses is None:
            raise ValueError("no slot left")
        for e in misses:
            self.planes_in[self.slot_of[e]] = 0
        have = {e: self.planes_in[self.slot_of[e]] for e in hot}
        # HEBF: hottest expert first, its planes in bit order, only those its widest pair needs
        seq = [(e, b) for e in hot for b in (2, 3, 4) if have[e] < b <= need[e]]
        phase_of = {u: i + 1 for i, u in enumerate(seq)}
        stats = OffloadStats(len(hot), len(hot) - len(misses),
                             sum(self.gu.plane_bytes(b) + self.dn.plane_bytes(b) for _, b in seq))
        key = np.empty(P, dtype=np.int32)
        for i in range(P):
            e, b = int(ids_h[i]), int(bits_h[i])
            ph = 0 if have[e] >= b else phase_of[(e, b)]
            key[i] = 3 * (ph * S + self.slot_of[e]) + 4 - b
        n_phase = 1 + len(seq)
        keys = torch.from_numpy(key.reshape(T, k)).to(x.device)
        perm = moe_permute(keys, 3 * S * n_phase)
        compute = torch.cuda.current_stream()
        self.copy_stream.wait_stream(compute)  # the copies may overwrite planes earlier work still reads
        landed = []
        for e, b in seq:
            s = self.slot_of[e]
            self.gu.copy_plane(e, s, b, self.copy_stream)
            self.dn.copy_plane(e, s, b, self.copy_stream)
            ev = torch.cuda.Event()
            ev.record(self.copy_stream)
            landed.append(ev)
        if seq and not overlap:
            compute.wait_event(landed[-1])
        for e in hot:
            s = self.slot_of[e]
            self.planes_in[s] = max(self.planes_in[s], int(need[e]))
        rows = np.bincount(key // (3 * S), minlength=n_phase)
        h, y = self._intermediates(P, x.device)
        for ph in range(n_phase):
            if rows[ph] == 0:
                continue
            if ph > 0:
                compute.wait_event(landed[ph - 1])
            seg = perm.seg_offsets[3 * S * ph:3 * S * (ph + 1) + 1]
            moe_grouped_qgemm(self.gu.view, x, seg, P, MOE_EPI_SWIGLU, gather_pair=perm.sorted_pair, k=k, out=h)
            moe_grouped_qgemm(self.dn.view, h, seg, P, MOE_EPI_NONE_F16, out=y)
        out = moe_unpermute_combine(y, perm.pair_pos, w, T, k)
        return out, stats

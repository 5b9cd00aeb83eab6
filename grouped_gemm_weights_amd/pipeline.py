"""Multi-layer MoE pipeline with the copy-stream prefetch one layer ahead.

The schedule is the one of the DWDP explainer's prefetch-schedule panel:
while the compute stream runs layer l's MoE block and layer l+1's attention
block (here a dense bf16 GEMM stands in for attention), the copy stream fills
the alternate half of the merged buffer with layer l+1's experts: the merge
copies the local experts and the prefetch pulls the whole remote share (the
routing of layer l+1 is not known yet).  Per layer on the compute stream:

    A_l = bf16(x_l W_l^T)                          moe_dense_gemm
    wait(ready[l % 2])                             <- the layer's experts are in place
    route -> permute -> grouped SwiGLU -> combine  on half l % 2
    free[l % 2]                                    -> the half may be refilled
    x_{l+1} = bf16(x_l + y_l)                      moe_residual_add

and on the copy stream: wait(free[(l+1) % 2]) -> merge + prefetch of layer
l+1 into half (l+1) % 2 -> ready[(l+1) % 2].  Per-layer latency is then
max(compute, prefetch) (explainer, per-layer latency panel).

Every step runs in the library (C ABI); this module only orders the calls
and records events.
"""
from __future__ import annotations

from typing import Dict, List, Optional

import numpy as np
import torch

from . import binding as B
from . import synth
from .layer import MoELayer


class MoEPipeline:
    """stitched=True: layer l's merged range is one virtual range over [layer l's local-expert
    block | half (l % 2)'s own block] (moe_vmm_*), so the merge copies nothing and the copy
    stream moves only the remote share; the halves' own blocks alternate between layers."""

    def __init__(self, cfg: synth.MoEConfig, device="cuda", copy_mode: int = B.MOE_COPY_KERNEL,
                 stitched: bool = False, fused_gather: bool = False, sdma_experts: int = 0,
                 chunks: int = 1):
        """sdma_experts > 0 splits each layer's pull over two copy engines: the first
        ``sdma_experts`` remote experts go as no-CU copies (MOE_COPY_SDMA) on a second copy
        stream while the rest go through ``copy_mode`` on the first, in ``chunks`` runs of
        whole experts.  Every part has its own ready event, and the MoE block runs the grouped
        GEMM per expert range as each part lands (the local experts first)."""
        assert cfg.dtype == "bf16", "the pipeline runs the bf16 workloads"
        assert 0 <= sdma_experts <= cfg.E - cfg.n_local and chunks >= 1
        self.cfg = cfg
        self.sdma_experts = sdma_experts
        self.chunks = chunks
        self.dev = torch.device(device)
        self.stitched = stitched
        self.L = MoELayer(cfg, device=self.dev, copy_mode=copy_mode, allocate_halves=not stitched,
                          fused_gather=fused_gather)
        L = self.L
        self.n = cfg.layers
        self.locals: List[torch.Tensor] = []
        self.remotes: List[torch.Tensor] = []
        self.local_pools, self.remote_pools = [], []
        self.logits: List[torch.Tensor] = []
        self.w_attn: List[torch.Tensor] = []
        for l in range(self.n):
            loc = synth.pool_torch(cfg, l, 0, cfg.n_local, self.dev)
            rem = synth.pool_torch(cfg, l, cfg.n_local, cfg.E - cfg.n_local, self.dev)
            self.locals.append(loc)
            self.remotes.append(rem)
            self.local_pools.append(B.pool(loc, L.eb, 0, cfg.n_local))
            self.remote_pools.append(B.pool(rem, L.eb, cfg.n_local, cfg.E - cfg.n_local))
            self.logits.append(torch.from_numpy(synth.logits(cfg, l)).to(self.dev))
            self.w_attn.append(synth.dense_weight_torch(cfg, l, self.dev))
        x0 = synth.activations(cfg, 0)
        self.x0 = torch.from_numpy(x0.view(np.int16)).view(torch.bfloat16).to(self.dev)
        # the pull's parts: (expert range, stream) in the order the GEMM consumes them; the
        # local experts [0, n_local) are ready once the merge has written the slot map
        self.copy_stream2 = torch.cuda.Stream(device=self.dev) if sdma_experts else None
        lo = cfg.n_local
        parts = []
        if sdma_experts:
            parts.append((lo, lo + sdma_experts, "sdma"))
            lo += sdma_experts
        if lo < cfg.E:
            bounds = np.linspace(lo, cfg.E, min(chunks, cfg.E - lo) + 1).round().astype(int)
            parts += [(int(a), int(b), "main") for a, b in zip(bounds[:-1], bounds[1:])]
        self.parts = parts
        self.split = bool(sdma_experts) or chunks > 1
        # ready events per half: [merge] + one per part
        self.part_ready = [[B.moe_event_create(False) for _ in range(len(parts) + 1)]
                           for _ in range(2)]
        self.x = torch.empty_like(self.x0)
        self.a = torch.empty_like(self.x0)
        self.all_ids = list(range(cfg.E))
        torch.cuda.current_stream(self.dev).synchronize()
        # merged range and local pool of each layer
        self._ranges, self._phys = [], []
        if stitched:
            dev_index = self.dev.index if self.dev.index is not None else torch.cuda.current_device()
            lb, ob = cfg.n_local * L.eb, (cfg.E - cfg.n_local) * L.eb
            own = [B.moe_vmm_create(ob, dev_index) for _ in range(2)]
            self._phys += own
            self.wbufs, self.merge_pools = [], []
            for l in range(self.n):
                loc = B.moe_vmm_create(lb, dev_index)
                self._phys.append(loc)
                va = B.moe_vmm_map([loc, own[l % 2]], [lb, ob], dev_index)
                self._ranges.append((va, [lb, ob]))
                wb = B.wbuf(va, L.eb, cfg.E, cfg.E, L.slot_maps[l % 2])
                self.wbufs.append(wb)
                self.merge_pools.append(B.pool(va, L.eb, 0, cfg.n_local))
                # the local experts of layer l are placed once in its local block
                B.moe_prefetch_layer(self.local_pools[l], list(range(cfg.n_local)), wb,
                                     L.copy_stream, copy_mode=B.MOE_COPY_ANY)
            L.copy_stream.synchronize()
        else:
            self.wbufs = [L.wbufs[l % 2] for l in range(self.n)]
            self.merge_pools = self.local_pools

    # -------------------------------------------------------------- pieces
    def fill(self, l: int, wait_free: bool = True, ev: Optional[Dict[str, list]] = None) -> None:
        """Copy stream: wait until half l % 2 is free, then merge layer l's local experts and
        prefetch its remote share into it; ``ev`` c0/c1 bracket the copies themselves."""
        if self.split:
            return self._fill_split(l, wait_free, ev)
        L, h = self.L, l % 2
        if wait_free:
            B.moe_stream_wait_event(L.copy_stream, L.free[h])
        if ev is not None:
            B.moe_event_record(ev["c0"][l], L.copy_stream)
        B.moe_merge_weights(self.merge_pools[l], self.all_ids, self.wbufs[l], L.copy_stream,
                            wait_free=None, ready=None, copy_mode=L.copy_mode)
        B.moe_prefetch_layer(self.remote_pools[l], self.all_ids, self.wbufs[l], L.copy_stream,
                             wait_free=None, ready=L.ready[h], copy_mode=L.copy_mode)
        if ev is not None:
            B.moe_event_record(ev["c1"][l], L.copy_stream)

    def _fill_split(self, l: int, wait_free: bool, ev) -> None:
        """The split pull: the merge and the main parts on copy stream 1 (``copy_mode``), the
        SDMA part on copy stream 2 (no-CU copies), one ready event per part.  c1 is recorded
        on stream 1 after stream 2's part has landed, so c0..c1 spans the whole pull."""
        L, h, cfg = self.L, l % 2, self.cfg
        s1, s2 = L.copy_stream, self.copy_stream2
        ready = self.part_ready[h]
        if wait_free:
            B.moe_stream_wait_event(s1, L.free[h])
            if s2 is not None:
                B.moe_stream_wait_event(s2, L.free[h])
        if ev is not None:
            B.moe_event_record(ev["c0"][l], s1)
            if s2 is not None:
                B.moe_stream_wait_event(s2, ev["c0"][l])
        B.moe_merge_weights(self.merge_pools[l], self.all_ids, self.wbufs[l], s1,
                            wait_free=None, ready=ready[0], copy_mode=L.copy_mode)
        rbase = self.remotes[l].data_ptr()
        for i, (lo, hi, eng) in enumerate(self.parts):
            sub = B.pool(rbase + (lo - cfg.n_local) * L.eb, L.eb, lo, hi - lo)
            if eng == "sdma":
                B.moe_prefetch_layer(sub, self.all_ids, self.wbufs[l], s2, ready=ready[i + 1],
                                     copy_mode=B.MOE_COPY_SDMA)
            else:
                B.moe_prefetch_layer(sub, self.all_ids, self.wbufs[l], s1, ready=ready[i + 1],
                                     copy_mode=L.copy_mode)
        if s2 is not None:
            B.moe_stream_wait_event(s1, ready[1])
        B.moe_event_record(L.ready[h], s1)
        if ev is not None:
            B.moe_event_record(ev["c1"][l], s1)

    def dense(self, l: int) -> None:
        cfg = self.cfg
        B.moe_dense_gemm(self.x, self.w_attn[l], cfg.T, cfg.H, cfg.H, self.a, self.L.compute_stream)

    def moe(self, l: int, ev: Optional[Dict[str, list]] = None) -> None:
        """Route -> permute -> (wait for the half) -> grouped SwiGLU -> combine for layer l."""
        L, cfg, cs, h = self.L, self.cfg, self.L.compute_stream, l % 2
        L.logits, L.x = self.logits[l], self.a
        L.route_permute()
        if ev is not None:
            B.moe_event_record(ev["wait0"][l], cs)
        if self.split:
            # per-part readiness: the local experts, then each part as it lands
            ready = self.part_ready[h]
            B.moe_stream_wait_event(cs, ready[0])
            L.grouped(self.wbufs[l], 0, cfg.n_local)
            for i, (lo, hi, _) in enumerate(self.parts):
                B.moe_stream_wait_event(cs, ready[i + 1])
                if ev is not None and i == len(self.parts) - 1:
                    B.moe_event_record(ev["wait1"][l], cs)
                L.grouped(self.wbufs[l], lo, hi)
        else:
            B.moe_stream_wait_event(cs, L.ready[h])
            if ev is not None:
                B.moe_event_record(ev["wait1"][l], cs)
            L.grouped(self.wbufs[l])
        if ev is not None and "g1" in ev:
            B.moe_event_record(ev["g1"][l], cs)
        B.moe_combine(L.y_perm, L.row_of, L.topk_w, cfg.T, cfg.k, cfg.H, L.y, cs)
        B.moe_event_record(L.free[h], cs)

    def residual(self) -> None:
        cfg = self.cfg
        B.moe_residual_add(self.x, self.L.y, cfg.T * cfg.H, self.x, self.L.compute_stream)

    # -------------------------------------------------------------- runs
    def reset(self) -> None:
        with torch.cuda.stream(self.L.compute_stream):
            self.x.copy_(self.x0)

    def forward(self, ev: Optional[Dict[str, list]] = None, layer_hook=None) -> None:
        """The pipelined pass over all layers.  ``ev`` (optional) holds per-layer timing events:
        c0/c1 around each fill on the copy stream, wait0/wait1 around the wait for the half,
        d0 at the start of the dense block and m1 at the end of each MoE block."""
        L, cs, ps = self.L, self.L.compute_stream, self.L.copy_stream
        self.reset()
        self.fill(0, wait_free=True, ev=ev)
        for l in range(self.n):
            if ev is not None:
                B.moe_event_record(ev["d0"][l], cs)
            self.dense(l)
            if l + 1 < self.n:
                self.fill(l + 1, wait_free=True, ev=ev)
            self.moe(l, ev)
            if ev is not None:
                B.moe_event_record(ev["m1"][l], cs)
            if layer_hook is not None:
                layer_hook(l)
            self.residual()

    def capture(self) -> "torch.cuda.CUDAGraph":
        """The pipelined pass over all layers captured into one HIP graph on the compute
        stream: the copy stream is forked in by an event at the start and joined back by the
        last layer's ready event.  Inside one pass the first two fills find their halves
        unused, so only later fills wait for a half's free event (recorded by the pass
        itself); replays on one stream run one after another.  replay() recomputes x from x0.
        The split pull is not captured.  The graph holds the pipeline's buffers by address:
        replay it only before close()."""
        assert not self.split, "the split pull is not captured"
        L, cs, ps = self.L, self.L.compute_stream, self.L.copy_stream
        if getattr(self, "_fork", None) is None:
            self._fork = B.moe_event_create(False)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cs, capture_error_mode="relaxed"):
            self.reset()
            B.moe_event_record(self._fork, cs)
            B.moe_stream_wait_event(ps, self._fork)
            self.fill(0, wait_free=False)
            for l in range(self.n):
                self.dense(l)
                if l + 1 < self.n:
                    self.fill(l + 1, wait_free=l + 1 >= 2)
                self.moe(l)
                self.residual()
        return g

    def forward_serial(self, ev: Optional[Dict[str, list]] = None) -> None:
        """Each layer's copies finish before its compute starts (no overlap): the compute
        time alone, for the contention-slowdown figure."""
        L, cs, ps = self.L, self.L.compute_stream, self.L.copy_stream
        self.reset()
        for l in range(self.n):
            cs.synchronize()               # the previous layer's compute is done
            self.fill(l, wait_free=True, ev=ev)
            ps.synchronize()
            if ev is not None:
                B.moe_event_record(ev["d0"][l], cs)
            self.dense(l)
            self.moe(l)
            if ev is not None:
                B.moe_event_record(ev["m1"][l], cs)
            self.residual()
        cs.synchronize()

    def synchronize(self) -> None:
        self.L.synchronize()
        if self.copy_stream2 is not None:
            self.copy_stream2.synchronize()

    def close(self) -> None:
        """Release the stitched ranges and blocks (and the layer's events)."""
        self.synchronize()
        for lst in self.part_ready:
            for e in lst:
                B.moe_event_destroy(e)
        self.part_ready = []
        if getattr(self, "_fork", None) is not None:
            B.moe_event_destroy(self._fork)
            self._fork = None
        self.L.close()
        for va, sizes in self._ranges:
            B.moe_vmm_unmap(va, sizes)
        for ph in self._phys:
            B.moe_vmm_release(ph)
        self._ranges, self._phys = [], []

"""Host orchestration of the MoE layer forward on one GPU, through the C ABI.

``MoELayer`` owns the device buffers of one layer (PyTorch is used only to
allocate device memory and to provide streams) and issues the library calls
of one forward step:

    compute stream:  moe_route -> moe_permute -> (counts to host)
    copy stream:     moe_merge_weights (local experts + slot map)
                     -> moe_prefetch_layer (remote experts) -> ready event
    compute stream:  wait(ready) -> moe_grouped_swiglu -> moe_combine
                     -> free event (the half may be refilled)

This is the layer step of the DWDP explainer's prefetch-schedule panel with
the merged buffer of its contiguous-buffer panel; the peers' share of the
experts is a separate device pool (or pinned host memory) on this GPU.
Every step of the arithmetic runs in the library's HIP kernels.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np
import torch

from . import binding as B
from .synth import MoEConfig, expert_block_bytes


def _dtype_code(cfg: MoEConfig) -> int:
    return B.MOE_F32 if cfg.dtype == "f32" else B.MOE_BF16


def _torch_dtype(cfg: MoEConfig):
    return torch.float32 if cfg.dtype == "f32" else torch.bfloat16


class MoELayer:
    """Buffers and streams for one MoE layer of shape ``cfg`` on ``device``.

    ``n_halves`` merged-buffer halves of ``n_slots`` slots each are allocated
    (two for the double buffer).  The pools are set with ``set_pools`` (device
    tensors [n, 3*H*I], or pinned host tensors for the remote pool).
    """

    def __init__(self, cfg: MoEConfig, device="cuda", n_slots: Optional[int] = None,
                 n_halves: int = 2, compute_stream=None, copy_stream=None,
                 copy_mode: int = B.MOE_COPY_KERNEL, stitched: bool = False,
                 allocate_halves: bool = True, fused_gather: bool = False,
                 combine_in_epilogue: bool = False):
        """stitched: each half is one virtual range over [the local-expert block | the half's own
        block], so merging the local experts copies nothing (page stitching, moe_vmm_*).
        allocate_halves=False leaves the halves to the caller (the pipeline builds per-layer ranges).
        fused_gather: the grouped GEMM reads its rows from x through src_of, and x_perm is not built.
        combine_in_epilogue: the down GEMM adds its w-scaled rows straight into y
        (moe_grouped_swiglu_combine; implies fused_gather), and y_perm is not written."""
        self.cfg = cfg
        self.stitched = stitched
        self.combine_in_epilogue = combine_in_epilogue
        fused_gather = fused_gather or combine_in_epilogue
        self.fused_gather = fused_gather
        self.dev = torch.device(device)
        self.copy_mode = copy_mode
        T, E, k, H, I = cfg.T, cfg.E, cfg.k, cfg.H, cfg.I
        R = T * k
        self.R = R
        self.eb = expert_block_bytes(cfg)
        self.dt = _dtype_code(cfg)
        tdt = _torch_dtype(cfg)
        d = self.dev
        i32 = dict(dtype=torch.int32, device=d)
        self.logits = torch.empty((T, E), dtype=torch.float32, device=d)
        self.x = torch.empty((T, H), dtype=tdt, device=d)
        self.topk_idx = torch.empty((T, k), **i32)
        self.topk_w = torch.empty((T, k), dtype=torch.float32, device=d)
        self.counts = torch.empty((E,), **i32)
        self.offsets = torch.empty((E + 1,), **i32)
        self.row_of = torch.empty((R,), **i32)
        self.src_of = torch.empty((R,), **i32)
        # with the gather fused into the GEMM's loads, x_perm is never written
        self.x_perm = torch.empty((1 if fused_gather else R, H), dtype=tdt, device=d)
        self.y_perm = torch.empty((1 if combine_in_epilogue else R, H), dtype=torch.float32, device=d)
        self.y = torch.empty((T, H), dtype=torch.float32, device=d)
        self.status = torch.zeros((1,), **i32)
        self.ws_perm_bytes = B.moe_permute_workspace_size(T, E, k)
        self.ws_perm = torch.empty((max(1, self.ws_perm_bytes),), dtype=torch.uint8, device=d)
        self.ws_gemm_bytes = B.moe_grouped_swiglu_workspace_size(R, E, H, I, self.dt)
        self.ws_gemm = torch.empty((self.ws_gemm_bytes,), dtype=torch.uint8, device=d)
        self.counts_host = torch.empty((E,), dtype=torch.int32, pin_memory=True)
        self.n_slots = E if n_slots is None else n_slots
        self.halves = []
        self.wbufs = []
        self.slot_maps = [torch.full((E,), -1, **i32) for _ in range(n_halves)]
        self._vmm_ranges, self._vmm_phys = [], []
        self.stitched_local_pools = []
        if allocate_halves and stitched:
            dev_index = d.index if d.index is not None else torch.cuda.current_device()
            local_bytes = cfg.n_local * self.eb
            own_bytes = (self.n_slots - cfg.n_local) * self.eb
            if local_bytes == 0 and own_bytes == 0:
                raise ValueError("stitched halves need at least one slot")
            self._local_phys = B.moe_vmm_create(local_bytes, dev_index) if local_bytes else None
            if self._local_phys is not None:
                self._vmm_phys.append(self._local_phys)
            for h in range(n_halves):
                own = B.moe_vmm_create(own_bytes, dev_index) if own_bytes else None
                if own is not None:
                    self._vmm_phys.append(own)
                # a block of zero bytes (no local experts, or no slots beyond them) is left out
                pieces = [(ph, nb) for ph, nb in ((self._local_phys, local_bytes), (own, own_bytes)) if nb]
                va = B.moe_vmm_map([ph for ph, _ in pieces], [nb for _, nb in pieces], dev_index)
                self._vmm_ranges.append((va, [nb for _, nb in pieces]))
                self.halves.append((va, self.slot_maps[h]))
                self.wbufs.append(B.wbuf(va, self.eb, self.n_slots, E, self.slot_maps[h]))
                self.stitched_local_pools.append(B.pool(va, self.eb, 0, cfg.n_local))
        elif allocate_halves:
            for h in range(n_halves):
                base = torch.empty((self.n_slots, self.eb), dtype=torch.uint8, device=d)
                self.halves.append((base, self.slot_maps[h]))
                self.wbufs.append(B.wbuf(base, self.eb, self.n_slots, E, self.slot_maps[h]))
        self.compute_stream = compute_stream or torch.cuda.Stream(device=d)
        self.copy_stream = copy_stream or torch.cuda.Stream(device=d)
        self.ready = [B.moe_event_create(False) for _ in range(n_halves)]
        self.free = [B.moe_event_create(False) for _ in range(n_halves)]
        self.counts_ready = B.moe_event_create(False)
        self.local_pool = None
        self.remote_pool = None
        self.last_ids = None
        torch.cuda.current_stream(d).synchronize()   # buffers initialised on torch's stream

    # ------------------------------------------------------------------ setup
    def set_pools(self, local: torch.Tensor, remote: torch.Tensor) -> None:
        """local: experts [0, n_local); remote: experts [n_local, E); each [n, 3*H*I]."""
        cfg = self.cfg
        assert local.shape[0] == cfg.n_local and remote.shape[0] == cfg.E - cfg.n_local
        assert local.is_contiguous() and remote.is_contiguous()
        self._local_t, self._remote_t = local, remote
        self.local_pool = B.pool(local, self.eb, 0, cfg.n_local)
        self.remote_pool = B.pool(remote, self.eb, cfg.n_local, cfg.E - cfg.n_local)
        torch.cuda.current_stream(self.dev).synchronize()
        if self.stitched_local_pools:
            # place the local experts once in the block every half maps at its head
            B.moe_prefetch_layer(self.local_pool, list(range(cfg.n_local)), self.wbufs[0],
                                 self.copy_stream, copy_mode=B.MOE_COPY_ANY)
            self.copy_stream.synchronize()

    def set_inputs(self, x, logits) -> None:
        """x: numpy [T,H] (float32, or uint16 bf16 bits) or torch; logits numpy f32 [T,E] or torch."""
        if isinstance(x, np.ndarray):
            if x.dtype == np.uint16:
                x = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
            else:
                x = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
        if isinstance(logits, np.ndarray):
            logits = torch.from_numpy(np.ascontiguousarray(logits, dtype=np.float32))
        self.x.copy_(x)
        self.logits.copy_(logits)
        torch.cuda.current_stream(self.dev).synchronize()   # inputs ready before the layer's streams run

    def expert_block(self, e: int) -> torch.Tensor:
        """The pool block of expert e (device or host tensor view)."""
        n_local = self.cfg.n_local
        return self._local_t[e] if e < n_local else self._remote_t[e - n_local]

    # ------------------------------------------------------------------ steps
    def route_permute(self) -> None:
        cfg, cs = self.cfg, self.compute_stream
        B.moe_route(self.logits, cfg.T, cfg.E, cfg.k, self.topk_idx, self.topk_w, self.status, cs)
        B.moe_permute(self.topk_idx, cfg.T, cfg.E, cfg.k, self.x, cfg.H, self.dt, self.counts,
                      self.offsets, self.row_of, self.src_of,
                      None if self.fused_gather else self.x_perm, self.ws_perm,
                      self.ws_perm_bytes, self.status, cs)

    def grouped(self, wbuf, e_begin: int = 0, e_end: Optional[int] = None, stream=None) -> None:
        """The grouped SwiGLU GEMM over experts [e_begin, e_end) of ``wbuf`` into y_perm."""
        cfg = self.cfg
        e_end = cfg.E if e_end is None else e_end
        cs = self.compute_stream if stream is None else stream
        if self.fused_gather:
            B.moe_grouped_swiglu_gathered(self.x, self.src_of, cfg.k, self.offsets, self.R, cfg.E,
                                          cfg.H, cfg.I, self.dt, wbuf, e_begin, e_end, self.ws_gemm,
                                          self.ws_gemm_bytes, self.y_perm, self.status, cs)
        else:
            B.moe_grouped_swiglu_range(self.x_perm, self.offsets, self.R, cfg.E, cfg.H, cfg.I,
                                       self.dt, wbuf, e_begin, e_end, self.ws_gemm,
                                       self.ws_gemm_bytes, self.y_perm, self.status, cs)

    def grouped_combine(self, wbuf, stream=None) -> None:
        """Grouped SwiGLU GEMM with the gather on load and the combine in the down GEMM's
        epilogue: writes y directly (every expert of ``wbuf``)."""
        cfg = self.cfg
        cs = self.compute_stream if stream is None else stream
        B.moe_grouped_swiglu_combine(self.x, self.src_of, self.topk_w, cfg.T, cfg.k, self.offsets,
                                     cfg.E, cfg.H, cfg.I, self.dt, wbuf, self.ws_gemm,
                                     self.ws_gemm_bytes, self.y, self.status, cs)

    def expert_output(self, wbuf) -> None:
        """y from the merged buffer: the grouped GEMM then the combine, or both in one call."""
        cfg = self.cfg
        if self.combine_in_epilogue:
            self.grouped_combine(wbuf)
        else:
            self.grouped(wbuf)
            B.moe_combine(self.y_perm, self.row_of, self.topk_w, cfg.T, cfg.k, cfg.H, self.y,
                          self.compute_stream)

    def routed_ids(self) -> Sequence[int]:
        """Read counts back (one small copy and a sync) and return the expert set of the buffer:
        every local expert plus the remote experts that received tokens, ascending."""
        cfg, cs = self.cfg, self.compute_stream
        with torch.cuda.stream(cs):
            self.counts_host.copy_(self.counts, non_blocking=True)
        cs.synchronize()
        c = self.counts_host.numpy()
        remote = np.nonzero(c[cfg.n_local:])[0] + cfg.n_local
        return list(range(cfg.n_local)) + [int(e) for e in remote]

    def fill_half(self, half: int, ids: Sequence[int], wait_free: bool = True) -> None:
        """Copy stream: merge the local experts (and the slot map) and prefetch the remote ones.
        With stitched halves the local experts already sit at their slots: only the map is written."""
        ws = self.free[half] if wait_free else None
        local = self.local_pool
        if self.stitched_local_pools:
            assert list(ids[: self.cfg.n_local]) == list(range(self.cfg.n_local)), \
                "a stitched half needs every local expert at the head of the expert set"
            local = self.stitched_local_pools[half]
        B.moe_merge_weights(local, ids, self.wbufs[half], self.copy_stream,
                            wait_free=ws, ready=None, copy_mode=self.copy_mode)
        B.moe_prefetch_layer(self.remote_pool, ids, self.wbufs[half], self.copy_stream,
                             wait_free=None, ready=self.ready[half], copy_mode=self.copy_mode)
        self.last_ids = list(ids)

    def fill_half_routed_on_device(self, half: int, wait_free: bool = True) -> None:
        """Copy stream: the local experts (merge of ids 0 .. n_local - 1) and the routed remote
        experts decided on the device from this step's counts (slot = expert id), with no count
        read-back.  Call after route_permute."""
        cfg = self.cfg
        local = self.stitched_local_pools[half] if self.stitched_local_pools else self.local_pool
        # the copy stream's first operation is the wait for the permute, so a capture of the step
        # on the compute stream takes the copy stream's work in too
        B.moe_event_record(self.counts_ready, self.compute_stream)
        B.moe_stream_wait_event(self.copy_stream, self.counts_ready)
        B.moe_merge_weights(local, range(cfg.n_local), self.wbufs[half], self.copy_stream,
                            wait_free=self.free[half] if wait_free else None, ready=None,
                            copy_mode=self.copy_mode)
        kernel = (self.copy_mode & 0xFF) == B.MOE_COPY_KERNEL
        B.moe_prefetch_routed(self.remote_pool, self.counts, self.wbufs[half], self.copy_stream,
                              ready=self.ready[half],
                              max_blocks=(self.copy_mode >> 8) if kernel else 0)
        self.last_ids = None                  # the expert set never reaches the host

    def capture_step(self, half: int = 0) -> "torch.cuda.CUDAGraph":
        """One device-routed layer step (route, permute, merge, routed pull, grouped GEMM,
        combine) captured into a HIP graph on this layer's compute stream, the copy stream's
        work forked into it by the permute's event and joined by the half's ready event.
        replay() reruns the step on whatever x and logits hold (set_inputs writes them in
        place).  The half's free event is not waited for inside the graph: replays on one
        stream run one after another, and the caller must not fill this half from elsewhere
        while a replay runs.  The graph holds this layer's buffers and pools by address: replay
        it only while the layer is open and its pools are alive."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=self.compute_stream, capture_error_mode="relaxed"):
            self.route_permute()
            self.fill_half_routed_on_device(half, wait_free=False)
            self.expert_compute(half)
        return g

    def expert_compute(self, half: int) -> None:
        """Compute stream: wait for the half, grouped SwiGLU GEMM, combine, release the half."""
        cs = self.compute_stream
        B.moe_stream_wait_event(cs, self.ready[half])
        self.expert_output(self.wbufs[half])
        B.moe_event_record(self.free[half], cs)

    def forward(self, half: int = 0, remote: str = "routed", chunks: int = 0, ev=None) -> None:
        """One whole layer step; remote = 'routed' (fetch only the remote experts that got
        tokens, after a count read-back), 'device' (the same set, picked on the device: no
        read-back, nothing waits on the host) or 'all' (fetch the whole remote share).
        chunks > 0 (not with 'device') splits the remote fetch into that many chunks with one
        ready event each, and the grouped GEMM runs per chunk as its weights land (the local
        experts first, while the copies run)."""
        self.route_permute()
        if remote == "device":
            if chunks > 0:
                raise ValueError("the device-routed pull is not chunked")
            self.fill_half_routed_on_device(half)
            self.expert_compute(half)
            return
        ids = self.routed_ids() if remote == "routed" else list(range(self.cfg.E))
        if chunks <= 0 or self.combine_in_epilogue:
            self.fill_half(half, ids)
            self.expert_compute(half)
        else:
            self.forward_chunked(half, ids, chunks, ev)

    def _chunk_events(self, half: int, n: int):
        if not hasattr(self, "_cev"):
            self._cev = {}
        lst = self._cev.setdefault(half, [])
        while len(lst) < n:
            lst.append(B.moe_event_create(False))
        return lst[:n]

    def forward_chunked(self, half: int, ids: Sequence[int], chunks: int, ev=None) -> None:
        """Merge + chunked prefetch on the copy stream, per-chunk grouped GEMM on the compute
        stream.  ``ev`` (optional): dict of timing-event lists 'g0'/'g1' (one pair per GEMM call)."""
        cfg, cs, ps = self.cfg, self.compute_stream, self.copy_stream
        remote_ids = [e for e in ids if e >= cfg.n_local]
        n_ch = max(1, min(chunks, len(remote_ids))) if remote_ids else 0
        groups = [list(g) for g in np.array_split(np.asarray(remote_ids, dtype=np.int64), n_ch)] if n_ch else []
        bounds = [g[0] for g in groups] + [cfg.E]
        ready = self._chunk_events(half, n_ch + 1)
        local = self.local_pool
        if self.stitched_local_pools:
            assert list(ids[: cfg.n_local]) == list(range(cfg.n_local))
            local = self.stitched_local_pools[half]
        wb = self.wbufs[half]
        B.moe_merge_weights(local, ids, wb, ps, wait_free=self.free[half], ready=ready[0],
                            copy_mode=self.copy_mode)
        rbase = self._remote_t.data_ptr()
        for c in range(n_ch):
            lo, hi = int(bounds[c]), int(bounds[c + 1])
            sub = B.pool(rbase + (lo - cfg.n_local) * self.eb, self.eb, lo, hi - lo)
            B.moe_prefetch_layer(sub, ids, wb, ps, ready=ready[c + 1], copy_mode=self.copy_mode)
        ranges = [(0, int(bounds[0]))] + [(int(bounds[c]), int(bounds[c + 1])) for c in range(n_ch)]
        for c, (lo, hi) in enumerate(ranges):
            B.moe_stream_wait_event(cs, ready[c])
            if ev is not None:
                B.moe_event_record(ev["g0"][c], cs)
            self.grouped(wb, lo, hi)
            if ev is not None:
                B.moe_event_record(ev["g1"][c], cs)
        B.moe_combine(self.y_perm, self.row_of, self.topk_w, cfg.T, cfg.k, cfg.H, self.y, cs)
        B.moe_event_record(self.free[half], cs)
        self.last_ids = list(ids)

    def synchronize(self) -> None:
        self.compute_stream.synchronize()
        self.copy_stream.synchronize()

    def read_status(self) -> int:
        self.synchronize()
        return int(self.status.item())

    def outputs(self) -> Dict[str, np.ndarray]:
        """Host copies of every output of the step (synchronises)."""
        self.synchronize()
        to = lambda t: t.detach().cpu()
        x_perm = to(self.x_perm)
        if x_perm.dtype == torch.bfloat16:
            x_perm = x_perm.view(torch.int16).numpy().view(np.uint16)
        else:
            x_perm = x_perm.numpy()
        return dict(idx=to(self.topk_idx).numpy(), w=to(self.topk_w).numpy(),
                    counts=to(self.counts).numpy(), offsets=to(self.offsets).numpy(),
                    row_of=to(self.row_of).numpy(), src_of=to(self.src_of).numpy(),
                    x_perm=x_perm, y_perm=to(self.y_perm).numpy(), y=to(self.y).numpy(),
                    status=int(self.status.item()))

    def close(self) -> None:
        self.synchronize()
        evs = self.ready + self.free + [e for l in getattr(self, "_cev", {}).values() for e in l]
        if self.counts_ready is not None:
            evs.append(self.counts_ready)
        for ev in evs:
            B.moe_event_destroy(ev)
        self.ready, self.free, self._cev, self.counts_ready = [], [], {}, None
        for va, sizes in self._vmm_ranges:
            B.moe_vmm_unmap(va, sizes)
        for ph in self._vmm_phys:
            B.moe_vmm_release(ph)
        self._vmm_ranges, self._vmm_phys = [], []


def block_to_numpy(block: torch.Tensor) -> np.ndarray:
    """An expert block (torch, any device) as a host numpy array: float32, or uint16 bf16 bits."""
    b = block.detach().cpu()
    if b.dtype == torch.bfloat16:
        return b.view(torch.int16).numpy().view(np.uint16)
    return b.numpy()

"""Two-stream decode pipeline over a pinned-host KV store: orchestration only.

Per layer the full K|V store stays in pinned host memory and a resident set
of top_k slots per KV head lives in HBM.  One layer-step is

  main stream:  wait for this layer's previous copy, then the fused step
                (attention of both query rows over the resident slots, and
                scan, top-K and plan for the next step);
  copy stream:  wait for that attention, then copy the planned blocks from
                host to their resident slots (oasis_copy_blocks reads the
                mapped pinned memory from the GPU).

The copy overwrites slots the attention has just read, so it is ordered after
it; the next step's attention of the same layer reads what the copy wrote, so
it is ordered after the copy.  Other layers run meanwhile.  This is the
pipelined transfer of the OasisKV paper (Section 4, the pinned-host path with a
background copy stream and events that keep each layer's order); the steps
themselves are the library's kernels, called through ``ops``.

With a decode-host cache (Section 3.2: remote memory holds the full prompt KV,
decode-host memory a bounded cache of whole blocks), each layer's cache has a
dispatcher thread (oasis_host_tier_submit): once the step's attention is done
it copies the plan back, fetches the absent whole blocks on the host, then
launches the gather through the cache's union map on the copy stream and
records the layer's copy event.  These are the remote-fetch and local-fetch
stages of Section 3.3's per-layer pipeline; the dispatchers of different
layers work side by side while the GPU runs other layers.  Before the main
stream waits on a layer's copy event, the host waits until that layer's
dispatcher has recorded it.  A layer's next fetch (which may evict cache
slots) follows its next step, which waits for this gather, so a gather never
reads a slot being replaced.
"""
from __future__ import annotations

import torch

from . import ops


class PipelineLayer:
    """State of one layer: host store views, resident store, slot tables
    (double-buffered: step t reads buffer t % 2 and plans into the other),
    per-layer plan buffers and the prepared calls."""

    def __init__(self, wl, host_store: torch.Tensor | None, summaries: torch.Tensor,
                 q0: torch.Tensor, device, opts=None, want_scores=False,
                 remote_store: torch.Tensor | None = None, host_capacity: int | None = None,
                 host_workers: int = 1):
        """host_store: pinned [R][H][n_blk][2][B][D], the full store the copies
        read.  Or, with a decode-host cache: remote_store pinned
        [R][n_blk][H][2][B][D] (whole blocks, standing in for remote memory;
        filled from the host), host_capacity blocks per request cached in
        decode-host memory, and host_workers threads per fetch (besides the
        layer's dispatcher thread)."""
        R, H, K, B, D = wl.R, wl.H, wl.K, wl.B, wl.D
        self.wl = wl
        self.tier = None
        if remote_store is not None:
            if not remote_store.is_pinned() or remote_store.shape[:1] != (R,) or \
                    remote_store.shape[2:] != (H, 2, B, D):
                raise ValueError("remote_store must be pinned [R][n_blk][H][2][B][D]")
            n_blk = remote_store.shape[1]
            cap = int(host_capacity)
            self.remote = remote_store
            self.cache = torch.empty((R, cap, H, 2, B, D), dtype=wl.dtype, pin_memory=True)
            self.map = torch.empty((R, n_blk), dtype=torch.int32, pin_memory=True)
            block_bytes = H * 2 * B * D * remote_store.element_size()
            self.tier = ops.HostTier(R, H, K, n_blk, [cap] * R, remote_store, self.cache,
                                     self.map, block_bytes, workers=host_workers)
        else:
            if host_store is None or not host_store.is_pinned():
                raise ValueError("the host store must be pinned")
            self.host = host_store
            self.host_k, self.host_v = ops.interleaved_kv(host_store)
        self.res = torch.empty((R, H, K, 2, B, D), dtype=wl.dtype, device=device)
        self.res_k, self.res_v = ops.interleaved_kv(self.res)
        self.summ = summaries
        self.blk = [torch.full((R, H, K), -1, dtype=torch.int32, device=device) for _ in range(2)]
        self.stamp = [torch.full((R, H, K), -1, dtype=torch.int32, device=device)
                      for _ in range(2)]
        self.ident = torch.arange(K, dtype=torch.int32, device=device).repeat(R, H, 1).contiguous()
        self.bufs = {}
        self.step_calls = [ops.prepare_lookahead_step(
            q0, summaries, K, self.blk[p], self.stamp[p], self.blk[1 - p], self.stamp[1 - p], 0,
            wl.cap, self.res_k, self.res_v, self.ident, K, B, pred_row=1, want_scores=want_scores,
            want_evicted=False, opts=opts, bufs=self.bufs) for p in range(2)]
        self.plan = {k: self.bufs[k] for k in ("plan_count", "plan_src", "plan_dst")}
        if self.tier is None:
            self.copy_call = ops.prepare_copy_blocks(self.host_k, self.host_v, self.res_k,
                                                     self.res_v, self.plan, B)
        else:
            self.submit = self.tier.prepare_submit(self.cache, self.res_k, self.res_v, self.plan, B)
        self.attn_done = torch.cuda.Event()
        self.copy_done = torch.cuda.Event()
        self.attn_done.record()  # created now: the dispatcher takes raw handles
        self.copy_done.record()

    def ready(self) -> None:
        """Host wait until this layer's last copy event has been recorded (a
        dispatcher records it; without a cache it already is)."""
        if self.tier is not None:
            self.tier.wait_issued()

    def seed(self, q0: torch.Tensor, copy_stream) -> None:
        """First working set from row 0 of the first queries (empty slots, no
        cap), copied on ``copy_stream``; the next step's attention waits for it."""
        wl = self.wl
        idx, _, _ = ops.score_topk(q0, self.summ, wl.K)
        ops.select_plan(idx, self.blk[0], self.stamp[0], 0, wl.cap, pred_row=0,
                        plan=dict(self.plan, plan_evicted=None))
        self.attn_done.record()
        self.copy(copy_stream, self.blk[0])

    def copy(self, stream, slot_block: torch.Tensor, events=None) -> None:
        """The planned blocks into their slots on `stream` after this layer's
        attn_done, then copy_done.  Through the decode-host cache when there is
        one (fetch and gather by the dispatcher).  `events`: timing events
        around the copy; with a cache they span submit to gather end, and the
        host waits for the dispatcher in between (for timing runs only)."""
        if self.tier is not None:
            if events:
                events[0].record(stream)
            self.submit(slot_block, self.attn_done, stream, self.copy_done)
            if events:
                self.tier.wait_issued()
                events[1].record(stream)
            return
        stream.wait_event(self.attn_done)
        if events:
            events[0].record(stream)
        self.copy_call(stream)
        if events:
            events[1].record(stream)
        self.copy_done.record(stream)


class Pipeline:
    """Layers sharing one main stream (the caller's current stream) and one
    background copy stream."""

    def __init__(self, layers: list[PipelineLayer], copy_stream=None):
        self.layers = layers
        self.copy_stream = copy_stream or torch.cuda.Stream()

    def seed(self, q0s) -> None:
        for layer, q0 in zip(self.layers, q0s):
            layer.seed(q0, self.copy_stream)

    def layer_step(self, t: int, l: int, q: torch.Tensor, step_events=None,
                   copy_events=None) -> dict:
        """Step t of layer l with stacked queries q; returns the fused call's
        result dict (its buffers are reused by this layer's next step).
        Optional timing events: around the fused step (main stream) and around
        the direct copy (copy stream)."""
        L = self.layers[l]
        main = torch.cuda.current_stream()
        L.ready()
        main.wait_event(L.copy_done)
        if step_events:
            step_events[0].record(main)
        res = L.step_calls[t % 2](t + 1, q)
        if step_events:
            step_events[1].record(main)
        L.attn_done.record(main)
        L.copy(self.copy_stream, L.blk[1 - t % 2], copy_events)
        return res

    def drain(self) -> None:
        """Host wait until every submitted copy has been issued; after this,
        waiting on the copy stream covers all of them."""
        for L in self.layers:
            L.ready()

    def resident_blocks(self, l: int, t: int) -> torch.Tensor:
        """Slot table that describes layer l's resident store during step t."""
        return self.layers[l].blk[t % 2]

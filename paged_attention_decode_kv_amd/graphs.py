"""Captured decode steps over padded row buckets.

A serving loop presents a different number of rows at each step, and a recorded graph
replays one shape at fixed addresses.  Following the capture list of the nanoserve
daily log (Day 55, "What I added today" and "Why it matters"), every bucket of a list of
row counts gets one graph, recorded while every row is padding: length 0, new K/V aimed
at the sink slot.  Such a recording is legal for any later step because it keeps only
addresses, and each step writes its own numbers through them.  A step of n rows runs on
the smallest bucket of at least n rows: its inputs fill the first n rows of the shared
buffers, rows n.. of the bucket become padding again, and the bucket's graph replays.

The pages' shape set is a product of row buckets and width buckets.  Here the block
table has one fixed width and the chunk length of the split is chosen on the device, so
a single list over row counts covers every step.  The graphs are recorded largest
first, as the pages order them; they share one set of buffers and one workspace, so
replays must stay on one stream.

Host bookkeeping only: the recording and every launch go through the library
(pkv_graph_capture, pkv_graph_launch), and the padding fill and input copies are plain
device copies.
"""

from __future__ import annotations

import torch

from . import binding


def default_buckets(max_rows: int) -> list[int]:
    """Powers of two below ``max_rows``, then ``max_rows`` itself."""
    if max_rows < 1:
        raise ValueError("max_rows must be positive")
    out, b = [], 1
    while b < max_rows:
        out.append(b)
        b *= 2
    out.append(max_rows)
    return out


def bucket_for(buckets, n: int) -> int:
    """The smallest bucket holding ``n`` rows."""
    if n < 1:
        raise binding.PagedKVError("EMPTY", "no rows")
    fits = [b for b in buckets if b >= n]
    if not fits:
        raise binding.PagedKVError("SHAPE", f"{n} rows exceed the largest bucket "
                                            f"{max(buckets)}")
    return min(fits)


class DecodeGraphs:
    """One recorded decode step per row bucket, over shared fixed-address buffers."""

    def __init__(self, k_cache: torch.Tensor, v_cache: torch.Tensor, *, num_heads: int,
                 max_blocks: int, scale: float, buckets=None, max_rows: int | None = None,
                 layout: str = "HND"):
        if buckets is None:
            if max_rows is None:
                raise ValueError("give buckets or max_rows")
            buckets = default_buckets(max_rows)
        self.buckets = sorted({int(b) for b in buckets})
        if not self.buckets or self.buckets[0] < 1:
            raise ValueError("buckets must be positive row counts")
        desc = binding.pool_desc(k_cache, layout)
        self.layout = layout
        self.k_cache, self.v_cache = k_cache, v_cache
        self.num_heads, self.max_blocks, self.scale = num_heads, max_blocks, float(scale)
        self.sink = binding.sink_slot(k_cache, layout)
        n, dev, dt = self.buckets[-1], k_cache.device, k_cache.dtype
        hkv, d = desc.num_kv_heads, desc.head_dim
        self.q = torch.zeros((n, num_heads, d), dtype=dt, device=dev)
        self.out = torch.zeros_like(self.q)
        self.k_new = torch.zeros((n, hkv, d), dtype=dt, device=dev)
        self.v_new = torch.zeros_like(self.k_new)
        self.slot_mapping = torch.full((n,), self.sink, dtype=torch.int64, device=dev)
        self.block_tables = torch.full((n, max_blocks), -1, dtype=torch.int32, device=dev)
        self.context_lens = torch.zeros((n,), dtype=torch.int32, device=dev)
        ws = binding.workspace_bytes(k_cache, n, num_heads, max_blocks, layout)
        self.workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=dev)
        self.graphs: dict[int, binding.StepGraph] = {}
        for b in reversed(self.buckets):          # largest first
            self.graphs[b] = binding.capture_step(
                self.k_new[:b], self.v_new[:b], self.slot_mapping[:b], self.q[:b],
                k_cache, v_cache, self.block_tables[:b], self.context_lens[:b],
                self.scale, self.out[:b], self.workspace, layout=layout)
        # the warm run: every bucket once over the all-padding batch
        for b in self.buckets:
            self.graphs[b].launch()

    def bucket_for(self, n: int) -> int:
        return bucket_for(self.buckets, n)

    def launch(self, n: int) -> torch.Tensor:
        """Replay the step for ``n`` rows already written into the first ``n`` rows of
        the buffers; returns ``out[:n]`` (valid once the current stream reaches it)."""
        b = self.bucket_for(n)
        if b > n:
            self.context_lens[n:b].zero_()
            self.slot_mapping[n:b].fill_(self.sink)
        self.graphs[b].launch()
        return self.out[:n]

    def step(self, q, k_new, v_new, slot_mapping, block_tables, context_lens) -> torch.Tensor:
        """Copy one step's inputs into the buffers and replay; returns ``out[:n]``.
        Inputs are not checked on the host: bad entries are clamped or skipped on the
        device and reported by the device status word."""
        n = int(context_lens.shape[0])
        self.bucket_for(n)
        width = int(block_tables.shape[1])
        if width > self.max_blocks:
            raise binding.PagedKVError("SHAPE", f"block table width {width} > "
                                                f"{self.max_blocks}")
        for t, buf, name in ((q, self.q, "q"), (k_new, self.k_new, "k_new"),
                             (v_new, self.v_new, "v_new"),
                             (slot_mapping, self.slot_mapping, "slot_mapping"),
                             (context_lens, self.context_lens, "context_lens")):
            if t.dtype != buf.dtype or tuple(t.shape) != (n,) + tuple(buf.shape[1:]):
                raise binding.PagedKVError(
                    "SHAPE", f"{name} must be {buf.dtype} {(n,) + tuple(buf.shape[1:])}, "
                             f"got {t.dtype} {tuple(t.shape)}")
        if block_tables.dtype != torch.int32 or block_tables.shape[0] != n:
            raise binding.PagedKVError("SHAPE", f"block_tables must be int32 [{n}, width]")
        self.q[:n].copy_(q)
        self.k_new[:n].copy_(k_new)
        self.v_new[:n].copy_(v_new)
        self.slot_mapping[:n].copy_(slot_mapping)
        self.block_tables[:n, :width].copy_(block_tables)
        if width < self.max_blocks:
            self.block_tables[:n, width:].fill_(-1)
        self.context_lens[:n].copy_(context_lens)
        return self.launch(n)

    def close(self) -> None:
        for g in self.graphs.values():
            g.destroy()
        self.graphs.clear()

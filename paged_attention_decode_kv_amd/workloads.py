"""Seeded synthetic inputs for the batched paged-attention decode step.

This module only *constructs inputs*: lengths, block placement, the step's write
slots, and N(0, 1) values for queries, new keys/values and the pool history.  It
holds none of the step's arithmetic (no scores, no softmax, no weighted sums) and
it is the one module that the HIP binding's tests and the CPU oracle's tests both
draw from.  It imports neither of them.

Workloads follow the nanoserve pages' synthetic decode batches (Day 59, "What I
added today": the streambench shapes of 8-256 rows, 32 heads, widths 2048-8192,
uniform, ragged and long-tail length spreads, scattered block placement).  The
five named configurations are:

1. ``tiny-f32``    2 rows, 4 heads, head_dim 64, fp32, pool of 8 blocks, lengths [16, 40]
2. ``uniform``     8 rows, 32 heads, head_dim 128, bf16, every length 2048, pool sized exactly
3. ``ragged``      32 rows + 2 pad rows, lengths uniform in [2048, 8192], pool 20% oversized
4. ``long-tail``   256 rows, width 2048, lengths lognormal(median 256, sigma 1.0), one row at 2048
5. ``full-width``  256 rows (16 pad), width 8192, lengths lognormal(median 1024, sigma 1.2),
                   8 rows at 8192; a 131072-block (~34 GB K+V) pool

All configurations use block_size 16 and one new token per row (its write slot is
the row's last live position; pad rows write the sink slot).

Draw order from ``numpy.random.default_rng(seed)``: lengths, pad positions, block
permutation, q, new k, new v.  The pool history comes from a second stream
(``seed + HISTORY_SEED_OFFSET``) on the host, or from a seeded ``torch.Generator`` on
the device for pools too large to build on the host.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

HISTORY_SEED_OFFSET = 7919
BF16_NAN = np.uint16(0x7FC0)
CONFIG_NAMES = {1: "tiny-f32", 2: "uniform", 3: "ragged", 4: "long-tail", 5: "full-width"}
# pools up to this many bytes (K + V together) are generated on the host
HOST_POOL_LIMIT = 1 << 30


def cdiv(a: int, b: int) -> int:
    return -(-int(a) // int(b))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (finite inputs)."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bias = ((b >> np.uint64(16)) & np.uint64(1)) + np.uint64(0x7FFF)
    return ((b + bias) >> np.uint64(16)).astype(np.uint16)


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32)
    if dtype == "bf16":
        return bf16_bits(x)
    raise ValueError(dtype)


def storage_nbytes(dtype: str) -> int:
    return {"f32": 4, "bf16": 2}[dtype]


@dataclass
class Workload:
    """One decode step's inputs, plus what is needed to build its pool."""

    name: str
    seed: int
    rows: int
    heads: int
    kv_heads: int
    head_dim: int
    block_size: int
    dtype: str
    layout: str
    num_blocks: int
    context_lens: np.ndarray          # int32 [rows]
    block_tables: np.ndarray          # int32 [rows, max_blocks], -1 past the live prefix
    slot_mapping: np.ndarray          # int64 [rows * query_len]: this step's write slots
    q: np.ndarray                     # storage [rows, heads, head_dim], or with
                                      # query_len > 1 [rows, query_len, heads, head_dim]
    k_new: np.ndarray                 # storage [rows * query_len, kv_heads, head_dim]
    v_new: np.ndarray
    scale: float
    meta: dict = field(default_factory=dict)
    query_len: int = 1                # new tokens (queries) per row this step

    @property
    def max_blocks(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def sink(self) -> int:
        return self.num_blocks * self.block_size

    @property
    def pool_shape(self) -> tuple:
        nb1 = self.num_blocks + 1
        if self.layout == "HND":
            return (nb1, self.kv_heads, self.block_size, self.head_dim)
        return (nb1, self.block_size, self.kv_heads, self.head_dim)

    @property
    def pool_bytes(self) -> int:
        """Bytes of K plus V pool storage."""
        return 2 * int(np.prod(self.pool_shape)) * storage_nbytes(self.dtype)

    @property
    def live_rows(self) -> np.ndarray:
        return np.nonzero(self.context_lens > 0)[0]

    @property
    def pad_rows(self) -> np.ndarray:
        return np.nonzero(self.context_lens == 0)[0]

    def history_on_host(self) -> bool:
        return self.pool_bytes <= HOST_POOL_LIMIT


# --------------------------------------------------------------------------- #
# construction helpers
# --------------------------------------------------------------------------- #
def _place_blocks(rng, context_lens, block_size, num_blocks, max_blocks):
    """Seeded random block placement: live blocks are taken, row by row, from one
    permutation of the pool's blocks, so no two rows share a block."""
    need = [cdiv(c, block_size) for c in context_lens]
    if sum(need) > num_blocks:
        raise ValueError("pool too small for the lengths")
    perm = rng.permutation(num_blocks).astype(np.int32)
    tables = np.full((len(context_lens), max_blocks), -1, dtype=np.int32)
    at = 0
    for r, n in enumerate(need):
        tables[r, :n] = perm[at:at + n]
        at += n
    return tables


def _write_slots(context_lens, block_tables, block_size, num_blocks, query_len=1):
    """The step's write slots, query_len per row: the row's last query_len live
    positions (its length includes the tokens written this step), or the sink slot for
    every token of a pad row."""
    slots = np.empty(len(context_lens) * query_len, dtype=np.int64)
    for r, c in enumerate(context_lens):
        for i in range(query_len):
            if c == 0:
                slots[r * query_len + i] = num_blocks * block_size
            else:
                pos = int(c) - query_len + i
                slots[r * query_len + i] = (int(block_tables[r, pos // block_size]) *
                                            block_size + pos % block_size)
    return slots


def _finish(name, seed, rng, lens, *, heads, kv_heads, head_dim, block_size, dtype,
            layout, num_blocks, max_blocks, meta=None, query_len=1):
    lens = np.asarray(lens, dtype=np.int32)
    if np.any((lens > 0) & (lens < query_len)):
        raise ValueError("a live row must hold at least its query_len new tokens")
    tables = _place_blocks(rng, lens, block_size, num_blocks, max_blocks)
    slots = _write_slots(lens, tables, block_size, num_blocks, query_len)
    rows = len(lens)
    q_shape = (rows, heads, head_dim) if query_len == 1 else \
        (rows, query_len, heads, head_dim)
    q = to_storage(rng.standard_normal(q_shape, dtype=np.float32), dtype)
    new_shape = (rows * query_len, kv_heads, head_dim)
    k_new = to_storage(rng.standard_normal(new_shape, dtype=np.float32), dtype)
    v_new = to_storage(rng.standard_normal(new_shape, dtype=np.float32), dtype)
    return Workload(name=name, seed=seed, rows=rows, heads=heads, kv_heads=kv_heads,
                    head_dim=head_dim, block_size=block_size, dtype=dtype, layout=layout,
                    num_blocks=num_blocks, context_lens=lens, block_tables=tables,
                    slot_mapping=slots, q=q, k_new=k_new, v_new=v_new,
                    scale=1.0 / math.sqrt(head_dim), meta=dict(meta or {}),
                    query_len=query_len)


def _lognormal_lens(rng, n, median, sigma, hi):
    x = rng.lognormal(mean=math.log(median), sigma=sigma, size=n)
    return np.clip(np.rint(x), 1, hi).astype(np.int64)


# --------------------------------------------------------------------------- #
# the five named configurations
# --------------------------------------------------------------------------- #
def make_config(index: int, layout: str = "HND", kv_heads: int | None = None,
                query_len: int = 1) -> Workload:
    """Build configuration ``index`` (1..5) with seed = index.

    ``kv_heads`` gives the grouped-query variant of a configuration: the same lengths,
    placement and query heads, with fewer KV heads (query head h reads KV head
    h // (heads // kv_heads)); the pool shrinks by heads / kv_heads.  The named
    configurations themselves have kv_heads == heads.

    ``query_len`` gives the multi-token variant: every row gets query_len new tokens
    (queries), its last query_len positions, and a live row shorter than query_len is
    lengthened to query_len.  The draws are the same up to the shapes of q and the new
    K/V."""
    w = _make_config(index, layout, kv_heads, query_len)
    if kv_heads is not None:
        w.name = f"{w.name}-gqa{w.heads // w.kv_heads}"
    if query_len != 1:
        w.name = f"{w.name}-q{query_len}"
    return w


def _make_config(index, layout, kv_heads_override, query_len=1):
    seed = int(index)
    rng = np.random.default_rng(seed)
    name = CONFIG_NAMES[index]
    bs = 16

    def fin(name, seed, rng, lens, **kw):   # multi-token: live rows hold query_len tokens
        lens = np.asarray(lens, dtype=np.int64)
        lens = np.where(lens > 0, np.maximum(lens, query_len), 0)
        return _finish(name, seed, rng, lens, query_len=query_len, **kw)
    if index == 1:
        lens = [16, 40]
        return fin(name, seed, rng, lens, heads=4, kv_heads=kv_heads_override or 4,
                       head_dim=64,
                       block_size=bs, dtype="f32", layout=layout, num_blocks=8,
                       max_blocks=3)
    if index == 2:
        lens = [2048] * 8
        nb = sum(cdiv(c, bs) for c in lens)
        return fin(name, seed, rng, lens, heads=32, kv_heads=kv_heads_override or 32, head_dim=128,
                       block_size=bs, dtype="bf16", layout=layout, num_blocks=nb,
                       max_blocks=2048 // bs)
    if index == 3:
        live = rng.integers(2048, 8192, size=32, endpoint=True)
        pads = np.sort(rng.choice(34, size=2, replace=False))
        lens = np.zeros(34, dtype=np.int64)
        lens[np.setdiff1d(np.arange(34), pads)] = live
        nb = math.ceil(1.2 * sum(cdiv(c, bs) for c in lens))
        return fin(name, seed, rng, lens, heads=32, kv_heads=kv_heads_override or 32, head_dim=128,
                       block_size=bs, dtype="bf16", layout=layout, num_blocks=nb,
                       max_blocks=8192 // bs, meta={"pad_rows": pads.tolist()})
    if index == 4:
        lens = _lognormal_lens(rng, 256, 256, 1.0, 2048)
        forced = int(rng.integers(256))
        lens[forced] = 2048
        return fin(name, seed, rng, lens, heads=32, kv_heads=kv_heads_override or 32, head_dim=128,
                       block_size=bs, dtype="bf16", layout=layout,
                       num_blocks=256 * 2048 // bs, max_blocks=2048 // bs,
                       meta={"forced_row": forced})
    if index == 5:
        body = _lognormal_lens(rng, 232, 1024, 1.2, 8192)
        lens = np.concatenate([body, np.full(8, 8192), np.zeros(16, dtype=np.int64)])
        lens = lens[rng.permutation(256)]
        return fin(name, seed, rng, lens, heads=32, kv_heads=kv_heads_override or 32, head_dim=128,
                       block_size=bs, dtype="bf16", layout=layout,
                       num_blocks=256 * 8192 // bs, max_blocks=8192 // bs)
    raise ValueError(f"no configuration {index}")


def make_custom(context_lens, *, heads=4, kv_heads=None, head_dim=64, block_size=16,
                dtype="f32", layout="HND", num_blocks=None, max_blocks=None, seed=0,
                name="custom", query_len=1) -> Workload:
    """A small workload for tests: explicit lengths, seeded placement and values."""
    kv_heads = heads if kv_heads is None else kv_heads
    lens = [int(c) for c in context_lens]
    need = sum(cdiv(c, block_size) for c in lens)
    if num_blocks is None:
        num_blocks = max(need + 3, 1)
    if max_blocks is None:
        max_blocks = max(1, max(cdiv(c, block_size) for c in lens) if lens else 1)
    rng = np.random.default_rng(seed)
    return _finish(name, seed, rng, lens, heads=heads, kv_heads=kv_heads,
                   head_dim=head_dim, block_size=block_size, dtype=dtype, layout=layout,
                   num_blocks=num_blocks, max_blocks=max_blocks, query_len=query_len)


# --------------------------------------------------------------------------- #
# pool history
# --------------------------------------------------------------------------- #
def history_host(w: Workload):
    """Host K/V pools with every slot (sink block included) drawn N(0, 1)."""
    rng = np.random.default_rng(w.seed + HISTORY_SEED_OFFSET)
    k = to_storage(rng.standard_normal(w.pool_shape, dtype=np.float32), w.dtype)
    v = to_storage(rng.standard_normal(w.pool_shape, dtype=np.float32), w.dtype)
    return k, v


def history_device(w: Workload, k_cache, v_cache, chunk_elems: int = 1 << 28):
    """Fill device pools (torch tensors of ``w.pool_shape``) with seeded N(0, 1)
    values, in chunks, with torch's device generator.  bf16 values are rounded by
    torch's float32 -> bfloat16 conversion (round to nearest even)."""
    import torch

    gen = torch.Generator(device=k_cache.device)
    gen.manual_seed(w.seed + HISTORY_SEED_OFFSET)
    for t in (k_cache, v_cache):
        flat = t.view(-1)
        for at in range(0, flat.numel(), chunk_elems):
            n = min(chunk_elems, flat.numel() - at)
            flat[at:at + n].copy_(torch.randn(n, generator=gen, device=t.device,
                                              dtype=torch.float32))


def live_blocks(w: Workload, rows=None) -> np.ndarray:
    """The distinct pool blocks the given rows' live table prefixes name."""
    rows = range(w.rows) if rows is None else rows
    ids = [w.block_tables[r, :cdiv(w.context_lens[r], w.block_size)] for r in rows]
    return np.unique(np.concatenate(ids)) if ids else np.zeros(0, dtype=np.int32)

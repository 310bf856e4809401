"""Host arithmetic about a decode step: tiles walked, rectangle size, bytes moved.

Day 59 ("What I added today" and its streambench table) counts the work of the
streamed read two ways: the KV tiles a per-(row, head) loop walks, one
``cdiv(len, tile)`` per row, against the tiles a rectangle of the batch's width
implies; and the bytes of the float32 score rectangle ``rows x heads x width``
against one tile's worth ``rows x heads x tile``.  Day 55 ("What I added today",
the pool-budget table) inverts the rectangle size: a byte budget caps the widest
rectangle at ``budget / (rows x heads x 4)`` tokens.

``algorithmic_bytes`` is the traffic the step cannot avoid: each live (row, KV head,
position) K and V vector once, q and out once, the live block-table prefix and the
lengths once, and the slot scatter's read of the new K/V plus its write into the
pool.  Pad rows and positions past a row's length cost nothing.
"""

from __future__ import annotations

import numpy as np

SCORE_BYTES = 4          # the rectangle's float32 scores
MB = 1e6


def cdiv(a, b):
    return -(-np.asarray(a, dtype=np.int64) // int(b))


def tiles_walked(context_lens, tile: int) -> int:
    """Tiles a per-row streamed loop visits: sum over rows of cdiv(len, tile)."""
    return int(np.sum(cdiv(context_lens, tile)))


def rectangle_tiles(rows: int, width: int, tile: int) -> int:
    """Tiles a [rows, width] rectangle holds."""
    return int(rows) * int(cdiv(width, tile))


def walk_ratio(context_lens, width: int, tile: int) -> float:
    return rectangle_tiles(len(context_lens), width, tile) / tiles_walked(context_lens, tile)


def rectangle_bytes(rows: int, heads: int, width: int, elem: int = SCORE_BYTES) -> int:
    """The [rows, heads, 1, width] score rectangle."""
    return int(rows) * int(heads) * int(width) * int(elem)


def tile_bytes(rows: int, heads: int, tile: int, elem: int = SCORE_BYTES) -> int:
    """One tile of scores per (row, head)."""
    return int(rows) * int(heads) * int(tile) * int(elem)


def widest_capture(budget_bytes: float, rows: int, heads: int,
                   elem: int = SCORE_BYTES) -> int:
    """The widest rectangle a byte budget holds."""
    return int(budget_bytes // (int(rows) * int(heads) * int(elem)))


def algorithmic_bytes(context_lens, *, heads: int, kv_heads: int, head_dim: int,
                      block_size: int, elem: int, write_tokens: int,
                      address: str = "blocks", query_len: int = 1) -> dict:
    """Bytes the step must move, split by component.  ``address`` is how the read is
    addressed: "blocks" reads one int32 block id per live block, "slots" one int64
    rectangle cell per live position (Day 51, "Why it matters": the same information,
    one cell per slot instead of one per block).  ``query_len`` new tokens per row
    each bring a query and an output; K and V are still read once per KV head."""
    ctx = np.asarray(context_lens, dtype=np.int64)
    rows = int(ctx.size)
    kv = int(ctx.sum()) * kv_heads * head_dim * elem * 2
    q_out = 2 * rows * query_len * heads * head_dim * elem
    if address == "blocks":
        tables = int(np.sum(cdiv(ctx, block_size))) * 4 + rows * 4
    elif address == "slots":
        tables = int(ctx.sum()) * 8 + rows * 4
    else:
        raise ValueError(f"unknown address {address!r}")
    write = 2 * int(write_tokens) * kv_heads * head_dim * elem * 2
    read_total = kv + q_out + tables
    return {"kv": kv, "q_out": q_out, "tables": tables, "attention": read_total,
            "kv_write": write, "total": read_total + write}


def row_heads(context_lens, heads: int) -> int:
    """(row, head) pairs with something to attend over."""
    return int(np.count_nonzero(np.asarray(context_lens) > 0)) * int(heads)

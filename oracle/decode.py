"""The oracle's arithmetic: slot scatter, rectangle mapping, masked softmax read.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use this module.

Conventions shared with the library's C boundary (restated here, not imported):

* storage dtype ``"f32"`` is a ``numpy.float32`` array; ``"bf16"`` is a
  ``numpy.uint16`` array holding bfloat16 bit patterns;
* the K and V pools each hold ``num_blocks + 1`` blocks of ``block_size`` slots;
  the extra last block holds the sink slot ``num_blocks * block_size``, which is a
  legal write target that no block table may name;
* layout ``"HND"`` stores a pool as ``[num_blocks + 1, kv_heads, block_size, head_dim]``
  and ``"NHD"`` as ``[num_blocks + 1, block_size, kv_heads, head_dim]``; both are the
  same slot-indexed pool ``[slots, kv_heads, head_dim]`` with a different order of
  the two middle axes;
* ``q`` and the output are ``[rows, heads, head_dim]``; query head ``h`` reads KV
  head ``h // (heads // kv_heads)``;
* ``block_tables`` is int32 ``[rows, max_blocks]`` and ``context_lens`` int32 ``[rows]``;
  ``slot_mapping`` is int64 ``[tokens]``;
* the read may instead be addressed by a slot rectangle, int64 ``[rows, width]``, whose
  cell (r, t) names the slot holding position t of row r (cells at or past the row's
  length may hold anything and are never read).

Every floating-point operation is float64.
"""

from __future__ import annotations

import numpy as np

LAYOUTS = ("HND", "NHD")
REFUSAL_CODES = ("EMPTY", "DTYPE", "SHAPE", "CONTEXT_BOUNDS", "BLOCK_ID", "SLOT")

_STORAGE = {"f32": np.float32, "bf16": np.uint16}


class Refusal(ValueError):
    """An input the step refuses.  ``code`` is one of ``REFUSAL_CODES``."""

    def __init__(self, code: str, detail: str):
        assert code in REFUSAL_CODES
        super().__init__(f"{code}: {detail}")
        self.code = code
        self.detail = detail


# --------------------------------------------------------------------------- #
# storage decoding
# --------------------------------------------------------------------------- #
def decode_storage(a: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array -> float64.

    bfloat16 is the upper half of an IEEE binary32, so a bf16 bit pattern widened
    by a 16-bit left shift is the same number as a float32; both widenings are
    exact.
    """
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def sink_slot(num_blocks: int, block_size: int) -> int:
    """The sink slot: one past the last slot the allocator hands out.

    Day 55 ("Why it matters"): a pad row's K/V goes to a slot that is a legal
    address but that no block table can name.  The pool's extra last block holds it.
    """
    return int(num_blocks) * int(block_size)


def _pool_shape(num_blocks, block_size, kv_heads, head_dim, layout):
    if layout == "HND":
        return (num_blocks + 1, kv_heads, block_size, head_dim)
    if layout == "NHD":
        return (num_blocks + 1, block_size, kv_heads, head_dim)
    raise ValueError(f"unknown layout {layout!r}")


def slot_view(cache: np.ndarray, layout: str) -> np.ndarray:
    """A pool as ``[slots, kv_heads, head_dim]`` (slot = block * block_size + offset)."""
    if layout == "NHD":
        nb1, bs, hkv, d = cache.shape
        return cache.reshape(nb1 * bs, hkv, d)
    if layout == "HND":
        nb1, hkv, bs, d = cache.shape
        return np.ascontiguousarray(cache.transpose(0, 2, 1, 3)).reshape(nb1 * bs, hkv, d)
    raise ValueError(f"unknown layout {layout!r}")


# --------------------------------------------------------------------------- #
# refusals
# --------------------------------------------------------------------------- #
def _check_pool(k_cache, v_cache, num_blocks, block_size, layout, dtype):
    if k_cache.dtype != _STORAGE[dtype] or v_cache.dtype != _STORAGE[dtype]:
        raise Refusal("DTYPE", "pool storage does not match the declared dtype")


def _pool_dims(k_cache, layout):
    if k_cache.ndim != 4:
        return None
    if layout == "HND":
        _, hkv, _, d = k_cache.shape
    else:
        _, _, hkv, d = k_cache.shape
    return hkv, d


def validate_write(k_cache, v_cache, k, v, slot_mapping, *, num_blocks, block_size,
                   layout, dtype):
    """Refusals of the slot scatter, checked in the order EMPTY, DTYPE, SHAPE, SLOT.

    The slot range [0, sink] follows Day 55 ("Why it matters"): every real write
    names a slot the allocator handed out and a pad row names the sink; nothing
    else is a legal address.
    """
    n = int(np.asarray(slot_mapping).shape[0]) if np.ndim(slot_mapping) >= 1 else 0
    if n == 0:
        raise Refusal("EMPTY", "no tokens to write")
    _check_pool(k_cache, v_cache, num_blocks, block_size, layout, dtype)
    if k.dtype != _STORAGE[dtype] or v.dtype != _STORAGE[dtype]:
        raise Refusal("DTYPE", "new K/V storage does not match the declared dtype")
    if np.asarray(slot_mapping).dtype != np.int64:
        raise Refusal("DTYPE", "slot_mapping must be int64")
    dims = _pool_dims(k_cache, layout)
    if dims is None:
        raise Refusal("SHAPE", "pool must be 4-D")
    hkv, d = dims
    want = _pool_shape(num_blocks, block_size, hkv, d, layout)
    if k_cache.shape != want or v_cache.shape != want:
        raise Refusal("SHAPE", f"pool shape {k_cache.shape} != {want}")
    if k.shape != (n, hkv, d) or v.shape != (n, hkv, d):
        raise Refusal("SHAPE", f"new K/V shape {k.shape} != {(n, hkv, d)}")
    if np.asarray(slot_mapping).shape != (n,):
        raise Refusal("SHAPE", "slot_mapping must be 1-D")
    sink = sink_slot(num_blocks, block_size)
    sm = np.asarray(slot_mapping)
    bad = np.nonzero((sm < 0) | (sm > sink))[0]
    if bad.size:
        i = int(bad[0])
        raise Refusal("SLOT", f"slot_mapping[{i}] = {int(sm[i])} outside [0, {sink}]")


def validate_attention(q, k_cache, v_cache, block_tables, context_lens, *, num_blocks,
                       block_size, layout, dtype):
    """Refusals of the read, checked in the order EMPTY, DTYPE, SHAPE, CONTEXT_BOUNDS,
    BLOCK_ID.

    * A length may not be negative, may not exceed what the row's table can address
      (max_blocks * block_size) and may not exceed the pool's slot count: Day 51
      ("What I added today") clamps the longest row to the pool for that reason.
    * Only the live prefix of a table row (entries j < cdiv(len, block_size)) is
      addressed; each such entry must be an allocatable block in [0, num_blocks).
      The sink block is not nameable (Day 55, "Why it matters").  Entries past the
      live prefix, -1 included, are never read (Day 59, "Why it matters") and are
      not checked.
    """
    limit = _check_read_shape(q, k_cache, v_cache, block_tables, context_lens,
                              num_blocks=num_blocks, block_size=block_size, layout=layout,
                              dtype=dtype)
    _check_lengths(context_lens, limit)
    _check_block_ids(block_tables, context_lens, num_blocks, block_size)


def _check_read_shape(q, k_cache, v_cache, block_tables, context_lens, *, num_blocks,
                      block_size, layout, dtype):
    """EMPTY, DTYPE and SHAPE of the read; returns the largest legal length."""
    ctx = np.asarray(context_lens)
    bt = np.asarray(block_tables)
    r = int(ctx.shape[0]) if ctx.ndim >= 1 else 0
    if r == 0:
        raise Refusal("EMPTY", "no rows")
    _check_pool(k_cache, v_cache, num_blocks, block_size, layout, dtype)
    if q.dtype != _STORAGE[dtype]:
        raise Refusal("DTYPE", "q storage does not match the declared dtype")
    if ctx.dtype != np.int32 or bt.dtype != np.int32:
        raise Refusal("DTYPE", "block_tables and context_lens must be int32")
    dims = _pool_dims(k_cache, layout)
    if dims is None:
        raise Refusal("SHAPE", "pool must be 4-D")
    hkv, d = dims
    want = _pool_shape(num_blocks, block_size, hkv, d, layout)
    if k_cache.shape != want or v_cache.shape != want:
        raise Refusal("SHAPE", f"pool shape {k_cache.shape} != {want}")
    if q.ndim != 3 or q.shape[0] != r or q.shape[2] != d:
        raise Refusal("SHAPE", f"q shape {q.shape} does not match rows={r}, head_dim={d}")
    h = q.shape[1]
    if h == 0 or h % hkv != 0:
        raise Refusal("SHAPE", f"{h} query heads is not a multiple of {hkv} KV heads")
    if ctx.shape != (r,) or bt.ndim != 2 or bt.shape[0] != r or bt.shape[1] < 1:
        raise Refusal("SHAPE", "block_tables must be [rows, max_blocks>=1], context_lens [rows]")
    return min(int(bt.shape[1]) * block_size, num_blocks * block_size)


def _check_lengths(context_lens, limit):
    ctx = np.asarray(context_lens)
    bad = np.nonzero((ctx < 0) | (ctx > limit))[0]
    if bad.size:
        i = int(bad[0])
        raise Refusal("CONTEXT_BOUNDS",
                      f"context_lens[{i}] = {int(ctx[i])} outside [0, {limit}]")


def _check_block_ids(block_tables, context_lens, num_blocks, block_size):
    ctx = np.asarray(context_lens)
    bt = np.asarray(block_tables)
    for row in range(int(ctx.shape[0])):
        live = -(-int(ctx[row]) // block_size)
        ids = bt[row, :live]
        wrong = np.nonzero((ids < 0) | (ids >= num_blocks))[0]
        if wrong.size:
            j = int(wrong[0])
            raise Refusal("BLOCK_ID", f"block_tables[{row}, {j}] = {int(ids[j])} "
                                      f"outside [0, {num_blocks})")


def validate_attention_slots(q, k_cache, v_cache, slot_rect, context_lens, *, num_blocks,
                             block_size, layout, dtype):
    """Refusals of the read addressed by a slot rectangle, in the order EMPTY, DTYPE,
    SHAPE, CONTEXT_BOUNDS, SLOT.

    Day 51 ("What I added today"): the decode step reads through a persistent
    [max_batch, max_model_len] int64 slot table, handed to the read as the window
    ``slots[:rows, :width]``, with the lengths passed beside it.

    * A length may not be negative, may not exceed the rectangle's width and may not
      exceed the pool's slot count.
    * Every live cell (t < len) must name an allocatable slot, in [0, num_blocks *
      block_size).  The sink holds padding writes only and is no row's token (Day 55,
      "Why it matters").  Cells past a row's length are never read and not checked:
      a re-tenanted row keeps its old tenant's slots there (Day 51, "What I learned").
    """
    ctx = np.asarray(context_lens)
    rect = np.asarray(slot_rect)
    r = int(ctx.shape[0]) if ctx.ndim >= 1 else 0
    if r == 0:
        raise Refusal("EMPTY", "no rows")
    _check_pool(k_cache, v_cache, num_blocks, block_size, layout, dtype)
    if q.dtype != _STORAGE[dtype]:
        raise Refusal("DTYPE", "q storage does not match the declared dtype")
    if ctx.dtype != np.int32 or rect.dtype != np.int64:
        raise Refusal("DTYPE", "the slot rectangle must be int64 and context_lens int32")
    dims = _pool_dims(k_cache, layout)
    if dims is None:
        raise Refusal("SHAPE", "pool must be 4-D")
    hkv, d = dims
    want = _pool_shape(num_blocks, block_size, hkv, d, layout)
    if k_cache.shape != want or v_cache.shape != want:
        raise Refusal("SHAPE", f"pool shape {k_cache.shape} != {want}")
    if q.ndim != 3 or q.shape[0] != r or q.shape[2] != d:
        raise Refusal("SHAPE", f"q shape {q.shape} does not match rows={r}, head_dim={d}")
    h = q.shape[1]
    if h == 0 or h % hkv != 0:
        raise Refusal("SHAPE", f"{h} query heads is not a multiple of {hkv} KV heads")
    if ctx.shape != (r,) or rect.ndim != 2 or rect.shape[0] != r or rect.shape[1] < 1:
        raise Refusal("SHAPE", "slot rectangle must be [rows, width>=1], context_lens [rows]")
    width = int(rect.shape[1])
    slots = num_blocks * block_size
    limit = min(width, slots)
    bad = np.nonzero((ctx < 0) | (ctx > limit))[0]
    if bad.size:
        i = int(bad[0])
        raise Refusal("CONTEXT_BOUNDS",
                      f"context_lens[{i}] = {int(ctx[i])} outside [0, {limit}]")
    for row in range(r):
        cells = rect[row, :int(ctx[row])]
        wrong = np.nonzero((cells < 0) | (cells >= slots))[0]
        if wrong.size:
            t = int(wrong[0])
            raise Refusal("SLOT", f"slot rectangle [{row}, {t}] = {int(cells[t])} "
                                  f"outside [0, {slots})")


def validate_attention_multi(q, k_cache, v_cache, block_tables, context_lens, *,
                             num_blocks, block_size, layout, dtype):
    """Refusals of the multi-token read, in the order EMPTY, DTYPE, SHAPE,
    CONTEXT_BOUNDS, BLOCK_ID: those of the decode read, with q
    ``[rows, query_len, heads, head_dim]`` and one more bound, a live row's length
    counting its query_len new tokens, so it is 0 or at least query_len."""
    ctx = np.asarray(context_lens)
    r = int(ctx.shape[0]) if ctx.ndim >= 1 else 0
    if r == 0:
        raise Refusal("EMPTY", "no rows")
    _check_pool(k_cache, v_cache, num_blocks, block_size, layout, dtype)
    if q.dtype != _STORAGE[dtype]:
        raise Refusal("DTYPE", "q storage does not match the declared dtype")
    if q.ndim != 4 or q.shape[0] != r or q.shape[1] < 1:
        raise Refusal("SHAPE", f"q shape {q.shape} is not [rows={r}, query_len>=1, heads, d]")
    n_q = int(q.shape[1])
    limit = _check_read_shape(q[:, 0], k_cache, v_cache, block_tables, context_lens,
                              num_blocks=num_blocks, block_size=block_size, layout=layout,
                              dtype=dtype)
    _check_lengths(context_lens, limit)
    short = np.nonzero((ctx > 0) & (ctx < n_q))[0]
    if short.size:
        i = int(short[0])
        raise Refusal("CONTEXT_BOUNDS", f"context_lens[{i}] = {int(ctx[i])} is live but "
                                        f"shorter than query_len {n_q}")
    _check_block_ids(block_tables, context_lens, num_blocks, block_size)


# --------------------------------------------------------------------------- #
# O1: the slot scatter
# --------------------------------------------------------------------------- #
def kv_write(k_cache, v_cache, k, v, slot_mapping, *, num_blocks, block_size, layout,
             dtype):
    """Write token i's K/V into slot ``slot_mapping[i]`` of each pool, in place.

    Day 55 ("Why it matters"): the whole padded batch is one indexed assignment;
    pad rows carry the sink slot.  Tokens are written in index order, so when the
    same slot appears twice (only the sink may) the last writer's values remain.
    """
    validate_write(k_cache, v_cache, k, v, slot_mapping, num_blocks=num_blocks,
                   block_size=block_size, layout=layout, dtype=dtype)
    for i, slot in enumerate(np.asarray(slot_mapping).tolist()):
        block, offset = divmod(int(slot), block_size)
        if layout == "HND":
            k_cache[block, :, offset, :] = k[i]
            v_cache[block, :, offset, :] = v[i]
        else:
            k_cache[block, offset, :, :] = k[i]
            v_cache[block, offset, :, :] = v[i]


# --------------------------------------------------------------------------- #
# O2-O3: width and mapping
# --------------------------------------------------------------------------- #
def rebuild_mapping(block_tables, context_lens, block_size):
    """The [rows, width] slot rectangle of a batch, and its live mask.

    width is the longest context in the batch.  Live cell (r, t), t < len_r, holds
    ``block_tables[r, t // block_size] * block_size + t % block_size`` (Day 51, "Why
    it matters": block id times block size plus offset).  Cells past a row's length
    hold slot 0: the reference only needs a legal index there because it gathers
    before it masks (Day 51, "What I learned").
    """
    ctx = np.asarray(context_lens, dtype=np.int64)
    width = int(ctx.max()) if ctx.size else 0
    t = np.arange(width, dtype=np.int64)
    live = t[None, :] < ctx[:, None]
    if width == 0:
        return np.zeros((ctx.size, 0), dtype=np.int64), live
    ids = np.asarray(block_tables, dtype=np.int64)[:, t // block_size]
    slots = ids * block_size + (t % block_size)[None, :]
    return np.where(live, slots, 0), live


# --------------------------------------------------------------------------- #
# O4: gather
# --------------------------------------------------------------------------- #
def gather(cache, mapping, layout, dtype):
    """K or V at every cell of the slot rectangle: ``[rows, width, kv_heads, head_dim]``
    in float64."""
    flat = slot_view(cache, layout)
    return decode_storage(flat[mapping], dtype)


# --------------------------------------------------------------------------- #
# O5-O9: scores, mask, softmax, weighted V
# --------------------------------------------------------------------------- #
def paged_attention(q, k_cache, v_cache, block_tables, context_lens, scale, *,
                    num_blocks, block_size, layout, dtype):
    """The masked-rectangle decode read, float64 ``[rows, heads, head_dim]``.

    Day 59 ("What I added today") describes it: the [batch, max_ctx] mapping is
    gathered into K and V, each query head scores the whole rectangle into
    [batch, heads, 1, max_ctx], the scores past each row's length are masked, and
    the softmax weights multiply V.  A row of length 0 attends over nothing and its
    output is zero (its whole score row is masked; Day 51, "Tomorrow", and Day 55,
    "Why it matters").
    """
    validate_attention(q, k_cache, v_cache, block_tables, context_lens,
                       num_blocks=num_blocks, block_size=block_size, layout=layout,
                       dtype=dtype)
    mapping, live = rebuild_mapping(block_tables, context_lens, block_size)
    return _attend(q, k_cache, v_cache, mapping, live, context_lens, scale, layout, dtype)


def paged_attention_slots(q, k_cache, v_cache, slot_rect, context_lens, scale, *,
                          num_blocks, block_size, layout, dtype):
    """The same read with the rectangle handed in rather than rebuilt from block
    tables, float64 ``[rows, heads, head_dim]``.

    Day 51 ("What I added today"): the read is given the window of the slot table and
    the lengths.  The mapping is the window's first max(len) columns, with the cells
    past each row's length replaced by slot 0, a legal index the mask then discards
    (Day 51, "What I learned": the reference gathers before it masks).
    """
    validate_attention_slots(q, k_cache, v_cache, slot_rect, context_lens,
                             num_blocks=num_blocks, block_size=block_size, layout=layout,
                             dtype=dtype)
    ctx = np.asarray(context_lens, dtype=np.int64)
    width = int(ctx.max())
    t = np.arange(width, dtype=np.int64)
    live = t[None, :] < ctx[:, None]
    mapping = np.where(live, np.asarray(slot_rect)[:, :width], 0)
    return _attend(q, k_cache, v_cache, mapping, live, context_lens, scale, layout, dtype)


def _attend(q, k_cache, v_cache, mapping, live, context_lens, scale, layout, dtype):
    """Gather, score, mask, softmax and weight V over a [rows, width] slot mapping
    whose cells outside ``live`` are legal but meaningless (Day 59, "What I added
    today")."""
    rows, heads, head_dim = q.shape
    kv_heads = k_cache.shape[1] if layout == "HND" else k_cache.shape[2]
    group = heads // kv_heads
    kv_of_head = np.arange(heads) // group                     # query head -> KV head

    width = mapping.shape[1]
    out = np.zeros((rows, heads, head_dim), dtype=np.float64)
    if width == 0:
        return out

    kg = gather(k_cache, mapping, layout, dtype)[:, :, kv_of_head, :]  # [R, W, H, D]
    vg = gather(v_cache, mapping, layout, dtype)[:, :, kv_of_head, :]
    qf = decode_storage(q, dtype)                                       # [R, H, D]

    # scores [R, H, 1, W] = scale * q . k
    scores = float(scale) * np.matmul(qf[:, :, None, :], kg.transpose(0, 2, 3, 1))
    # mask columns past each row's length
    scores = np.where(live[:, None, None, :], scores, -np.inf)
    # softmax over the width axis, shifted by the row maximum
    has_keys = np.asarray(context_lens) > 0
    peak = np.max(scores, axis=-1, keepdims=True)
    peak = np.where(has_keys[:, None, None, None], peak, 0.0)
    weights = np.exp(scores - peak)
    denom = np.sum(weights, axis=-1, keepdims=True)
    denom = np.where(has_keys[:, None, None, None], denom, 1.0)
    probs = weights / denom
    # weighted sum of V: [R, H, 1, W] @ [R, H, W, D]
    out = np.matmul(probs, vg.transpose(0, 2, 1, 3))[:, :, 0, :]
    out[~has_keys] = 0.0
    return out


# --------------------------------------------------------------------------- #
# several new tokens per row
# --------------------------------------------------------------------------- #
def paged_attention_multi(q, k_cache, v_cache, block_tables, context_lens, scale, *,
                          num_blocks, block_size, layout, dtype):
    """The read with query_len new tokens per row, float64
    ``[rows, query_len, heads, head_dim]``.

    The rectangle of Day 59 ("Why it matters") has a query_len axis beside rows and
    heads; query i of row r is the token at position len_r - query_len + i, and it
    attends causally, over the positions t <= its own.  The scores are
    [rows, heads, query_len, width]; a length-0 row's outputs are zero.
    """
    validate_attention_multi(q, k_cache, v_cache, block_tables, context_lens,
                             num_blocks=num_blocks, block_size=block_size, layout=layout,
                             dtype=dtype)
    rows, n_q, heads, head_dim = q.shape
    kv_heads = k_cache.shape[1] if layout == "HND" else k_cache.shape[2]
    kv_of_head = np.arange(heads) // (heads // kv_heads)
    mapping, live = rebuild_mapping(block_tables, context_lens, block_size)
    width = mapping.shape[1]
    out = np.zeros((rows, n_q, heads, head_dim), dtype=np.float64)
    if width == 0:
        return out
    ctx = np.asarray(context_lens, dtype=np.int64)
    kg = gather(k_cache, mapping, layout, dtype)[:, :, kv_of_head, :]  # [R, W, H, D]
    vg = gather(v_cache, mapping, layout, dtype)[:, :, kv_of_head, :]
    qf = decode_storage(q, dtype).transpose(0, 2, 1, 3)                 # [R, H, n_q, D]
    scores = float(scale) * np.matmul(qf, kg.transpose(0, 2, 3, 1))     # [R, H, n_q, W]
    # query i sees t <= len - n_q + i (which also keeps t < len)
    last = ctx[:, None] - n_q + np.arange(n_q)[None, :]                 # [R, n_q]
    t = np.arange(width)
    visible = t[None, None, :] <= last[:, :, None]                      # [R, n_q, W]
    scores = np.where(visible[:, None, :, :], scores, -np.inf)
    has_keys = ctx > 0
    peak = np.max(scores, axis=-1, keepdims=True)
    peak = np.where(has_keys[:, None, None, None], peak, 0.0)
    weights = np.exp(scores - peak)
    denom = np.sum(weights, axis=-1, keepdims=True)
    denom = np.where(has_keys[:, None, None, None], denom, 1.0)
    probs = weights / denom
    res = np.matmul(probs, vg.transpose(0, 2, 1, 3))                   # [R, H, n_q, D]
    out = res.transpose(0, 2, 1, 3).copy()
    out[~has_keys] = 0.0
    return out

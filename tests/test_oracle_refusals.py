"""The oracle refuses exactly the inputs the step refuses, with the same codes."""

import numpy as np
import pytest

import oracle
from paged_attention_decode_kv_amd import workloads as wl


def _setup(lens=(16, 40, 0), dtype="f32", layout="HND"):
    w = wl.make_custom(list(lens), heads=4, kv_heads=2, head_dim=16, dtype=dtype,
                       layout=layout, seed=2)
    k, v = wl.history_host(w)
    return w, k, v


def _attn(w, k, v, **over):
    a = dict(q=w.q, block_tables=w.block_tables, context_lens=w.context_lens)
    a.update(over)
    return oracle.paged_attention(a["q"], k, v, a["block_tables"], a["context_lens"],
                                  w.scale, num_blocks=w.num_blocks,
                                  block_size=w.block_size, layout=w.layout, dtype=w.dtype)


def _code(fn):
    with pytest.raises(oracle.Refusal) as e:
        fn()
    return e.value.code


def test_legal_edges_are_accepted():
    w, k, v = _setup()
    _attn(w, k, v)
    # a length that fills its table exactly
    bt = np.full((1, 2), -1, dtype=np.int32)
    bt[0] = [1, 2]
    _attn(w, k, v, q=w.q[:1], block_tables=bt, context_lens=np.array([32], np.int32))
    # -1 past the live prefix, and an all-padding batch with -1 tables
    _attn(w, k, v, q=w.q[:1], block_tables=np.array([[3, -1]], np.int32),
          context_lens=np.array([16], np.int32))
    _attn(w, k, v, q=w.q[:2], block_tables=np.full((2, 3), -1, np.int32),
          context_lens=np.zeros(2, np.int32))
    # the sink is a legal write target, several times over
    sm = np.full(3, w.sink, dtype=np.int64)
    oracle.kv_write(k, v, w.k_new, w.v_new, sm, num_blocks=w.num_blocks,
                    block_size=w.block_size, layout=w.layout, dtype=w.dtype)


def test_attention_refusals():
    w, k, v = _setup()
    assert _code(lambda: _attn(w, k, v, q=w.q[:0], block_tables=w.block_tables[:0],
                               context_lens=w.context_lens[:0])) == "EMPTY"
    assert _code(lambda: _attn(w, k, v, context_lens=w.context_lens.astype(np.int64))) == "DTYPE"
    assert _code(lambda: _attn(w, k, v, q=w.q.astype(np.float64))) == "DTYPE"
    assert _code(lambda: _attn(w, k, v, q=w.q[:, :3])) == "SHAPE"          # 3 % 2 != 0
    assert _code(lambda: _attn(w, k, v, q=w.q[:, :, :8])) == "SHAPE"
    assert _code(lambda: _attn(w, k, v, block_tables=w.block_tables[:2])) == "SHAPE"
    lens = w.context_lens.copy(); lens[1] = -1
    assert _code(lambda: _attn(w, k, v, context_lens=lens)) == "CONTEXT_BOUNDS"
    lens = w.context_lens.copy(); lens[1] = w.max_blocks * w.block_size + 1
    assert _code(lambda: _attn(w, k, v, context_lens=lens)) == "CONTEXT_BOUNDS"
    bt = w.block_tables.copy(); bt[1, 2] = -1
    assert _code(lambda: _attn(w, k, v, block_tables=bt)) == "BLOCK_ID"
    bt = w.block_tables.copy(); bt[1, 0] = w.num_blocks        # the sink block
    assert _code(lambda: _attn(w, k, v, block_tables=bt)) == "BLOCK_ID"


def test_length_is_capped_by_the_pool():
    w = wl.make_custom([16], heads=2, head_dim=16, num_blocks=2, max_blocks=4, seed=1)
    k, v = wl.history_host(w)
    bt = np.array([[0, 1, -1, -1]], np.int32)
    _attn(w, k, v, block_tables=bt, context_lens=np.array([32], np.int32))
    assert _code(lambda: _attn(w, k, v, block_tables=bt,
                               context_lens=np.array([33], np.int32))) == "CONTEXT_BOUNDS"


def test_write_refusals():
    w, k, v = _setup()
    def wr(**o):
        a = dict(k=w.k_new, v=w.v_new, sm=w.slot_mapping)
        a.update(o)
        oracle.kv_write(k, v, a["k"], a["v"], a["sm"], num_blocks=w.num_blocks,
                        block_size=w.block_size, layout=w.layout, dtype=w.dtype)
    assert _code(lambda: wr(k=w.k_new[:0], v=w.v_new[:0], sm=w.slot_mapping[:0])) == "EMPTY"
    assert _code(lambda: wr(sm=w.slot_mapping.astype(np.int32))) == "DTYPE"
    assert _code(lambda: wr(k=w.k_new[:, :1])) == "SHAPE"
    sm = w.slot_mapping.copy(); sm[0] = w.sink + 1
    assert _code(lambda: wr(sm=sm)) == "SLOT"
    sm = w.slot_mapping.copy(); sm[2] = -1
    assert _code(lambda: wr(sm=sm)) == "SLOT"


def test_refused_write_touches_nothing():
    w, k, v = _setup()
    k0, v0 = k.copy(), v.copy()
    sm = w.slot_mapping.copy(); sm[-1] = -5
    with pytest.raises(oracle.Refusal):
        oracle.kv_write(k, v, w.k_new, w.v_new, sm, num_blocks=w.num_blocks,
                        block_size=w.block_size, layout=w.layout, dtype=w.dtype)
    assert np.array_equal(k, k0) and np.array_equal(v, v0)

"""Pins of the CPU oracle against things other than itself.

* brute force: per-(row, head) softmax attention in plain Python floats, reading the
  pool through block id and offset (not through the oracle's rectangle), and taking
  each row's newest token from the step's new K/V rather than from the pool;
* a library routine: torch's CPU float64 scaled_dot_product_attention per row;
* closed forms: one key, two keys (a logistic weight), zero scale / zero query
  (plain mean of V), equal keys, one dominant key;
* invariants: a constant added to every key, an affine map of V, row permutation,
  physical block relabelling, head independence, stale-tail and unnamed-block
  independence, pad rows inert;
* the slot scatter: written slots bit-exact, everything else untouched, only the
  sink receives pad-row writes, the last writer wins on the sink.
"""

import math
import struct
import zlib

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from paged_attention_decode_kv_amd import workloads as wl

LAYOUTS = ("HND", "NHD")


# --------------------------------------------------------------------------- #
# helpers written independently of the oracle
# --------------------------------------------------------------------------- #
def _scalar(bits_or_value, dtype):
    if dtype == "bf16":
        return struct.unpack("<f", struct.pack("<I", int(bits_or_value) << 16))[0]
    return float(bits_or_value)


def _vec(arr, dtype):
    return [_scalar(x, dtype) for x in np.asarray(arr).ravel().tolist()]


def _pool_vec(cache, layout, block, kvh, offset, dtype):
    if layout == "HND":
        return _vec(cache[block, kvh, offset, :], dtype)
    return _vec(cache[block, offset, kvh, :], dtype)


def brute_force(w, k_pool, v_pool, *, scale=None, q=None):
    """Per-(row, head) softmax attention, Python floats, no rectangle.

    ``k_pool``/``v_pool`` are the pools *before* the step's write; position len-1 of
    each live row is read from the step's new K/V instead.
    """
    scale = w.scale if scale is None else scale
    q = w.q if q is None else q
    group = w.heads // w.kv_heads
    out = np.zeros((w.rows, w.heads, w.head_dim))
    for r in range(w.rows):
        n = int(w.context_lens[r])
        for h in range(w.heads):
            kvh = h // group
            qv = _vec(q[r, h], w.dtype)
            keys, vals = [], []
            for t in range(n):
                if t == n - 1:
                    keys.append(_vec(w.k_new[r, kvh], w.dtype))
                    vals.append(_vec(w.v_new[r, kvh], w.dtype))
                    continue
                b, o = divmod(t, w.block_size)
                blk = int(w.block_tables[r, b])
                keys.append(_pool_vec(k_pool, w.layout, blk, kvh, o, w.dtype))
                vals.append(_pool_vec(v_pool, w.layout, blk, kvh, o, w.dtype))
            if n == 0:
                continue
            s = [scale * math.fsum(a * b for a, b in zip(qv, kk)) for kk in keys]
            top = max(s)
            e = [math.exp(x - top) for x in s]
            z = math.fsum(e)
            for d in range(w.head_dim):
                out[r, h, d] = math.fsum(e[t] * vals[t][d] for t in range(n)) / z
    return out


def run_oracle(w, k_pool, v_pool, **over):
    k = k_pool.copy()
    v = v_pool.copy()
    oracle.kv_write(k, v, w.k_new, w.v_new, w.slot_mapping, num_blocks=w.num_blocks,
                    block_size=w.block_size, layout=w.layout, dtype=w.dtype)
    args = dict(q=w.q, block_tables=w.block_tables, context_lens=w.context_lens,
                scale=w.scale)
    args.update(over)
    out = oracle.paged_attention(args["q"], k, v, args["block_tables"],
                                 args["context_lens"], args["scale"],
                                 num_blocks=w.num_blocks, block_size=w.block_size,
                                 layout=w.layout, dtype=w.dtype)
    return out, k, v


def small_cases():
    cases = []
    for layout in LAYOUTS:
        for dtype in ("f32", "bf16"):
            for heads, kvh in ((4, 4), (4, 2), (4, 1)):
                for lens, bs in (([1, 15, 16, 17], 16), ([32, 33, 0, 5], 16),
                                 ([7, 9, 1], 4)):
                    cases.append((layout, dtype, heads, kvh, tuple(lens), bs))
    return cases


# --------------------------------------------------------------------------- #
# brute force
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("layout", LAYOUTS)
def test_config1_matches_brute_force(layout):
    w = wl.make_config(1, layout=layout)
    k, v = wl.history_host(w)
    got, _, _ = run_oracle(w, k, v)
    want = brute_force(w, k, v)
    assert np.max(np.abs(got - want)) <= 1e-12


@pytest.mark.parametrize("layout,dtype,heads,kvh,lens,bs", small_cases())
def test_small_shapes_match_brute_force(layout, dtype, heads, kvh, lens, bs):
    w = wl.make_custom(lens, heads=heads, kv_heads=kvh, head_dim=16, block_size=bs,
                       dtype=dtype, layout=layout,
                       seed=zlib.crc32(repr((layout, dtype, heads, kvh, lens, bs)).encode()))
    k, v = wl.history_host(w)
    got, _, _ = run_oracle(w, k, v)
    want = brute_force(w, k, v)
    assert np.max(np.abs(got - want)) <= 1e-12


def test_brute_force_detects_planted_mistakes():
    """Plausible oracle mistakes (transposed head map, off-by-one mask, missing scale)
    are caught by the brute-force comparison."""
    w = wl.make_custom([17, 33, 5], heads=4, kv_heads=2, head_dim=16, dtype="f32")
    k, v = wl.history_host(w)
    want = brute_force(w, k, v)
    got, _, _ = run_oracle(w, k, v)
    assert np.max(np.abs(got - want)) <= 1e-12
    # an oracle that forgot the scale
    bad, _, _ = run_oracle(w, k, v, scale=1.0)
    assert np.max(np.abs(bad - want)) > 1e-3
    # an oracle that dropped each row's newest token (length off by one)
    lens = w.context_lens.copy()
    lens[lens > 1] -= 1
    bad, _, _ = run_oracle(w, k, v, context_lens=lens)
    assert np.max(np.abs(bad - want)) > 1e-3
    # an oracle that read the other KV head (GQA map reversed)
    q_swapped = w.q[:, ::-1, :].copy()
    bad, _, _ = run_oracle(w, k, v, q=q_swapped)
    assert np.max(np.abs(bad[:, ::-1, :] - want)) > 1e-3


# --------------------------------------------------------------------------- #
# a library routine
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("kvh", [4, 2])
def test_matches_torch_sdpa(layout, kvh):
    w = wl.make_custom([40, 1, 0, 23, 64], heads=4, kv_heads=kvh, head_dim=32,
                       dtype="bf16", layout=layout, seed=11)
    k, v = wl.history_host(w)
    got, kw, vw = run_oracle(w, k, v)
    kf = oracle.slot_view(kw, layout)
    vf = oracle.slot_view(vw, layout)
    group = w.heads // w.kv_heads
    for r in range(w.rows):
        n = int(w.context_lens[r])
        if n == 0:
            assert np.all(got[r] == 0)
            continue
        slots = [int(w.block_tables[r, t // w.block_size]) * w.block_size
                 + t % w.block_size for t in range(n)]
        kr = torch.from_numpy(oracle.decode_storage(kf[slots], "bf16"))   # [n, Hkv, D]
        vr = torch.from_numpy(oracle.decode_storage(vf[slots], "bf16"))
        kr = kr.repeat_interleave(group, dim=1).permute(1, 0, 2).contiguous()
        vr = vr.repeat_interleave(group, dim=1).permute(1, 0, 2).contiguous()
        qr = torch.from_numpy(oracle.decode_storage(w.q[r], "bf16"))[:, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(
            qr, kr, vr, scale=w.scale)[:, 0, :].numpy()
        assert np.max(np.abs(got[r] - ref)) <= 1e-12


# --------------------------------------------------------------------------- #
# closed forms
# --------------------------------------------------------------------------- #
def _rows_kv(w, kw, vw, r, kvh):
    kf = oracle.decode_storage(oracle.slot_view(kw, w.layout), w.dtype)
    vf = oracle.decode_storage(oracle.slot_view(vw, w.layout), w.dtype)
    n = int(w.context_lens[r])
    slots = [int(w.block_tables[r, t // w.block_size]) * w.block_size + t % w.block_size
             for t in range(n)]
    return kf[slots, kvh, :], vf[slots, kvh, :]


@pytest.mark.parametrize("layout", LAYOUTS)
def test_single_key_returns_its_value_exactly(layout):
    w = wl.make_custom([1, 1, 1], heads=4, head_dim=64, dtype="bf16", layout=layout, seed=3)
    k, v = wl.history_host(w)
    got, _, _ = run_oracle(w, k, v)
    assert np.array_equal(got, oracle.decode_storage(w.v_new, "bf16"))


def test_two_keys_logistic_weight():
    w = wl.make_custom([2, 2], heads=2, head_dim=16, dtype="f32", seed=5)
    k, v = wl.history_host(w)
    got, kw, vw = run_oracle(w, k, v)
    qf = oracle.decode_storage(w.q, "f32")
    for r in range(2):
        for h in range(2):
            kk, vv = _rows_kv(w, kw, vw, r, h)
            s0, s1 = w.scale * qf[r, h] @ kk[0], w.scale * qf[r, h] @ kk[1]
            want = scipy.special.expit(s0 - s1) * vv[0] + scipy.special.expit(s1 - s0) * vv[1]
            assert np.max(np.abs(got[r, h] - want)) <= 1e-13


@pytest.mark.parametrize("how", ["zero_scale", "zero_q", "equal_keys"])
def test_uniform_weights_give_plain_mean(how):
    w = wl.make_custom([37, 5, 16], heads=2, head_dim=16, dtype="f32", seed=8)
    k, v = wl.history_host(w)
    over = {}
    if how == "zero_scale":
        over["scale"] = 0.0
    elif how == "zero_q":
        over["q"] = np.zeros_like(w.q)
    else:
        k[...] = k[0, 0, 0, :]       # every slot gets the same key
        w.k_new[...] = k[0, 0, 0, :]
    got, kw, vw = run_oracle(w, k, v, **over)
    for r in range(w.rows):
        for h in range(w.heads):
            _, vv = _rows_kv(w, kw, vw, r, h)
            assert np.max(np.abs(got[r, h] - vv.mean(axis=0))) <= 1e-13


def test_dominant_key_selects_its_value():
    w = wl.make_custom([20], heads=1, head_dim=16, dtype="f32", seed=9)
    k, v = wl.history_host(w)
    qf = w.q[0, 0].astype(np.float64)
    blk = int(w.block_tables[0, 0])
    k[blk, 0, 3, :] = (1000.0 * qf).astype(np.float32)   # position 3 of the row
    got, _, vw = run_oracle(w, k, v)
    assert np.array_equal(got[0, 0], v[blk, 0, 3, :].astype(np.float64))


# --------------------------------------------------------------------------- #
# invariants
# --------------------------------------------------------------------------- #
def _case(layout="HND", dtype="f32", seed=21, lens=(37, 5, 0, 16, 48), heads=4, kvh=4):
    w = wl.make_custom(list(lens), heads=heads, kv_heads=kvh, head_dim=16, dtype=dtype,
                       layout=layout, seed=seed)
    k, v = wl.history_host(w)
    return w, k, v


def test_key_shift_invariance():
    w, k, v = _case()
    base, _, _ = run_oracle(w, k, v)
    c = np.linspace(-1, 1, w.head_dim, dtype=np.float32) * 0.25
    k2 = (k.astype(np.float64) + c).astype(np.float32)
    w.k_new = (w.k_new.astype(np.float64) + c).astype(np.float32)
    shifted, _, _ = run_oracle(w, k2, v)
    # The shift changes scores by the per-(row, head) constant scale*q.c only up to
    # float32 rounding of the shifted keys; tolerance covers that rounding.
    assert np.max(np.abs(shifted - base)) <= 1e-5


@pytest.mark.parametrize("a,b,tol", [(2.0, 0.0, 1e-12), (1.0, 1.0, 2e-6), (-0.5, 0.25, 2e-6)])
def test_value_affine_map(a, b, tol):
    """V -> aV + b maps out -> a out + b.  Scaling by a power of two is exact in
    float32 storage; a shift rounds each stored value by at most 2^-24 of its
    magnitude (|v| < 6 here), which bounds the tolerance."""
    w, k, v = _case()
    base, _, _ = run_oracle(w, k, v)
    w.v_new = (w.v_new.astype(np.float64) * a + b).astype(np.float32)
    mapped, _, _ = run_oracle(w, k, (v.astype(np.float64) * a + b).astype(np.float32))
    live = w.context_lens > 0
    assert np.max(np.abs(mapped[live] - (a * base[live] + b))) <= tol
    assert np.all(mapped[~live] == 0)


def test_row_permutation_permutes_outputs():
    w, k, v = _case()
    base, kw, vw = run_oracle(w, k, v)
    perm = np.array([3, 0, 4, 2, 1])
    out = oracle.paged_attention(w.q[perm], kw, vw, w.block_tables[perm],
                                 w.context_lens[perm], w.scale, num_blocks=w.num_blocks,
                                 block_size=w.block_size, layout=w.layout, dtype=w.dtype)
    assert np.max(np.abs(out - base[perm])) <= 1e-12


@pytest.mark.parametrize("layout", LAYOUTS)
def test_block_relabelling_is_invisible(layout):
    w, k, v = _case(layout=layout, dtype="bf16")
    base, kw, vw = run_oracle(w, k, v)
    rng = np.random.default_rng(4)
    pi = rng.permutation(w.num_blocks)               # physical block b moves to pi[b]
    k2, v2 = kw.copy(), vw.copy()
    k2[pi] = kw[:w.num_blocks]
    v2[pi] = vw[:w.num_blocks]
    bt = w.block_tables.copy()
    live = bt >= 0
    bt[live] = pi[bt[live]]
    out = oracle.paged_attention(w.q, k2, v2, bt, w.context_lens, w.scale,
                                 num_blocks=w.num_blocks, block_size=w.block_size,
                                 layout=layout, dtype=w.dtype)
    assert np.array_equal(out, base)


def test_heads_are_independent():
    w, k, v = _case()
    base, kw, vw = run_oracle(w, k, v)
    k2, v2 = kw.copy(), vw.copy()
    k2[:, 2] += 3.0          # HND: axis 1 is the KV head
    v2[:, 2] -= 1.0
    out = oracle.paged_attention(w.q, k2, v2, w.block_tables, w.context_lens, w.scale,
                                 num_blocks=w.num_blocks, block_size=w.block_size,
                                 layout=w.layout, dtype=w.dtype)
    keep = [0, 1, 3]
    assert np.array_equal(out[:, keep], base[:, keep])
    assert not np.allclose(out[:, 2][w.context_lens > 0], base[:, 2][w.context_lens > 0])


def test_stale_tail_and_unnamed_blocks_do_not_matter():
    w, k, v = _case()
    base, kw, vw = run_oracle(w, k, v)
    k2, v2 = kw.copy(), vw.copy()
    named = set(wl.live_blocks(w).tolist())
    for b in range(w.num_blocks + 1):
        if b not in named:
            k2[b] = 1e6
            v2[b] = -1e6
    for r in range(w.rows):
        n = int(w.context_lens[r])
        if n % w.block_size:
            blk = int(w.block_tables[r, n // w.block_size])
            k2[blk, :, n % w.block_size:, :] = 1e6      # HND: positions past the length
            v2[blk, :, n % w.block_size:, :] = -1e6
    # slot 0 is the rectangle's pad target; keep it unchanged so the gather stays finite
    k2[0], v2[0] = kw[0], vw[0]
    out = oracle.paged_attention(w.q, k2, v2, w.block_tables, w.context_lens, w.scale,
                                 num_blocks=w.num_blocks, block_size=w.block_size,
                                 layout=w.layout, dtype=w.dtype)
    assert np.array_equal(out, base)


def test_pad_rows_are_zero_and_ignore_their_tables():
    w, k, v = _case(lens=(0, 9, 0, 0))
    base, kw, vw = run_oracle(w, k, v)
    assert np.all(base[[0, 2, 3]] == 0)
    bt = w.block_tables.copy()
    bt[[0, 2, 3]] = -1
    out = oracle.paged_attention(w.q, kw, vw, bt, w.context_lens, w.scale,
                                 num_blocks=w.num_blocks, block_size=w.block_size,
                                 layout=w.layout, dtype=w.dtype)
    assert np.array_equal(out, base)


def test_all_padding_batch_is_all_zero():
    w, k, v = _case(lens=(0, 0, 0))
    out, kw, vw = run_oracle(w, k, v)
    assert np.all(out == 0)


def test_batch_composition_does_not_change_a_row():
    w, k, v = _case()
    base, kw, vw = run_oracle(w, k, v)
    for r in range(w.rows):
        one = oracle.paged_attention(w.q[r:r + 1], kw, vw, w.block_tables[r:r + 1],
                                     w.context_lens[r:r + 1], w.scale,
                                     num_blocks=w.num_blocks, block_size=w.block_size,
                                     layout=w.layout, dtype=w.dtype)
        assert np.max(np.abs(one[0] - base[r])) <= 1e-12


def test_nan_in_the_pad_target_poisons_the_rectangle():
    """The rectangle reads slot 0 for every cell past a row's length and masks the
    scores afterwards, so a NaN there reaches rows shorter than the batch width.
    This is the expected weakness of the reference read, not of the kernel."""
    for seed in range(64):           # a placement in which block 0 holds no live token
        w = wl.make_custom([37, 5, 16], heads=4, head_dim=16, dtype="f32",
                           num_blocks=24, seed=seed)
        if 0 not in set(wl.live_blocks(w).tolist()):
            break
    k, v = wl.history_host(w)
    base, kw, vw = run_oracle(w, k, v)
    vw[0, :, 0, :] = np.nan
    out = oracle.paged_attention(w.q, kw, vw, w.block_tables, w.context_lens, w.scale,
                                 num_blocks=w.num_blocks, block_size=w.block_size,
                                 layout=w.layout, dtype=w.dtype)
    short = w.context_lens < w.context_lens.max()
    assert np.all(np.isnan(out[short]))
    assert np.array_equal(out[~short], base[~short])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_layouts_agree(dtype):
    w, k, v = _case(layout="NHD", dtype=dtype)
    base, _, _ = run_oracle(w, k, v)
    w2, _, _ = _case(layout="HND", dtype=dtype)
    out, _, _ = run_oracle(w2, np.ascontiguousarray(k.transpose(0, 2, 1, 3)),
                           np.ascontiguousarray(v.transpose(0, 2, 1, 3)))
    assert np.array_equal(out, base)


# --------------------------------------------------------------------------- #
# the slot scatter
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_scatter_writes_exactly_the_named_slots(layout, dtype):
    w = wl.make_custom([0, 17, 0, 1, 32], heads=4, kv_heads=2, head_dim=16, dtype=dtype,
                       layout=layout, seed=17)
    k, v = wl.history_host(w)
    kw, vw = k.copy(), v.copy()
    oracle.kv_write(kw, vw, w.k_new, w.v_new, w.slot_mapping, num_blocks=w.num_blocks,
                    block_size=w.block_size, layout=layout, dtype=dtype)
    sink = w.num_blocks * w.block_size
    changed = set()
    for slot in range((w.num_blocks + 1) * w.block_size):
        b, o = divmod(slot, w.block_size)
        for h in range(w.kv_heads):
            if layout == "HND":
                a0, a1, b0, b1 = k[b, h, o], kw[b, h, o], v[b, h, o], vw[b, h, o]
            else:
                a0, a1, b0, b1 = k[b, o, h], kw[b, o, h], v[b, o, h], vw[b, o, h]
            if not (np.array_equal(a0, a1) and np.array_equal(b0, b1)):
                changed.add(slot)
    live_slots = {int(w.slot_mapping[r]) for r in w.live_rows}
    assert changed <= live_slots | {sink}
    assert live_slots <= changed
    for r in w.live_rows:
        b, o = divmod(int(w.slot_mapping[r]), w.block_size)
        got_k = kw[b, :, o] if layout == "HND" else kw[b, o]
        got_v = vw[b, :, o] if layout == "HND" else vw[b, o]
        assert np.array_equal(got_k, w.k_new[r]) and np.array_equal(got_v, w.v_new[r])
    # pad rows hit the sink; the last of them wins
    last_pad = int(w.pad_rows[-1])
    sink_k = kw[w.num_blocks, :, 0] if layout == "HND" else kw[w.num_blocks, 0]
    assert np.array_equal(sink_k, w.k_new[last_pad])


def test_every_write_slot_is_the_last_live_position():
    for idx in (1, 2, 3, 4):
        w = wl.make_config(idx)
        mapping, live = oracle.rebuild_mapping(w.block_tables, w.context_lens,
                                               w.block_size)
        for r in range(w.rows):
            n = int(w.context_lens[r])
            if n == 0:
                assert w.slot_mapping[r] == w.sink
            else:
                assert mapping[r, n - 1] == w.slot_mapping[r]

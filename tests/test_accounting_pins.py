"""The host accounting reproduces every number the pages print for the streamed
read's work and the score rectangle's size (fixtures under tests/golden/)."""

import csv
import os

import numpy as np
import pytest

from paged_attention_decode_kv_amd import accounting as acc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TILE = 128
HEADS = 32


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        lines = [ln for ln in f if not ln.startswith("#")]
    return list(csv.DictReader(lines))


def spread_lengths(rows, width, spread):
    """Length patterns behind the page's spread labels.  'uniform' and 'long tail'
    (one row in eight at full width, seven at width/8) reproduce every walk count;
    '2x' (full, half alternating) and '4x' (full, 1/2, 1/4, 1/8 repeating) are this
    build's reading of two labels the page does not define."""
    if spread == "uniform":
        pat = [width]
    elif spread == "2x":
        pat = [width, width // 2]
    elif spread == "4x":
        pat = [width, width // 2, width // 4, width // 8]
    elif spread == "long tail":
        pat = [width] + [width // 8] * 7
    else:
        raise ValueError(spread)
    return np.array([pat[i % len(pat)] for i in range(rows)])


def _round_like(x, printed):
    decimals = len(printed.split(".")[1]) if "." in printed else 0
    return round(x, decimals)


@pytest.mark.parametrize("row", _rows("day59_streambench.csv"),
                         ids=lambda r: f"{r['rows']}x{r['width']}-{r['spread']}")
def test_streambench_table(row):
    rows, width = int(row["rows"]), int(row["width"])
    lens = spread_lengths(rows, width, row["spread"])
    assert acc.tiles_walked(lens, TILE) == int(row["walked"])
    assert acc.rectangle_tiles(rows, width, TILE) == int(row["rect_tiles"])
    ratio = acc.walk_ratio(lens, width, TILE)
    assert _round_like(ratio, row["walks"]) == float(row["walks"])
    rect = acc.rectangle_bytes(rows, HEADS, width) / acc.MB
    tile = acc.tile_bytes(rows, HEADS, TILE) / acc.MB
    assert _round_like(rect, row["rect_mb"]) == float(row["rect_mb"])
    assert _round_like(tile, row["tile_mb"]) == float(row["tile_mb"])
    assert acc.rectangle_bytes(rows, HEADS, width) // acc.tile_bytes(rows, HEADS, TILE) \
        == int(row["holds"])


def test_long_tail_example():
    (row,) = _rows("day59_long_tail_example.csv")
    lens = np.array([2048] + [256] * 7)
    walked = acc.tiles_walked(lens, TILE)
    rect = acc.rectangle_tiles(8, 2048, TILE)
    assert (rect, rect - walked, walked) == (int(row["rect_tiles"]),
                                             int(row["padding_tiles"]), int(row["walked"]))


@pytest.mark.parametrize("row", _rows("day55_pool_budget.csv"), ids=lambda r: r["budget_bytes"])
def test_pool_budget_table(row):
    assert acc.widest_capture(float(row["budget_bytes"]), 256, HEADS) == int(row["widest_tokens"])


def test_algorithmic_bytes_components():
    lens = np.array([16, 40, 0])
    b = acc.algorithmic_bytes(lens, heads=4, kv_heads=2, head_dim=64, block_size=16,
                              elem=2, write_tokens=3)
    assert b["kv"] == 56 * 2 * 64 * 2 * 2
    assert b["q_out"] == 2 * 3 * 4 * 64 * 2
    assert b["tables"] == (1 + 3 + 0) * 4 + 3 * 4
    assert b["kv_write"] == 2 * 3 * 2 * 64 * 2 * 2
    assert b["total"] == b["kv"] + b["q_out"] + b["tables"] + b["kv_write"]
    assert acc.row_heads(lens, 4) == 8


def test_slot_addressing_bytes():
    """One int64 cell per live position instead of one int32 id per live block: at
    block size 16 the rectangle holds 16x the cells (Day 51, "Why it matters"), 32x the
    bytes."""
    lens = np.array([16, 48, 0, 160])
    kw = dict(heads=4, kv_heads=2, head_dim=64, block_size=16, elem=2, write_tokens=4)
    blocks = acc.algorithmic_bytes(lens, **kw)
    slots = acc.algorithmic_bytes(lens, address="slots", **kw)
    assert slots["tables"] == (16 + 48 + 160) * 8 + 4 * 4
    assert (slots["tables"] - 16) == 32 * (blocks["tables"] - 16)
    assert slots["kv"] == blocks["kv"] and slots["kv_write"] == blocks["kv_write"]
    with pytest.raises(ValueError):
        acc.algorithmic_bytes(lens, address="rows", **kw)


def test_multi_token_bytes():
    lens = np.array([16, 48, 0])
    kw = dict(heads=4, kv_heads=2, head_dim=64, block_size=16, elem=2)
    one = acc.algorithmic_bytes(lens, write_tokens=3, **kw)
    four = acc.algorithmic_bytes(lens, write_tokens=12, query_len=4, **kw)
    assert four["kv"] == one["kv"] and four["tables"] == one["tables"]
    assert four["q_out"] == 4 * one["q_out"]
    assert four["kv_write"] == 4 * one["kv_write"]

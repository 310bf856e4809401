"""Host logic of bench.py (no GPU): the one-GPU refusal, the flags, and the lookup of
the committed HBM-traffic records that fill the roofline's ``traffic`` field."""
import importlib.util
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def _bench_module():
    spec = importlib.util.spec_from_file_location("bench_under_test", BENCH)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)       # top level imports the standard library only
    return mod


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, BENCH, *args], capture_output=True, text=True,
                          env=env, timeout=120)


@pytest.mark.parametrize("args,env", [(["--gpus", "2"], None), (["--gpus", "8"], None),
                                      ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(args, env):
    r = _run(args, env)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""                # no JSON line for a run that did not happen


def test_help_lists_the_flags():
    r = _run(["--help"])
    assert r.returncode == 0
    for flag in ("--steps", "--warmup", "--config", "--kv-heads", "--query-len", "--address",
                 "--launch", "--solo-tokens", "--no-cpu-baseline", "--copy-calibration"):
        assert flag in r.stdout


def test_traffic_is_reported_only_for_the_current_kernel_source(tmp_path):
    b = _bench_module()
    src = b.kernel_source_hash()
    recs = {"records": [
        {"workload": "full-width", "layout": "HND", "kernel_source_sha256": "0" * 64,
         "bytes_per_launch": 111},
        {"workload": "full-width", "layout": "NHD", "kernel_source_sha256": src,
         "bytes_per_launch": 222},
        {"workload": "full-width", "layout": "HND", "kernel_source_sha256": src,
         "bytes_per_launch": 333},
    ]}
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(recs))
    b.TRAFFIC_FILE = str(path)
    assert b.traffic_per_launch("full-width", "HND") == 333
    assert b.traffic_per_launch("full-width", "NHD") == 222
    assert b.traffic_per_launch("ragged", "HND") is None
    recs["records"] = recs["records"][:1]          # only a stale record left
    path.write_text(json.dumps(recs))
    assert b.traffic_per_launch("full-width", "HND") is None
    path.write_text("not json")
    assert b.traffic_per_launch("full-width", "HND") is None
    b.TRAFFIC_FILE = str(tmp_path / "missing.json")
    assert b.traffic_per_launch("full-width", "HND") is None


def test_committed_traffic_records_are_consistent():
    """Every committed record taken on the current kernel source: fetch + write bytes
    make its per-launch figure, within a few percent of the algorithmic bytes (the
    excess is split partials) for launches of at least 100 MB (a launch of a few hundred
    KB reads mostly its fixed bytes: arguments, counters, work list), from counters
    scaled by a 1 GiB copy's readings."""
    b = _bench_module()
    with open(b.TRAFFIC_FILE) as f:
        records = json.load(f)["records"]
    src = b.kernel_source_hash()
    current = [r for r in records if r["kernel_source_sha256"] == src]
    assert current, "no traffic record for the current kernel source"
    for r in current:
        assert r["bytes_per_launch"] == r["fetch_bytes"] + r["write_bytes"]
        if r["algorithmic_bytes_per_launch"] >= 100e6:
            assert 0.99 < r["traffic_over_algorithmic"] < 1.05, r["tag"]
        cal = r["calibration"]
        assert abs(cal["fetch_scale"] * cal["fetch_kib"] - 1048576) < 1024
        assert abs(cal["write_scale"] * cal["write_kib"] - 1048576) < 1024
        assert all("rocprofv3 --pmc" in c and "bench.py" in c for c in r["commands"])


@pytest.mark.parametrize("layout", ["HND", "NHD"])
def test_gather_pieces_are_the_pieces_the_read_streams(layout):
    """The reference read's piece list (gather_offsets) holds each piece the decode reads
    exactly once and nothing else: for an HND pool every (live block, KV head) piece, for
    an NHD pool every live (position, KV head) token vector, and for rows read token by
    token every (listed slot, KV head) token vector; all inside the pool."""
    import numpy as np

    from paged_attention_decode_kv_amd import workloads as wl

    bench = _bench_module()
    w = wl.make_custom([37, 0, 16, 100, 1], heads=8, kv_heads=2, head_dim=64, block_size=16,
                       dtype="bf16", layout=layout, seed=5)
    vec = w.head_dim * 2
    pool_bytes = int(np.prod(w.pool_shape)) * 2

    def token_bytes(slot, h):       # from the pool shape, independently of the bench
        blk, off = divmod(int(slot), w.block_size)
        idx = (blk, h, off) if layout == "HND" else (blk, off, h)
        return int(np.ravel_multi_index(idx, w.pool_shape[:3])) * vec

    offs, piece = bench.gather_offsets(w)
    want = []
    for r in range(w.rows):
        n = int(w.context_lens[r])
        for t in range(n):
            slot = int(w.block_tables[r, t // w.block_size]) * w.block_size + t % w.block_size
            for h in range(w.kv_heads):
                if layout == "NHD":
                    want.append(token_bytes(slot, h))
                elif t % w.block_size == 0:          # a whole (block, KV head) piece
                    want.append(token_bytes(slot, h))
    assert piece == (w.block_size * vec if layout == "HND" else vec)
    assert sorted(offs.tolist()) == sorted(want)
    assert offs.min() >= 0 and offs.max() + piece <= pool_bytes

    rng = np.random.default_rng(1)
    slot_rows = {3: rng.permutation(np.arange(40, 140)), 0: np.array([5, 200, 17])}
    offs, piece = bench.gather_offsets(w, slot_rows=slot_rows)
    want = [token_bytes(s, h) for r in slot_rows for h in range(w.kv_heads)
            for s in slot_rows[r]]
    assert piece == vec
    assert offs.tolist() == want                      # row by row, head by head, in order
    assert bench.gather_offsets(w, rows=[1]) is None  # a padding row reads nothing

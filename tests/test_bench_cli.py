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

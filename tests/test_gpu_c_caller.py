"""One decode step driven by a plain C program (tests/c_abi_step.c) through the C ABI,
with device memory from the HIP C runtime and no Python in the process: its pools after
the scatter equal the oracle's bit for bit, and its outputs equal the oracle's to the
parity tolerances (2e-6 for float32; 2e-2 and 2^-8 relative + 2e-5 for bfloat16)."""

import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
from paged_attention_decode_kv_amd import _capi
from paged_attention_decode_kv_amd import workloads as wl

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DTYPE_CODE = {"f32": 0, "bf16": 1}
LAYOUT_CODE = {"HND": 0, "NHD": 1}


def say(msg):
    print(f"[gpu-test] {msg}", flush=True)


@pytest.fixture(scope="module")
def program(tmp_path_factory):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    exe = str(tmp_path_factory.mktemp("cabi") / "c_abi_step")
    libdir = os.path.dirname(_capi.LIB_PATH)
    build = subprocess.run(
        [gcc, "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror",
         "-D__HIP_PLATFORM_AMD__", "-isystem", "/opt/rocm/include",
         "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c_abi_step.c"),
         "-o", exe, "-L", libdir, "-lpagedkv", "-L", "/opt/rocm/lib", "-lamdhip64",
         f"-Wl,-rpath,{libdir}", "-Wl,-rpath,/opt/rocm/lib"],
        capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    return exe


CASES = [
    dict(lens=[17, 0, 300, 64, 1], heads=8, kv_heads=2, head_dim=128, dtype="bf16",
         layout="HND", seed=11),
    dict(lens=[5, 33, 129], heads=4, kv_heads=4, head_dim=64, dtype="f32", layout="NHD",
         seed=12),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c['dtype']}-{c['layout']}-h{c['heads']}/{c['kv_heads']}")
def test_a_c_program_runs_one_step_through_the_abi(program, case, tmp_path):
    w = wl.make_custom(case["lens"], heads=case["heads"], kv_heads=case["kv_heads"],
                       head_dim=case["head_dim"], dtype=case["dtype"], layout=case["layout"],
                       seed=case["seed"], name="c-caller")
    say(f"c caller: {case}")
    k_host, v_host = wl.history_host(w)
    d = str(tmp_path)
    with open(os.path.join(d, "shape.txt"), "w") as f:
        f.write(f"{w.num_blocks} {w.block_size} {w.kv_heads} {w.head_dim} "
                f"{DTYPE_CODE[w.dtype]} {LAYOUT_CODE[w.layout]} {w.rows} {w.heads} "
                f"{w.max_blocks} {len(w.slot_mapping)}\n")
    files = {"scale.bin": np.float32(w.scale), "k_pool.bin": k_host, "v_pool.bin": v_host,
             "q.bin": w.q, "k_new.bin": w.k_new, "v_new.bin": w.v_new,
             "slots.bin": w.slot_mapping.astype(np.int64),
             "tables.bin": w.block_tables.astype(np.int32),
             "lens.bin": w.context_lens.astype(np.int32)}
    for name, arr in files.items():
        with open(os.path.join(d, name), "wb") as f:
            f.write(np.ascontiguousarray(arr).tobytes())
    run = subprocess.run([program, d], capture_output=True, text=True, timeout=120)
    say(run.stdout.strip())
    assert run.returncode == 0, run.stdout + run.stderr

    store = k_host.dtype
    got_out = np.fromfile(os.path.join(d, "out.bin"), dtype=store).reshape(w.q.shape)
    got_k = np.fromfile(os.path.join(d, "k_pool_out.bin"), dtype=store).reshape(k_host.shape)
    got_v = np.fromfile(os.path.join(d, "v_pool_out.bin"), dtype=store).reshape(v_host.shape)

    kw, vw = k_host.copy(), v_host.copy()
    oracle.kv_write(kw, vw, w.k_new, w.v_new, w.slot_mapping, num_blocks=w.num_blocks,
                    block_size=w.block_size, layout=w.layout, dtype=w.dtype)
    assert np.array_equal(got_k.view(np.uint8), kw.view(np.uint8))
    assert np.array_equal(got_v.view(np.uint8), vw.view(np.uint8))
    ref = oracle.paged_attention(w.q, kw, vw, w.block_tables, w.context_lens, w.scale,
                                 num_blocks=w.num_blocks, block_size=w.block_size,
                                 layout=w.layout, dtype=w.dtype)
    g = oracle.decode_storage(got_out, w.dtype)
    err = np.abs(g - ref)
    if w.dtype == "f32":
        assert err.max() <= 2e-6, err.max()
    else:
        assert err.max() <= 2e-2, err.max()
        assert np.all(err <= 2.0 ** -8 * np.abs(ref) + 2e-5)
    pad = np.asarray(w.context_lens) == 0
    assert np.all(g[pad] == 0)

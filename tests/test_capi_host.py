"""The C-ABI library loads without a GPU, exports every declared symbol, and its host
validator refuses exactly what the oracle refuses (no kernel is launched here)."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from paged_attention_decode_kv_amd import _capi, binding
from paged_attention_decode_kv_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pagedkv.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_capi.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return _capi.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 10
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(_capi.SIGNATURES), "binding and header disagree"


def test_abi_and_status_strings(lib):
    assert lib.pkv_abi_version() == 4
    for code, name in enumerate(_capi.STATUS_NAMES):
        assert lib.pkv_status_str(code).decode() == name


def test_descriptor_arithmetic(lib):
    d = binding.host_desc(131072, 16, 32, 128)
    assert lib.pkv_sink_slot(ctypes.byref(d)) == 131072 * 16
    assert lib.pkv_pool_elements(ctypes.byref(d)) == 131073 * 16 * 32 * 128
    assert lib.pkv_check_pool(ctypes.byref(d)) == 0
    for bad, code in ((binding.host_desc(8, 16, 4, 64, dtype="f16"), "DTYPE"),
                      (binding.host_desc(0, 16, 4, 64), "SHAPE"),
                      (binding.host_desc(8, 16, 4, 64, layout="XYZ"), "SHAPE"),
                      (binding.host_desc(8, 12, 4, 64), "UNSUPPORTED"),
                      (binding.host_desc(8, 16, 4, 96), "UNSUPPORTED")):
        assert _capi.STATUS_NAMES[lib.pkv_check_pool(ctypes.byref(bad))] == code
        assert lib.pkv_sink_slot(ctypes.byref(bad)) == -1


def test_workspace_size_depends_on_shape_only(lib):
    d = binding.host_desc(131072, 16, 32, 128)
    small = lib.pkv_workspace_bytes(ctypes.byref(d), 8, 32, 128)
    big = lib.pkv_workspace_bytes(ctypes.byref(d), 256, 32, 512)
    assert 0 < small < big
    assert lib.pkv_workspace_bytes(ctypes.byref(d), 0, 32, 128) == 0


def _align(x, a=256):
    return (x + a - 1) // a * a


def _expected_workspace(rows, vectors, head_dim, max_blocks, block_size, cmin, cmax):
    """The documented layout: counters, work list, four row arrays, split-row records
    (at most 16 MiB between the shortest and longest chunk's needs)."""
    width = max_blocks * block_size
    mc_min, mc_max = -(-width // cmin), -(-width // cmax)
    at_min = rows * mc_min if mc_min > 1 else 0
    at_max = rows * mc_max if mc_max > 1 else 0
    budget = (16 << 20) // ((head_dim + 4) * 4 * vectors)
    recs = min(at_min, max(at_max, budget))
    return (256 + _align(rows * max(mc_min, 1) * 16) + 3 * _align(rows * 4) +
            _align(rows * 16) + _align(recs * vectors * (head_dim + 4) * 4))


@pytest.mark.parametrize("rows,heads,d,mb,bs,qlen", [
    (256, 32, 128, 512, 16, 1),    # the full-width batch: ~17 MB, not 138 MB
    (8, 32, 128, 128, 16, 1),      # small: every row may split into the shortest chunks
    (34, 32, 128, 512, 16, 1),
    (4, 8, 64, 8, 16, 1),          # a table narrower than the shortest chunk: no records
    (64, 16, 256, 4096, 16, 4),    # multi-token
])
def test_workspace_layout_and_record_budget(lib, rows, heads, d, mb, bs, qlen):
    desc = binding.host_desc(1 << 20, bs, heads, d)
    binding.set_tuning(chunk_min=128, chunk_max=8192)
    got = lib.pkv_workspace_bytes_multi(ctypes.byref(desc), rows, qlen, heads, mb)
    assert got == _expected_workspace(rows, qlen * heads, d, mb, bs, 128, 8192)
    if (rows, mb) == (256, 512):
        assert got < 20 << 20
    # pinning the chunk leaves the plan no room: every row's chunks get records
    binding.set_tuning(chunk_min=256, chunk_max=256)
    try:
        pinned = lib.pkv_workspace_bytes_multi(ctypes.byref(desc), rows, qlen, heads, mb)
        assert pinned == _expected_workspace(rows, qlen * heads, d, mb, bs, 256, 256)
    finally:
        binding.set_tuning(chunk_min=128, chunk_max=8192)


def test_tuning_reads_are_one_snapshot_under_concurrent_sets(lib):
    """A thread flips the chunk range between two settings while this one sizes
    workspaces and reads the tuning: every read sees one setting or the other, never
    one field of each (the pair (32, 8192) would even be an illegal range)."""
    import threading
    desc = binding.host_desc(131072, 16, 32, 128)
    a, b = (128, 8192), (32, 2048)
    sizes = set()
    for lo, hi in (a, b):
        binding.set_tuning(chunk_min=lo, chunk_max=hi)
        sizes.add(lib.pkv_workspace_bytes(ctypes.byref(desc), 256, 32, 512))
    assert len(sizes) == 2
    stop = threading.Event()

    def flip():
        t = [_capi.Tuning(*a, 0, 0, 0, 0, 0, 0, 0, 0), _capi.Tuning(*b, 0, 0, 0, 0, 0, 0, 0, 0)]
        i = 0
        while not stop.is_set():
            assert lib.pkv_set_tuning(ctypes.byref(t[i & 1])) == 0
            i += 1

    th = threading.Thread(target=flip)
    th.start()
    try:
        seen = set()
        for _ in range(20000):
            sz = lib.pkv_workspace_bytes(ctypes.byref(desc), 256, 32, 512)
            assert sz in sizes, sz
            tu = _capi.Tuning()
            assert lib.pkv_get_tuning(ctypes.byref(tu)) == 0
            assert (tu.chunk_min, tu.chunk_max) in (a, b), (tu.chunk_min, tu.chunk_max)
            seen.add(sz)
    finally:
        stop.set()
        th.join()
        binding.set_tuning(chunk_min=128, chunk_max=8192)


def test_error_detail_is_per_thread(lib):
    """Two threads make refused host checks with different bad entries at the same time;
    each reads back the detail naming its own entry."""
    import threading
    w, _ = _attention_cases()
    d = binding.host_desc(w.num_blocks, w.block_size, w.kv_heads, w.head_dim, w.dtype,
                          w.layout)
    errors = []

    def worker(row, n):
        ctx = w.context_lens.copy()
        ctx[row] = -1 - row
        bt = np.ascontiguousarray(w.block_tables, dtype=np.int32)
        for _ in range(n):
            st = lib.pkv_check_attention_host(
                ctypes.byref(d), bt.ctypes.data_as(ctypes.c_void_p), bt.shape[1],
                ctx.ctypes.data_as(ctypes.c_void_p), ctx.shape[0], w.heads)
            detail = lib.pkv_last_error_detail().decode()
            if _capi.STATUS_NAMES[st] != "CONTEXT_BOUNDS" or \
                    f"context_lens[{row}] = {-1 - row}" not in detail:
                errors.append((row, st, detail))
                return

    threads = [threading.Thread(target=worker, args=(r, 5000)) for r in (0, 3)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors[:3]


def _oracle_code(fn):
    try:
        fn()
    except oracle.Refusal as e:
        return e.code
    return "OK"


def _attention_cases():
    w = wl.make_custom([16, 40, 0, 7], heads=4, kv_heads=2, head_dim=64, num_blocks=12,
                       max_blocks=4, seed=5)
    cases = [("legal", w.block_tables, w.context_lens)]
    ctx = w.context_lens.copy(); ctx[1] = -3
    cases.append(("negative length", w.block_tables, ctx))
    ctx = w.context_lens.copy(); ctx[3] = 4 * 16 + 1
    cases.append(("past the table", w.block_tables, ctx))
    bt = w.block_tables.copy(); bt[1, 2] = -1
    cases.append(("-1 inside the live prefix", bt, w.context_lens))
    bt = w.block_tables.copy(); bt[3, 0] = w.num_blocks
    cases.append(("sink block named", bt, w.context_lens))
    bt = w.block_tables.copy(); bt[0, 1:] = -1; bt[2, :] = 99
    cases.append(("junk past the live prefix", bt, w.context_lens))
    ctx = np.zeros_like(w.context_lens)
    cases.append(("all padding", np.full_like(w.block_tables, -1), ctx))
    ctx = w.context_lens.copy(); ctx[0] = 64
    bt = w.block_tables.copy(); bt[0] = [0, 1, 2, 3]
    cases.append(("length fills the table", bt, ctx))
    return w, cases


@pytest.mark.parametrize("idx", range(8))
def test_attention_refusals_match_the_oracle(lib, idx):
    w, cases = _attention_cases()
    name, bt, ctx = cases[idx]
    k, v = wl.history_host(w)
    want = _oracle_code(lambda: oracle.validate_attention(
        w.q, k, v, bt, ctx, num_blocks=w.num_blocks, block_size=w.block_size,
        layout=w.layout, dtype=w.dtype))
    d = binding.host_desc(w.num_blocks, w.block_size, w.kv_heads, w.head_dim, w.dtype,
                          w.layout)
    assert binding.check_attention_host(d, bt, ctx, w.heads) == want, name


def test_empty_and_shape_refusals_match_the_oracle(lib):
    w, _ = _attention_cases()
    d = binding.host_desc(w.num_blocks, w.block_size, w.kv_heads, w.head_dim, w.dtype,
                          w.layout)
    k, v = wl.history_host(w)
    want = _oracle_code(lambda: oracle.validate_attention(
        w.q[:0], k, v, w.block_tables[:0], w.context_lens[:0], num_blocks=w.num_blocks,
        block_size=w.block_size, layout=w.layout, dtype=w.dtype))
    assert binding.check_attention_host(d, w.block_tables[:0], w.context_lens[:0],
                                        w.heads) == want == "EMPTY"
    want = _oracle_code(lambda: oracle.validate_attention(
        w.q[:, :3], k, v, w.block_tables, w.context_lens, num_blocks=w.num_blocks,
        block_size=w.block_size, layout=w.layout, dtype=w.dtype))
    assert binding.check_attention_host(d, w.block_tables, w.context_lens, 3) == want == "SHAPE"


@pytest.mark.parametrize("slots", [[0, 5, 8 * 16], [8 * 16, 8 * 16], [8 * 16 + 1, 3],
                                   [2, -1], [127, 128, 129]])
def test_write_refusals_match_the_oracle(lib, slots):
    w = wl.make_custom([3] * len(slots), heads=2, head_dim=64, num_blocks=8, seed=1)
    k, v = wl.history_host(w)
    sm = np.array(slots, dtype=np.int64)
    want = _oracle_code(lambda: oracle.validate_write(
        k, v, w.k_new, w.v_new, sm, num_blocks=8, block_size=16, layout="HND", dtype="f32"))
    d = binding.host_desc(8, 16, w.kv_heads, w.head_dim, "f32", "HND")
    assert binding.check_write_host(d, sm) == want


def test_empty_write_is_refused(lib):
    d = binding.host_desc(8, 16, 2, 64, "f32", "HND")
    assert binding.check_write_host(d, np.zeros(0, dtype=np.int64)) == "EMPTY"


def test_graph_capture_refusals_need_no_gpu(lib):
    """pkv_graph_capture makes the shape refusals of the two calls before touching HIP."""
    desc = binding.host_desc(64, 16, 4, 128, "bf16", "HND")
    handle = ctypes.c_void_p(123)
    p = ctypes.c_void_p(16)         # never dereferenced: every case below is refused first

    def cap(rows, heads, ws_bytes, max_blocks=8, d=desc, out=ctypes.byref(handle)):
        return _capi.STATUS_NAMES[lib.pkv_graph_capture(
            ctypes.byref(d), p, p, p, p, p, p, p, p, max_blocks, p, rows, heads, 1.0, p,
            ws_bytes, out)]

    need = lib.pkv_workspace_bytes(ctypes.byref(desc), 4, 8, 8)
    assert cap(0, 8, need) == "EMPTY"
    assert handle.value is None          # cleared on refusal
    assert cap(4, 6, need) == "SHAPE"    # 6 query heads over 4 KV heads
    assert cap(4, 8, need, max_blocks=0) == "SHAPE"
    assert cap(4, 8, need - 1) == "WORKSPACE"
    bad = binding.host_desc(64, 16, 4, 96, "bf16", "HND")
    assert cap(4, 8, need, d=bad) == "UNSUPPORTED"
    assert cap(4, 8, need, out=None) == "NULL"
    assert _capi.STATUS_NAMES[lib.pkv_graph_launch(None, None)] == "NULL"
    assert _capi.STATUS_NAMES[lib.pkv_graph_destroy(None)] == "OK"


def test_reference_read_refusals_need_no_gpu(lib):
    """pkv_stream_read and pkv_gather_read refuse bad sizes and shapes before launching."""
    p = ctypes.c_void_p(16)         # never dereferenced: every case below is refused first

    def gather(n=4, piece=4096, gpc=1, waves=4, ppw=2, ptr=p):
        return _capi.STATUS_NAMES[lib.pkv_gather_read(ptr, p, p, n, piece, p, gpc, waves, ppw,
                                                      None)]

    def stream(nbytes=4096, gpc=1, ptr=p):
        return _capi.STATUS_NAMES[lib.pkv_stream_read(ptr, nbytes, p, gpc, None)]

    assert gather(ptr=None) == "NULL"
    assert gather(n=0) == "SHAPE"
    assert gather(piece=8) == "SHAPE"
    assert gather(piece=4100) == "SHAPE"
    assert gather(piece=(1 << 20) + 16) == "SHAPE"
    assert gather(gpc=0) == "SHAPE" and gather(gpc=17) == "SHAPE"
    for waves, ppw, field in ((2, 2, "waves_per_group 2"), (16, 1, "waves_per_group 16"),
                              (4, 3, "pieces_per_wave 3"), (8, 8, "pieces_per_wave 8"),
                              (4, 0, "pieces_per_wave 0")):
        assert gather(waves=waves, ppw=ppw) == "SHAPE"
        assert field in lib.pkv_last_error_detail().decode()
    assert stream(ptr=None) == "NULL"
    assert stream(nbytes=0) == "SHAPE" and stream(nbytes=24) == "SHAPE"
    assert stream(gpc=0) == "SHAPE" and stream(gpc=17) == "SHAPE"
    assert len(binding.GATHER_SHAPES) == 6


def test_a_c99_program_includes_the_header_and_links_the_library(lib, tmp_path):
    """The boundary is plain C: tests/c_abi_consumer.c compiles as C99 with -pedantic
    -Werror against include/pagedkv.h, links libpagedkv.so, and its host-only calls
    return what the header states."""
    import shutil
    import subprocess

    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    src = os.path.join(ROOT, "tests", "c_abi_consumer.c")
    exe = str(tmp_path / "c_abi_consumer")
    libdir = os.path.dirname(_capi.LIB_PATH)
    build = subprocess.run(
        [gcc, "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror", "-I",
         os.path.join(ROOT, "include"), src, "-o", exe, "-L", libdir, "-lpagedkv",
         f"-Wl,-rpath,{libdir}"], capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "0 failure(s)" in run.stdout


def test_row_buckets():
    from paged_attention_decode_kv_amd.graphs import bucket_for, default_buckets
    assert default_buckets(1) == [1]
    assert default_buckets(256) == [1, 2, 4, 8, 16, 32, 64, 128, 256]
    assert default_buckets(24) == [1, 2, 4, 8, 16, 24]
    b = [4, 8, 16]
    assert [bucket_for(b, n) for n in (1, 4, 5, 8, 9, 16)] == [4, 4, 8, 8, 16, 16]
    with pytest.raises(binding.PagedKVError, match="SHAPE"):
        bucket_for(b, 17)
    with pytest.raises(binding.PagedKVError, match="EMPTY"):
        bucket_for(b, 0)


def _slot_cases():
    w = wl.make_custom([16, 40, 0, 7], heads=4, kv_heads=2, head_dim=64, num_blocks=12,
                       max_blocks=4, seed=5)
    sink = w.num_blocks * w.block_size
    table = np.full((w.rows, 64), -7, dtype=np.int64)
    for r in range(w.rows):
        for t in range(int(w.context_lens[r])):
            table[r, t] = int(w.block_tables[r, t // 16]) * 16 + t % 16
    rect = table[:, :48]                            # a window on a wider table
    cases = [("legal window", rect, w.context_lens)]
    ctx = w.context_lens.copy(); ctx[1] = -3
    cases.append(("negative length", rect, ctx))
    ctx = w.context_lens.copy(); ctx[3] = 49
    cases.append(("past the window", rect, ctx))
    ctx = w.context_lens.copy(); ctx[3] = 48
    cases.append(("length fills the window", rect, ctx))
    for bad in (-1, sink, sink + 5):
        r2 = table.copy()[:, :48]
        r2[1, 39] = bad
        cases.append((f"live cell {bad}", r2, w.context_lens))
    r2 = table.copy()[:, :48]
    r2[1, 40:] = sink + 99
    r2[2, :] = -1
    cases.append(("junk past the length", r2, w.context_lens))
    r2 = table.copy()[:, :48]
    r2[0, 0] = -1
    ctx = w.context_lens.copy(); ctx[3] = 49
    cases.append(("bounds before slots", r2, ctx))
    cases.append(("zero width", table[:, :0], np.zeros_like(w.context_lens)))
    assert len(cases) == 10
    return w, cases


@pytest.mark.parametrize("idx", range(10))
def test_slot_refusals_match_the_oracle(lib, idx):
    w, cases = _slot_cases()
    name, rect, ctx = cases[idx]
    k, v = wl.history_host(w)
    want = _oracle_code(lambda: oracle.validate_attention_slots(
        w.q, k, v, rect, ctx, num_blocks=w.num_blocks, block_size=w.block_size,
        layout=w.layout, dtype=w.dtype))
    d = binding.host_desc(w.num_blocks, w.block_size, w.kv_heads, w.head_dim, w.dtype,
                          w.layout)
    assert binding.check_attention_slots_host(d, rect, ctx, w.heads) == want, name


def test_slot_shape_refusals(lib):
    w, cases = _slot_cases()
    rect, ctx = cases[0][1], cases[0][2]
    d = binding.host_desc(w.num_blocks, w.block_size, w.kv_heads, w.head_dim, w.dtype,
                          w.layout)
    assert binding.check_attention_slots_host(d, rect[:0], ctx[:0], w.heads) == "EMPTY"
    assert binding.check_attention_slots_host(d, rect, ctx, 3) == "SHAPE"
    p = ctypes.c_void_p(16)
    # a row stride shorter than the width
    assert _capi.STATUS_NAMES[lib.pkv_check_attention_slots_host(
        ctypes.byref(d), p, 48, 47, p, 4, 4)] == "SHAPE"
    assert _capi.STATUS_NAMES[lib.pkv_check_attention_slots_host(
        ctypes.byref(d), p, (1 << 24) + 1, (1 << 24) + 1, p, 4, 4)] == "UNSUPPORTED"
    assert lib.pkv_workspace_bytes_slots(ctypes.byref(d), 4, 4, 0) == 0
    assert lib.pkv_workspace_bytes_slots(ctypes.byref(d), 4, 4, 48) > \
        lib.pkv_workspace_bytes(ctypes.byref(d), 4, 4, 3)


def _multi_cases():
    w = wl.make_custom([16, 40, 0, 7], heads=4, kv_heads=2, head_dim=64, num_blocks=12,
                       max_blocks=4, seed=5, query_len=4)
    cases = [("legal", w.block_tables, w.context_lens)]
    ctx = w.context_lens.copy(); ctx[3] = 3
    cases.append(("live row shorter than its queries", w.block_tables, ctx))
    ctx = w.context_lens.copy(); ctx[3] = 4
    cases.append(("exactly its queries", w.block_tables, ctx))
    ctx = w.context_lens.copy(); ctx[1] = 65
    cases.append(("past the table", w.block_tables, ctx))
    bt = w.block_tables.copy(); bt[1, 2] = -1
    cases.append(("-1 inside the live prefix", bt, w.context_lens))
    ctx = w.context_lens.copy(); ctx[3] = 2
    cases.append(("short row before a bad block", bt, ctx))
    ctx = w.context_lens.copy(); ctx[3] = 2; ctx[0] = -1
    cases.append(("range before short", w.block_tables, ctx))
    return w, cases


@pytest.mark.parametrize("idx", range(7))
def test_multi_refusals_match_the_oracle(lib, idx):
    w, cases = _multi_cases()
    name, bt, ctx = cases[idx]
    k, v = wl.history_host(w)
    want = _oracle_code(lambda: oracle.validate_attention_multi(
        w.q, k, v, bt, ctx, num_blocks=w.num_blocks, block_size=w.block_size,
        layout=w.layout, dtype=w.dtype))
    d = binding.host_desc(w.num_blocks, w.block_size, w.kv_heads, w.head_dim, w.dtype,
                          w.layout)
    assert binding.check_attention_multi_host(d, bt, ctx, 4, w.heads) == want, name


def test_multi_query_len_limits(lib):
    w, cases = _multi_cases()
    d = binding.host_desc(w.num_blocks, w.block_size, w.kv_heads, w.head_dim, w.dtype,
                          w.layout)
    bt, ctx = cases[0][1], cases[0][2]
    assert binding.check_attention_multi_host(d, bt, ctx, 0, w.heads) == "SHAPE"
    assert binding.check_attention_multi_host(d, bt, ctx, 65, w.heads) == "UNSUPPORTED"
    assert binding.check_attention_multi_host(d, bt[:0], ctx[:0], 4, w.heads) == "EMPTY"
    one = lib.pkv_workspace_bytes(ctypes.byref(d), 4, 4, 4)
    assert lib.pkv_workspace_bytes_multi(ctypes.byref(d), 4, 1, 4, 4) == one
    # a table narrower than the shortest chunk splits no row: no records either way
    assert lib.pkv_workspace_bytes_multi(ctypes.byref(d), 4, 4, 4, 4) == one
    # a wider one holds a record per query vector of every chunk of a split row
    wide = lib.pkv_workspace_bytes(ctypes.byref(d), 4, 4, 64)
    assert lib.pkv_workspace_bytes_multi(ctypes.byref(d), 4, 4, 4, 64) > wide
    assert lib.pkv_workspace_bytes_multi(ctypes.byref(d), 4, 0, 4, 4) == 0


def test_row_and_width_limits(lib):
    """The library is built for at most 65535 rows and 2^24-token rows."""
    d = binding.host_desc(64, 16, 4, 64, "bf16", "HND")
    p = ctypes.c_void_p(16)
    at = lambda rows, m: _capi.STATUS_NAMES[lib.pkv_check_attention_host(
        ctypes.byref(d), p, m, p, rows, 4)]
    assert at(65536, 4) == "UNSUPPORTED"
    assert at(4, (1 << 24) // 16 + 1) == "UNSUPPORTED"
    assert lib.pkv_workspace_bytes(ctypes.byref(d), 65535, 4, 4) > 0
    assert lib.pkv_workspace_bytes(ctypes.byref(d), 65536, 4, 4) == 0


def test_decode_kernel_choice(lib):
    """The kernel a shape runs: query vectors per KV head (heads per KV head x new
    tokens) decide it, bfloat16 pools of head_dim <= 128 go to the matrix cores from 4."""
    def name(kvh, heads, d=128, dtype="bf16", q=1):
        desc = binding.host_desc(64, 16, kvh, d, dtype, "HND")
        return lib.pkv_decode_kernel_for(ctypes.byref(desc), heads, q).decode()
    assert name(32, 32) == "decode_kernel, 1 query vector per item"
    assert name(16, 32) == "decode_kernel, 2 query vectors per item"
    assert name(8, 32) == "decode_mfma_kernel, 4 query vectors per item"
    assert name(4, 32) == "decode_mfma_kernel, 8 query vectors per item"
    assert name(2, 32) == "decode_mfma_kernel, 16 query vectors per item"
    assert name(32, 32, q=4) == "decode_mfma_kernel, 4 query vectors per item"
    assert name(32, 32, q=3) == "decode_kernel, 1 query vector per item"
    assert name(8, 32, dtype="f32") == "decode_kernel, 4 query vectors per item"
    assert name(4, 32, d=256) == "decode_kernel, 4 query vectors per item"
    assert name(4, 6) == ""


def test_tuning_is_validated_before_it_changes(lib):
    """A refused tuning changes nothing; solo_tokens takes 1 (none) or a power of two in
    [32, 1024], and the chunk range must be powers of two within a ratio of 64."""
    before = binding.get_tuning()
    try:
        for bad in (dict(solo_tokens=16), dict(solo_tokens=2048), dict(solo_tokens=300),
                    dict(chunk_min=64, chunk_max=8192), dict(chunk_min=96),
                    dict(decode_waves=3), dict(groups_per_cu=17), dict(solo_tokens=-1)):
            with pytest.raises(binding.PagedKVError, match="UNSUPPORTED"):
                binding.set_tuning(**bad)
            assert binding.get_tuning() == before
        binding.set_tuning(solo_tokens=1)
        assert binding.get_tuning()["solo_tokens"] == 1
        binding.set_tuning(solo_tokens=1024, chunk_min=32, chunk_max=2048)
        t = binding.get_tuning()
        assert (t["solo_tokens"], t["chunk_min"], t["chunk_max"]) == (1024, 32, 2048)
    finally:
        binding.set_tuning(**before)
    assert binding.get_tuning() == before

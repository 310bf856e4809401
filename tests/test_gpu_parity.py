"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Tolerances (written here, derived from the arithmetic):
* float32 pools: max |gpu - oracle| <= 2e-6;
* bfloat16 pools: max |gpu - oracle| <= 2e-2, and the tighter per-element bound
  |gpu - oracle| <= 2^-8 |oracle| + 2e-5: the kernel accumulates in float32 (relative
  error ~1e-6 on these sizes) and rounds once to bfloat16 (half an ulp, 2^-9 relative);
* the slot scatter: bit-exact.
Every case compares every output row.  The large configurations (pools of 2-34 GB)
recompute each row with the oracle from a host copy of just the blocks that row group
names (block relabelling leaves the oracle's result unchanged, a pinned invariant), on
a pool of host threads.
"""

import os
import zlib
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
from paged_attention_decode_kv_amd import _capi, accounting, binding
from paged_attention_decode_kv_amd import workloads as wl

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)
TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


# --------------------------------------------------------------------------- #
# helpers
# --------------------------------------------------------------------------- #
def say(msg):
    print(f"[gpu-test] {msg}", flush=True)


def to_dev(a, dtype=None):
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(a).to(DEV)


def to_host(t, dtype):
    t = t.detach().contiguous()
    if dtype == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bits(t):
    """Integer view of a tensor, for bit-exact comparison."""
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def assert_close(got_storage, ref, dtype, where=""):
    got = oracle.decode_storage(got_storage, dtype)
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got)), f"non-finite output {where}"
    err = np.abs(got - ref)
    if dtype == "f32":
        assert err.max() <= 2e-6, f"max err {err.max():.3e} {where}"
    else:
        assert err.max() <= 2e-2, f"max err {err.max():.3e} {where}"
        bound = 2.0 ** -8 * np.abs(ref) + 2e-5
        worst = np.argmax(err - bound)
        assert np.all(err <= bound), (f"err {err.flat[worst]:.3e} > bound "
                                      f"{bound.flat[worst]:.3e} at {worst} {where}")
    return float(err.max())


class Step:
    """Device tensors of one workload, before and after a decode step."""

    def __init__(self, w, *, host_history=None):
        self.w = w
        host_history = w.history_on_host() if host_history is None else host_history
        self.k_host = self.v_host = None
        if host_history:
            self.k_host, self.v_host = wl.history_host(w)
            self.k_cache = to_dev(self.k_host, w.dtype)
            self.v_cache = to_dev(self.v_host, w.dtype)
        else:
            self.k_cache = torch.empty(w.pool_shape, dtype=TORCH_DT[w.dtype], device=DEV)
            self.v_cache = torch.empty_like(self.k_cache)
            wl.history_device(w, self.k_cache, self.v_cache)
        self.q = to_dev(w.q, w.dtype)
        self.k_new = to_dev(w.k_new, w.dtype)
        self.v_new = to_dev(w.v_new, w.dtype)
        self.slots = to_dev(w.slot_mapping)
        self.tables = to_dev(w.block_tables)
        self.lens = to_dev(w.context_lens)

    def run(self, validate=True, out=None, workspace=None):
        """kv_write then the read (the multi-token read when the workload has several
        new tokens per row), in the given workspace if any."""
        w = self.w
        binding.kv_write(self.k_new, self.v_new, self.slots, self.k_cache, self.v_cache,
                         layout=w.layout, validate=validate)
        read = binding.paged_attention if w.query_len == 1 else binding.paged_attention_multi
        out = read(self.q, self.k_cache, self.v_cache, self.tables, self.lens, w.scale,
                   layout=w.layout, out=out, workspace=workspace, validate=validate)
        torch.cuda.synchronize()
        return out

    def workspace(self):
        w = self.w
        if w.query_len == 1:
            n = binding.workspace_bytes(self.k_cache, w.rows, w.heads, w.max_blocks, w.layout)
        else:
            n = binding.workspace_bytes_multi(self.k_cache, w.rows, w.query_len, w.heads,
                                              w.max_blocks, w.layout)
        return torch.empty(n, dtype=torch.uint8, device=DEV)

    def host_pools_for(self, rows):
        """Host copies of the pre-step blocks the given rows name, relabelled 0..n-1,
        with the tables and write slots (query_len per row) of those rows remapped to
        match."""
        w = self.w
        nq = w.query_len
        blocks = wl.live_blocks(w, rows)
        remap = {int(b): i for i, b in enumerate(blocks)}
        n = len(blocks)
        idx = torch.from_numpy(np.append(blocks, w.num_blocks).astype(np.int64)).to(DEV)
        k = to_host(self.k_cache.index_select(0, idx), w.dtype)
        v = to_host(self.v_cache.index_select(0, idx), w.dtype)
        bt = np.full((len(rows), w.max_blocks), -1, dtype=np.int32)
        sm = np.empty(len(rows) * nq, dtype=np.int64)
        for i, r in enumerate(rows):
            live = wl.cdiv(w.context_lens[r], w.block_size)
            bt[i, :live] = [remap[int(b)] for b in w.block_tables[r, :live]]
            for j in range(nq):
                s = int(w.slot_mapping[r * nq + j])
                if w.context_lens[r] == 0:
                    sm[i * nq + j] = n * w.block_size
                else:
                    sm[i * nq + j] = remap[s // w.block_size] * w.block_size + s % w.block_size
        return k, v, bt, sm, n


def oracle_full(w, k_host, v_host):
    kw, vw = k_host.copy(), v_host.copy()
    oracle.kv_write(kw, vw, w.k_new, w.v_new, w.slot_mapping, num_blocks=w.num_blocks,
                    block_size=w.block_size, layout=w.layout, dtype=w.dtype)
    out = oracle.paged_attention(w.q, kw, vw, w.block_tables, w.context_lens, w.scale,
                                 num_blocks=w.num_blocks, block_size=w.block_size,
                                 layout=w.layout, dtype=w.dtype)
    return out, kw, vw


# host threads for the oracle (numpy releases the interpreter lock in its gathers,
# products and elementwise loops); a few, so that the float64 rectangles in flight
# stay within a few GB of host memory
ORACLE_THREADS = max(1, min(8, len(os.sched_getaffinity(0))))


def _row_groups(lens, rows, per_row, cells):
    """Rows sorted by length, cut into groups whose oracle rectangle (rows x longest
    length x per_row elements) stays within `cells` (a longer row goes alone)."""
    order = sorted(range(len(rows)), key=lambda i: int(lens[rows[i]]))
    groups, at = [], 0
    while at < len(order):
        end = at + 1
        while end < len(order) and \
                (end + 1 - at) * max(1, int(lens[rows[order[end]]])) * per_row <= cells:
            end += 1
        groups.append(order[at:end])
        at = end
    return groups


def oracle_rows(step, rows, cells=1 << 23):
    """Oracle outputs of the given rows (all of a full-size batch's rows, as the tests
    ask): groups of rows of similar length, each from a host copy of just the blocks it
    names (copied in this thread), computed on ORACLE_THREADS host threads."""
    w = step.w
    rows = [int(r) for r in rows]
    nq = w.query_len
    out = np.zeros((len(rows),) + w.q.shape[1:])
    kv_shape = (w.rows, nq, w.kv_heads, w.head_dim)
    read = oracle.paged_attention if nq == 1 else oracle.paged_attention_multi

    def compute(part, k, v, bt, sm, n):
        k_new = w.k_new.reshape(kv_shape)[part].reshape(-1, w.kv_heads, w.head_dim)
        v_new = w.v_new.reshape(kv_shape)[part].reshape(-1, w.kv_heads, w.head_dim)
        oracle.kv_write(k, v, k_new, v_new, sm, num_blocks=n, block_size=w.block_size,
                        layout=w.layout, dtype=w.dtype)
        return read(w.q[part], k, v, bt, w.context_lens[part], w.scale, num_blocks=n,
                    block_size=w.block_size, layout=w.layout, dtype=w.dtype)

    groups = _row_groups(w.context_lens, rows, w.heads * w.head_dim * nq, cells)
    with ThreadPoolExecutor(ORACLE_THREADS) as ex:
        pending = []
        for g in groups:
            part = [rows[i] for i in g]
            pending.append((g, ex.submit(compute, part, *step.host_pools_for(part))))
            while len(pending) >= 2 * ORACLE_THREADS:   # bound the host copies in flight
                g0, f0 = pending.pop(0)
                out[g0] = f0.result()
        for g0, f0 in pending:
            out[g0] = f0.result()
    return out


def check_plan(w, info):
    """The plan and the decode kernel's own walk count against the host's accounting
    of the same lengths (Day 59, "What I learned" 5: the helper's tile count and the
    kernel's loop are held to the same lengths)."""
    lens = w.context_lens.astype(np.int64)
    P = info["chunk_tokens"]
    assert P > 0 and P & (P - 1) == 0, info
    live = lens[lens > 0]
    assert info["live_entries"] == accounting.tiles_walked(live, P), info
    assert info["entries"] == info["live_entries"] + int(np.count_nonzero(lens == 0)), info
    assert info["full_chunks"] == int(np.sum(live // P)), info
    split = live[live > P]
    assert info["split_rows"] == len(split), info
    assert info["records"] == accounting.tiles_walked(split, P), info
    assert info["records"] <= info["record_capacity"], info
    T = info["tile_tokens"]
    assert T in (4, 8, 16), info
    assert info["vector_groups"] >= 1, info
    assert info["tiles_walked"] == info["vector_groups"] * accounting.tiles_walked(live, T), info
    assert info["status"] == 0, info


def check_full(w):
    say(f"{w.name}: rows={w.rows} heads={w.heads}/{w.kv_heads} d={w.head_dim} "
        f"bs={w.block_size} {w.dtype} {w.layout} lens={w.context_lens.tolist()[:8]}")
    st = Step(w, host_history=True)
    out = st.run()
    ref, kw, vw = oracle_full(w, st.k_host, st.v_host)
    err = assert_close(to_host(out, w.dtype), ref, w.dtype, w.name)
    # the scatter: bit-exact everywhere but the sink, whose value is one pad row's
    sink_b = w.num_blocks
    gk, gv = to_host(st.k_cache, w.dtype), to_host(st.v_cache, w.dtype)
    ints = np.uint16 if w.dtype == "bf16" else np.uint32
    for got, want in ((gk, kw), (gv, vw)):
        assert np.array_equal(got[:sink_b].view(ints), want[:sink_b].view(ints))
    return err


# --------------------------------------------------------------------------- #
# the named configurations
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("layout", ["HND", "NHD"])
def test_config1_tiny_fp32(layout):
    err = check_full(wl.make_config(1, layout=layout))
    say(f"tiny fp32 {layout}: max err {err:.3e}")


def test_config2_uniform_bf16():
    err = check_full(wl.make_config(2))
    say(f"uniform bf16: max err {err:.3e}")


def _full_size(idx, kv_heads=None, query_len=1):
    """A full-size configuration (or its grouped or multi-token variant): every live
    row against the oracle, pad rows zero, the scatter bit-exact at every written slot
    with the rest of the pool untouched, and the plan's counts and the kernel's own
    walk count against the host accounting."""
    w = wl.make_config(idx, kv_heads=kv_heads, query_len=query_len)
    say(f"{w.name} kv_heads={w.kv_heads} query_len={w.query_len}: building "
        f"{w.pool_bytes / 1e9:.1f} GB of pools on the device")
    st = Step(w, host_history=False)
    k_before = st.k_cache.clone()
    v_before = st.v_cache.clone()
    ws = st.workspace()
    out = st.run(workspace=ws)
    info = binding.plan_info(ws)
    say(f"{w.name}: plan {info}")
    check_plan(w, info)
    live = w.live_rows
    say(f"{w.name}: oracle on all {len(live)} live rows, {ORACLE_THREADS} host threads")
    ref = oracle_rows(st, live)
    got = to_host(out, w.dtype)[live]
    err = assert_close(got, ref, w.dtype, w.name)
    # scatter: every live row's slots hold its new K/V bit-exactly, nothing else moved
    nq = w.query_len
    tokens = (live[:, None] * nq + np.arange(nq)[None, :]).reshape(-1)
    slots = torch.from_numpy(w.slot_mapping[tokens]).to(DEV)
    blk, off = slots // w.block_size, slots % w.block_size
    tok_dev = torch.from_numpy(tokens).to(DEV)
    sink_b = w.num_blocks
    for pool, before, new in ((st.k_cache, k_before, st.k_new),
                              (st.v_cache, v_before, st.v_new)):
        if w.layout == "HND":
            assert torch.equal(bits(pool[blk, :, off, :]), bits(new[tok_dev]))
            before[blk, :, off, :] = new[tok_dev]
            before[sink_b, :, 0, :] = pool[sink_b, :, 0, :]
        else:
            assert torch.equal(bits(pool[blk, off]), bits(new[tok_dev]))
            before[blk, off] = new[tok_dev]
            before[sink_b, 0] = pool[sink_b, 0]
        assert torch.equal(bits(before), bits(pool)), "the scatter touched another slot"
    # padding rows: zero output
    pads = w.pad_rows
    if len(pads):
        assert torch.count_nonzero(out[torch.from_numpy(pads).to(DEV)]).item() == 0
    say(f"{w.name}: every row, max err {err:.3e}")
    del k_before, v_before, st
    torch.cuda.empty_cache()


def test_config3_ragged_every_row():
    _full_size(3)


def test_config4_long_tail_every_row():
    _full_size(4)


def test_config5_full_width_every_row():
    _full_size(5)


PLAN_TUNINGS = [
    {},                                               # the plan's own choice
    {"chunk_min": 512, "chunk_max": 512},             # pinned
    {"chunk_min": 8192, "chunk_max": 8192},           # pinned: no row of width 8192 split
    {"chunk_min": 32, "chunk_max": 2048, "solo_tokens": 1, "decode_waves": 4},
]


@pytest.mark.parametrize("tuning", PLAN_TUNINGS,
                         ids=lambda t: "-".join(f"{k}{v}" for k, v in t.items()) or "default")
@pytest.mark.parametrize("idx,kv_heads,query_len", [(2, None, 1), (3, None, 1), (4, None, 1),
                                                    (5, None, 1), (5, 8, 1), (5, None, 4)])
def test_plan_counts_equal_the_kernel_walk(idx, kv_heads, query_len, tuning):
    """Day 59, "What I learned" 5: the host's tile accounting and the kernel's loop,
    held to the same lengths.  The plan's entries are sum(cdiv(len, P)) plus the pad
    rows; the decode kernel's own count of the tiles it streamed is the vector groups
    times sum(cdiv(len, tile)).  The counts depend on the lengths alone, so the rows'
    tables here name blocks of a small shared pool (rows may share blocks for a read)."""
    w = wl.make_config(idx, kv_heads=kv_heads, query_len=query_len)
    nb = 2048
    j = np.arange(w.max_blocks, dtype=np.int64)[None, :]
    r = np.arange(w.rows, dtype=np.int64)[:, None]
    tables = to_dev(((j * 7 + r * 131) % nb).astype(np.int32))
    shape = (nb + 1, w.kv_heads, w.block_size, w.head_dim)
    gen = torch.Generator(device=DEV).manual_seed(idx)
    k = torch.randn(shape, generator=gen, device=DEV).to(torch.bfloat16)
    v = torch.randn(shape, generator=gen, device=DEV).to(torch.bfloat16)
    q = to_dev(w.q, w.dtype)
    lens = to_dev(w.context_lens)
    saved = binding.get_tuning()
    binding.set_tuning(**tuning)
    try:
        if query_len == 1:
            n = binding.workspace_bytes(k, w.rows, w.heads, w.max_blocks)
            read = binding.paged_attention
        else:
            n = binding.workspace_bytes_multi(k, w.rows, query_len, w.heads, w.max_blocks)
            read = binding.paged_attention_multi
        ws = torch.empty(n, dtype=torch.uint8, device=DEV)
        read(q, k, v, tables, lens, w.scale, workspace=ws, validate=False)
        info = binding.plan_info(ws)
    finally:
        binding.set_tuning(**saved)
    say(f"config {idx} kv_heads={w.kv_heads} query_len={query_len} {tuning}: {info}")
    check_plan(w, info)
    if "chunk_max" in tuning and tuning["chunk_min"] == tuning["chunk_max"]:
        assert info["chunk_tokens"] == tuning["chunk_min"]


def _budget_batch():
    """64 rows of 4096 tokens, float32 pools, 32 query heads over 4 KV heads (8 query
    vectors to an item on the vector units).  8 waves per CU need 4096 items; 256-token
    chunks are the longest that give them (64 x 16 entries x 4 head groups), and their
    records (64 x 16 chunks of 32 vectors, 17.3 MB) exceed the workspace's cap of 992
    record chunks, while 512-token chunks (512 record chunks) fit."""
    return wl.make_custom([4096] * 64, heads=32, kv_heads=4, head_dim=128, block_size=16,
                          dtype="f32", layout="HND", seed=64)


@pytest.mark.parametrize("chunk_max", [0, 256], ids=["budget-binds", "budget-fits"])
def test_record_budget_moves_the_plan_to_longer_chunks(chunk_max):
    """The split rows' partial records have a fixed budget in the workspace: the
    records every row needs at the longest chunk length, or 16 MiB, whichever is more.
    With the default range the plan's first choice does not fit and it takes the next
    longer chunk; with the range capped at 256 tokens the cap is that range's own need
    and the first choice stands.  Every row against the oracle both ways."""
    w = _budget_batch()
    st = Step(w)
    saved = binding.get_tuning()
    if chunk_max:
        binding.set_tuning(chunk_min=128, chunk_max=chunk_max)
    try:
        ws = st.workspace()
        out = st.run(workspace=ws)
        info = binding.plan_info(ws)
    finally:
        binding.set_tuning(**saved)
    say(f"record budget, chunk_max {chunk_max or 'default'}: {info}")
    check_plan(w, info)
    lens = w.context_lens.astype(np.int64)
    cap = info["record_capacity"]
    if chunk_max:
        assert cap == accounting.tiles_walked(lens, 256), info
        assert info["chunk_tokens"] == 256 and info["records"] == cap, info
    else:
        assert cap == 992, info
        assert accounting.tiles_walked(lens, 256) > cap, info    # the first choice
        assert info["chunk_tokens"] == 512 and info["records"] == 512, info
    ref = oracle_rows(st, w.live_rows)
    err = assert_close(to_host(out, w.dtype)[w.live_rows], ref, w.dtype, "record budget")
    say(f"record budget: every row, max err {err:.3e}")


@pytest.mark.parametrize("chunk", [0, 8192], ids=["default", "chunk8192"])
def test_rows_longer_than_the_longest_chunk(chunk):
    """Rows of up to 20000 tokens (a table 20000 wide): even at the longest chunk
    (8192 tokens) they split, into up to 3 chunks, and the merge joins them.  8 query
    heads over 2 KV heads (4 vectors to an item, the matrix cores), bf16."""
    lens = [20000, 16384, 8193, 8192, 100, 0, 1]
    w = wl.make_custom(lens, heads=8, kv_heads=2, head_dim=128, block_size=16, dtype="bf16",
                       layout="HND", seed=2000)
    st = Step(w, host_history=False)
    saved = binding.get_tuning()
    if chunk:
        binding.set_tuning(chunk_min=chunk, chunk_max=chunk)
    try:
        ws = st.workspace()
        out = st.run(workspace=ws)
        info = binding.plan_info(ws)
    finally:
        binding.set_tuning(**saved)
    say(f"rows past the longest chunk, chunk {chunk or 'default'}: {info}")
    check_plan(w, info)
    if chunk:
        assert info["chunk_tokens"] == chunk and info["split_rows"] == 3, info
    ref = oracle_rows(st, w.live_rows)
    err = assert_close(to_host(out, w.dtype)[w.live_rows], ref, w.dtype,
                       "rows past the longest chunk")
    assert torch.all(out[torch.from_numpy(w.pad_rows).to(DEV)] == 0)
    say(f"rows past the longest chunk: max err {err:.3e}")


def test_a_row_of_a_quarter_million_tokens():
    """One row of 2^18 tokens beside a row of 3: a table 2^18 wide, the row cut into
    about a thousand chunks and merged from as many partial records (the merge's loop
    over more chunks than it holds at once).  2 query heads over 1 KV head, head_dim 64,
    bf16; every output against the oracle."""
    w = wl.make_custom([1 << 18, 3], heads=2, kv_heads=1, head_dim=64, block_size=16,
                       dtype="bf16", layout="HND", seed=20)
    st = Step(w, host_history=False)
    ws = st.workspace()
    out = st.run(workspace=ws)
    info = binding.plan_info(ws)
    say(f"2^18 tokens: {info}")
    check_plan(w, info)
    assert info["split_rows"] >= 1 and (1 << 18) // info["chunk_tokens"] > 8, info
    ref = oracle_rows(st, w.live_rows)
    err = assert_close(to_host(out, w.dtype)[w.live_rows], ref, w.dtype, "2^18 tokens")
    say(f"2^18 tokens: max err {err:.3e}")


@pytest.mark.parametrize("chunk", [0, 1024], ids=["default", "chunk1024"])
def test_the_most_rows(chunk):
    """65535 rows, the most the library takes: the plan walks them 1024 at a time and
    keeps each thread's first four rows in registers, so rows past 4096 take its other
    path (lengths and record offsets reloaded from memory).  Short rows with pad rows
    among them, and long rows past index 4096; with 1024-token chunks those split, so
    their record offsets come back from memory too.  Every row against the oracle, and
    the plan against the host accounting."""
    rng = np.random.default_rng(65535)
    lens = rng.integers(0, 41, 65535)
    for r in (5000, 30000, 65534, 4100):
        lens[r] = 3000 + r % 7
    w = wl.make_custom(lens.tolist(), heads=2, kv_heads=1, head_dim=64, dtype="bf16",
                       layout="HND", seed=65535)
    st = Step(w, host_history=False)
    saved = binding.get_tuning()
    if chunk:
        binding.set_tuning(chunk_min=chunk, chunk_max=chunk)
    try:
        ws = st.workspace()
        out = st.run(workspace=ws)
        info = binding.plan_info(ws)
    finally:
        binding.set_tuning(**saved)
    say(f"65535 rows, chunk {chunk or 'default'}: {info}")
    check_plan(w, info)
    if chunk:
        assert info["chunk_tokens"] == chunk and info["split_rows"] == 4, info
    ref = oracle_rows(st, w.live_rows)
    err = assert_close(to_host(out, w.dtype)[w.live_rows], ref, w.dtype, "65535 rows")
    assert torch.all(out[torch.from_numpy(w.pad_rows).to(DEV)] == 0)
    say(f"65535 rows: every row, max err {err:.3e}")


# --------------------------------------------------------------------------- #
# shapes, ragged tails and edges at sizes the oracle finishes quickly
# --------------------------------------------------------------------------- #
SWEEP = [
    # lens, heads, kv_heads, head_dim, block_size, dtype, layout
    ([1, 15, 16, 17, 255, 256, 257, 700], 8, 8, 128, 16, "bf16", "HND"),
    ([1, 15, 16, 17, 255, 256, 257, 700], 8, 8, 128, 16, "f32", "HND"),
    ([513, 0, 33, 1024, 5], 8, 2, 128, 16, "bf16", "NHD"),
    ([513, 0, 33, 1024, 5], 8, 2, 128, 16, "f32", "NHD"),
    ([300, 64, 1, 0, 97], 4, 4, 64, 16, "bf16", "HND"),
    ([300, 64, 1, 0, 97], 4, 1, 64, 32, "f32", "NHD"),
    ([130, 257, 2], 4, 2, 256, 16, "bf16", "HND"),
    ([130, 257, 2], 4, 4, 256, 64, "f32", "HND"),
    ([777, 512, 31], 16, 4, 128, 32, "bf16", "NHD"),
    ([1000, 3], 4, 4, 64, 128, "bf16", "HND"),
    ([2049, 40], 4, 4, 128, 256, "f32", "NHD"),
]


@pytest.mark.parametrize("case", SWEEP, ids=lambda c: f"{c[5]}-{c[6]}-d{c[3]}-bs{c[4]}-h{c[1]}/{c[2]}")
def test_shape_sweep(case):
    lens, h, hkv, d, bs, dtype, layout = case
    w = wl.make_custom(lens, heads=h, kv_heads=hkv, head_dim=d, block_size=bs, dtype=dtype,
                       layout=layout, seed=sum(lens) + d + bs)
    check_full(w)


def test_all_padding_batch():
    w = wl.make_custom([0, 0, 0], heads=4, head_dim=128, dtype="bf16", seed=2)
    st = Step(w, host_history=True)
    out = st.run()
    assert torch.count_nonzero(out).item() == 0
    gk = to_host(st.k_cache, w.dtype)
    assert np.array_equal(gk[:w.num_blocks], st.k_host[:w.num_blocks])


def test_full_table_single_row():
    w = wl.make_custom([4096], heads=4, kv_heads=4, head_dim=128, block_size=16,
                       dtype="f32", max_blocks=256, num_blocks=256, seed=4)
    check_full(w)


def test_poisoned_pad_slots_are_never_read():
    """NaN in every slot no live position names (stale tails and unnamed blocks) and -1
    past each live table prefix leave the output equal to the unpoisoned oracle's."""
    w = wl.make_custom([37, 5, 0, 16, 300, 1], heads=4, head_dim=128, dtype="bf16",
                       num_blocks=64, max_blocks=24, seed=6)
    k_host, v_host = wl.history_host(w)
    ref, _, _ = oracle_full(w, k_host, v_host)
    live = {}
    for r in range(w.rows):
        for t in range(int(w.context_lens[r])):
            live.setdefault(int(w.block_tables[r, t // 16]), set()).add(t % 16)
    kp, vp = k_host.copy(), v_host.copy()
    for b in range(w.num_blocks + 1):
        for o in range(16):
            if o not in live.get(b, ()):
                kp[b, :, o, :] = wl.BF16_NAN
                vp[b, :, o, :] = wl.BF16_NAN
    st = Step(w, host_history=True)
    st.k_cache.copy_(to_dev(kp, "bf16"))
    st.v_cache.copy_(to_dev(vp, "bf16"))
    # the written slots receive finite new K/V; the sink keeps NaN
    out = st.run()
    assert_close(to_host(out, w.dtype), ref, w.dtype, "poisoned")


def test_block_placement_is_bit_invisible():
    w = wl.make_custom([300, 45, 513, 0, 16], heads=8, kv_heads=4, head_dim=128,
                       dtype="bf16", num_blocks=96, max_blocks=40, seed=8)
    st = Step(w, host_history=True)
    base = to_host(st.run(), w.dtype)
    pi = np.random.default_rng(3).permutation(w.num_blocks)
    k2, v2 = st.k_host.copy(), st.v_host.copy()
    k2[pi] = st.k_host[:w.num_blocks]
    v2[pi] = st.v_host[:w.num_blocks]
    w2 = wl.make_custom([300, 45, 513, 0, 16], heads=8, kv_heads=4, head_dim=128,
                        dtype="bf16", num_blocks=96, max_blocks=40, seed=8)
    bt = w2.block_tables.copy()
    bt[bt >= 0] = pi[bt[bt >= 0]]
    w2.block_tables = bt
    sm = w2.slot_mapping.copy()
    livem = w2.context_lens > 0
    sm[livem] = pi[sm[livem] // 16] * 16 + sm[livem] % 16
    w2.slot_mapping = sm
    st2 = Step(w2, host_history=True)
    st2.k_cache.copy_(to_dev(k2, "bf16"))
    st2.v_cache.copy_(to_dev(v2, "bf16"))
    moved = to_host(st2.run(), w2.dtype)
    assert np.array_equal(base, moved)


def test_runs_are_bit_deterministic():
    w = wl.make_config(4)
    st = Step(w, host_history=False)
    a = to_host(st.run(validate=False), w.dtype)
    b = to_host(st.run(validate=False), w.dtype)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("kind", ["vector", "vector-single-wave", "matrix-cores",
                                  "matrix-cores-single-wave"])
def test_bad_block_ids_without_validation_are_skipped_and_reported(kind):
    """validate=False on every decode path: a live block id outside [0, num_blocks) (the
    sink block, -1, far past the pool) is never read, its 16 tokens drop out of the
    row's softmax, and the BLOCK_ID status bit is raised.  The decode read has no
    positional term, so such a row equals the oracle over its table without that entry;
    the other rows are untouched."""
    solo = kind.endswith("single-wave")
    heads, kvh = (16, 4) if kind.startswith("matrix") else (4, 4)
    lens = _solo_lens(560, 8, 17) if solo else [700, 40, 1500, 0, 33, 260, 2100]
    w = wl.make_custom(lens, heads=heads, kv_heads=kvh, head_dim=128, dtype="bf16", seed=17)
    bs = w.block_size
    # rows of at least three blocks; a bad id goes in a block before the last (the last
    # holds the step's own token)
    cand = [r for r in range(w.rows) if w.context_lens[r] >= 3 * bs]
    long_row = int(np.argmax(w.context_lens))
    short_rows = [r for r in cand if w.context_lens[r] < 300][:2]
    bad = {long_row: (1, w.num_blocks)}
    for r, v in zip(short_rows, (-1, w.num_blocks + 1000)):
        bad[r] = (wl.cdiv(int(w.context_lens[r]), bs) - 2, v)
    tables = w.block_tables.copy()
    for r, (j, v) in bad.items():
        tables[r, j] = v
    st = Step(w, host_history=True)
    st.tables = to_dev(tables)
    saved = binding.get_tuning()
    binding.set_tuning(groups_per_cu=1, solo_tokens=512 if solo else 1)
    try:
        binding.device_status(DEV, clear=True)
        ws = st.workspace()
        clean_ws = st.workspace()
        got = to_host(st.run(validate=False, workspace=ws), "bf16")
        # the bit belongs to this call: its workspace has it, a clean call's has not,
        # and the device-wide word keeps it until cleared
        clean = Step(w, host_history=True)
        clean.run(validate=False, workspace=clean_ws)
        assert binding.workspace_status(ws) == _capi.DEVERR_BLOCK_ID
        assert binding.workspace_status(clean_ws) == 0
        assert binding.device_status(DEV, clear=True) & _capi.DEVERR_BLOCK_ID
        # a later clean call in the same workspace starts its status afresh
        clean.run(validate=False, workspace=ws)
        assert binding.workspace_status(ws) == 0
    finally:
        binding.set_tuning(**saved)
    ref, kw, vw = _oracle_by_rows(w, st.k_host, st.v_host)
    for r, (j, _) in bad.items():
        n = int(w.context_lens[r])
        row = np.delete(w.block_tables[r], j)
        bt = np.full((1, w.max_blocks), -1, dtype=np.int32)
        bt[0, :len(row)] = row
        ref[r] = oracle.paged_attention(w.q[[r]], kw, vw, bt, np.array([n - bs], np.int32),
                                        w.scale, num_blocks=w.num_blocks, block_size=bs,
                                        layout=w.layout, dtype="bf16")[0]
    say(f"{kind}: bad ids in rows {sorted(bad)} of {w.rows}")
    assert_close(got, ref, "bf16", kind)


@pytest.mark.parametrize("kind", ["vector", "matrix"])
def test_bad_lengths_without_validation_are_clamped_and_reported(kind):
    """validate=False: a length below 0 reads as 0 (the row gives zeros), and one past
    what its table addresses reads as the table's capacity (the whole table).  The
    CONTEXT_BOUNDS status bit is raised in the call's workspace and in the device word.
    Every row against the oracle over the clamped lengths."""
    heads, kvh = (16, 4) if kind == "matrix" else (4, 4)
    lens = [100, 0, 4096, 50, 0, 777]      # row 2 fills its table: 256 blocks of 16
    w = wl.make_custom(lens, heads=heads, kv_heads=kvh, head_dim=128, dtype="bf16",
                       max_blocks=256, seed=23)
    st = Step(w, host_history=True)
    binding.kv_write(st.k_new, st.v_new, st.slots, st.k_cache, st.v_cache, layout=w.layout)
    bad = st.lens.clone()
    bad[1] = -5                            # clamps to 0: the pad row it is
    bad[2] = 4096 + 777                    # clamps to 4096: the row as it is
    ws = st.workspace()
    binding.device_status(DEV, clear=True)
    out = binding.paged_attention(st.q, st.k_cache, st.v_cache, st.tables, bad, w.scale,
                                  layout=w.layout, workspace=ws, validate=False)
    torch.cuda.synchronize()
    assert binding.workspace_status(ws) == _capi.DEVERR_CONTEXT_BOUNDS
    assert binding.device_status(DEV, clear=True) & _capi.DEVERR_CONTEXT_BOUNDS
    ref, _, _ = oracle_full(w, st.k_host, st.v_host)
    err = assert_close(to_host(out, w.dtype), ref, w.dtype, f"clamped lengths, {kind}")
    say(f"clamped lengths ({kind}): max err {err:.3e}")


def test_bad_write_slots_without_validation_are_skipped_and_reported():
    """validate=False: a write slot outside [0, sink] (below 0, past the sink) is
    skipped, so its token's K/V go nowhere, every other token lands bit-exactly, the
    rest of the pool is untouched, and the SLOT status bit is raised."""
    w = wl.make_custom([40, 17, 0, 99, 5], heads=4, kv_heads=2, head_dim=128, dtype="bf16",
                       layout="NHD", seed=29)
    st = Step(w, host_history=True)
    sink = binding.sink_slot(st.k_cache, w.layout)
    assert sink == w.num_blocks * w.block_size
    slots = w.slot_mapping.copy()
    slots[1] = -3
    slots[3] = sink + 5
    binding.device_status(DEV, clear=True)
    binding.kv_write(st.k_new, st.v_new, to_dev(slots), st.k_cache, st.v_cache,
                     layout=w.layout, validate=False)
    torch.cuda.synchronize()
    assert binding.device_status(DEV, clear=True) & _capi.DEVERR_SLOT
    keep = np.array([i for i in range(len(slots)) if 0 <= slots[i] <= sink])
    kw, vw = st.k_host.copy(), st.v_host.copy()
    oracle.kv_write(kw, vw, w.k_new[keep], w.v_new[keep], slots[keep],
                    num_blocks=w.num_blocks, block_size=w.block_size, layout=w.layout,
                    dtype=w.dtype)
    for got, want in ((st.k_cache, kw), (st.v_cache, vw)):
        g = to_host(got, w.dtype)
        assert np.array_equal(g.view(np.uint16), want.view(np.uint16)), \
            "a skipped token's K/V landed, or a slot other than the named ones changed"
    say(f"bad write slots: tokens 1 and 3 skipped, {len(keep)} written")


def test_first_launches_from_two_host_threads():
    """A fresh process whose first decode launches come from two host threads at once
    (each on its own stream; one shape on the vector units and one on the matrix cores,
    then one shape from both): every output matches the oracle."""
    import subprocess
    import sys
    helper = os.path.join(os.path.dirname(os.path.abspath(__file__)), "two_thread_first_launch.py")
    r = subprocess.run([sys.executable, helper], capture_output=True, text=True, timeout=240)
    say(r.stdout.strip().replace("\n", " | "))
    assert r.returncode == 0 and "OK" in r.stdout, r.stdout + r.stderr[-2000:]


def test_refusals_touch_nothing():
    w = wl.make_custom([37, 5, 16], heads=4, head_dim=128, dtype="bf16", seed=9)
    st = Step(w, host_history=True)
    out = torch.full_like(st.q, 7.0)
    bad = st.tables.clone()
    bad[1, 0] = w.num_blocks                       # the sink block named in a live prefix
    with pytest.raises(binding.PagedKVError) as e:
        binding.paged_attention(st.q, st.k_cache, st.v_cache, bad, st.lens, w.scale,
                                out=out)
    assert e.value.code == "BLOCK_ID"
    lens = st.lens.clone()
    lens[2] = w.max_blocks * w.block_size + 1
    with pytest.raises(binding.PagedKVError) as e:
        binding.paged_attention(st.q, st.k_cache, st.v_cache, st.tables, lens, w.scale,
                                out=out)
    assert e.value.code == "CONTEXT_BOUNDS"
    slots = st.slots.clone()
    slots[0] = w.sink + 1
    with pytest.raises(binding.PagedKVError) as e:
        binding.kv_write(st.k_new, st.v_new, slots, st.k_cache, st.v_cache)
    assert e.value.code == "SLOT"
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
    assert np.array_equal(to_host(st.k_cache, "bf16"), st.k_host)
    assert np.array_equal(to_host(st.v_cache, "bf16"), st.v_host)
    with pytest.raises(binding.PagedKVError) as e:
        binding.paged_attention(st.q[:0], st.k_cache, st.v_cache, st.tables[:0],
                                st.lens[:0], w.scale)
    assert e.value.code == "EMPTY"


TUNINGS = [
    dict(chunk_min=128, chunk_max=1024, decode_waves=8, items_per_group=8, deal=2),
    dict(chunk_min=32, chunk_max=32, decode_waves=1, items_per_group=1, staging=2),
    dict(chunk_min=2048, chunk_max=2048, decode_waves=4, items_per_group=1),
    dict(chunk_min=64, chunk_max=2048, decode_waves=2, items_per_group=64, staging=2),
    dict(chunk_min=128, chunk_max=2048, decode_waves=8, items_per_group=16, staging=2),
    dict(chunk_min=256, chunk_max=256, decode_waves=8, items_per_group=1, deal=1),
    # chunks of up to 512 blocks: an item's block ids span all eight id registers
    dict(chunk_min=4096, chunk_max=8192, decode_waves=8, items_per_group=1),
    dict(chunk_min=8192, chunk_max=8192, decode_waves=8, items_per_group=16, staging=2),
]


@pytest.mark.parametrize("tuning", TUNINGS, ids=lambda t: "-".join(f"{k}{v}" for k, v in t.items()))
def test_work_split_variants(tuning):
    """Every work split (chunk range, waves per workgroup, items per wave) gives oracle
    parity."""
    before = binding.get_tuning()
    binding.set_tuning(**tuning)
    try:
        for dtype in ("bf16", "f32"):
            w = wl.make_custom([4100, 0, 1, 255, 256, 257, 2049, 31, 700, 8192, 8177], heads=8,
                               kv_heads=2,
                               head_dim=128, block_size=16, dtype=dtype, layout="HND",
                               seed=77)
            check_full(w)
    finally:
        binding.set_tuning(**before)


LONG_CHUNKS = [
    # lens, heads, kv_heads, head_dim, block_size, dtype, layout, chunk, waves: chunks of
    # thousands of tokens, so a wave's block ids fill one or more id registers; block
    # sizes above 16 put several sub-chunks in a block, and float32 (and head_dim 256)
    # has sub-chunks of 8 (4) tokens
    ([8000, 4097, 31], 4, 4, 128, 32, "bf16", "HND", 8192, 8),
    ([8192, 5000], 4, 4, 128, 256, "bf16", "NHD", 8192, 8),
    ([6000, 100], 4, 4, 128, 16, "f32", "HND", 8192, 8),
    ([4100, 2], 2, 2, 256, 64, "f32", "HND", 4096, 8),
    ([7000, 300], 8, 2, 128, 64, "bf16", "HND", 8192, 8),
    ([8192, 1500, 0], 4, 4, 128, 16, "bf16", "HND", 8192, 1),
]


@pytest.mark.parametrize("case", LONG_CHUNKS,
                         ids=lambda c: f"{c[5]}-d{c[3]}-bs{c[4]}-h{c[1]}/{c[2]}-c{c[7]}-w{c[8]}")
def test_long_chunks_across_block_sizes(case):
    """Pinned chunks of 4096-8192 tokens over long rows give oracle parity for every
    block size and sub-chunk width (each wave's block ids span 64+ sub-chunks)."""
    lens, h, hkv, d, bs, dtype, layout, chunk, waves = case
    before = binding.get_tuning()
    binding.set_tuning(chunk_min=chunk, chunk_max=chunk, decode_waves=waves)
    try:
        w = wl.make_custom(lens, heads=h, kv_heads=hkv, head_dim=d, block_size=bs, dtype=dtype,
                           layout=layout, seed=sum(lens) + bs + chunk)
        check_full(w)
    finally:
        binding.set_tuning(**before)


def _solo_lens(n_short, n_long, seed, short_max=300, low=1):
    """Many short rows (below the single-wave bound), a few long ones and two pad rows."""
    rng = np.random.default_rng(seed)
    lens = np.concatenate([rng.integers(low, short_max, n_short),
                           rng.integers(600, 1600, n_long), [0, 0]])
    rng.shuffle(lens)
    return [int(x) for x in lens]


SOLO_CASES = [
    # name, lens, query_len, heads, kv_heads, head_dim, block_size, dtype, layout, tuning.
    # The test pins 256 workgroups (groups_per_cu 1), and every case has at least one
    # short chunk per wave (>= 2048 for 8-wave workgroups), so the plan keeps the
    # single-wave phase; the long rows still go through the shared 8-wave items.
    ("vec-bf16", _solo_lens(560, 8, 1), 1, 4, 4, 128, 16, "bf16", "HND",
     dict(solo_tokens=512)),
    # 128-token chunks under a 1024 bound: every item single-wave, split rows included
    ("vec-bf16-all", _solo_lens(100, 40, 2), 1, 4, 4, 128, 16, "bf16", "HND",
     dict(solo_tokens=1024, chunk_min=128, chunk_max=128)),
    # four query heads per item on the vector units, float32
    ("vec-f32-gqa4", _solo_lens(1100, 8, 3), 1, 8, 2, 128, 16, "f32", "NHD",
     dict(solo_tokens=512, mfma=2)),
    # 4-token sub-chunks: items of up to 1023 tokens span four id registers of one wave
    ("vec-f32-d256", _solo_lens(140, 2, 4, short_max=1024), 1, 2, 2, 256, 32, "f32", "HND",
     dict(solo_tokens=1024, decode_waves=1)),
    ("vec-d64-registers", _solo_lens(560, 8, 5, short_max=128), 1, 4, 4, 64, 16, "bf16",
     "HND", dict(solo_tokens=128, staging=1)),
    ("vec-one-wave", _solo_lens(300, 4, 6, short_max=256), 1, 4, 4, 128, 64, "bf16", "HND",
     dict(solo_tokens=256, decode_waves=1)),
    ("vec-four-waves", _solo_lens(300, 4, 7, short_max=64), 1, 4, 4, 128, 16, "bf16", "HND",
     dict(solo_tokens=64, decode_waves=4)),
    ("vec-off", _solo_lens(560, 8, 1), 1, 4, 4, 128, 16, "bf16", "HND", dict(solo_tokens=1)),
    # several new tokens: causal limits inside single-wave items
    ("vec-q2-f32", _solo_lens(300, 4, 8, low=2), 2, 4, 4, 128, 16, "f32", "HND",
     dict(solo_tokens=256, chunk_min=64, chunk_max=64)),
    ("vec-q4", _solo_lens(560, 4, 9, low=4), 4, 4, 4, 128, 16, "bf16", "HND",
     dict(solo_tokens=1024, mfma=2)),
    # the matrix cores: 4, 8 and 16 vectors per item, written from one wave's tiles
    ("mfma-gqa4", _solo_lens(560, 8, 10), 1, 16, 4, 128, 16, "bf16", "HND",
     dict(solo_tokens=512)),
    ("mfma-gqa16-d64", _solo_lens(1100, 4, 11), 1, 32, 2, 64, 16, "bf16", "NHD",
     dict(solo_tokens=512)),
    ("mfma-q4", _solo_lens(560, 4, 12, low=4), 4, 4, 4, 128, 16, "bf16", "HND",
     dict(solo_tokens=1024)),
    ("mfma-gqa4-split", _solo_lens(200, 30, 13), 1, 16, 4, 128, 32, "bf16", "HND",
     dict(solo_tokens=1024, chunk_min=128, chunk_max=128)),
]


def _oracle_by_rows(w, k_host, v_host, cells=1 << 23, slot_rect=None):
    """The oracle's step over a large batch: one scatter, then the read a few rows at a
    time (a row's output depends on that row alone), rows of similar length together so
    that each call's rectangle stays narrow.  With slot_rect, the read through that slot
    window instead of the block tables."""
    kw, vw = k_host.copy(), v_host.copy()
    oracle.kv_write(kw, vw, w.k_new, w.v_new, w.slot_mapping, num_blocks=w.num_blocks,
                    block_size=w.block_size, layout=w.layout, dtype=w.dtype)
    if slot_rect is not None:
        read, addr = oracle.paged_attention_slots, slot_rect
    elif w.query_len == 1:
        read, addr = oracle.paged_attention, w.block_tables
    else:
        read, addr = oracle.paged_attention_multi, w.block_tables
    per_row = w.heads * w.head_dim * w.query_len
    out = np.zeros(w.q.shape)
    order = np.argsort(w.context_lens, kind="stable")
    at = 0
    while at < w.rows:
        end = at + 1
        while end < w.rows and (end + 1 - at) * max(1, int(w.context_lens[order[end]])) * \
                per_row <= cells:
            end += 1
        part = order[at:end]
        out[part] = read(w.q[part], kw, vw, addr[part], w.context_lens[part], w.scale,
                         num_blocks=w.num_blocks, block_size=w.block_size, layout=w.layout,
                         dtype=w.dtype)
        at = end
    return out, kw, vw


@pytest.mark.parametrize("case", SOLO_CASES, ids=[c[0] for c in SOLO_CASES])
def test_single_wave_items(case):
    """Chunks shorter than solo_tokens are read one wave each, before the shared items;
    every output against the oracle for every bound, sub-chunk width, staging path,
    query group and kernel."""
    name, lens, n_q, h, hkv, d, bs, dtype, layout, tuning = case
    w = wl.make_custom(lens, heads=h, kv_heads=hkv, head_dim=d, block_size=bs, dtype=dtype,
                       layout=layout, query_len=n_q, seed=zlib.crc32(name.encode()))
    say(f"{name}: rows {w.rows} heads {h}/{hkv} d {d} q {n_q} {dtype} {layout} {tuning}")
    before = binding.get_tuning()
    binding.set_tuning(groups_per_cu=1, **tuning)
    try:
        st = Step(w, host_history=True)
        got = st.run() if n_q == 1 else _multi_run(w, st)
    finally:
        binding.set_tuning(**before)
    assert binding.device_status(DEV, clear=True) == 0
    ref, kw, vw = _oracle_by_rows(w, st.k_host, st.v_host)
    assert_close(to_host(got, dtype), ref, dtype, name)
    ints = np.uint16 if dtype == "bf16" else np.uint32
    for dev_pool, want in ((st.k_cache, kw), (st.v_cache, vw)):
        got_pool = to_host(dev_pool, dtype)
        assert np.array_equal(got_pool[:w.num_blocks].view(ints), want[:w.num_blocks].view(ints))


NARROW_SOLO_CASES = [
    # name, lens, query_len, dtype, layout (32 heads, head_dim 128, block 16).  Small,
    # near-uniform batches whose 256-token chunks give about one item per wave at 8
    # waves per CU but not 16 items per workgroup: on a 256-CU MI355X the plan takes
    # 256-token single-wave chunks at 8 waves per CU, by the single-wave branch alone
    ("16x1024-bf16", [1024] * 16, 1, "bf16", "HND"),
    ("ragged8-bf16-nhd", [2135, 2202, 1811, 2203, 2034, 2057, 2115, 1942], 1, "bf16", "NHD"),
    ("16x1024-f32", [1024] * 16, 1, "f32", "HND"),
    ("16x1024-q2", [1024] * 16, 2, "bf16", "HND"),
]


@pytest.mark.parametrize("case", NARROW_SOLO_CASES, ids=[c[0] for c in NARROW_SOLO_CASES])
def test_single_wave_chunks_at_eight_waves_per_cu(case):
    """Default tuning on batches whose chunks are all single-wave items, one per wave of
    an 8-waves-per-CU launch: every output against the oracle, the scatter bit-exact."""
    name, lens, n_q, dtype, layout = case
    w = wl.make_custom(lens, heads=32, kv_heads=32, head_dim=128, block_size=16, dtype=dtype,
                       layout=layout, query_len=n_q, seed=zlib.crc32(name.encode()))
    say(f"{name}: rows {w.rows} lens {lens[:4]}.. q {n_q} {dtype} {layout}")
    st = Step(w, host_history=True)
    got = st.run() if n_q == 1 else _multi_run(w, st)
    assert binding.device_status(DEV, clear=True) == 0
    ref, kw, vw = _oracle_by_rows(w, st.k_host, st.v_host)
    assert_close(to_host(got, dtype), ref, dtype, name)
    ints = np.uint16 if dtype == "bf16" else np.uint32
    for dev_pool, want in ((st.k_cache, kw), (st.v_cache, vw)):
        got_pool = to_host(dev_pool, dtype)
        assert np.array_equal(got_pool[:w.num_blocks].view(ints), want[:w.num_blocks].view(ints))


GQA_CASES = [
    # lens, heads, kv_heads, head_dim, dtype, layout: query groups 8, 4, 2 and 16 (two items)
    ([700, 1, 0, 2049, 31], 16, 2, 128, "bf16", "HND"),
    ([700, 1, 0, 2049, 31], 16, 2, 128, "f32", "NHD"),
    ([513, 64, 1000], 32, 8, 64, "bf16", "HND"),
    ([257, 5], 8, 4, 256, "f32", "HND"),
    ([300, 90], 32, 2, 128, "bf16", "NHD"),
    ([130, 2500], 16, 4, 256, "bf16", "HND"),
]


@pytest.mark.parametrize("case", GQA_CASES, ids=lambda c: f"{c[4]}-{c[5]}-d{c[3]}-h{c[1]}/{c[2]}")
@pytest.mark.parametrize("max_group", [16, 8, 1])
def test_grouped_query_heads(case, max_group):
    """Grouped-query attention: one K/V load serves up to 8 query heads (max_group 8) or
    one (max_group 1); both match the oracle."""
    lens, h, hkv, d, dtype, layout = case
    before = binding.get_tuning()
    binding.set_tuning(max_query_group=max_group)
    try:
        w = wl.make_custom(lens, heads=h, kv_heads=hkv, head_dim=d, dtype=dtype,
                           layout=layout, seed=sum(lens) + h)
        check_full(w)
    finally:
        binding.set_tuning(**before)


@pytest.mark.parametrize("kv_heads", [8, 4])
def test_config5_grouped_variant_every_row(kv_heads):
    """The full-width batch with 32 query heads over 8 or 4 KV heads."""
    _full_size(5, kv_heads=kv_heads)



# --------------------------------------------------------------------------- #
# captured steps
# --------------------------------------------------------------------------- #
def _graph_step_workload(n, seed, num_blocks, max_blocks, heads, kv_heads, max_len):
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, max_len + 1, n)
    return wl.make_custom(lens.tolist(), heads=heads, kv_heads=kv_heads, head_dim=128,
                          block_size=16, dtype="bf16", layout="HND", num_blocks=num_blocks,
                          max_blocks=max_blocks, seed=seed)


@pytest.mark.parametrize("heads,kv_heads", [(8, 8), (8, 2)])
def test_bucketed_graphs_replay_real_steps(heads, kv_heads):
    """Graphs recorded per row bucket over an all-padding batch replay a sequence of
    real steps of other sizes on one evolving pool; every step matches the oracle."""
    from paged_attention_decode_kv_amd.graphs import DecodeGraphs
    mb, nb = 48, 16 * 48 + 8
    first = _graph_step_workload(16, 100, nb, mb, heads, kv_heads, 700)
    k_host, v_host = wl.history_host(first)
    k_cache, v_cache = to_dev(k_host, "bf16"), to_dev(v_host, "bf16")
    say(f"bucketed graphs heads={heads}/{kv_heads} pool={first.pool_shape}")
    binding.device_status(DEV, clear=True)
    graphs = DecodeGraphs(k_cache, v_cache, num_heads=heads, max_blocks=mb, scale=first.scale,
                          buckets=[4, 8, 16])
    torch.cuda.synchronize()
    # the warm runs wrote only the sink and left zeros
    assert torch.count_nonzero(graphs.out).item() == 0
    assert np.array_equal(to_host(k_cache, "bf16")[:nb], k_host[:nb])
    kh, vh = k_host.copy(), v_host.copy()
    plan = [(16, 700, mb), (5, 700, mb), (8, 250, 16), (1, 700, mb), (13, 700, mb)]
    for i, (n, max_len, width) in enumerate(plan):
        w = _graph_step_workload(n, 200 + i, nb, width, heads, kv_heads, max_len)
        say(f"  step {i}: rows {n} bucket {graphs.bucket_for(n)} width {width} "
            f"lens {w.context_lens.tolist()}")
        got = graphs.step(to_dev(w.q, "bf16"), to_dev(w.k_new, "bf16"),
                          to_dev(w.v_new, "bf16"), to_dev(w.slot_mapping),
                          to_dev(w.block_tables), to_dev(w.context_lens))
        torch.cuda.synchronize()
        oracle.kv_write(kh, vh, w.k_new, w.v_new, w.slot_mapping, num_blocks=nb,
                        block_size=16, layout="HND", dtype="bf16")
        ref = oracle.paged_attention(w.q, kh, vh, w.block_tables, w.context_lens, w.scale,
                                     num_blocks=nb, block_size=16, layout="HND",
                                     dtype="bf16")
        assert_close(to_host(got, "bf16"), ref, "bf16", f"graph step {i}")
        assert np.array_equal(to_host(k_cache, "bf16")[:nb], kh[:nb])
        assert np.array_equal(to_host(v_cache, "bf16")[:nb], vh[:nb])
        # rows past n in the bucket are padding: their output is zero
        b = graphs.bucket_for(n)
        assert torch.count_nonzero(graphs.out[n:b]).item() == 0
    assert binding.device_status(DEV, clear=True) == 0
    graphs.close()


def test_graph_replays_switch_the_single_wave_phase():
    """One recorded 640-row step, 256 workgroups pinned at capture, replayed on batches
    that do and do not keep the single-wave phase (the plan decides it on the device per
    replay): mostly short rows, long rows, a mix, and a few rows.  Every replay against
    the oracle on the evolving pool."""
    from paged_attention_decode_kv_amd.graphs import DecodeGraphs
    heads, kvh, d, mb = 4, 4, 64, 80
    nb = 640 * mb + 8
    saved = binding.get_tuning()
    binding.set_tuning(groups_per_cu=1, solo_tokens=512)
    try:
        def batch(n_short, n_long, seed):
            rng = np.random.default_rng(seed)
            lens = np.concatenate([rng.integers(1, 300, n_short),
                                   rng.integers(600, mb * 16 - 16, n_long)])
            rng.shuffle(lens)
            return wl.make_custom(lens.tolist(), heads=heads, kv_heads=kvh, head_dim=d,
                                  block_size=16, dtype="bf16", layout="HND",
                                  num_blocks=nb, max_blocks=mb, seed=seed)
        first = batch(4, 4, 900)
        k_host, v_host = wl.history_host(first)
        k_cache, v_cache = to_dev(k_host, "bf16"), to_dev(v_host, "bf16")
        graphs = DecodeGraphs(k_cache, v_cache, num_heads=heads, max_blocks=mb,
                              scale=first.scale, buckets=[640])
        torch.cuda.synchronize()
        kh, vh = k_host.copy(), v_host.copy()
        for i, (n_short, n_long) in enumerate([(600, 0), (0, 600), (560, 40), (3, 2),
                                               (600, 20)]):
            w = batch(n_short, n_long, 910 + i)
            say(f"  replay {i}: {n_short} short rows, {n_long} long")
            got = graphs.step(to_dev(w.q, "bf16"), to_dev(w.k_new, "bf16"),
                              to_dev(w.v_new, "bf16"), to_dev(w.slot_mapping),
                              to_dev(w.block_tables), to_dev(w.context_lens))
            torch.cuda.synchronize()
            ref, kh, vh = _oracle_by_rows(w, kh, vh)
            assert_close(to_host(got, "bf16"), ref, "bf16", f"replay {i}")
            assert np.array_equal(to_host(k_cache, "bf16")[:nb], kh[:nb])
            assert torch.count_nonzero(graphs.out[w.rows:]).item() == 0
        assert binding.device_status(DEV, clear=True) == 0
        graphs.close()
    finally:
        binding.set_tuning(**saved)


def test_caller_stream_capture_of_the_step():
    """The two entry points with validate=0 are capturable by a caller's own stream
    capture: recorded over padding, replayed several times on real batches written into
    the same tensors, with eager work between replays."""
    rows, mb = 24, 64
    nb = rows * mb + 8
    rng = np.random.default_rng(5)
    batches = [_graph_step_workload(rows, 40 + i, nb, mb, 16, 4, 1024) for i in range(2)]
    w0 = batches[0]
    st = Step(w0, host_history=True)
    k_host, v_host = st.k_host, st.v_host
    out = torch.empty_like(st.q)
    ws = torch.empty(binding.workspace_bytes(st.k_cache, rows, 16, mb), dtype=torch.uint8,
                     device=DEV)
    st.lens.zero_()
    st.slots.fill_(w0.sink)
    st.tables.fill_(-1)
    say(f"caller capture: rows={rows} lens {[w.context_lens.tolist()[:6] for w in batches]}")
    torch.cuda.synchronize()
    binding.paged_attention(st.q, st.k_cache, st.v_cache, st.tables, st.lens, w0.scale,
                            out=out, workspace=ws, validate=False)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        binding.kv_write(st.k_new, st.v_new, st.slots, st.k_cache, st.v_cache, validate=False)
        binding.paged_attention(st.q, st.k_cache, st.v_cache, st.tables, st.lens, w0.scale,
                                out=out, workspace=ws, validate=False)
    st.k_cache.copy_(to_dev(k_host, "bf16"))
    st.v_cache.copy_(to_dev(v_host, "bf16"))
    out.fill_(7.0)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0
    assert np.array_equal(to_host(st.k_cache, "bf16")[:nb], k_host[:nb])
    for w in batches:
        st.k_cache.copy_(to_dev(k_host, "bf16"))
        st.v_cache.copy_(to_dev(v_host, "bf16"))
        for dst, src, dt in ((st.q, w.q, "bf16"), (st.k_new, w.k_new, "bf16"),
                             (st.v_new, w.v_new, "bf16"), (st.slots, w.slot_mapping, None),
                             (st.tables, w.block_tables, None), (st.lens, w.context_lens, None)):
            dst.copy_(to_dev(src, dt))
        torch.cuda.synchronize()
        for rep in range(2):
            graph.replay()
            torch.cuda.synchronize()
            if rep == 0:
                ref, kw, vw = oracle_full(w, k_host, v_host)
            assert_close(to_host(out, "bf16"), ref, "bf16", f"replay {rep} seed {w.seed}")
            # the second replay writes the same vectors into the same slots
            assert np.array_equal(to_host(st.k_cache, "bf16")[:nb], kw[:nb])
            assert np.array_equal(to_host(st.v_cache, "bf16")[:nb], vw[:nb])


# --------------------------------------------------------------------------- #
# the read through a per-token slot rectangle
# --------------------------------------------------------------------------- #
def _block_table_rect(w, width, stride, junk=-7):
    """The slot window a slot table holds for ``w``'s block placement, as a
    [rows, width] view of a [rows, stride] table; junk past each row's length."""
    t = np.arange(width)
    bt = np.where(w.block_tables >= 0, w.block_tables, 0).astype(np.int64)
    rect = bt[:, t // w.block_size] * w.block_size + t % w.block_size
    table = np.full((w.rows, stride), junk, dtype=np.int64)
    table[:, :width] = np.where(t[None, :] < w.context_lens[:, None], rect, junk)
    return table


def _scatter_rows(w, table, rows, rng):
    """Rewrite the live cells of ``rows`` (but each row's newest cell, its write slot)
    with distinct random slots that no other row uses."""
    sink = w.num_blocks * w.block_size
    used = set()
    for r in range(w.rows):
        n = int(w.context_lens[r])
        if r not in rows:
            used.update(table[r, :n].tolist())
        elif n:
            used.add(int(table[r, n - 1]))
    free = iter(s for s in rng.permutation(sink).tolist() if s not in used)
    for r in rows:
        n = int(w.context_lens[r])
        for t in range(n - 1):
            table[r, t] = next(free)
    return table


def _slot_run(st, table, width, *, validate=True, out=None):
    w = st.w
    binding.kv_write(st.k_new, st.v_new, st.slots, st.k_cache, st.v_cache, layout=w.layout,
                     validate=validate)
    tab = to_dev(table)
    got = binding.paged_attention_slots(st.q, st.k_cache, st.v_cache, tab[:, :width],
                                        st.lens, w.scale, layout=w.layout, out=out,
                                        validate=validate)
    torch.cuda.synchronize()
    return got


def _slot_oracle(w, k_host, v_host, table, width):
    kw, vw = k_host.copy(), v_host.copy()
    oracle.kv_write(kw, vw, w.k_new, w.v_new, w.slot_mapping, num_blocks=w.num_blocks,
                    block_size=w.block_size, layout=w.layout, dtype=w.dtype)
    return oracle.paged_attention_slots(w.q, kw, vw, table[:, :width], w.context_lens,
                                        w.scale, num_blocks=w.num_blocks,
                                        block_size=w.block_size, layout=w.layout,
                                        dtype=w.dtype)


SLOT_CASES = [
    # name, lens, heads, kv_heads, head_dim, block_size, dtype, layout
    ("tiny-f32-HND", [16, 40], 4, 4, 64, 16, "f32", "HND"),
    ("tiny-f32-NHD", [16, 40, 0, 3], 4, 4, 64, 16, "f32", "NHD"),
    ("ragged-bf16", [1, 17, 0, 300, 1024, 1025, 2100, 64], 8, 8, 128, 16, "bf16", "HND"),
    ("gqa-bf16", [700, 0, 33, 1500, 129], 16, 4, 128, 16, "bf16", "HND"),
    ("d256-bs32", [90, 513, 0, 1], 4, 2, 256, 32, "bf16", "NHD"),
]


@pytest.mark.parametrize("case", SLOT_CASES, ids=[c[0] for c in SLOT_CASES])
def test_block_structured_slots_equal_block_tables(case):
    """A window whose live cells follow the block placement takes the block path: bit
    for bit the block-table read, and the oracle's value."""
    name, lens, heads, kvh, d, bs, dtype, layout = case
    w = wl.make_custom(lens, heads=heads, kv_heads=kvh, head_dim=d, block_size=bs,
                       dtype=dtype, layout=layout, seed=zlib.crc32(name.encode()))
    width = w.max_blocks * w.block_size
    table = _block_table_rect(w, width, width + 37)
    say(f"slots {name}: lens {lens} width {width}")
    st = Step(w, host_history=True)
    ref_block = st.run()
    blk = to_host(ref_block, dtype).copy()
    st2 = Step(w, host_history=True)
    got = _slot_run(st2, table, width)
    assert np.array_equal(to_host(got, dtype), blk), "slot window differs from block tables"
    ref = _slot_oracle(w, st.k_host, st.v_host, table, width)
    assert_close(to_host(got, dtype), ref, dtype, name)
    assert binding.device_status(DEV, clear=True) == 0


@pytest.mark.parametrize("chunk", [0, 32])
@pytest.mark.parametrize("case", SLOT_CASES, ids=[c[0] for c in SLOT_CASES])
def test_scattered_slots_are_read_token_by_token(case, chunk):
    """Rows whose live cells name scattered slots (and a mix with block-structured
    rows and padding) match the oracle; chunk=32 splits the token-by-token rows into
    many chunks, merged by the combine kernel."""
    name, lens, heads, kvh, d, bs, dtype, layout = case
    w = wl.make_custom(lens, heads=heads, kv_heads=kvh, head_dim=d, block_size=bs,
                       dtype=dtype, layout=layout, num_blocks=sum(wl.cdiv(c, bs) for c in lens) + 40,
                       seed=zlib.crc32(name.encode()) + 1)
    width = w.max_blocks * w.block_size
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    live = [r for r in range(w.rows) if w.context_lens[r] > 0]
    scattered = live[::2]
    table = _scatter_rows(w, _block_table_rect(w, width, width), scattered, rng)
    say(f"scattered {name} chunk {chunk}: rows {scattered} of {w.rows}")
    st = Step(w, host_history=True)
    saved = binding.get_tuning()
    if chunk:
        binding.set_tuning(chunk_min=chunk, chunk_max=chunk)
    try:
        got = _slot_run(st, table, width)
    finally:
        binding.set_tuning(**saved)
    ref = _slot_oracle(w, st.k_host, st.v_host, table, width)
    assert_close(to_host(got, dtype), ref, dtype, name)
    assert binding.device_status(DEV, clear=True) == 0


@pytest.mark.parametrize("chunk", [0, 64])
def test_many_token_rows_share_one_queue(chunk):
    """Every live row of a 1500-row batch scattered: more token-by-token rows than one
    pass of the plan's threads, their chunks (full ones, then remainders by length) in
    one shared queue; chunk=64 splits most rows.  Against the oracle."""
    rows = 1500
    rng = np.random.default_rng(31)
    lens = rng.integers(0, 300, rows)
    lens[::50] = rng.integers(600, 2500, len(lens[::50]))
    w = wl.make_custom(lens.tolist(), heads=2, kv_heads=2, head_dim=64, dtype="bf16", seed=31)
    width = w.max_blocks * w.block_size
    live = [r for r in range(rows) if lens[r] > 0]
    table = _scatter_rows(w, _block_table_rect(w, width, width), live, rng)
    st = Step(w, host_history=True)
    saved = binding.get_tuning()
    if chunk:
        binding.set_tuning(chunk_min=chunk, chunk_max=chunk)
    try:
        got = _slot_run(st, table, width)
    finally:
        binding.set_tuning(**saved)
    assert binding.device_status(DEV, clear=True) == 0
    ref = _oracle_by_rows(w, st.k_host, st.v_host, slot_rect=table[:, :width])[0]
    assert_close(to_host(got, "bf16"), ref, "bf16", f"1500 token rows, chunk {chunk}")


@pytest.mark.parametrize("chunk", [0, 128])
def test_short_token_rows_one_wave_each(chunk):
    """Every live row of a 1200-row batch scattered, mostly shorter than solo_tokens:
    more short chunks than the token kernels have waves, so token_rows_short_kernel
    reads them one wave each after the shared ones; a few long rows stay shared
    (chunk=128 splits everything into short chunks).  Against the oracle."""
    rng = np.random.default_rng(51)
    lens = np.concatenate([rng.integers(1, 400, 1150), rng.integers(600, 3000, 50), [0]])
    rng.shuffle(lens)
    w = wl.make_custom(lens.tolist(), heads=4, kv_heads=2, head_dim=128, dtype="bf16",
                       layout="NHD", seed=51)
    width = w.max_blocks * w.block_size
    live = [r for r in range(w.rows) if lens[r] > 0]
    table = _scatter_rows(w, _block_table_rect(w, width, width), live, rng)
    st = Step(w, host_history=True)
    saved = binding.get_tuning()
    if chunk:
        binding.set_tuning(chunk_min=chunk, chunk_max=chunk)
    try:
        got = _slot_run(st, table, width)
    finally:
        binding.set_tuning(**saved)
    assert binding.device_status(DEV, clear=True) == 0
    ref = _oracle_by_rows(w, st.k_host, st.v_host, slot_rect=table[:, :width])[0]
    assert_close(to_host(got, "bf16"), ref, "bf16", f"short token rows, chunk {chunk}")


def test_token_rows_beside_single_wave_items():
    """A slot window with both kinds of rows while the single-wave phase runs: 600 short
    block-structured rows (2400 short chunks, more than one per wave of 256 workgroups),
    long block rows whose 2048-token chunks and remainders stay shared, and scattered
    rows for the token kernel, whose list the plan builds in the same bins after it has
    placed the block rows' chunks.  Against the oracle."""
    rng = np.random.default_rng(41)
    lens = np.concatenate([rng.integers(1, 300, 600), rng.integers(2500, 4000, 20),
                           rng.integers(700, 3000, 20), [0]])
    rng.shuffle(lens)
    w = wl.make_custom(lens.tolist(), heads=4, kv_heads=4, head_dim=64, dtype="bf16", seed=41)
    width = w.max_blocks * w.block_size
    scattered = [r for r in range(w.rows) if 700 <= lens[r] < 3000 and lens[r] > 300]
    scattered = [r for r in scattered if not 2500 <= lens[r] < 4000][:20]
    table = _scatter_rows(w, _block_table_rect(w, width, width), scattered, rng)
    st = Step(w, host_history=True)
    saved = binding.get_tuning()
    binding.set_tuning(groups_per_cu=1, chunk_min=2048, chunk_max=2048, solo_tokens=512)
    try:
        got = _slot_run(st, table, width)
    finally:
        binding.set_tuning(**saved)
    assert binding.device_status(DEV, clear=True) == 0
    ref = _oracle_by_rows(w, st.k_host, st.v_host, slot_rect=table[:, :width])[0]
    assert_close(to_host(got, "bf16"), ref, "bf16", "token rows beside single-wave items")


def test_one_moved_token_past_the_first_translation_chunk():
    """A single cell that breaks the block structure at position > 1024 sends its row
    token by token; the other rows stay on the block path, bit for bit."""
    w = wl.make_custom([3000, 2500, 900], heads=8, kv_heads=8, head_dim=128, dtype="bf16",
                       num_blocks=600, seed=77)
    width = w.max_blocks * w.block_size
    table = _block_table_rect(w, width, width)
    used = set(np.concatenate([table[r, :w.context_lens[r]] for r in range(3)]).tolist())
    spare = next(s for s in range(w.num_blocks * 16) if s not in used)
    table[0, 2049] = spare                      # translation chunk 2 of row 0
    say("moved token: row 0 position 2049")
    st = Step(w, host_history=True)
    got = to_host(_slot_run(st, table, width), "bf16")
    ref = _slot_oracle(w, st.k_host, st.v_host, table, width)
    assert_close(got, ref, "bf16", "moved token")
    blk = to_host(Step(w, host_history=True).run(), "bf16")
    assert np.array_equal(got[1:], blk[1:])     # untouched rows: the block path
    assert not np.array_equal(got[0], blk[0])


def test_slot_refusals_touch_nothing():
    w = wl.make_custom([40, 16, 0], heads=4, kv_heads=4, head_dim=64, dtype="f32", seed=9)
    width = w.max_blocks * w.block_size
    st = Step(w, host_history=True)
    tab = to_dev(_block_table_rect(w, width, width))
    out = torch.full_like(st.q, 3.0)
    sink = w.num_blocks * w.block_size
    for row, t, bad, code in ((0, 39, -1, "SLOT"), (1, 0, sink, "SLOT"),
                              (0, 5, sink + 1, "SLOT")):
        t2 = tab.clone()
        t2[row, t] = bad
        with pytest.raises(binding.PagedKVError, match=code):
            binding.paged_attention_slots(st.q, st.k_cache, st.v_cache, t2, st.lens,
                                          w.scale, out=out)
    lens = st.lens.clone()
    lens[1] = width + 1
    with pytest.raises(binding.PagedKVError, match="CONTEXT_BOUNDS"):
        binding.paged_attention_slots(st.q, st.k_cache, st.v_cache, tab, lens, w.scale,
                                      out=out)
    with pytest.raises(binding.PagedKVError, match="DTYPE"):
        binding.paged_attention_slots(st.q, st.k_cache, st.v_cache, tab.int(), st.lens,
                                      w.scale, out=out)
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)


def test_bad_live_slot_without_validation_is_skipped_and_reported():
    """validate=False: a live cell outside the slots is skipped (the kernel never reads
    it) and raises the SLOT status bit; rows without one are still exact."""
    w = wl.make_custom([40, 16, 33], heads=4, kv_heads=4, head_dim=64, dtype="f32", seed=4)
    width = w.max_blocks * w.block_size
    table = _block_table_rect(w, width, width)
    table[0, 3] = -(1 << 40)
    table[2, 7] = w.num_blocks * w.block_size + 12345
    st = Step(w, host_history=True)
    binding.device_status(DEV, clear=True)
    got = to_host(_slot_run(st, table, width, validate=False), "f32")
    assert binding.device_status(DEV, clear=True) & _capi.DEVERR_SLOT
    ok = table.copy()
    ok[0, 3] = ok[0, 2]
    ok[2, 7] = ok[2, 6]
    ref = _slot_oracle(w, st.k_host, st.v_host, ok, width)
    assert_close(got[1:2], ref[1:2], "f32", "clean row")
    assert np.all(np.isfinite(got))


def test_config5_as_a_slot_window():
    """The full-width batch read through its slot window (256 x 8192 int64 cells, a
    view of a wider table): every output bit-identical to the block-table read, and
    every row against the oracle."""
    w = wl.make_config(5)
    width = w.max_blocks * w.block_size
    st = Step(w)
    say(f"config 5 slot window {w.rows} x {width}")
    blk = to_host(st.run(validate=False), "bf16").copy()
    t = torch.arange(width, device=DEV)
    tables = st.tables.long().clamp_min(0)
    rect = tables[:, t // w.block_size] * w.block_size + t % w.block_size
    table = torch.full((w.rows, width + 64), -1, dtype=torch.int64, device=DEV)
    table[:, :width] = torch.where(t[None, :] < st.lens[:, None].long(), rect, -1)
    got = binding.paged_attention_slots(st.q, st.k_cache, st.v_cache, table[:, :width],
                                        st.lens, w.scale)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(got, "bf16"), blk)
    live = w.live_rows
    ref = oracle_rows(st, live)
    assert_close(blk[live], ref, "bf16", "config 5 slot window")


def test_captured_slot_window_step():
    """pkv_graph_capture_slots recorded over an all-padding batch replays real steps
    whose slot windows are written into the same table: bit for bit the eager slot
    read, with block-structured and scattered rows."""
    w = wl.make_custom([300, 0, 1100, 57, 2000, 16], heads=8, kv_heads=2, head_dim=128,
                       dtype="bf16", num_blocks=400, seed=31)
    width = w.max_blocks * w.block_size
    table_host = _block_table_rect(w, width, width + 16)
    table_host = _scatter_rows(w, table_host, [2, 3], np.random.default_rng(2))
    st = Step(w, host_history=True)
    k_host, v_host = st.k_host, st.v_host
    table = torch.full((w.rows, width + 16), -1, dtype=torch.int64, device=DEV)
    out = torch.empty_like(st.q)
    ws = torch.empty(binding.workspace_bytes_slots(st.k_cache, w.rows, w.heads, width),
                     dtype=torch.uint8, device=DEV)
    real = [t.clone() for t in (st.q, st.k_new, st.v_new, st.slots, st.lens)]
    st.lens.zero_()
    st.slots.fill_(w.sink)
    say(f"captured slot window: rows {w.rows} width {width}")
    graph = binding.capture_step_slots(st.k_new, st.v_new, st.slots, st.q, st.k_cache,
                                       st.v_cache, table[:, :width], st.lens, w.scale, out,
                                       ws)
    out.fill_(5.0)
    graph.launch()
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0
    for dst, src in zip((st.q, st.k_new, st.v_new, st.slots, st.lens), real):
        dst.copy_(src)
    table.copy_(to_dev(table_host))
    torch.cuda.synchronize()
    replays = []
    for _ in range(2):
        st.k_cache.copy_(to_dev(k_host, "bf16"))
        st.v_cache.copy_(to_dev(v_host, "bf16"))
        graph.launch()
        torch.cuda.synchronize()
        replays.append(to_host(out, "bf16").copy())
    graph.destroy()
    st2 = Step(w, host_history=True)
    eager = to_host(_slot_run(st2, table_host, width), "bf16")
    for got in replays:
        assert np.array_equal(got, eager)
    ref = _slot_oracle(w, k_host, v_host, table_host, width)
    assert_close(eager, ref, "bf16", "captured slot window")
    assert binding.device_status(DEV, clear=True) == 0


# --------------------------------------------------------------------------- #
# several new tokens (queries) per row
# --------------------------------------------------------------------------- #
def _multi_run(w, st, *, validate=True, out=None):
    binding.kv_write(st.k_new, st.v_new, st.slots, st.k_cache, st.v_cache, layout=w.layout,
                     validate=validate)
    got = binding.paged_attention_multi(st.q, st.k_cache, st.v_cache, st.tables, st.lens,
                                        w.scale, layout=w.layout, out=out, validate=validate)
    torch.cuda.synchronize()
    return got


def _multi_oracle(w, k_host, v_host):
    kw, vw = k_host.copy(), v_host.copy()
    oracle.kv_write(kw, vw, w.k_new, w.v_new, w.slot_mapping, num_blocks=w.num_blocks,
                    block_size=w.block_size, layout=w.layout, dtype=w.dtype)
    return oracle.paged_attention_multi(w.q, kw, vw, w.block_tables, w.context_lens, w.scale,
                                        num_blocks=w.num_blocks, block_size=w.block_size,
                                        layout=w.layout, dtype=w.dtype)


MULTI_CASES = [
    # name, lens, query_len, heads, kv_heads, head_dim, block_size, dtype, layout
    ("q2-f32", [16, 40, 0, 130], 2, 4, 4, 64, 16, "f32", "HND"),
    ("q4-gqa4-bf16", [4, 300, 1025, 2050, 0, 77], 4, 16, 4, 128, 16, "bf16", "HND"),
    ("q3-mha-nhd", [3, 50, 129, 700], 3, 8, 8, 128, 16, "bf16", "NHD"),
    ("q5-gqa2-bs32", [5, 64, 900], 5, 8, 4, 64, 32, "bf16", "HND"),
    ("q8-d256", [8, 200, 513], 8, 4, 2, 256, 16, "bf16", "HND"),
    ("q16-mha", [16, 600, 2100, 0], 16, 8, 8, 128, 16, "bf16", "HND"),
    ("q4-f32-d128", [4, 1000, 33], 4, 8, 2, 128, 16, "f32", "NHD"),
]


@pytest.mark.parametrize("chunk", [0, 32])
@pytest.mark.parametrize("case", MULTI_CASES, ids=[c[0] for c in MULTI_CASES])
def test_multi_token_rows(case, chunk):
    """Several new tokens per row, each attending causally: every output against the
    oracle, the written slots bit-exact.  chunk=32 pins 32-token chunks, so causal
    limits fall inside and before split chunks."""
    name, lens, n_q, heads, kvh, d, bs, dtype, layout = case
    w = wl.make_custom(lens, heads=heads, kv_heads=kvh, head_dim=d, block_size=bs,
                       dtype=dtype, layout=layout, query_len=n_q,
                       seed=zlib.crc32(name.encode()))
    say(f"multi {name} chunk {chunk}: lens {lens} q {n_q} heads {heads}/{kvh}")
    saved = binding.get_tuning()
    if chunk:
        binding.set_tuning(chunk_min=chunk, chunk_max=chunk)
    try:
        st = Step(w, host_history=True)
        got = _multi_run(w, st)
    finally:
        binding.set_tuning(**saved)
    ref = _multi_oracle(w, st.k_host, st.v_host)
    assert_close(to_host(got, dtype), ref, dtype, name)
    assert binding.device_status(DEV, clear=True) == 0


def test_one_query_per_row_is_the_decode_read():
    w = wl.make_config(3)
    st = Step(w)
    blk = to_host(st.run(validate=False), "bf16").copy()
    got = binding.paged_attention_multi(st.q[:, None], st.k_cache, st.v_cache, st.tables,
                                        st.lens, w.scale)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(got[:, 0], "bf16"), blk)


def test_multi_refusals_touch_nothing():
    w = wl.make_custom([16, 40], heads=4, kv_heads=4, head_dim=64, dtype="f32",
                       query_len=4, seed=3)
    st = Step(w, host_history=True)
    out = torch.full_like(st.q, 2.0)
    lens = st.lens.clone()
    lens[0] = 3
    with pytest.raises(binding.PagedKVError, match="CONTEXT_BOUNDS"):
        binding.paged_attention_multi(st.q, st.k_cache, st.v_cache, st.tables, lens,
                                      w.scale, out=out)
    with pytest.raises(binding.PagedKVError, match="SHAPE"):
        binding.paged_attention_multi(st.q[:, 0], st.k_cache, st.v_cache, st.tables,
                                      st.lens, w.scale)
    torch.cuda.synchronize()
    assert torch.all(out == 2.0)


def test_config5_with_four_new_tokens_every_row():
    """The full-width batch with four new tokens per row (a speculative-decoding step
    of three drafts)."""
    _full_size(5, query_len=4)


# --------------------------------------------------------------------------- #
# the matrix-core fold (4, 8 or 16 query vectors per KV head, bfloat16, d 64/128)
# --------------------------------------------------------------------------- #
MFMA_CASES = [
    # name, lens, query_len, heads, kv_heads, head_dim, layout
    ("gqa4-d128", [9, 300, 0, 1500, 33], 1, 16, 4, 128, "HND"),
    ("q4-mha-d64", [4, 77, 2049, 500], 4, 4, 4, 64, "NHD"),
    ("gqa8-d128", [1, 17, 0, 300, 1025, 2050, 64], 1, 32, 4, 128, "HND"),
    ("gqa16-d128-nhd", [5, 700, 129, 0, 2000], 1, 32, 2, 128, "NHD"),
    ("gqa16-d64", [33, 1, 900, 16], 1, 16, 1, 64, "HND"),
    ("q4-gqa4", [4, 90, 1500, 0, 77], 4, 8, 2, 128, "HND"),
    ("q8-mha-d64-nhd", [8, 300, 31, 1100], 8, 4, 4, 64, "NHD"),
    ("q16-mha", [16, 600, 2100], 16, 4, 4, 128, "HND"),
    ("q2-gqa8", [2, 40, 513], 2, 32, 4, 128, "HND"),
]


@pytest.mark.parametrize("mfma", [1, 2])
@pytest.mark.parametrize("chunk", [0, 32])
@pytest.mark.parametrize("case", MFMA_CASES, ids=[c[0] for c in MFMA_CASES])
def test_matrix_core_groups(case, chunk, mfma):
    """Groups of 4, 8 or 16 query vectors per KV head on the matrix cores (mfma=1) and on
    the vector units (mfma=2), default and 32-token chunks: every output against the
    oracle."""
    name, lens, n_q, heads, kvh, d, layout = case
    w = wl.make_custom(lens, heads=heads, kv_heads=kvh, head_dim=d, dtype="bf16",
                       layout=layout, query_len=n_q, seed=zlib.crc32(name.encode()) + 5)
    say(f"matrix cores {name} chunk {chunk} mfma {mfma}")
    saved = binding.get_tuning()
    binding.set_tuning(chunk_min=chunk, chunk_max=chunk, mfma=mfma)
    try:
        st = Step(w, host_history=True)
        if n_q == 1:
            got = st.run()
        else:
            got = _multi_run(w, st)
    finally:
        binding.set_tuning(**saved)
    ref = _multi_oracle(w, st.k_host, st.v_host) if n_q > 1 else \
        oracle_full(w, st.k_host, st.v_host)[0]
    assert_close(to_host(got, "bf16"), ref, "bf16", name)
    assert binding.device_status(DEV, clear=True) == 0


# --------------------------------------------------------------------------- #
# many rows: the plan kernel walks the rows in several passes of 1024
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("rows,hi,dtype", [(4100, 64, "f32"), (65535, 16, "bf16")])
def test_many_rows(rows, hi, dtype):
    """Batches wider than the plan kernel's 1024 threads (its scans carry over from pass
    to pass), up to the largest supported batch; every output against the oracle."""
    rng = np.random.default_rng(rows)
    lens = rng.integers(0, hi + 1, rows)
    lens[rng.choice(rows, rows // 10, replace=False)] = 0
    w = wl.make_custom(lens.tolist(), heads=2, kv_heads=1, head_dim=64, dtype=dtype,
                       seed=rows)
    say(f"many rows: {rows} rows, lengths 0..{hi}, {int(lens.sum())} tokens")
    err = check_full(w)
    say(f"  max err {err:.3e}")


def test_many_rows_through_a_slot_window():
    rows = 3000
    rng = np.random.default_rng(8)
    lens = rng.integers(0, 200, rows)
    w = wl.make_custom(lens.tolist(), heads=2, kv_heads=2, head_dim=64, dtype="bf16", seed=8)
    width = w.max_blocks * w.block_size
    table = _block_table_rect(w, width, width + 3)
    table = _scatter_rows(w, table, list(range(0, rows, 97)), rng)
    st = Step(w, host_history=True)
    got = _slot_run(st, table, width)
    ref = _slot_oracle(w, st.k_host, st.v_host, table, width)
    assert_close(to_host(got, "bf16"), ref, "bf16", "3000-row slot window")


# --------------------------------------------------------------------------- #
# seeded random configurations: shapes and work splits drawn together
# --------------------------------------------------------------------------- #
def _random_case(seed):
    """One drawn configuration: a workload and a tuning, both seeded."""
    rng = np.random.default_rng(1000 + seed)
    dtype = ["bf16", "f32"][int(rng.integers(2))]
    d = [64, 128, 256][int(rng.integers(3))]
    bs = [16, 32, 64, 128, 256][int(rng.integers(5))]
    kvh = [1, 2, 4][int(rng.integers(3))]
    group = [1, 2, 4, 8][int(rng.integers(4))]
    n_q = [1, 1, 2, 4][int(rng.integers(4))]
    many = bool(rng.integers(4) == 0)     # enough short rows for the single-wave phase
    if many:
        lens = rng.integers(n_q, 200, 520 if group * n_q >= 4 else 560).tolist()
        kvh, group = 4, 1
    else:
        lens = rng.integers(0, 900, int(rng.integers(1, 12))).tolist()
        lens = [0 if x < n_q and x > 0 else x for x in lens]
    chunk_min = [32, 64, 128, 256][int(rng.integers(4))]
    tuning = dict(chunk_min=chunk_min,
                  chunk_max=min(8192, chunk_min * [1, 4, 16, 64][int(rng.integers(4))]),
                  decode_waves=[1, 2, 4, 8][int(rng.integers(4))],
                  staging=[1, 2][int(rng.integers(2))],
                  mfma=[1, 2][int(rng.integers(2))],
                  solo_tokens=[1, 64, 256, 1024][int(rng.integers(4))],
                  groups_per_cu=1 if many else [1, 2, 16][int(rng.integers(3))])
    # drawn after the rest, so that the draws above stay what they were
    tuning.update(deal=[1, 2][int(rng.integers(2))],
                  items_per_group=[1, 4, 16, 64][int(rng.integers(4))],
                  max_query_group=[16, 8, 4, 1][int(rng.integers(4))])
    return dict(context_lens=lens, heads=kvh * group, kv_heads=kvh, head_dim=d, block_size=bs,
                dtype=dtype, layout=["HND", "NHD"][int(rng.integers(2))], query_len=n_q,
                seed=seed), tuning


@pytest.mark.parametrize("seed", range(40))
def test_random_configurations(seed):
    """Drawn shapes (dtype, head_dim, block size, head grouping, new tokens per row,
    layout, lengths) under drawn work splits (chunk range, waves, staging, matrix cores,
    single-wave bound, workgroups per CU, static deal or all tickets, items per
    workgroup, query-group cap): every output against the oracle, the scatter
    bit-exact."""
    kw, tuning = _random_case(seed)
    w = wl.make_custom(**kw)
    say(f"random {seed}: rows {w.rows} heads {w.heads}/{w.kv_heads} d {w.head_dim} "
        f"bs {w.block_size} {w.dtype} {w.layout} q {w.query_len} {tuning}")
    before = binding.get_tuning()
    binding.set_tuning(**tuning)
    try:
        st = Step(w, host_history=True)
        got = st.run() if w.query_len == 1 else _multi_run(w, st)
    finally:
        binding.set_tuning(**before)
    assert binding.device_status(DEV, clear=True) == 0
    ref, kwp, vwp = _oracle_by_rows(w, st.k_host, st.v_host)
    assert_close(to_host(got, w.dtype), ref, w.dtype, f"random {seed}")
    ints = np.uint16 if w.dtype == "bf16" else np.uint32
    for dev_pool, want in ((st.k_cache, kwp), (st.v_cache, vwp)):
        assert np.array_equal(to_host(dev_pool, w.dtype)[:w.num_blocks].view(ints),
                              want[:w.num_blocks].view(ints))


@pytest.mark.parametrize("seed", range(12))
def test_random_slot_windows(seed):
    """Drawn shapes and work splits read through a slot window in which a drawn share of
    the live rows is scattered (token by token) and the rest block-structured: every
    output against the oracle."""
    kw, tuning = _random_case(500 + seed)
    kw["query_len"] = 1
    kw["context_lens"] = [max(x, 1) if x else 0 for x in kw["context_lens"]]
    rng = np.random.default_rng(600 + seed)
    w = wl.make_custom(num_blocks=sum(wl.cdiv(c, kw["block_size"])
                                      for c in kw["context_lens"]) + 40, **kw)
    width = w.max_blocks * w.block_size
    live = [r for r in range(w.rows) if w.context_lens[r] > 1]
    share = [0.3, 0.6, 1.0][seed % 3]
    scattered = sorted(rng.choice(live, int(round(share * len(live))), replace=False).tolist()) \
        if live else []
    table = _scatter_rows(w, _block_table_rect(w, width, width + 5), scattered, rng)
    say(f"random slots {seed}: rows {w.rows} scattered {len(scattered)} heads "
        f"{w.heads}/{w.kv_heads} d {w.head_dim} bs {w.block_size} {w.dtype} {w.layout} "
        f"{tuning}")
    st = Step(w, host_history=True)
    before = binding.get_tuning()
    binding.set_tuning(**tuning)
    try:
        got = _slot_run(st, table, width)
    finally:
        binding.set_tuning(**before)
    assert binding.device_status(DEV, clear=True) == 0
    ref = _oracle_by_rows(w, st.k_host, st.v_host, slot_rect=table[:, :width])[0]
    assert_close(to_host(got, w.dtype), ref, w.dtype, f"random slots {seed}")

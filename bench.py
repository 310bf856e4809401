#!/usr/bin/env python3
"""Throughput of one batched paged-attention decode step on one MI355X.

A step is the whole hot path over one batch: the slot scatter of every row's new K/V
(pad rows into the sink) followed by the paged attention read of every (row, head).
The default workload is the full-width decode batch: 256 rows (16 of them padding),
32 query heads = 32 KV heads, head_dim 128, block_size 16, bf16 K/V, table width 8192
tokens, lengths long-tail lognormal (median 1024, sigma 1.2) with 8 rows at 8192, and
a 131072-block pool (~34 GB of K+V).  Every input is resident in HBM before timing.

Prints one JSON line on stdout.  ``value`` is KV GB/s: the bytes of K and V the read
must stream (every live (row, KV head, position) once) divided by the wall-clock time
per step.  The step is timed twice over the same tensors: as the two library calls
per step (eager), and as replays of one HIP graph recorded from those calls (graph, the
default ``value``; ``--launch eager`` reports the other).  ``roofline`` reports the
decode kernel alone, timed with HIP events on its launch stream over a third pass of
the same library-call steps, against MI355X's 8 TB/s HBM peak, and beside the rate a
plain streaming read of the same byte count reaches on the same GPU (``achievable``)
and the best rate a plain read of exactly the decode's scattered pieces reaches over
every load shape of the gathering read (``achievable_gather``; ``--gather-sweep`` logs
each shape, and the same pieces sorted by address).
``cpu_baseline`` times the CPU oracle over the same batch (every row by default) on a
pool of host threads, one per core of the process's CPU affinity (at most 16); its
outputs check every GPU output row.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode paged-attn KV GB/s and % HBM peak; (row,head)/s at 256 rows × 8192"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published peak
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.json")
KERNEL_SOURCE = os.path.join(ROOT, "paged_attention_decode_kv_amd", "csrc", "kernels.hip")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=5, help="workload 1..5 (default 5)")
    ap.add_argument("--layout", default="HND", choices=["HND", "NHD"])
    ap.add_argument("--cpu-rows", type=int, default=0,
                    help="rows of the batch the CPU oracle runs (a seeded sample; 0: every "
                         "row)")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="host threads of the CPU oracle (0: the process's CPU affinity, "
                         "at most 16)")
    ap.add_argument("--chunk-min", type=int, default=0,
                    help="shortest decode work-item length in tokens (0: library default)")
    ap.add_argument("--chunk-max", type=int, default=0,
                    help="longest decode work-item length in tokens (0: library default)")
    ap.add_argument("--decode-waves", type=int, default=0,
                    help="waves per decode work item (0: library default)")
    ap.add_argument("--items-per-group", type=int, default=0,
                    help="work items per decode workgroup the plan aims for (0: default)")
    ap.add_argument("--deal", type=int, default=0,
                    help="1: deal full-chunk rounds statically, 2: queue every item")
    ap.add_argument("--staging", type=int, default=0,
                    help="1: K/V straight to registers, 2: through an LDS stage")
    ap.add_argument("--max-query-group", type=int, default=0,
                    help="query heads sharing one K/V load under GQA (0: default)")
    ap.add_argument("--mfma", type=int, default=0,
                    help="1: groups of 8 or 16 query vectors per KV head on the matrix "
                         "cores (library default), 2: always on the vector units")
    ap.add_argument("--groups-per-cu", type=int, default=0,
                    help="at most this many decode workgroups per compute unit")
    ap.add_argument("--solo-tokens", type=int, default=0,
                    help="chunks shorter than this are read by one wave each (1: none)")
    ap.add_argument("--kv-heads", type=int, default=0,
                    help="override the workload's KV heads (grouped-query variant)")
    ap.add_argument("--launch", default="graph", choices=["graph", "eager"],
                    help="graph (default): time the two library calls per step, then replays "
                         "of one HIP graph recorded from them, and report the replays as "
                         "value; eager: time and report the library calls only")
    ap.add_argument("--query-len", type=int, default=1,
                    help="new tokens (queries) per row: >1 runs the multi-token read "
                         "(speculative decoding's drafts) on the same lengths")
    ap.add_argument("--address", default="blocks", choices=["blocks", "slots"],
                    help="how the read is addressed: block tables (default), or the "
                         "per-token int64 slot window of a wider slot table")
    ap.add_argument("--scatter-rows", type=int, default=0,
                    help="with --address slots: shuffle the live cells of this many of "
                         "the longest rows among themselves (the same tokens, so the same "
                         "result, but no block structure: those rows take the "
                         "token-by-token kernel)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain elementwise kernel over 1 GiB (for counter scaling)")
    ap.add_argument("--gather-sweep", action="store_true",
                    help="log the gathering read's rate for every load shape, in the decode's "
                         "piece order and sorted by address")
    ap.add_argument("--flush-mb", type=int, default=0,
                    help="read a buffer of this many MB before each event-timed step, so that "
                         "the per-kernel times see no K/V left in the 256 MB MALL by the step "
                         "before (a read leaves no dirty lines to write back during the step; "
                         "the step-time loops are unchanged)")
    return ap.parse_args()


def kernel_source_hash():
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def traffic_per_launch(config_name, layout):
    """HBM bytes per decode launch from committed counter runs, if they were taken on
    the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            records = json.load(f).get("records", [])
    except (OSError, ValueError, AttributeError):
        return None
    src = kernel_source_hash()
    for rec in records:
        if (rec.get("kernel_source_sha256") == src and rec.get("workload") == config_name
                and rec.get("layout") == layout):
            return rec.get("bytes_per_launch")
    return None


MAX_ORACLE_THREADS = 16    # a one-GPU machine's share of its host's cores


def cpu_info():
    """Host CPUs as this process sees them: the model, the logical CPUs of the machine
    and those of the process's affinity."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"model": model, "cpu_count": os.cpu_count(),
            "affinity": len(os.sched_getaffinity(0))}


def _host(t, dtype):
    import numpy as np
    import torch
    if dtype == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def _row_groups(lens, rows, per_row, cells=1 << 23):
    """Rows sorted by length, cut into groups whose oracle rectangle (rows x longest
    length x per_row elements) stays within `cells` (a longer row goes alone)."""
    rows = sorted(rows, key=lambda r: int(lens[r]))
    groups, at = [], 0
    while at < len(rows):
        end = at + 1
        while end < len(rows) and (end + 1 - at) * max(1, int(lens[rows[end]])) * per_row <= cells:
            end += 1
        groups.append(rows[at:end])
        at = end
    return groups


def cpu_baseline(w, k_cache, v_cache, sample_rows=0, threads=0):
    """The oracle (kv_write + masked-rectangle read) over the batch's rows (every row,
    or a seeded sample of ``sample_rows``), in groups of rows of similar length on a pool
    of host threads (numpy releases the interpreter lock in its gathers, products and
    loops; BLAS is held to one thread per worker).  Runs on the pool before any GPU
    step touches it.  The host copies of each group's blocks are made first, untimed;
    the wall clock from the first group's start to the last group's end is the time.
    Returns the timing record and the oracle outputs of the rows it covered."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    import oracle
    from paged_attention_decode_kv_amd import workloads as wl

    info = cpu_info()
    n_threads = threads or max(1, min(MAX_ORACLE_THREADS, info["affinity"]))
    rows = list(range(w.rows))
    if sample_rows and sample_rows < w.rows:
        rows = sorted(np.random.default_rng(1234).permutation(w.rows)[:sample_rows].tolist())
    nq = w.query_len
    kv_shape = (w.rows, nq, w.kv_heads, w.head_dim)
    read = oracle.paged_attention if nq == 1 else oracle.paged_attention_multi
    groups = _row_groups(w.context_lens, rows, w.heads * w.head_dim * nq)
    jobs = []
    for part in groups:                     # host copies, untimed
        blocks = wl.live_blocks(w, part)
        remap = {int(b): i for i, b in enumerate(blocks)}
        n = len(blocks)
        idx = torch.from_numpy(np.append(blocks, w.num_blocks).astype(np.int64)).to(k_cache.device)
        kh = _host(k_cache.index_select(0, idx), w.dtype)
        vh = _host(v_cache.index_select(0, idx), w.dtype)
        bt = np.full((len(part), w.max_blocks), -1, dtype=np.int32)
        sm = np.empty(len(part) * nq, dtype=np.int64)
        for i, r in enumerate(part):
            live = wl.cdiv(w.context_lens[r], w.block_size)
            bt[i, :live] = [remap[int(b)] for b in w.block_tables[r, :live]]
            for j in range(nq):
                s = int(w.slot_mapping[r * nq + j])
                sm[i * nq + j] = (n * w.block_size if w.context_lens[r] == 0 else
                                  remap[s // w.block_size] * w.block_size + s % w.block_size)
        k_new = w.k_new.reshape(kv_shape)[part].reshape(-1, w.kv_heads, w.head_dim)
        v_new = w.v_new.reshape(kv_shape)[part].reshape(-1, w.kv_heads, w.head_dim)
        jobs.append((part, kh, vh, bt, sm, n, k_new, v_new))

    def compute(job):
        part, kh, vh, bt, sm, n, k_new, v_new = job
        oracle.kv_write(kh, vh, k_new, v_new, sm, num_blocks=n, block_size=w.block_size,
                        layout=w.layout, dtype=w.dtype)
        return read(w.q[part], kh, vh, bt, w.context_lens[part], w.scale, num_blocks=n,
                    block_size=w.block_size, layout=w.layout, dtype=w.dtype)

    with threadpool_limits(limits=1, user_api="blas"), ThreadPoolExecutor(n_threads) as ex:
        t0 = time.perf_counter()
        outs = list(ex.map(compute, jobs))
        spent = time.perf_counter() - t0
    done = [r for part in groups for r in part]
    lens = w.context_lens[done]
    elem = 2 if w.dtype == "bf16" else 4
    kv_bytes = int(lens.sum()) * w.kv_heads * w.head_dim * 2 * elem
    row_heads = int(np.count_nonzero(lens)) * w.heads
    rec = {
        "value": round(kv_bytes / spent / 1e9, 4),
        "unit": "GB/s",
        "cores": n_threads,
        "kind": "oracle",
        "sample": (f"{'every row' if len(done) == w.rows else f'{len(done)} seeded rows'} of "
                   f"the same batch ({len(done)} rows, {int(lens.sum())} tokens, {row_heads} "
                   f"live (row, head) pairs) in {len(groups)} row groups on {n_threads} host "
                   f"threads (BLAS 1 thread each), float64 numpy; {spent:.2f} s wall; "
                   f"{row_heads / spent:.1f} (row, head)/s"),
        "seconds": round(spent, 3),
        "row_heads_per_s": round(row_heads / spent, 3),
        "cpu": info,
    }
    return rec, np.array(done), np.concatenate(outs)


def achievable_read(nbytes, device, reps=5):
    """The best rate (GB/s) a plain streaming read of ``nbytes`` reaches on this GPU
    (pkv_stream_read, 1 to 8 workgroups of 256 threads per CU), each launch timed with
    events on the stream it runs on; returns (GB/s, workgroups per CU, microseconds)."""
    import torch

    from paged_attention_decode_kv_amd import binding

    nbytes = max(16, nbytes // 16 * 16)
    buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
    sink = torch.zeros(1, dtype=torch.int32, device=device)
    best = None
    for gpc in (1, 2, 4, 8):
        for _ in range(2):
            binding.stream_read(buf, sink, gpc)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * reps)]
        for i in range(reps):
            ev[2 * i].record()
            binding.stream_read(buf, sink, gpc)
            ev[2 * i + 1].record()
        torch.cuda.synchronize()
        us = min(ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(reps)) * 1e3
        if best is None or us < best[2]:
            best = (nbytes / us / 1e3, gpc, us)
    del buf, sink
    return best


def gather_offsets(w, rows=None, slot_rows=None):
    """Byte offsets of the pieces of K and V a decode read streams, in its order, with the
    piece size: (offsets, piece bytes), or None.
    * Block tables, HND pool: one (block, KV head) piece of block_size x head_dim
      elements per block and KV head, row by row, in groups of 8 blocks (a decode item's
      waves take one block each), every KV head of a group before the next group, so that
      concurrent waves read all heads' pieces (one head's pieces sit at the same offset of
      every block, and reading them alone leaves most HBM channels idle).
    * Block tables, NHD pool: a (block, KV head) is block_size separate token vectors, so
      each live token's head vector is a piece, in the same order.
    * ``slot_rows`` ({row: its live slots, in window order}): the rows read token by
      token; a piece per (row, KV head, token), in that order.
    ``rows`` limits the block-table rows (default: every row)."""
    import numpy as np

    from paged_attention_decode_kv_amd import workloads as wl

    elem = 2 if w.dtype == "bf16" else 4
    vec = w.head_dim * elem
    heads = np.arange(w.kv_heads, dtype=np.int64)

    def token_offset(slot, h):     # byte offset of (slot, KV head h) in either layout
        if w.layout == "NHD":
            return (slot * w.kv_heads + h) * vec
        blk, off = slot // w.block_size, slot % w.block_size
        return ((blk * w.kv_heads + h) * w.block_size + off) * vec

    offs = []
    if slot_rows is not None:
        for r, sl in slot_rows.items():
            sl = np.asarray(sl, dtype=np.int64)
            offs.append(token_offset(sl[None, :], heads[:, None]).reshape(-1))
        return (np.concatenate(offs), vec) if offs else None
    t_in = np.arange(w.block_size, dtype=np.int64)
    for r in (range(w.rows) if rows is None else rows):
        n = int(w.context_lens[r])
        nb = wl.cdiv(n, w.block_size)
        if nb == 0:
            continue
        blocks = w.block_tables[r, :nb].astype(np.int64)
        for g0 in range(0, nb, 8):
            grp = blocks[g0:g0 + 8]
            if w.layout == "HND":
                offs.append(((grp[None, :] * w.kv_heads + heads[:, None]) * w.block_size *
                             vec).reshape(-1))
            else:   # live tokens only: position g0 * block_size + j * block_size + t
                pos = (g0 + np.arange(len(grp), dtype=np.int64))[:, None] * w.block_size + t_in
                slot = grp[:, None] * w.block_size + t_in
                o = token_offset(slot[None, :, :], heads[:, None, None])
                offs.append(o[:, pos < n].reshape(-1))
    if not offs:
        return None
    return np.concatenate(offs), (w.block_size * vec if w.layout == "HND" else vec)


def gather_rates(pieces, reps=5):
    """Every (waves per workgroup, pieces per wave, workgroups per CU) of the gathering
    read over ``pieces``: a list of (GB/s, waves, pieces per wave, workgroups per CU,
    microseconds), fastest of ``reps`` launches each, timed with events on the stream the
    read runs on."""
    import torch

    from paged_attention_decode_kv_amd import binding

    sink = torch.zeros(1, dtype=torch.int32, device=pieces.k_cache.device)
    nbytes = pieces.offsets.numel() * pieces.piece_bytes * 2
    out = []
    for waves, ppw in binding.GATHER_SHAPES:
        for gpc in (1, 2, 4) if waves == 8 else (1, 2, 4, 8):
            def launch():
                binding.gather_read(pieces, sink, gpc, waves, ppw)
            for _ in range(2):
                launch()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * reps)]
            for i in range(reps):
                ev[2 * i].record()
                launch()
                ev[2 * i + 1].record()
            torch.cuda.synchronize()
            us = min(ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(reps)) * 1e3
            out.append((nbytes / us / 1e3, waves, ppw, gpc, us))
    del sink
    return out


def achievable_gather(w, k_cache, v_cache, sweep_log=None, rows=None, slot_rows=None):
    """The best rate (GB/s) a plain read of exactly the pieces of K and V the dominant
    kernel streams, in its order (gather_offsets), reaches over every load shape of
    pkv_gather_read (4 or 8 waves per workgroup, 1, 2 or 4 loads in flight per wave, 1 to
    8 workgroups per CU).  With ``sweep_log``, every shape's rate goes to it, and so do
    those of the same pieces sorted by address (a locality the decode's order does not
    have: context only).  Returns (GB/s, description, microseconds, bytes) or None."""
    import numpy as np

    from paged_attention_decode_kv_amd import binding

    got = gather_offsets(w, rows=rows, slot_rows=slot_rows)
    if got is None:
        return None
    offs, piece = got
    pieces = binding.GatherPieces(k_cache, v_cache, offs, piece)
    nbytes = offs.size * piece * 2
    rates = gather_rates(pieces)
    del pieces
    best = max(rates)
    if sweep_log:
        per = 1024 // piece if piece <= 1024 and 1024 % piece == 0 else 1
        sweep_log(f"gathering read of {nbytes} B in {offs.size} pieces of {piece} B "
                  f"(GB/s by waves per workgroup x loads in flight per wave, a load being "
                  f"{per} piece(s), and workgroups per CU):")
        orders = [("decode order", rates)]
        sorted_pieces = binding.GatherPieces(k_cache, v_cache, np.sort(offs), piece)
        orders.append(("sorted by address", gather_rates(sorted_pieces)))
        del sorted_pieces
        for name, rr in orders:
            for waves, ppw in binding.GATHER_SHAPES:
                cells = [f"{gpc}: {gbs:.0f}" for gbs, wv, pp, gpc, _ in rr
                         if (wv, pp) == (waves, ppw)]
                sweep_log(f"  {name}, {waves} waves x {ppw} pieces: " + ", ".join(cells))
            top = max(rr)
            sweep_log(f"  {name}: best {top[0]:.1f} GB/s ({top[1]} waves x {top[2]} pieces, "
                      f"{top[3]} workgroups per CU)")
    kern = "gather_small_kernel" if piece <= 1024 and 1024 % piece == 0 else "gather_read_kernel"
    loads = (f"{best[2]} loads of {1024 // piece} pieces a wave" if kern == "gather_small_kernel"
             else f"{best[2]} pieces a wave")
    desc = (f"{kern}, {best[3]} x {best[1]}-wave workgroups per CU, {loads}, best of "
            f"{len(rates)} shapes, {nbytes} B in pieces of {piece} B")
    return best[0], desc, best[4], nbytes


def check_outputs(out, rows, ref, dtype):
    """GPU outputs of the sampled rows against the oracle's (same tolerances as the
    parity tests: 2e-6 for float32, 2e-2 and 2^-8 relative + 2e-5 for bfloat16)."""
    import numpy as np
    import torch

    got = out[torch.from_numpy(rows).to(out.device)].float().cpu().numpy().astype(np.float64)
    err = np.abs(got - ref)
    if dtype == "f32":
        ok = bool(err.max() <= 2e-6)
    else:
        ok = bool(err.max() <= 2e-2 and np.all(err <= 2.0 ** -8 * np.abs(ref) + 2e-5))
    return {"rows": int(len(rows)), "max_abs_err": float(err.max()), "ok": ok}


class _CallerGraph:
    """A step whose library calls are recorded by torch's stream capture (the calls are
    capturable with validate off), replayed like the library's own captured steps."""

    def __init__(self, step, torch):
        self._g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self._g):
            step()

    def launch(self):
        self._g.replay()

    def destroy(self):
        self._g = None


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the decode step is built and timed on a "
              "single MI355X; run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from paged_attention_decode_kv_amd import accounting as acc
    from paged_attention_decode_kv_amd import binding
    from paged_attention_decode_kv_amd import workloads as wl
    from paged_attention_decode_kv_amd import _capi

    if not os.path.exists(_capi.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    binding.set_tuning(args.chunk_min, args.chunk_max, args.decode_waves,
                       args.items_per_group, args.deal, args.staging, args.max_query_group,
                       args.mfma, args.groups_per_cu, args.solo_tokens)
    tuning = binding.get_tuning()
    if args.query_len > 1 and args.address != "blocks":
        raise SystemExit("--query-len > 1 reads through block tables only")
    w = wl.make_config(args.config, layout=args.layout, kv_heads=args.kv_heads or None,
                       query_len=args.query_len)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}[w.dtype]
    log(f"workload {w.name}: rows={w.rows} heads={w.heads} d={w.head_dim} bs={w.block_size} "
        f"{w.dtype} {w.layout}; pool {w.pool_bytes / 1e9:.2f} GB; "
        f"tokens {int(w.context_lens.sum())}")

    def dev_array(a, dtype=None):
        a = np.ascontiguousarray(a)
        if dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    k_cache = torch.empty(w.pool_shape, dtype=tdt, device=dev)
    v_cache = torch.empty_like(k_cache)
    wl.history_device(w, k_cache, v_cache)
    q = dev_array(w.q, w.dtype)
    k_new = dev_array(w.k_new, w.dtype)
    v_new = dev_array(w.v_new, w.dtype)
    slots = dev_array(w.slot_mapping)
    tables = dev_array(w.block_tables)
    lens = dev_array(w.context_lens)
    out = torch.empty_like(q)
    width = w.max_blocks * w.block_size
    slot_win = None
    scattered = [] if args.address != "slots" else \
        np.argsort(-w.context_lens, kind="stable")[:args.scatter_rows].tolist()
    if args.address == "slots":
        # the slot table a serving loop keeps: [rows, width + 64] int64, each row's live
        # positions holding block id * block size + offset of the same placement, junk
        # (-1) elsewhere; the read gets its first `width` columns as a window
        t = torch.arange(width, device=dev)
        cells = tables.long().clamp_min(0)[:, t // w.block_size] * w.block_size + \
            t % w.block_size
        slot_table = torch.full((w.rows, width + 64), -1, dtype=torch.int64, device=dev)
        slot_table[:, :width] = torch.where(t[None, :] < lens[:, None].long(), cells, -1)
        if args.scatter_rows:
            gen = torch.Generator(device=dev).manual_seed(99)
            for r in scattered:
                n = int(w.context_lens[r])
                perm = torch.randperm(n, generator=gen, device=dev)
                slot_table[r, :n] = slot_table[r, :n][perm]
        slot_win = slot_table[:, :width]
        del t, cells
        ws_bytes = binding.workspace_bytes_slots(k_cache, w.rows, w.heads, width, w.layout)
    elif w.query_len > 1:
        ws_bytes = binding.workspace_bytes_multi(k_cache, w.rows, w.query_len, w.heads,
                                                 w.max_blocks, w.layout)
    else:
        ws_bytes = binding.workspace_bytes(k_cache, w.rows, w.heads, w.max_blocks, w.layout)
    ws = torch.empty(max(1, ws_bytes), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    # the CPU oracle runs first, on the untouched pool: its timing is the baseline and
    # its outputs check the GPU step's outputs afterwards
    if args.no_cpu_baseline:   # the oracle still checks a few rows
        sample = min(w.rows, 8)
    else:
        sample = args.cpu_rows
    log(f"cpu oracle on {sample or 'every'} row(s) of the batch")
    base_rec, check_rows, check_ref = cpu_baseline(w, k_cache, v_cache, sample,
                                                   args.cpu_threads)
    log(f"cpu oracle: {base_rec['sample']}")

    def step(validate=False):
        binding.kv_write(k_new, v_new, slots, k_cache, v_cache, layout=w.layout,
                         validate=validate)
        if slot_win is not None:
            binding.paged_attention_slots(q, k_cache, v_cache, slot_win, lens, w.scale,
                                          layout=w.layout, out=out, workspace=ws,
                                          validate=validate)
        elif w.query_len > 1:
            binding.paged_attention_multi(q, k_cache, v_cache, tables, lens, w.scale,
                                          layout=w.layout, out=out, workspace=ws,
                                          validate=validate)
        else:
            binding.paged_attention(q, k_cache, v_cache, tables, lens, w.scale,
                                    layout=w.layout, out=out, workspace=ws,
                                    validate=validate)

    # one validated step: the library checks every length, block id and slot on the host
    step(validate=True)
    binding.device_status(dev, clear=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # K library-call steps as a caller makes them, with nothing recorded between kernels
    torch.cuda.synchronize()            # barrier: one process, one GPU
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    eager_s = (t1 - t0) / args.steps

    # the same step recorded once into a HIP graph over the same tensors, then replayed:
    # identical kernels and arguments, without a host launch per kernel.  Timed before
    # the event-timed loop: for a few ms after hundreds of event pairs, replays of a
    # small step run up to 1.5x slower
    graph_s = None
    if args.launch == "graph":
        if slot_win is not None:
            graph = binding.capture_step_slots(k_new, v_new, slots, q, k_cache, v_cache,
                                               slot_win, lens, w.scale, out, ws,
                                               layout=w.layout)
        elif w.query_len > 1:
            graph = _CallerGraph(step, torch)     # the calls captured on a side stream
        else:
            graph = binding.capture_step(k_new, v_new, slots, q, k_cache, v_cache, tables,
                                         lens, w.scale, out, ws, layout=w.layout)
        for _ in range(args.warmup):
            graph.launch()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            graph.launch()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        graph_s = (t1 - t0) / args.steps
        graph.destroy()

    # the same K steps again with a HIP event pair around every kernel, on the stream it
    # runs on: the per-kernel averages (the events add ~10 us of idle time per kernel
    # boundary, so this loop's wall clock is reported but is not the step time)
    flush = (torch.ones(args.flush_mb << 18, dtype=torch.float32, device=dev)
             if args.flush_mb > 0 else None)
    sink = torch.empty((), dtype=torch.float32, device=dev)
    binding.timing_enable(True)
    for ph in _capi.PHASES:
        binding.timing_read(ph, reset=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if flush is not None:
            torch.sum(flush, dim=0, out=sink)   # outside the library's event pairs
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    phases = {ph: binding.timing_read(ph, reset=True) for ph in _capi.PHASES}
    binding.timing_enable(False)
    event_s = (t1 - t0) / args.steps
    del flush, sink

    flags = binding.device_status(dev, clear=True)
    if flags:
        raise SystemExit(f"kernels clamped or skipped inputs (status bits {flags}); "
                         "the measurement is invalid")
    log(f"step: eager {eager_s * 1e3:.4f} ms" +
        (f", graph replay {graph_s * 1e3:.4f} ms" if graph_s else ""))

    if args.copy_calibration:
        # an elementwise kernel that reads 1 GiB and writes 1 GiB (torch's vectorized
        # multiply): the known-size reference for the HBM byte counters
        a = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            torch.mul(a, 1.0, out=b)
        torch.cuda.synchronize()
        log("ran 3 elementwise multiplies over 1 GiB (1073741824 B read + written each)")
        del a, b

    step_s = graph_s if args.launch == "graph" else eager_s
    elem = 2 if w.dtype == "bf16" else 4
    shape = dict(heads=w.heads, kv_heads=w.kv_heads, head_dim=w.head_dim,
                 block_size=w.block_size, elem=elem, write_tokens=w.rows * w.query_len,
                 query_len=w.query_len)
    b = acc.algorithmic_bytes(w.context_lens, address=args.address, **shape)
    # the decode kernel reads block ids in both modes (with slots, the table the
    # translation pass derived from the window); rows whose slots were scattered are
    # read by the token-by-token kernel instead, which reads their slot cells
    reg_lens = w.context_lens.copy()
    reg_lens[scattered] = 0
    dec_bytes = acc.algorithmic_bytes(reg_lens, **shape)["attention"]
    rh = acc.row_heads(w.context_lens, w.heads)
    avg = {ph: (ms / n if n else None) for ph, (ms, n) in phases.items()}
    for ph, (ms, n) in phases.items():
        if n:
            log(f"  {ph:9s} {n:5d} launches, avg {ms / n * 1e3:9.2f} us")
    dec_s = avg["decode"] * 1e-3
    kernel, kern_s, kern_bytes = (binding.decode_kernel_for(k_cache, w.heads, w.query_len,
                                                            w.layout), dec_s, dec_bytes)
    traffic = traffic_per_launch(w.name, w.layout)
    # the plan of the last step (every step plans the same batch): chunk length,
    # workgroups taking part, entries, split rows
    plan = binding.plan_info(ws)
    if scattered and avg.get("token_rows"):
        tok_lens = np.zeros_like(w.context_lens)
        tok_lens[scattered] = w.context_lens[scattered]
        tok_s = avg["token_rows"] * 1e-3
        if tok_s > dec_s:   # the dominant kernel is the token-by-token one
            kernel, kern_s = "token_rows_kernel", tok_s
            kern_bytes = acc.algorithmic_bytes(tok_lens, address="slots", **shape)["attention"]
        traffic = None        # the committed counters are for the unscattered batch
    achieved = kern_bytes / kern_s / 1e9
    ach_gbps, ach_gpc, ach_us = achievable_read(kern_bytes, dev)
    log(f"streaming read of {kern_bytes} B: {ach_us:.2f} us at {ach_gpc} workgroups/CU, "
        f"{ach_gbps:.1f} GB/s")
    # the reference read takes the dominant kernel's pieces: the rows read token by token
    # (their live slots, in window order) or the rows read through block tables
    sweep = log if args.gather_sweep else None
    if kernel == "token_rows_kernel":
        win = slot_win[scattered].cpu().numpy()
        slot_rows = {r: win[i, :int(w.context_lens[r])] for i, r in enumerate(scattered)}
        gather = achievable_gather(w, k_cache, v_cache, sweep, slot_rows=slot_rows)
    else:
        gather = achievable_gather(w, k_cache, v_cache, sweep,
                                   rows=[r for r in range(w.rows) if r not in set(scattered)])
    if gather:
        log(f"gathering read of the dominant kernel's {gather[3]} B of pieces: "
            f"{gather[2]:.2f} us, {gather[0]:.1f} GB/s ({gather[1]})")
    roofline = {
        "bound": "hbm",
        "achieved": round(achieved, 2),
        "peak": HBM_PEAK_GBPS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBPS, 4),
        "traffic": traffic,
        "kernel": kernel,
        "kernel_avg_us": round(kern_s * 1e6, 2),
        "bytes_per_launch": kern_bytes,
        # a plain streaming read of the same byte count on this GPU (best of 1-8
        # workgroups/CU, fastest of 5 launches): the rate a kernel that only reads reaches
        "achievable": round(ach_gbps, 2),
        "achievable_kernel": f"stream_read_kernel, {ach_gpc} x 256-thread workgroups per CU",
        "frac_of_achievable": round(achieved / ach_gbps, 4),
        # the same for a plain read of exactly the pieces the dominant kernel reads, in
        # its order: the best of every load shape
        "achievable_gather": round(gather[0], 2) if gather else None,
        "achievable_gather_kernel": gather[1] if gather else None,
        "frac_of_gather": round(achieved / gather[0], 4) if gather else None,
    }
    result = {
        "metric": METRIC,
        "value": round(b["kv"] / step_s / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": (f"{w.name} decode step: {w.rows} rows ({len(w.pad_rows)} padding) x "
                         f"{w.heads} heads x head_dim {w.head_dim}, {w.dtype} KV, block "
                         f"{w.block_size}, table width {w.max_blocks * w.block_size}, "
                         f"{int(w.context_lens.sum())} live tokens; kv_write + "
                         + ("paged_attention" if args.address == "blocks" else
                            "paged_attention_slots through a [rows, width] int64 slot "
                            "window")),
            "address": args.address,
            "scattered_rows": args.scatter_rows,
            "query_len": w.query_len,
            "rows": w.rows,
            "heads": w.heads,
            "kv_heads": w.kv_heads,
            "head_dim": w.head_dim,
            "block_size": w.block_size,
            "width": w.max_blocks * w.block_size,
            "layout": w.layout,
            "tuning": tuning,
            "launch": args.launch,
            "parallelism": "single GPU",
        },
        "eager_ms_per_step": round(eager_s * 1e3, 4),
        "event_timed_ms_per_step": round(event_s * 1e3, 4),
        "flush_mb_before_event_timed_steps": args.flush_mb,
        "graph_ms_per_step": round(graph_s * 1e3, 4) if graph_s else None,
        "hbm_frac": round(b["total"] / step_s / 1e9 / HBM_PEAK_GBPS, 4),
        "total_algorithmic_GBps": round(b["total"] / step_s / 1e9, 2),
        "row_heads_per_s": round(rh / step_s, 1),
        "phase_avg_us": {ph: (round(v * 1e3, 2) if v is not None else None)
                         for ph, v in avg.items()},
        "algorithmic_bytes": b,
        "plan": {k: plan[k] for k in ("chunk_tokens", "decode_groups", "entries",
                                      "full_chunks", "split_rows", "records",
                                      "record_capacity", "token_rows")},
        "roofline": roofline,
    }
    result["cpu_baseline"] = None if args.no_cpu_baseline else base_rec
    result["check"] = check_outputs(out, check_rows, check_ref, w.dtype)
    print(json.dumps(result), flush=True)
    if not result["check"]["ok"]:
        raise SystemExit(f"GPU outputs disagree with the oracle: {result['check']}")


if __name__ == "__main__":
    main()

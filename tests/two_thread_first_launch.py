"""Helper of test_first_launches_from_two_host_threads (run in a fresh process, so that
these are the process's first launches): two host threads, each on its own stream, make
their first decode steps at the same moment, one through the vector units and one
through the matrix cores, plus a third shape shared by both; every output is compared
with the oracle.  Prints OK and exits 0 on success."""

import os
import sys
import threading

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import oracle  # noqa: E402
from paged_attention_decode_kv_amd import binding  # noqa: E402
from paged_attention_decode_kv_amd import workloads as wl  # noqa: E402

DEV = torch.device("cuda", 0)


def to_dev(a, bf16):
    a = np.ascontiguousarray(a)
    t = torch.from_numpy(a.view(np.int16) if bf16 else a).to(DEV)
    return t.view(torch.bfloat16) if bf16 else t


def run(w, barrier, results, key):
    bf = w.dtype == "bf16"
    k_host, v_host = wl.history_host(w)
    stream = torch.cuda.Stream(device=DEV)
    with torch.cuda.stream(stream):
        k, v = to_dev(k_host, bf), to_dev(v_host, bf)
        args = [to_dev(w.q, bf), to_dev(w.k_new, bf), to_dev(w.v_new, bf),
                to_dev(w.slot_mapping, False), to_dev(w.block_tables, False),
                to_dev(w.context_lens, False)]
        stream.synchronize()
        barrier.wait()   # both threads launch their first kernels together
        q, kn, vn, sm, bt, ln = args
        binding.kv_write(kn, vn, sm, k, v, layout=w.layout, validate=False)
        out = binding.paged_attention(q, k, v, bt, ln, w.scale, layout=w.layout, validate=False)
        stream.synchronize()
    got = out.view(torch.int16).cpu().numpy().view(np.uint16) if bf else out.cpu().numpy()
    kw, vw = k_host.copy(), v_host.copy()
    oracle.kv_write(kw, vw, w.k_new, w.v_new, w.slot_mapping, num_blocks=w.num_blocks,
                    block_size=w.block_size, layout=w.layout, dtype=w.dtype)
    ref = oracle.paged_attention(w.q, kw, vw, w.block_tables, w.context_lens, w.scale,
                                 num_blocks=w.num_blocks, block_size=w.block_size,
                                 layout=w.layout, dtype=w.dtype)
    err = np.abs(oracle.decode_storage(got, w.dtype) - ref)
    if w.dtype == "f32":
        ok = err.max() <= 2e-6
    else:
        ok = err.max() <= 2e-2 and bool(np.all(err <= 2.0 ** -8 * np.abs(ref) + 2e-5))
    results[key] = (bool(ok), float(err.max()))


def main():
    cases = {
        "vector": wl.make_custom([700, 40, 0, 1500, 33], heads=8, kv_heads=8, head_dim=128,
                                 dtype="bf16", seed=71),
        "matrix": wl.make_custom([900, 17, 2100, 0, 64], heads=32, kv_heads=2, head_dim=128,
                                 dtype="bf16", seed=72),
        "f32": wl.make_custom([100, 300, 5], heads=4, kv_heads=4, head_dim=64, dtype="f32",
                              seed=73),
    }
    for round_ in (("vector", "matrix"), ("f32", "f32")):
        barrier = threading.Barrier(2)
        results = {}
        threads = [threading.Thread(target=run, args=(cases[c], barrier, results, f"{c}{i}"))
                   for i, c in enumerate(round_)]
        for t in threads:
            t.start()
        for t in threads:
            t.join()
        print(f"round {round_}: {results}", flush=True)
        if len(results) != 2 or not all(ok for ok, _ in results.values()):
            sys.exit(1)
    print("OK", flush=True)


if __name__ == "__main__":
    main()

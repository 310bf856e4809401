"""The entry point that allocates nothing (pkv_paged_attention_noalloc, the read in the
library's static scratch) against pkv_paged_attention with a workspace of its own: two
calls in a row through the C ABI, the second with a smaller batch, each bit-identical
to the workspace call and within the oracle's tolerance."""

import numpy as np
import pytest
import torch

import oracle
from paged_attention_decode_kv_amd import _capi, binding
from paged_attention_decode_kv_amd import workloads as wl

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)
TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


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


def _run_both(w):
    """kv_write, then the read with a workspace and the read in the static scratch;
    returns both outputs (storage arrays) and the oracle's."""
    say(f"no-alloc: rows={w.rows} heads={w.heads}/{w.kv_heads} d={w.head_dim} {w.dtype} "
        f"lens={w.context_lens.tolist()[:10]}")
    k_host, v_host = wl.history_host(w)
    k_cache, v_cache = to_dev(k_host, w.dtype), to_dev(v_host, w.dtype)
    q, tables, lens = to_dev(w.q, w.dtype), to_dev(w.block_tables), to_dev(w.context_lens)
    binding.kv_write(to_dev(w.k_new, w.dtype), to_dev(w.v_new, w.dtype),
                     to_dev(w.slot_mapping), k_cache, v_cache, layout=w.layout)
    need = binding.workspace_bytes(k_cache, w.rows, w.heads, w.max_blocks, w.layout)
    assert 0 < need <= _capi.NOALLOC_SCRATCH_BYTES
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    ref_out = binding.paged_attention(q, k_cache, v_cache, tables, lens, w.scale,
                                      layout=w.layout, workspace=ws, validate=True)
    out = torch.full_like(q, 3.0)
    binding.device_status(DEV, clear=True)
    got = binding.paged_attention_noalloc(q, k_cache, v_cache, tables, lens, w.scale, out,
                                          layout=w.layout)
    torch.cuda.synchronize()
    assert got.data_ptr() == out.data_ptr()
    assert binding.device_status(DEV, clear=True) == 0
    kw, vw = k_host.copy(), v_host.copy()
    oracle.kv_write(kw, vw, w.k_new, w.v_new, w.slot_mapping, num_blocks=w.num_blocks,
                    block_size=w.block_size, layout=w.layout, dtype=w.dtype)
    ref = oracle.paged_attention(w.q, kw, vw, w.block_tables, w.context_lens, w.scale,
                                 num_blocks=w.num_blocks, block_size=w.block_size,
                                 layout=w.layout, dtype=w.dtype)
    return to_host(out, w.dtype), to_host(ref_out, w.dtype), ref


def _assert_oracle(got, ref, dtype):
    g = oracle.decode_storage(got, dtype)
    err = np.abs(g - ref)
    if dtype == "f32":
        assert err.max() <= 2e-6, err.max()
    else:
        assert err.max() <= 2e-2, err.max()
        assert np.all(err <= 2.0 ** -8 * np.abs(ref) + 2e-5)
    return float(err.max())


def test_no_alloc_read_matches_the_workspace_read_twice():
    rng = np.random.default_rng(31)
    # first call: rows long enough to split into chunks (partial records in the scratch),
    # grouped heads, padding rows
    lens1 = rng.integers(1, 5000, 22).tolist() + [0, 8192, 0, 4096]
    w1 = wl.make_custom(lens1, heads=16, kv_heads=4, head_dim=128, dtype="bf16",
                        layout="HND", max_blocks=512, seed=41)
    # second call: a smaller batch of another shape, over the scratch the first left
    lens2 = [1, 300, 17, 0, 1000, 64]
    w2 = wl.make_custom(lens2, heads=8, kv_heads=8, head_dim=64, dtype="f32", layout="NHD",
                        max_blocks=64, seed=42)
    for w in (w1, w2):
        got, want, ref = _run_both(w)
        assert np.array_equal(got, want), "the scratch read differs from the workspace read"
        err = _assert_oracle(got, ref, w.dtype)
        pads = w.context_lens == 0
        assert np.all(got[pads] == 0)
        say(f"no-alloc: bit-identical to the workspace call, max err {err:.3e}")


def _named_step(idx):
    """A named configuration's pools (built on the device), after its kv_write; returns
    the read's tensors."""
    w = wl.make_config(idx)
    k_cache = torch.empty(w.pool_shape, dtype=TORCH_DT[w.dtype], device=DEV)
    v_cache = torch.empty_like(k_cache)
    wl.history_device(w, k_cache, v_cache)
    binding.kv_write(to_dev(w.k_new, w.dtype), to_dev(w.v_new, w.dtype),
                     to_dev(w.slot_mapping), k_cache, v_cache, layout=w.layout)
    return (w, to_dev(w.q, w.dtype), k_cache, v_cache, to_dev(w.block_tables),
            to_dev(w.context_lens))


def test_no_alloc_at_the_full_width_step():
    """The full-width batch (256 rows of up to 8192 tokens, 34 GB of pools; its
    workspace is about 17 MB, inside the scratch) read both ways: bit-identical.  Then a
    smaller batch (8 rows of 2048, every row split) over the scratch the first call
    left: bit-identical again."""
    for idx in (5, 2):
        w, q, k_cache, v_cache, tables, lens = _named_step(idx)
        need = binding.workspace_bytes(k_cache, w.rows, w.heads, w.max_blocks, w.layout)
        assert 0 < need <= _capi.NOALLOC_SCRATCH_BYTES
        say(f"no-alloc, config {idx}: workspace {need} bytes")
        ws = torch.empty(need, dtype=torch.uint8, device=DEV)
        want = binding.paged_attention(q, k_cache, v_cache, tables, lens, w.scale,
                                       layout=w.layout, workspace=ws, validate=True)
        out = torch.full_like(q, 3.0)
        binding.device_status(DEV, clear=True)
        binding.paged_attention_noalloc(q, k_cache, v_cache, tables, lens, w.scale, out,
                                        layout=w.layout)
        torch.cuda.synchronize()
        assert binding.device_status(DEV, clear=True) == 0
        assert torch.equal(out.view(torch.int16), want.view(torch.int16)), \
            f"config {idx}: the scratch read differs from the workspace read"
        pads = torch.from_numpy(w.pad_rows).to(DEV)
        assert torch.all(out[pads] == 0)
        say(f"no-alloc, config {idx}: bit-identical to the workspace read")
        del k_cache, v_cache, ws
        torch.cuda.empty_cache()


def test_no_alloc_refuses_a_batch_larger_than_the_scratch():
    """A batch whose workspace exceeds the scratch is refused before anything runs."""
    w = wl.make_custom([8192] * 2, heads=32, kv_heads=32, head_dim=256, dtype="bf16",
                       num_blocks=1024, max_blocks=2048, seed=43)
    k = torch.zeros((w.num_blocks + 1, w.kv_heads, w.block_size, w.head_dim),
                    dtype=torch.bfloat16, device=DEV)
    q = to_dev(w.q, w.dtype)
    rows = 1200   # many rows of a 32768-token table: every row splits at any chunk
    q = q[:1].expand(rows, -1, -1).contiguous()
    tables = torch.zeros((rows, 2048), dtype=torch.int32, device=DEV)
    lens = torch.zeros(rows, dtype=torch.int32, device=DEV)
    need = binding.workspace_bytes(k, rows, w.heads, 2048)
    assert need > _capi.NOALLOC_SCRATCH_BYTES
    out = torch.full_like(q, 5.0)
    with pytest.raises(binding.PagedKVError) as e:
        binding.paged_attention_noalloc(q, k, k, tables, lens, w.scale, out)
    assert e.value.code == "WORKSPACE"
    torch.cuda.synchronize()
    assert torch.all(out == 5.0)

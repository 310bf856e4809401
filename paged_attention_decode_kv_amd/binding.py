"""Python face of libpagedkv.so: torch tensors in, device pointers and sizes out.

Argument marshalling only.  Every step of the decode path runs in the library's HIP
kernels; this module checks tensor types and shapes, turns them into the C ABI's
plain pointers and sizes, and raises ``PagedKVError`` on any status but OK.  There is
no CPU fallback: without the built library every call raises.
"""

from __future__ import annotations

import ctypes

import numpy as np
import torch

from . import _capi

_DTYPES = {torch.float32: _capi.F32, torch.bfloat16: _capi.BF16}


class PagedKVError(ValueError):
    """A refusal or failure of the library; ``code`` is the status name."""

    def __init__(self, code: str, detail: str):
        super().__init__(f"{code}: {detail}")
        self.code = code
        self.detail = detail


def _raise(code: str, detail: str):
    raise PagedKVError(code, detail)


def _check(status: int):
    if status != 0:
        lib = _capi.lib()
        name = _capi.STATUS_NAMES[status] if status < len(_capi.STATUS_NAMES) else str(status)
        _raise(name, lib.pkv_last_error_detail().decode())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t: torch.Tensor):
    return ctypes.c_void_p(t.data_ptr())


def pool_desc(k_cache: torch.Tensor, layout: str = "HND") -> _capi.PoolDesc:
    """Descriptor of a pool tensor: HND ``[NB+1, Hkv, BS, D]`` or NHD ``[NB+1, BS, Hkv, D]``."""
    if layout not in _capi.LAYOUT_CODES:
        _raise("SHAPE", f"unknown layout {layout!r}")
    if k_cache.dtype not in _DTYPES:
        _raise("DTYPE", f"pool dtype {k_cache.dtype} is not float32 or bfloat16")
    if k_cache.dim() != 4:
        _raise("SHAPE", "pool must be 4-D")
    nb1 = k_cache.shape[0]
    if layout == "HND":
        hkv, bs = k_cache.shape[1], k_cache.shape[2]
    else:
        bs, hkv = k_cache.shape[1], k_cache.shape[2]
    return _capi.PoolDesc(nb1 - 1, bs, hkv, k_cache.shape[3], _DTYPES[k_cache.dtype],
                          _capi.LAYOUT_CODES[layout])


def _pool_pair(k_cache, v_cache, layout):
    desc = pool_desc(k_cache, layout)
    if v_cache.dtype != k_cache.dtype:
        _raise("DTYPE", "K and V pools differ in dtype")
    if v_cache.shape != k_cache.shape:
        _raise("SHAPE", "K and V pools differ in shape")
    for t in (k_cache, v_cache):
        if not t.is_cuda or not t.is_contiguous():
            _raise("SHAPE", "pools must be contiguous device tensors")
    return desc


def _device_tensor(t, name, dtype, device):
    if t.dtype != dtype:
        _raise("DTYPE", f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda or t.device != device or not t.is_contiguous():
        _raise("SHAPE", f"{name} must be a contiguous tensor on {device}")


def sink_slot(k_cache: torch.Tensor, layout: str = "HND") -> int:
    """The sink slot of a pool (num_blocks * block_size)."""
    desc = pool_desc(k_cache, layout)
    s = _capi.lib().pkv_sink_slot(ctypes.byref(desc))
    if s < 0:
        _check(_capi.lib().pkv_check_pool(ctypes.byref(desc)))
    return int(s)


def kv_write(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor,
             k_cache: torch.Tensor, v_cache: torch.Tensor, *, layout: str = "HND",
             validate: bool = True) -> None:
    """Scatter token i's K/V into slot ``slot_mapping[i]`` of the pools, in place."""
    n = int(slot_mapping.shape[0]) if slot_mapping.dim() >= 1 else 0
    if n == 0:
        _raise("EMPTY", "no tokens to write")
    desc = _pool_pair(k_cache, v_cache, layout)
    dev = k_cache.device
    _device_tensor(k, "k", k_cache.dtype, dev)
    _device_tensor(v, "v", k_cache.dtype, dev)
    _device_tensor(slot_mapping, "slot_mapping", torch.int64, dev)
    want = (n, desc.num_kv_heads, desc.head_dim)
    if tuple(k.shape) != want or tuple(v.shape) != want or slot_mapping.dim() != 1:
        _raise("SHAPE", f"k, v must be {want}, slot_mapping [{n}]")
    with torch.cuda.device(dev):
        _check(_capi.lib().pkv_kv_write(ctypes.byref(desc), _ptr(k_cache), _ptr(v_cache),
                                        _ptr(k), _ptr(v), _ptr(slot_mapping), n,
                                        int(bool(validate)), _stream(k_cache)))


def workspace_bytes(k_cache: torch.Tensor, num_rows: int, num_heads: int, max_blocks: int,
                    layout: str = "HND") -> int:
    desc = pool_desc(k_cache, layout)
    return int(_capi.lib().pkv_workspace_bytes(ctypes.byref(desc), num_rows, num_heads,
                                               max_blocks))


def paged_attention(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                    block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float, *,
                    layout: str = "HND", out: torch.Tensor | None = None,
                    workspace: torch.Tensor | None = None,
                    validate: bool = True) -> torch.Tensor:
    """The batched decode read; returns ``out`` ``[rows, heads, head_dim]``."""
    rows = int(context_lens.shape[0]) if context_lens.dim() >= 1 else 0
    if rows == 0:
        _raise("EMPTY", "no rows")
    desc = _pool_pair(k_cache, v_cache, layout)
    dev = k_cache.device
    _device_tensor(q, "q", k_cache.dtype, dev)
    _device_tensor(block_tables, "block_tables", torch.int32, dev)
    _device_tensor(context_lens, "context_lens", torch.int32, dev)
    if q.dim() != 3 or q.shape[0] != rows or q.shape[2] != desc.head_dim:
        _raise("SHAPE", f"q must be [{rows}, heads, {desc.head_dim}], got {tuple(q.shape)}")
    heads = int(q.shape[1])
    if context_lens.dim() != 1 or block_tables.dim() != 2 or block_tables.shape[0] != rows:
        _raise("SHAPE", "block_tables must be [rows, max_blocks], context_lens [rows]")
    max_blocks = int(block_tables.shape[1])
    if out is None:
        out = torch.empty_like(q)
    else:
        _device_tensor(out, "out", q.dtype, dev)
        if out.shape != q.shape:
            _raise("SHAPE", "out must have q's shape")
    lib = _capi.lib()
    need = int(lib.pkv_workspace_bytes(ctypes.byref(desc), rows, heads, max_blocks))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    elif workspace.device != dev or not workspace.is_contiguous():
        _raise("WORKSPACE", "workspace must be a contiguous tensor on the pool's device")
    ws_bytes = workspace.numel() * workspace.element_size()
    with torch.cuda.device(dev):
        _check(lib.pkv_paged_attention(ctypes.byref(desc), _ptr(out), _ptr(q), _ptr(k_cache),
                                       _ptr(v_cache), _ptr(block_tables), max_blocks,
                                       _ptr(context_lens), rows, heads, float(scale),
                                       _ptr(workspace), ws_bytes, int(bool(validate)),
                                       _stream(k_cache)))
    return out


def paged_attention_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                            block_tables: torch.Tensor, context_lens: torch.Tensor,
                            scale: float, out: torch.Tensor, *,
                            layout: str = "HND") -> torch.Tensor:
    """The decode read in the library's static scratch (pkv_paged_attention_noalloc):
    nothing is allocated, by the library or here, so ``out`` must be given; no host
    checks (bad inputs are clamped or skipped and reported in device_status)."""
    rows = int(context_lens.shape[0]) if context_lens.dim() >= 1 else 0
    if rows == 0:
        _raise("EMPTY", "no rows")
    desc = _pool_pair(k_cache, v_cache, layout)
    dev = k_cache.device
    _device_tensor(q, "q", k_cache.dtype, dev)
    _device_tensor(out, "out", k_cache.dtype, dev)
    _device_tensor(block_tables, "block_tables", torch.int32, dev)
    _device_tensor(context_lens, "context_lens", torch.int32, dev)
    if q.dim() != 3 or q.shape[0] != rows or q.shape[2] != desc.head_dim or \
            out.shape != q.shape:
        _raise("SHAPE", f"q and out must be [{rows}, heads, {desc.head_dim}]")
    if context_lens.dim() != 1 or block_tables.dim() != 2 or block_tables.shape[0] != rows:
        _raise("SHAPE", "block_tables must be [rows, max_blocks], context_lens [rows]")
    with torch.cuda.device(dev):
        _check(_capi.lib().pkv_paged_attention_noalloc(
            ctypes.byref(desc), _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
            _ptr(block_tables), int(block_tables.shape[1]), _ptr(context_lens), rows,
            int(q.shape[1]), float(scale), _stream(k_cache)))
    return out


def workspace_bytes_multi(k_cache: torch.Tensor, num_rows: int, query_len: int,
                          num_heads: int, max_blocks: int, layout: str = "HND") -> int:
    desc = pool_desc(k_cache, layout)
    return int(_capi.lib().pkv_workspace_bytes_multi(ctypes.byref(desc), num_rows, query_len,
                                                     num_heads, max_blocks))


def paged_attention_multi(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                          block_tables: torch.Tensor, context_lens: torch.Tensor,
                          scale: float, *, layout: str = "HND",
                          out: torch.Tensor | None = None,
                          workspace: torch.Tensor | None = None,
                          validate: bool = True) -> torch.Tensor:
    """The read with ``q`` [rows, query_len, heads, head_dim]: query i of a row is its
    token at position len - query_len + i and attends causally; returns ``out``."""
    rows = int(context_lens.shape[0]) if context_lens.dim() >= 1 else 0
    if rows == 0:
        _raise("EMPTY", "no rows")
    desc = _pool_pair(k_cache, v_cache, layout)
    dev = k_cache.device
    _device_tensor(q, "q", k_cache.dtype, dev)
    _device_tensor(block_tables, "block_tables", torch.int32, dev)
    _device_tensor(context_lens, "context_lens", torch.int32, dev)
    if q.dim() != 4 or q.shape[0] != rows or q.shape[3] != desc.head_dim:
        _raise("SHAPE", f"q must be [{rows}, query_len, heads, {desc.head_dim}], "
                        f"got {tuple(q.shape)}")
    query_len, heads = int(q.shape[1]), int(q.shape[2])
    if context_lens.dim() != 1 or block_tables.dim() != 2 or block_tables.shape[0] != rows:
        _raise("SHAPE", "block_tables must be [rows, max_blocks], context_lens [rows]")
    max_blocks = int(block_tables.shape[1])
    if out is None:
        out = torch.empty_like(q)
    else:
        _device_tensor(out, "out", q.dtype, dev)
        if out.shape != q.shape:
            _raise("SHAPE", "out must have q's shape")
    lib = _capi.lib()
    need = int(lib.pkv_workspace_bytes_multi(ctypes.byref(desc), rows, query_len, heads,
                                             max_blocks))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    elif workspace.device != dev or not workspace.is_contiguous():
        _raise("WORKSPACE", "workspace must be a contiguous tensor on the pool's device")
    ws_bytes = workspace.numel() * workspace.element_size()
    with torch.cuda.device(dev):
        _check(lib.pkv_paged_attention_multi(
            ctypes.byref(desc), _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
            _ptr(block_tables), max_blocks, _ptr(context_lens), rows, query_len, heads,
            float(scale), _ptr(workspace), ws_bytes, int(bool(validate)), _stream(k_cache)))
    return out


def _slot_window(slot_table: torch.Tensor, rows: int, dev: torch.device):
    """(width, row_stride) of a [rows, width] int64 window whose cells are contiguous
    along a row; the window may be a column slice of a wider table."""
    if slot_table.dtype != torch.int64:
        _raise("DTYPE", f"slot_table must be int64, got {slot_table.dtype}")
    if not slot_table.is_cuda or slot_table.device != dev:
        _raise("SHAPE", f"slot_table must be on {dev}")
    if slot_table.dim() != 2 or slot_table.shape[0] != rows:
        _raise("SHAPE", f"slot_table must be [{rows}, width]")
    width = int(slot_table.shape[1])
    if width < 1:
        _raise("SHAPE", "slot_table width must be at least 1")
    if slot_table.stride(1) != 1 or (rows > 1 and slot_table.stride(0) < width):
        _raise("SHAPE", "slot_table rows must be contiguous, one row after another")
    return width, int(slot_table.stride(0)) if rows > 1 else width


def workspace_bytes_slots(k_cache: torch.Tensor, num_rows: int, num_heads: int, width: int,
                          layout: str = "HND") -> int:
    desc = pool_desc(k_cache, layout)
    return int(_capi.lib().pkv_workspace_bytes_slots(ctypes.byref(desc), num_rows, num_heads,
                                                     width))


def paged_attention_slots(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                          slot_table: torch.Tensor, context_lens: torch.Tensor, scale: float,
                          *, layout: str = "HND", out: torch.Tensor | None = None,
                          workspace: torch.Tensor | None = None,
                          validate: bool = True) -> torch.Tensor:
    """The decode read through a per-token slot rectangle ``slot_table`` [rows, width]
    (int64, possibly a column window of a wider table); returns ``out``."""
    rows = int(context_lens.shape[0]) if context_lens.dim() >= 1 else 0
    if rows == 0:
        _raise("EMPTY", "no rows")
    desc = _pool_pair(k_cache, v_cache, layout)
    dev = k_cache.device
    _device_tensor(q, "q", k_cache.dtype, dev)
    _device_tensor(context_lens, "context_lens", torch.int32, dev)
    if q.dim() != 3 or q.shape[0] != rows or q.shape[2] != desc.head_dim:
        _raise("SHAPE", f"q must be [{rows}, heads, {desc.head_dim}], got {tuple(q.shape)}")
    if context_lens.dim() != 1:
        _raise("SHAPE", "context_lens must be [rows]")
    width, row_stride = _slot_window(slot_table, rows, dev)
    heads = int(q.shape[1])
    if out is None:
        out = torch.empty_like(q)
    else:
        _device_tensor(out, "out", q.dtype, dev)
        if out.shape != q.shape:
            _raise("SHAPE", "out must have q's shape")
    lib = _capi.lib()
    need = int(lib.pkv_workspace_bytes_slots(ctypes.byref(desc), rows, heads, width))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    elif workspace.device != dev or not workspace.is_contiguous():
        _raise("WORKSPACE", "workspace must be a contiguous tensor on the pool's device")
    ws_bytes = workspace.numel() * workspace.element_size()
    with torch.cuda.device(dev):
        _check(lib.pkv_paged_attention_slots(
            ctypes.byref(desc), _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
            _ptr(slot_table), width, row_stride, _ptr(context_lens), rows, heads,
            float(scale), _ptr(workspace), ws_bytes, int(bool(validate)), _stream(k_cache)))
    return out


class StepGraph:
    """One captured decode step (pkv_graph_capture): kv_write then paged_attention over
    the tensors it was captured with, replayed by ``launch``.  Holds references to those
    tensors so their storage outlives the graph."""

    def __init__(self, handle: ctypes.c_void_p, device: torch.device, keep: tuple):
        self._handle = handle
        self.device = device
        self._keep = keep

    def launch(self, stream=None) -> None:
        if self._handle is None:
            _raise("NULL", "graph already destroyed")
        s = torch.cuda.current_stream(self.device) if stream is None else stream
        with torch.cuda.device(self.device):
            _check(_capi.lib().pkv_graph_launch(self._handle, ctypes.c_void_p(s.cuda_stream)))

    def destroy(self) -> None:
        if self._handle is not None:
            handle, self._handle = self._handle, None
            _check(_capi.lib().pkv_graph_destroy(handle))
            self._keep = ()

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def capture_step(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor,
                 q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                 block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                 out: torch.Tensor, workspace: torch.Tensor, *,
                 layout: str = "HND") -> StepGraph:
    """Record kv_write + paged_attention over these tensors into a graph; nothing runs."""
    rows = int(context_lens.shape[0]) if context_lens.dim() == 1 else 0
    if rows == 0:
        _raise("EMPTY", "no rows")
    desc = _pool_pair(k_cache, v_cache, layout)
    dev = k_cache.device
    for t, name in ((k, "k"), (v, "v"), (q, "q"), (out, "out")):
        _device_tensor(t, name, k_cache.dtype, dev)
    _device_tensor(slot_mapping, "slot_mapping", torch.int64, dev)
    _device_tensor(block_tables, "block_tables", torch.int32, dev)
    _device_tensor(context_lens, "context_lens", torch.int32, dev)
    if workspace.device != dev or not workspace.is_contiguous():
        _raise("WORKSPACE", "workspace must be a contiguous tensor on the pool's device")
    kv_shape = (rows, desc.num_kv_heads, desc.head_dim)
    if tuple(k.shape) != kv_shape or tuple(v.shape) != kv_shape or \
            tuple(slot_mapping.shape) != (rows,):
        _raise("SHAPE", f"k, v must be {kv_shape}, slot_mapping [{rows}]")
    if q.dim() != 3 or q.shape[0] != rows or q.shape[2] != desc.head_dim or \
            out.shape != q.shape:
        _raise("SHAPE", f"q and out must be [{rows}, heads, {desc.head_dim}]")
    if block_tables.dim() != 2 or block_tables.shape[0] != rows:
        _raise("SHAPE", "block_tables must be [rows, max_blocks]")
    handle = ctypes.c_void_p()
    with torch.cuda.device(dev):
        _check(_capi.lib().pkv_graph_capture(
            ctypes.byref(desc), _ptr(k_cache), _ptr(v_cache), _ptr(k), _ptr(v),
            _ptr(slot_mapping), _ptr(out), _ptr(q), _ptr(block_tables),
            int(block_tables.shape[1]), _ptr(context_lens), rows, int(q.shape[1]),
            float(scale), _ptr(workspace), workspace.numel() * workspace.element_size(),
            ctypes.byref(handle)))
    return StepGraph(handle, dev, (k, v, slot_mapping, q, k_cache, v_cache, block_tables,
                                   context_lens, out, workspace))


def capture_step_slots(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor,
                       q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                       slot_table: torch.Tensor, context_lens: torch.Tensor, scale: float,
                       out: torch.Tensor, workspace: torch.Tensor, *,
                       layout: str = "HND") -> StepGraph:
    """Record kv_write + paged_attention_slots over these tensors into a graph."""
    rows = int(context_lens.shape[0]) if context_lens.dim() == 1 else 0
    if rows == 0:
        _raise("EMPTY", "no rows")
    desc = _pool_pair(k_cache, v_cache, layout)
    dev = k_cache.device
    for t, name in ((k, "k"), (v, "v"), (q, "q"), (out, "out")):
        _device_tensor(t, name, k_cache.dtype, dev)
    _device_tensor(slot_mapping, "slot_mapping", torch.int64, dev)
    _device_tensor(context_lens, "context_lens", torch.int32, dev)
    width, row_stride = _slot_window(slot_table, rows, dev)
    if workspace.device != dev or not workspace.is_contiguous():
        _raise("WORKSPACE", "workspace must be a contiguous tensor on the pool's device")
    kv_shape = (rows, desc.num_kv_heads, desc.head_dim)
    if tuple(k.shape) != kv_shape or tuple(v.shape) != kv_shape or \
            tuple(slot_mapping.shape) != (rows,):
        _raise("SHAPE", f"k, v must be {kv_shape}, slot_mapping [{rows}]")
    if q.dim() != 3 or q.shape[0] != rows or q.shape[2] != desc.head_dim or \
            out.shape != q.shape:
        _raise("SHAPE", f"q and out must be [{rows}, heads, {desc.head_dim}]")
    handle = ctypes.c_void_p()
    with torch.cuda.device(dev):
        _check(_capi.lib().pkv_graph_capture_slots(
            ctypes.byref(desc), _ptr(k_cache), _ptr(v_cache), _ptr(k), _ptr(v),
            _ptr(slot_mapping), _ptr(out), _ptr(q), _ptr(slot_table), width, row_stride,
            _ptr(context_lens), rows, int(q.shape[1]), float(scale), _ptr(workspace),
            workspace.numel() * workspace.element_size(), ctypes.byref(handle)))
    return StepGraph(handle, dev, (k, v, slot_mapping, q, k_cache, v_cache, slot_table,
                                   context_lens, out, workspace))


def device_status(device=None, clear: bool = True) -> int:
    """Bitwise OR of the device-side refusal bits raised since the last clear."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else device
    flags = ctypes.c_uint32(0)
    with torch.cuda.device(dev):
        stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        _check(_capi.lib().pkv_device_status(ctypes.byref(flags), int(bool(clear)), stream))
    return int(flags.value)


def _workspace_args(workspace: torch.Tensor):
    if not workspace.is_cuda or not workspace.is_contiguous():
        _raise("WORKSPACE", "workspace must be a contiguous device tensor")
    return _ptr(workspace), workspace.numel() * workspace.element_size()


def workspace_status(workspace: torch.Tensor) -> int:
    """PKV_DEVERR_* bits raised by the last attention call that used this workspace
    (and by no other call); synchronises the current stream."""
    flags = ctypes.c_uint32(0)
    ptr, nbytes = _workspace_args(workspace)
    with torch.cuda.device(workspace.device):
        stream = ctypes.c_void_p(torch.cuda.current_stream(workspace.device).cuda_stream)
        _check(_capi.lib().pkv_workspace_status(ptr, nbytes, ctypes.byref(flags), stream))
    return int(flags.value)


def plan_info(workspace: torch.Tensor) -> dict:
    """The plan and the decode kernel's walk count of the last attention call that used
    this workspace (pkv_plan_info_read); synchronises the current stream."""
    info = _capi.PlanInfo()
    ptr, nbytes = _workspace_args(workspace)
    with torch.cuda.device(workspace.device):
        stream = ctypes.c_void_p(torch.cuda.current_stream(workspace.device).cuda_stream)
        _check(_capi.lib().pkv_plan_info_read(ptr, nbytes, ctypes.byref(info), stream))
    return {f: int(getattr(info, f)) for f, _ in _capi.PlanInfo._fields_}


def stream_read(buf: torch.Tensor, sink: torch.Tensor, groups_per_cu: int = 4) -> None:
    """Enqueue a plain streaming read of ``buf`` (pkv_stream_read) on the current
    stream; ``sink`` is a device int32/uint32 scalar tensor."""
    if not buf.is_cuda or not buf.is_contiguous() or not sink.is_cuda:
        _raise("SHAPE", "buf and sink must be contiguous device tensors")
    nbytes = buf.numel() * buf.element_size() // 16 * 16
    with torch.cuda.device(buf.device):
        _check(_capi.lib().pkv_stream_read(_ptr(buf), nbytes, _ptr(sink), int(groups_per_cu),
                                           _stream(buf)))


class GatherPieces:
    """Byte offsets of pieces of both pools for gather_read, checked on the host to lie
    inside the pools and then copied to the device."""

    def __init__(self, k_cache: torch.Tensor, v_cache: torch.Tensor, offsets: np.ndarray,
                 piece_bytes: int):
        offsets = np.ascontiguousarray(offsets, dtype=np.int64)
        nbytes = min(k_cache.numel() * k_cache.element_size(),
                     v_cache.numel() * v_cache.element_size())
        if offsets.ndim != 1 or offsets.size == 0:
            _raise("SHAPE", "offsets must be a non-empty 1-D array")
        if piece_bytes < 16 or piece_bytes % 16 or offsets.min() < 0 or \
                offsets.max() + piece_bytes > nbytes:
            _raise("SHAPE", "a piece lies outside the pools")
        self.k_cache, self.v_cache = k_cache, v_cache
        self.offsets = torch.from_numpy(offsets).to(k_cache.device)
        self.piece_bytes = int(piece_bytes)


GATHER_SHAPES = ((4, 1), (4, 2), (4, 4), (8, 1), (8, 2), (8, 4))
"""(waves per workgroup, pieces per wave) that pkv_gather_read takes."""


def gather_read(pieces: GatherPieces, sink: torch.Tensor, groups_per_cu: int = 4,
                waves_per_group: int = 4, pieces_per_wave: int = 2) -> None:
    """Enqueue a plain read of checked pieces of both pools (pkv_gather_read) on the
    current stream."""
    k_cache, v_cache, offsets = pieces.k_cache, pieces.v_cache, pieces.offsets
    piece_bytes = pieces.piece_bytes
    with torch.cuda.device(k_cache.device):
        _check(_capi.lib().pkv_gather_read(_ptr(k_cache), _ptr(v_cache), _ptr(offsets),
                                           offsets.numel(), int(piece_bytes), _ptr(sink),
                                           int(groups_per_cu), int(waves_per_group),
                                           int(pieces_per_wave), _stream(k_cache)))


def decode_kernel_for(k_cache: torch.Tensor, num_heads: int, query_len: int = 1,
                      layout: str = "HND") -> str:
    """Which decode kernel (and query-vector group) a read of this shape runs."""
    desc = pool_desc(k_cache, layout)
    return _capi.lib().pkv_decode_kernel_for(ctypes.byref(desc), num_heads, query_len).decode()


def set_tuning(chunk_min: int = 0, chunk_max: int = 0, decode_waves: int = 0,
               items_per_group: int = 0, deal: int = 0, staging: int = 0,
               max_query_group: int = 0, mfma: int = 0, groups_per_cu: int = 0,
               solo_tokens: int = 0) -> None:
    """Set the decode work split (0 keeps a value); see pkv_set_tuning."""
    t = _capi.Tuning(chunk_min, chunk_max, decode_waves, items_per_group, deal, staging,
                     max_query_group, mfma, groups_per_cu, solo_tokens)
    _check(_capi.lib().pkv_set_tuning(ctypes.byref(t)))


def get_tuning() -> dict:
    t = _capi.Tuning()
    _check(_capi.lib().pkv_get_tuning(ctypes.byref(t)))
    return {f: int(getattr(t, f)) for f, _ in _capi.Tuning._fields_}


def timing_enable(on: bool = True) -> None:
    """Start (or stop) bracketing every kernel launch with HIP events."""
    _check(_capi.lib().pkv_timing_enable(int(bool(on))))


def timing_read(phase: str, reset: bool = True) -> tuple[float, int]:
    """(summed milliseconds, launches) of one phase: kv_write, plan, decode, combine."""
    ms = ctypes.c_double(0.0)
    n = ctypes.c_int64(0)
    _check(_capi.lib().pkv_timing_read(_capi.PHASES[phase], ctypes.byref(ms), ctypes.byref(n),
                                       int(bool(reset))))
    return float(ms.value), int(n.value)


# ---------------------------------------------------------------------------- #
# host-side checks (no GPU needed)
# ---------------------------------------------------------------------------- #
def host_desc(num_blocks, block_size, kv_heads, head_dim, dtype="bf16", layout="HND"):
    return _capi.PoolDesc(num_blocks, block_size, kv_heads, head_dim,
                          {"f32": _capi.F32, "bf16": _capi.BF16}.get(dtype, 99),
                          _capi.LAYOUT_CODES.get(layout, 99))


def check_write_host(desc: _capi.PoolDesc, slot_mapping: np.ndarray) -> str:
    """Status name the library's host validator gives a write."""
    sm = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    st = _capi.lib().pkv_check_write_host(ctypes.byref(desc),
                                          sm.ctypes.data_as(ctypes.c_void_p), sm.shape[0])
    return _capi.STATUS_NAMES[st]


def check_attention_slots_host(desc: _capi.PoolDesc, slot_table: np.ndarray,
                               context_lens: np.ndarray, num_heads: int) -> str:
    """Status name the library's host validator gives a read through a slot rectangle:
    a [rows, width] int64 numpy array whose rows are contiguous (a column slice of a
    wider table is passed with that table's row stride)."""
    rect = np.asarray(slot_table)
    ctx = np.ascontiguousarray(context_lens, dtype=np.int32)
    if rect.dtype != np.int64 or rect.ndim != 2 or rect.shape[0] != ctx.shape[0] or \
            rect.strides[1] != 8 or rect.strides[0] % 8 != 0:
        raise ValueError("slot_table must be a 2-D int64 array with contiguous rows, "
                         "one per length")
    st = _capi.lib().pkv_check_attention_slots_host(
        ctypes.byref(desc), rect.ctypes.data_as(ctypes.c_void_p), rect.shape[1],
        rect.strides[0] // 8, ctx.ctypes.data_as(ctypes.c_void_p), ctx.shape[0], num_heads)
    return _capi.STATUS_NAMES[st]


def check_attention_multi_host(desc: _capi.PoolDesc, block_tables: np.ndarray,
                               context_lens: np.ndarray, query_len: int,
                               num_heads: int) -> str:
    """Status name the library's host validator gives a multi-token read."""
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    ctx = np.ascontiguousarray(context_lens, dtype=np.int32)
    m = bt.shape[1] if bt.ndim == 2 else 0
    st = _capi.lib().pkv_check_attention_multi_host(
        ctypes.byref(desc), bt.ctypes.data_as(ctypes.c_void_p), m,
        ctx.ctypes.data_as(ctypes.c_void_p), ctx.shape[0], query_len, num_heads)
    return _capi.STATUS_NAMES[st]


def check_attention_host(desc: _capi.PoolDesc, block_tables: np.ndarray,
                         context_lens: np.ndarray, num_heads: int) -> str:
    """Status name the library's host validator gives a read."""
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    ctx = np.ascontiguousarray(context_lens, dtype=np.int32)
    m = bt.shape[1] if bt.ndim == 2 else 0
    st = _capi.lib().pkv_check_attention_host(
        ctypes.byref(desc), bt.ctypes.data_as(ctypes.c_void_p), m,
        ctx.ctypes.data_as(ctypes.c_void_p), ctx.shape[0], num_heads)
    return _capi.STATUS_NAMES[st]

"""ctypes declarations of libpagedkv.so (include/pagedkv.h).  Loading only; no logic."""

from __future__ import annotations

import ctypes
import os

# PAGEDKV_LIB names another build of the same library (for side-by-side comparisons)
LIB_PATH = os.environ.get("PAGEDKV_LIB") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libpagedkv.so")

F32, BF16 = 0, 1
LAYOUT_CODES = {"HND": 0, "NHD": 1}
STATUS_NAMES = ("OK", "EMPTY", "DTYPE", "SHAPE", "CONTEXT_BOUNDS", "BLOCK_ID", "SLOT",
                "UNSUPPORTED", "WORKSPACE", "NULL", "HIP")
DEVERR_SLOT, DEVERR_CONTEXT_BOUNDS, DEVERR_BLOCK_ID = 1, 2, 4
NOALLOC_SCRATCH_BYTES = 32 << 20   # PKV_NOALLOC_SCRATCH_BYTES

# every function include/pagedkv.h declares: name -> (restype, argtypes)
_i32, _i64, _sz, _p, _f = (ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p,
                           ctypes.c_float)


class PoolDesc(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int64), ("block_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("layout", ctypes.c_int32)]


class Tuning(ctypes.Structure):
    _fields_ = [("chunk_min", ctypes.c_int32), ("chunk_max", ctypes.c_int32),
                ("decode_waves", ctypes.c_int32), ("items_per_group", ctypes.c_int32),
                ("deal", ctypes.c_int32), ("staging", ctypes.c_int32),
                ("max_query_group", ctypes.c_int32), ("mfma", ctypes.c_int32),
                ("groups_per_cu", ctypes.c_int32), ("solo_tokens", ctypes.c_int32)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("chunk_tokens", ctypes.c_int32), ("entries", ctypes.c_int32),
                ("full_chunks", ctypes.c_int32), ("live_entries", ctypes.c_int32),
                ("wide_entries", ctypes.c_int32), ("split_rows", ctypes.c_int32),
                ("records", ctypes.c_int32), ("record_capacity", ctypes.c_int32),
                ("decode_groups", ctypes.c_int32), ("vector_groups", ctypes.c_int32),
                ("tile_tokens", ctypes.c_int32), ("token_rows", ctypes.c_int32),
                ("tiles_walked", ctypes.c_int64), ("token_entries", ctypes.c_int32),
                ("status", ctypes.c_uint32)]


_PD = ctypes.POINTER(PoolDesc)
SIGNATURES = {
    "pkv_abi_version": (_i32, []),
    "pkv_status_str": (ctypes.c_char_p, [_i32]),
    "pkv_last_error_detail": (ctypes.c_char_p, []),
    "pkv_sink_slot": (_i64, [_PD]),
    "pkv_pool_elements": (_i64, [_PD]),
    "pkv_check_pool": (_i32, [_PD]),
    "pkv_check_write_host": (_i32, [_PD, _p, _i64]),
    "pkv_check_attention_host": (_i32, [_PD, _p, _i32, _p, _i64, _i32]),
    "pkv_kv_write": (_i32, [_PD, _p, _p, _p, _p, _p, _i64, _i32, _p]),
    "pkv_workspace_bytes": (_sz, [_PD, _i64, _i32, _i32]),
    "pkv_paged_attention": (_i32, [_PD, _p, _p, _p, _p, _p, _i32, _p, _i64, _i32, _f, _p,
                                   _sz, _i32, _p]),
    "pkv_device_status": (_i32, [ctypes.POINTER(ctypes.c_uint32), _i32, _p]),
    "pkv_workspace_status": (_i32, [_p, _sz, ctypes.POINTER(ctypes.c_uint32), _p]),
    "pkv_plan_info_read": (_i32, [_p, _sz, ctypes.POINTER(PlanInfo), _p]),
    "pkv_decode_kernel_for": (ctypes.c_char_p, [_PD, _i32, _i32]),
    "pkv_set_tuning": (_i32, [ctypes.POINTER(Tuning)]),
    "pkv_get_tuning": (_i32, [ctypes.POINTER(Tuning)]),
    "pkv_timing_enable": (_i32, [_i32]),
    "pkv_timing_read": (_i32, [_i32, ctypes.POINTER(ctypes.c_double),
                               ctypes.POINTER(ctypes.c_int64), _i32]),
    "pkv_graph_capture": (_i32, [_PD, _p, _p, _p, _p, _p, _p, _p, _p, _i32, _p, _i64, _i32,
                                 _f, _p, _sz, ctypes.POINTER(ctypes.c_void_p)]),
    "pkv_graph_capture_slots": (_i32, [_PD, _p, _p, _p, _p, _p, _p, _p, _p, _i32, _i64, _p,
                                       _i64, _i32, _f, _p, _sz,
                                       ctypes.POINTER(ctypes.c_void_p)]),
    "pkv_graph_launch": (_i32, [_p, _p]),
    "pkv_paged_attention_noalloc": (_i32, [_PD, _p, _p, _p, _p, _p, _i32, _p, _i64, _i32,
                                           _f, _p]),
    "pkv_stream_read": (_i32, [_p, _sz, _p, _i32, _p]),
    "pkv_gather_read": (_i32, [_p, _p, _p, _i64, _i32, _p, _i32, _i32, _i32, _p]),
    "pkv_workspace_bytes_multi": (_sz, [_PD, _i64, _i32, _i32, _i32]),
    "pkv_paged_attention_multi": (_i32, [_PD, _p, _p, _p, _p, _p, _i32, _p, _i64, _i32, _i32,
                                         _f, _p, _sz, _i32, _p]),
    "pkv_check_attention_multi_host": (_i32, [_PD, _p, _i32, _p, _i64, _i32, _i32]),
    "pkv_workspace_bytes_slots": (_sz, [_PD, _i64, _i32, _i32]),
    "pkv_paged_attention_slots": (_i32, [_PD, _p, _p, _p, _p, _p, _i32, _i64, _p, _i64, _i32,
                                         _f, _p, _sz, _i32, _p]),
    "pkv_check_attention_slots_host": (_i32, [_PD, _p, _i32, _i64, _p, _i64, _i32]),
    "pkv_graph_destroy": (_i32, [_p]),
}
PHASES = {"kv_write": 0, "plan": 1, "decode": 2, "combine": 3, "translate": 4,
          "token_rows": 5}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library.  Raises if it has not been built: there is no fallback."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib

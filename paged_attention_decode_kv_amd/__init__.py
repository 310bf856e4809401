"""MI355X-native (gfx950) batched paged-attention decode step.

``kv_write`` scatters a decode step's new K/V into a paged pool (pad rows into the
sink slot); ``paged_attention`` reads every (row, query head) through its block table
with an online softmax.  Both run as hand-written HIP kernels in ``libpagedkv.so``
(C ABI in ``include/pagedkv.h``); this package only marshals torch tensors into it.
"""

from .binding import (  # noqa: F401
    PagedKVError,
    check_attention_host,
    check_write_host,
    device_status,
    host_desc,
    kv_write,
    paged_attention,
    pool_desc,
    get_tuning,
    set_tuning,
    sink_slot,
    timing_enable,
    timing_read,
    workspace_bytes,
)

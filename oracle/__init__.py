"""CPU oracle for the batched paged-attention decode step.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The HIP library never routes through it, and this package imports
nothing from the HIP library or its Python binding.

What it computes is the plain definition of the step described on the nanoserve
pages:

* ``kv_write``: the slot scatter of each row's new K/V into the pool, pad rows
  aimed at the sink slot (Day 55, "Why it matters": a pad row has length 0 and
  writes to the sink, one slot past everything the allocator hands out).
* ``paged_attention``: the masked-rectangle read that the Day-59 page grades its
  streamed kernel against (Day 59, "What I added today": gather the whole
  [batch, max_ctx] slot mapping into K/V, score a [batch, heads, 1, max_ctx]
  rectangle, mask by length, softmax, multiply by V), built on the Day-50
  ``rebuild_mapping`` construction (Day 51, "What I added today") and the
  block-id addressing ``block_id * block_size + offset`` (Day 51, "Why it
  matters").
* ``paged_attention_multi``: several new tokens (queries) per row, each
  attending causally over the positions up to its own (Day 59, "Why it
  matters": the rectangle's query_len axis).
* ``paged_attention_slots``: the same read addressed by a per-token slot
  rectangle handed in directly, a window on the persistent slot table (Day 51,
  "What I added today").

Every floating-point step runs in float64.  Parity is pinned by the tests under
``tests/test_oracle_*.py`` (brute force, library routines, closed forms,
invariants and the pages' printed arithmetic); no function here is "parity
unpinned".
"""

from .decode import (  # noqa: F401
    LAYOUTS,
    REFUSAL_CODES,
    Refusal,
    decode_storage,
    gather,
    kv_write,
    paged_attention,
    paged_attention_multi,
    paged_attention_slots,
    rebuild_mapping,
    sink_slot,
    slot_view,
    validate_attention,
    validate_attention_multi,
    validate_attention_slots,
    validate_write,
)

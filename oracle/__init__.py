"""CPU oracle for the paged-KV decode path (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The library (``paged_kv_cache_83_amd``)
never imports it, and it never imports the library: the two share no code. The
only inputs both receive come from the seeded generators in ``synth``.

Everything here is plain and slow on purpose: numpy and Python loops, float64
for every floating-point result, one obvious step at a time, each function
citing the passage of the pages it follows. The pages are:

* "KV Cache Management" (Harvard Edge cs249r book, vol. 3): Eq. (1), the
  PagedAttention virtual memory model, block-size trade-offs, copy-on-write
  branching, chunked-prefill online softmax, asynchronous paged swapping.
* "EfficientAgent: What Makes KV Cache Offloading Work for Concurrent Agents?":
  per-rank KV footprint, Eq. (1) and Table 6.
* "PagedAttention" (programmer.ie Inference book, ch. 14): block allocator,
  block tables, fork and copy-on-write, the waste table.

Modules:
  footprint      -- KV bytes per token / block, blocks per sequence, tail waste
  layout         -- how a pool array is addressed (the library's documented layout)
  kv_ops         -- slot-mapped append, block copy, gather and scatter
  attention      -- contiguous rebuild from block tables + softmax attention
  block_manager  -- free list, reference counts, fork, copy-on-write, release, swap

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against values the pages print, closed forms, invariants or an independent
library routine. Nothing here is "parity unpinned".
"""

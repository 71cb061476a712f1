"""Paged KV writes and paged attention for one AMD Instinct MI355X (gfx950).

* ``libpa.so`` (``csrc/``, C ABI in ``include/pa.h``): HIP kernels for the KV
  write (fp16 copy, int8 per-token requantisation), block copies for
  copy-on-write, and attention over paged K/V (vector split-K path for
  decode, MFMA path for prefill / chunked prefill).
* ``pa``: the ctypes binding, one function per C entry point.
* ``host``: host-side integer bookkeeping (allocator, tables, refcounts,
  copy-on-write) that produces the metadata the kernels consume.
* ``workload``: drives a seeded synthetic workload through ``host`` and the
  device calls.
"""
from .host import BlockAllocator, KVCacheExhausted, PagedKVManager, StepBatch  # noqa: F401
from .pa import (  # noqa: F401
    PagedAttentionError, load_library, pa_attend, pa_attend_workspace_bytes, pa_copy_blocks, pa_write_kv,
)

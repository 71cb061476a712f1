"""CPU oracle for paged attention: test infrastructure, not the product.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call anything in this package.  It shares no code
with ``paged_kv_cache_47_amd`` (neither imports the other); the two meet only
in the seeded inputs of ``synthetic``.

What it computes, each part written from the pages' own description:

* ``paging``     - a LIFO free stack with an allocated set and refcounts, block
                   tables, address translation ``pos // bs`` / ``pos % bs``,
                   slot numbers, and copy-on-write copies for beam forks.
* ``kv_write``   - the pool after a step's writes: an fp16 scatter, and the
                   int8 per-token dequantise / append / re-max / requantise
                   replay with one fp16 scale per (block, KV head).
* ``attention``  - gather each sequence's K/V through its block table into a
                   contiguous buffer, then plain scaled dot-product attention in
                   float64 with GQA head sharing and the causal rule at each
                   query's true position.
* ``brute``      - the same attention as pure-Python loops for tiny inputs.

Pages cited (by title):
  [manager]   "Build a paged KV cache manager from scratch" (martinuke0.github.io)
  [pytorch]   "How to Implement Paged Attention in PyTorch and vLLM" (swarnava.dev)
  [nanoserve] "Day 14: the block allocator, paging for attention starts as pure
              bookkeeping" (pjdurden.github.io/nanoserve)
  [engine]    "Building a paged inference engine from scratch, and measuring it
              honestly" (vrajpatel105.github.io/paged-inference)

Parity pins for every function live in ``tests/test_oracle_pins.py``.  The
pages print no attention output values, so numeric attention results are
pinned by closed forms, brute force, permutation invariance and equality with
contiguous (unpaged) attention rather than by printed numbers.
"""

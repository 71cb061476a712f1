"""Reference paging bookkeeping (test infrastructure; see ``oracle/__init__``).

Written from:
* [nanoserve] "What I learned": a free stack plus an allocated set; freeing an
  id that is not allocated raises ``ValueError``; a multi-block reservation of
  ``ceil(tokens / bs)`` blocks is all-or-nothing; exhaustion has its own error;
  reuse is last-in-first-out.
* [pytorch] "Represent blocks, sequences, and free capacity" and "Allocate,
  append, and free KV-cache blocks": the stack starts so the first pops give
  0, 1, 2, ...; a new block is popped when ``pos % bs == 0``; the write lands
  in block ``table[pos // bs]`` at offset ``pos % bs``.
* [manager] "Step 2: The Block Pool" / "Step 3: The Block Table": refcounts,
  and a fork that shares every block id and retains each one.
* [pytorch] "Map the PyTorch design to vLLM PagedAttention": a shared block is
  copied only on the first divergent write (copy-on-write).

Readings where the pages are silent: a block whose refcount reaches zero goes
straight back on the free stack; a slot number is ``block * bs + offset``; all
copy-on-write copies of a step happen before that step's writes.

Sliding window ([pytorch] "PagedAttention vs sliding-window attention,
RadixAttention, and SSMs": the window caps retained history while paging
manages the blocks that hold it).  Reading: after a sequence's new positions
are reserved, every block of it that holds no position at or after the
step's earliest visible key (``L - Q - w + 1``, L after the step) is
released, in table order; its table entry becomes -1.
"""
from __future__ import annotations

import numpy as np


class Exhausted(Exception):
    """The pool cannot supply the blocks asked for ([nanoserve] "What I learned")."""


def blocks_for(num_tokens: int, block_size: int) -> int:
    """ceil(num_tokens / block_size) ([pytorch] "Size the paged KV cache and choose a block size")."""
    return -(-int(num_tokens) // int(block_size))


def translate(pos: int, block_size: int) -> tuple:
    """(logical block, offset) of token position ``pos`` ([pytorch] "How to implement
    paged attention: the minimal data flow", steps 2 and 3)."""
    return pos // block_size, pos % block_size


class RefPool:
    """Free stack, allocated set and refcounts over ``num_blocks`` ids."""

    def __init__(self, num_blocks: int, first_pops=None):
        order = range(num_blocks) if first_pops is None else [int(b) for b in first_pops]
        assert sorted(order) == list(range(num_blocks))
        self.num_blocks = num_blocks
        self.stack = list(reversed(list(order)))   # top of the stack is the end of the list
        self.refs: dict = {}                        # allocated id -> refcount

    @property
    def num_free(self) -> int:
        return len(self.stack)

    def pop(self) -> int:
        if not self.stack:
            raise Exhausted("no free block")
        b = self.stack.pop()
        self.refs[b] = 1
        return b

    def pop_for(self, num_tokens: int, block_size: int) -> list:
        n = blocks_for(num_tokens, block_size)
        if n > len(self.stack):
            raise Exhausted(f"need {n} blocks, {len(self.stack)} free")
        return [self.pop() for _ in range(n)]

    def push(self, b: int) -> None:
        if b not in self.refs:
            raise ValueError(f"block {b} is not allocated")
        del self.refs[b]
        self.stack.append(b)

    def push_all(self, ids) -> None:
        for b in ids:
            self.push(b)

    def retain(self, b: int) -> None:
        if b not in self.refs:
            raise ValueError(f"block {b} is not allocated")
        self.refs[b] += 1

    def release(self, b: int) -> None:
        if b not in self.refs:
            raise ValueError(f"block {b} is not allocated")
        self.refs[b] -= 1
        if self.refs[b] == 0:
            self.push(b)


class RefState:
    """Sequences (block table + length) over one ``RefPool``."""

    def __init__(self, num_blocks, block_size, first_pops=None):
        self.pool = RefPool(num_blocks, first_pops)
        self.bs = block_size
        self.tables: list = []
        self.lens: list = []

    def add(self, num_tokens: int) -> int:
        self.tables.append(self.pool.pop_for(num_tokens, self.bs))
        self.lens.append(int(num_tokens))
        return len(self.tables) - 1

    def fork(self, i: int) -> int:
        t = list(self.tables[i])
        for b in t:
            self.pool.retain(b)
        self.tables.append(t)
        self.lens.append(self.lens[i])
        return len(self.tables) - 1

    def append(self, i: int, n: int):
        """Reserve positions len..len+n-1 of sequence ``i``; returns (slots, copies)
        where ``copies`` lists (src, dst) block pairs to copy before writing."""
        table = self.tables[i]
        slots, copies = [], []
        for j in range(n):
            pos = self.lens[i] + j
            lb, off = translate(pos, self.bs)
            if lb == len(table):
                table.append(self.pool.pop())
            elif self.pool.refs[table[lb]] > 1:
                old = table[lb]
                new = self.pool.pop()
                copies.append((old, new))
                self.pool.release(old)
                table[lb] = new
            slots.append(table[lb] * self.bs + off)
        self.lens[i] += n
        return slots, copies


def build_state(w) -> RefState:
    """Tables of a ``synthetic.Workload`` before its first step.

    Sequences take their cached-context blocks in order.  With a shared
    prefix, the prefix chain is taken first, every request holds it (one
    reference each), then each request takes its own suffix blocks; request r
    is then forked into ``beams[r]`` sequences, listed request by request."""
    st = RefState(w.num_blocks, w.block_size, w.first_pops)
    if w.beams is None:
        for c in w.ctx_lens:
            st.add(int(c))
        return st
    bs = w.block_size
    prefix = st.pool.pop_for(w.shared_prefix, bs)
    req_tables, req_lens = [], []
    for r, c in enumerate(w.ctx_lens):
        if r > 0:
            for b in prefix:
                st.pool.retain(b)
        suffix = st.pool.pop_for(int(c) - w.shared_prefix, bs)
        req_tables.append(list(prefix) + suffix)
        req_lens.append(int(c))
    order = []
    for r in range(len(req_tables)):
        st.tables.append(req_tables[r])
        st.lens.append(req_lens[r])
        order.append(len(st.tables) - 1)
    seqs = []
    for r, base in enumerate(order):
        seqs.append(base)
        for _ in range(int(w.beams[r]) - 1):
            seqs.append(st.fork(base))
    # canonical order: request by request, the original first, then its forks
    st.tables = [st.tables[i] for i in seqs]
    st.lens = [st.lens[i] for i in seqs]
    return st


def release_out_of_window(st: RefState, i: int, q_len: int, window: int) -> None:
    """Release sequence ``i``'s blocks that only hold positions before the
    step's earliest visible key; their table entries become -1."""
    lo = max(0, st.lens[i] - int(q_len) - int(window) + 1)
    table = st.tables[i]
    for lb in range(min(lo // st.bs, len(table))):
        if table[lb] >= 0:
            st.pool.release(table[lb])
            table[lb] = -1


def apply_step(st: RefState, q_lens, window: int = 0):
    """Reserve every sequence's new positions; returns (slot_mapping, copies).
    With ``window > 0`` each sequence then releases its out-of-window blocks."""
    slots, copies = [], []
    for i, n in enumerate(q_lens):
        s, c = st.append(i, int(n))
        slots += s
        copies += c
        if window:
            release_out_of_window(st, i, int(n), window)
    return np.asarray(slots, np.int64), copies


def table_array(st: RefState, width=None) -> np.ndarray:
    width = max([len(t) for t in st.tables] + [1]) if width is None else width
    out = np.zeros((len(st.tables), width), np.int64)
    for i, t in enumerate(st.tables):
        out[i, :len(t)] = t
    return out

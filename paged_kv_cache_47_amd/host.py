"""Host-side integer bookkeeping that feeds the paged-attention kernels.

Block allocator, per-sequence block tables and lengths, refcounts,
fork/copy-on-write, and the per-step metadata arrays (slot mapping, block
tables, lengths, copy pairs) handed to ``pa_write_kv`` / ``pa_attend`` /
``pa_copy_blocks``.  Pure integers, no device work.

Behaviour follows the pages:
* [nanoserve] "Day 14: the block allocator ...", "What I learned": ids live
  either on a LIFO free stack or in the allocated set; a free of an id that is
  not allocated raises ``ValueError``; ``allocate_for`` reserves
  ``ceil(tokens / block_size)`` blocks or none and raises
  ``KVCacheExhausted``.
* [pytorch] "How to Implement Paged Attention in PyTorch and vLLM",
  "Allocate, append, and free KV-cache blocks": first pops give 0, 1, 2, ...;
  a sequence takes a new block when ``pos % block_size == 0``; its token at
  ``pos`` lives in block ``table[pos // block_size]`` at offset
  ``pos % block_size``.
* [engine] "Building a paged inference engine ...", "02 The engine":
  ``can_allocate`` and ``num_free`` for admission decisions.
* [manager] "Build a paged KV cache manager from scratch", steps 2-3 and its
  tests: retain/release refcounts; ``fork`` shares every block and retains it;
  finishing a sequence twice is harmless.
* [pytorch] "Map the PyTorch design to vLLM PagedAttention": a shared block
  is copied on its first divergent write (copy-on-write).
* [pytorch] "PagedAttention vs sliding-window attention, RadixAttention, and
  SSMs": with a sliding window of ``w`` tokens, a step's queries see nothing
  before position ``seq_len - q_len - w + 1``; once a sequence has reserved
  its positions for the step, every block holding only earlier positions is
  released (in table order) and its table entry becomes -1.
A block whose refcount drops to zero goes straight back on the free stack.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Iterable, List, Optional, Sequence

import numpy as np


class KVCacheExhausted(RuntimeError):
    """The pool cannot supply the requested blocks."""


class BlockAllocator:
    """Fixed pool of block ids: LIFO free stack, allocated set, refcounts."""

    def __init__(self, num_blocks: int, first_pops: Optional[Sequence[int]] = None):
        if num_blocks <= 0:
            raise ValueError("num_blocks must be positive")
        self.num_blocks = int(num_blocks)
        order = np.arange(num_blocks) if first_pops is None else np.asarray(first_pops, np.int64)
        if order.shape != (num_blocks,) or not np.array_equal(np.sort(order), np.arange(num_blocks)):
            raise ValueError("first_pops must be a permutation of range(num_blocks)")
        # the stack's top is the end of the list: reverse so successive pops follow `order`
        self._free: List[int] = order[::-1].tolist()
        self._refs: List[int] = [0] * self.num_blocks   # a list: per-token scalar lookups stay cheap

    @property
    def num_free(self) -> int:
        return len(self._free)

    def can_allocate(self, num_blocks: int) -> bool:
        return num_blocks <= len(self._free)

    def allocate(self) -> int:
        if not self._free:
            raise KVCacheExhausted(f"all {self.num_blocks} blocks are allocated")
        b = self._free.pop()
        self._refs[b] = 1
        return b

    def allocate_for(self, num_tokens: int, block_size: int) -> List[int]:
        need = -(-int(num_tokens) // int(block_size))
        if need > len(self._free):
            raise KVCacheExhausted(f"{need} blocks needed for {num_tokens} tokens, {len(self._free)} free")
        return [self.allocate() for _ in range(need)]

    def is_allocated(self, b: int) -> bool:
        return 0 <= b < self.num_blocks and self._refs[b] > 0

    def refcount(self, b: int) -> int:
        return self._refs[b]

    def retain(self, b: int) -> None:
        if not self.is_allocated(b):
            raise ValueError(f"retain of block {b}, which is not allocated")
        self._refs[b] += 1

    def release(self, b: int) -> bool:
        """Drop one reference; returns True when the block went back on the free stack."""
        if not self.is_allocated(b):
            raise ValueError(f"release of block {b}, which is not allocated")
        self._refs[b] -= 1
        if self._refs[b] == 0:
            self._free.append(int(b))
            return True
        return False

    def free(self, b: int) -> None:
        """Return a block held by exactly one owner (double or foreign frees raise)."""
        if not self.is_allocated(b):
            raise ValueError(f"free of block {b}, which is not allocated")
        if self._refs[b] != 1:
            raise ValueError(f"free of block {b} with refcount {self._refs[b]}; use release")
        self.release(b)

    def free_all(self, ids: Iterable[int]) -> None:
        for b in ids:
            self.free(b)

    def allocated_ids(self) -> np.ndarray:
        return np.nonzero(np.asarray(self._refs))[0]

    def free_ids(self) -> List[int]:
        return list(self._free)


@dataclass
class _Seq:
    blocks: List[int] = field(default_factory=list)
    length: int = 0
    live: bool = True


@dataclass
class StepBatch:
    """Metadata of one step for the device calls (all int32, host memory)."""
    seq_ids: List[int]
    slot_mapping: np.ndarray      # [T]
    copy_pairs: np.ndarray        # [n, 2] (src, dst), to run before the write
    block_tables: np.ndarray      # [S, width]
    seq_lens: np.ndarray          # [S] after the step's writes
    q_lens: np.ndarray            # [S]


class PagedKVManager:
    """Block tables and lengths of many sequences over one ``BlockAllocator``.
    ``window`` > 0: sliding-window attention of that many tokens (blocks that
    leave every query's window are released at each step)."""

    def __init__(self, num_blocks: int, block_size: int = 16, first_pops: Optional[Sequence[int]] = None,
                 window: int = 0):
        if window < 0:
            raise ValueError("window must be >= 0")
        self.block_size = int(block_size)
        self.window = int(window)
        self.alloc = BlockAllocator(num_blocks, first_pops)
        self._seqs: List[_Seq] = []
        self._tab = None          # last block-table array built, its sequence list and row contents
        self._tab_ids: List[int] = []
        self._tab_rows: List[tuple] = []

    # -- sequences --------------------------------------------------------
    def add_sequence(self, num_tokens: int = 0, shared_from: Optional[int] = None, shared_tokens: int = 0) -> int:
        """New sequence holding ``num_tokens`` cached tokens.  With ``shared_from``,
        its first ``shared_tokens`` tokens (a whole number of blocks) reuse that
        sequence's blocks (one more reference each) and only the rest is allocated."""
        bs = self.block_size
        shared: List[int] = []
        if shared_from is not None:
            if shared_tokens % bs != 0 or shared_tokens > self._seqs[shared_from].length:
                raise ValueError("shared prefix must be whole blocks of the source sequence")
            shared = self._seqs[shared_from].blocks[: shared_tokens // bs]
        own = self.alloc.allocate_for(num_tokens - len(shared) * bs, bs)
        for b in shared:
            self.alloc.retain(b)
        self._seqs.append(_Seq(blocks=list(shared) + own, length=int(num_tokens)))
        return len(self._seqs) - 1

    def fork(self, sid: int) -> int:
        s = self._seqs[sid]
        for b in s.blocks:
            if b >= 0:
                self.alloc.retain(b)
        self._seqs.append(_Seq(blocks=list(s.blocks), length=s.length))
        return len(self._seqs) - 1

    def finish(self, sid: int) -> None:
        s = self._seqs[sid]
        if not s.live:
            return
        for b in s.blocks:
            if b >= 0:
                self.alloc.release(b)
        s.blocks = []
        s.live = False

    def seq_len(self, sid: int) -> int:
        return self._seqs[sid].length

    def blocks(self, sid: int) -> List[int]:
        return list(self._seqs[sid].blocks)

    def slots(self, sid: int, start: int, n: int) -> np.ndarray:
        """Slot numbers of the existing positions start..start+n-1 of ``sid``."""
        s = self._seqs[sid]
        if start < 0 or start + n > s.length:
            raise ValueError("positions outside the sequence")
        pos = np.arange(start, start + n, dtype=np.int64)
        bl = np.asarray(s.blocks, np.int64)
        if n and bl[start // self.block_size] < 0:
            raise ValueError("positions in blocks released by the sliding window")
        return (bl[pos // self.block_size] * self.block_size + pos % self.block_size).astype(np.int32)

    # -- writes -----------------------------------------------------------
    def append(self, sid: int, n: int, slots: Optional[list] = None, copies: Optional[list] = None):
        """Reserve the next ``n`` positions of ``sid``: returns (slots, copy_pairs)
        (appended to the given lists when passed)."""
        s = self._seqs[sid]
        bs = self.block_size
        blocks, refs, alloc = s.blocks, self.alloc._refs, self.alloc
        slots = [] if slots is None else slots
        copies = [] if copies is None else copies
        for pos in range(s.length, s.length + int(n)):
            idx, off = divmod(pos, bs)
            if idx == len(blocks):
                blocks.append(alloc.allocate())
            elif refs[blocks[idx]] > 1:              # shared: copy before the first divergent write
                b = blocks[idx]
                nb = alloc.allocate()
                copies.append((b, nb))
                alloc.release(b)
                blocks[idx] = nb
            slots.append(blocks[idx] * bs + off)
        s.length += int(n)
        return slots, copies

    def release_out_of_window(self, sid: int, q_len: int) -> None:
        """Release the blocks of ``sid`` that hold no position the step's
        queries (its last ``q_len`` positions) can see; entries become -1."""
        s = self._seqs[sid]
        lo = max(0, s.length - int(q_len) - self.window + 1)
        blocks = s.blocks
        for lb in range(min(lo // self.block_size, len(blocks))):
            if blocks[lb] >= 0:
                self.alloc.release(blocks[lb])
                blocks[lb] = -1

    def step(self, seq_ids: Sequence[int], q_lens: Sequence[int], width: Optional[int] = None) -> StepBatch:
        """Reserve ``q_lens[i]`` new positions of each listed sequence (in order)
        and return the metadata of the step."""
        slots: List[int] = []
        copies: List[tuple] = []
        for sid, n in zip(seq_ids, q_lens):
            self.append(sid, n, slots, copies)
            if self.window:
                self.release_out_of_window(sid, n)
        return StepBatch(
            seq_ids=list(seq_ids),
            slot_mapping=np.asarray(slots, np.int32),
            copy_pairs=np.asarray(copies, np.int32).reshape(-1, 2),
            block_tables=self.block_tables(seq_ids, width),
            seq_lens=np.asarray([self._seqs[s].length for s in seq_ids], np.int32),
            q_lens=np.asarray(q_lens, np.int32),
        )

    def block_tables(self, seq_ids: Sequence[int], width: Optional[int] = None) -> np.ndarray:
        """[S, width] int32 tables (zero past each sequence's blocks).  Rows that
        did not change since the last call for the same sequences and width
        are taken from that call's array."""
        seqs = self._seqs
        rows = [tuple(seqs[s].blocks) for s in seq_ids]
        need = max([len(r) for r in rows] + [1])
        width = need if width is None else int(width)
        if width < need:
            raise ValueError(f"table width {width} < {need} blocks")
        prev = self._tab
        if prev is not None and prev.shape == (len(rows), width) and self._tab_ids == list(seq_ids):
            out = prev.copy()
            for r, (new, old) in enumerate(zip(rows, self._tab_rows)):
                if new != old:
                    out[r, :] = 0
                    out[r, : len(new)] = new
        else:
            out = np.zeros((len(rows), width), np.int32)
            for r, bl in enumerate(rows):
                out[r, : len(bl)] = bl
        self._tab, self._tab_ids, self._tab_rows = out, list(seq_ids), rows
        return out

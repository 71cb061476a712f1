"""Host-side integer bookkeeping that feeds the paged-attention kernels.

Block allocator, per-sequence block tables and lengths, refcounts,
fork/copy-on-write, the sliding-window release, and the per-step metadata
arrays (slot mapping, block tables, lengths, copy pairs) handed to
``pa_write_kv`` / ``pa_attend`` / ``pa_copy_blocks``.  The work is done by
the native manager in libpa.so (``include/pa_host.h``); this module only
marshals arguments and turns statuses into exceptions.  No device work.

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
* [manager] "Step 4: The Prefix Tree (Radix Trie)" and "Step 2: The Block
  Pool": published full blocks form a tree keyed by their token ids, so a
  prompt starting with a known prefix reuses its blocks
  (``add_sequence_prefix``, ``publish``); zero-refcount blocks are reclaimed
  least recently used first.
A block whose refcount drops to zero goes straight back on the free stack,
unless it is published in the prefix cache: then it stays cached until an
allocation finds the free stack empty and evicts the least recently released
cached block (with its subtree).  A step either reserves every listed
sequence's positions or changes nothing.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Iterable, List, Optional, Sequence

import numpy as np

from ._lib import cdll

_OK, _ARG, _EXHAUSTED, _NOT_ALLOCATED, _SHARED, _CAPACITY, _RELEASED = 0, -1, -2, -3, -4, -5, -6


class KVCacheExhausted(RuntimeError):
    """The pool cannot supply the requested blocks."""


_bound = None


def _native():
    """libpa.so with the host-manager signatures set (once)."""
    global _bound
    if _bound is not None:
        return _bound
    lib = cdll()
    vp, i32 = ctypes.c_void_p, ctypes.c_int32
    sig = {
        "pa_mgr_create": ([i32, i32, vp, i32], vp),
        "pa_mgr_destroy": ([vp], None),
        "pa_mgr_num_blocks": ([vp], i32),
        "pa_mgr_num_free": ([vp], i32),
        "pa_mgr_num_cached": ([vp], i32),
        "pa_mgr_add_sequence_prefix": ([vp, vp, i32, vp, vp], i32),
        "pa_mgr_publish": ([vp, i32, vp, i32], i32),
        "pa_mgr_allocate": ([vp, i32, vp], i32),
        "pa_mgr_refcount": ([vp, i32], i32),
        "pa_mgr_retain": ([vp, i32], i32),
        "pa_mgr_release": ([vp, i32, vp], i32),
        "pa_mgr_free": ([vp, i32], i32),
        "pa_mgr_free_all": ([vp, vp, i32], i32),
        "pa_mgr_free_ids": ([vp, vp, i32], i32),
        "pa_mgr_refcounts": ([vp, vp, i32], i32),
        "pa_mgr_add_sequence": ([vp, i32, i32, i32, vp], i32),
        "pa_mgr_fork": ([vp, i32, vp], i32),
        "pa_mgr_finish": ([vp, i32], i32),
        "pa_mgr_num_seqs": ([vp], i32),
        "pa_mgr_seq_len": ([vp, i32], i32),
        "pa_mgr_seq_blocks": ([vp, i32, vp, i32], i32),
        "pa_mgr_slots": ([vp, i32, i32, i32, vp], i32),
        "pa_mgr_append": ([vp, i32, i32, vp, vp, i32, vp], i32),
        "pa_mgr_release_out_of_window": ([vp, i32, i32], i32),
        "pa_mgr_step_width": ([vp, vp, vp, i32], i32),
        "pa_mgr_step": ([vp, vp, vp, i32, i32, vp, vp, i32, vp, vp, vp], i32),
        "pa_mgr_block_tables": ([vp, vp, i32, i32, vp], i32),
        "pa_host_status_str": ([i32], ctypes.c_char_p),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    _bound = lib
    return lib


def _raise(status: int, what: str):
    msg = f"{what}: {_native().pa_host_status_str(status).decode()}"
    if status == _EXHAUSTED:
        raise KVCacheExhausted(msg)
    if status in (_ARG, _NOT_ALLOCATED, _SHARED, _RELEASED):
        raise ValueError(msg)
    raise RuntimeError(msg)


def _ok(status: int, what: str) -> int:
    if status < 0:
        _raise(status, what)
    return status


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int32)


class _Handle:
    """Owns one native manager; destroyed with the last Python reference."""

    def __init__(self, num_blocks: int, block_size: int, first_pops, window: int):
        if num_blocks <= 0:
            raise ValueError("num_blocks must be positive")
        if window < 0:
            raise ValueError("window must be >= 0")
        lib = _native()
        pops = None
        if first_pops is not None:
            pops = _i32(first_pops)
            if pops.shape != (num_blocks,):
                raise ValueError("first_pops must be a permutation of range(num_blocks)")
        ptr = lib.pa_mgr_create(int(num_blocks), int(block_size), None if pops is None else pops.ctypes.data,
                                int(window))
        if not ptr:
            raise ValueError("first_pops must be a permutation of range(num_blocks)")
        self.ptr = ptr
        self._lib = lib

    def __del__(self):
        if getattr(self, "ptr", None):
            self._lib.pa_mgr_destroy(self.ptr)
            self.ptr = None


class BlockAllocator:
    """Fixed pool of block ids: LIFO free stack, allocated set, refcounts."""

    def __init__(self, num_blocks: int, first_pops: Optional[Sequence[int]] = None, _handle: _Handle = None):
        self._h = _handle if _handle is not None else _Handle(num_blocks, 1, first_pops, 0)
        self._lib = _native()
        self.num_blocks = self._lib.pa_mgr_num_blocks(self._h.ptr)

    @property
    def num_free(self) -> int:
        """Blocks on the free stack."""
        return self._lib.pa_mgr_num_free(self._h.ptr)

    @property
    def num_cached(self) -> int:
        """Blocks held by nobody but kept in the prefix cache (reclaimable)."""
        return self._lib.pa_mgr_num_cached(self._h.ptr)

    def can_allocate(self, num_blocks: int) -> bool:
        return num_blocks <= self.num_free + self.num_cached

    def allocate(self) -> int:
        out = ctypes.c_int32()
        st = self._lib.pa_mgr_allocate(self._h.ptr, 1, ctypes.addressof(out))
        if st == _EXHAUSTED:
            raise KVCacheExhausted(f"all {self.num_blocks} blocks are allocated")
        _ok(st, "allocate")
        return out.value

    def allocate_for(self, num_tokens: int, block_size: int) -> List[int]:
        need = max(0, -(-int(num_tokens) // int(block_size)))
        out = np.empty(max(need, 1), np.int32)
        st = self._lib.pa_mgr_allocate(self._h.ptr, need, out.ctypes.data)
        if st == _EXHAUSTED:
            raise KVCacheExhausted(f"{need} blocks needed for {num_tokens} tokens, {self.num_free} free")
        _ok(st, "allocate_for")
        return out[:need].tolist()

    def is_allocated(self, b: int) -> bool:
        return self._lib.pa_mgr_refcount(self._h.ptr, int(b)) > 0

    def refcount(self, b: int) -> int:
        r = self._lib.pa_mgr_refcount(self._h.ptr, int(b))
        if r < 0:
            raise IndexError(f"block {b} is outside the pool")
        return r

    def retain(self, b: int) -> None:
        st = self._lib.pa_mgr_retain(self._h.ptr, int(b))
        if st == _NOT_ALLOCATED:
            raise ValueError(f"retain of block {b}, which is not allocated")
        _ok(st, "retain")

    def release(self, b: int) -> bool:
        """Drop one reference; returns True when the block went back on the free stack."""
        freed = ctypes.c_int32()
        st = self._lib.pa_mgr_release(self._h.ptr, int(b), ctypes.addressof(freed))
        if st == _NOT_ALLOCATED:
            raise ValueError(f"release of block {b}, which is not allocated")
        _ok(st, "release")
        return bool(freed.value)

    def free(self, b: int) -> None:
        """Return a block held by exactly one owner (double or foreign frees raise)."""
        st = self._lib.pa_mgr_free(self._h.ptr, int(b))
        if st == _NOT_ALLOCATED:
            raise ValueError(f"free of block {b}, which is not allocated")
        if st == _SHARED:
            raise ValueError(f"free of block {b} with refcount {self.refcount(b)}; use release")
        _ok(st, "free")

    def free_all(self, ids: Iterable[int]) -> None:
        for b in ids:
            self.free(b)

    def refcounts(self) -> np.ndarray:
        out = np.empty(self.num_blocks, np.int32)
        _ok(self._lib.pa_mgr_refcounts(self._h.ptr, out.ctypes.data, self.num_blocks), "refcounts")
        return out

    def allocated_ids(self) -> np.ndarray:
        return np.nonzero(self.refcounts())[0]

    def free_ids(self) -> List[int]:
        n = self.num_free
        out = np.empty(max(n, 1), np.int32)
        n = _ok(self._lib.pa_mgr_free_ids(self._h.ptr, out.ctypes.data, n), "free_ids")
        return out[:n].tolist()


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
        if block_size <= 0:
            raise ValueError("block_size must be positive")
        self._h = _Handle(num_blocks, block_size, first_pops, window)
        self._lib = _native()
        self.block_size = int(block_size)
        self.window = int(window)
        self.alloc = BlockAllocator(num_blocks, _handle=self._h)

    # -- sequences --------------------------------------------------------
    def add_sequence(self, num_tokens: int = 0, shared_from: Optional[int] = None, shared_tokens: int = 0) -> int:
        """New sequence holding ``num_tokens`` cached tokens.  With ``shared_from``,
        its first ``shared_tokens`` tokens (a whole number of blocks) reuse that
        sequence's blocks (one more reference each) and only the rest is allocated."""
        sid = ctypes.c_int32()
        src = -1 if shared_from is None else int(shared_from)
        st = self._lib.pa_mgr_add_sequence(self._h.ptr, int(num_tokens), src,
                                           0 if shared_from is None else int(shared_tokens), ctypes.addressof(sid))
        if st == _ARG and shared_from is not None:
            raise ValueError("shared prefix must be whole blocks of the source sequence")
        _ok(st, "add_sequence")
        return sid.value

    def add_sequence_prefix(self, tokens: Sequence[int]) -> tuple:
        """New sequence for a prompt: it starts with the longest chain of
        published full blocks matching ``tokens`` (leaving at least one token);
        returns (sequence id, cached tokens = its length)."""
        t = _i32(tokens)
        sid, cached = ctypes.c_int32(), ctypes.c_int32()
        _ok(self._lib.pa_mgr_add_sequence_prefix(self._h.ptr, t.ctypes.data, len(t), ctypes.addressof(sid),
                                                 ctypes.addressof(cached)), "add_sequence_prefix")
        return sid.value, cached.value

    def publish(self, sid: int, tokens: Sequence[int]) -> None:
        """Enter the sequence's full blocks holding ``tokens`` into the prefix cache."""
        t = _i32(tokens)
        _ok(self._lib.pa_mgr_publish(self._h.ptr, int(sid), t.ctypes.data, len(t)), "publish")

    def fork(self, sid: int) -> int:
        child = ctypes.c_int32()
        _ok(self._lib.pa_mgr_fork(self._h.ptr, int(sid), ctypes.addressof(child)), "fork")
        return child.value

    def finish(self, sid: int) -> None:
        _ok(self._lib.pa_mgr_finish(self._h.ptr, int(sid)), "finish")

    @property
    def num_seqs(self) -> int:
        return self._lib.pa_mgr_num_seqs(self._h.ptr)

    def seq_len(self, sid: int) -> int:
        n = self._lib.pa_mgr_seq_len(self._h.ptr, int(sid))
        if n < 0:
            raise IndexError(f"no sequence {sid}")
        return n

    def blocks(self, sid: int) -> List[int]:
        cap = -(-self.seq_len(sid) // self.block_size) + 1
        out = np.empty(cap, np.int32)
        n = _ok(self._lib.pa_mgr_seq_blocks(self._h.ptr, int(sid), out.ctypes.data, cap), "blocks")
        return out[:n].tolist()

    def slots(self, sid: int, start: int, n: int) -> np.ndarray:
        """Slot numbers of the existing positions start..start+n-1 of ``sid``."""
        out = np.empty(max(int(n), 1), np.int32)
        st = self._lib.pa_mgr_slots(self._h.ptr, int(sid), int(start), int(n), out.ctypes.data)
        if st == _RELEASED:
            raise ValueError("positions in blocks released by the sliding window")
        if st == _ARG:
            raise ValueError("positions outside the sequence")
        _ok(st, "slots")
        return out[:int(n)]

    # -- writes -----------------------------------------------------------
    def append(self, sid: int, n: int, slots: Optional[list] = None, copies: Optional[list] = None):
        """Reserve the next ``n`` positions of ``sid``: returns (slots, copy_pairs)
        (appended to the given lists when passed)."""
        n = int(n)
        cap = n // self.block_size + 2
        sl = np.empty(max(n, 1), np.int32)
        cp = np.empty((cap, 2), np.int32)
        nc = ctypes.c_int32()
        _ok(self._lib.pa_mgr_append(self._h.ptr, int(sid), n, sl.ctypes.data, cp.ctypes.data, cap,
                                    ctypes.addressof(nc)), "append")
        slots = [] if slots is None else slots
        copies = [] if copies is None else copies
        slots += sl[:n].tolist()
        copies += [tuple(p) for p in cp[:nc.value].tolist()]
        return slots, copies

    def release_out_of_window(self, sid: int, q_len: int) -> None:
        """Release the blocks of ``sid`` that hold no position the step's
        queries (its last ``q_len`` positions) can see; entries become -1."""
        _ok(self._lib.pa_mgr_release_out_of_window(self._h.ptr, int(sid), int(q_len)), "release_out_of_window")

    def step_width(self, seq_ids, q_lens) -> int:
        """Table width a step of these sequences needs (no state change)."""
        sids, ql = _i32(seq_ids), _i32(q_lens)
        return _ok(self._lib.pa_mgr_step_width(self._h.ptr, sids.ctypes.data, ql.ctypes.data, len(sids)), "step")

    def step(self, seq_ids: Sequence[int], q_lens: Sequence[int], width: Optional[int] = None) -> StepBatch:
        """Reserve ``q_lens[i]`` new positions of each listed sequence (in order,
        ids distinct) and return the metadata of the step.  Either every
        position is reserved or nothing changes (``KVCacheExhausted``)."""
        sids, ql = _i32(seq_ids), _i32(q_lens)
        if sids.shape != ql.shape or sids.ndim != 1:
            raise ValueError("one q_len per sequence id")
        S = len(sids)
        need = self.step_width(sids, ql)
        width = need if width is None else int(width)
        if width < need:
            raise ValueError(f"table width {width} < {need} blocks")
        cap = int((ql // self.block_size).sum()) + 2 * S
        slots = np.empty(int(ql.sum()), np.int32)
        copies = np.empty((max(cap, 1), 2), np.int32)
        tables = np.empty((S, width), np.int32)
        lens = np.empty(S, np.int32)
        nc = ctypes.c_int32()
        _ok(self._lib.pa_mgr_step(self._h.ptr, sids.ctypes.data, ql.ctypes.data, S, width, slots.ctypes.data,
                                  copies.ctypes.data, cap, ctypes.addressof(nc), tables.ctypes.data,
                                  lens.ctypes.data), "step")
        return StepBatch(seq_ids=list(seq_ids), slot_mapping=slots, copy_pairs=copies[:nc.value],
                         block_tables=tables, seq_lens=lens, q_lens=ql)

    def block_tables(self, seq_ids: Sequence[int], width: Optional[int] = None) -> np.ndarray:
        """[S, width] int32 tables (zero past each sequence's blocks)."""
        sids = _i32(seq_ids)
        need = max([len(self.blocks(int(s))) for s in sids] + [1])
        width = need if width is None else int(width)
        if width < need:
            raise ValueError(f"table width {width} < {need} blocks")
        out = np.empty((len(sids), width), np.int32)
        _ok(self._lib.pa_mgr_block_tables(self._h.ptr, sids.ctypes.data, len(sids), width, out.ctypes.data),
            "block_tables")
        return out

"""Continuous-batching scheduler (``include/pa_sched.h``): ctypes wrapper of
the native scheduler in libpa.so.  It owns its block manager; each ``step``
runs the four phases (release finished requests, grow the running ones,
admit waiting ones with look-ahead and a blocking fallback, assemble the
batch) and reserves the batch's positions.  Host-only.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

from ._lib import cdll
from .host import PagedKVManager, _ok

_bound = None


def _native():
    global _bound
    if _bound is not None:
        return _bound
    lib = cdll()
    vp, i32 = ctypes.c_void_p, ctypes.c_int32
    sig = {
        "pa_sched_create": ([vp, i32, i32, i32, i32], vp),
        "pa_sched_destroy": ([vp], None),
        "pa_sched_add": ([vp, i32, i32, vp], i32),
        "pa_sched_add_tokens": ([vp, vp, i32, i32, vp], i32),
        "pa_sched_cached_tokens": ([vp], ctypes.c_int64),
        "pa_sched_max_width": ([vp], i32),
        "pa_sched_step": ([vp, vp, vp, vp, vp, vp, i32, vp, i32, vp, vp, vp], i32),
        "pa_sched_counts": ([vp, vp, vp, vp, vp, vp], i32),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    _bound = lib
    return lib


@dataclass
class SchedStep:
    """One scheduled step (views into the scheduler's buffers, valid until
    the next step)."""
    rids: np.ndarray          # [S] request of each sequence of the batch
    sids: np.ndarray          # [S] its manager sequence id
    q_lens: np.ndarray        # [S] rows: 1 for a decode, the prompt length for a prefill
    finished: np.ndarray      # requests released at the start of this step
    slot_mapping: np.ndarray  # [sum q_lens]
    block_tables: np.ndarray  # [S, width]
    seq_lens: np.ndarray      # [S]


class Scheduler:
    """Requests over a pool of ``num_blocks`` blocks of ``block_size`` tokens."""

    def __init__(self, num_blocks: int, block_size: int = 16, max_batch_tokens: int = 8192, max_seqs: int = 256,
                 lookahead: int = 4, max_skips: int = 8, first_pops: Optional[Sequence[int]] = None):
        self.mgr = PagedKVManager(num_blocks, block_size, first_pops)
        self._lib = _native()
        ptr = self._lib.pa_sched_create(self.mgr._h.ptr, int(max_batch_tokens), int(max_seqs), int(lookahead),
                                        int(max_skips))
        if not ptr:
            raise ValueError("invalid scheduler limits")
        self.ptr = ptr
        self.max_tokens, self.max_seqs = int(max_batch_tokens), int(max_seqs)
        self._bufs = None
        self._width = 0

    def __del__(self):
        if getattr(self, "ptr", None):
            self._lib.pa_sched_destroy(self.ptr)
            self.ptr = None

    def add(self, prompt_len: int, new_tokens: int) -> int:
        rid = ctypes.c_int32()
        _ok(self._lib.pa_sched_add(self.ptr, int(prompt_len), int(new_tokens), ctypes.addressof(rid)), "add")
        return rid.value

    def add_tokens(self, tokens, new_tokens: int) -> int:
        """Queue a request whose prompt is ``tokens`` (matched against and then
        published into the prefix cache)."""
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        rid = ctypes.c_int32()
        _ok(self._lib.pa_sched_add_tokens(self.ptr, t.ctypes.data, len(t), int(new_tokens), ctypes.addressof(rid)),
            "add")
        return rid.value

    @property
    def cached_tokens(self) -> int:
        return self._lib.pa_sched_cached_tokens(self.ptr)

    @property
    def max_width(self) -> int:
        return self._lib.pa_sched_max_width(self.ptr)

    def counts(self) -> dict:
        v = [ctypes.c_int32() for _ in range(4)]
        g = ctypes.c_int64()
        _ok(self._lib.pa_sched_counts(self.ptr, *[ctypes.addressof(x) for x in v], ctypes.addressof(g)), "counts")
        return {"waiting": v[0].value, "running": v[1].value, "finished": v[2].value,
                "blocking": bool(v[3].value), "generated": g.value}

    def done(self) -> bool:
        c = self.counts()
        return c["waiting"] == 0 and c["running"] == 0

    def _buffers(self, width: int):
        if self._bufs is None or self._width < width:
            S, T = self.max_seqs, self.max_tokens
            self._width = max(width, 1)
            self._bufs = {
                "rids": np.empty(S, np.int32), "sids": np.empty(S, np.int32), "q_lens": np.empty(S, np.int32),
                "finished": np.empty(S, np.int32), "slots": np.empty(T, np.int32),
                "tables": np.empty(S * self._width, np.int32), "lens": np.empty(S, np.int32),
                "n": ctypes.c_int32(), "nf": ctypes.c_int32(),
            }
        return self._bufs

    def step(self, width: Optional[int] = None) -> SchedStep:
        """Schedule and reserve one step.  ``width``: block-table width of the
        output (at least ``max_width``; default exactly that)."""
        width = self.max_width if width is None else int(width)
        b = self._buffers(width)
        _ok(self._lib.pa_sched_step(self.ptr, b["rids"].ctypes.data, b["sids"].ctypes.data, b["q_lens"].ctypes.data,
                                    ctypes.addressof(b["n"]), b["finished"].ctypes.data, self.max_seqs,
                                    ctypes.addressof(b["nf"]), width, b["slots"].ctypes.data,
                                    b["tables"].ctypes.data, b["lens"].ctypes.data), "schedule")
        n, nf = b["n"].value, b["nf"].value
        q = b["q_lens"][:n]
        return SchedStep(rids=b["rids"][:n], sids=b["sids"][:n], q_lens=q, finished=b["finished"][:nf],
                         slot_mapping=b["slots"][:int(q.sum())], block_tables=b["tables"][:n * width].reshape(n, width),
                         seq_lens=b["lens"][:n])

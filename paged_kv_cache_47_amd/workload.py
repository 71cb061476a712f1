"""Run a seeded synthetic workload (``synthetic.Workload``) through the
host bookkeeping and libpa.so.

Sequences are set up the way the workloads describe them: each takes the
blocks of its cached context in order; with a shared prefix, the first
request's prefix blocks are shared by every other request (one reference
each) and beam requests are then forked; int8 pools get their cached context
written token by token through ``pa_write_kv``.  A step reserves the new
positions (growing tables, copy-on-write of shared blocks), then runs
``pa_copy_blocks`` -> ``pa_write_kv`` -> ``pa_attend`` on the current stream.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional

import numpy as np
import torch

from . import pa
from .host import PagedKVManager, StepBatch


def build_manager(w) -> tuple:
    """(manager, sequence ids in the workload's canonical order)."""
    mgr = PagedKVManager(w.num_blocks, w.block_size, w.first_pops)
    if w.beams is None:
        return mgr, [mgr.add_sequence(int(c)) for c in w.ctx_lens]
    reqs: List[int] = []
    for r, c in enumerate(w.ctx_lens):
        if r == 0:
            reqs.append(mgr.add_sequence(int(c)))
        else:
            reqs.append(mgr.add_sequence(int(c), shared_from=reqs[0], shared_tokens=w.shared_prefix))
    ids: List[int] = []
    for r, sid in enumerate(reqs):
        ids.append(sid)
        ids += [mgr.fork(sid) for _ in range(int(w.beams[r]) - 1)]
    return mgr, ids


@dataclass
class StepInputs:
    batch: StepBatch
    slot_mapping: torch.Tensor
    copy_pairs: torch.Tensor
    block_tables: torch.Tensor
    seq_lens: torch.Tensor
    q_lens: torch.Tensor
    new_k: torch.Tensor
    new_v: torch.Tensor
    q: torch.Tensor


class DeviceRun:
    """Device pools plus host bookkeeping for one workload."""

    def __init__(self, w, device: str = "cuda", context_batch_tokens: int = 1 << 18):
        self.w = w
        self.device = torch.device(device)
        self.mgr, self.ids = build_manager(w)
        self.k_cache = torch.from_numpy(w.pool_k).to(self.device)
        self.v_cache = torch.from_numpy(w.pool_v).to(self.device)
        self.i8 = w.kv_dtype == "i8"
        self.k_scale = torch.from_numpy(w.pool_k_scale).to(self.device) if self.i8 else None
        self.v_scale = torch.from_numpy(w.pool_v_scale).to(self.device) if self.i8 else None
        if w.context is not None:
            self._write_context(context_batch_tokens)

    def _write_context(self, batch_tokens: int) -> None:
        pend_k, pend_v, pend_s, n = [], [], [], 0

        def flush():
            nonlocal pend_k, pend_v, pend_s, n
            if n:
                k = torch.from_numpy(np.concatenate(pend_k)).to(self.device)
                v = torch.from_numpy(np.concatenate(pend_v)).to(self.device)
                s = torch.from_numpy(np.concatenate(pend_s)).to(self.device)
                pa.pa_write_kv(k, v, s, self.k_cache, self.v_cache, self.k_scale, self.v_scale)
            pend_k, pend_v, pend_s, n = [], [], [], 0

        for i, sid in enumerate(self.ids):
            c = int(self.w.ctx_lens[i])
            if c == 0:
                continue
            k, v = self.w.context(i)
            pend_k.append(k)
            pend_v.append(v)
            pend_s.append(self.mgr.slots(sid, 0, c))
            n += c
            if n >= batch_tokens:
                flush()
        flush()

    def prepare(self, s: int = 0, width: Optional[int] = None) -> StepInputs:
        st = self.w.step(s)
        b = self.mgr.step(self.ids, st.q_lens, width)
        d = self.device

        def dev(a):
            return torch.from_numpy(np.ascontiguousarray(a)).to(d)

        return StepInputs(b, dev(b.slot_mapping), dev(b.copy_pairs), dev(b.block_tables), dev(b.seq_lens),
                          dev(b.q_lens), dev(st.new_k), dev(st.new_v), dev(st.q))

    def write(self, x: StepInputs) -> None:
        if x.copy_pairs.shape[0]:
            pa.pa_copy_blocks(self.k_cache, self.v_cache, x.copy_pairs, self.k_scale, self.v_scale)
        pa.pa_write_kv(x.new_k, x.new_v, x.slot_mapping, self.k_cache, self.v_cache, self.k_scale, self.v_scale)

    def attend(self, x: StepInputs, out=None, workspace=None, **opts) -> torch.Tensor:
        return pa.pa_attend(x.q, self.k_cache, self.v_cache, x.block_tables, x.seq_lens, x.q_lens,
                            x.batch.seq_lens, x.batch.q_lens, self.w.scale, out=out, workspace=workspace,
                            k_scale=self.k_scale, v_scale=self.v_scale, **opts)

    def run(self, x: StepInputs, **opts) -> torch.Tensor:
        self.write(x)
        return self.attend(x, **opts)

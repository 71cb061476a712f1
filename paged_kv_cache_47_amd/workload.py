"""Run a seeded synthetic workload (``synthetic.Workload``) through the
host bookkeeping and libpa.so.

Sequences are set up the way the workloads describe them: each takes the
blocks of its cached context in order; with a shared prefix, the first
request's prefix blocks are shared by every other request (one reference
each) and beam requests are then forked; int8 pools get their cached context
written token by token through ``pa_write_kv``.  A step reserves the new
positions (growing tables, copy-on-write of shared blocks), then runs
``pa_copy_blocks`` -> ``pa_write_kv`` -> ``pa_attend`` on the current stream.
With several layers the pools hold every layer of a block; one step's
metadata serves all layers, and each layer's write and attention follow
each other (as in a model), the attention of layers after the first reusing
the first layer's plan.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import List, Optional

import numpy as np
import torch

from . import pa
from .host import PagedKVManager, StepBatch


def build_manager(w) -> tuple:
    """(manager, sequence ids in the workload's canonical order)."""
    mgr = PagedKVManager(w.num_blocks, w.block_size, w.first_pops, window=w.window)
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
        # bf16 values are drawn as float32 (exactly representable) and narrowed on the device
        self.act_dtype = torch.bfloat16 if w.kv_dtype == "bf16" else torch.float16
        self.k_cache = self._dev(w.pool_k, w.kv_dtype == "bf16")
        self.v_cache = self._dev(w.pool_v, w.kv_dtype == "bf16")
        self.i8 = w.kv_dtype == "i8"
        self.layers = int(w.num_layers)
        self.k_scale = torch.from_numpy(w.pool_k_scale).to(self.device) if self.i8 else None
        self.v_scale = torch.from_numpy(w.pool_v_scale).to(self.device) if self.i8 else None
        if w.context is not None:
            self._write_context(context_batch_tokens)
        self._pinned = [None, None]   # two pinned staging buffers for step metadata, used in turn
        self._copied = [None, None]   # event after the last copy out of each
        self._turn = 0
        self._ws = None               # attention workspace, grown as needed

    def _dev(self, a, narrow: bool = True) -> torch.Tensor:
        t = torch.from_numpy(np.ascontiguousarray(a)).to(self.device)
        return t.to(torch.bfloat16) if (narrow and self.act_dtype == torch.bfloat16) else t

    def _upload_i32(self, arrays) -> list:
        """The step's int32 metadata arrays packed into one pinned host buffer
        and copied to the device in one asynchronous transfer on the current
        stream; returns device views shaped like the inputs.  The device
        buffer is fresh each step, so earlier steps' views stay valid."""
        flat = [np.ascontiguousarray(a, dtype=np.int32).reshape(-1) for a in arrays]
        n = max(1, sum(a.size for a in flat))
        t = self._turn = self._turn ^ 1
        if self._copied[t] is not None:
            self._copied[t].synchronize()          # the copy that last read this buffer is done
        if self._pinned[t] is None or self._pinned[t].numel() < n:
            self._pinned[t] = torch.empty(2 * n, dtype=torch.int32, pin_memory=True)
        host = self._pinned[t].numpy()
        off = 0
        for a in flat:
            host[off:off + a.size] = a
            off += a.size
        dev = torch.empty(n, dtype=torch.int32, device=self.device)
        dev.copy_(self._pinned[t][:n], non_blocking=True)
        ev = torch.cuda.Event()
        ev.record()
        self._copied[t] = ev
        out, off = [], 0
        for a, f in zip(arrays, flat):
            out.append(dev[off:off + f.size].view(np.shape(a)))
            off += f.size
        return out

    def _write_context(self, batch_tokens: int) -> None:
        pend_k, pend_v, pend_s, n = [], [], [], 0

        ax = 0 if self.layers == 1 else 1   # token axis of the context draws

        def flush():
            nonlocal pend_k, pend_v, pend_s, n
            if n:
                k = torch.from_numpy(np.concatenate(pend_k, axis=ax)).to(self.device)
                v = torch.from_numpy(np.concatenate(pend_v, axis=ax)).to(self.device)
                s = torch.from_numpy(np.concatenate(pend_s)).to(self.device)
                for layer in range(self.layers):
                    kl, vl = (k, v) if self.layers == 1 else (k[layer], v[layer])
                    pa.pa_write_kv(kl, vl, s, self.k_cache, self.v_cache, self.k_scale, self.v_scale, layer=layer)
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

    def activations(self, s: int) -> tuple:
        """Step ``s``'s new K, new V and queries on the device (what a model
        would hand over; a leading layer axis with several layers), drawn and
        copied outside any timed region."""
        st = self.w.step(s)
        return tuple(self._dev(a) for a in (st.new_k, st.new_v, st.q))

    def prepare(self, s: int = 0, width: Optional[int] = None, acts: Optional[tuple] = None) -> StepInputs:
        """Host bookkeeping of step ``s`` (table growth, slots, copy-on-write
        pairs) and the copies of its metadata to the device; the activations
        are copied too unless ``acts`` (from ``activations``) is given."""
        st = self.w.step(s)
        b = self.mgr.step(self.ids, st.q_lens, width)
        nk, nv, q = acts if acts is not None else (self._dev(st.new_k), self._dev(st.new_v), self._dev(st.q))
        sm, cp, bt, sl, ql = self._upload_i32([b.slot_mapping, b.copy_pairs, b.block_tables, b.seq_lens, b.q_lens])
        return StepInputs(b, sm, cp, bt, sl, ql, nk, nv, q)

    def layer_acts(self, x: StepInputs, layer: int) -> tuple:
        if self.layers == 1:
            return x.new_k, x.new_v, x.q
        return x.new_k[layer], x.new_v[layer], x.q[layer]

    def copy(self, x: StepInputs) -> None:
        """The step's copy-on-write block copies (every layer of each block)."""
        if x.copy_pairs.shape[0]:
            pa.pa_copy_blocks(self.k_cache, self.v_cache, x.copy_pairs, self.k_scale, self.v_scale)

    def write_layer(self, x: StepInputs, layer: int) -> None:
        nk, nv, _ = self.layer_acts(x, layer)
        pa.pa_write_kv(nk, nv, x.slot_mapping, self.k_cache, self.v_cache, self.k_scale, self.v_scale, layer=layer)

    def write(self, x: StepInputs) -> None:
        """Copies, then every layer's KV write."""
        self.copy(x)
        for layer in range(self.layers):
            self.write_layer(x, layer)

    def attend(self, x: StepInputs, out=None, workspace=None, layer: int = 0, **opts) -> torch.Tensor:
        if workspace is None:
            need = pa.pa_attend_workspace_bytes(self.k_cache, self.w.num_q_heads, x.batch.seq_lens,
                                                x.batch.q_lens, opts.get("partition_tokens", 0),
                                                opts.get("mfma_min_rows", 0), self.w.window,
                                                opts.get("mfma_split_steps", 0))
            if self._ws is None or self._ws.numel() < need:
                self._ws = torch.empty(2 * need, dtype=torch.uint8, device=self.device)
            workspace = self._ws
        return pa.pa_attend(self.layer_acts(x, layer)[2], self.k_cache, self.v_cache, x.block_tables, x.seq_lens,
                            x.q_lens, x.batch.seq_lens, x.batch.q_lens, self.w.scale, out=out, workspace=workspace,
                            k_scale=self.k_scale, v_scale=self.v_scale, window=self.w.window, layer=layer, **opts)

    def run(self, x: StepInputs, **opts):
        """One step: copies, then per layer its write and its attention (the
        layers after the first reuse the first one's plan).  Returns the
        output (one layer) or the list of per-layer outputs."""
        if self.layers == 1:
            self.write(x)
            return self.attend(x, **opts)
        self.copy(x)
        outs = []
        for layer in range(self.layers):
            self.write_layer(x, layer)
            outs.append(self.attend(x, layer=layer, reuse_plan=layer > 0, **opts))
        return outs


class StaticSteps:
    """Fixed-shape steps of a ``DeviceRun`` issued from buffers at fixed
    device addresses, so that a whole step (block copies, then every layer's
    KV write and attention) is a list of prepared library calls, which can
    also be captured once in a HIP graph and replayed.

    Every step reserves ``q_len`` new positions for each of the run's
    sequences.  The native manager writes the step's metadata straight into
    a pinned host buffer (two of them, used in turn) laid out like the
    device buffer, and one asynchronous copy moves it over.  The attention
    launches are shaped for an upper bound on the lengths (``width`` blocks
    per sequence), so the same launches serve every step up to that bound;
    the plan kernel builds the work lists from the true device lengths.
    Copy-on-write pairs are padded to one per sequence (a step copies at most
    one block per sequence: only the block holding its first new position
    can already exist) with (-1, -1), which the copy kernel skips.
    """

    def __init__(self, run: DeviceRun, width: int, q_len: int = 1, partition_tokens: int = 0,
                 copies: bool = False):
        from . import host
        w = run.w
        self.run, self.w = run, w
        self.S = S = len(run.ids)
        self.T = T = S * int(q_len)
        self.W = W = int(width)
        self.copies = bool(copies)
        self.partition_tokens = int(partition_tokens)
        o = self.off = {"ql": 0, "sl": S, "slots": 2 * S, "cp": 2 * S + T, "tab": 4 * S + T}
        n = o["tab"] + S * W
        self.pinned = [torch.empty(n, dtype=torch.int32, pin_memory=True) for _ in range(2)]
        self.host = [p.numpy() for p in self.pinned]
        self.base = [p.data_ptr() for p in self.pinned]
        for h in self.host:
            h[:S] = q_len
        self.done = [None, None]
        self.turn = 0
        dev = self.dev = torch.zeros(n, dtype=torch.int32, device=run.device)
        self.q_lens = dev[0:S]
        self.seq_lens = dev[S:2 * S]
        self.slots = dev[2 * S:2 * S + T]
        self.pairs = dev[o["cp"]:o["cp"] + 2 * S].view(S, 2)
        self.tables = dev[o["tab"]:].view(S, W)
        # host lengths handed to the attention calls: the upper bound until a step says otherwise
        self.h_len = np.full(S, W * w.block_size, np.int32)
        self.h_ql = np.full(S, q_len, np.int32)
        L, hq, hkv, d = run.layers, w.num_q_heads, w.num_kv_heads, w.head_dim
        f16 = dict(dtype=run.act_dtype, device=run.device)
        self.new_k = torch.zeros((L, T, hkv, d), **f16)
        self.new_v = torch.zeros((L, T, hkv, d), **f16)
        self.q = torch.zeros((L, T, hq, d), **f16)
        self.out = torch.zeros((L, T, hq, d), **f16)
        # The automatic split size depends on the batch's total keys, so steps with shorter true
        # lengths could pick a smaller partition and need more split units than the bound; fixing
        # the partition the bound gets keeps every step's units (and workspace) within it.
        # The split of long row tiles is fixed the same way; with a window a tile's step count
        # depends on the alignment of its window start, not only on the length, so there row
        # tiles are never split.
        info = pa.pa_attend_plan_info(run.k_cache, hq, self.h_len, self.h_ql, window=w.window)
        if self.partition_tokens == 0:
            self.partition_tokens = info["partition_tokens"] or -1
        self.split_steps = -1 if w.window > 0 else (info["mfma_split_steps"] or -1)
        need = pa.pa_attend_workspace_bytes(run.k_cache, hq, self.h_len, self.h_ql, self.partition_tokens, 0,
                                            w.window, self.split_steps)
        self.ws = torch.empty(need, dtype=torch.uint8, device=run.device)
        self._lib = host._native()
        self._ok = host._ok
        self.mgr = run.mgr._h.ptr
        self.sids = np.asarray(run.ids, np.int32)
        self.sids_ptr = self.sids.__array_interface__["data"][0]
        self.nc = ctypes.c_int32()
        self.nc_ptr = ctypes.addressof(self.nc)
        self.calls = self._calls()
        self.graph = None

    def _calls(self) -> list:
        """The step's library calls, on the current stream."""
        run, w = self.run, self.w
        kc, vc, ks, vs = run.k_cache, run.v_cache, run.k_scale, run.v_scale
        calls = []
        if self.copies:
            calls.append(pa.prepare_copy_blocks(kc, vc, self.pairs, ks, vs))
        for layer in range(run.layers):
            calls.append(pa.prepare_write_kv(self.new_k[layer], self.new_v[layer], self.slots, kc, vc, ks, vs,
                                             layer=layer))
            calls.append(pa.prepare_attend(self.q[layer], kc, vc, self.tables, self.seq_lens, self.q_lens,
                                           self.h_len, self.h_ql, w.scale, out=self.out[layer], workspace=self.ws,
                                           k_scale=ks, v_scale=vs, partition_tokens=self.partition_tokens,
                                           window=w.window, layer=layer, reuse_plan=layer > 0,
                                           mfma_split_steps=self.split_steps))
        return calls

    def set_activations(self, s: int = None, acts=None) -> None:
        """Copy step ``s``'s activations (or ``acts`` = (new_k, new_v, q) device
        tensors with a leading layer axis when there are several layers) into
        the fixed buffers."""
        if acts is None:
            acts = self.run.activations(s)
        for dst, src in zip((self.new_k, self.new_v, self.q), acts):
            dst.copy_(src.view(dst.shape), non_blocking=True)

    def host_step(self, exact_lengths: bool = True) -> None:
        """Bookkeeping of the next step (native, into pinned memory) and the
        asynchronous copy of its metadata to the device on the current
        stream.  ``exact_lengths``: hand the step's true lengths to the
        prepared attention calls (a captured graph keeps the upper bound)."""
        t = self.turn = self.turn ^ 1
        if self.done[t] is not None:
            self.done[t].synchronize()           # the copy that last read this buffer has finished
        b, o, S = self.base[t], self.off, self.S
        self._ok(self._lib.pa_mgr_step(self.mgr, self.sids_ptr, b + 4 * o["ql"], S, self.W, b + 4 * o["slots"],
                                       b + 4 * o["cp"], S, self.nc_ptr, b + 4 * o["tab"], b + 4 * o["sl"]),
                 "step")
        h = self.host[t]
        if self.copies:
            h[o["cp"] + 2 * self.nc.value:o["cp"] + 2 * S] = -1
        elif self.nc.value:
            raise RuntimeError("a step made copy-on-write pairs but these steps were set up without copies")
        self.dev.copy_(self.pinned[t], non_blocking=True)
        ev = torch.cuda.Event()
        ev.record()
        self.done[t] = ev
        if exact_lengths:
            self.h_len[:] = h[S:2 * S]

    def lengths(self) -> np.ndarray:
        """The last step's lengths (host copy)."""
        return self.host[self.turn][self.S:2 * self.S].copy()

    def launch(self) -> None:
        """Issue the step's calls (copies, then per layer write and attention)."""
        for c in self.calls:
            c()

    def capture(self) -> None:
        """Capture the step's calls once in a HIP graph, shaped for the upper
        bound on the lengths."""
        self.h_len[:] = self.W * self.w.block_size
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            calls = self._calls()                # bound to the capture stream
            for c in calls:
                c()
        self.graph = g

    def replay(self) -> None:
        self.graph.replay()


class ServeRun:
    """A request stream (``synthetic.RequestStream``) through the native
    continuous-batching scheduler and the library: each step the scheduler
    releases finished requests, admits waiting ones and reserves the batch's
    positions (decode rows of running requests, then prefill rows of the new
    ones, packed); the step's metadata goes to the device in one copy; then
    per layer the KV write and the attention (the layers after the first
    reuse the first one's plan).  Requests with token ids start from the
    blocks the prefix cache holds for their prompt's prefix: their first step
    writes and attends only the rest of the prompt.  Shared blocks are full
    and never written again, so there are no block copies."""

    def __init__(self, rs, device: str = "cuda", acts=None):
        from .sched import Scheduler
        self.rs = rs
        self.device = torch.device(device)
        self.sched = Scheduler(rs.num_blocks, rs.block_size, rs.max_batch_tokens, rs.max_seqs, rs.lookahead,
                               rs.max_skips)
        self.next_arrival = 0
        self.step_index = 0
        self.act_dtype = torch.bfloat16 if rs.kv_dtype == "bf16" else torch.float16
        lead = () if rs.num_layers == 1 else (rs.num_layers,)
        shape = (rs.num_blocks, *lead, rs.num_kv_heads, rs.block_size, rs.head_dim)
        pool_dtype = torch.int8 if rs.kv_dtype == "i8" else self.act_dtype
        self.k_cache = torch.zeros(shape, dtype=pool_dtype, device=self.device)
        self.v_cache = torch.zeros(shape, dtype=pool_dtype, device=self.device)
        self.k_scale = self.v_scale = None
        if rs.kv_dtype == "i8":   # one fp16 scale per (block, layer, KV head)
            self.k_scale = torch.zeros(shape[:-2], dtype=torch.float16, device=self.device)
            self.v_scale = torch.zeros(shape[:-2], dtype=torch.float16, device=self.device)
        self.acts = acts          # None: draw each step's activations; else a callable (step, rows) -> tensors
        self._pinned = [None, None]
        self._copied = [None, None]
        self._turn = 0
        self._ws = None
        self._meta = None         # device int32 buffer of the step's metadata, reused every step
        self.width = 0
        # Per-step calls go straight to the library: the pools, their descriptors, the options and
        # the stream are fixed for the run and checked once here; the step's own arguments are
        # produced by the scheduler.  The library calls go to the stream current at construction,
        # the metadata copy to the current stream: step with that same stream current.
        self._lib = pa.load_library()
        self._descs = [pa.cache_desc(self.k_cache, layer) for layer in range(rs.num_layers)]
        self._dptr = [ctypes.pointer(d) for d in self._descs]
        self._opts = [pa._opts(reuse_plan=layer > 0) for layer in range(rs.num_layers)]
        self._optr = [ctypes.pointer(o) for o in self._opts]
        self._stream = ctypes.c_void_p(torch.cuda.current_stream(self.device).cuda_stream)
        self._pools = tuple(None if t is None else t.data_ptr()
                            for t in (self.k_cache, self.v_cache, self.k_scale, self.v_scale))
        for _ in range(int(np.sum(rs.arrivals <= 0))):
            self._arrive()

    def _arrive(self) -> None:
        i = self.next_arrival
        if self.rs.tokens is not None:
            self.sched.add_tokens(self.rs.tokens[i], int(self.rs.new_tokens[i]))
        else:
            self.sched.add(int(self.rs.prompts[i]), int(self.rs.new_tokens[i]))
        self.next_arrival += 1

    def done(self) -> bool:
        return self.next_arrival == len(self.rs.prompts) and self.sched.done()

    def _upload(self, arrays) -> list:
        flat = [np.ascontiguousarray(a, dtype=np.int32).reshape(-1) for a in arrays]
        n = max(1, sum(a.size for a in flat))
        t = self._turn = self._turn ^ 1
        if self._copied[t] is not None:
            self._copied[t].synchronize()
        if self._pinned[t] is None or self._pinned[t].numel() < n:
            self._pinned[t] = torch.empty(2 * n, dtype=torch.int32, pin_memory=True)
        host = self._pinned[t].numpy()
        off = 0
        for a in flat:
            host[off:off + a.size] = a
            off += a.size
        # one device buffer for every step: this copy is ordered after the previous step's kernels
        if self._meta is None or self._meta.numel() < n:
            self._meta = torch.empty(2 * n, dtype=torch.int32, device=self.device)
        dev = self._meta[:n]
        dev.copy_(self._pinned[t][:n], non_blocking=True)
        ev = torch.cuda.Event()
        ev.record()
        self._copied[t] = ev
        out, off = [], 0
        for a, f in zip(arrays, flat):
            out.append(dev[off:off + f.size].view(np.shape(a)))
            off += f.size
        return out

    def step(self):
        """One scheduled step; returns (the schedule, the per-layer outputs,
        or None for an empty batch)."""
        rs = self.rs
        while self.next_arrival < len(rs.prompts) and rs.arrivals[self.next_arrival] <= self.step_index:
            self._arrive()
        st = self.sched.step()
        s = self.step_index
        self.step_index += 1
        if len(st.rids) == 0:
            return st, None
        T = int(st.q_lens.sum())
        if self.acts is not None:
            nk, nv, q = self.acts(s, T)
        else:
            nk, nv, q = (torch.from_numpy(np.ascontiguousarray(a)).to(self.device).to(self.act_dtype)
                         for a in rs.acts(s, T))
        sm, bt, sl, ql = self._upload([st.slot_mapping, st.block_tables, st.seq_lens, st.q_lens])
        hl, hq = np.ascontiguousarray(st.seq_lens, np.int32), np.ascontiguousarray(st.q_lens, np.int32)
        S = len(hl)
        ha, qa = hl.ctypes.data, hq.ctypes.data
        lib, kc, vc, ks, vs = self._lib, *self._pools
        need = lib.pa_attend_workspace_bytes(self._dptr[0], rs.num_q_heads, S, ha, qa, self._optr[0])
        if need == 0:
            raise pa.PagedAttentionError("pa_attend_workspace_bytes: invalid arguments")
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(2 * need, dtype=torch.uint8, device=self.device)
        outs = []
        for layer in range(rs.num_layers):
            lk, lv, lq = (nk, nv, q) if rs.num_layers == 1 else (nk[layer], nv[layer], q[layer])
            # the library trusts these sizes: check them (and the type and layout) every step
            if (tuple(lk.shape) != (T, rs.num_kv_heads, rs.head_dim) or lv.shape != lk.shape
                    or tuple(lq.shape) != (T, rs.num_q_heads, rs.head_dim)):
                raise ValueError(f"step {s}: activations must be [{T}, heads, {rs.head_dim}]")
            if not (lk.dtype == lv.dtype == lq.dtype == self.act_dtype and lk.is_cuda and lv.is_cuda and lq.is_cuda
                    and lk.is_contiguous() and lv.is_contiguous() and lq.is_contiguous()):
                raise ValueError(f"step {s}: activations must be contiguous device {self.act_dtype} tensors")
            out = torch.empty_like(lq)
            r = lib.pa_write_kv(self._dptr[layer], lk.data_ptr(), lv.data_ptr(), sm.data_ptr(), T, kc, vc, ks, vs,
                                self._stream)
            if r == 0:
                r = lib.pa_attend(self._dptr[layer], lq.data_ptr(), rs.num_q_heads, kc, vc, ks, vs, bt.data_ptr(),
                                  bt.shape[1], sl.data_ptr(), ql.data_ptr(), S, ha, qa, ctypes.c_float(rs.scale),
                                  out.data_ptr(), self._ws.data_ptr(), self._ws.numel(), self._optr[layer],
                                  self._stream)
            if r != 0:
                pa._check(r, f"serve step {s} layer {layer}")
            outs.append(out)
        return st, outs

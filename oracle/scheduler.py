"""Reference continuous-batching scheduler (test infrastructure; see
``oracle/__init__``).  Plain Python over ``oracle.paging.RefState``.

Written from [engine] "02 The engine":
* requests are admitted roughly in order, but the scheduler may look a few
  requests ahead and admit whichever of them fit;
* if too many requests are skipped in a row it falls back to blocking mode
  until memory frees up;
* new requests join the batch that is already running;
* every call runs four phases: release the blocks of sequences that finished
  in the last step, grow the running sequences, admit waiting requests,
  assemble the step's batch; whether a sequence is prefilling or decoding
  follows from its token counts (no flag).

Readings where the page is silent (stated once, used by the native
scheduler too):
* a request has a prompt of P tokens and generates N tokens: its first step
  reserves its P prompt positions (a prefill row block of q_len P) and yields
  token 1; each later step reserves one position (the token produced in the
  step before) and yields the next token; after N tokens it is finished and
  its blocks are released at the start of the next step.  Its lifetime is
  P + N - 1 positions.
* "fit": the request's whole lifetime, ceil((P + N - 1) / bs) blocks, fits in
  the free blocks left after the blocks still owed to the running requests
  (their lifetime blocks minus the blocks they hold), its P rows fit in the
  step's row budget, and a sequence slot is free.  Admission reserves the
  lifetime, so running requests never run out of blocks.
* look-ahead: the first ``lookahead`` waiting requests are considered in
  arrival order; each that fits is admitted.  When the oldest waiting request
  is passed over while a later one is admitted, its skip count grows; when it
  exceeds ``max_skips`` the scheduler blocks: only the oldest request may be
  admitted, and only once it fits; then it leaves blocking mode.
* the batch lists the running requests first (in admission order), then the
  requests admitted in this step (in admission order).
* requests that carry token ids ([manager]'s prefix tree, ``oracle.prefix``)
  are matched against the published blocks on admission: their first step
  reserves only the positions after the cached prefix, and after it their
  full prompt blocks are published.  Cached blocks count as available.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List

from . import paging as opg
from .prefix import RefPrefixPool


@dataclass
class Req:
    rid: int
    prompt: int
    new: int
    sid: int = -1
    generated: int = 0
    tokens: tuple = ()
    first_rows: int = 0
    state: str = "waiting"     # waiting | running | finished


@dataclass
class Step:
    rids: List[int] = field(default_factory=list)    # one entry per sequence of the batch
    q_lens: List[int] = field(default_factory=list)
    admitted: List[int] = field(default_factory=list)
    finished: List[int] = field(default_factory=list)  # released at the start of this step
    blocking: bool = False


def lifetime_blocks(r: Req, bs: int) -> int:
    return opg.blocks_for(r.prompt + r.new - 1, bs)


class RefScheduler:
    def __init__(self, num_blocks: int, block_size: int, max_batch_tokens: int, max_seqs: int,
                 lookahead: int, max_skips: int, first_pops=None):
        self.st = opg.RefState(num_blocks, block_size, first_pops)
        self.st.pool = RefPrefixPool(num_blocks, first_pops)
        self.cached_tokens = 0
        self.bs = block_size
        self.max_tokens, self.max_seqs = max_batch_tokens, max_seqs
        self.lookahead, self.max_skips = lookahead, max_skips
        self.reqs: List[Req] = []
        self.waiting: List[int] = []
        self.running: List[int] = []
        self.blocking = False
        self.head_skips = 0

    def add(self, prompt: int, new: int) -> int:
        r = Req(len(self.reqs), int(prompt), int(new))
        if r.prompt < 1 or r.new < 1 or lifetime_blocks(r, self.bs) > self.st.pool.num_blocks \
                or r.prompt > self.max_tokens:
            raise ValueError("a request that can never be admitted")
        self.reqs.append(r)
        self.waiting.append(r.rid)
        return r.rid

    def add_tokens(self, tokens, new: int) -> int:
        rid = self.add(len(tokens), new)
        self.reqs[rid].tokens = tuple(int(t) for t in tokens)
        return rid

    def _owed(self) -> int:
        owed = 0
        for rid in self.running:
            r = self.reqs[rid]
            held = len([b for b in self.st.tables[r.sid] if b >= 0])
            owed += lifetime_blocks(r, self.bs) - held
        return owed

    def schedule(self) -> Step:
        out = Step()
        # 1. release finished requests
        for rid in list(self.running):
            r = self.reqs[rid]
            if r.generated == r.new:
                for b in self.st.tables[r.sid]:
                    if b >= 0:
                        self.st.pool.release(b)
                self.st.tables[r.sid] = []
                r.state = "finished"
                self.running.remove(rid)
                out.finished.append(rid)
        # 2. running requests decode one token each
        decode = list(self.running)
        # 3. admission
        avail = self.st.pool.num_free + self.st.pool.num_cached - self._owed()
        tokens = self.max_tokens - len(decode)
        seqs = self.max_seqs - len(decode)
        admitted = []

        def fits(r):
            return lifetime_blocks(r, self.bs) <= avail and r.prompt <= tokens and seqs >= 1

        if self.blocking:
            if self.waiting:
                r = self.reqs[self.waiting[0]]
                if fits(r):
                    admitted.append(r.rid)
                    self.blocking = False
                    self.head_skips = 0
        else:
            for pos, rid in enumerate(list(self.waiting[:self.lookahead])):
                r = self.reqs[rid]
                if fits(r):
                    admitted.append(rid)
                    avail -= lifetime_blocks(r, self.bs)
                    tokens -= r.prompt
                    seqs -= 1
            head = self.waiting[0] if self.waiting else None
            if head is not None and head in admitted:
                self.head_skips = 0
            elif head is not None and admitted:
                self.head_skips += 1
                if self.head_skips > self.max_skips:
                    self.blocking = True
        for rid in admitted:
            self.waiting.remove(rid)
            r = self.reqs[rid]
            r.sid = self.st.add(0)
            cached = []
            if r.tokens:
                cached = self.st.pool.match(r.tokens, self.bs)
                self.st.tables[r.sid] = list(cached)
                self.st.lens[r.sid] = len(cached) * self.bs
            r.first_rows = r.prompt - len(cached) * self.bs
            self.cached_tokens += len(cached) * self.bs
            r.state = "running"
            self.running.append(rid)
        # 4. the batch: running first, then the newly admitted
        for rid in decode:
            out.rids.append(rid)
            out.q_lens.append(1)
        for rid in admitted:
            out.rids.append(rid)
            out.q_lens.append(self.reqs[rid].first_rows)
        out.admitted = admitted
        out.blocking = self.blocking
        return out

    def reserve(self, step: Step):
        """Reserve the batch's positions (``RefState.append`` per sequence, in
        batch order) and count one generated token per request; returns the
        slot mapping."""
        slots = []
        for rid, q in zip(step.rids, step.q_lens):
            r = self.reqs[rid]
            s, copies = self.st.append(r.sid, q)
            assert not copies
            slots += s
            r.generated += 1
        for rid in step.admitted:
            r = self.reqs[rid]
            if r.tokens:
                self.st.pool.publish(self.st.tables[r.sid], self.st.lens[r.sid], r.tokens, self.bs)
        return slots

    def done(self) -> bool:
        return not self.waiting and not self.running

"""The five synthetic paged-attention workloads, as seeded random draws.

Every array is drawn from ``numpy.random.default_rng`` keyed by
``[seed, stream, ...]``.  Large arrays are drawn in fixed chunks of the
flattened array, chunk ``c`` from the key ``[..., c]``, so a result never
depends on how many threads drew it.  Queries and K/V values are N(0,1) in
float32 rounded to fp16 (round to nearest even).

Shapes follow the five workloads:

1. tiny MHA decode: 12/12 heads, d64, 8-block pool, lengths 40/20/16/30;
2. GPT-2-small-shaped batch: 12/12 heads, d64, 32 prompts of 32..512 tokens
   prefilled, then 64 decode steps;
3. GQA decode: 32/8 heads, d128, 256 sequences of 1..4096 tokens;
4. shared 1024-token prefix with 4-beam copy-on-write, GQA 32/8, d128;
5. packed chunked prefill + decode over an int8 pool, GQA 32/8, d128.

Every constructor takes overrides so tests can build the same structure at a
size the CPU oracle finishes in seconds.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Callable, Optional

import numpy as np

BLOCK_SIZE = 16
CHUNK = 1 << 20  # elements per independently seeded draw chunk

# stream ids inside one workload's seed
S_META, S_POOL_K, S_POOL_V, S_NEW_K, S_NEW_V, S_Q, S_KSCALE, S_VSCALE, S_CTX_K, S_CTX_V, S_LAYERS = range(11)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _chunked(key, shape, dtype, fill_chunk):
    n = int(np.prod(shape, dtype=np.int64))
    out = np.empty(n, dtype)
    nchunks = max(1, -(-n // CHUNK))

    def one(c):
        lo = c * CHUNK
        hi = min(n, lo + CHUNK)
        if hi > lo:
            fill_chunk(np.random.default_rng([*key, c]), out[lo:hi])

    if nchunks == 1:
        one(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(one, range(nchunks)))
    return out.reshape(shape)


def normal_f16(key, shape) -> np.ndarray:
    """N(0,1) float32 draws rounded to fp16 (RNE)."""
    def fill(rng, dst):
        dst[:] = rng.standard_normal(dst.shape[0], dtype=np.float32)
    return _chunked(tuple(key), tuple(shape), np.float16, fill)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 values rounded to the nearest bfloat16 (ties to even), kept as
    float32 (every bf16 value is exactly a float32); inputs are finite."""
    b = np.ascontiguousarray(x, np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def normal_bf16(key, shape) -> np.ndarray:
    """N(0,1) float32 draws rounded to bf16 (RNE), held as float32."""
    def fill(rng, dst):
        dst[:] = round_bf16(rng.standard_normal(dst.shape[0], dtype=np.float32))
    return _chunked(tuple(key), tuple(shape), np.float32, fill)


def normal_act(kv_dtype: str):
    """The draw of 16-bit activations and pool values for a pool type."""
    return normal_bf16 if kv_dtype == "bf16" else normal_f16


def uniform_i8(key, shape) -> np.ndarray:
    """Uniform integers in [-127, 127] (filler for unused int8 pool slots)."""
    def fill(rng, dst):
        dst[:] = rng.integers(-127, 128, dst.shape[0], dtype=np.int8)
    return _chunked(tuple(key), tuple(shape), np.int8, fill)


def uniform_scale_f16(key, shape) -> np.ndarray:
    """Uniform (0.005, 0.05) rounded to fp16 (filler scales for unused blocks)."""
    def fill(rng, dst):
        dst[:] = rng.uniform(0.005, 0.05, dst.shape[0]).astype(np.float32)
    return _chunked(tuple(key), tuple(shape), np.float16, fill)


@dataclass
class StepDraw:
    """One step: every sequence (in canonical order) appends ``q_lens[i]`` new
    tokens, which are written and then queried (packed, sequence-major)."""
    q_lens: np.ndarray            # int64 [S]
    new_k: np.ndarray             # fp16 [T, Hkv, D]
    new_v: np.ndarray             # fp16 [T, Hkv, D]
    q: np.ndarray                 # fp16 [T, Hq, D]


@dataclass
class Workload:
    name: str
    seed: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    kv_dtype: str                 # "f16", "bf16" (values held as float32) or "i8"
    scale: float
    num_blocks: int
    first_pops: Optional[np.ndarray]   # free-list order: successive pops return these ids
    ctx_lens: np.ndarray          # tokens cached per sequence before the first step
    # initial pool contents, drawn on first access: fp16 [NB, Hkv, bs, D]
    # (int8 codes for int8 pools) and fp16 [NB, Hkv] scales for int8 pools
    pool_draws: dict = field(default_factory=dict, repr=False)
    steps: list = field(default_factory=list)   # list[StepDraw] or a callable(step)->StepDraw
    num_steps: int = 1
    # sharing (workload 4): request r holds ctx_lens[r] tokens whose first
    # ``shared_prefix`` tokens are one chain of blocks common to all requests;
    # request r is forked into ``beams[r]`` sequences before the step.
    shared_prefix: int = 0
    beams: Optional[np.ndarray] = None
    # int8 pools: the fp16 K/V of the cached context of sequence i, written
    # token by token into the pool before the first step.
    context: Optional[Callable[[int], tuple]] = None
    # sliding-window attention over this many tokens (0 = full causal)
    window: int = 0
    # layers per block: pools [NB, layers, Hkv, bs, D] and per-layer step
    # activations [layers, T, H, D] when > 1 (one block table for all layers)
    num_layers: int = 1

    _cache: dict = field(default_factory=dict, repr=False)
    _step_cache: dict = field(default_factory=dict, repr=False)

    def _pool(self, name):
        if name not in self.pool_draws:
            return None
        if name not in self._cache:
            self._cache[name] = self.pool_draws[name]()
        return self._cache[name]

    @property
    def pool_k(self) -> np.ndarray:
        return self._pool("k")

    @property
    def pool_v(self) -> np.ndarray:
        return self._pool("v")

    @property
    def pool_k_scale(self) -> Optional[np.ndarray]:
        return self._pool("k_scale")

    @property
    def pool_v_scale(self) -> Optional[np.ndarray]:
        return self._pool("v_scale")

    def drop_pools(self) -> None:
        """Forget the drawn pool arrays (they are redrawn identically on access)."""
        self._cache.clear()

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def step(self, s: int) -> StepDraw:
        """Step ``s``'s draws; the same object on every call (callers may edit it)."""
        if callable(self.steps):
            if s not in self._step_cache:
                self._step_cache[s] = self.steps(s)
            return self._step_cache[s]
        return self.steps[s]

    def layer_acts(self, s: int, layer: int) -> tuple:
        """(new_k, new_v, q) of step ``s`` for one layer."""
        st = self.step(s)
        if self.num_layers == 1:
            return st.new_k, st.new_v, st.q
        return st.new_k[layer], st.new_v[layer], st.q[layer]

    @property
    def num_seqs(self) -> int:
        if self.beams is not None:
            return int(np.sum(self.beams))
        return len(self.ctx_lens)


def _ceil_div(a, b):
    return -(-a // b)


def _lk(layers):
    """Shape prefix and key suffix of per-layer draws (none for one layer)."""
    return ((), ()) if layers == 1 else ((layers,), (S_LAYERS,))


def _f16_pool(seed, nb, hkv, d, layers=1, kv_dtype="f16"):
    _, key = _lk(layers)
    shape = (nb, hkv, BLOCK_SIZE, d) if layers == 1 else (nb, layers, hkv, BLOCK_SIZE, d)
    draw = normal_act(kv_dtype)
    return {
        "k": lambda: draw((seed, S_POOL_K, *key), shape),
        "v": lambda: draw((seed, S_POOL_V, *key), shape),
    }


def _i8_pool(seed, nb, hkv, d, layers=1):
    _, key = _lk(layers)
    lead = (nb,) if layers == 1 else (nb, layers)
    return {
        "k": lambda: uniform_i8((seed, S_POOL_K, *key), (*lead, hkv, BLOCK_SIZE, d)),
        "v": lambda: uniform_i8((seed, S_POOL_V, *key), (*lead, hkv, BLOCK_SIZE, d)),
        "k_scale": lambda: uniform_scale_f16((seed, S_KSCALE, *key), (*lead, hkv)),
        "v_scale": lambda: uniform_scale_f16((seed, S_VSCALE, *key), (*lead, hkv)),
    }


def _step(seed, tag, q_lens, hq, hkv, d, layers=1, kv_dtype="f16"):
    t = int(np.sum(q_lens))
    lead, key = _lk(layers)
    draw = normal_act(kv_dtype)
    return StepDraw(
        q_lens=np.asarray(q_lens, np.int64),
        new_k=draw((seed, S_NEW_K, *tag, *key), (*lead, t, hkv, d)),
        new_v=draw((seed, S_NEW_V, *tag, *key), (*lead, t, hkv, d)),
        q=draw((seed, S_Q, *tag, *key), (*lead, t, hq, d)),
    )


def config1(seed: int = 47001) -> Workload:
    """Tiny MHA decode: 12/12 heads, d64, bs 16, an 8-block pool; post-write
    lengths 40/20/16/30; the free list is a seeded permutation of 0..7."""
    hq = hkv = 12
    d = 64
    nb = 8
    rng = np.random.default_rng([seed, S_META])
    perm = rng.permutation(nb)
    post = np.array([40, 20, 16, 30], np.int64)
    return Workload(
        name="tiny-mha-decode", seed=seed, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
        block_size=BLOCK_SIZE, kv_dtype="f16", scale=1.0 / math.sqrt(d), num_blocks=nb,
        first_pops=perm, ctx_lens=post - 1,
        pool_draws=_f16_pool(seed, nb, hkv, d),
        steps=[_step(seed, (0,), np.ones(4, np.int64), hq, hkv, d)],
    )


def config2(seed: int = 47002, num_seqs: int = 32, min_prompt: int = 32, max_prompt: int = 512,
            decode_steps: int = 64, num_layers: int = 1, kv_dtype: str = "f16") -> Workload:
    """GPT-2-small-shaped batch: 12/12 heads, d64; prompts U[32,512] prefilled
    (step 0, causal), then ``decode_steps`` steps of one token per sequence.
    Plain free list (first pops 0, 1, 2, ...); blocks grow on demand.
    ``num_layers`` > 1 (GPT-2 small has 12): a multi-layer pool and per-layer
    activations over the same tables."""
    hq = hkv = 12
    d = 64
    rng = np.random.default_rng([seed, S_META])
    prompts = rng.integers(min_prompt, max_prompt + 1, num_seqs).astype(np.int64)
    nb = num_seqs * _ceil_div(max_prompt + decode_steps, BLOCK_SIZE)

    def steps(s):
        if s == 0:
            return _step(seed, (0,), prompts, hq, hkv, d, num_layers, kv_dtype)
        return _step(seed, (s,), np.ones(num_seqs, np.int64), hq, hkv, d, num_layers, kv_dtype)

    return Workload(
        name="gpt2-continuous-batch", seed=seed, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
        block_size=BLOCK_SIZE, kv_dtype=kv_dtype, scale=1.0 / math.sqrt(d), num_blocks=nb,
        first_pops=None, ctx_lens=np.zeros(num_seqs, np.int64),
        pool_draws=_f16_pool(seed, nb, hkv, d, num_layers, kv_dtype),
        steps=steps, num_steps=1 + decode_steps, num_layers=num_layers,
    )


def config3(seed: int = 47003, num_seqs: int = 256, max_len: int = 4096, min_len: int = 1,
            num_q_heads: int = 32, num_kv_heads: int = 8, head_dim: int = 128, kv_dtype: str = "f16") -> Workload:
    """GQA decode: 32/8 heads, d128; post-write lengths U[1,4096]; pool = the
    blocks needed plus 10%, free list a seeded permutation of the pool."""
    hq, hkv, d = num_q_heads, num_kv_heads, head_dim
    rng = np.random.default_rng([seed, S_META])
    post = rng.integers(min_len, max_len + 1, num_seqs).astype(np.int64)
    nb = int(math.ceil(1.1 * int(np.sum(_ceil_div(post, BLOCK_SIZE)))))
    perm = rng.permutation(nb)
    return Workload(
        name="gqa-decode", seed=seed, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
        block_size=BLOCK_SIZE, kv_dtype=kv_dtype, scale=1.0 / math.sqrt(d), num_blocks=nb,
        first_pops=perm, ctx_lens=post - 1,
        pool_draws=_f16_pool(seed, nb, hkv, d, kv_dtype=kv_dtype),
        steps=[_step(seed, (0,), np.ones(num_seqs, np.int64), hq, hkv, d, kv_dtype=kv_dtype)],
    )


def config4(seed: int = 47004, num_requests: int = 64, prefix: int = 1024, min_suffix: int = 16,
            max_suffix: int = 256, beam_requests: int = 16, beam_width: int = 4, share: bool = True,
            decode_steps: int = 1) -> Workload:
    """Shared prefix + beam copy-on-write: every request's table starts with
    the same ``prefix``-token chain; suffixes U[16,256]; requests
    0..beam_requests-1 are forked into ``beam_width`` sequences; one decode
    token per sequence.  Free list is a seeded permutation.

    ``share=False`` is the control with the same sequences and lengths but
    nothing shared: every sequence (each beam too) owns all of its blocks.
    ``decode_steps`` > 1 adds further one-token steps (step s drawn under its
    own tag; step 0 is the same either way)."""
    hq, hkv, d = 32, 8, 128
    rng = np.random.default_rng([seed, S_META])
    suffix = rng.integers(min_suffix, max_suffix + 1, num_requests).astype(np.int64)
    beams = np.ones(num_requests, np.int64)
    beams[:beam_requests] = beam_width
    need = _ceil_div(prefix, BLOCK_SIZE) + int(np.sum(beams * _ceil_div(suffix + 1, BLOCK_SIZE)))
    nb = int(math.ceil(1.1 * need))
    perm = rng.permutation(nb)
    nseq = int(np.sum(beams))

    def steps(s):
        return _step(seed, (s,), np.ones(nseq, np.int64), hq, hkv, d)

    if decode_steps > 1:
        nb += nseq * _ceil_div(decode_steps, BLOCK_SIZE)
        perm = rng.permutation(nb)
    if not share:
        lens = np.repeat(prefix + suffix, beams)
        nb = int(math.ceil(1.1 * int(np.sum(_ceil_div(lens + 1, BLOCK_SIZE)))))
        return Workload(
            name="prefix-copies-control", seed=seed, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
            block_size=BLOCK_SIZE, kv_dtype="f16", scale=1.0 / math.sqrt(d), num_blocks=nb,
            first_pops=rng.permutation(nb), ctx_lens=lens,
            pool_draws=_f16_pool(seed, nb, hkv, d),
            steps=[_step(seed, (0,), np.ones(nseq, np.int64), hq, hkv, d)],
        )
    return Workload(
        name="prefix-share-beam-cow", seed=seed, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
        block_size=BLOCK_SIZE, kv_dtype="f16", scale=1.0 / math.sqrt(d), num_blocks=nb,
        first_pops=perm, ctx_lens=prefix + suffix,
        pool_draws=_f16_pool(seed, nb, hkv, d),
        steps=steps if decode_steps > 1 else [steps(0)], num_steps=int(decode_steps),
        shared_prefix=prefix, beams=beams,
    )


def config5(seed: int = 47005, num_chunks: int = 8, chunk_q: int = 512, max_chunk_ctx: int = 8192,
            num_decode: int = 192, max_decode_len: int = 32768, kv_dtype: str = "i8",
            num_q_heads: int = 32, chunk_ctx: Optional[int] = None) -> Workload:
    """Packed chunked prefill + decode over an int8 pool: ``num_chunks``
    segments of ``chunk_q`` query tokens with cached context U[0,8192], then
    ``num_decode`` decode sequences with post-write length U[1,32768].  The
    cached context is N(0,1) fp16 K/V, written into the int8 pool token by
    token before the step.  Unused pool slots hold uniform int8 filler.

    ``kv_dtype`` "f16" / "bf16": the same batch over a 16-bit pool whose
    contents are N(0,1) (the context already in place, as in workload 3);
    with ``num_decode=0`` that is the chunks alone (the same contexts: they
    are drawn first).  ``num_q_heads`` 64 gives groups of eight query
    heads per KV head (the same draws otherwise).  ``chunk_ctx`` gives every
    chunk that cached context instead of the draw (which is still made, so
    the other draws stay the same)."""
    hq, hkv, d = num_q_heads, 8, 128
    rng = np.random.default_rng([seed, S_META])
    cctx = rng.integers(0, max_chunk_ctx + 1, num_chunks).astype(np.int64)
    if chunk_ctx is not None:
        cctx[:] = int(chunk_ctx)
    dpost = rng.integers(1, max_decode_len + 1, num_decode).astype(np.int64)
    ctx = np.concatenate([cctx, dpost - 1])
    q_lens = np.concatenate([np.full(num_chunks, chunk_q, np.int64), np.ones(num_decode, np.int64)])
    post = ctx + q_lens
    nb = int(math.ceil(1.1 * int(np.sum(_ceil_div(post, BLOCK_SIZE)))))
    perm = rng.permutation(nb)

    def context(i):
        n = int(ctx[i])
        return (normal_f16((seed, S_CTX_K, i), (n, hkv, d)),
                normal_f16((seed, S_CTX_V, i), (n, hkv, d)))

    if kv_dtype != "i8":
        return Workload(
            name=f"packed-{kv_dtype}-prefill" + ("-decode" if num_decode else ""), seed=seed, num_q_heads=hq,
            num_kv_heads=hkv, head_dim=d, block_size=BLOCK_SIZE, kv_dtype=kv_dtype, scale=1.0 / math.sqrt(d),
            num_blocks=nb, first_pops=perm, ctx_lens=ctx, pool_draws=_f16_pool(seed, nb, hkv, d, kv_dtype=kv_dtype),
            steps=[_step(seed, (0,), q_lens, hq, hkv, d, kv_dtype=kv_dtype)],
        )
    return Workload(
        name="packed-int8-prefill-decode", seed=seed, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
        block_size=BLOCK_SIZE, kv_dtype="i8", scale=1.0 / math.sqrt(d), num_blocks=nb,
        first_pops=perm, ctx_lens=ctx,
        pool_draws={
            "k": lambda: uniform_i8((seed, S_POOL_K), (nb, hkv, BLOCK_SIZE, d)),
            "v": lambda: uniform_i8((seed, S_POOL_V), (nb, hkv, BLOCK_SIZE, d)),
            "k_scale": lambda: uniform_scale_f16((seed, S_KSCALE), (nb, hkv)),
            "v_scale": lambda: uniform_scale_f16((seed, S_VSCALE), (nb, hkv)),
        },
        steps=[_step(seed, (0,), q_lens, hq, hkv, d)],
        context=context,
    )


CONFIGS = {1: config1, 2: config2, 3: config3, 4: config4, 5: config5}


def custom(seed: int, kv_lens, q_lens, num_q_heads: int = 8, num_kv_heads: int = 2, head_dim: int = 128,
           kv_dtype: str = "f16", extra_blocks: int = 3, permute: bool = True, window: int = 0,
           num_layers: int = 1) -> Workload:
    """A one-step workload with explicit post-write lengths ``kv_lens`` and
    query rows ``q_lens`` (the cached context is kv_len - q_len tokens).  For
    int8 pools the cached context is drawn as N(0,1) fp16 and written token
    by token before the step; fp16 pools hold N(0,1) everywhere.  With
    ``num_layers`` > 1 every draw gets a leading layer axis (after the block
    axis in the pools)."""
    hq, hkv, d = num_q_heads, num_kv_heads, head_dim
    post = np.asarray(kv_lens, np.int64)
    ql = np.asarray(q_lens, np.int64)
    ctx = post - ql
    nb = int(np.sum(_ceil_div(post, BLOCK_SIZE))) + extra_blocks
    rng = np.random.default_rng([seed, S_META])
    perm = rng.permutation(nb) if permute else None
    lead, key = _lk(num_layers)
    if kv_dtype == "i8":
        draws = _i8_pool(seed, nb, hkv, d, num_layers)

        def context(i):
            n = int(ctx[i])
            return (normal_f16((seed, S_CTX_K, i, *key), (*lead, n, hkv, d)),
                    normal_f16((seed, S_CTX_V, i, *key), (*lead, n, hkv, d)))
    else:
        draws = _f16_pool(seed, nb, hkv, d, num_layers, kv_dtype)
        context = None
    return Workload(
        name=f"custom-{seed}", seed=seed, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=BLOCK_SIZE,
        kv_dtype=kv_dtype, scale=1.0 / math.sqrt(d), num_blocks=nb, first_pops=perm, ctx_lens=ctx,
        pool_draws=draws, steps=[_step(seed, (0,), ql, hq, hkv, d, num_layers, kv_dtype)], context=context,
        window=int(window), num_layers=int(num_layers),
    )


@dataclass
class RequestStream:
    """Requests for the continuous-batching scheduler: arrival step, prompt
    length and tokens to generate each, the attention shape, the pool and the
    scheduler's limits.  Activations of step s are drawn under tag (s,)."""
    name: str
    seed: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    kv_dtype: str
    scale: float
    num_blocks: int
    arrivals: np.ndarray          # step at which each request is queued
    prompts: np.ndarray
    new_tokens: np.ndarray
    max_batch_tokens: int
    max_seqs: int
    lookahead: int
    max_skips: int
    num_layers: int = 1
    tokens: Optional[list] = None   # per request, its prompt's token ids (for the prefix cache)

    def acts(self, s: int, rows: int) -> tuple:
        """(new_k, new_v, q) of step ``s`` with ``rows`` packed rows (a leading
        layer axis with several layers)."""
        st = _step(self.seed, (s,), [rows], self.num_q_heads, self.num_kv_heads, self.head_dim, self.num_layers,
                   self.kv_dtype)
        return st.new_k, st.new_v, st.q


def config6(seed: int = 47006, num_requests: int = 256, min_prompt: int = 32, max_prompt: int = 512,
            new_tokens: int = 64, num_blocks: int = 1152, max_batch_tokens: int = 4096, max_seqs: int = 64,
            lookahead: int = 4, max_skips: int = 8, arrive_per_step: int = 0, num_layers: int = 1,
            kv_dtype: str = "f16", system_prompts: int = 0, min_system: int = 64,
            max_system: int = 256) -> RequestStream:
    """Continuous batching under churn, GPT-2-small-shaped (12/12 heads, d64):
    ``num_requests`` requests with prompts U[32,512] each generating 64
    tokens (every request of the engine page's workload generates 64), over
    a 1152-block pool (the 32-request batch of workload 2), at most 4096 rows
    and 64 sequences per step.  ``arrive_per_step`` = 0 queues every request
    at once; k > 0 queues k per step.  ``system_prompts`` = k > 0 gives every
    request token ids: one of k shared system prompts (U[64,256] tokens) then
    its own U[min_prompt, max_prompt] tokens, ids uniform over GPT-2's 50257,
    so the prefix cache can serve the shared parts."""
    hq = hkv = 12
    d = 64
    rng = np.random.default_rng([seed, S_META])
    prompts = rng.integers(min_prompt, max_prompt + 1, num_requests).astype(np.int64)
    tokens = None
    if system_prompts > 0:
        trng = np.random.default_rng([seed, S_META, 1])
        systems = [trng.integers(0, 50257, int(trng.integers(min_system, max_system + 1))).astype(np.int32)
                   for _ in range(system_prompts)]
        pick = trng.integers(0, system_prompts, num_requests)
        tokens = [np.concatenate([systems[int(pick[i])],
                                  trng.integers(0, 50257, int(prompts[i])).astype(np.int32)])
                  for i in range(num_requests)]
        prompts = np.asarray([len(t) for t in tokens], np.int64)
    arrivals = (np.zeros(num_requests, np.int64) if arrive_per_step <= 0
                else np.arange(num_requests, dtype=np.int64) // int(arrive_per_step))
    return RequestStream(
        name="gpt2-continuous-batching-churn", seed=seed, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
        block_size=BLOCK_SIZE, kv_dtype=kv_dtype, scale=1.0 / math.sqrt(d), num_blocks=num_blocks,
        arrivals=arrivals, prompts=prompts, new_tokens=np.full(num_requests, new_tokens, np.int64),
        max_batch_tokens=max_batch_tokens, max_seqs=max_seqs, lookahead=lookahead, max_skips=max_skips,
        num_layers=num_layers, tokens=tokens,
    )

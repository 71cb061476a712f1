"""Reference paged attention in float64 (test infrastructure; see ``oracle/__init__``).

Written from [pytorch] "Compute reference attention without hiding the
layout": each position's K/V is gathered through the block table into a
contiguous buffer; each KV head is repeated ``q_heads / kv_heads`` times along
a new axis after the KV-head axis (so query head ``hq`` reads KV head
``hq // G``); scores are ``q . k * head_dim ** -0.5`` (the caller passes the
scale); softmax over keys; the output is the weighted sum of V.

The causal rule for several query tokens of one sequence follows [engine]
"03 Correctness, and the bugs a real model found": the query at packed
offset ``t`` of a sequence with ``q_len`` new tokens and ``kv_len`` cached
tokens (after this step's writes) sits at position ``kv_len - q_len + t`` and
sees keys ``0 .. kv_len - q_len + t``.  A decode query (q_len 1) sees all
``kv_len`` keys, itself included (write, then attend).

int8 pools are read as ``code * scale[block, head]`` ([engine] "INT8 KV cache
design": dequantise before each of the two dot products).

Sliding window ([pytorch] "PagedAttention vs sliding-window attention,
RadixAttention, and SSMs": each query attends only to the most recent ``w``
tokens): with ``window = w > 0`` the query at position ``P`` sees keys
``max(0, P - w + 1) .. P``.  Blocks that hold no key any query of the step can
see may already be freed, so the gather starts at the step's earliest
visible key.
"""
from __future__ import annotations

import numpy as np


def gather(pool, table, length, block_size, scales=None, start=0):
    """Contiguous ``[length - start, kv_heads, D]`` float64 copy of positions
    ``start .. length - 1`` of one sequence's K or V."""
    pos = np.arange(int(start), int(length))
    blocks = np.asarray(table, np.int64)[pos // block_size]
    offs = pos % block_size
    x = pool[blocks, :, offs, :].astype(np.float64)
    if scales is not None:
        x *= scales[blocks, :].astype(np.float64)[:, :, None]
    return x


def query_positions(kv_len: int, q_len: int) -> np.ndarray:
    return int(kv_len) - int(q_len) + np.arange(int(q_len))


def attend(q, positions, Kc, Vc, scale, window=0, key0=0):
    """Attention of query rows ``q [n, Hq, D]`` at ``positions [n]`` over the
    contiguous ``Kc, Vc [L, Hkv, D]`` holding positions ``key0 ..``; returns
    float64 ``[n, Hq, D]``.  ``window > 0`` hides keys before ``P - window + 1``."""
    q = np.asarray(q, np.float64)
    n, hq, _ = q.shape
    hkv = Kc.shape[1]
    G = hq // hkv
    Ke = np.repeat(Kc, G, axis=1).transpose(1, 2, 0)      # [Hq, D, L]
    Ve = np.repeat(Vc, G, axis=1).transpose(1, 0, 2)      # [Hq, L, D]
    s = np.matmul(q.transpose(1, 0, 2), Ke) * float(scale)  # [Hq, n, L]
    keys = int(key0) + np.arange(Kc.shape[0])[None, :]
    P = np.asarray(positions)[:, None]
    hidden = keys > P                                                      # [n, L]
    if window:
        hidden |= keys < P - int(window) + 1
    s = np.where(hidden[None], -np.inf, s)
    s = s - s.max(axis=-1, keepdims=True)
    w = np.exp(s)
    w /= w.sum(axis=-1, keepdims=True)
    return np.matmul(w, Ve).transpose(1, 0, 2)             # [n, Hq, D]


def window_start(kv_len: int, q_len: int, window: int) -> int:
    """Earliest key any query of the step can see (0 without a window)."""
    return max(0, int(kv_len) - int(q_len) - int(window) + 1) if window else 0


def paged_attention(q, pool_k, pool_v, tables, kv_lens, q_lens, scale, block_size,
                    k_scale=None, v_scale=None, seqs=None, window=0):
    """Attention for a packed batch (sequence-major query rows).

    ``seqs`` optionally restricts the work to some sequences; rows of other
    sequences are left as NaN."""
    q = np.asarray(q)
    out = np.full(q.shape, np.nan, np.float64)
    start = 0
    for i, (L, Q) in enumerate(zip(kv_lens, q_lens)):
        L, Q = int(L), int(Q)
        if seqs is None or i in seqs:
            if Q > 0:
                lo = window_start(L, Q, window)
                Kc = gather(pool_k, tables[i], L, block_size, k_scale, lo)
                Vc = gather(pool_v, tables[i], L, block_size, v_scale, lo)
                out[start:start + Q] = attend(q[start:start + Q], query_positions(L, Q), Kc, Vc, scale,
                                              window, lo)
        start += Q
    return out

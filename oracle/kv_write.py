"""Reference KV writes (test infrastructure; see ``oracle/__init__``).

Pool layout (a reading: the pages disagree, [manager] "Step 1: The Block" vs
[pytorch] "Allocate, append, and free KV-cache blocks"): separate K and V
pools of shape ``[num_blocks, kv_heads, block_size, head_dim]``.

fp16: token ``t`` with slot ``s >= 0`` lands at block ``s // bs``, offset
``s % bs``, every KV head ([pytorch] "Allocate, append, and free KV-cache
blocks", the index-put of ``append_token``).  A negative slot is skipped.

int8 ([engine] "INT8 KV cache design"): symmetric, no zero point, one scale
per block per head; on every token write the block's valid entries are
dequantised with the stored scale, the new token is appended, a new max-abs
scale is taken over the whole set and every entry is requantised.  The pages
fix neither the constant, the rounding nor the precision; the reading used
(and shared with the kernel, since these floats decide integer codes):

    x_j   = float32(code_j) * float32(scale)        j < o   (exact)
    x_o   = float32(new)
    amax  = max_j |x_j|                              (float32)
    scale = fp16_round_nearest_even(amax / 127.0f)   (IEEE float32 division)
    code_j = clamp(round_half_even(x_j / float32(scale)), -127, 127)
             (all zero when the new scale is zero)

where ``o = slot % bs`` is the number of valid entries before the write
(tokens of a block arrive in position order).  K and V are quantised
separately, each per (block, KV head).
"""
from __future__ import annotations

import numpy as np


def write_f16(pool_k, pool_v, new_k, new_v, slots, block_size):
    """Pools after scattering ``new_k/new_v[t]`` to ``slots[t]`` (copies returned)."""
    K = pool_k.copy()
    V = pool_v.copy()
    for t, s in enumerate(np.asarray(slots).tolist()):
        if s < 0:
            continue
        b, o = divmod(s, block_size)
        K[b, :, o, :] = new_k[t]
        V[b, :, o, :] = new_v[t]
    return K, V


def copy_blocks(pools, pairs):
    """Copy whole blocks ``src -> dst`` in every array of ``pools`` (in place).
    The copies of one call read sources before any destination is written."""
    pairs = list(pairs)
    for arr in pools:
        if arr is None:
            continue
        src = [p[0] for p in pairs]
        dst = [p[1] for p in pairs]
        if pairs:
            arr[dst] = arr[src].copy()


def quant_append(codes_bd, scale, o, new_d):
    """One int8 token write into one (block, head).

    codes_bd: int8 [bs, D]; scale: float16 scalar; o: offset of the new token
    (entries 0..o-1 are valid); new_d: float16 [D].  Returns (codes, scale)."""
    f32 = np.float32
    x = np.empty((o + 1, codes_bd.shape[1]), f32)
    x[:o] = codes_bd[:o].astype(f32) * f32(scale)
    x[o] = new_d.astype(f32)
    amax = f32(np.max(np.abs(x)))
    s = np.float16(amax / f32(127.0))
    out = codes_bd.copy()
    if s == 0:
        out[:o + 1] = 0
    else:
        out[:o + 1] = np.clip(np.rint(x / f32(s)), -127, 127).astype(np.int8)
    return out, s


def write_i8(pool_k, pool_v, k_scale, v_scale, new_k, new_v, slots, block_size):
    """Pools and scales after replaying the tokens in increasing t (copies returned)."""
    K, V, KS, VS = pool_k.copy(), pool_v.copy(), k_scale.copy(), v_scale.copy()
    hkv = K.shape[1]
    for t, s in enumerate(np.asarray(slots).tolist()):
        if s < 0:
            continue
        b, o = divmod(s, block_size)
        for h in range(hkv):
            K[b, h], KS[b, h] = quant_append(K[b, h], KS[b, h], o, new_k[t, h])
            V[b, h], VS[b, h] = quant_append(V[b, h], VS[b, h], o, new_v[t, h])
    return K, V, KS, VS


def quant_append_many(codes, scales, o, new):
    """``quant_append`` applied independently to many (block, head) pairs at one offset.

    codes: int8 [n, H, bs, D]; scales: float16 [n, H]; new: float16 [n, H, D].
    Each (i, h) is exactly ``quant_append(codes[i, h], scales[i, h], o, new[i, h])``."""
    f32 = np.float32
    n, H, bs, D = codes.shape
    x = np.empty((n, H, o + 1, D), f32)
    x[:, :, :o] = codes[:, :, :o].astype(f32) * scales.astype(f32)[:, :, None, None]
    x[:, :, o] = new.astype(f32)
    amax = np.max(np.abs(x), axis=(2, 3)).astype(f32)
    s = (amax / f32(127.0)).astype(np.float16)
    out = codes.copy()
    s32 = s.astype(f32)[:, :, None, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.clip(np.rint(x / s32), -127, 127)
    q = np.where(s32 == 0, 0, q)
    out[:, :, :o + 1] = q.astype(np.int8)
    return out, s


def fill_context_i8(pool_k, pool_v, k_scale, v_scale, table, ctx_k, ctx_v, block_size):
    """Write a sequence's first ``n = len(ctx_k)`` tokens into its blocks, token by
    token in position order (in place).  Blocks are independent, so offset ``o``
    of every block is written in one vectorised ``quant_append_many`` step."""
    n = ctx_k.shape[0]
    nblk = -(-n // block_size)
    blocks = np.asarray(table[:nblk], np.int64)
    for o in range(block_size):
        idx = np.arange(nblk) * block_size + o
        live = idx < n
        if not live.any():
            break
        b = blocks[live]
        for pool, sc, src in ((pool_k, k_scale, ctx_k), (pool_v, v_scale, ctx_v)):
            c, s = quant_append_many(pool[b], sc[b], o, src[idx[live]])
            pool[b] = c
            sc[b] = s

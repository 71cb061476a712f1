"""Pure-Python brute force for tiny inputs (test infrastructure; see ``oracle/__init__``).

No numpy arithmetic: nested loops over Python floats and ``math.exp``.  It
walks the block table for every key (no gathered buffer) and applies the
causal rule and GQA head mapping as stated in ``oracle.attention``.
"""
from __future__ import annotations

import math


def paged_attention(q, pool_k, pool_v, tables, kv_lens, q_lens, scale, block_size,
                    k_scale=None, v_scale=None, window=0):
    """q: nested lists [T][Hq][D]; pools: nested lists [NB][Hkv][bs][D];
    scales: [NB][Hkv] or None.  Returns nested lists [T][Hq][D].  With
    ``window > 0`` the query at position P sees keys P - window + 1 .. P only."""
    hq = len(q[0]) if q else 0
    hkv = len(pool_k[0]) if pool_k else 1
    G = hq // hkv if hkv else 1
    out = []
    row = 0
    for i, (L, Q) in enumerate(zip(kv_lens, q_lens)):
        for t in range(Q):
            pos = L - Q + t
            first = max(0, pos - window + 1) if window else 0
            out_row = []
            for h in range(hq):
                g = h // G
                scores = []
                for j in range(first, pos + 1):
                    b = tables[i][j // block_size]
                    o = j % block_size
                    ks = 1.0 if k_scale is None else float(k_scale[b][g])
                    dot = 0.0
                    for d in range(len(q[row][h])):
                        dot += float(q[row][h][d]) * float(pool_k[b][g][o][d]) * ks
                    scores.append(dot * scale)
                m = max(scores)
                ws = [math.exp(x - m) for x in scores]
                tot = sum(ws)
                vec = []
                for d in range(len(q[row][h])):
                    acc = 0.0
                    for jj, j in enumerate(range(first, pos + 1)):
                        b = tables[i][j // block_size]
                        o = j % block_size
                        vs = 1.0 if v_scale is None else float(v_scale[b][g])
                        acc += ws[jj] * float(pool_v[b][g][o][d]) * vs
                    vec.append(acc / tot)
                out_row.append(vec)
            out.append(out_row)
            row += 1
    return out

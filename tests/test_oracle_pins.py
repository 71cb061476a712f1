"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each test names what fixes the expected value: a trace the pages print
(``tests/golden``), a closed form, a library routine on contiguous data,
brute force, or an invariance.  A plausible slip in the oracle (a dropped
scale, a wrong sign, a transposed operand, an off-by-one in the causal rule,
a wrong GQA head mapping, a wrong rounding mode or constant in the int8 rule)
fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention as oatt
from oracle import brute
from oracle import kv_write as okv
from oracle import paging as opg
import synthetic

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- paging ----

def test_nanoserve_allocator_trace():
    g = _gold("nanoserve_allocator_trace.json")
    pool = opg.RefPool(g["num_blocks"])
    held = {}
    for op in g["ops"]:
        if op["op"] == "allocate_for":
            if "expect_error" in op:
                with pytest.raises(opg.Exhausted):
                    pool.pop_for(op["tokens"], g["block_size"])
            else:
                held[op["name"]] = pool.pop_for(op["tokens"], g["block_size"])
                assert held[op["name"]] == op["expect_ids"]
        else:
            pool.push_all(held.pop(op["name"]))
        assert pool.num_free == op["expect_free"]


def test_pytorch_lookup_trace():
    g = _gold("pytorch_lookup_trace.json")
    bs = g["block_size"]
    order = g["initial_table"] + [g["next_free_block"]]
    order += [b for b in range(10) if b not in order]
    st = opg.RefState(10, bs, first_pops=order)
    st.add(g["initial_len"])
    assert st.tables[0] == g["initial_table"]
    for lk in g["lookups"]:
        lb, off = opg.translate(lk["pos"], bs)
        assert (lb, off) == (lk["logical_block"], lk["offset"])
        assert st.tables[0][lb] == lk["physical_block"]
    for ap in g["appends"]:
        slots, copies = st.append(0, 1)
        assert copies == []
        assert opg.translate(ap["pos"], bs) == (ap["logical_block"], ap["offset"])
        assert st.tables[0] == ap["table_after"] and st.lens[0] == ap["len_after"]
        assert slots == [ap["table_after"][ap["logical_block"]] * bs + ap["offset"]]


def test_block_math():
    g = _gold("block_math.json")
    for n, bs, want in g["block_counts"]:
        assert opg.blocks_for(n, bs) == want
    assert 2 * 32 * 4096 * 8 * 128 * 2 == g["contiguous_bytes_per_seq"]
    assert 256 * g["contiguous_bytes_per_seq"] == g["contiguous_bytes_256_seqs"]
    for pos, bs, lb, off in g["translate"]:
        assert opg.translate(pos, bs) == (lb, off)


def test_atomic_reserve_and_double_free():
    pool = opg.RefPool(4)
    a = pool.pop_for(20, 16)
    before = list(pool.stack)
    with pytest.raises(opg.Exhausted):
        pool.pop_for(3 * 16 + 1, 16)          # needs 4 blocks, 2 free
    assert pool.stack == before and pool.num_free == 2
    pool.push_all(a)
    with pytest.raises(ValueError):
        pool.push(a[0])                        # double free
    with pytest.raises(ValueError):
        pool.push(99)                          # never belonged to the pool


def test_interleaved_invariants():
    """Random interleaving of add / fork / append / finish keeps: free and
    allocated disjoint and covering the pool; refcount = number of tables
    holding the block; fragmentation below one block per sequence; finishing
    everything returns every block."""
    rng = np.random.default_rng(7)
    nb, bs = 64, 4
    st = opg.RefState(nb, bs, first_pops=rng.permutation(nb))
    live = []
    for _ in range(400):
        op = rng.integers(0, 4)
        try:
            if op == 0 or not live:
                live.append(st.add(int(rng.integers(0, 9))))
            elif op == 1:
                live.append(st.fork(live[rng.integers(len(live))]))
            elif op == 2:
                i = live[rng.integers(len(live))]
                st.append(i, int(rng.integers(1, 6)))
            else:
                i = live.pop(rng.integers(len(live)))
                for b in st.tables[i]:
                    st.pool.release(b)
                st.tables[i] = []
        except opg.Exhausted:
            pass
        held = {}
        for i in live:
            for b in st.tables[i]:
                held[b] = held.get(b, 0) + 1
            assert len(st.tables[i]) * bs - st.lens[i] in range(0, bs)
        assert held == st.pool.refs
        assert set(st.pool.stack).isdisjoint(st.pool.refs)
        assert len(st.pool.stack) + len(st.pool.refs) == nb
    for i in live:
        for b in st.tables[i]:
            st.pool.release(b)
    assert st.pool.num_free == nb


def test_workload1_tables():
    w = synthetic.config1()
    st = opg.build_state(w)
    assert [len(t) for t in st.tables] == [3, 2, 1, 2]
    assert sum(st.tables, []) == list(w.first_pops)
    slots, copies = opg.apply_step(st, w.step(0).q_lens)
    assert copies == [] and st.lens == [40, 20, 16, 30]
    assert [len(t) for t in st.tables] == [3, 2, 1, 2]


def test_workload4_refcounts_and_cow():
    w = synthetic.config4(num_requests=8, beam_requests=3)
    # before forking: one reference per request on every prefix block
    w1 = synthetic.config4(num_requests=8, beam_requests=0)
    st1 = opg.build_state(w1)
    prefix = st1.tables[0][:w1.shared_prefix // 16]
    assert all(st1.pool.refs[b] == 8 for b in prefix)
    st = opg.build_state(w)
    prefix = st.tables[0][:w.shared_prefix // 16]
    assert all(st.pool.refs[b] == 8 + 3 * 3 for b in prefix)
    slots, copies = opg.apply_step(st, w.step(0).q_lens)
    # every beam of a request whose next position is mid-block, except the last, copies
    exp = sum(3 for r in range(3) if int(w.ctx_lens[r]) % 16 != 0)
    assert len(copies) == exp
    assert all(st.pool.refs[b] == 8 + 9 for b in prefix)
    for i in range(len(st.tables)):
        assert slots[i] // 16 == st.tables[i][int(st.lens[i] - 1) // 16]
    # after the step no block a sequence writes is shared
    written = [s // 16 for s in slots]
    assert len(set(written)) == len(written)


# -------------------------------------------------------------- kv write ----

def test_write_roundtrip():
    """Known K/V written within a block, across a block boundary and across
    non-contiguous blocks read back unchanged through the table
    ([pytorch] 'Test and benchmark ...': write-read roundtrips)."""
    rng = np.random.default_rng(3)
    nb, hkv, bs, d = 12, 2, 4, 8
    st = opg.RefState(nb, bs, first_pops=rng.permutation(nb))
    i = st.add(0)
    K = rng.standard_normal((nb, hkv, bs, d)).astype(np.float16)
    V = rng.standard_normal((nb, hkv, bs, d)).astype(np.float16)
    written_k, written_v = [], []
    for n in (3, 1, 6, 9):       # within, up to the boundary, across, across several
        slots, _ = st.append(i, n)
        nk = rng.standard_normal((n, hkv, d)).astype(np.float16)
        nv = rng.standard_normal((n, hkv, d)).astype(np.float16)
        K, V = okv.write_f16(K, V, nk, nv, slots, bs)
        written_k.append(nk)
        written_v.append(nv)
    L = st.lens[i]
    assert np.array_equal(oatt.gather(K, st.tables[i], L, bs), np.concatenate(written_k).astype(np.float64))
    assert np.array_equal(oatt.gather(V, st.tables[i], L, bs), np.concatenate(written_v).astype(np.float64))
    assert len(set(st.tables[i])) == len(st.tables[i])


def test_write_skips_negative_slots_and_touches_nothing_else():
    rng = np.random.default_rng(4)
    K = rng.standard_normal((4, 2, 4, 8)).astype(np.float16)
    V = rng.standard_normal((4, 2, 4, 8)).astype(np.float16)
    nk = rng.standard_normal((3, 2, 8)).astype(np.float16)
    K2, V2 = okv.write_f16(K, V, nk, nk, [5, -1, 14], 4)
    mask = np.zeros(K.shape, bool)
    mask[1, :, 1] = True
    mask[3, :, 2] = True
    assert np.array_equal(K2[~mask], K[~mask])
    assert np.array_equal(K2[1, :, 1], nk[0]) and np.array_equal(K2[3, :, 2], nk[2])


def test_copy_blocks_reads_before_writing():
    a = np.arange(5 * 3).reshape(5, 3)
    okv.copy_blocks([a], [(0, 1), (1, 2)])   # both copies read the original contents
    assert a[1].tolist() == [0, 1, 2] and a[2].tolist() == [3, 4, 5]


# ------------------------------------------------------------------ int8 ----

def test_int8_hand_worked_example():
    """Values derived by hand from the int8 reading (max-abs / 127, fp16 scale,
    round half to even):
    token A = [3.96875, 0.078125, 0.109375, -0.078125] into an empty block:
      amax = 3.96875 = 127/32 -> scale = 1/32 exactly; A/scale = [127, 2.5, 3.5, -2.5]
      -> codes [127, 2, 4, -2] (ties to even).
    token B = [7.9375, 0, 0, 0] appended at offset 1:
      A dequantises to [3.96875, 0.0625, 0.125, -0.0625]; amax = 7.9375 = 127/16
      -> scale 1/16; A/scale = [63.5, 1, 2, -1] -> [64, 1, 2, -1]; B -> [127, 0, 0, 0].
    """
    codes = np.full((4, 4), 99, np.int8)
    A = np.array([3.96875, 0.078125, 0.109375, -0.078125], np.float16)
    B = np.array([7.9375, 0, 0, 0], np.float16)
    c1, s1 = okv.quant_append(codes, np.float16(0.5), 0, A)
    assert s1 == np.float16(1 / 32) and c1[0].tolist() == [127, 2, 4, -2]
    assert c1[1:].tolist() == codes[1:].tolist()       # entries past the write untouched
    c2, s2 = okv.quant_append(c1, s1, 1, B)
    assert s2 == np.float16(1 / 16)
    assert c2[0].tolist() == [64, 1, 2, -1] and c2[1].tolist() == [127, 0, 0, 0]


def test_int8_first_write_scale_bits():
    """x = [1, -0.5, 0.25]: 1/127 = 0.0078740... rounds to fp16 0x2008
    (2^-7 * (1 + 8/1024) = 0.00787353515625); x/scale = [127.008, -63.504, 31.752]
    -> codes [127, -64, 32]."""
    c, s = okv.quant_append(np.zeros((2, 3), np.int8), np.float16(0), 0,
                            np.array([1, -0.5, 0.25], np.float16))
    assert s.view(np.uint16) == 0x2008
    assert c[0].tolist() == [127, -64, 32]


def test_int8_zero_and_underflow():
    c, s = okv.quant_append(np.ones((2, 3), np.int8), np.float16(1), 0, np.zeros(3, np.float16))
    assert s == 0 and c[0].tolist() == [0, 0, 0]
    # amax / 127 below half the smallest fp16 subnormal: the scale rounds to zero
    c, s = okv.quant_append(np.ones((2, 3), np.int8), np.float16(1), 0,
                            np.array([2e-7, 0, -1e-7], np.float16))
    assert s == 0 and c[0].tolist() == [0, 0, 0]


def test_int8_properties():
    rng = np.random.default_rng(11)
    for _ in range(200):
        o = int(rng.integers(0, 16))
        codes = rng.integers(-127, 128, (16, 32)).astype(np.int8)
        scale = np.float16(rng.uniform(0.005, 0.1))
        new = rng.standard_normal(32).astype(np.float16)
        c, s = okv.quant_append(codes, scale, o, new)
        # the new token's dequantised error is at most half a step
        err = np.abs(c[o].astype(np.float64) * float(s) - new.astype(np.float64))
        assert np.all(err <= float(s) / 2 + 1e-12)
        # old entries requantised within half a step of their old values
        old = codes[:o].astype(np.float64) * float(scale)
        assert np.all(np.abs(c[:o].astype(np.float64) * float(s) - old) <= float(s) / 2 + 1e-12)
        # the max-abs entry maps to +-127 and all codes lie in range
        allx = np.concatenate([old, new[None].astype(np.float64)])
        j = np.unravel_index(np.argmax(np.abs(allx)), allx.shape)
        assert abs(int(c[:o + 1][j])) == 127
        assert np.all(np.abs(c[:o + 1].astype(int)) <= 127)
        # sign symmetry and power-of-two scale invariance
        cn, sn = okv.quant_append(-codes, scale, o, -new)
        assert sn == s and np.array_equal(cn[:o + 1], -c[:o + 1])
        c2, s2 = okv.quant_append(codes, np.float16(2 * float(scale)), o, (2 * new.astype(np.float32)).astype(np.float16))
        assert s2 == np.float16(2 * float(s)) and np.array_equal(c2[:o + 1], c[:o + 1])


def test_int8_exact_multiples_roundtrip():
    s = np.float16(2.0 ** -5)
    k = np.array([127, -3, 0, 55, -127, 1], np.int8)
    c, s1 = okv.quant_append(np.zeros((2, 6), np.int8), np.float16(0), 0,
                             (k.astype(np.float32) * np.float32(s)).astype(np.float16))
    assert s1 == s and np.array_equal(c[0], k)


def test_int8_vectorised_equals_scalar():
    rng = np.random.default_rng(12)
    n, H, bs, D = 7, 3, 16, 8
    for o in (0, 1, 5, 15):
        codes = rng.integers(-127, 128, (n, H, bs, D)).astype(np.int8)
        sc = rng.uniform(0.005, 0.1, (n, H)).astype(np.float16)
        new = rng.standard_normal((n, H, D)).astype(np.float16)
        new[0, 0] = 0
        codes[0, 0] = 0
        c, s = okv.quant_append_many(codes, sc, o, new)
        for i in range(n):
            for h in range(H):
                cc, ss = okv.quant_append(codes[i, h], sc[i, h], o, new[i, h])
                assert ss == s[i, h] and np.array_equal(cc, c[i, h])


def test_int8_context_fill_equals_token_replay():
    rng = np.random.default_rng(13)
    nb, H, bs, D = 9, 2, 16, 8
    K = rng.integers(-127, 128, (nb, H, bs, D)).astype(np.int8)
    V = rng.integers(-127, 128, (nb, H, bs, D)).astype(np.int8)
    KS = rng.uniform(0.01, 0.05, (nb, H)).astype(np.float16)
    VS = rng.uniform(0.01, 0.05, (nb, H)).astype(np.float16)
    n = 53
    table = list(rng.permutation(nb)[:4])
    ck = rng.standard_normal((n, H, D)).astype(np.float16)
    cv = rng.standard_normal((n, H, D)).astype(np.float16)
    slots = [int(table[p // bs]) * bs + p % bs for p in range(n)]
    K1, V1, KS1, VS1 = okv.write_i8(K, V, KS, VS, ck, cv, slots, bs)
    K2, V2, KS2, VS2 = K.copy(), V.copy(), KS.copy(), VS.copy()
    okv.fill_context_i8(K2, V2, KS2, VS2, table, ck, cv, bs)
    for a, b in ((K1, K2), (V1, V2), (KS1, KS2), (VS1, VS2)):
        assert np.array_equal(a, b)


# ------------------------------------------------------------- attention ----

def _random_paged(rng, lens, hkv, d, bs, nb_extra=3, dtype=np.float16):
    nb = sum(opg.blocks_for(L, bs) for L in lens) + nb_extra
    st = opg.RefState(nb, bs, first_pops=rng.permutation(nb))
    for L in lens:
        st.add(int(L))
    K = rng.standard_normal((nb, hkv, bs, d)).astype(dtype)
    V = rng.standard_normal((nb, hkv, bs, d)).astype(dtype)
    return st, K, V


def test_attention_equals_contiguous_sdpa():
    """Contiguous K/V written into pages through the oracle's own tables and
    slots, then paged attention == torch SDPA (fp64, CPU) on the contiguous
    originals: decode rows see all keys; chunk row t sees the first
    L - Q + t + 1 keys; a full prefill (Q == L) is SDPA's own causal mask."""
    rng = np.random.default_rng(21)
    hq, hkv, d, bs = 8, 2, 16, 4
    lens = [1, 5, 16, 23, 9]
    qls = [1, 2, 16, 7, 9]
    nb = sum(opg.blocks_for(L, bs) for L in lens) + 2
    st = opg.RefState(nb, bs, first_pops=rng.permutation(nb))
    K = rng.standard_normal((nb, hkv, bs, d)).astype(np.float16)
    V = rng.standard_normal((nb, hkv, bs, d)).astype(np.float16)
    conts = []
    for L in lens:
        i = st.add(0)
        slots, _ = st.append(i, L)
        ck = rng.standard_normal((L, hkv, d)).astype(np.float16)
        cv = rng.standard_normal((L, hkv, d)).astype(np.float16)
        K, V = okv.write_f16(K, V, ck, cv, slots, bs)
        conts.append((ck, cv))
    q = rng.standard_normal((sum(qls), hq, d)).astype(np.float16)
    scale = d ** -0.5
    out = oatt.paged_attention(q, K, V, st.tables, lens, qls, scale, bs)
    F = torch.nn.functional
    r = 0
    for (ck, cv), L, Q in zip(conts, lens, qls):
        kt = torch.from_numpy(ck.astype(np.float64)).permute(1, 0, 2)[None]   # [1, Hkv, L, D]
        vt = torch.from_numpy(cv.astype(np.float64)).permute(1, 0, 2)[None]
        for t in range(Q):
            n = L - Q + t + 1
            qt = torch.from_numpy(q[r + t].astype(np.float64))[None, :, None, :]  # [1, Hq, 1, D]
            ref = F.scaled_dot_product_attention(qt, kt[:, :, :n], vt[:, :, :n], scale=scale, enable_gqa=True)
            assert np.allclose(out[r + t], ref[0, :, 0].numpy(), rtol=0, atol=1e-12)
        if Q == L:
            qa = torch.from_numpy(q[r:r + Q].astype(np.float64)).permute(1, 0, 2)[None]
            ref = F.scaled_dot_product_attention(qa, kt, vt, is_causal=True, scale=scale, enable_gqa=True)
            assert np.allclose(out[r:r + Q], ref[0].permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)
        r += Q


def test_permutation_invariance():
    rng = np.random.default_rng(22)
    hq, hkv, d, bs = 4, 2, 8, 4
    lens, qls = [7, 12, 3], [1, 5, 3]
    st, K, V = _random_paged(rng, lens, hkv, d, bs)
    q = rng.standard_normal((sum(qls), hq, d)).astype(np.float16)
    base = oatt.paged_attention(q, K, V, st.tables, lens, qls, 0.3, bs)
    perm = rng.permutation(K.shape[0])
    K2 = np.empty_like(K)
    V2 = np.empty_like(V)
    K2[perm] = K
    V2[perm] = V
    tables2 = [[int(perm[b]) for b in t] for t in st.tables]
    assert np.array_equal(oatt.paged_attention(q, K2, V2, tables2, lens, qls, 0.3, bs), base)


def test_closed_forms():
    rng = np.random.default_rng(23)
    hq, hkv, d, bs = 4, 2, 8, 4
    st, K, V = _random_paged(rng, [1, 9, 14], hkv, d, bs)
    q = rng.standard_normal((3, hq, d)).astype(np.float16)
    # L = 1: the output is v_0 exactly
    out = oatt.paged_attention(q[:1], K, V, st.tables[:1], [1], [1], 0.7, bs)
    b0 = st.tables[0][0]
    assert np.array_equal(out[0], np.repeat(V[b0, :, 0, :].astype(np.float64), hq // hkv, axis=0))
    # q = 0: uniform weights, output = mean of the visible V
    out = oatt.paged_attention(np.zeros((1, hq, d), np.float16), K, V, st.tables[1:2], [9], [1], 0.7, bs)
    Vc = oatt.gather(V, st.tables[1], 9, bs)
    assert np.allclose(out[0], np.repeat(Vc.mean(0), hq // hkv, axis=0), atol=1e-14)
    # constant V: the output is that constant whatever the scores
    Vk = np.full_like(V, np.float16(-1.375))
    out = oatt.paged_attention(q[2:3], K, Vk, st.tables[2:3], [14], [1], 0.7, bs)
    assert np.allclose(out, -1.375, rtol=0, atol=1e-14)
    # a single dominant key takes all the weight
    Kd = np.zeros_like(K)
    b, o = st.tables[1][1], 2          # position 6 of sequence 1
    Kd[b, :, o, :] = 1
    qd = np.full((1, hq, d), 8, np.float16)
    out = oatt.paged_attention(qd, Kd, V, st.tables[1:2], [9], [1], 1.0, bs)
    assert np.allclose(out[0], np.repeat(V[b, :, o, :].astype(np.float64), hq // hkv, axis=0), atol=1e-12)


def test_gqa_equals_repeated_mha():
    rng = np.random.default_rng(24)
    hq, hkv, d, bs = 8, 2, 8, 4
    lens, qls = [6, 11], [1, 4]
    st, K, V = _random_paged(rng, lens, hkv, d, bs)
    q = rng.standard_normal((5, hq, d)).astype(np.float16)
    gqa = oatt.paged_attention(q, K, V, st.tables, lens, qls, 0.4, bs)
    Km = np.repeat(K, hq // hkv, axis=1)
    Vm = np.repeat(V, hq // hkv, axis=1)
    mha = oatt.paged_attention(q, Km, Vm, st.tables, lens, qls, 0.4, bs)
    assert np.allclose(gqa, mha, rtol=0, atol=1e-13)


def test_chunk_row_equals_decode():
    rng = np.random.default_rng(25)
    hq, hkv, d, bs = 4, 1, 8, 4
    st, K, V = _random_paged(rng, [13], hkv, d, bs)
    Q = 6
    q = rng.standard_normal((Q, hq, d)).astype(np.float16)
    chunk = oatt.paged_attention(q, K, V, st.tables, [13], [Q], 0.5, bs)
    for t in range(Q):
        dec = oatt.paged_attention(q[t:t + 1], K, V, st.tables, [13 - Q + t + 1], [1], 0.5, bs)
        assert np.allclose(chunk[t], dec[0], rtol=0, atol=1e-13)


@pytest.mark.parametrize("int8", [False, True])
def test_brute_force_tiny(int8):
    rng = np.random.default_rng(26 + int8)
    hq, hkv, d, bs = 4, 2, 4, 4
    lens, qls = [5, 9, 2], [1, 3, 2]
    nb = sum(opg.blocks_for(L, bs) for L in lens) + 1
    st = opg.RefState(nb, bs, first_pops=rng.permutation(nb))
    for L in lens:
        st.add(L)
    if int8:
        K = rng.integers(-127, 128, (nb, hkv, bs, d)).astype(np.int8)
        V = rng.integers(-127, 128, (nb, hkv, bs, d)).astype(np.int8)
        ks = rng.uniform(0.01, 0.05, (nb, hkv)).astype(np.float16)
        vs = rng.uniform(0.01, 0.05, (nb, hkv)).astype(np.float16)
    else:
        K = rng.standard_normal((nb, hkv, bs, d)).astype(np.float16)
        V = rng.standard_normal((nb, hkv, bs, d)).astype(np.float16)
        ks = vs = None
    q = rng.standard_normal((sum(qls), hq, d)).astype(np.float16)
    vec = oatt.paged_attention(q, K, V, st.tables, lens, qls, 0.5, bs, ks, vs)
    bf = brute.paged_attention(q.tolist(), K.tolist(), V.tolist(), st.tables, lens, qls, 0.5, bs,
                               None if ks is None else ks.tolist(), None if vs is None else vs.tolist())
    assert np.allclose(vec, np.array(bf), rtol=0, atol=1e-12)


def test_scale_enters_scores():
    """Doubling the scale equals doubling q (scores are scale * q.k)."""
    rng = np.random.default_rng(27)
    st, K, V = _random_paged(rng, [10], 1, 8, 4)
    q = rng.standard_normal((1, 1, 8)).astype(np.float16)
    a = oatt.paged_attention(q, K, V, st.tables, [10], [1], 0.5, 4)
    b = oatt.paged_attention((2 * q.astype(np.float32)).astype(np.float16), K, V, st.tables, [10], [1], 0.25, 4)
    assert np.allclose(a, b, rtol=0, atol=1e-13)
    c = oatt.paged_attention(q, K, V, st.tables, [10], [1], 1.0, 4)
    assert not np.allclose(a, c, atol=1e-6)


# --------------------------------------------------------- sliding window ----
# [pytorch] "PagedAttention vs sliding-window attention, RadixAttention, and
# SSMs": each query attends only to the most recent w tokens; the window caps
# the retained history while paging manages the blocks that hold it.

def test_window_attention_equals_sdpa_on_the_window():
    """Row at position P with window w == SDPA (fp64) over keys max(0, P-w+1)..P of
    the contiguous originals; w >= L is plain causal attention, bit for bit."""
    rng = np.random.default_rng(41)
    hq, hkv, d, bs = 8, 2, 16, 4
    lens, qls = [1, 9, 23, 17], [1, 3, 7, 17]
    nb = sum(opg.blocks_for(L, bs) for L in lens) + 2
    st = opg.RefState(nb, bs, first_pops=rng.permutation(nb))
    K = rng.standard_normal((nb, hkv, bs, d)).astype(np.float16)
    V = rng.standard_normal((nb, hkv, bs, d)).astype(np.float16)
    conts = []
    for L in lens:
        i = st.add(0)
        slots, _ = st.append(i, L)
        ck = rng.standard_normal((L, hkv, d)).astype(np.float16)
        cv = rng.standard_normal((L, hkv, d)).astype(np.float16)
        K, V = okv.write_f16(K, V, ck, cv, slots, bs)
        conts.append((ck, cv))
    q = rng.standard_normal((sum(qls), hq, d)).astype(np.float16)
    F = torch.nn.functional
    full = oatt.paged_attention(q, K, V, st.tables, lens, qls, 0.25, bs)
    assert np.array_equal(oatt.paged_attention(q, K, V, st.tables, lens, qls, 0.25, bs, window=max(lens)), full)
    for w in (1, 2, 5, 8):
        out = oatt.paged_attention(q, K, V, st.tables, lens, qls, 0.25, bs, window=w)
        r = 0
        for (ck, cv), L, Q in zip(conts, lens, qls):
            for t in range(Q):
                P = L - Q + t
                lo = max(0, P - w + 1)
                kt = torch.from_numpy(ck[lo:P + 1].astype(np.float64)).permute(1, 0, 2)[None]
                vt = torch.from_numpy(cv[lo:P + 1].astype(np.float64)).permute(1, 0, 2)[None]
                qt = torch.from_numpy(q[r + t].astype(np.float64))[None, :, None, :]
                ref = F.scaled_dot_product_attention(qt, kt, vt, scale=0.25, enable_gqa=True)
                assert np.allclose(out[r + t], ref[0, :, 0].numpy(), rtol=0, atol=1e-12), (w, L, t)
                if w == 1:   # one visible key: its V exactly
                    assert np.array_equal(out[r + t], np.repeat(cv[P].astype(np.float64), hq // hkv, axis=0))
            r += Q


@pytest.mark.parametrize("int8", [False, True])
def test_window_brute_force_tiny(int8):
    rng = np.random.default_rng(43 + int8)
    hq, hkv, d, bs = 4, 2, 4, 4
    lens, qls = [5, 11, 7], [1, 4, 7]
    nb = sum(opg.blocks_for(L, bs) for L in lens) + 1
    st = opg.RefState(nb, bs, first_pops=rng.permutation(nb))
    for L in lens:
        st.add(L)
    if int8:
        K = rng.integers(-127, 128, (nb, hkv, bs, d)).astype(np.int8)
        V = rng.integers(-127, 128, (nb, hkv, bs, d)).astype(np.int8)
        ks = rng.uniform(0.01, 0.05, (nb, hkv)).astype(np.float16)
        vs = rng.uniform(0.01, 0.05, (nb, hkv)).astype(np.float16)
    else:
        K = rng.standard_normal((nb, hkv, bs, d)).astype(np.float16)
        V = rng.standard_normal((nb, hkv, bs, d)).astype(np.float16)
        ks = vs = None
    q = rng.standard_normal((sum(qls), hq, d)).astype(np.float16)
    for w in (1, 3, 6):
        vec = oatt.paged_attention(q, K, V, st.tables, lens, qls, 0.5, bs, ks, vs, window=w)
        bf = brute.paged_attention(q.tolist(), K.tolist(), V.tolist(), st.tables, lens, qls, 0.5, bs,
                                   None if ks is None else ks.tolist(), None if vs is None else vs.tolist(), window=w)
        assert np.allclose(vec, np.array(bf), rtol=0, atol=1e-12)


def test_window_releases_blocks_that_leave_it():
    """bs 4, w 6, one sequence growing by decode steps from 3 tokens: after the
    step that makes it L tokens long, keys before L - 1 - 6 + 1 = L - 6 are
    out of every present and future window, so blocks whose last position is
    below L - 6 are released (table entry -1) and come back on the stack."""
    st = opg.RefState(8, 4)                 # first pops 0, 1, 2, ...
    st.add(3)                               # [0]
    held = []
    for L in range(4, 21):
        opg.apply_step(st, [1], window=6)
        held.append(list(st.tables[0]))
        lo = max(0, L - 6)
        for lb, b in enumerate(st.tables[0]):
            assert (b == -1) == ((lb + 1) * 4 <= lo), (L, st.tables[0])
        live = [b for b in st.tables[0] if b >= 0]
        assert len(live) <= -(-6 // 4) + 1
        assert sorted(live + st.pool.stack) == list(range(8))
    # L = 10 releases block 0 (positions 0-3 < 4); block 0 is then reused at L = 13 for logical
    # block 3, and L = 14 releases block 1 (positions 4-7 < 8)
    assert held[10 - 4] == [-1, 1, 2]
    assert held[13 - 4] == [-1, 1, 2, 0]
    assert held[14 - 4] == [-1, -1, 2, 0]
    # a step with 3 query tokens keeps what its first query still sees
    st = opg.RefState(8, 4)
    st.add(10)                              # blocks 0, 1, 2 (positions 0-9)
    opg.apply_step(st, [3], window=4)       # L = 13, earliest visible key 13 - 3 - 4 + 1 = 7
    assert st.tables[0] == [-1, 1, 2, 3]

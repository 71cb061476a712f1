"""Host bookkeeping (paged_kv_cache_47_amd.host) on the CPU.

* The allocator contract of the pages: [nanoserve] "What I learned" (distinct
  blocks, atomic multi-block reserve, LIFO reuse after free, double and
  foreign frees rejected, exhaustion raises its own error), [engine] "02 The
  engine" (interleaved out-of-order allocate/free keeps counts and ownership
  consistent), [manager] "Running and Testing It" (fork doubles refcounts, a
  second finish is harmless).
* Bit-exact agreement of tables, slot mappings, lengths and copy-on-write
  pairs with the oracle's own bookkeeping on all five workloads at full size.
"""
import json
import os

import numpy as np
import pytest

import synthetic
from oracle import paging as opg
from paged_kv_cache_47_amd.host import BlockAllocator, KVCacheExhausted, PagedKVManager
from paged_kv_cache_47_amd.workload import build_manager

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_nanoserve_trace():
    with open(os.path.join(GOLD, "nanoserve_allocator_trace.json")) as f:
        g = json.load(f)
    a = BlockAllocator(g["num_blocks"])
    held = {}
    for op in g["ops"]:
        if op["op"] == "allocate_for":
            if "expect_error" in op:
                with pytest.raises(KVCacheExhausted):
                    a.allocate_for(op["tokens"], g["block_size"])
            else:
                held[op["name"]] = a.allocate_for(op["tokens"], g["block_size"])
                assert held[op["name"]] == op["expect_ids"]
        else:
            a.free_all(held.pop(op["name"]))
        assert a.num_free == op["expect_free"]


def test_distinct_blocks_and_exhaustion():
    a = BlockAllocator(5)
    ids = [a.allocate() for _ in range(5)]
    assert sorted(ids) == list(range(5))
    assert not a.can_allocate(1)
    with pytest.raises(KVCacheExhausted):
        a.allocate()


def test_atomic_reserve():
    a = BlockAllocator(6)
    a.allocate_for(33, 16)                   # 3 blocks
    before = a.free_ids()
    with pytest.raises(KVCacheExhausted):
        a.allocate_for(4 * 16, 16)           # needs 4, 3 free
    assert a.free_ids() == before and a.num_free == 3
    assert a.allocate_for(0, 16) == []


def test_reuse_after_free_is_lifo():
    a = BlockAllocator(6)
    x = a.allocate_for(40, 16)
    a.allocate_for(20, 16)
    a.free_all(x)                            # pushes 0, 1, 2
    assert a.allocate_for(30, 16) == [2, 1]


@pytest.mark.parametrize("bad", ["double", "foreign", "negative", "shared"])
def test_bad_frees_raise(bad):
    a = BlockAllocator(4)
    b = a.allocate()
    if bad == "double":
        a.free(b)
        with pytest.raises(ValueError):
            a.free(b)
    elif bad == "foreign":
        with pytest.raises(ValueError):
            a.free(99)
    elif bad == "negative":
        with pytest.raises(ValueError):
            a.free(-1)
    else:
        a.retain(b)
        with pytest.raises(ValueError):
            a.free(b)                         # two owners: release, do not free
        a.release(b)
        a.free(b)
    assert a.num_free + len(a.allocated_ids()) == 4


def test_first_pops_order_and_validation():
    a = BlockAllocator(4, first_pops=[2, 0, 3, 1])
    assert [a.allocate() for _ in range(4)] == [2, 0, 3, 1]
    with pytest.raises(ValueError):
        BlockAllocator(4, first_pops=[0, 1, 1, 2])


def test_interleaved_out_of_order():
    rng = np.random.default_rng(5)
    nb, bs = 48, 16
    m = PagedKVManager(nb, bs, first_pops=rng.permutation(nb))
    live = []
    for _ in range(600):
        op = int(rng.integers(0, 5))
        try:
            if op == 0 or not live:
                live.append(m.add_sequence(int(rng.integers(0, 70))))
            elif op == 1:
                live.append(m.fork(live[int(rng.integers(len(live)))]))
            elif op in (2, 3):
                m.append(live[int(rng.integers(len(live)))], int(rng.integers(1, 20)))
            else:
                m.finish(live.pop(int(rng.integers(len(live)))))
        except KVCacheExhausted:
            pass
        owners = {}
        for s in live:
            for b in m.blocks(s):
                owners[b] = owners.get(b, 0) + 1
            assert len(m.blocks(s)) == -(-m.seq_len(s) // bs)
        assert owners == {int(b): m.alloc.refcount(b) for b in m.alloc.allocated_ids()}
        assert m.alloc.num_free + len(owners) == nb
        assert set(m.alloc.free_ids()).isdisjoint(owners)
    for s in live:
        m.finish(s)
    assert m.alloc.num_free == nb


def test_fork_doubles_refcounts_and_finish_twice():
    m = PagedKVManager(8, 16)
    p = m.add_sequence(16 * 3)
    before = [m.alloc.refcount(b) for b in m.blocks(p)]
    c = m.fork(p)
    assert [m.alloc.refcount(b) for b in m.blocks(p)] == [2 * r for r in before]
    m.finish(p)
    m.finish(p)
    assert [m.alloc.refcount(b) for b in m.blocks(c)] == before
    m.finish(c)
    assert m.alloc.num_free == 8


def test_copy_on_write_pairs():
    m = PagedKVManager(10, 4)
    p = m.add_sequence(6)                     # blocks [0, 1], block 1 half full
    c = m.fork(p)
    slots, copies = m.append(c, 1)            # writes into shared block 1: copy first
    assert copies == [(1, 2)] and slots == [2 * 4 + 2]
    assert m.blocks(c) == [0, 2] and m.blocks(p) == [0, 1]
    slots, copies = m.append(p, 1)            # now sole owner of block 1: in place
    assert copies == [] and slots == [1 * 4 + 2]
    slots, copies = m.append(c, 3)            # fills block 2, then a fresh block
    assert copies == [] and slots == [2 * 4 + 3, 3 * 4 + 0, 3 * 4 + 1]


def test_slots_of_existing_positions():
    m = PagedKVManager(8, 4, first_pops=[5, 2, 7, 0, 1, 3, 4, 6])
    s = m.add_sequence(7)
    assert m.slots(s, 0, 7).tolist() == [20, 21, 22, 23, 8, 9, 10]
    with pytest.raises(ValueError):
        m.slots(s, 5, 3)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_metadata_matches_oracle_full_size(cfg):
    w = synthetic.CONFIGS[cfg]()
    mgr, ids = build_manager(w)
    st = opg.build_state(w)
    assert [mgr.blocks(s) for s in ids] == st.tables
    for s in range(w.num_steps):
        q_lens = w.step(s).q_lens
        b = mgr.step(ids, q_lens)
        slots, copies = opg.apply_step(st, q_lens)
        assert np.array_equal(b.slot_mapping, slots.astype(np.int32)), f"step {s}"
        assert [tuple(p) for p in b.copy_pairs.tolist()] == [tuple(p) for p in copies]
        assert b.seq_lens.tolist() == st.lens
        assert np.array_equal(b.block_tables, opg.table_array(st, b.block_tables.shape[1]).astype(np.int32))
    if cfg == 1:
        assert [len(t) for t in st.tables] == [3, 2, 1, 2]
    if cfg == 4:
        prefix = st.tables[0][:64]
        assert all(mgr.alloc.refcount(b) == 64 + 16 * 3 for b in prefix)
        assert len(b.copy_pairs) == 3 * sum(1 for r in range(16) if int(w.ctx_lens[r]) % 16)


def test_window_release_trace():
    # the hand-worked trace of the oracle's pin, through the host manager:
    # block size 4, window 6, first pops 0, 1, 2, ...
    m = PagedKVManager(8, 4, window=6)
    s = m.add_sequence(9)                      # blocks [0, 1, 2]
    b = m.step([s], [1])                       # L=10: keys 4..9 visible -> block 0 released
    assert m.blocks(s) == [-1, 1, 2] and b.block_tables.tolist() == [[-1, 1, 2]]
    m.step([s], [3])                           # L=13: positions 12 take block 0 again; keys 7..12
    assert m.blocks(s) == [-1, 1, 2, 0]
    m.step([s], [1])                           # L=14: keys 8..13 -> block 1 released
    assert m.blocks(s) == [-1, -1, 2, 0] and m.alloc.free_ids()[-1] == 1
    with pytest.raises(ValueError):
        m.slots(s, 0, 2)                       # released positions have no slots
    m.finish(s)
    assert m.alloc.num_free == 8


@pytest.mark.parametrize("cfg,window", [(2, 1), (2, 16), (2, 100), (4, 17), (4, 2000), (3, 300), (5, 1000)])
def test_window_metadata_matches_oracle(cfg, window):
    w = synthetic.CONFIGS[cfg](**({"decode_steps": 20} if cfg == 2 else {}))
    w.window = window
    mgr, ids = build_manager(w)
    st = opg.build_state(w)
    for s in range(w.num_steps):
        q_lens = w.step(s).q_lens
        b = mgr.step(ids, q_lens)
        slots, copies = opg.apply_step(st, q_lens, window)
        assert np.array_equal(b.slot_mapping, slots.astype(np.int32)), f"step {s}"
        assert [tuple(p) for p in b.copy_pairs.tolist()] == [tuple(p) for p in copies]
        assert b.seq_lens.tolist() == st.lens
        assert np.array_equal(b.block_tables, opg.table_array(st, b.block_tables.shape[1]).astype(np.int32))
        assert mgr.alloc.free_ids() == st.pool.stack
    assert any(-1 in mgr.blocks(i) for i in ids) == (window < max(st.lens))


def _snapshot(m, ids):
    return ([m.blocks(s) for s in ids], [m.seq_len(s) for s in ids], m.alloc.free_ids(),
            m.alloc.refcounts().tolist())


def test_step_is_atomic_when_the_pool_runs_out():
    m = PagedKVManager(6, 4)
    a = m.add_sequence(7)                     # 2 blocks
    b = m.add_sequence(4)                     # 1 block
    c = m.fork(a)                             # shares a's 2 blocks
    before = _snapshot(m, [a, b, c])
    # a: copy of the shared block 1 (pos 7) + a new block (pos 8); c: then sole owner of block 1,
    # a new block for pos 8; b: 2 new blocks -> 5 > 3 free
    with pytest.raises(KVCacheExhausted):
        m.step([a, c, b], [2, 2, 5])
    assert _snapshot(m, [a, b, c]) == before
    with pytest.raises(ValueError):           # a sequence listed twice
        m.step([a, a], [1, 1])
    with pytest.raises(ValueError):           # a table narrower than the step needs
        m.step([a], [2], width=2)
    assert _snapshot(m, [a, b, c]) == before
    x = m.step([a, c, b], [2, 2, 0])          # 2 + 1 + 0 blocks: fits exactly
    assert m.alloc.num_free == 0 and x.copy_pairs.tolist() == [[1, 3]]


def test_window_release_counts_toward_the_same_step():
    # a block one sequence's window releases is free for the later sequences of that step
    m = PagedKVManager(4, 4, window=2)
    a = m.add_sequence(6)                     # blocks [0, 1]
    b = m.add_sequence(8)                     # blocks [2, 3]: the pool is full
    before = _snapshot(m, [a, b])
    with pytest.raises(KVCacheExhausted):     # b first: it needs a block before anything is released
        m.step([b, a], [1, 2])
    assert _snapshot(m, [a, b]) == before
    x = m.step([a, b], [2, 1])                # a: L=8, keys 5.. -> block 0 released; b takes it for pos 8
    assert x.slot_mapping.tolist() == [6, 7, 0]
    assert m.blocks(a) == [-1, 1] and m.blocks(b) == [-1, 3, 0]   # b: L=9, keys 7.. -> its block 2 released
    assert m.alloc.free_ids() == [2]


def _oracle_finish(st, i):
    for b in st.tables[i]:
        if b >= 0:
            st.pool.release(b)
    st.tables[i] = []


@pytest.mark.parametrize("seed,window", [(1, 0), (2, 0), (3, 5), (4, 17), (5, 1)])
def test_random_interleavings_match_the_oracle(seed, window):
    rng = np.random.default_rng(seed)
    nb, bs = 96, 4
    perm = rng.permutation(nb)
    m = PagedKVManager(nb, bs, first_pops=perm, window=window)
    st = opg.RefState(nb, bs, first_pops=perm)
    live = []
    for _ in range(300):
        op = rng.integers(0, 10)
        if op < 2 and m.alloc.num_free >= 8:
            n = int(rng.integers(0, 20))
            live.append(m.add_sequence(n))
            assert st.add(n) == live[-1]
        elif op < 3 and live and not window:
            src = live[int(rng.integers(len(live)))]
            live.append(m.fork(src))
            assert st.fork(src) == live[-1]
        elif op < 4 and live:
            sid = live.pop(int(rng.integers(len(live))))
            m.finish(sid)
            _oracle_finish(st, sid)
        elif live:
            k = int(rng.integers(1, len(live) + 1))
            sids = [int(s) for s in rng.choice(live, size=k, replace=False)]
            qls = [int(q) for q in rng.integers(0, 6, size=k)]
            pool_before = list(st.pool.stack)
            try:
                b = m.step(sids, qls)
            except KVCacheExhausted:
                st.pool.stack = pool_before
                assert m.alloc.free_ids() == st.pool.stack
                continue
            slots, copies = [], []
            for s, q in zip(sids, qls):
                sl, cp = st.append(s, q)
                slots += sl
                copies += cp
                if window:
                    opg.release_out_of_window(st, s, q, window)
            assert b.slot_mapping.tolist() == slots
            assert [tuple(p) for p in b.copy_pairs.tolist()] == copies
        for s in live:
            assert m.blocks(s) == st.tables[s] and m.seq_len(s) == st.lens[s]
        assert m.alloc.free_ids() == st.pool.stack

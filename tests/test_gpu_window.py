"""Sliding-window attention on the GPU, through the C ABI, against the oracle.

[pytorch] "PagedAttention vs sliding-window attention, RadixAttention, and
SSMs": a query at position P sees keys max(0, P - w + 1) .. P, and blocks
that no query of a step can see any more are released (their table entries
become -1).  Covered: windows from 1 key to more than the longest sequence,
on both dispatch paths (vector and MFMA, each forced for every row too) and
every split-K partition size, fp16 and int8 pools, several decode steps with
releases and block reuse, and poison in every released block (no kernel may
read a block its window has left behind).
"""
import dataclasses

import numpy as np
import pytest
import torch

import synthetic
from tests.oracle_side import OracleSide
from tests.test_gpu_parity import SPLITS, _check_step

pytestmark = pytest.mark.gpu

LENS = [1, 2, 15, 16, 17, 33, 100, 257, 700, 90, 1500]
QLS = [1, 1, 1, 1, 2, 3, 16, 40, 1, 90, 300]
BOTH_PATHS = SPLITS + ({"mfma_min_rows": 1}, {"mfma_min_rows": 2 ** 31 - 1})


def _run(w):
    from paged_kv_cache_47_amd.workload import DeviceRun
    return DeviceRun(w)


@pytest.mark.parametrize("window", [1, 2, 15, 16, 17, 64, 100, 257, 5000])
def test_window_mixed_batch_f16(window):
    w = synthetic.custom(200 + window, LENS, QLS, 8, 2, 128, window=window)
    _check_step(_run(w), OracleSide(w), 0, BOTH_PATHS)


@pytest.mark.parametrize("window", [1, 17, 100, 700])
def test_window_mixed_batch_int8(window):
    w = synthetic.custom(300 + window, LENS, QLS, 8, 2, 128, "i8", window=window)
    _check_step(_run(w), OracleSide(w), 0, BOTH_PATHS)


@pytest.mark.parametrize("hq,hkv,d,dt,window", [
    (12, 12, 64, "f16", 33), (32, 4, 128, "f16", 129), (16, 2, 64, "i8", 48), (8, 1, 128, "f16", 16),
    (16, 2, 128, "i8", 17), (64, 8, 128, "i8", 100),   # int8 groups of eight at head dim 128 (quad K layout)
])
def test_window_groups_and_head_dims(hq, hkv, d, dt, window):
    w = synthetic.custom(400 + window, LENS, QLS, hq, hkv, d, dt, window=window)
    _check_step(_run(w), OracleSide(w), 0, ({}, {"partition_tokens": 16}, {"mfma_min_rows": 1}))


def test_window_prefill_then_decode_steps():
    # causal prefill of every prompt, then decode steps that release blocks and reuse them
    w = synthetic.config2(num_seqs=6, min_prompt=17, max_prompt=150, decode_steps=20)
    w.window = 24
    run, ora = _run(w), OracleSide(w)
    _check_step(run, ora, 0, ({}, {"mfma_min_rows": 2 ** 31 - 1, "partition_tokens": 16}))
    for s in range(1, 21):
        _check_step(run, ora, s, SPLITS if s % 5 == 0 else ({},))
    assert any(-1 in run.mgr.blocks(i) for i in run.ids)


@pytest.mark.parametrize("dt", ["f16", "i8"])
def test_released_blocks_are_never_read(dt):
    w = synthetic.custom(500, [700, 257, 1500, 90, 33], [1, 40, 300, 1, 1], 8, 2, 128, dt, window=100)
    run = _run(w)
    x = run.prepare(0)
    run.write(x)
    clean = [run.attend(x, **o).clone() for o in BOTH_PATHS]
    free = run.mgr.alloc.free_ids()
    assert (x.block_tables < 0).any() and free
    idx = torch.tensor(free, dtype=torch.long, device="cuda")
    if dt == "f16":
        run.k_cache[idx] = float("nan")
        run.v_cache[idx] = float("nan")
    else:
        run.k_cache[idx] = 127
        run.v_cache[idx] = -127
        run.k_scale[idx] = float("nan")
        run.v_scale[idx] = float("inf")
    bt = x.block_tables.clone()
    bt[bt < 0] = free[0]
    poisoned = dataclasses.replace(x, block_tables=bt)
    for o, ref in zip(BOTH_PATHS, clean):
        got = run.attend(poisoned, **o)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), o


def test_window_rejects_negative():
    from paged_kv_cache_47_amd import pa
    w = synthetic.custom(501, [40], [1], 8, 2, 128)
    run = _run(w)
    x = run.prepare(0)
    with pytest.raises(pa.PagedAttentionError):
        pa.pa_attend(x.q, run.k_cache, run.v_cache, x.block_tables, x.seq_lens, x.q_lens, x.batch.seq_lens,
                     x.batch.q_lens, 0.1, window=-1)

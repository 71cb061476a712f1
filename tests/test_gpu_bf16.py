"""bf16 pools on the GPU, through the C ABI, against the oracle.

[pytorch] "Compute reference attention without hiding the layout" checks a
paged bf16 cache against its own tolerance (absolute 5e-3).  bf16 pools take
bf16 new rows and queries and return bf16 outputs; the products run on
v_dot2_f32_bf16 (vector path) and v_mfma_f32_16x16x32_bf16 (MFMA path) with
fp32 accumulation.  Covered: bit-exact writes, both dispatch paths (each
forced for every row), every split-K partition size, group sizes and head
dims, a multi-layer pool, a sliding window, and the exact case of a single
visible key.  The inputs are N(0,1) draws rounded to bf16.
"""
import numpy as np
import pytest
import torch

import synthetic
from tests.oracle_side import OracleSide, assert_attn_close, dev_np
from tests.test_gpu_parity import SPLITS, _check_step

pytestmark = pytest.mark.gpu

LENS = [1, 2, 15, 16, 17, 33, 100, 257, 700, 90, 1500]
QLS = [1, 1, 1, 1, 2, 3, 16, 40, 1, 90, 300]
BOTH_PATHS = SPLITS + ({"mfma_min_rows": 1}, {"mfma_min_rows": 2 ** 31 - 1})


def _run(w):
    from paged_kv_cache_47_amd.workload import DeviceRun
    return DeviceRun(w)


@pytest.mark.parametrize("hq,hkv,d", [(8, 2, 128), (32, 8, 128), (12, 12, 64), (16, 2, 64), (8, 1, 128)])
def test_bf16_mixed_batch(hq, hkv, d):
    w = synthetic.custom(700 + hq + d, LENS, QLS, hq, hkv, d, "bf16")
    _check_step(_run(w), OracleSide(w), 0, BOTH_PATHS)


def test_bf16_window():
    w = synthetic.custom(720, LENS, QLS, 8, 2, 128, "bf16", window=100)
    _check_step(_run(w), OracleSide(w), 0, BOTH_PATHS)


def test_bf16_prefill_then_decode():
    w = synthetic.config2(num_seqs=6, min_prompt=17, max_prompt=150, decode_steps=3, kv_dtype="bf16")
    run, ora = _run(w), OracleSide(w)
    _check_step(run, ora, 0, ({}, {"mfma_min_rows": 2 ** 31 - 1, "partition_tokens": 32}))
    for s in (1, 2, 3):
        _check_step(run, ora, s, SPLITS)


def test_bf16_single_key_is_exact():
    # one visible key: its weight is exactly 1, so the output is that key's V, exactly
    w = synthetic.custom(721, [1, 1, 1], [1, 1, 1], 8, 2, 128, "bf16")
    run = _run(w)
    x = run.prepare(0)
    run.write(x)
    for opts in ({}, {"mfma_min_rows": 1}):
        out = dev_np(run.attend(x, **opts))
        torch.cuda.synchronize()
        v = np.repeat(w.step(0).new_v, 4, axis=1)     # query head h reads KV head h // 4
        assert np.array_equal(out.view(np.uint32), v.view(np.uint32)), opts


def test_bf16_error_statistics():
    # the observed error sits well inside the gate: report it
    w = synthetic.custom(722, [40, 300, 1200, 3000], [1, 1, 64, 1], 32, 8, 128, "bf16")
    run, ora = _run(w), OracleSide(w)
    x = run.prepare(0)
    slots, copies = ora.reserve(0)
    run.write(x)
    ora.write(0, slots, copies)
    ref = ora.attend(0)
    for opts in ({}, {"mfma_min_rows": 1}):
        got = dev_np(run.attend(x, **opts))
        torch.cuda.synchronize()
        st = assert_attn_close(got, ref, "bf16", str(opts))
        print("bf16", opts, st, "mean abs", float(np.abs(got - ref).mean()))
        assert st["max_abs"] < 0.02

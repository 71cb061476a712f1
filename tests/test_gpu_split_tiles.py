"""Split row tiles on the GPU, through the C ABI, against the CPU oracle.

A row tile (256 query rows of a sequence on the MFMA path) whose keys span
more 64-key steps than the split is cut into parts of equal step counts;
each part is its own workgroup and writes its rows' normalised outputs and
log-sum-exps, which a merge kernel combines into the rows (the log-sum-exp
merge of split-K partitions, as for long decode rows).  Covered: parts of
one, two, three and five steps and the automatic split; rows that see no key
of a part (causal rows before a part's first key, windows that end before
it); fp16, bf16 and int8 pools; groups of 1, 4, 8 and 16; head dims 64 and
128; windows; a chunked prefill with a long context; several layers reusing
one plan; and the workspace-free entry point.
"""
import numpy as np
import pytest
import torch

import synthetic
from tests.oracle_side import OracleSide
from tests.test_gpu_parity import _check_step

pytestmark = pytest.mark.gpu

# chunked prefill rows over contexts of 0 to ~1000 keys, a whole prompt, and decode rows
LENS = [600, 1100, 90, 257, 1000, 40, 700]
QLS = [100, 64, 90, 17, 1, 1, 300]
FORCED = ({"mfma_split_steps": 1}, {"mfma_split_steps": 2}, {"mfma_split_steps": 3},
          {"mfma_split_steps": 5, "partition_tokens": 64}, {"mfma_split_steps": -1})


def _run(w):
    from paged_kv_cache_47_amd.workload import DeviceRun
    return DeviceRun(w)


@pytest.mark.parametrize("hq,hkv,d,dt", [
    (8, 2, 128, "f16"), (8, 8, 64, "f16"), (32, 4, 128, "bf16"), (16, 2, 128, "i8"),
    (32, 8, 128, "i8"), (4, 4, 64, "i8"), (32, 2, 128, "f16"),
])
def test_split_row_tiles(hq, hkv, d, dt):
    w = synthetic.custom(500 + hq + d, LENS, QLS, hq, hkv, d, dt)
    _check_step(_run(w), OracleSide(w), 0, FORCED + ({"mfma_split_steps": 1, "mfma_min_rows": 1},))


@pytest.mark.parametrize("window", [1, 40, 100, 300])
def test_split_row_tiles_with_a_window(window):
    # parts whose keys lie entirely before some rows' windows, or after others' positions
    w = synthetic.custom(600 + window, LENS, QLS, 8, 2, 128, window=window)
    _check_step(_run(w), OracleSide(w), 0, FORCED)
    w = synthetic.custom(650 + window, LENS, QLS, 16, 2, 128, "i8", window=window)
    _check_step(_run(w), OracleSide(w), 0, FORCED[:2])


def test_long_context_chunk_automatic_split():
    # one 512-query chunk (group 4: 8 row tiles of ~95-102 steps, 64 workgroups) over
    # 6000 cached keys: the automatic split (the row-tile work spread over 256 compute
    # units: ~25 steps) cuts each tile into about four parts
    from paged_kv_cache_47_amd import pa
    w = synthetic.custom(700, [6512, 300], [512, 1], 32, 8, 128)
    run = _run(w)
    info = pa.pa_attend_plan_info(run.k_cache, 32, [6512, 300], [512, 1])
    assert info["mfma_units"] > info["mfma_tiles"] == 8
    _check_step(run, OracleSide(w), 0, ({}, {"mfma_split_steps": -1}))


def test_split_tiles_across_layers_reuse_the_plan():
    w = synthetic.custom(710, LENS, QLS, 8, 2, 128, "i8", num_layers=3)
    run, ora = _run(w), OracleSide(w)
    x = run.prepare(0)
    slots, _ = ora.reserve(0)
    run.write(x)
    ora.write(0, slots, [])
    ws = torch.empty(1 << 26, dtype=torch.uint8, device="cuda")
    from tests.oracle_side import assert_attn_close, dev_np
    for layer in range(3):
        out = run.attend(x, workspace=ws, layer=layer, reuse_plan=layer > 0, mfma_split_steps=2)
        torch.cuda.synchronize()
        assert_attn_close(dev_np(out), ora.attend(0, layer=layer), "i8", f"layer {layer}")


def test_split_tiles_without_a_workspace():
    from paged_kv_cache_47_amd import pa
    w = synthetic.custom(720, LENS, QLS, 8, 2, 128)
    run, ora = _run(w), OracleSide(w)
    x = run.prepare(0)
    slots, _ = ora.reserve(0)
    run.write(x)
    ora.write(0, slots, [])
    out = pa.pa_attend_noalloc(run.layer_acts(x, 0)[2], run.k_cache, run.v_cache, x.block_tables, x.seq_lens,
                               x.q_lens, x.batch.seq_lens, x.batch.q_lens, w.scale, mfma_split_steps=1)
    ref = pa.pa_attend(run.layer_acts(x, 0)[2], run.k_cache, run.v_cache, x.block_tables, x.seq_lens,
                       x.q_lens, x.batch.seq_lens, x.batch.q_lens, w.scale, mfma_split_steps=1)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    from tests.oracle_side import assert_attn_close, dev_np
    assert_attn_close(dev_np(out), ora.attend(0), "f16", "noalloc split")


def test_more_parts_than_one_wave_of_lanes():
    # a 64-query chunk over ~5000 cached keys cut into one-step parts: ~80 parts per tile, more
    # than the 64 log-sum-exps the merge takes per pass
    from paged_kv_cache_47_amd import pa
    w = synthetic.custom(730, [5100, 300], [64, 1], 16, 4, 128)
    run = _run(w)
    info = pa.pa_attend_plan_info(run.k_cache, 16, [5100, 300], [64, 1], mfma_split_steps=1)
    assert info["mfma_units"] >= 65 * info["mfma_tiles"]
    _check_step(run, OracleSide(w), 0, ({"mfma_split_steps": 1}, {"mfma_split_steps": 2}))

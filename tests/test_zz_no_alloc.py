"""pa_attend_noalloc through the C ABI: the entry point for callers that
cannot allocate device memory runs pa_attend on the library's fixed per-GPU
scratch.  Its outputs must equal pa_attend's (same kernels, same plan: bit
for bit) and stay within the oracle's tolerance, on two calls in a row, the
second with a smaller batch, so whatever the first call left in the shared
scratch cannot leak into the second."""
import numpy as np
import pytest
import torch

import synthetic
from tests.oracle_side import OracleSide, assert_attn_close, dev_np

pytestmark = pytest.mark.gpu


def _step(w):
    from paged_kv_cache_47_amd.workload import DeviceRun
    run, ora = DeviceRun(w), OracleSide(w)
    x = run.prepare(0)
    slots, copies = ora.reserve(0)
    run.write(x)
    ora.write(0, slots, copies)
    return run, x, ora.attend(0)


def _noalloc(run, x, **opts):
    from paged_kv_cache_47_amd import pa
    return pa.pa_attend_noalloc(x.q, run.k_cache, run.v_cache, x.block_tables, x.seq_lens, x.q_lens,
                                x.batch.seq_lens, x.batch.q_lens, run.w.scale, k_scale=run.k_scale,
                                v_scale=run.v_scale, window=run.w.window, **opts)


@pytest.mark.parametrize("dt", ["f16", "i8"])
def test_noalloc_equals_pa_attend_on_two_calls_in_a_row(dt):
    rng = np.random.default_rng(46)
    # first call: 96 decode rows (several split), a 40-row chunk on the MFMA path and a 3-row sequence
    big_L = [int(v) for v in rng.integers(1, 5000, 96)] + [900, 60]
    big_Q = [1] * 96 + [40, 3]
    # second call: a smaller batch (fewer, shorter sequences)
    small_L = [int(v) for v in rng.integers(1, 700, 20)]
    small_Q = [1] * 20
    for seed, L, Q in ((4601, big_L, big_Q), (4602, small_L, small_Q)):
        w = synthetic.custom(seed, L, Q, 32, 8, 128, dt)
        run, x, ref = _step(w)
        for opts in ({}, {"partition_tokens": 64}, {"partition_tokens": -1}):
            got = _noalloc(run, x, **opts)
            want = run.attend(x, **opts)
            torch.cuda.synchronize()
            assert torch.equal(got, want), (seed, opts)
            assert_attn_close(dev_np(got), ref, dt, f"noalloc {seed} {opts}")


def test_noalloc_reuses_its_own_plan_across_layers():
    w = synthetic.custom(4603, [300, 2500, 17, 1200], [1, 1, 1, 20], 32, 8, 128, num_layers=2)
    run, x, _ = _step(w)
    from paged_kv_cache_47_amd import pa
    outs = []
    for layer in range(2):
        q = run.layer_acts(x, layer)[2]
        outs.append(pa.pa_attend_noalloc(q, run.k_cache, run.v_cache, x.block_tables, x.seq_lens, x.q_lens,
                                         x.batch.seq_lens, x.batch.q_lens, w.scale, layer=layer,
                                         partition_tokens=256, reuse_plan=layer > 0))
    for layer in range(2):
        want = run.attend(x, layer=layer, partition_tokens=256)
        torch.cuda.synchronize()
        assert torch.equal(outs[layer], want), layer

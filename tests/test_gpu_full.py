"""GPU parity at the workloads' full sizes, in the launch configuration
bench.py times (default dispatch options).

Workloads 2-4 are checked in full: every slot of both pools bit-exact after
each step, every output row within tolerance.  Workload 5 (an int8 pool of
220k blocks and 3.2M cached tokens) is checked on all 8 prefill chunks and
48 of the 192 decode sequences (the longest included): the oracle replays
the context of those sequences only, and their blocks (codes and scales)
must match bit for bit before and after the step.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import synthetic
from oracle import kv_write as okv
from tests.oracle_side import OracleSide, assert_attn_close
from tests.test_gpu_parity import _check_step

pytestmark = pytest.mark.gpu


def _run(w):
    from paged_kv_cache_47_amd.workload import DeviceRun
    return DeviceRun(w)


@pytest.mark.timeout(600)
def test_workload2_full_all_steps():
    w = synthetic.config2()
    run = _run(w)
    ora = OracleSide(w)
    for s in range(w.num_steps):
        _check_step(run, ora, s, ({},))


@pytest.mark.timeout(600)
def test_workload3_full():
    w = synthetic.config3()
    _check_step(_run(w), OracleSide(w), 0, ({},))


@pytest.mark.timeout(600)
def test_workload4_full():
    w = synthetic.config4()
    _check_step(_run(w), OracleSide(w), 0, ({},))


@pytest.mark.timeout(900)
def test_workload5_full_sampled():
    """Every row of all 8 chunks (the longest MFMA row tiles included) and 48
    of the 192 decode rows, the longest among them, at full size."""
    w = synthetic.config5()
    rng = np.random.default_rng(47)
    nch = 8
    dec = nch + rng.choice(192, 47, replace=False)
    dec = np.concatenate([dec, [nch + int(np.argmax(w.ctx_lens[nch:]))]])   # the longest decode sequence
    sample = sorted(set(list(range(nch)) + dec.tolist()))
    assert len(sample) >= nch + 48
    run = _run(w)
    torch.cuda.synchronize()
    # the oracle replays the sampled sequences' context token by token; sequences own disjoint
    # blocks, so their replays run side by side (numpy releases the GIL in the array work)
    ora = OracleSide(w, context_seqs=[])
    tabs = ora.st.tables

    def fill(i):
        c = int(w.ctx_lens[i])
        if c:
            ck, cv = w.context(i)
            okv.fill_context_i8(ora.K, ora.V, ora.KS, ora.VS, tabs[i], ck, cv, w.block_size)

    with ThreadPoolExecutor(8) as ex:
        for n, _ in enumerate(ex.map(fill, sorted(sample, key=lambda i: -int(w.ctx_lens[i])))):
            if n % 8 == 7:
                print(f"workload 5: oracle context of {n + 1}/{len(sample)} sequences replayed", flush=True)

    def check_blocks(when):
        for i in sample:
            blk = torch.tensor(tabs[i], dtype=torch.long, device="cuda")
            for dev, ref in ((run.k_cache, ora.K), (run.v_cache, ora.V)):
                assert np.array_equal(dev[blk].cpu().numpy(), ref[tabs[i]]), f"{when}: codes of seq {i}"
            for dev, ref in ((run.k_scale, ora.KS), (run.v_scale, ora.VS)):
                assert np.array_equal(dev[blk].cpu().numpy().view(np.uint16), ref[tabs[i]].view(np.uint16)), \
                    f"{when}: scales of seq {i}"

    check_blocks("context")
    x = run.prepare(0)
    slots, copies = ora.reserve(0)
    assert np.array_equal(x.batch.slot_mapping, slots.astype(np.int32)) and not copies
    run.write(x)
    # the oracle replays only the sampled sequences' new tokens
    starts, ql = ora.row_ranges(0)
    keep = np.full(len(slots), -1, np.int64)
    for i in sample:
        keep[starts[i]:starts[i] + ql[i]] = slots[starts[i]:starts[i] + ql[i]]
    ora.write(0, keep, copies)
    torch.cuda.synchronize()
    check_blocks("after write")
    out = run.attend(x).cpu().numpy()
    print("workload 5: blocks match after the write; oracle attention", flush=True)
    with ThreadPoolExecutor(8) as ex:
        parts = list(ex.map(lambda i: ora.attend(0, seqs={i})[starts[i]:starts[i] + ql[i]].copy(), sample))
    for i, ref in zip(sample, parts):
        assert_attn_close(out[starts[i]:starts[i] + ql[i]], ref, True, f"workload 5 sequence {i} ({int(ql[i])} rows)")

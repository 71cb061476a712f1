"""Fixed-address steps (``StaticSteps``): prepared calls and a captured HIP
graph against the oracle and against each other.

[engine] "07 Open items" names per-step host overhead as the main cost and
proposes building the step's metadata once and capturing the step in a
graph.  Here the native manager writes each step's metadata into pinned
memory, one copy moves it to fixed device buffers, and one graph replays the
block copies and every layer's write and attention.  Each replay is checked
against the oracle (writes bit-exact, outputs to tolerance) and against the
same step issued eagerly from prepared calls with the exact lengths
(bit-identical: the graph's launches are shaped for an upper bound, and the
surplus work items exit), with the program's own eager work and
synchronisations between replays.
"""
import numpy as np
import pytest
import torch

import synthetic
from oracle import paging as opg
from tests.oracle_side import OracleSide, assert_attn_close

pytestmark = pytest.mark.gpu


def _run(w):
    from paged_kv_cache_47_amd.workload import DeviceRun
    return DeviceRun(w)


def _static(run, width, **kw):
    from paged_kv_cache_47_amd.workload import StaticSteps
    return StaticSteps(run, width, **kw)


def _oracle_step(ora, s, st):
    slots, copies = ora.reserve(s)
    ora.write(s, slots, copies)
    h = st.host[st.turn]
    S, T = st.S, st.T
    assert np.array_equal(h[2 * S:2 * S + T], np.asarray(slots, np.int32))
    pairs = h[st.off["cp"]:st.off["cp"] + 2 * S].reshape(S, 2)
    assert [tuple(p) for p in pairs[:len(copies)].tolist()] == [tuple(p) for p in copies]
    if st.copies:
        assert (pairs[len(copies):] == -1).all()
    else:
        assert not copies
    tab = h[st.off["tab"]:].reshape(S, st.W)
    assert np.array_equal(tab, opg.table_array(ora.st, st.W).astype(np.int32))


def _check_pools(run, ora):
    assert np.array_equal(run.k_cache.cpu().numpy(), ora.K)
    assert np.array_equal(run.v_cache.cpu().numpy(), ora.V)


@pytest.mark.parametrize("layers", [1, 3])
def test_graph_replays_match_eager_and_the_oracle(layers):
    w = synthetic.config2(num_seqs=6, min_prompt=17, max_prompt=150, decode_steps=8, num_layers=layers)
    run, ora = _run(w), OracleSide(w)
    x = run.prepare(0)                         # the prefill step, eagerly
    run.run(x)
    s0, c0 = ora.reserve(0)
    ora.write(0, s0, c0)
    width = -(-(150 + 8) // 16)
    st = _static(run, width, partition_tokens=32)
    st.capture()
    for s in range(1, 9):
        st.set_activations(s)
        st.host_step(exact_lengths=True)
        st.replay()
        got = st.out.clone()
        torch.cuda.synchronize()
        _oracle_step(ora, s, st)
        _check_pools(run, ora)
        for layer in range(layers):
            assert_attn_close(got[layer].cpu().numpy(), ora.attend(s, layer=layer), False, f"step {s} layer {layer}")
        # the same step again from the prepared calls with the exact lengths: fp16 writes are
        # idempotent, so the pools stay the same and the outputs must be bit-identical
        st.launch()
        torch.cuda.synchronize()
        assert torch.equal(st.out, got), s
        _check_pools(run, ora)


def test_graph_with_copy_on_write():
    w = synthetic.config4(num_requests=6, prefix=32, min_suffix=1, max_suffix=40, beam_requests=3, beam_width=3,
                          decode_steps=4)
    run, ora = _run(w), OracleSide(w)
    width = max(len(run.mgr.blocks(i)) for i in run.ids) + 1
    st = _static(run, width, partition_tokens=16, copies=True)
    st.capture()
    n_copies = 0
    for s in range(4):
        st.set_activations(s)
        st.host_step()
        st.replay()
        torch.cuda.synchronize()
        n_copies += st.nc.value
        _oracle_step(ora, s, st)
        _check_pools(run, ora)
        assert_attn_close(st.out[0].cpu().numpy(), ora.attend(s), False, f"step {s}")
    assert n_copies > 0


def test_prepared_calls_without_graph():
    w = synthetic.config2(num_seqs=4, min_prompt=40, max_prompt=90, decode_steps=3, num_layers=2)
    run, ora = _run(w), OracleSide(w)
    x = run.prepare(0)
    run.run(x)
    s0, c0 = ora.reserve(0)
    ora.write(0, s0, c0)
    st = _static(run, -(-(90 + 3) // 16))
    for s in range(1, 4):
        st.set_activations(s)
        st.host_step()
        st.launch()
        torch.cuda.synchronize()
        _oracle_step(ora, s, st)
        _check_pools(run, ora)
        assert np.array_equal(st.lengths(), np.asarray(ora.st.lens, np.int32))
        for layer in range(2):
            assert_attn_close(st.out[layer].cpu().numpy(), ora.attend(s, layer=layer), False, f"step {s}")

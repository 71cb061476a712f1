"""Seeded random crossings of the features, each step against the CPU oracle.

Every case draws one combination of pool type (fp16, int8, bf16), head size,
GQA group (1 to 8 query heads per KV head; rows of several queries reach the
matrix-core path), layer count, sliding window, ragged lengths (block-edge
values and random ones), query rows (decode rows and chunks), split size and
dispatch threshold.  The
writes must match bit for bit, the attention within the pool type's
tolerance; with two layers the second layer is attended with the first
layer's plan.  The per-feature tests pin each feature alone; these catch
interactions between them.  A second family appends random runs of tokens
to int8 blocks in the states earlier writes leave, most of them keeping the
block's scale (only the new row is quantised) and some raising it (every
earlier code requantised), bit for bit against the oracle's replay.
"""
import numpy as np
import pytest
import torch

import synthetic
from tests.oracle_side import OracleSide, assert_attn_close, dev_np
from tests.test_gpu_parity import _check_step

HEADS = [(8, 8), (8, 4), (16, 4), (32, 8), (16, 2), (8, 1), (32, 4)]
EDGE_LENS = [1, 2, 15, 16, 17, 31, 33, 64, 100]
OPTS = [{}, {"partition_tokens": 16}, {"partition_tokens": 64}, {"partition_tokens": 256},
        {"partition_tokens": -1}, {"mfma_min_rows": 1}, {"mfma_min_rows": 2 ** 31 - 1}]


def draw_case(i: int):
    """The i-th case: everything the workload and the calls need, from one seeded generator."""
    rng = np.random.default_rng([4711, i])
    hq, hkv = HEADS[int(rng.integers(len(HEADS)))]
    d = int(rng.choice([64, 128]))
    dt = str(rng.choice(["f16", "i8", "bf16"]))
    layers = int(rng.choice([1, 1, 2]))
    n = int(rng.integers(1, 9))
    lens, qls = [], []
    for _ in range(n):
        L = int(rng.choice(EDGE_LENS)) if rng.random() < 0.5 else int(rng.integers(1, 2500))
        q = 1 if rng.random() < 0.6 else int(rng.integers(1, min(L, 80) + 1))
        lens.append(L)
        qls.append(q)
    window = 0 if rng.random() < 0.5 else int(rng.integers(1, 400))
    picks = rng.choice(len(OPTS), size=2, replace=False)
    opts = [OPTS[int(k)] for k in picks]
    return dict(seed=900 + i, hq=hq, hkv=hkv, d=d, dt=dt, layers=layers, lens=lens, qls=qls, window=window,
                opts=opts)


def test_draws_cover_the_features():   # host only: what the seeded draws contain
    cases = [draw_case(i) for i in range(48)]
    assert {c["dt"] for c in cases} == {"f16", "i8", "bf16"}
    assert {c["d"] for c in cases} == {64, 128}
    assert {c["layers"] for c in cases} == {1, 2}
    assert any(c["window"] for c in cases) and any(not c["window"] for c in cases)
    assert any(c["hq"] // c["hkv"] == 8 for c in cases) and any(c["hq"] == c["hkv"] for c in cases)
    assert any(max(c["qls"]) > 1 for c in cases)


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(48))
def test_random_case(i):
    from paged_kv_cache_47_amd.workload import DeviceRun
    c = draw_case(i)
    print(f"case {i}: {c}", flush=True)
    w = synthetic.custom(c["seed"], c["lens"], c["qls"], c["hq"], c["hkv"], c["d"], c["dt"], window=c["window"],
                         num_layers=c["layers"])
    run, ora = DeviceRun(w), OracleSide(w)
    x = _check_step(run, ora, 0, tuple(c["opts"]))
    if c["layers"] > 1:
        # the last call above left its plan in the run's workspace
        got = run.attend(x, layer=1, reuse_plan=True, **c["opts"][-1])
        torch.cuda.synchronize()
        assert_attn_close(dev_np(got), ora.attend(0, layer=1), w.kv_dtype, f"case {i} layer 1")


def draw_int8_writes(i: int):
    """Pools whose blocks hold the codes and scales earlier writes leave (each block's first o0
    tokens replayed through the oracle from N(0,1) rows), then one call's runs: per block a start
    offset and a run of consecutive slots, rows mostly small enough to keep the block's scale."""
    from oracle import kv_write as okv
    rng = np.random.default_rng([4712, i])
    hkv = int(rng.choice([1, 2, 8]))
    d = int(rng.choice([64, 128]))
    nb = 12
    K = rng.integers(-127, 128, (nb, hkv, 16, d)).astype(np.int8)   # filler past each block's tokens
    V = rng.integers(-127, 128, (nb, hkv, 16, d)).astype(np.int8)
    KS = np.zeros((nb, hkv), np.float16)
    VS = np.zeros((nb, hkv), np.float16)
    order = rng.permutation(nb)
    slots = []
    for b in order[: int(rng.integers(4, nb + 1))]:
        o0 = int(rng.integers(0, 16))
        for o in range(o0):   # the block's earlier tokens, written one at a time
            for h in range(hkv):
                K[b, h], KS[b, h] = okv.quant_append(K[b, h], KS[b, h], o, rng.standard_normal(d).astype(np.float16))
                V[b, h], VS[b, h] = okv.quant_append(V[b, h], VS[b, h], o, rng.standard_normal(d).astype(np.float16))
        n = int(rng.integers(1, 16 - o0 + 1))
        slots += [int(b) * 16 + o0 + j for j in range(n)]
    T = len(slots)
    sig = rng.choice([0.3, 0.3, 0.3, 1.0, 3.0], size=T)
    nk = (rng.standard_normal((T, hkv, d)) * sig[:, None, None]).astype(np.float16)
    nv = (rng.standard_normal((T, hkv, d)) * sig[:, None, None]).astype(np.float16)
    return K, V, KS, VS, nk, nv, np.asarray(slots, np.int32)


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(12))
def test_random_int8_writes(i):
    from oracle import kv_write as okv
    from paged_kv_cache_47_amd import pa
    K, V, KS, VS, nk, nv, slots = draw_int8_writes(i)
    print(f"int8 writes {i}: hkv {K.shape[1]} d {K.shape[3]} tokens {len(slots)}", flush=True)
    dev = [torch.from_numpy(a.copy()).cuda() for a in (K, V, KS, VS)]
    pa.pa_write_kv(torch.from_numpy(nk).cuda(), torch.from_numpy(nv).cuda(), torch.from_numpy(slots).cuda(),
                   dev[0], dev[1], dev[2], dev[3])
    eK, eV, eKS, eVS = okv.write_i8(K, V, KS, VS, nk, nv, slots, 16)
    torch.cuda.synchronize()
    gK, gV, gKS, gVS = (t.cpu().numpy() for t in dev)
    assert np.array_equal(gK, eK) and np.array_equal(gV, eV)
    assert np.array_equal(gKS.view(np.uint16), eKS.view(np.uint16))
    assert np.array_equal(gVS.view(np.uint16), eVS.view(np.uint16))

"""GPU edge cases through the C ABI, each against the CPU oracle.

Shapes and group sizes on both dispatch paths, sequences with no query rows,
empty batches, a single 32k-key sequence, poison in every slot no query may
read, int8 writes of special values and of runs crossing blocks, negative
slots, and block copies.
"""
import numpy as np
import pytest
import torch

import synthetic
from oracle import kv_write as okv
from tests.oracle_side import OracleSide, assert_attn_close
from tests.test_gpu_parity import SPLITS, _check_step

pytestmark = pytest.mark.gpu

LENS = [1, 2, 15, 16, 17, 33, 100, 257, 700, 90]
QLS = [1, 1, 1, 1, 2, 3, 16, 40, 1, 90]


def _run(w):
    from paged_kv_cache_47_amd.workload import DeviceRun
    return DeviceRun(w)


@pytest.mark.parametrize("hq,hkv,d,dt", [
    (8, 1, 128, "f16"), (16, 2, 128, "f16"), (8, 4, 64, "f16"), (4, 4, 128, "f16"),
    (4, 4, 64, "i8"), (16, 2, 64, "i8"), (8, 8, 128, "i8"), (32, 8, 128, "i8"),
    (16, 2, 128, "i8"),   # int8 groups of eight at head dim 128: K read four lanes per token row
])
def test_shapes_and_groups(hq, hkv, d, dt):
    w = synthetic.custom(101 + hq + d, LENS, QLS, hq, hkv, d, dt)
    _check_step(_run(w), OracleSide(w), 0, SPLITS + ({"mfma_min_rows": 1}, {"mfma_min_rows": 2 ** 31 - 1}))


def test_rows_at_the_mfma_threshold():
    # q_len * group = 15, 16, 17 rows; 64-row tiles with 1, 63, 64, 65 rows
    lens = [40, 40, 40, 80, 80, 80, 200]
    qls = [15, 16, 17, 1, 63, 64, 65]
    w = synthetic.custom(7, lens, qls, 4, 4, 128)
    _check_step(_run(w), OracleSide(w), 0, ({}, {"partition_tokens": 16}))


def test_rows_at_the_row_tile_edges():
    # q_len * group = 127, 128, 129, 255, 256, 257, 511, 513 rows: partial, full and spilling row tiles
    lens = [300, 300, 300, 600, 600, 600, 900, 900]
    qls = [127, 128, 129, 255, 256, 257, 511, 513]
    w = synthetic.custom(16, lens, qls, 2, 2, 64)
    _check_step(_run(w), OracleSide(w), 0, ({},))
    w = synthetic.custom(17, [1000, 700], [400, 65], 8, 2, 128, "i8")
    _check_step(_run(w), OracleSide(w), 0, ({},))


def test_zero_query_rows_and_empty_batch():
    from paged_kv_cache_47_amd import pa
    w = synthetic.custom(8, [5, 40, 1, 300, 17], [0, 1, 0, 20, 0], 8, 2, 128)
    _check_step(_run(w), OracleSide(w), 0, SPLITS)
    run = _run(synthetic.custom(9, [5], [1], 8, 2, 128))
    x = run.prepare(0)
    empty = torch.empty((0, 8, 128), dtype=torch.float16, device="cuda")
    none = torch.empty((0,), dtype=torch.int32, device="cuda")
    before = run.k_cache.clone()
    pa.pa_write_kv(torch.empty((0, 2, 128), dtype=torch.float16, device="cuda"),
                   torch.empty((0, 2, 128), dtype=torch.float16, device="cuda"), none, run.k_cache, run.v_cache)
    out = pa.pa_attend(empty, run.k_cache, run.v_cache, torch.zeros((0, 1), dtype=torch.int32, device="cuda"),
                       none, none, np.zeros(0, np.int32), np.zeros(0, np.int32), 0.1)
    torch.cuda.synchronize()
    assert out.shape == (0, 8, 128) and torch.equal(before, run.k_cache)


def test_single_long_sequence():
    w = synthetic.custom(10, [32768], [1], 32, 8, 128)
    _check_step(_run(w), OracleSide(w), 0, SPLITS)


def _poison_mask(run, w, L):
    """[NB, bs] True where no query may read: slots past each sequence's length
    in its blocks, and every block no table holds."""
    nb, bs = w.num_blocks, w.block_size
    mask = np.ones((nb, bs), bool)
    for sid, n in zip(run.ids, L):
        for j, b in enumerate(run.mgr.blocks(sid)):
            valid = min(bs, n - j * bs)
            mask[b, :valid] = False
    return torch.from_numpy(mask).cuda()


@pytest.mark.parametrize("dt", ["f16", "i8"])
def test_poison_in_unused_slots_changes_nothing(dt):
    lens = [1, 5, 16, 31, 100, 333, 64]
    qls = [1, 1, 1, 1, 30, 1, 64]
    w = synthetic.custom(11, lens, qls, 16, 4, 128, dt)
    run = _run(w)
    x = run.prepare(0)
    run.write(x)
    opts_list = SPLITS + ({"mfma_min_rows": 1},)
    clean = [run.attend(x, **o).clone() for o in opts_list]
    mask = _poison_mask(run, w, x.batch.seq_lens)
    m4 = mask[:, None, :, None].expand_as(run.k_cache)
    if dt == "f16":
        run.k_cache[m4] = float("nan")
        run.v_cache[m4] = float("nan")
    else:
        run.k_cache[m4] = 127
        run.v_cache[m4] = -127
        free = mask.all(dim=1)
        run.k_scale[free] = float("nan")
        run.v_scale[free] = float("inf")
    for o, ref in zip(opts_list, clean):
        got = run.attend(x, **o)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), o


def test_int8_write_special_values():
    lens = [20, 40, 16, 3, 48]
    qls = [20, 40, 1, 3, 33]          # runs that start at offset 0 and cross blocks, and one at offset 15
    w = synthetic.custom(12, lens, qls, 8, 2, 128, "i8")
    st = w.step(0)
    st.new_k[0:5] = 0                                   # a zero block: scale 0, codes 0
    st.new_k[20:24] = np.float16(65504)                 # largest fp16 (softmax saturates on these keys)
    st.new_k[60] = np.float16(2e-7)                     # amax / 127 rounds to a zero scale
    st.new_v[61, :, ::2] = np.float16(6e-5)             # subnormal scales
    st.new_k[62] = -st.new_k[62]
    _check_step(_run(w), OracleSide(w), 0, ({},))


def test_int8_values_near_the_fp16_limit():
    # V rows of +-60000 give block scales near the fp16 limit (60000 / 127 -> 472.5): the weight
    # times V scale products of both paths must stay finite; the new keys are aligned with their
    # queries so the decode rows also weight them heavily
    lens, qls = [120, 100, 90, 300], [40, 1, 1, 1]   # 160 rows on the MFMA path, three decode rows
    w = synthetic.custom(18, lens, qls, 8, 2, 128, "i8")
    st = w.step(0)
    st.new_v[:, :, 0::2] = np.float16(60000)
    st.new_v[:, :, 1::2] = np.float16(-60000)
    st.new_k[:] = (0.6 * st.q[:, ::4, :].astype(np.float32)).astype(np.float16)
    run, ora = _run(w), OracleSide(w)
    x = run.prepare(0)
    slots, copies = ora.reserve(0)
    run.write(x)
    ora.write(0, slots, copies)
    ref = ora.attend(0)
    for opts in ({}, {"partition_tokens": 32}, {"mfma_min_rows": 1}):
        got = run.attend(x, **opts).cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(got)), opts
        err = np.abs(got - ref)
        assert np.all(err <= np.maximum(5e-2, 1e-2 * np.abs(ref))), (opts, float((err / np.maximum(np.abs(ref), 1)).max()))


@pytest.mark.parametrize("d", [128, 64])
def test_int8_write_from_crafted_block_states(d):
    # Appends to blocks whose earlier codes and scale are set by hand, against the oracle's
    # per-token replay from the same state: a scale the new rows leave unchanged (only the new
    # rows are quantised), a largest code below 127 (the scale moves), a stray -128 code, zero,
    # negative and negative-zero scales, and a run that keeps the scale for some tokens only
    from paged_kv_cache_47_amd import pa
    rng = np.random.default_rng(41 + d)
    nb, hkv, bs = 7, 2, 16
    K = rng.integers(-127, 128, (nb, hkv, bs, d)).astype(np.int8)
    V = rng.integers(-127, 128, (nb, hkv, bs, d)).astype(np.int8)
    K[:, :, 0, 0] = 127
    V[:, :, 0, 1] = -127
    KS = np.full((nb, hkv), 0.02, np.float16)
    VS = np.full((nb, hkv), 0.03, np.float16)
    K[1] = np.clip(K[1], -100, 100)                    # largest code 100: the scale moves
    V[1] = np.clip(V[1], -100, 100)
    K[2, :, 1, 5] = -128                                # a code outside the written range
    V[2, :, 2, 7] = -128
    KS[3], VS[3] = 0, 0                                 # zero scale over nonzero codes
    KS[4], VS[4] = -0.02, -0.03                         # negative scales
    KS[5], VS[5] = np.float16(-0.0), np.float16(-0.0)
    # (block, first offset, tokens); blocks 0 and 6 get rows within the old range, block 6 then larger ones
    runs = [(0, 5, 3), (1, 8, 2), (2, 4, 1), (3, 6, 1), (4, 3, 2), (5, 2, 1), (6, 1, 6)]
    slots, nk, nv = [], [], []
    for b, o0, n in runs:
        for i in range(n):
            slots.append(b * bs + o0 + i)
            big = b == 6 and i >= 3
            nk.append((rng.standard_normal((hkv, d)) * (3.0 if big else 0.4)).clip(-2.5, 2.5) if not big
                      else rng.standard_normal((hkv, d)) * 3.0)
            nv.append((rng.standard_normal((hkv, d)) * 0.4).clip(-3.5, 3.5))
    nk = np.asarray(nk).astype(np.float16)
    nv = np.asarray(nv).astype(np.float16)
    nk[9] = 0                                           # block 5: a zero row gives a zero scale
    nv[9] = 0
    slots = np.asarray(slots, np.int32)
    dev = [torch.from_numpy(a.copy()).cuda() for a in (K, V, KS, VS)]
    pa.pa_write_kv(torch.from_numpy(nk).cuda(), torch.from_numpy(nv).cuda(), torch.from_numpy(slots).cuda(),
                   dev[0], dev[1], dev[2], dev[3])
    eK, eV, eKS, eVS = okv.write_i8(K, V, KS, VS, nk, nv, slots, bs)
    torch.cuda.synchronize()
    gK, gV, gKS, gVS = (t.cpu().numpy() for t in dev)
    assert np.array_equal(gK, eK) and np.array_equal(gV, eV)
    assert np.array_equal(gKS.view(np.uint16), eKS.view(np.uint16))
    assert np.array_equal(gVS.view(np.uint16), eVS.view(np.uint16))
    # the cases are what they claim to be
    assert eKS[0, 0] == KS[0, 0] and eKS[1, 0] != KS[1, 0] and eK[2, 0, 1, 5] == -127
    assert eKS[4, 0] == -KS[4, 0] and eKS[5, 0] == 0 and eKS[6, 0] != KS[6, 0]


@pytest.mark.parametrize("n,q2,hq,dt", [(100, False, 32, "f16"), (128, False, 32, "f16"), (129, False, 32, "f16"),
                                        (160, False, 32, "f16"), (100, True, 32, "f16"), (128, False, 64, "i8")])
def test_pure_decode_batches_with_and_without_the_plan(n, q2, hq, dt):
    # one query row per sequence, no split, at most 1024 (sequence, KV head) pairs: the decode kernel
    # reads the lengths itself (100 and 128 x 8; int8 group 8 takes the query-rows-in-LDS kernel); more
    # pairs (129 and 160 x 8) or a row with two queries go through the plan kernel; all against the
    # oracle, with a window on half of them.  The library's own plan query says which path each took.
    from paged_kv_cache_47_amd import pa
    rng = np.random.default_rng(5 + n + q2)
    lens = [int(x) for x in rng.integers(1, 600, n)]
    qls = [1] * n
    if q2:
        qls[7] = 2
        lens[7] = max(lens[7], 2)
    for window in (0, 100):
        w = synthetic.custom(70 + n, lens, qls, hq, 8, 128, dt, window=window)
        run = _run(w)
        for opts in ({}, {"partition_tokens": -1}):
            info = pa.pa_attend_plan_info(run.k_cache, hq, lens, qls, window=window, **opts)
            want = 0 if q2 else (1 if (n <= 128 and info["max_parts"] == 1) else 2)
            assert info["plan_free"] == want, (n, q2, opts, info)
        _check_step(run, OracleSide(w), 0, ({}, {"partition_tokens": -1}))


@pytest.mark.parametrize("n,hi,hq,hkv,dt,window", [
    (256, 6000, 32, 8, "f16", 0), (1024, 400, 32, 8, "f16", 0), (300, 3000, 64, 8, "i8", 0),
    (200, 5000, 16, 2, "bf16", 700), (97, 9000, 8, 8, "f16", 0), (130, 2000, 4, 4, "i8", 100),
])
def test_self_planned_decode_batches(n, hi, hq, hkv, dt, window):
    # pure-decode batches that split rows or exceed 1024 (sequence, KV head) pairs: no plan kernel,
    # every decode workgroup derives the bucketed unit order from the device lengths and takes its unit
    from paged_kv_cache_47_amd import pa
    rng = np.random.default_rng(900 + n + hi)
    lens = [int(x) for x in rng.integers(1, hi, n)]
    lens[n // 2] = hi                                       # the longest row sits mid-batch
    w = synthetic.custom(800 + n, lens, [1] * n, hq, hkv, 128, dt, window=window)
    run = _run(w)
    opts_list = ({}, {"partition_tokens": 16}, {"partition_tokens": 256}, {"partition_tokens": 4096},
                 {"partition_tokens": -1})
    for opts in opts_list:
        info = pa.pa_attend_plan_info(run.k_cache, hq, lens, [1] * n, window=window, **opts)
        assert info["plan_free"] == (1 if (info["max_parts"] == 1 and n * hkv <= 1024) else 2), (opts, info)
    _check_step(run, OracleSide(w), 0, opts_list)


def test_write_skips_negative_and_out_of_range_slots():
    from paged_kv_cache_47_amd import pa
    rng = np.random.default_rng(13)
    nb, hkv, d = 6, 2, 64
    K = rng.standard_normal((nb, hkv, 16, d)).astype(np.float16)
    V = rng.standard_normal((nb, hkv, 16, d)).astype(np.float16)
    nk = rng.standard_normal((5, hkv, d)).astype(np.float16)
    nv = rng.standard_normal((5, hkv, d)).astype(np.float16)
    slots = np.array([3, -1, 40, nb * 16, -7], np.int32)
    kc, vc = torch.from_numpy(K).cuda(), torch.from_numpy(V).cuda()
    pa.pa_write_kv(torch.from_numpy(nk).cuda(), torch.from_numpy(nv).cuda(), torch.from_numpy(slots).cuda(), kc, vc)
    eK, eV = okv.write_f16(K, V, nk, nv, [3, -1, 40, -1, -1], 16)
    torch.cuda.synchronize()
    assert np.array_equal(kc.cpu().numpy(), eK) and np.array_equal(vc.cpu().numpy(), eV)


@pytest.mark.parametrize("dt", ["f16", "i8"])
def test_copy_blocks(dt):
    from paged_kv_cache_47_amd import pa
    rng = np.random.default_rng(14)
    nb, hkv, d = 12, 4, 128
    if dt == "f16":
        K = rng.standard_normal((nb, hkv, 16, d)).astype(np.float16)
        V = rng.standard_normal((nb, hkv, 16, d)).astype(np.float16)
        KS = VS = None
    else:
        K = rng.integers(-127, 128, (nb, hkv, 16, d)).astype(np.int8)
        V = rng.integers(-127, 128, (nb, hkv, 16, d)).astype(np.int8)
        KS = rng.uniform(0.01, 0.05, (nb, hkv)).astype(np.float16)
        VS = rng.uniform(0.01, 0.05, (nb, hkv)).astype(np.float16)
    pairs = [(0, 5), (3, 7), (3, 8), (11, 1)]
    dev = [None if a is None else torch.from_numpy(a.copy()).cuda() for a in (K, V, KS, VS)]
    pa.pa_copy_blocks(dev[0], dev[1], torch.tensor(pairs, dtype=torch.int32, device="cuda"), dev[2], dev[3])
    okv.copy_blocks([K, V, KS, VS], pairs)
    torch.cuda.synchronize()
    for a, t in zip((K, V, KS, VS), dev):
        if a is not None:
            assert np.array_equal(t.cpu().numpy(), a)


def test_decode_of_length_one_is_v0():
    w = synthetic.custom(15, [1, 1, 1], [1, 1, 1], 8, 2, 128)
    run = _run(w)
    ora = OracleSide(w)
    x = run.prepare(0)
    run.write(x)
    out = run.attend(x).cpu().numpy()
    torch.cuda.synchronize()
    # the only key a query sees is its own token: the output is that token's V, exactly
    v = w.step(0).new_v
    assert np.array_equal(out, np.repeat(v, 4, axis=1))
    ora.reserve(0)


@pytest.mark.parametrize("hq", [8, 16, 32])
def test_int8_block_with_zero_key_scale(hq):
    # A block whose written K rows are all exactly zero gets a zero K scale ([engine] "INT8 KV
    # cache design": scale = max |x| / 127, zero codes).  Here each chosen sequence's new token
    # opens a block, so that block holds one visible key with a zero scale and 15 masked slots:
    # the masked scores must stay -inf (not -inf * 0) on the vector path, the eight-row quad layout
    # and the matrix-core decode alike, and the outputs must match the oracle.
    lens = [17, 33, 161, 49, 1, 400, 65, 2]
    w = synthetic.custom(77 + hq, lens, [1] * len(lens), hq, 2, 128, "i8")
    st = w.step(0)
    for i, L in enumerate(lens):
        if (L - 1) % 16 == 0:                 # the new token is the first of its block
            st.new_k[i] = 0
    run = _run(w)
    x = _check_step(run, OracleSide(w), 0, SPLITS + ({"mfma_min_rows": 1}, {"mfma_min_rows": 2 ** 31 - 1}))
    tab = x.batch.block_tables
    zero = [int(tab[i][(L - 1) // 16]) for i, L in enumerate(lens) if (L - 1) % 16 == 0]
    assert len(zero) == 6 and (run.k_scale[zero].float() == 0).all()

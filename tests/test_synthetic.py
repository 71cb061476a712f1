"""The seeded input generator (CPU): determinism and the bf16 rounding it
applies to its draws (checked against torch's own float32 -> bfloat16
conversion, round to nearest with ties to even)."""
import numpy as np
import torch

import synthetic
from synthetic.configs import normal_bf16, round_bf16


def test_round_bf16_matches_torch():
    rng = np.random.default_rng(3)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * np.float32(3.0),
        np.array([0.0, -0.0, 1.0, -1.0, 1e-38, -1e-38, 3.0e38, 65504.0], np.float32),
        # exact ties: the low 16 bits are 0x8000, so rounding goes to the even neighbour
        (np.arange(1, 2000, dtype=np.uint32) << 16 | np.uint32(0x8000)).view(np.float32),
    ])
    want = torch.from_numpy(x.copy()).to(torch.bfloat16).float().numpy()
    got = round_bf16(x)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_bf16_draws_are_bf16_and_deterministic():
    a = normal_bf16((5, 1), (3, 70000))
    b = normal_bf16((5, 1), (3, 70000))
    assert a.dtype == np.float32 and np.array_equal(a, b)
    assert np.all((a.view(np.uint32) & np.uint32(0xFFFF)) == 0)
    assert abs(float(a.mean())) < 0.02 and abs(float(a.std()) - 1.0) < 0.02


def test_layered_workload_shapes():
    w = synthetic.custom(9, [40, 20], [1, 3], 8, 2, 64, "bf16", num_layers=3)
    assert w.pool_k.shape == (w.num_blocks, 3, 2, 16, 64)
    assert w.step(0).q.shape == (3, 4, 8, 64)
    assert w.layer_acts(0, 2)[2].shape == (4, 8, 64)
    single = synthetic.custom(9, [40, 20], [1, 3], 8, 2, 64)
    assert single.pool_k.shape == (single.num_blocks, 2, 16, 64) and single.pool_k.dtype == np.float16

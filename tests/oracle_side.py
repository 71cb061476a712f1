"""Oracle side of a workload: the oracle's own tables, pools and expected
outputs, built from the same seeded draws as the device run (nothing taken
from the HIP path)."""
from __future__ import annotations

import numpy as np

from oracle import attention as oatt
from oracle import kv_write as okv
from oracle import paging as opg

# Tolerances stated for fp16 outputs (max-abs 2e-3; max-rel 1e-2, taken over
# elements whose reference magnitude is at least 0.2, below which the absolute
# bound is the tighter one) and for int8 KV (max-abs 5e-2).
ATOL_F16 = 2e-3
RTOL_F16 = 1e-2
REL_FLOOR = 0.2
ATOL_I8 = 5e-2


def assert_attn_close(got, ref, int8: bool, what: str = "") -> dict:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    diff = np.abs(got - ref)
    mx = float(diff.max()) if diff.size else 0.0
    if int8:
        assert mx <= ATOL_I8, f"{what}: max abs diff {mx} > {ATOL_I8}"
        return {"max_abs": mx}
    assert mx <= ATOL_F16, f"{what}: max abs diff {mx} > {ATOL_F16}"
    big = np.abs(ref) >= REL_FLOOR
    rel = float((diff[big] / np.abs(ref[big])).max()) if big.any() else 0.0
    assert rel <= RTOL_F16, f"{what}: max rel diff {rel} > {RTOL_F16}"
    return {"max_abs": mx, "max_rel": rel}


class OracleSide:
    def __init__(self, w, with_pools: bool = True, context_seqs=None):
        self.w = w
        self.st = opg.build_state(w)
        self.K = self.V = self.KS = self.VS = None
        if with_pools:
            self.K = w.pool_k.copy()
            self.V = w.pool_v.copy()
            if w.kv_dtype == "i8":
                self.KS = w.pool_k_scale.copy()
                self.VS = w.pool_v_scale.copy()
            if w.context is not None:
                seqs = range(len(self.st.tables)) if context_seqs is None else context_seqs
                for i in seqs:
                    c = int(w.ctx_lens[i])
                    if c:
                        ck, cv = w.context(i)
                        okv.fill_context_i8(self.K, self.V, self.KS, self.VS, self.st.tables[i], ck, cv,
                                            w.block_size)

    def reserve(self, s: int):
        """Reserve step ``s``'s positions: (slot_mapping, copies)."""
        return opg.apply_step(self.st, self.w.step(s).q_lens, self.w.window)

    def write(self, s: int, slots, copies) -> None:
        w = self.w
        step = w.step(s)
        okv.copy_blocks([self.K, self.V, self.KS, self.VS], copies)
        if w.kv_dtype == "i8":
            self.K, self.V, self.KS, self.VS = okv.write_i8(self.K, self.V, self.KS, self.VS, step.new_k,
                                                          step.new_v, slots, w.block_size)
        else:
            self.K, self.V = okv.write_f16(self.K, self.V, step.new_k, step.new_v, slots, w.block_size)

    def attend(self, s: int, seqs=None) -> np.ndarray:
        w = self.w
        step = w.step(s)
        return oatt.paged_attention(step.q, self.K, self.V, self.st.tables, self.st.lens, step.q_lens, w.scale,
                                    w.block_size, self.KS, self.VS, seqs=seqs, window=self.w.window)

    def row_ranges(self, s: int):
        q = np.asarray(self.w.step(s).q_lens)
        starts = np.concatenate([[0], np.cumsum(q)[:-1]])
        return starts, q

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
# bound is the tighter one) and for int8 KV (max-abs 5e-2).  bf16 ([pytorch]
# "Compute reference attention without hiding the layout" gives bf16 an
# absolute tolerance of 5e-3 against a float reference): 5e-3 plus one bf16
# unit in the last place of the reference (2^-7 relative), since the outputs
# themselves are stored in bf16.
ATOL_F16 = 2e-3
RTOL_F16 = 1e-2
REL_FLOOR = 0.2
ATOL_I8 = 5e-2
ATOL_BF16 = 5e-3
RTOL_BF16 = 2.0 ** -7


def dev_np(t):
    """A device tensor as numpy in the oracle's representation (bf16 as float32)."""
    import torch
    return (t.float() if t.dtype == torch.bfloat16 else t).cpu().numpy()


def same_bits(a, b) -> bool:
    """Bit-for-bit equality of two arrays of one dtype (float32 compared as words)."""
    a, b = np.asarray(a), np.asarray(b)
    if a.shape != b.shape or a.dtype != b.dtype:
        return False
    if a.dtype == np.float32:
        return np.array_equal(a.view(np.uint32), b.view(np.uint32))
    if a.dtype == np.float16:
        return np.array_equal(a.view(np.uint16), b.view(np.uint16))
    return np.array_equal(a, b)


def assert_attn_close(got, ref, kind, what: str = "") -> dict:
    """``kind``: the pool type ("f16", "bf16", "i8"; True / False stand for
    int8 / fp16)."""
    kind = "i8" if kind is True else ("f16" if kind is False else kind)
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    diff = np.abs(got - ref)
    mx = float(diff.max()) if diff.size else 0.0
    if kind == "i8":
        assert mx <= ATOL_I8, f"{what}: max abs diff {mx} > {ATOL_I8}"
        return {"max_abs": mx}
    if kind == "bf16":
        excess = float((diff - (ATOL_BF16 + RTOL_BF16 * np.abs(ref))).max()) if diff.size else -1.0
        assert excess <= 0, f"{what}: max abs diff {mx} exceeds 5e-3 + 2^-7 |ref| by {excess}"
        return {"max_abs": mx, "max_excess": excess}
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
                        for layer in range(w.num_layers):
                            K, V, KS, VS = self._layer(layer)
                            lk, lv = (ck, cv) if w.num_layers == 1 else (ck[layer], cv[layer])
                            okv.fill_context_i8(K, V, KS, VS, self.st.tables[i], lk, lv, w.block_size)

    def _layer(self, layer: int):
        """Views of one layer's pools and scales ([NB, Hkv, bs, D] / [NB, Hkv])."""
        if self.w.num_layers == 1:
            return self.K, self.V, self.KS, self.VS
        pick = (lambda a: None if a is None else a[:, layer])
        return pick(self.K), pick(self.V), pick(self.KS), pick(self.VS)

    def reserve(self, s: int):
        """Reserve step ``s``'s positions: (slot_mapping, copies)."""
        return opg.apply_step(self.st, self.w.step(s).q_lens, self.w.window)

    def write(self, s: int, slots, copies) -> None:
        w = self.w
        okv.copy_blocks([self.K, self.V, self.KS, self.VS], copies)   # whole blocks: every layer
        for layer in range(w.num_layers):
            nk, nv, _ = w.layer_acts(s, layer)
            K, V, KS, VS = self._layer(layer)
            if w.kv_dtype == "i8":
                K[...], V[...], KS[...], VS[...] = okv.write_i8(K, V, KS, VS, nk, nv, slots, w.block_size)
            else:
                K[...], V[...] = okv.write_f16(K, V, nk, nv, slots, w.block_size)

    def attend(self, s: int, seqs=None, layer: int = 0) -> np.ndarray:
        w = self.w
        step = w.step(s)
        K, V, KS, VS = self._layer(layer)
        return oatt.paged_attention(w.layer_acts(s, layer)[2], K, V, self.st.tables, self.st.lens, step.q_lens,
                                    w.scale, w.block_size, KS, VS, seqs=seqs, window=self.w.window)

    def row_ranges(self, s: int):
        q = np.asarray(self.w.step(s).q_lens)
        starts = np.concatenate([[0], np.cumsum(q)[:-1]])
        return starts, q

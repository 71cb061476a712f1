"""Resource use of the built gfx950 kernels, read from the library's own code
objects (no GPU needed): no kernel keeps registers or arrays in private
scratch memory, and the attention kernels spill no scalar registers either.

The library's device code sits in clang offload bundles (one per HIP source)
inside libpa.so; each gfx950 entry is an ELF whose AMDGPU metadata note
(msgpack) lists every kernel with its register counts, spill counts and
private segment size.
"""
import os
import re
import struct

import pytest

msgpack = pytest.importorskip("msgpack")

from paged_kv_cache_47_amd import _lib  # noqa: E402

NT_AMDGPU_METADATA = 32
BUNDLE_MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"

# kernels on the attention path: no scalar spills (each costs lane writes and reads every use)
HOT = ("decode_kernel", "decode_mfma_kernel", "prefill_kernel", "prefill_merge_kernel", "reduce_kernel",
       "write_f16_kernel")


def _gfx950_objects(blob: bytes):
    for m in re.finditer(re.escape(BUNDLE_MAGIC), blob):
        base = m.start()
        (n,) = struct.unpack_from("<Q", blob, base + 24)
        p = base + 32
        for _ in range(n):
            off, size, tlen = struct.unpack_from("<QQQ", blob, p)
            p += 24
            triple = blob[p:p + tlen].decode()
            p += tlen
            if "gfx950" in triple and size:
                yield blob[base + off:base + off + size]


def _metadata_notes(elf: bytes):
    assert elf[:4] == b"\x7fELF" and elf[4] == 2, "64-bit ELF code object expected"
    (shoff,) = struct.unpack_from("<Q", elf, 0x28)
    shentsize, shnum = struct.unpack_from("<HH", elf, 0x3A)
    for k in range(shnum):
        sh = shoff + k * shentsize
        if struct.unpack_from("<I", elf, sh + 4)[0] != 7:   # SHT_NOTE
            continue
        off, size = struct.unpack_from("<QQ", elf, sh + 0x18)
        p = off
        while p < off + size:
            nsz, dsz, ntype = struct.unpack_from("<III", elf, p)
            p += 12
            p += (nsz + 3) & ~3
            desc = elf[p:p + dsz]
            p += (dsz + 3) & ~3
            if ntype == NT_AMDGPU_METADATA:
                yield msgpack.unpackb(desc, raw=False)


def _kernels():
    path = _lib.LIB_PATH
    if not os.path.exists(path):
        pytest.skip("libpa.so is not built")
    with open(path, "rb") as f:
        blob = f.read()
    out = []
    for elf in _gfx950_objects(blob):
        for md in _metadata_notes(elf):
            out.extend(md["amdhsa.kernels"])
    return out


def test_no_private_scratch_and_no_vector_spills():
    ks = _kernels()
    assert len(ks) > 50, "expected the library's kernels in its gfx950 code objects"
    bad = [(k[".name"], k.get(".private_segment_fixed_size"), k.get(".vgpr_spill_count"))
           for k in ks if k.get(".private_segment_fixed_size", 0) or k.get(".vgpr_spill_count", 0)]
    assert not bad, f"kernels using private scratch or spilling vector registers: {bad}"


def test_attention_kernels_spill_no_scalar_registers():
    ks = _kernels()
    hot = [k for k in ks if any(h in k[".name"] for h in HOT)]
    assert hot, "no attention kernels found"
    bad = [(k[".name"], k.get(".sgpr_spill_count")) for k in hot if k.get(".sgpr_spill_count", 0)]
    assert not bad, f"attention kernels spilling scalar registers: {bad}"


def test_every_kernel_leaves_room_for_two_waves_per_simd():
    # 512 vector registers per lane per SIMD, shared by the waves on it; on gfx950 a kernel's
    # .vgpr_count is its unified total (architectural registers, then the accumulator ones from
    # accum_offset), so above 256 only one wave fits per SIMD
    ks = _kernels()
    bad = [(k[".name"], k.get(".vgpr_count"), k.get(".agpr_count")) for k in ks if k.get(".vgpr_count", 0) > 256]
    assert not bad, f"kernels above 256 vector registers (one wave per SIMD): {bad}"

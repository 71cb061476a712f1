"""The HBM-ceiling reads (pa_ceiling.h) on the GPU: they must read every
word they claim to read, and nothing else.  A lane writes the sink only when
the xor of the words it read equals a fixed constant, so a buffer of zeros
with that constant in one word shows whether that word was read."""
import pytest
import torch

from paged_kv_cache_47_amd import pa

pytestmark = pytest.mark.gpu

MAGIC = 0x9E3779B9


def _sink():
    return torch.zeros(1, dtype=torch.int32, device="cuda")


def _words(nbytes):
    return torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda")


def _as_i32(v):
    return v - (1 << 32) if v >= 1 << 31 else v


@pytest.mark.parametrize("nbytes,workgroups", [(16, 0), (4096, 1), (1 << 20, 1024), ((1 << 20) + 48, 3)])
def test_stream_read_reads_every_word(nbytes, workgroups):
    for word in sorted({0, nbytes // 16 // 2, nbytes // 16 - 1}):
        buf = _words(nbytes)
        buf[4 * word] = _as_i32(MAGIC)
        sink = _sink()
        print(f"stream read {nbytes} B, {workgroups} workgroups, marked word {word}", flush=True)
        pa.pa_ceiling_stream_read(buf, sink, workgroups=workgroups)
        torch.cuda.synchronize()
        assert int(sink.item()) & 0xFFFFFFFF == MAGIC
    sink = _sink()
    pa.pa_ceiling_stream_read(_words(nbytes), sink, workgroups=workgroups)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0


@pytest.mark.parametrize("depth", [1, 2])
@pytest.mark.parametrize("num_ids,per_wave", [(1, 16), (37, 16), (64, 5)])
def test_tile_gather_reads_the_listed_tiles_only(depth, num_ids, per_wave):
    num_tiles = 64
    g = torch.Generator().manual_seed(num_ids * 10 + depth)
    ids = torch.randperm(num_tiles, generator=g)[:num_ids].to(torch.int32)
    listed = set(ids.tolist())
    unlisted = [t for t in range(num_tiles) if t not in listed]
    cases = [("k", ids[-1].item(), True), ("v", ids[0].item(), True)]
    if unlisted:
        cases += [("k", unlisted[0], False), ("v", unlisted[-1], False)]
    for pool, tile, read in cases:
        k, v = _words(num_tiles * 4096), _words(num_tiles * 4096)
        (k if pool == "k" else v)[tile * 1024 + 1023] = _as_i32(MAGIC)   # the tile's last word
        sink = _sink()
        print(f"gather {num_ids} ids, {per_wave} per wave, depth {depth}: {pool} tile {tile}", flush=True)
        pa.pa_ceiling_gather(k, v, ids.cuda(), sink, ids_per_wave=per_wave, depth=depth)
        torch.cuda.synchronize()
        assert (int(sink.item()) & 0xFFFFFFFF == MAGIC) == read


def test_tile_gather_clamps_ids_to_tile_zero():
    k, v = _words(4 * 4096), _words(4 * 4096)
    k[5] = _as_i32(MAGIC)                      # a word of tile 0
    ids = torch.tensor([-1, 4, 1 << 30], dtype=torch.int32, device="cuda")
    sink = _sink()
    pa.pa_ceiling_gather(k, v, ids, sink, ids_per_wave=1, depth=2)
    torch.cuda.synchronize()
    assert int(sink.item()) & 0xFFFFFFFF == MAGIC

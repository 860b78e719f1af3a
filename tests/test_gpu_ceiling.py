"""pa_read_tiles, the read-only bandwidth probe: every tile's XOR of 32-bit words equals the
host's, bit for bit, for contiguous runs and for scattered tiles (ids out of range skipped)."""

import numpy as np
import pytest

from gpu_helpers import need_gpu, say
from paged_kv_cache_05_amd import ops

pytestmark = pytest.mark.gpu


def _xor_tiles(words, tile_bytes, ids):
    per = tile_bytes // 4
    tiles = words.reshape(-1, per)
    out = np.zeros(len(ids), np.uint32)
    for k, t in enumerate(ids):
        if 0 <= t < tiles.shape[0]:
            out[k] = np.bitwise_xor.reduce(tiles[t])
    return out


@pytest.mark.parametrize("tile_bytes", [1024, 2048, 4096, 8192])
def test_read_tiles_xor(tile_bytes):
    import torch
    dev = need_gpu()
    rng = np.random.default_rng(tile_bytes)
    ntiles = 203                                   # not a multiple of the 16 tiles per workgroup
    words = rng.integers(0, 2**32, size=ntiles * tile_bytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).to(dev)
    # contiguous run over the whole buffer
    out = torch.zeros(ntiles, dtype=torch.int32, device=dev)
    ops.read_tiles(buf, tile_bytes, out)
    # scattered tiles, repeats and ids outside the buffer
    ids = rng.permutation(ntiles)[:150].astype(np.int32)
    ids[[3, 40, 149]] = [-1, ntiles, 2**31 - 1]
    ids[7] = ids[8]
    out2 = torch.zeros(len(ids), dtype=torch.int32, device=dev)
    ops.read_tiles(buf, tile_bytes, out2, torch.from_numpy(ids).to(dev))
    torch.cuda.synchronize()
    say(f"read_tiles {tile_bytes} B: {ntiles} contiguous, {len(ids)} scattered")
    assert np.array_equal(out.cpu().numpy().view(np.uint32), _xor_tiles(words, tile_bytes, range(ntiles)))
    assert np.array_equal(out2.cpu().numpy().view(np.uint32), _xor_tiles(words, tile_bytes, ids))

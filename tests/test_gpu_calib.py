"""The bandwidth calibration calls (include/rss_calib.h) on the GPU: what they
read, copy and write, at sizes that are not a multiple of one grid pass."""
import numpy as np
import pytest
import torch

from gpu_util import DEV
from recurrent_state_storage_amd import rss

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nvec,blocks", [(1, 0), (1000, 3), (262147, 64)])
def test_calibration_read_copy_write(nvec, blocks):
    src = torch.randn((nvec, 4), device=DEV)
    keep = src.clone()
    sink = torch.zeros((4,), device=DEV)
    rss.rss_calib_read(src, sink, blocks)
    dst = torch.full_like(src, float("nan"))
    rss.rss_calib_copy(src, dst, blocks)
    torch.cuda.synchronize()
    assert torch.equal(src, keep) and torch.equal(dst, src)
    out = torch.full_like(src, float("nan"))
    rss.rss_calib_write(out, blocks)
    torch.cuda.synchronize()
    i = torch.arange(nvec, device=DEV)
    want = torch.stack([(i & 0xffffff).float(), torch.ones_like(i, dtype=torch.float32),
                        torch.full((nvec,), 2.0, device=DEV), torch.full((nvec,), 3.0, device=DEV)], dim=1)
    assert torch.equal(out, want)


@pytest.mark.parametrize("order", [0, 1])
@pytest.mark.parametrize("tile_bytes,n_tiles,write_bytes", [(32768, 37, 672), (4096, 9, 16), (65536, 5, 4096),
                                                            (8192, 3, 0), (32768, 300, 672), (65536, 77, 16),
                                                            (4096, 1100, 16)])
def test_calibration_tiles(tile_bytes, n_tiles, write_bytes, order):
    """Tile t's 16-byte vector i: (sum of thread i's floats, i, t, 1). The
    source holds small integers, so every fp32 sum is exact in any order. The
    larger cases span whole groups of the decode kernels' tile order (8 runs of
    up to 512 KiB) and a ragged tail, so every tile being served exactly once
    checks that order's workgroup-to-tile map."""
    L = tile_bytes // 4096
    g = np.random.default_rng(tile_bytes + n_tiles)
    host = g.integers(0, 8, size=(n_tiles, L, 256, 4)).astype(np.float32)
    src = torch.from_numpy(host).to(DEV)
    keep = src.clone()
    wv = write_bytes // 16
    dst = torch.full((max(n_tiles * wv, 1), 4), float("nan"), device=DEV)
    rss.rss_calib_tiles(src, tile_bytes, n_tiles, dst if write_bytes else None, write_bytes, order)
    torch.cuda.synchronize()
    assert torch.equal(src, keep)
    if not write_bytes:
        assert torch.isnan(dst).all()
        return
    sums = host.sum(axis=(1, 3))                      # (n_tiles, 256): thread i's floats of tile t
    want = np.zeros((n_tiles, wv, 4), np.float32)
    want[..., 0] = sums[:, :wv]
    want[..., 1] = np.arange(wv)[None, :]
    want[..., 2] = np.arange(n_tiles)[:, None]
    want[..., 3] = 1.0
    assert np.array_equal(dst.cpu().numpy().reshape(n_tiles, wv, 4), want)


@pytest.mark.parametrize("order", [0, 1])
@pytest.mark.parametrize("tile_bytes,n_tiles", [(32768, 37), (4096, 9), (65536, 5), (32768, 300), (16384, 531)])
def test_calibration_tile_copy(tile_bytes, n_tiles, order):
    """write_bytes = tile_bytes copies every tile to the same place in dst."""
    src = torch.randn((n_tiles * tile_bytes // 4,), device=DEV)
    keep = src.clone()
    dst = torch.full_like(src, float("nan"))
    rss.rss_calib_tiles(src, tile_bytes, n_tiles, dst, tile_bytes, order)
    torch.cuda.synchronize()
    assert torch.equal(src, keep) and torch.equal(dst, src)

"""The bandwidth calibration calls (include/rss_calib.h) on the GPU: what they
read, copy and write, at sizes that are not a multiple of one grid pass."""
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

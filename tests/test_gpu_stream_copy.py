"""GPU checks of the copy-kernel calibration (mrr_stream_copy): every byte
copied, tails shorter than one 16-byte vector, workgroups that walk several
tiles (MRR_MAX_GRID) and the persistent launch (MRR_LDS_CAP=0)."""
import pytest
import torch

import allreduce_reduction_nranks_amd as mrr
from gpu_common import announce

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [1, 15, 16, 17, 4096 + 9, 3 * 64 * 4 * 16 + 5, (64 << 20) + 13])
@pytest.mark.parametrize("mode", ["default", "walk", "persistent"])
def test_stream_copy_exact(nbytes, mode, mrr_env):
    announce("stream copy", nbytes, mode)
    g = torch.Generator().manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=g).cuda()
    dst = torch.full((nbytes + 32,), 0xA5, dtype=torch.uint8, device="cuda")
    if mode == "walk":
        mrr_env("MRR_MAX_GRID", "3")
    elif mode == "persistent":
        mrr_env("MRR_LDS_CAP", "0")
    assert mrr.mrr_stream_copy(src, dst, nbytes) == mrr.MRR_OK
    torch.cuda.synchronize()
    mrr_env("MRR_MAX_GRID", None)
    mrr_env("MRR_LDS_CAP", None)
    assert torch.equal(dst[:nbytes], src)
    assert torch.all(dst[nbytes:] == 0xA5), "wrote past the end"

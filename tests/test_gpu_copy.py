"""The bandwidth reference copy (mxq_copy16) copies every byte, for sizes
that leave a partial last round and for both store kinds."""
import pytest
import torch

import fp8_mx_activation_amd as mxq
from gpu_util import DEV, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 48, 4096 * 4 + 16, (1 << 20) + 48,
                                    64 << 20])
@pytest.mark.parametrize("nt", [0, 1, 2, 3])
def test_copy16_copies_every_byte(nbytes, nt):
    g = torch.Generator(device=DEV).manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device=DEV,
                        generator=g)
    dst = torch.full((nbytes,), 0xA5, dtype=torch.uint8, device=DEV)
    say("copy16", nbytes, nt)
    mxq.mxq_copy16(src, dst, nt)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)

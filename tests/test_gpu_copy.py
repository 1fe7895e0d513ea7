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


@pytest.mark.parametrize("R,W,G,K", [(300, 7168 * 2, 50, 8), (17, 48, 9, 3),
                                     (64, 40000, 5, 64)])
def test_gather_read16_reads_the_named_rows(R, W, G, K):
    """Every block's XOR word equals the XOR of the 32-bit words of the rows
    its indices name (indices outside [0, R) skipped); rows wider than one
    block's 16 KB pass take several passes."""
    import numpy as np
    rng = np.random.default_rng(R + W)
    rows_h = rng.integers(0, 2 ** 32, (R, W // 4), dtype=np.uint64).astype(
        np.uint32)
    idx_h = rng.integers(-3, R + 3, (G, K)).astype(np.int32)
    rows = torch.from_numpy(rows_h.view(np.int32)).to(DEV)
    idx = torch.from_numpy(idx_h).to(DEV)
    say("gather_read16", R, W, G, K)
    sink = mxq.mxq_gather_read16(rows, idx)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    want = np.zeros(G, np.uint32)
    for g in range(G):
        for d in idx_h[g]:
            if 0 <= d < R:
                want[g] ^= np.bitwise_xor.reduce(rows_h[d])
    assert np.array_equal(got, want)


def test_fill_rows16_writes_every_row_byte():
    dst = torch.zeros((37, 80), dtype=torch.int32, device=DEV)
    view = dst[:, :68]                      # row stride 320 B, 272 B written
    say("fill_rows16")
    mxq.mxq_fill_rows16(view, 0x5A5A1234)
    torch.cuda.synchronize()
    h = dst.cpu()
    assert (h[:, :68] == 0x5A5A1234).all() and (h[:, 68:] == 0).all()

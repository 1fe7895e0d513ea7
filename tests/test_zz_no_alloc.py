"""moe_layout_noalloc (the layout without a workspace argument, whose
per-chunk counts live in the library's static device array) against
moe_layout with a caller workspace, through the C ABI: every output must be
identical, over two calls in a row, the second with a smaller routing, so
stale counts left in the shared array by the first call cannot leak into the
second."""
import numpy as np
import pytest
import torch

import synthetic_inputs as si
from gpu_util import DEV, say

pytestmark = pytest.mark.gpu

KEYS = ("counts", "expert_offsets", "m_indices", "masked_m", "src2dst",
        "overflow_flag")


@pytest.fixture(scope="module")
def mxq():
    import fp8_mx_activation_amd as m
    m.lib()
    return m


def outputs(E, T, K, rows, fill):
    """Output buffers pre-filled with a canary, so a value the call does not
    write shows up."""
    shapes = dict(counts=(E,), expert_offsets=(E + 1,), m_indices=(rows,),
                  masked_m=(E,), src2dst=(T, K), overflow_flag=(1,))
    return {k: torch.full(s, fill, dtype=torch.int32, device=DEV)
            for k, s in shapes.items()}


def call_noalloc(mxq, ids, E, kind, block_e, cap, rows, o):
    T, K = ids.shape
    s = torch.cuda.current_stream().cuda_stream
    return mxq.lib().moe_layout_noalloc(
        ids.data_ptr(), T, K, 0, E, mxq.LAYOUT_KINDS[kind], block_e, cap,
        rows, *(o[k].data_ptr() for k in KEYS), s)


def call_with_workspace(mxq, ids, E, kind, block_e, cap, rows, o):
    T, K = ids.shape
    need = mxq.moe_layout_workspace_bytes(T, K, E)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=DEV)
    s = torch.cuda.current_stream().cuda_stream
    st = mxq.lib().moe_layout(
        ids.data_ptr(), T, K, 0, E, mxq.LAYOUT_KINDS[kind], block_e, cap,
        rows, *(o[k].data_ptr() for k in KEYS), ws.data_ptr(), ws.numel(), s)
    torch.cuda.synchronize()
    return st


CASES = (
    # (name, T, K, E, kind, cap): routings whose per-chunk counts go through
    # the shared array (more than 256 experts, or more than 2^17
    # assignments): first a prefill-sized one, then a smaller one that uses
    # fewer chunks of it, then a masked one
    ("prefill-zipf", 8192, 8, 384, "compact", 0),
    ("smaller-zipf", 1500, 8, 384, "compact", 0),
    ("masked-after", 20000, 8, 32, "masked", 1024),
)


def test_noalloc_matches_workspace_layout(mxq):
    rng = np.random.default_rng(si.SEEDS["prefill_compact"] + 17)
    for name, T, K, E, kind, cap in CASES:
        if kind == "compact":
            ids_h = si.zipf_topk(rng, T, E, K, n_zero=8)
            rows = mxq.moe_compact_row_bound(T * K, E, 128)
        else:
            ids_h = si.uniform_topk(rng, T, 256, K)
            rows = E * cap
        assert mxq.moe_layout_workspace_bytes(T, K, E) > 0   # uses scratch
        ids = torch.from_numpy(np.ascontiguousarray(ids_h, np.int32)).to(DEV)
        a = outputs(E, T, K, rows, -7)
        b = outputs(E, T, K, rows, -9)
        say("moe_layout (workspace)", name, T, K, E, kind)
        assert call_with_workspace(mxq, ids, E, kind, 128, cap, rows, a) == 0
        say("moe_layout_noalloc", name, T, K, E, kind)
        assert call_noalloc(mxq, ids, E, kind, 128, cap, rows, b) == 0
        torch.cuda.synchronize()
        for k in KEYS:
            got, want = b[k].cpu().numpy(), a[k].cpu().numpy()
            assert np.array_equal(got, want), (name, k)
        # the layout itself is right, not only equal: slots of every local
        # assignment are distinct rows holding their expert
        s2d = b["src2dst"].cpu().numpy()
        m = b["m_indices"].cpu().numpy()
        local = (ids_h >= 0) & (ids_h < E)
        d = s2d[local]
        assert len(np.unique(d)) == len(d)
        if kind == "compact":
            assert np.array_equal(m[d], ids_h[local])


def test_noalloc_single_launch_and_limit(mxq):
    """A routing small enough for one launch needs no scratch; one beyond the
    array's size is refused before anything is enqueued."""
    rng = np.random.default_rng(5)
    T, K, E = 200, 8, 64
    ids_h = si.uniform_topk(rng, T, E, K)
    ids = torch.from_numpy(np.ascontiguousarray(ids_h, np.int32)).to(DEV)
    rows = mxq.moe_compact_row_bound(T * K, E, 128)
    a = outputs(E, T, K, rows, -7)
    b = outputs(E, T, K, rows, -9)
    say("noalloc single-launch routing", T, K, E)
    assert call_with_workspace(mxq, ids, E, "compact", 128, 0, rows, a) == 0
    assert call_noalloc(mxq, ids, E, "compact", 128, 0, rows, b) == 0
    torch.cuda.synchronize()
    for k in KEYS:
        assert np.array_equal(b[k].cpu().numpy(), a[k].cpu().numpy()), k
    # 2^24 assignments over 1024 experts: 2048 chunks x 1024 counts (8 MiB)
    big_T, big_K, big_E = 1 << 21, 8, 1024
    assert mxq.moe_layout_workspace_bytes(big_T, big_K, big_E) > \
        mxq.LAYOUT_NOALLOC_SCRATCH_BYTES
    s = torch.cuda.current_stream().cuda_stream
    FAKE = 0x10000  # never dereferenced: the call returns before any launch
    st = mxq.lib().moe_layout_noalloc(
        FAKE, big_T, big_K, 0, big_E, 0, 128, 0,
        mxq.moe_compact_row_bound(big_T * big_K, big_E, 128),
        FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, s)
    assert st == mxq.MXQ_ERR_SCRATCH_LIMIT

"""Host-side checks of the Python binding that need no GPU: every wrapper
refuses host tensors before anything reaches the library (there is no CPU
path), and the shape helpers give the documented geometry."""
import os

import pytest
import torch


@pytest.fixture(scope="module")
def mxq():
    import fp8_mx_activation_amd as m
    if not os.path.exists(m.LIB_PATH):
        from fp8_mx_activation_amd import build
        build.build(verbose=False)
    return m


def test_wrappers_refuse_host_tensors(mxq):
    x = torch.zeros((4, 256), dtype=torch.bfloat16)
    ids = torch.zeros((4, 2), dtype=torch.int32)
    w = torch.zeros((4, 2), dtype=torch.float32)
    q = torch.zeros((4, 256), dtype=torch.uint8)
    sc = torch.ones((4, 2), dtype=torch.float32)
    calls = [
        lambda: mxq.moe_layout(ids, 0, 4),
        lambda: mxq.moe_scatter_quant(x, ids, 8),
        lambda: mxq.moe_scatter_quant_ex(x, ids, 8, rule="ocp_floor"),
        lambda: mxq.mx_quant_live_rows(x, 2, torch.zeros(2, dtype=torch.int32)),
        lambda: mxq.mx_quant_live_rows_ex(x, 2,
                                          torch.zeros(2, dtype=torch.int32)),
        lambda: mxq.requant_per_token_to_per_tensor(q, torch.ones(4)),
        lambda: mxq.moe_combine(x, ids, w),
        lambda: mxq.moe_scatter_rows(q, ids, 8),
        lambda: mxq.upscale_fp8_to_bf16(q, sc),
        lambda: mxq.requant_weight_block_ue8m0(
            torch.zeros((128, 128), dtype=torch.uint8), torch.ones((1, 1))),
        lambda: mxq.moe_m_indices_from_psum(torch.zeros(4, dtype=torch.int32),
                                            16, 16),
        lambda: mxq.moe_expand_to_masked_slab(
            q, torch.zeros(4, dtype=torch.int32), 16, 16),
        lambda: mxq.moe_masked_slab_to_expand(
            x, torch.zeros(4, dtype=torch.int32),
            torch.zeros(4, dtype=torch.int32), 16, 16, out_rows=8),
    ]
    for c in calls:
        with pytest.raises(ValueError, match="must be a GPU tensor"):
            c()


def test_packed_mn_scale_shape(mxq):
    """Four scale bytes per int32 word, rows contiguous, rows aligned to 4."""
    t = mxq.packed_mn_scales(98048, 56, "cpu")
    assert t.dtype == torch.int32 and tuple(t.shape) == (14, 98048)
    t = mxq.packed_mn_scales(5, 3, "cpu")
    assert tuple(t.shape) == (1, 8)
    t = mxq.packed_mn_scales(0, 224, "cpu")
    assert tuple(t.shape) == (56, 0)


def test_format_and_rule_tables(mxq):
    assert mxq.SCALE_FORMATS == {"ue8m0_g128": (0, 128), "e8m0_g32": (1, 32)}
    assert mxq.SCALE_RULES == {"no_clip": 0, "ocp_floor": 1}

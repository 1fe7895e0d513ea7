"""The declared limits, on the GPU against the oracle: 2^24 assignments with
1024 local experts, hidden 32768, top-64."""
import numpy as np
import pytest
import torch

import fp8_mx_activation_amd as mxq
import synthetic_inputs as si
from gpu_util import (CANARY, DEV, assert_equal, bf16_to_dev, bf16_to_host,
                      f32_to_dev, host, i32_to_dev, say)

pytestmark = pytest.mark.gpu


def test_layout_at_max_assignments(ora):
    """T*K = 2^24 (the most a layout takes) over 1024 local experts, skewed
    routing: counts, offsets, src2dst and m_indices compared in full."""
    T, K, E = 1 << 21, 8, 1024
    rng = np.random.default_rng(24)
    ids = si.strided_topk(rng, T, E, K)
    assert T * K == 1 << 24
    assert (np.sort(ids, axis=1)[:, 1:] != np.sort(ids, axis=1)[:, :-1]).all()
    say("layout max", T, K, E)
    lay = mxq.moe_layout(i32_to_dev(ids), 0, E, "compact")
    torch.cuda.synchronize()
    ref = ora.moe_layout(ids, 0, E, "compact")
    assert lay["num_rows"] == ref["num_rows"]
    for k in ("counts", "expert_offsets", "src2dst", "m_indices"):
        assert_equal(host(lay[k]), ref[k], k)


@pytest.mark.parametrize("G", [128, 32])
def test_scatter_and_combine_at_max_hidden(ora, G):
    """Hidden 32768 (the largest row the scatter stages in LDS) for both
    group sizes, and the combine at the same width."""
    H, T, K, E = 32768, 40, 4, 16
    rng = np.random.default_rng(G)
    x = si.gaussian_bf16(rng, (T, H))
    ids = si.uniform_topk(rng, T, E, K)
    w = si.softmax_weights(rng, T, K)
    ref = ora.moe_layout(ids, 0, E, "compact", block_e=8)
    R = ref["num_rows"]
    say("max hidden", H, G, R)
    lay = mxq.moe_layout(i32_to_dev(ids), 0, E, "compact", block_e=8,
                         num_rows=R)
    q = torch.full((R, H), CANARY, dtype=torch.uint8, device=DEV)
    s = torch.full((R, H // G), CANARY, dtype=torch.uint8, device=DEV)
    fmt = "ue8m0_g128" if G == 128 else "e8m0_g32"
    mxq.moe_scatter_quant(bf16_to_dev(x), lay["src2dst"], R, fmt, q=q,
                          scales=s)
    torch.cuda.synchronize()
    q_ref = np.full((R, H), CANARY, np.uint8)
    s_ref = np.full((R, H // G), CANARY, np.uint8)
    ora.scatter_quant(x, ref["src2dst"], G, R, q_ref, s_ref)
    assert_equal(host(q), q_ref, "fp8 bytes")
    assert_equal(host(s), s_ref, "scales")
    y = si.gaussian_bf16(rng, (R, H))
    out = mxq.moe_combine(bf16_to_dev(y), lay["src2dst"], f32_to_dev(w))
    torch.cuda.synchronize()
    assert_equal(bf16_to_host(out), ora.combine(y, ref["src2dst"], w),
                 "combine")


def test_top64_masked_at_capacity(ora):
    """K = 64 (the largest top-k) with 64 local experts and a masked slab of
    capacity T: every token reaches every expert, so each count equals the
    capacity exactly and nothing overflows."""
    T, K, E, H = 48, 64, 64, 256
    rng = np.random.default_rng(64)
    ids = np.stack([rng.permutation(E) for _ in range(T)]).astype(np.int32)
    x = si.gaussian_bf16(rng, (T, H))
    w = si.softmax_weights(rng, T, K)
    ref = ora.moe_layout(ids, 0, E, "masked", capacity=T)
    assert ref["overflow"] == 0 and (ref["masked_m"] == T).all()
    say("top64", T, K, E)
    lay = mxq.moe_layout(i32_to_dev(ids), 0, E, "masked", capacity=T)
    q, s = mxq.moe_scatter_quant(bf16_to_dev(x), lay["src2dst"], E * T)
    torch.cuda.synchronize()
    assert mxq.moe_read_overflow(lay["overflow_flag"]) == 0
    assert_equal(host(lay["src2dst"]), ref["src2dst"], "src2dst")
    q_ref, s_ref = ora.scatter_quant(x, ref["src2dst"], 128, E * T)
    assert_equal(host(q), q_ref, "fp8 bytes")
    assert_equal(host(s), s_ref, "scales")
    y = si.gaussian_bf16(rng, (E * T, H))
    out = mxq.moe_combine(bf16_to_dev(y), lay["src2dst"], f32_to_dev(w))
    torch.cuda.synchronize()
    assert_equal(bf16_to_host(out), ora.combine(y, ref["src2dst"], w),
                 "combine")

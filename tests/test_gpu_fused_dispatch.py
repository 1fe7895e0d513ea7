"""moe_layout_scatter_quant (layout and scatter+quant in one launch) on the
GPU against the oracle's layout followed by its scatter: every layout output
and every fp8 and scale byte bit-exact, rows that are no destination keep
their canary; the same outputs as the two GPU calls."""
import numpy as np
import pytest
import torch

import fp8_mx_activation_amd as mxq
import synthetic_inputs as si
from gpu_util import (CANARY, DEV, assert_equal, bf16_to_dev, host,
                      i32_to_dev, say)

pytestmark = pytest.mark.gpu

FMT = {128: "ue8m0_g128", 32: "e8m0_g32"}


def fused_case(ora, x_bits, ids, begin, E, kind, G, cap=0, block_e=128,
               num_rows=None, m_indices=True):
    T, H = x_bits.shape
    ref = ora.moe_layout(ids, begin, E, kind, block_e=block_e, capacity=cap,
                         num_rows=num_rows)
    R = ref["num_rows"]
    say("fused layout+scatter", kind, "T=%d K=%d E=%d H=%d G=%d rows=%d"
        % (T, ids.shape[1], E, H, G, R))
    q = torch.full((R, H), CANARY, dtype=torch.uint8, device=DEV)
    s = torch.full((R, H // G), CANARY, dtype=torch.uint8, device=DEV)
    lay, _, _ = mxq.moe_layout_scatter_quant(
        i32_to_dev(ids), bf16_to_dev(x_bits), begin, E, kind,
        block_e=block_e, capacity=cap, num_rows=R, fmt=FMT[G],
        m_indices=m_indices, q=q, scales=s)
    torch.cuda.synchronize()
    for key in ("counts", "expert_offsets", "masked_m", "src2dst"):
        assert_equal(host(lay[key]), ref[key], key)
    if m_indices:
        assert_equal(host(lay["m_indices"]), ref["m_indices"], "m_indices")
    assert int(host(lay["overflow_flag"])[0]) == ref["overflow"]
    q_ref = np.full((R, H), CANARY, np.uint8)
    s_ref = np.full((R, H // G), CANARY, np.uint8)
    ora.scatter_quant(x_bits, ref["src2dst"], G, R, q_ref, s_ref)
    assert_equal(host(q), q_ref, "fp8 bytes")
    assert_equal(host(s), s_ref, "scale bytes")
    return lay, q, s


def test_decode_masked(ora):
    b = si.decode_masked()
    fused_case(ora, b.x, b.topk_ids, 0, 32, "masked", 128, cap=128)


def test_decode_masked_g32_second_window(ora):
    """Experts [32, 64) of the same routing: a different set of tokens is
    local, the rest have no destination."""
    b = si.decode_masked()
    fused_case(ora, b.x, b.topk_ids, 32, 32, "masked", 32, cap=128)


def test_tiny_compact(ora):
    b = si.tiny()
    fused_case(ora, b.x, b.topk_ids, 0, 8, "compact", 128)


def test_largest_routing_compact_and_masked(ora):
    """4096 assignments (512 tokens of top-8 over 256 experts), the most
    the fused launch takes; each thread loads several of the ids."""
    rng = np.random.default_rng(31)
    T, K, H = 512, 8, 1024
    x = si.gaussian_bf16(rng, (T, H))
    ids = si.uniform_topk(rng, T, 256, K)
    fused_case(ora, x, ids, 0, 256, "compact", 128)
    fused_case(ora, x, ids, 64, 64, "masked", 32, cap=64)


def test_overflow_duplicates_and_k1(ora):
    """A hot expert over the slab capacity (slots past it dropped, flag
    set), repeated experts within a token (each its own row), and K = 1."""
    rng = np.random.default_rng(32)
    T, H = 200, 256
    x = si.gaussian_bf16(rng, (T, H))
    ids = rng.integers(0, 6, size=(T, 4)).astype(np.int32)
    ids[:, 0] = 2                                 # expert 2: 200+ assignments
    lay, _, _ = fused_case(ora, x, ids, 0, 6, "masked", 128, cap=64)
    assert mxq.moe_read_overflow(lay["overflow_flag"]) == 1
    fused_case(ora, x, ids, 0, 6, "compact", 32, block_e=32)
    fused_case(ora, x, ids[:, :1].copy(), 0, 6, "compact", 128)


def test_many_experts_wide_rows_and_extra_rows(ora):
    """1024 local experts (LDS tables at their largest) with and without
    m_indices and with a num_rows above the bound; hidden 32768 (four row
    chunks per lane) over 16 experts."""
    rng = np.random.default_rng(33)
    T, K = 64, 8
    ids = si.uniform_topk(rng, T, 1024, K)
    x = si.gaussian_bf16(rng, (T, 96))            # 3 groups of 32
    fused_case(ora, x, ids, 0, 1024, "compact", 32)
    bound = mxq.moe_compact_row_bound(T * K, 1024, 128)
    fused_case(ora, x, ids, 0, 1024, "compact", 32, num_rows=bound + 300,
               m_indices=False)
    ids16 = si.uniform_topk(rng, T, 16, K)
    xw = si.gaussian_bf16(rng, (T, 32768))
    fused_case(ora, xw, ids16, 0, 16, "compact", 128)


def test_block_size_boundary(ora):
    """512 local experts (the last count a 512-thread block scans) and 513
    (the first on 1024 threads), with rows wider than one pass of either
    block, and local ids spread over the whole window."""
    rng = np.random.default_rng(34)
    T, K, H = 40, 8, 17408
    x = si.gaussian_bf16(rng, (T, H))
    ids = si.uniform_topk(rng, T, 1024, K)
    for E in (512, 513):
        fused_case(ora, x, ids, 0, E, "compact", 128)
        fused_case(ora, x, ids, 511, E, "masked", 32, cap=2)


def test_many_experts_and_many_ids_per_thread(ora):
    """700 local experts (1024-thread blocks) with 3200 assignments, so each
    thread loads four ids of the routing; the layout alone takes the same
    block shape (one block per token) and is compared too."""
    rng = np.random.default_rng(36)
    T, K, H = 400, 8, 512
    x = si.gaussian_bf16(rng, (T, H))
    ids = si.uniform_topk(rng, T, 800, K)
    fused_case(ora, x, ids, 50, 700, "compact", 32)
    fused_case(ora, x, ids, 0, 700, "masked", 128, cap=6)
    ref = ora.moe_layout(ids, 50, 700, "compact")
    lay = mxq.moe_layout(i32_to_dev(ids), 50, 700, "compact")
    torch.cuda.synchronize()
    for key in ("counts", "expert_offsets", "masked_m", "src2dst",
                "m_indices"):
        assert_equal(host(lay[key]), ref[key], "layout " + key)


def test_same_as_two_calls_and_limits():
    """Byte-identical to moe_layout + moe_scatter_quant on the GPU; more than
    4096 assignments is refused; T = 0 gives the empty layout."""
    b = si.decode_masked()
    ids = i32_to_dev(b.topk_ids)
    x = bf16_to_dev(b.x)
    lay2 = mxq.moe_layout(ids, 0, 32, "masked", capacity=128)
    q2 = torch.zeros((32 * 128, b.H), dtype=torch.uint8, device=DEV)
    s2 = torch.zeros((32 * 128, b.H // 128), dtype=torch.uint8, device=DEV)
    mxq.moe_scatter_quant(x, lay2["src2dst"], 32 * 128, q=q2, scales=s2)
    q1 = torch.zeros_like(q2)
    s1 = torch.zeros_like(s2)
    lay1, _, _ = mxq.moe_layout_scatter_quant(ids, x, 0, 32, "masked",
                                              capacity=128, q=q1, scales=s1)
    torch.cuda.synchronize()
    for key in ("counts", "expert_offsets", "masked_m", "src2dst",
                "m_indices", "overflow_flag"):
        assert torch.equal(lay1[key], lay2[key]), key
    assert torch.equal(q1, q2) and torch.equal(s1, s2)

    big = torch.zeros((513, 8), dtype=torch.int32, device=DEV)
    xb = torch.zeros((513, 128), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(mxq.MxqError, match="unsupported"):
        mxq.moe_layout_scatter_quant(big, xb, 0, 32, "masked", capacity=128)

    empty = torch.zeros((0, 8), dtype=torch.int32, device=DEV)
    x0 = torch.zeros((0, 128), dtype=torch.bfloat16, device=DEV)
    lay0, _, _ = mxq.moe_layout_scatter_quant(empty, x0, 0, 4, "compact")
    torch.cuda.synchronize()
    assert (host(lay0["counts"]) == 0).all()
    assert (host(lay0["m_indices"]) == -1).all()


def test_graph_replay(ora):
    """Captured once in a hipGraph and replayed three times with new
    routings and rows (some ids non-local, one routing over the slab
    capacity); every replay checked against the oracle, with eager work and
    synchronizations between the replays."""
    T, K, E, H, cap = 96, 8, 16, 512, 64
    R = E * cap
    ids_s = torch.zeros((T, K), dtype=torch.int32, device=DEV)
    x_s = torch.zeros((T, H), dtype=torch.bfloat16, device=DEV)
    out = {k: torch.empty(shape, dtype=torch.int32, device=DEV)
           for k, shape in (("counts", (E,)), ("expert_offsets", (E + 1,)),
                            ("m_indices", (R,)), ("masked_m", (E,)),
                            ("src2dst", (T, K)), ("overflow_flag", (1,)))}
    q_s = torch.empty((R, H), dtype=torch.uint8, device=DEV)
    s_s = torch.empty((R, H // 128), dtype=torch.uint8, device=DEV)

    def step():
        mxq.moe_layout_scatter_quant(ids_s, x_s, 0, E, "masked", capacity=cap,
                                     out=out, q=q_s, scales=s_s)

    say("fused graph: warm-up on a side stream")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    say("fused graph: capture")
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        rng = np.random.default_rng(5000 + rep)
        ids = si.uniform_topk(rng, T, 24, K)
        if rep == 1:
            ids[:, 0] = 3                         # 96 assignments, cap 64
        x = si.gaussian_bf16(rng, (T, H))
        ids_s.copy_(i32_to_dev(ids))
        x_s.copy_(bf16_to_dev(x))
        q_s.fill_(CANARY)
        s_s.fill_(CANARY)
        torch.cuda.synchronize()
        say("fused graph: replay %d" % rep)
        g.replay()
        torch.cuda.synchronize()
        ref = ora.moe_layout(ids, 0, E, "masked", capacity=cap)
        for key in ("counts", "expert_offsets", "masked_m", "src2dst",
                    "m_indices"):
            assert_equal(host(out[key]), ref[key], "%s replay %d" % (key, rep))
        assert int(host(out["overflow_flag"])[0]) == ref["overflow"]
        assert ref["overflow"] == (1 if rep == 1 else 0)
        q_ref = np.full((R, H), CANARY, np.uint8)
        s_ref = np.full((R, H // 128), CANARY, np.uint8)
        ora.scatter_quant(x, ref["src2dst"], 128, R, q_ref, s_ref)
        assert_equal(host(q_s), q_ref, "fp8 bytes replay %d" % rep)
        assert_equal(host(s_s), s_ref, "scale bytes replay %d" % rep)

"""moe_layout on the GPU against the oracle: counts, region starts, src2dst,
m_indices, masked_m and the overflow flag must match exactly."""
import numpy as np
import pytest

import fp8_mx_activation_amd as mxq
import synthetic_inputs as si
from gpu_util import assert_equal, host, i32_to_dev, say

pytestmark = pytest.mark.gpu


def run_both(ora, ids, begin, E, kind, block_e=128, cap=0, num_rows=None,
             m_indices=True):
    ids = np.ascontiguousarray(ids, np.int32)
    ref = ora.moe_layout(ids, begin, E, kind, block_e=block_e, capacity=cap,
                         num_rows=num_rows)
    say("layout", kind, "T=%d K=%d E=%d begin=%d block=%d cap=%d rows=%d"
        % (ids.shape[0], ids.shape[1], E, begin, block_e, cap,
           ref["num_rows"]))
    got = mxq.moe_layout(i32_to_dev(ids), begin, E, kind, block_e=block_e,
                         capacity=cap, num_rows=ref["num_rows"],
                         m_indices=m_indices)
    assert_equal(host(got["counts"]), ref["counts"], "counts")
    assert_equal(host(got["expert_offsets"]), ref["expert_offsets"],
                 "expert_offsets")
    assert_equal(host(got["src2dst"]), ref["src2dst"], "src2dst")
    if m_indices:
        assert_equal(host(got["m_indices"]), ref["m_indices"], "m_indices")
    assert_equal(host(got["masked_m"]), ref["masked_m"], "masked_m")
    assert mxq.moe_read_overflow(got["overflow_flag"]) == ref["overflow"]
    return got, ref


def test_tiny(ora):
    b = si.tiny()
    run_both(ora, b.topk_ids, 0, 8, "compact")


def test_decode_masked(ora):
    b = si.decode_masked()
    got, ref = run_both(ora, b.topk_ids, 0, 32, "masked", cap=128)
    assert ref["overflow"] == 0


def test_decode_as_compact(ora):
    b = si.decode_masked()
    run_both(ora, b.topk_ids, 0, 32, "compact")


def test_prefill_compact_full(ora):
    b = si.prefill_compact(H=128)   # routing only; H does not matter here
    got, ref = run_both(ora, b.topk_ids, 0, 256, "compact")
    assert ref["num_rows"] == 98048
    assert (ref["counts"] == 0).any()          # Zipf tail leaves experts empty


def test_large_combine_routing(ora):
    ids, _ = si.large_combine_routing()
    got, ref = run_both(ora, ids, 0, 128, "compact")
    assert ref["num_rows"] == 147328


def test_expert_window_and_nonlocal(ora):
    rng = np.random.default_rng(1)
    ids = si.uniform_topk(rng, 500, 256, 8)
    run_both(ora, ids, 64, 32, "compact")
    run_both(ora, ids, 224, 32, "masked", cap=64)
    run_both(ora, np.full((33, 3), 999, np.int32), 0, 16, "compact")


def test_masked_overflow_flag(ora):
    T, cap = 300, 128
    ids = np.zeros((T, 2), np.int32)
    ids[:, 0] = 5
    ids[:, 1] = np.arange(T) % 7 + 8
    got, ref = run_both(ora, ids, 0, 16, "masked", cap=cap)
    assert ref["overflow"] == 1


@pytest.mark.parametrize("seed", range(4))
def test_random_shapes(ora, seed):
    rng = np.random.default_rng(100 + seed)
    E = int(rng.choice([1, 2, 3, 17, 64, 255, 256, 1000, 1024]))
    K = int(rng.integers(1, min(E, 12) + 1))
    T = int(rng.choice([1, 7, 64, 65, 513, 4099]))
    block = int(rng.choice([1, 3, 64, 128]))
    ids = si.uniform_topk(rng, T, E, K)
    run_both(ora, ids, 0, E, "compact", block_e=block)
    run_both(ora, ids, 0, E, "masked", cap=int(rng.integers(1, 40)))


def test_ragged_adjacent_experts(ora):
    counts = [127, 129, 1, 255, 256, 0, 2, 128]
    ids = np.concatenate([np.full(c, e) for e, c in enumerate(counts)])
    ids = np.random.default_rng(0).permutation(ids).reshape(-1, 1)
    run_both(ora, ids, 0, len(counts), "compact")


def test_spare_rows_and_no_m_indices(ora):
    b = si.tiny()
    run_both(ora, b.topk_ids, 0, 8, "compact", num_rows=1024 + 300)
    run_both(ora, b.topk_ids, 0, 8, "masked", cap=20, num_rows=8 * 20 + 5)
    run_both(ora, b.topk_ids, 0, 8, "compact", m_indices=False)


def test_empty_batch(ora):
    ids = np.zeros((0, 8), np.int32)
    got, ref = run_both(ora, ids, 0, 256, "compact")
    got, ref = run_both(ora, ids, 0, 32, "masked", cap=128)
    assert (host(got["m_indices"]) == -1).all()


@pytest.mark.parametrize("T,K,E", [(512, 8, 1024), (513, 8, 1024),
                                   (341, 12, 300), (342, 12, 300),
                                   (129, 8, 256), (4096, 1, 7), (4097, 1, 7),
                                   (128, 8, 32)])
def test_single_launch_boundary(ora, T, K, E):
    """Around T*K = 4096, where one launch with every block ranking the
    whole routing gives way to the slot kernel over chunks: 4096, 4092, 1032
    and 1024 take the single launch; 4104 (1024 experts) and 4104 (300
    experts) the histogram + slots pair, 4097 over 7 experts the slot kernel
    counting the routing in every block; masked capacity small enough to
    overflow."""
    rng = np.random.default_rng(T * K + E)
    ids = si.zipf_topk(rng, T, E, K) if E >= 2 * K else si.uniform_topk(
        rng, T, E, K)
    run_both(ora, ids, 0, E, "compact")
    run_both(ora, ids, 0, E, "compact", block_e=1)
    got, ref = run_both(ora, ids, 0, E, "masked", cap=max(1, T * K // E // 2))


@pytest.mark.parametrize("T,K,E", [(2048, 2, 256), (2049, 1, 256),
                                   (1024, 4, 300), (1025, 3, 300),
                                   (1, 64, 1024), (1, 1, 1), (7, 64, 64)])
def test_per_token_boundary(ora, T, K, E):
    """Around the switch from one block per token (up to 2048 tokens with at
    most 256 experts, up to 1024 with more) to one block ranking the whole
    routing, at most 4096 assignments: 2048 x 2 and 1024 x 4 over 300
    experts take a block per token, 2049 x 1 and 1025 x 3 over 300 the
    single ranking block; one token with 64 assignments; duplicates of an
    expert inside one token (7 x 64 over 64 experts)."""
    rng = np.random.default_rng(T * 131 + K * 7 + E)
    ids = si.zipf_topk(rng, T, E, K) if E >= 2 * K else si.uniform_topk(
        rng, T, E, K)
    if T == 7:
        ids[:, 1::2] = ids[:, 0:1]  # the same expert in half of a token
    run_both(ora, ids, 0, E, "compact")
    run_both(ora, ids, 0, E, "compact", block_e=1)
    run_both(ora, ids, 0, E, "masked", cap=max(1, T * K // E // 2))


@pytest.mark.parametrize("T,K,E", [(4097, 1, 256), (4097, 1, 257),
                                   (2048, 8, 256), (2049, 8, 256),
                                   (2048, 8, 128), (1024, 8, 32),
                                   (8192, 2, 1), (1024, 8, 300)])
def test_counted_in_block_boundary(ora, T, K, E):
    """Where every block of the slot kernel counts the whole routing itself
    (4096 < T*K <= 2^14, at most 256 experts) against where the histogram
    launch counts it: 4097 and 16384 assignments over 256 experts, 16384
    over 128 and 1 and 8192 over 32 take the in-block count; 257 and 300
    experts and 16392 assignments the histogram; compact, one-row blocks
    and masked (with overflow) for each.  An expert window puts part of the
    ids out of range."""
    rng = np.random.default_rng(T * K + E + 7)
    ids = si.zipf_topk(rng, T, E + 16, K, n_zero=4) if E + 16 >= 2 * K \
        else si.uniform_topk(rng, T, E + 16, K)
    run_both(ora, ids, 8, E, "compact")
    run_both(ora, ids, 8, E, "compact", block_e=1)
    run_both(ora, ids, 8, E, "masked", cap=max(1, T * K // E // 2))


def test_many_assignments(ora):
    """Two million assignments: 256 chunks of 8192."""
    rng = np.random.default_rng(9)
    ids = si.zipf_topk(rng, 262144, 256, 8)
    run_both(ora, ids, 0, 256, "compact")

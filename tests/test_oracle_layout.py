"""Pins for the oracle's layout step: histogram, block-aligned regions, the
static compact bound, stable slots, m_indices and the masked slab."""
import itertools
import json
import os

import numpy as np
import pytest

import synthetic_inputs as si

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")


def rows_needed(counts, block):
    return sum(-(-c // block) * block for c in counts)


# -------------------------------------------------------------- the bound

def test_compact_bound_vs_brute_force(ora):
    """Over every top-K-distinct routing of T tokens to E experts, the rows a
    compact layout needs never exceed the bound, and the bound is reached for
    K = 1 (every count vector is realisable there), which is what makes it
    tight and routing-independent."""
    cases = 0
    for E in range(1, 5):
        for K in range(1, E + 1):
            subsets = list(itertools.combinations(range(E), K))
            for T in range(0, 5):
                if len(subsets) ** T > 4096:
                    continue
                for block in range(1, 5):
                    A = T * K
                    bound = ora.compact_row_bound(A, E, block)
                    best = 0
                    for routing in itertools.product(subsets, repeat=T):
                        c = [0] * E
                        for sub in routing:
                            for e in sub:
                                c[e] += 1
                        best = max(best, rows_needed(c, block))
                    assert best <= bound, (E, K, T, block)
                    if K == 1:
                        assert best == bound, (E, T, block)
                    cases += 1
    assert cases > 150
    # the bound can be loose for K > 1 (two tokens, two experts, both top-2)
    assert ora.compact_row_bound(4, 2, 2) == 6


def test_compact_bound_closed_forms(ora):
    assert ora.compact_row_bound(64 * 2, 8, 128) == 1024
    assert ora.compact_row_bound(8192 * 8, 256, 128) == 98048
    assert ora.compact_row_bound(16384 * 8, 128, 128) == 147328
    assert ora.compact_row_bound(0, 256, 128) == 0
    assert ora.compact_row_bound(3, 256, 128) == 3 * 128


def test_layout_rule_truth_table(ora):
    facts = json.load(open(GOLDEN))["layout_rule_cases"]
    for n_global, n_local, masked in facts["cases"]:
        assert ora.should_use_masked(n_global, n_local) == masked


# ------------------------------------------------------------ compact map

def m_indices_by_definition(counts, starts, num_rows):
    """m_indices from its definition: row r holds e exactly when
    start_e <= r < start_e + c_e; every other row, padding inside a region
    and the tail past the last region alike, holds -1 (sglang PR #33128 page,
    Implementation breakdown item 3 and Key source snippets: padding rows
    carry expert index -1)."""
    counts = np.asarray(counts, np.int64)
    starts = np.asarray(starts, np.int64)
    m = np.full(num_rows, -1, np.int64)
    labels = np.repeat(np.arange(len(counts)), counts)
    # position of each real row inside its expert's run
    first = np.repeat(np.cumsum(counts) - counts, counts)
    rows = np.repeat(starts, counts) + (np.arange(len(labels)) - first)
    m[rows] = labels
    return m


def psum_starts(counts, align):
    """Region starts by the psum geometry: expert e occupies
    [align(psum[e-1]), psum[e]) with psum[-1] = 0, where psum[e] is the
    previous region's aligned end plus c_e (a fold over the counts)."""
    up = lambda n: -(-n // align) * align  # noqa: E731
    psum = list(itertools.accumulate(counts, lambda end, c: up(end) + c,
                                     initial=0))
    return [up(p) for p in psum[:-1]], up(psum[-1])


def check_compact_invariants(lay, ids, b, E, block):
    counts, off = lay["counts"], lay["expert_offsets"]
    s2d, m = lay["src2dst"], lay["m_indices"]
    local = (ids >= b) & (ids < b + E)
    assert counts.sum() == local.sum()
    assert np.array_equal(np.bincount(ids[local] - b, minlength=E), counts)
    assert (off % block == 0).all()
    assert np.array_equal(np.diff(off), -(-counts // block) * block)
    assert (s2d[~local] == -1).all()
    d = s2d[local]
    assert len(np.unique(d)) == len(d)                 # injective
    assert set(d.tolist()) == set(np.flatnonzero(m >= 0).tolist())  # onto
    # a destination row carries its expert id
    assert np.array_equal(m[d], (ids[local] - b))
    # stable: inside an expert, slots grow with the flat index t*K + j
    flat_e = np.where(local, ids - b, -1).reshape(-1)
    flat_d = s2d.reshape(-1)
    for e in range(E):
        de = flat_d[flat_e == e]
        assert np.array_equal(de, np.arange(off[e], off[e] + counts[e]))


@pytest.mark.parametrize("seed", range(6))
def test_compact_layout_random(ora, seed):
    rng = np.random.default_rng(seed)
    E = int(rng.integers(1, 40))
    K = int(rng.integers(1, min(E, 8) + 1))
    T = int(rng.integers(0, 300))
    block = int(rng.choice([1, 4, 16, 128]))
    ids = si.uniform_topk(rng, T, E, K)
    lay = ora.moe_layout(ids, 0, E, "compact", block_e=block)
    check_compact_invariants(lay, ids, 0, E, block)
    # m_indices equals its definition over the psum geometry, the tail past
    # the last region included
    starts, end = psum_starts(lay["counts"].tolist(), block)
    assert starts == lay["expert_offsets"][:-1].tolist()
    assert end == lay["expert_offsets"][-1]
    want = m_indices_by_definition(lay["counts"], starts, lay["num_rows"])
    assert np.array_equal(lay["m_indices"], want)


def test_compact_layout_expert_window(ora):
    """Only experts in [begin, begin + E) are local; the rest get -1."""
    rng = np.random.default_rng(5)
    ids = si.uniform_topk(rng, 200, 64, 6)
    lay = ora.moe_layout(ids, 16, 16, "compact", block_e=128)
    check_compact_invariants(lay, ids, 16, 16, 128)


def test_psum_geometry_page_example(ora):
    """counts [3, 0, 130, 1] with alignment 128: starts 0, 128, 128, 384 and
    an aligned end of 512, on both the psum rule and the oracle layout."""
    counts = [3, 0, 130, 1]
    starts, end = psum_starts(counts, 128)
    assert starts == [0, 128, 128, 384] and end == 512
    ids = np.concatenate([np.full(c, e) for e, c in enumerate(counts)])
    lay = ora.moe_layout(ids.reshape(-1, 1).astype(np.int32), 0, 4, "compact")
    assert lay["expert_offsets"].tolist() == starts + [end]
    m = lay["m_indices"]
    assert (m[0:3] == 0).all() and (m[3:128] == -1).all()
    assert (m[128:258] == 2).all() and (m[258:384] == -1).all()
    assert m[384] == 3 and (m[385:] == -1).all()


def test_adjacent_ragged_experts(ora):
    """Neighbouring experts whose counts are not multiples of 128: padding
    rows of one must never carry the next expert's id."""
    counts = [127, 129, 1, 255, 256, 0, 2]
    ids = np.concatenate([np.full(c, e) for e, c in enumerate(counts)])
    rng = np.random.default_rng(0)
    ids = rng.permutation(ids).reshape(-1, 1).astype(np.int32)
    lay = ora.moe_layout(ids, 0, len(counts), "compact")
    check_compact_invariants(lay, ids, 0, len(counts), 128)
    off = lay["expert_offsets"]
    for e, c in enumerate(counts):
        seg = lay["m_indices"][off[e]:off[e + 1]]
        assert (seg[:c] == e).all() and (seg[c:] == -1).all()


def test_empty_batch_layout(ora):
    ids = np.zeros((0, 8), np.int32)
    lay = ora.moe_layout(ids, 0, 256, "compact")
    assert lay["num_rows"] == 0
    assert (lay["counts"] == 0).all() and (lay["expert_offsets"] == 0).all()


def test_num_rows_too_small_rejected(ora):
    ids = np.zeros((4, 1), np.int32)
    with pytest.raises(ValueError):
        ora.moe_layout(ids, 0, 1, "compact", num_rows=64)


# ------------------------------------------------------------- masked slab

def test_masked_layout_decode_shape(ora):
    b = si.decode_masked(H=256)
    lay = ora.moe_layout(b.topk_ids, 0, 32, "masked", capacity=128)
    assert lay["overflow"] == 0
    local = b.topk_ids < 32
    assert 60 < local.sum() < 200  # about 1/8 of 1024 assignments
    assert np.array_equal(lay["masked_m"], lay["counts"])
    s2d, ids = lay["src2dst"], b.topk_ids
    d = s2d[local]
    assert np.array_equal(d // 128, ids[local])
    assert len(np.unique(d)) == len(d)
    m = lay["m_indices"]
    for e in range(32):
        seg = m[e * 128:(e + 1) * 128]
        c = lay["counts"][e]
        assert (seg[:c] == e).all() and (seg[c:] == -1).all()
        de = s2d.reshape(-1)[(ids.reshape(-1) == e)]
        assert np.array_equal(de, e * 128 + np.arange(c))


def test_masked_overflow_fails_fast(ora):
    """A hot expert with more assignments than the slab capacity: the extra
    assignments get no slot, masked_m is clipped and the flag is raised."""
    T, cap = 40, 16
    ids = np.zeros((T, 2), np.int32)
    ids[:, 0] = 3
    ids[:, 1] = np.arange(T) % 3 + 4
    lay = ora.moe_layout(ids, 0, 8, "masked", capacity=cap)
    assert lay["overflow"] == 1
    assert lay["counts"][3] == T and lay["masked_m"][3] == cap
    col = lay["src2dst"][:, 0]
    assert np.array_equal(col[:cap], 3 * cap + np.arange(cap))
    assert (col[cap:] == -1).all()
    assert (lay["src2dst"][:, 1] >= 0).all()
    under = ora.moe_layout(ids[:cap], 0, 8, "masked", capacity=cap)
    assert under["overflow"] == 0

"""Pins for the oracle's psum (expanded) layout repack: m_indices from psum,
expanded -> masked slab, masked slab -> expanded with fused weights.

Geometry (DeepEPv2 page, Key source snippets, the layout fixture's
docstring): expert e occupies rows [align(psum[e-1]), psum[e]) with
psum[-1] = 0.  The fixture keeps that page's row values (real row r holds
r mod 200 + 1, twice that on odd columns), so a row or column mix-up
changes a value; the arrays are built here from the geometry alone."""
import itertools

import numpy as np
import pytest

import synthetic_inputs as si


def align_up(n, a):
    return -(-n // a) * a


def psum_of(counts, align):
    """psum by its defining recurrence psum[e] = align(psum[e-1]) + c_e,
    psum[-1] = 0, as a fold over the counts."""
    return list(itertools.accumulate(counts, lambda end, c: align_up(end, align)
                                     + c, initial=0))[1:]


def real_rows(counts, starts, n):
    """Boolean mask of the rows that hold an assignment."""
    r = np.arange(n)
    e = np.searchsorted(np.asarray(starts), r, side="right") - 1
    ok = e >= 0
    ee = np.where(ok, e, 0)
    return ok & (r - np.asarray(starts)[ee] < np.asarray(counts)[ee])


def build_layout(counts, align, hidden):
    """Rows of the expanded layout (float32), psum, region starts and the
    padded total (at least one row, so an all-empty layout still has a
    buffer)."""
    psum = psum_of(counts, align)
    starts = [align_up(p, align) for p in [0] + psum[:-1]]
    total = max(align_up(psum[-1], align) if psum else 0, 1)
    real = real_rows(counts, starts, total)
    row_val = np.where(real, np.arange(total) % 200 + 1, 0).astype(np.float32)
    gain = 1.0 + (np.arange(hidden) % 2).astype(np.float32)
    base = row_val[:, None] * gain[None, :]
    return base, np.array(psum, np.int32), starts, total


def bits(a):
    return si.to_bf16_bits(a)


def vals(b):
    return (np.asarray(b, np.uint32) << 16).view(np.float32)


def test_psum_geometry_matches_compact_layout(ora):
    """psum built from a routing's counts with alignment block_e reproduces
    the compact layout's region starts and m_indices (same geometry)."""
    rng = np.random.default_rng(3)
    for E, T, K in ((8, 300, 2), (32, 128, 8), (256, 1000, 8)):
        ids = si.zipf_topk(rng, T, E, K, n_zero=min(8, E // 4))
        lay = ora.moe_layout(ids, 0, E, "compact")
        _, psum, starts, total = build_layout(lay["counts"].tolist(), 128, 4)
        assert starts == lay["expert_offsets"][:-1].tolist()
        m = ora.m_indices_from_psum(psum, 128, lay["num_rows"])
        assert np.array_equal(m, lay["m_indices"])


def test_m_indices_tail_masks(ora):
    """Adjacent experts with ragged counts: rows past psum[e] are -1, never
    the next expert's id, and rows past the last range are -1."""
    counts = [3, 0, 130, 1, 127, 128, 129]
    _, psum, starts, total = build_layout(counts, 128, 1)
    m = ora.m_indices_from_psum(psum, 128, total + 200)
    for e, (s, c) in enumerate(zip(starts, counts)):
        assert (m[s:s + c] == e).all()
    real = real_rows(counts, starts, total + 200)
    assert (m[~real] == -1).all()
    assert starts[:4] == [0, 128, 128, 384]


@pytest.mark.parametrize("counts", [[5, 0, 17, 3], [0, 0, 0], [64, 1, 0, 63],
                                    [1] * 9, [40, 2]])
def test_expand_slab_roundtrip(ora, counts):
    H, max_m, align = 96, 64, 16
    base, psum, starts, total = build_layout(counts, align, H)
    xb = bits(base)
    slab, _, mm, flags = ora.expand_to_masked_slab(xb.view(np.uint8), psum,
                                                   align, max_m)
    assert flags == 0
    assert mm.tolist() == counts
    slab16 = slab.view(np.uint16).reshape(len(counts) * max_m, H)
    for e, (s, c) in enumerate(zip(starts, counts)):
        for j in range(c):
            assert np.array_equal(slab16[e * max_m + j], xb[s + j])
    canary = np.full((total, H), 0x7FC0, np.uint16)
    back = ora.masked_slab_to_expand(slab16, mm, psum, align, max_m,
                                     out=canary.copy())
    real = real_rows(counts, starts, total)
    assert np.array_equal(back[real], xb[real])
    assert (back[~real] == 0x7FC0).all()


def test_overflow_fails_fast(ora):
    """Counts at and over the slab capacity: at capacity is fine; over it
    sets the flag and copies only max_m rows (never past the slab)."""
    H, max_m = 32, 8
    for counts, over in (([8, 3], 0), ([9, 3], 1), ([3, 20, 0], 1)):
        base, psum, starts, total = build_layout(counts, 8, H)
        slab, _, mm, flags = ora.expand_to_masked_slab(
            bits(base).view(np.uint8), psum, 8, max_m)
        assert (flags & 1) == over
        assert mm.tolist() == [min(c, max_m) for c in counts]
        assert slab.shape[0] == len(counts) * max_m


def test_psum_past_source_rows_is_flagged(ora):
    base, psum, _, total = build_layout([4, 4], 8, 16)
    psum = psum.copy()
    psum[1] = total + 5            # claims rows the source does not have
    _, _, mm, flags = ora.expand_to_masked_slab(bits(base).view(np.uint8),
                                                psum, 8, 64)
    assert flags & 2
    assert mm[1] == total - 8


def test_weights_fused_on_real_rows_only(ora):
    counts = [7, 0, 12]
    H, max_m, align = 64, 16, 8
    base, psum, starts, total = build_layout(counts, align, H)
    xb = bits(base)
    slab, _, mm, _ = ora.expand_to_masked_slab(xb.view(np.uint8), psum, align,
                                               max_m)
    rng = np.random.default_rng(0)
    w = rng.uniform(0.01, 1.0, total).astype(np.float32)
    out = np.full((total, H), 0x1234, np.uint16)
    ora.masked_slab_to_expand(slab.view(np.uint16).reshape(-1, H), mm, psum,
                              align, max_m, weights=w, out=out)
    for s, c in zip(starts, counts):
        for j in range(c):
            exact = vals(xb[s + j]).astype(np.float64) * np.float64(w[s + j])
            got = vals(out[s + j]).astype(np.float64)
            # one bf16 rounding: at most half an ulp, 2^-8 of the value
            assert (np.abs(got - exact) <= 2.0 ** -8 * np.abs(exact)).all()
            # every odd column is twice its even neighbour before rounding
            assert np.allclose(got[1::2], 2 * got[0::2], rtol=2 ** -7)
    real = real_rows(counts, starts, total)
    assert (out[~real] == 0x1234).all()


@pytest.mark.parametrize("col_major", [False, True])
def test_scale_copy_by_stride(ora, col_major):
    """Scales copied by their source strides.  Seven scale columns (hidden
    896 in groups of 128) do not divide a pack of four, the case a hidden of
    512 hid."""
    counts = [5, 9, 0, 2]
    H, max_m, align, s_cols = 896, 16, 4, 7
    base, psum, starts, total = build_layout(counts, align, H)
    q = np.random.default_rng(1).integers(0, 255, (total, H), np.uint8)
    # a distinct value per (real row, column); other rows stay 0
    real = real_rows(counts, starts, total)
    row_code = np.where(real, (np.arange(total) % 50 + 1) * 0.5, 0.0)
    sc = np.where(real[:, None], row_code[:, None] + np.arange(s_cols),
                  0.0).astype(np.float32)
    src = np.ascontiguousarray(sc.T) if col_major else sc
    slab, slab_s, mm, flags = ora.expand_to_masked_slab(
        q, psum, align, max_m, scales=src, scales_col_major=col_major)
    assert flags == 0
    for e, (s, c) in enumerate(zip(starts, counts)):
        for j in range(c):
            assert np.array_equal(slab[e * max_m + j], q[s + j])
            assert np.array_equal(slab_s[e * max_m + j], sc[s + j])

"""Pins for the oracle's scatter of already-quantized rows (the prefill path
that writes a dispatcher's fp8 rows and scales into the contiguous layout at
its psum offsets): against numpy fancy indexing, with scales in either
orientation, skipped destinations and canaries on untouched rows."""
import numpy as np
import pytest

import synthetic_inputs as si
from test_oracle_psum import build_layout


def numpy_scatter(x, d, num_rows, out):
    t_idx = np.repeat(np.arange(x.shape[0]), d.shape[1]).reshape(d.shape)
    sel = (d >= 0) & (d < num_rows)
    out[d[sel]] = x[t_idx[sel]]
    return out


@pytest.mark.parametrize("elem,in_cm,out_cm", [(1, False, False),
                                               (4, True, False),
                                               (4, False, True),
                                               (1, True, True)])
def test_against_fancy_indexing(ora, elem, in_cm, out_cm):
    rng = np.random.default_rng(elem * 10 + in_cm * 2 + out_cm)
    T, K, E, rb, cols = 77, 4, 9, 448, 7
    ids = si.uniform_topk(rng, T, 12, K)            # experts 9..11 non-local
    lay = ora.moe_layout(ids, 0, E, "compact", block_e=16)
    R = lay["num_rows"]
    x = rng.integers(0, 256, (T, rb), dtype=np.uint8)
    dt = np.uint8 if elem == 1 else np.float32
    sc = rng.integers(0, 250, (T, cols)).astype(dt)
    canary_q = np.full((R, rb), 0xA5, np.uint8)
    canary_s = np.full((cols, R) if out_cm else (R, cols), 77, dt)
    q, s = ora.scatter_rows(x, lay["src2dst"], R,
                            scales=np.ascontiguousarray(sc.T) if in_cm else sc,
                            scales_col_major=in_cm, out=canary_q.copy(),
                            out_scales=canary_s.copy(),
                            out_scales_col_major=out_cm)
    want_q = numpy_scatter(x, lay["src2dst"], R, canary_q.copy())
    want_s = numpy_scatter(sc, lay["src2dst"], R,
                           (canary_s.T.copy() if out_cm else canary_s.copy()))
    assert np.array_equal(q, want_q)
    assert np.array_equal(s.T if out_cm else s, want_s)
    pad = lay["m_indices"] < 0
    assert (q[pad] == 0xA5).all()


def test_rows_land_at_psum_offsets(ora):
    """With psum built from the routing's counts (128-aligned, the page's
    fixture geometry), each expert's rows start at align(psum[e-1]) and come
    in ascending token order; the compact layout of the same routing gives
    these destinations."""
    rng = np.random.default_rng(3)
    T, K, E = 300, 8, 32
    ids = si.zipf_topk(rng, T, E, K, n_zero=4)
    lay = ora.moe_layout(ids, 0, E, "compact", block_e=128)
    _, psum, starts, total = build_layout(lay["counts"].tolist(), 128, 1)
    assert starts == lay["expert_offsets"][:-1].tolist()
    x = np.repeat(np.arange(T, dtype=np.uint32)[:, None], 4, 1).view(np.uint8)
    q, _ = ora.scatter_rows(x, lay["src2dst"], lay["num_rows"],
                            out=np.full((lay["num_rows"], 16), 0xFF, np.uint8))
    tok = q.view(np.uint32)[:, 0]
    for e in range(E):
        c = lay["counts"][e]
        rows = tok[starts[e]:starts[e] + c]
        want = np.flatnonzero((ids == e).any(axis=1))
        assert np.array_equal(rows, want)
        assert (tok[starts[e] + c:psum[e] + (128 - c % 128) % 128] ==
                0xFFFFFFFF).all()


def test_out_of_range_destinations_are_skipped(ora):
    x = np.arange(3 * 32, dtype=np.uint8).reshape(3, 32)
    d = np.array([[0, 5], [-1, 2], [7, 1]], np.int32)   # 5, 7 >= num_rows
    q, _ = ora.scatter_rows(x, d, 4, out=np.zeros((4, 32), np.uint8))
    assert np.array_equal(q[0], x[0]) and np.array_equal(q[2], x[1])
    assert np.array_equal(q[1], x[2]) and (q[3] == 0).all()

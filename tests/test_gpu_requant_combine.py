"""requant_per_token_to_per_tensor and moe_combine on the GPU against the
oracle.  Requant: bytes and the tensor scale bit-exact.  Combine: bit-exact
against the oracle's fp32 accumulation order, and within rel 1e-3 of the
float64 sum (|gpu - exact| <= 1e-3 * sum_j |w_j y_j|)."""
import numpy as np
import pytest
import torch

import fp8_mx_activation_amd as mxq
import synthetic_inputs as si
from gpu_util import (DEV, assert_equal, bf16_to_dev, bf16_to_host,
                      f32_to_dev, host, i32_to_dev, say, u8_to_dev)

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------ requant

def requant_both(ora, q, s, ld_pad=0, in_place=False):
    T, H = q.shape
    say("requant T=%d H=%d pad=%d in_place=%s" % (T, H, ld_pad, in_place))
    qin_full = torch.zeros((T, H + ld_pad), dtype=torch.uint8, device=DEV)
    qin_full[:, :H] = u8_to_dev(q)
    qin = qin_full[:, :H]
    qout = qin if in_place else None
    out, S = mxq.requant_per_token_to_per_tensor(qin, f32_to_dev(s),
                                                 q_out=qout)
    torch.cuda.synchronize()
    ref, S_ref = ora.requant_per_token_to_per_tensor(q, s)
    assert np.float32(host(S)[0]) == np.float32(S_ref)
    assert_equal(host(out), ref, "requant bytes")


def test_requant_full(ora):
    rb = si.requant_input()
    requant_both(ora, rb.q, rb.scales)


def test_requant_identity_and_zero(ora):
    rng = np.random.default_rng(2)
    q, _ = si.per_token_fp8(rng, 100, 512)
    requant_both(ora, q, np.full(100, 2.0 ** -3, np.float32))
    requant_both(ora, np.zeros((5, 64), np.uint8), np.ones(5, np.float32))


def test_requant_ragged_in_place(ora):
    rng = np.random.default_rng(3)
    q, s = si.per_token_fp8(rng, 37, 100)
    requant_both(ora, q, s, ld_pad=12)
    requant_both(ora, q, s, ld_pad=12, in_place=True)
    q1, s1 = si.per_token_fp8(rng, 1, 4096)
    requant_both(ora, q1, s1)
    q2, s2 = si.per_token_fp8(rng, 3000, 48, log2_lo=-30, log2_hi=30)
    requant_both(ora, q2, s2)


def fp8_rows_with_amax(rng, amax, H):
    """e4m3 rows (torch's float32 cast) whose largest magnitude is about
    amax[t]; amax[t] = 0 gives an all-zero row."""
    T = amax.shape[0]
    z = rng.standard_normal((T, H), dtype=np.float32)
    m = np.abs(z).max(axis=1, keepdims=True)
    m[m == 0] = 1.0
    y = np.clip(z * (amax.astype(np.float32)[:, None] / m), -448.0, 448.0)
    return torch.from_numpy(y.astype(np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def test_requant_max_from_rows_below_the_top_scale(ora):
    """The max pass reads a row only while its bound 448 * s_t can still
    raise the maximum.  Here the rows with the largest scale hold small
    values, so the maximum comes from rows with smaller scales, which the
    pass must still read; blocks of 16 rows see different top scales."""
    rng = np.random.default_rng(11)
    T, H = 777, 100              # H % 16 != 0 (row stride 112): byte tail read
    u = rng.integers(-8, 5, size=T)
    s = np.exp2(u).astype(np.float32)
    amax = np.where(u == 4, 0.5, 448.0)
    q = fp8_rows_with_amax(rng, amax, H)
    requant_both(ora, q, s, ld_pad=12)
    # ties: bound of the 2^3 rows (3584) equals the value of the 2^4 rows
    # that hold 224, and one 2^2 row holds the max of its block
    amax = np.where(u == 4, 224.0, np.where(u == 3, 448.0, 300.0))
    q = fp8_rows_with_amax(rng, amax, H)
    requant_both(ora, q, s, ld_pad=12)


def test_requant_non_power_of_two_scales(ora):
    """Scales that are not powers of two and row maxima spread over the
    whole e4m3 range: bounds of many distinct values, so both read phases
    of the max pass select rows."""
    rng = np.random.default_rng(12)
    for T, H in ((1000, 64), (3001, 208), (16389, 32)):   # 16389: 17 rows/block
        s = rng.uniform(0.25, 4.0, size=T).astype(np.float32)
        amax = np.exp2(rng.uniform(-9.0, np.log2(448.0), size=T))
        amax[rng.random(T) < 0.05] = 0.0
        q = fp8_rows_with_amax(rng, amax, H)
        requant_both(ora, q, s)


def test_requant_more_rows_than_one_ranking_round(ora):
    """T = 1.1M rows: each block of the max pass owns 1075 rows and screens
    them in runs of 64, carrying its maximum across runs."""
    rng = np.random.default_rng(13)
    T, H = 1_100_000, 16
    u = rng.integers(-6, 3, size=T)
    s = np.exp2(u).astype(np.float32)
    amax = np.exp2(rng.uniform(0.0, np.log2(448.0), size=T))
    q = fp8_rows_with_amax(rng, amax, H)
    requant_both(ora, q, s)


def test_requant_equal_bounds_below_448(ora):
    """Equal token scales and no row holding 448: every row's bound equals
    the largest, no row attains it, so the max pass reads every row, four
    at a time, and the maximum may sit in any of them.  Then the same rows
    with one row per 64 reaching 448 at a random place."""
    rng = np.random.default_rng(14)
    for T, H in ((1000, 64), (4099, 4096), (130, 112)):
        s = np.full(T, 2.0 ** -3, np.float32)
        amax = rng.uniform(1.0, 400.0, size=T)
        q = fp8_rows_with_amax(rng, amax, H)
        requant_both(ora, q, s)
        for r0 in range(0, T, 64):
            amax[r0 + int(rng.integers(0, min(64, T - r0)))] = 448.0
        q = fp8_rows_with_amax(rng, amax, H)
        requant_both(ora, q, s)


def test_requant_rows_of_several_batches(ora):
    """Rows longer than one 4 KB batch of the rewrite pass (which loads the
    next batch before storing the current one), with a byte tail, in place
    and out of place; and rows shorter than 16 bytes."""
    rng = np.random.default_rng(15)
    for T, H, pad in ((700, 7168, 0), (333, 8200, 8), (64, 12296, 24),
                      (50, 8, 8)):
        q, s = si.per_token_fp8(rng, T, H)
        requant_both(ora, q, s, ld_pad=pad)
        requant_both(ora, q, s, ld_pad=pad, in_place=True)


def test_requant_operation_order_cases(ora):
    """Rows where two other operation orders round to other bytes than R6's
    (built in test_oracle_paths): the kernel gives R6's bytes."""
    from test_oracle_paths import requant_order_cases
    q, scales, _, _ = requant_order_cases()
    requant_both(ora, q, scales)


def test_requant_empty():
    say("requant T=0")
    q = torch.zeros((0, 64), dtype=torch.uint8, device=DEV)
    _, S = mxq.requant_per_token_to_per_tensor(
        q, torch.zeros(0, dtype=torch.float32, device=DEV))
    assert host(S)[0] == 1.0


# ------------------------------------------------------------------ combine

def combine_both(ora, y_dev, src2dst, w, out_dtype=torch.bfloat16,
                 y_host=None, tokens=None):
    """src2dst entries outside [0, rows) are skipped by the kernel; the
    oracle gets them as -1, the same meaning."""
    T, K = src2dst.shape
    R, H = y_dev.shape
    say("combine T=%d K=%d rows=%d H=%d out=%s" % (T, K, R, H, out_dtype))
    out = mxq.moe_combine(y_dev, i32_to_dev(src2dst), f32_to_dev(w),
                          out_dtype=out_dtype)
    torch.cuda.synchronize()
    if y_host is None:
        y_host = bf16_to_host(y_dev)
    sel = np.arange(T) if tokens is None else np.asarray(tokens)
    d_sel = np.where(src2dst[sel] >= R, -1, src2dst[sel]).astype(np.int32)
    w_sel = w[sel]
    acc = ora.combine_f32(y_host, d_sel, w_sel)
    exact, mag = ora.combine_f64(y_host, d_sel, w_sel)
    if out_dtype == torch.float32:
        got = host(out)[sel]
        assert_equal(got.view(np.uint32), acc.view(np.uint32),
                     "combine fp32 bits")
        assert (np.abs(got - exact) <= 1e-3 * mag).all()
    else:
        got_bits = bf16_to_host(out)[sel]
        assert_equal(got_bits, ora.bf16_round(acc), "combine bf16 bits")
        gotv = (got_bits.astype(np.uint32) << 16).view(np.float32)
        # bf16 output adds one rounding of at most 2^-8 relative
        assert (np.abs(gotv - exact) <= 1e-3 * mag + 2.0 ** -8 *
                np.abs(exact)).all()
        assert np.isfinite(gotv).all()
    return out


def layout_and_outputs(ora, ids, E, kind, H, seed, cap=0):
    ref = ora.moe_layout(ids, 0, E, kind, capacity=cap)
    y = si.expert_outputs_bf16(seed, ref["num_rows"], H)
    si.poison_padding_rows(y, ref["m_indices"])
    return ref, y


def test_tiny(ora):
    b = si.tiny()
    ref, y = layout_and_outputs(ora, b.topk_ids, 8, "compact", b.H, 11)
    combine_both(ora, bf16_to_dev(y), ref["src2dst"], b.topk_weights,
                 y_host=y)
    combine_both(ora, bf16_to_dev(y), ref["src2dst"], b.topk_weights,
                 out_dtype=torch.float32, y_host=y)


def test_decode_masked_equals_compact(ora):
    """Same per-assignment expert outputs placed in both layouts: the GPU
    combine gives identical tokens from either."""
    b = si.decode_masked()
    rng = np.random.default_rng(12)
    ya = si.gaussian_bf16(rng, (b.T, b.K, b.H))
    outs = []
    for kind, cap in (("compact", 0), ("masked", 128)):
        ref = ora.moe_layout(b.topk_ids, 0, 32, kind, capacity=cap)
        y = np.full((ref["num_rows"], b.H), 0x7FC0, np.uint16)
        sel = ref["src2dst"] >= 0
        y[ref["src2dst"][sel]] = ya[sel]
        outs.append(bf16_to_host(combine_both(
            ora, bf16_to_dev(y), ref["src2dst"], b.topk_weights, y_host=y)))
    assert_equal(outs[0], outs[1], "masked vs compact")


def test_prefill_compact_full(ora):
    b = si.prefill_compact(H=128)
    ref = ora.moe_layout(b.topk_ids, 0, 256, "compact")
    H = 7168
    say("prefill combine: drawing", ref["num_rows"], "x", H, "on device")
    y = si.gaussian_bf16_device(303, (ref["num_rows"], H), DEV)
    y[torch.from_numpy(ref["m_indices"] < 0).to(DEV)] = float("nan")
    y_host = bf16_to_host(y)
    combine_both(ora, y, ref["src2dst"], b.topk_weights, y_host=y_host)


def test_large_combine_sampled(ora):
    """16384 tokens x 4096 from 147328 rows; every token is checked."""
    ids, w = si.large_combine_routing()
    ref = ora.moe_layout(ids, 0, 128, "compact")
    say("large combine: drawing", ref["num_rows"], "x 4096 on device")
    y = si.gaussian_bf16_device(505, (ref["num_rows"], 4096), DEV)
    y[torch.from_numpy(ref["m_indices"] < 0).to(DEV)] = float("nan")
    y_host = bf16_to_host(y)
    combine_both(ora, y, ref["src2dst"], w, y_host=y_host)
    combine_both(ora, y, ref["src2dst"], w, out_dtype=torch.float32,
                 y_host=y_host, tokens=np.arange(0, 16384, 7))


def test_skip_rules_and_ragged(ora):
    rng = np.random.default_rng(6)
    T, K, H = 90, 11, 136
    ids = si.uniform_topk(rng, T, 40, K)
    ref, y = layout_and_outputs(ora, ids, 20, "compact", H, 13)
    s2d = ref["src2dst"].copy()
    s2d[::5, 3] = ref["num_rows"] + 7          # out of range: skipped
    w = si.softmax_weights(rng, T, K)
    combine_both(ora, bf16_to_dev(y), s2d, w, y_host=y)
    combine_both(ora, bf16_to_dev(y), s2d, w, out_dtype=torch.float32,
                 y_host=y)


def test_no_local_assignment_gives_zero(ora):
    y = np.zeros((128, 64), np.uint16)
    s2d = np.full((10, 4), -1, np.int32)
    w = np.ones((10, 4), np.float32)
    out = combine_both(ora, bf16_to_dev(y), s2d, w, y_host=y)
    assert (bf16_to_host(out) == 0).all()


@pytest.mark.parametrize("T,H", [(1, 1032), (192, 1032), (193, 1032),
                                 (192, 7168), (193, 7168), (5, 1024)])
def test_row_slices_and_their_boundary(ora, T, H):
    """Up to 192 tokens a row is combined in slices of 1024 channels, one
    block each (H = 1032: a last slice of 8 channels; H = 1024: one slice);
    from 193 tokens one block takes the whole row.  Both out dtypes, every
    token compared, out-of-range entries skipped."""
    rng = np.random.default_rng(T * 7 + H)
    K = 8
    ids = si.uniform_topk(rng, T, 64, K)
    ref, y = layout_and_outputs(ora, ids, 48, "compact", H, T + H)
    s2d = ref["src2dst"].copy()
    s2d[::7, 2] = ref["num_rows"] + 3
    w = si.softmax_weights(rng, T, K)
    yd = bf16_to_dev(y)
    combine_both(ora, yd, s2d, w, y_host=y)
    combine_both(ora, yd, s2d, w, out_dtype=torch.float32, y_host=y)

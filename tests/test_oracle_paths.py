"""Pins for the oracle's data-moving steps: scatter+quant, live-row MX quant,
per-token -> per-tensor requant and the weighted combine."""
import numpy as np
import pytest
import torch

import synthetic_inputs as si

CANARY = 0xA5


def dec(b):
    return torch.from_numpy(np.ascontiguousarray(b, np.uint8)).view(
        torch.float8_e4m3fn).to(torch.float64).numpy()


def bf16_vals(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(
        np.float64)


def check_rows_bound(x_bits, q, s, G):
    x = bf16_vals(x_bits)
    e = np.repeat(s.astype(np.int64) - 127, G, axis=-1)
    deq = dec(q) * np.exp2(e.astype(np.float64))
    tol = np.maximum(np.abs(x) * 2.0 ** -4, np.exp2((e - 10).astype(float)))
    assert (np.abs(deq - x) <= tol).all()


# --------------------------------------------------------- scatter + quant

@pytest.mark.parametrize("G,H", [(128, 256), (32, 96), (128, 640), (32, 7168)])
def test_scatter_quant_copies_and_canary(ora, G, H):
    rng = np.random.default_rng(G + H)
    T, E, K = 37, 6, 3
    x = si.gaussian_bf16(rng, (T, H))
    ids = si.uniform_topk(rng, T, 9, K)   # experts 6..8 are not local
    lay = ora.moe_layout(ids, 0, E, "compact", block_e=16)
    R = lay["num_rows"]
    q = np.full((R, H), CANARY, np.uint8)
    s = np.full((R, H // G), CANARY, np.uint8)
    ora.scatter_quant(x, lay["src2dst"], G, R, q, s)
    m = lay["m_indices"]
    assert (q[m < 0] == CANARY).all() and (s[m < 0] == CANARY).all()
    for t in range(T):
        rq, rs = ora.quant_row(x[t], G)
        for d in lay["src2dst"][t]:
            if d >= 0:
                assert np.array_equal(q[d], rq) and np.array_equal(s[d], rs)
    live = m >= 0
    src_tok = np.empty(R, np.int64)
    for t in range(T):
        for d in lay["src2dst"][t]:
            if d >= 0:
                src_tok[d] = t
    check_rows_bound(x[src_tok[live]], q[live], s[live], G)


def test_scatter_quant_row_column_fixture(ora):
    """Each token row holds its own value, doubled on odd columns: a row mix-up
    or a column shift in the scatter lands on a different dequantized value."""
    T, H, G = 50, 640, 128
    base = (np.arange(T) % 200 + 1).astype(np.float32)[:, None]
    gain = 1.0 + (np.arange(H) % 2).astype(np.float32)[None, :]
    x = si.to_bf16_bits(base * gain)
    ids = (np.arange(T * 2).reshape(T, 2) % 5).astype(np.int32)
    lay = ora.moe_layout(ids, 0, 5, "compact", block_e=8)
    q, s = ora.scatter_quant(x, lay["src2dst"], G, lay["num_rows"])
    for t in range(T):
        for d in lay["src2dst"][t]:
            e = np.repeat(s[d].astype(np.int64) - 127, G)
            v = dec(q[d]) * np.exp2(e.astype(float))
            want = bf16_vals(x[t])
            assert np.allclose(v, want, rtol=2.0 ** -4)
            assert np.all(v[1::2] > v[0::2])


def test_masked_scatter_matches_compact_bytes(ora):
    """Both layouts hold byte-identical rows for each assignment."""
    b = si.decode_masked(H=512)
    comp = ora.moe_layout(b.topk_ids, 0, 32, "compact")
    mask = ora.moe_layout(b.topk_ids, 0, 32, "masked", capacity=128)
    qc, sc = ora.scatter_quant(b.x, comp["src2dst"], 128, comp["num_rows"])
    qm, sm = ora.scatter_quant(b.x, mask["src2dst"], 128, mask["num_rows"])
    dc, dm = comp["src2dst"], mask["src2dst"]
    assert np.array_equal(dc >= 0, dm >= 0)
    sel = dc >= 0
    assert np.array_equal(qc[dc[sel]], qm[dm[sel]])
    assert np.array_equal(sc[dc[sel]], sm[dm[sel]])


# ----------------------------------------------------------- live rows (MX)

def test_live_rows_only_live_written(ora):
    lr = si.live_rows(num_segments=4, rows_per_segment=24, H=256,
                      live_counts=[3, 0, 24, 7])
    rows, H = lr.x.shape
    q = np.full((rows, H), CANARY, np.uint8)
    s = np.full((rows, H // 32), CANARY, np.uint8)
    ora.mx_quant_live_rows(lr.x, 4, lr.live_counts, 32, q, s)
    for g in range(4):
        for r in range(24):
            row = g * 24 + r
            if r < lr.live_counts[g]:
                rq, rs = ora.quant_row(lr.x[row], 32)
                assert np.array_equal(q[row], rq) and np.array_equal(s[row], rs)
            else:
                assert (q[row] == CANARY).all() and (s[row] == CANARY).all()


def test_live_rows_counts_above_segment_are_clipped(ora):
    lr = si.live_rows(num_segments=2, rows_per_segment=4, H=64,
                      live_counts=[9, 1])
    q = np.full((8, 64), CANARY, np.uint8)
    s = np.full((8, 2), CANARY, np.uint8)
    ora.mx_quant_live_rows(lr.x, 2, lr.live_counts, 32, q, s)
    assert (q[0:4] != CANARY).any(axis=1).all()
    assert (q[5:8] == CANARY).all()


# ---------------------------------------------------------------- requant

def test_requant_identity_for_equal_power_of_two_scales(ora):
    """Every token scale 2^k and every row's largest magnitude 448: the
    per-tensor scale is 2^k and every byte is unchanged."""
    rng = np.random.default_rng(1)
    q, _ = si.per_token_fp8(rng, 64, 256)
    for k in (-8, 0, 3):
        s = np.full(64, 2.0 ** k, np.float32)
        out, S = ora.requant_per_token_to_per_tensor(q, s)
        assert S == 2.0 ** k
        assert np.array_equal(out, q)


def test_requant_properties(ora):
    rb = si.requant_input(T=300, H=512)
    out, S = ora.requant_per_token_to_per_tensor(rb.q, rb.scales)
    x = dec(rb.q) * rb.scales[:, None].astype(np.float64)
    t, j = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert out[t, j] & 0x7F == 0x7E                   # argmax -> 448
    assert np.float32(np.abs(x).max() / 448.0) == np.float32(S)
    assert ((out & 0x7F) <= 0x7E).all()               # no NaN, |q'| <= 448
    y = dec(out) * S
    tol = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * S) + \
        np.abs(x) * 2.0 ** -22
    assert (np.abs(y - x) <= tol).all()


def test_requant_bytes_equal_an_independent_construction(ora):
    """R6 built with other tools: torch's e4m3 decode, numpy float32
    products in the stated order (dec(q) * s_t, then * fl(1/S) with
    S = fl(amax / 448)), and torch's float32 -> e4m3fn cast, which rounds to
    nearest even and agrees with the saturating encoder below 464 (every
    |y| here is at most 448 (1 + 2^-23)).  Power-of-two scales, scales
    spread over 2^-30 .. 2^30, and scales that are not powers of two."""
    rng = np.random.default_rng(41)
    for T, H, lo, hi in ((300, 512, -8.0, 4.0), (200, 96, -30.0, 30.0)):
        q, s = si.per_token_fp8(rng, T, H, log2_lo=lo, log2_hi=hi)
        s_np2 = (s * rng.uniform(0.5, 2.0, T)).astype(np.float32)
        for sc in (s, s_np2):
            out, S = ora.requant_per_token_to_per_tensor(q, sc)
            d = torch.from_numpy(q).view(torch.float8_e4m3fn).float().numpy()
            rq = d * sc[:, None]                      # float32 products
            S_ref = np.float32(np.abs(rq).max()) / np.float32(448.0)
            inv = np.float32(1.0) / S_ref
            y = rq * inv
            assert y.dtype == np.float32 and np.abs(y).max() < 464.0
            ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(
                torch.uint8).numpy()
            assert np.float32(S) == S_ref
            assert np.array_equal(out, ref)


def e4m3_cast(y):
    return torch.from_numpy(np.ascontiguousarray(y, np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def requant_order_cases():
    """Rows on which R6's order, fl(fl(dec * s_t) * fl(1/S)), and two
    plausible other orders, dec * fl(s_t * fl(1/S)) and fl(dec * s_t) / S,
    round to different e4m3 bytes.  Row 0 holds 448 with the largest scale
    s0, which fixes S; every other row holds one code d (then -0 and zeros)
    with a scale a few ulps from m * S / d, m an e4m3 midpoint, where a
    one-ulp change of y can cross the midpoint.  Returns (q, scales, S,
    stated-order bytes of column 0 of rows 1..)."""
    codes = np.arange(0x01, 0x7F, dtype=np.uint8)
    d = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    vals = torch.arange(0, 0x7F, dtype=torch.uint8).view(
        torch.float8_e4m3fn).float().numpy()
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)
    mids = mids[(mids >= 1.0) & (mids < 440.0)]
    s0 = np.float32(3.1)
    S = np.float32(np.float32(448.0) * s0) / np.float32(448.0)
    inv = np.float32(1.0) / S
    k = np.arange(-16, 17).astype(np.float32) * np.float32(2.0 ** -23)
    D = np.broadcast_to(d[:, None, None], (d.size, mids.size, k.size))
    sc = (mids[None, :, None] * S / d[:, None, None] *
          (1 + k[None, None, :])).astype(np.float32)
    D, sc = D.ravel(), sc.ravel()
    keep = D * sc < np.float32(448.0) * s0 * np.float32(0.999)
    D, sc = D[keep], sc[keep]
    rq = D * sc
    ref = e4m3_cast(rq * inv)
    diff_a = ref != e4m3_cast(D * (sc * inv))
    diff_b = ref != e4m3_cast(rq / S)
    assert diff_a.sum() >= 64 and diff_b.sum() >= 64
    pick = np.concatenate([np.flatnonzero(diff_a)[:64],
                           np.flatnonzero(diff_b)[:64]])
    code_of = dict(zip(d.tolist(), codes.tolist()))
    q = np.zeros((1 + pick.size, 16), np.uint8)
    q[0, 0] = 0x7E
    q[1:, 0] = [code_of[float(v)] for v in D[pick]]
    q[1:, 1] = 0x80                                        # -0 stays -0
    scales = np.concatenate([[s0], sc[pick]]).astype(np.float32)
    return q, scales, S, ref[pick]


def test_requant_operation_order_is_pinned(ora):
    """The oracle follows R6's order on rows where two other orders give
    other bytes (requant_order_cases)."""
    q, scales, S, want = requant_order_cases()
    out, S_got = ora.requant_per_token_to_per_tensor(q, scales)
    assert np.float32(S_got) == S
    assert np.array_equal(out[1:, 0], want)
    assert (out[1:, 1] == 0x80).all() and out[0, 0] == 0x7E
    assert (out[1:, 2:] == 0).all()


def test_requant_zero_input(ora):
    q = np.zeros((4, 64), np.uint8)
    q[1] = 0x80
    out, S = ora.requant_per_token_to_per_tensor(q, np.ones(4, np.float32))
    assert S == 1.0 and np.array_equal(out, q)


# ---------------------------------------------------------------- combine

def place_expert_outputs(yv_per_assign, src2dst, num_rows, H):
    """Put the per-assignment expert outputs at their layout rows; every other
    row is NaN (padding is never read)."""
    y = np.full((num_rows, H), 0x7FC0, np.uint16)
    sel = src2dst >= 0
    y[src2dst[sel]] = yv_per_assign[sel]
    return y


def test_masked_and_compact_combine_identically(ora):
    """Same routing, same per-assignment expert outputs, two layouts: the
    combined tokens are bit-identical (the masked-vs-compact end-to-end
    equivalence the standard-dispatch tests check)."""
    b = si.decode_masked(H=384)
    rng = np.random.default_rng(9)
    ya = si.gaussian_bf16(rng, (b.T, b.K, b.H))
    comp = ora.moe_layout(b.topk_ids, 0, 32, "compact")
    mask = ora.moe_layout(b.topk_ids, 0, 32, "masked", capacity=128)
    yc = place_expert_outputs(ya, comp["src2dst"], comp["num_rows"], b.H)
    ym = place_expert_outputs(ya, mask["src2dst"], mask["num_rows"], b.H)
    oc = ora.combine(yc, comp["src2dst"], b.topk_weights)
    om = ora.combine(ym, mask["src2dst"], b.topk_weights)
    assert np.array_equal(oc, om)
    assert np.isfinite(bf16_vals(oc)).all()


def test_combine_one_hot_and_empty_tokens(ora):
    rng = np.random.default_rng(2)
    T, H, E = 20, 128, 4
    ids = si.uniform_topk(rng, T, 8, 2)
    lay = ora.moe_layout(ids, 0, E, "compact", block_e=4)
    y = si.gaussian_bf16(rng, (lay["num_rows"], H))
    si.poison_padding_rows(y, lay["m_indices"])
    w = np.zeros((T, 2), np.float32)
    w[:, 0] = 1.0
    out = ora.combine(y, lay["src2dst"], w)
    for t in range(T):
        d0 = lay["src2dst"][t, 0]
        if d0 >= 0:
            assert np.array_equal(out[t], y[d0])
        elif lay["src2dst"][t, 1] < 0:
            assert (out[t] == 0).all()                # +0 rows
    assert np.isfinite(bf16_vals(out)).all()


def f32_nearest(fr):
    """The float32 nearest to the exact rational fr (ties to even),
    returned as a Python float; |fr| < 2^100 here, so no overflow."""
    from fractions import Fraction
    if fr == 0:
        return 0.0
    neg = fr < 0
    a = -fr if neg else fr
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1                                  # 2^e <= a < 2^(e+1)
    q = max(e - 23, -149)                       # 24-bit significand
    m = a / Fraction(2) ** q
    n = m.numerator // m.denominator
    r = m - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    v = float(n) * 2.0 ** q
    return -v if neg else v


def test_combine_fp32_order_equals_exact_fma(ora):
    """R7 built independently: each fused multiply-add w * y + acc computed
    exactly in rationals and rounded once to float32 (nearest, ties to
    even), over j ascending from +0, skipping assignments without a row.
    Multiply-then-add (two roundings) or j descending, planted in the
    oracle, fail here."""
    from fractions import Fraction
    rng = np.random.default_rng(5)
    T, K, H, E = 24, 8, 32, 16
    ids = si.uniform_topk(rng, T, E + 4, K)         # some ids non-local
    lay = ora.moe_layout(ids, 0, E, "compact")
    y = si.gaussian_bf16(rng, (lay["num_rows"], H))
    w = si.softmax_weights(rng, T, K)
    acc = ora.combine_f32(y, lay["src2dst"], w)
    yv = bf16_vals(y)
    want = np.zeros((T, H), np.float32)
    for t in range(T):
        for h in range(H):
            a = 0.0
            for j in range(K):
                d = lay["src2dst"][t, j]
                if d < 0:
                    continue
                a = f32_nearest(Fraction(float(w[t, j])) *
                                Fraction(float(yv[d, h])) + Fraction(a))
            want[t, h] = a
    assert np.array_equal(want.view(np.uint32), acc.view(np.uint32))


def test_combine_vs_float64(ora):
    b = si.tiny()
    lay = ora.moe_layout(b.topk_ids, 0, 8, "compact")
    rng = np.random.default_rng(4)
    y = si.gaussian_bf16(rng, (lay["num_rows"], b.H))
    si.poison_padding_rows(y, lay["m_indices"])
    acc = ora.combine_f32(y, lay["src2dst"], b.topk_weights)
    ref, mag = ora.combine_f64(y, lay["src2dst"], b.topk_weights)
    assert (np.abs(acc - ref) <= 1e-6 * mag + 1e-30).all()
    out = bf16_vals(ora.combine(y, lay["src2dst"], b.topk_weights))
    assert (np.abs(out - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6 * mag).all()
    # the plain float64 numpy sum agrees as well
    w = b.topk_weights.astype(np.float64)
    yv = bf16_vals(y)
    manual = np.zeros((b.T, b.H))
    for t in range(b.T):
        for j in range(b.K):
            d = lay["src2dst"][t, j]
            if d >= 0:
                manual[t] += w[t, j] * yv[d]
    assert np.allclose(manual, ref, rtol=1e-12, atol=1e-12)

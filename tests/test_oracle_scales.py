"""Pins for the scale variants: the OCP Microscaling exponent rule beside
the no-clipping rule, and the packed MN-major placement of scale bytes."""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import synthetic_inputs as si


def f32_from_bits(w):
    return np.asarray(w, np.uint32).view(np.float32)


def exact_floor_log2(v: float) -> int:
    """floor(log2 v) for v > 0 in exact rationals."""
    a = Fraction(v)
    k = 0
    while Fraction(2) ** (k + 1) <= a:
        k += 1
    while Fraction(2) ** k > a:
        k -= 1
    return k


def test_ocp_exponent_every_positive_bf16(ora):
    bits = np.arange(1, 0x7F80, dtype=np.uint32) << 16
    vals = f32_from_bits(bits).astype(np.float64)
    got = np.array([ora.ocp_mx_exponent(v) for v in vals])
    for v, e in zip(vals[::41], got[::41]):
        assert e == max(-127, min(127, exact_floor_log2(v) - 8))
    assert ora.ocp_mx_exponent(0.0) == -127
    # against the no-clipping rule: one larger exactly when the significand
    # of amax exceeds 1.75 (448 = 1.75 * 2^8), equal otherwise
    ceil = np.array([ora.pow2_scale_exponent(v) for v in vals])
    m, _ = np.frexp(vals)                     # vals = m * 2^E, m in [0.5, 1)
    sig = 2 * m
    live = (got > -127) & (ceil > -127)
    assert np.array_equal((ceil - got)[live], (sig > 1.75)[live].astype(int))


def test_ocp_rule_bound_and_saturation(ora):
    """Under the OCP rule |x / 2^e| < 512; exactly the elements above 448
    saturate to 0x7E | sign, the rest stay within the format's bound."""
    rng = np.random.default_rng(8)
    G = 32
    for _ in range(30):
        mags = np.exp2(rng.uniform(-20, 20, (8, 1)))
        x = (rng.standard_normal((8, G)) * mags).reshape(-1).astype(np.float32)
        xb = si.to_bf16_bits(x)
        xv = f32_from_bits(xb.astype(np.uint32) << 16).astype(np.float64)
        q, s = ora.quant_row(xb, G, rule="ocp_floor")
        e = np.repeat(s.astype(np.int64) - 127, G)
        y = xv / np.exp2(e.astype(float))
        assert (np.abs(y) < 512).all()
        sat = np.abs(y) > 448
        assert ((q[sat] & 0x7F) == 0x7E).all()
        deq = torch.from_numpy(q).view(torch.float8_e4m3fn).to(
            torch.float64).numpy()
        ok = ~sat
        tol = np.maximum(np.abs(y[ok]) * 2.0 ** -4, 2.0 ** -10)
        assert (np.abs(deq[ok] - y[ok]) <= tol).all()


def test_ocp_rule_clips_where_ceil_does_not(ora):
    x = np.zeros(32, np.float32)
    x[3] = 460.0
    x[9] = -1.0
    xb = si.to_bf16_bits(x)
    q, s = ora.quant_row(xb, 32, rule="ocp_floor")
    assert s[0] == 127 and q[3] == 0x7E            # 460 clipped to 448
    q2, s2 = ora.quant_row(xb, 32, rule="ceil")
    assert s2[0] == 128 and q2[3] == 0x76          # 460 / 2 = 230 -> 224
    for k in (-30, 0, 11):
        y = np.zeros(32, np.float32)
        y[0] = 448.0 * 2.0 ** k                    # both rules agree here
        qa, sa = ora.quant_row(si.to_bf16_bits(y), 32, rule="ocp_floor")
        qb, sb = ora.quant_row(si.to_bf16_bits(y), 32, rule="ceil")
        assert sa[0] == sb[0] == k + 127 and qa[0] == qb[0] == 0x7E


@pytest.mark.parametrize("G,H", [(32, 7168), (32, 96), (128, 640)])
def test_packed_mn_layout(ora, G, H):
    """Four scale bytes per 32-bit word, rows contiguous (MN-major), row
    count aligned to four: unpacking by the word/byte formula gives back
    the row-major scales, unused bytes keep their fill."""
    rng = np.random.default_rng(H)
    T, E = 41, 6
    x = si.gaussian_bf16(rng, (T, H))
    ids = si.uniform_topk(rng, T, 8, 3)
    lay = ora.moe_layout(ids, 0, E, "compact", block_e=8)
    R = lay["num_rows"]
    q1, s_rows = ora.scatter_quant_ex(x, lay["src2dst"], G, R, "ceil", "rows")
    ng = H // G
    nk, ld_mn = -(-ng // 4), -(-R // 4) * 4
    packed0 = np.full((nk, ld_mn), 0xA5A5A5A5, np.uint32)
    q2, packed = ora.scatter_quant_ex(x, lay["src2dst"], G, R, "ceil",
                                      "packed_mn", s=packed0.copy())
    assert np.array_equal(q1, q2)
    live = lay["m_indices"] >= 0
    for r in np.flatnonzero(live)[:50]:
        for g in range(ng):
            word = int(packed[g // 4, r])
            assert (word >> (8 * (g % 4))) & 0xFF == s_rows[r, g]
    un = ora.unpack_mn_scales(packed, R, ng)
    assert np.array_equal(un[live], s_rows[live])
    if ng % 4:
        pad = (packed[nk - 1, np.flatnonzero(live)] >> (8 * (ng % 4)))
        full = 0xA5A5A5A5 >> (8 * (ng % 4))
        assert (pad == full).all()

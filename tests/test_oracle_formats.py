"""Pins for the oracle's number formats: e4m3fn codec, bf16 rounding and the
power-of-two group scale.  Each is checked against something other than the
oracle itself: torch's own dtype casts, exact rational arithmetic, and values
fixed by the format definitions or stated on the pages."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")


def f32_from_bits(w):
    return np.asarray(w, np.uint32).view(np.float32)


def torch_e4m3(y: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(y, np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def torch_e4m3_decode(b: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(b, np.uint8)).view(
        torch.float8_e4m3fn).to(torch.float64).numpy()


def e4m3_grid():
    """All finite non-negative e4m3fn values, from torch's decoder."""
    v = torch_e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    return np.unique(v)


# ------------------------------------------------------------------- decode

def test_decode_all_bytes_matches_torch(ora):
    b = np.arange(256, dtype=np.uint8)
    mine = ora.e4m3_decode(b)
    ref = torch_e4m3_decode(b)
    nan = np.isnan(ref)
    assert set(np.flatnonzero(nan)) == {0x7F, 0xFF}
    assert np.isnan(mine[nan]).all()
    assert np.array_equal(mine[~nan], ref[~nan])
    # signed zero kept
    assert math.copysign(1.0, mine[0x80]) == -1.0


def test_decode_format_fixed_points(ora):
    facts = json.load(open(GOLDEN))
    d = ora.e4m3_decode(np.array([0x7E, 0x01, 0x08, 0x38, 0xFE], np.uint8))
    assert d[0] == facts["e4m3_max_finite"]["value"] == 448.0
    assert d[1] == 2.0 ** -9          # smallest subnormal
    assert d[2] == 2.0 ** -6          # smallest normal
    assert d[3] == 1.0
    assert d[4] == -448.0


# ------------------------------------------------------------------- encode

def test_encode_roundtrip_every_finite_byte(ora):
    b = np.array([i for i in range(256) if i not in (0x7F, 0xFF)], np.uint8)
    vals = ora.e4m3_decode(b).astype(np.float32)
    assert np.array_equal(ora.e4m3_encode(vals), b)


def test_encode_fixed_values(ora):
    cases = {
        448.0: 0x7E, 449.0: 0x7E, 463.9: 0x7E, 464.0: 0x7E, 1e30: 0x7E,
        float("inf"): 0x7E, -448.0: 0xFE, -1e30: 0xFE,
        2.0 ** -10: 0x00, 1.5 * 2.0 ** -10: 0x01, -0.0: 0x80,
        -(2.0 ** -12): 0x80, 2.0 ** -9: 0x01, 2.0 ** -6: 0x08, 1.0: 0x38,
        1.0625: 0x38,  # tie between 1.0 and 1.125 -> even mantissa (1.0)
        1.1875: 0x3A,  # tie between 1.125 (odd) and 1.25 (even) -> 1.25
        240.0: 0x77, 256.0: 0x78, 432.0: 0x7E,  # 432 ties 416/448 -> 448 (even)
    }
    ys = np.array(list(cases.keys()), np.float32)
    got = ora.e4m3_encode(ys)
    want = np.array(list(cases.values()), np.uint8)
    assert np.array_equal(got, want), list(zip(ys, got, want))


def test_encode_nan(ora):
    got = ora.e4m3_encode(np.array([np.nan, -np.nan], np.float32))
    assert (got & 0x7F).tolist() == [0x7F, 0x7F]


def test_encode_matches_torch_strided_sweep(ora):
    """Every 1021st binary32 pattern below 464, both signs, against torch's
    float32 -> float8_e4m3fn cast (round to nearest even).  Above 464 torch
    returns NaN while the oracle saturates, so that range is not compared."""
    top = int(np.float32(464.0).view(np.uint32))
    w = np.arange(0, top, 1021, dtype=np.uint32)
    y = f32_from_bits(w)
    y = np.concatenate([y, -y])
    assert np.array_equal(ora.e4m3_encode(y), torch_e4m3(y))


def test_encode_matches_torch_at_midpoints(ora):
    """Exact midpoints between neighbouring grid values and the floats just
    beside them: the cases where a wrong tie rule or an off-by-one shows."""
    g = e4m3_grid()
    g = np.concatenate([g, [480.0]])  # the value after 448 if the grid went on
    mids = ((g[:-1] + g[1:]) / 2).astype(np.float32)
    mids = mids[mids < 464.0]
    lo = np.nextafter(mids, np.float32(-np.inf))
    hi = np.nextafter(mids, np.float32(np.inf))
    y = np.concatenate([mids, lo, hi, g[:-1].astype(np.float32)])
    y = np.concatenate([y, -y])
    assert np.array_equal(ora.e4m3_encode(y), torch_e4m3(y))


def test_encode_subnormal_binary32_inputs(ora):
    y = f32_from_bits(np.array([1, 2, 0x7FFFFF, 0x800000], np.uint32))
    y = np.concatenate([y, -y])
    assert np.array_equal(ora.e4m3_encode(y), torch_e4m3(y))


# --------------------------------------------------------------------- bf16

def test_bf16_round_matches_torch(ora):
    rng = np.random.default_rng(7)
    w = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(
        np.uint32)
    # ties and near-ties: low half 0x8000 and 0x7FFF / 0x8001
    base = rng.integers(0, 2 ** 16, size=20_000, dtype=np.uint32) << 16
    ties = np.concatenate([base | 0x8000, base | 0x7FFF, base | 0x8001])
    w = np.concatenate([w, ties, np.array([0x7F7F8000, 0x7F7FFFFF, 0x00008000,
                                           0x80008000], np.uint32)])
    x = f32_from_bits(w)
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy(
    ).view(np.uint16)
    assert np.array_equal(ora.bf16_round(x), ref)


# ------------------------------------------------------ power-of-two scale

def exact_scale_exponent(amax: float) -> int:
    """Smallest integer e with amax <= 448 * 2^e, in exact rationals."""
    a = Fraction(amax)
    if a == 0:
        return -127
    e = 0
    while Fraction(448) * Fraction(2) ** e < a:
        e += 1
    while Fraction(448) * Fraction(2) ** (e - 1) >= a:
        e -= 1
    return max(-127, min(127, e))


def test_scale_exponent_every_positive_bf16(ora):
    """All 32639 positive finite bf16 values (and zero) against exact rational
    arithmetic.  Also pins the unclamped exponent range over bf16,
    -141 ... 120, so the -127 clamp is live for tiny groups."""
    bits = np.arange(0, 0x7F80, dtype=np.uint32) << 16
    vals = f32_from_bits(bits).astype(np.float64)
    got = np.array([ora.pow2_scale_exponent(v) for v in vals])
    # exact rule via integer frexp: amax = m * 2^k with m odd integer
    want = np.array([exact_scale_exponent(v) for v in vals[::37]])
    assert np.array_equal(got[::37], want)
    # every value: definition holds (upper) and is minimal (lower) unless clamped
    for v, e in zip(vals, got):
        if v == 0:
            assert e == -127
            continue
        assert v <= 448.0 * 2.0 ** e
        if e > -127:
            assert v > 448.0 * 2.0 ** (e - 1)
    nz = vals > 0
    raw = np.ceil(np.log2(vals[nz] / 448.0))
    assert raw.min() == -141 and raw.max() == 120
    assert got.min() == -127 and got.max() == 120


def test_scale_exponent_powers_of_two_times_448(ora):
    for k in range(-120, 121, 7):
        assert ora.pow2_scale_exponent(448.0 * 2.0 ** k) == k
        assert ora.pow2_scale_exponent(np.nextafter(448.0 * 2.0 ** k,
                                                    np.inf)) == k + 1


# ------------------------------------------------------------ group quant

def _bf16_vals(bits):
    return f32_from_bits(np.asarray(bits, np.uint32) << 16).astype(np.float64)


def _check_bound(x_bits, q, s, G):
    """|dec(q)*2^e - x| <= max(2^-4 |x|, 2^(e-10)) and |x / 2^e| <= 448, with
    dec from torch's fp8 decoder."""
    x = _bf16_vals(x_bits)
    H = x.shape[0]
    e = s.astype(np.int64) - 127
    ee = np.repeat(e, G)[:H]
    deq = torch_e4m3_decode(q) * np.exp2(ee.astype(np.float64))
    err = np.abs(deq - x)
    tol = np.maximum(np.abs(x) * 2.0 ** -4, np.exp2((ee - 10).astype(
        np.float64)))
    assert (err <= tol).all()
    assert (np.abs(x) / np.exp2(ee.astype(np.float64)) <= 448.0).all()


@pytest.mark.parametrize("G", [32, 128])
def test_quant_row_error_bound(ora, G):
    rng = np.random.default_rng(11)
    from synthetic_inputs import to_bf16_bits
    for trial in range(20):
        mags = np.exp2(rng.uniform(-30, 30, size=(1024 // G, 1)))
        x = (rng.standard_normal((1024 // G, G)) * mags).reshape(-1)
        xb = to_bf16_bits(x.astype(np.float32))
        q, s = ora.quant_row(xb, G)
        _check_bound(xb, q, s, G)


def test_quant_row_exact_448_powers(ora):
    """x = +-448 * 2^k maps to 0x7E | sign with scale byte k + 127."""
    from synthetic_inputs import to_bf16_bits
    for k in (-100, -3, 0, 5, 100):
        x = np.zeros(128, np.float32)
        x[17] = 448.0 * 2.0 ** k
        x[90] = -448.0 * 2.0 ** k
        q, s = ora.quant_row(to_bf16_bits(x), 128)
        assert s[0] == k + 127
        assert q[17] == 0x7E and q[90] == 0xFE


def test_quant_row_zero_and_subnormal_groups(ora):
    """An all-zero group gets byte 0 (e = -127) and zero payload with signs
    kept; a group of bf16 subnormals is clamped to e = -127 and still
    encodes to non-zero bytes (x * 2^127 lies in the e4m3 range)."""
    xb = np.zeros(96, np.uint16)
    xb[32:64] = 0x8000            # -0.0
    xb[64:96] = np.arange(1, 33, dtype=np.uint16)  # bf16 subnormals
    xb[70] |= 0x8000
    q, s = ora.quant_row(xb, 32)
    assert s.tolist() == [0, 0, 0]
    assert (q[:32] == 0).all() and (q[32:64] == 0x80).all()
    assert (q[64:96] & 0x7F != 0).all()
    assert q[70] & 0x80
    _check_bound(xb, q, s, 32)


def test_page_constants(ora):
    """7168 / 32 = 224 one-byte scales, 7168 / 128 = 56, and an empty live
    batch gives a (0, 224) scale view."""
    facts = json.load(open(GOLDEN))
    H = facts["mx_hidden_and_scales"]["hidden"]
    G = facts["mx_group_size"]["value"]
    xb = np.zeros(H, np.uint16)
    _, s = ora.quant_row(xb, G)
    assert s.shape == (facts["mx_hidden_and_scales"]["scales_per_row"],)
    assert s.dtype.itemsize == facts["e8m0_scale_bytes"]["value"]
    _, s128 = ora.quant_row(xb, facts["ue8m0_group_size"]["value"])
    assert s128.shape == (facts["ue8m0_group_size"]["scales_per_row_at_7168"],)
    live = np.zeros(2, np.int32)
    x = np.zeros((2 * 4, H), np.uint16)
    q, sc = ora.mx_quant_live_rows(x, 2, live, G)
    rows = [r for g in range(2) for r in range(g * 4, g * 4 + int(live[g]))]
    assert sc[rows].shape == tuple(facts["empty_batch_scale_shape"]["value"])
    buf = facts["padded_receive_buffer"]
    assert buf["rows_per_segment"] * buf["segments"] == buf["rows"]


def test_direct_power_of_two_scale_avoids_double_error(ora):
    """Quantizing with an fp32 scale amax/448 and then rounding that scale up
    to a power of two (keeping the payload) misrepresents values by up to a
    factor of two; the direct power-of-two quantization stays inside the
    format's error bound on the same data."""
    from synthetic_inputs import to_bf16_bits
    rng = np.random.default_rng(3)
    x = rng.standard_normal(128).astype(np.float32) * 3.3
    xb = to_bf16_bits(x)
    xv = _bf16_vals(xb)
    q, s = ora.quant_row(xb, 128)
    _check_bound(xb, q, s, 128)
    amax = np.abs(xv).max()
    s_f32 = amax / 448.0
    q_ind = torch_e4m3(xv / s_f32)
    s_pow2 = 2.0 ** math.ceil(math.log2(s_f32))
    deq_ind = torch_e4m3_decode(q_ind) * s_pow2
    rel = np.abs(deq_ind - xv) / np.abs(xv)
    assert rel.max() > 2 * 2.0 ** -4          # breaks the bound
    assert np.isclose(np.median(deq_ind / xv), s_pow2 / s_f32, rtol=0.07)
    deq = torch_e4m3_decode(q) * 2.0 ** (int(s[0]) - 127)
    big = np.abs(xv) > amax / 8
    assert (np.abs(deq - xv)[big] / np.abs(xv)[big]).max() <= 2.0 ** -4

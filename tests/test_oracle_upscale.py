"""Pins for the oracle's receive-side upscale (fp8 + group fp32 scales ->
bf16) and its single rounding of an exact product to bf16.

The reference rounding here is independent of the oracle's: a sorted table
of every finite bf16 value is searched for the two neighbours of the exact
product (the float64 distances to them are exact: the product has at most 28
significant bits), and a tie goes to the even bit pattern."""
import numpy as np
import pytest
import torch


def bf16_table():
    bits = np.arange(0, 0x7F81, dtype=np.uint32)          # +0 .. +inf
    vals = (bits << 16).view(np.float32).astype(np.float64)
    return bits.astype(np.uint16), vals


BITS, VALS = bf16_table()


def nearest_bf16(x: np.ndarray) -> np.ndarray:
    """Round exact float64 values to bf16 bits: nearest, ties to even,
    overflow to inf, NaN -> 0x7FC0."""
    x = np.asarray(x, np.float64)
    a = np.abs(x)
    i = np.clip(np.searchsorted(VALS, a, side="right") - 1, 0, len(VALS) - 2)
    lo, hi = VALS[i], VALS[i + 1]
    hi_fin = np.where(np.isinf(hi), 2.0 ** 128, hi)        # inf as 2^128
    dlo, dhi = a - lo, hi_fin - a
    up = (dhi < dlo) | ((dhi == dlo) & (BITS[i] & 1 == 1))
    mag = np.where(up, BITS[i + 1], BITS[i]).astype(np.uint16)
    mag = np.where(a >= 2.0 ** 128, 0x7F80, mag)
    mag = np.where(a == lo, BITS[i], mag)
    out = mag | np.where(np.signbit(x), 0x8000, 0).astype(np.uint16)
    return np.where(np.isnan(x), 0x7FC0, out).astype(np.uint16)


def torch_decode(q: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(q, np.uint8)).view(
        torch.float8_e4m3fn).to(torch.float64).numpy()


def test_bf16_round_f64_against_table(ora):
    rng = np.random.default_rng(1)
    x = rng.standard_normal(20000) * np.exp2(rng.uniform(-140, 130, 20000))
    # exact ties and their neighbours
    base = VALS[rng.integers(1, 0x7F7F, 2000)]
    nxt = (base.astype(np.float32).view(np.uint32) + 0x10000).view(
        np.float32).astype(np.float64)
    mid = (base + nxt) / 2
    x = np.concatenate([x, mid, np.nextafter(mid, 0), np.nextafter(mid, 1e300),
                        -mid, [0.0, -0.0, np.inf, -np.inf, np.nan,
                               2.0 ** 128, 3.3961e38, 2.0 ** -134,
                               2.0 ** -134 * 1.0000001, 2.0 ** -135]])
    assert np.array_equal(ora.bf16_round_f64(x), nearest_bf16(x))


def test_bf16_round_f64_matches_float_rounding(ora):
    """On inputs that are float32 values the double rounding function agrees
    with the float one (two different constructions)."""
    rng = np.random.default_rng(2)
    w = rng.integers(0, 0xFFFFFFFF, 50000, dtype=np.uint64).astype(np.uint32)
    f = w.view(np.float32)
    f = f[np.isfinite(f)]
    assert np.array_equal(ora.bf16_round_f64(f.astype(np.float64)),
                          ora.bf16_round(f))


def test_every_byte_times_powers_of_two(ora):
    """Every e4m3 byte times 2^k is exactly representable in bf16 (4
    significant bits), so the upscale returns the decoded value itself; the
    NaN bytes give 0x7FC0."""
    q = np.tile(np.arange(256, dtype=np.uint8), (41, 1))
    k = np.arange(-20, 21)
    s = np.exp2(k).astype(np.float32)[:, None].repeat(2, axis=1)  # H=256, G=128
    out = ora.upscale_fp8(q, s)
    ref = torch.from_numpy(torch_decode(q) * np.exp2(k)[:, None]).to(
        torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(
        np.uint16)
    nan = np.isin(np.arange(256), [0x7F, 0xFF])
    assert np.array_equal(out[:, ~nan], ref[:, ~nan])
    assert (out[:, nan] == 0x7FC0).all()


def test_random_scales_round_once(ora):
    rng = np.random.default_rng(3)
    rows, H, G = 37, 384, 128
    q = rng.integers(0, 256, (rows, H), dtype=np.uint8)
    q[q == 0x7F] = 0x7E
    q[q == 0xFF] = 0xFE
    s = (rng.uniform(0.5, 2, (rows, H // G)) *
         np.exp2(rng.integers(-30, 10, (rows, H // G)))).astype(np.float32)
    out = ora.upscale_fp8(q, s)
    exact = torch_decode(q) * np.repeat(s.astype(np.float64), G, axis=1)
    assert np.array_equal(out, nearest_bf16(exact))


def double_rounding_traps(rng, n=64):
    """(byte, scale) pairs whose float32 product lies exactly on a bf16
    midpoint while the exact product does not: rounding the float32 product
    to bf16 would go the wrong way on about half of them."""
    a = 3.0                                         # byte 0x44
    out = []
    while len(out) < n:
        m = VALS[rng.integers(0x3000, 0x5000)]
        nxt = (np.float32(m).view(np.uint32) + 0x10000).view(np.float32)
        mid = (m + float(nxt)) / 2
        b0 = np.float32(mid / a)
        for d in range(-3, 4):
            b = (b0.view(np.uint32) + np.uint32(d) if d >= 0 else
                 b0.view(np.uint32) - np.uint32(-d)).view(np.float32)
            exact = a * float(b)                     # exact in float64
            if float(np.float32(exact)) == mid and exact != mid:
                out.append((0x44, b, exact))
                break
    return out


def test_double_rounding_traps(ora):
    rng = np.random.default_rng(4)
    traps = double_rounding_traps(rng)
    q = np.array([[t[0]] * 128 for t in traps], np.uint8)
    s = np.array([[t[1]] for t in traps], np.float32)
    exact = np.array([t[2] for t in traps])
    got = ora.upscale_fp8(q, s)[:, 0]
    want = nearest_bf16(exact)
    assert np.array_equal(got, want)
    naive = torch.from_numpy(exact.astype(np.float32)).to(
        torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (naive != want).sum() >= len(traps) // 4   # the traps are real


def test_rows_past_count_untouched_and_scale_strides(ora):
    rng = np.random.default_rng(5)
    rows, H = 20, 512
    q = rng.integers(0, 0x7E, (rows, H), dtype=np.uint8)
    s = rng.uniform(1e-3, 1e-1, (rows, H // 128)).astype(np.float32)
    canary = np.full((rows, H), 0x1234, np.uint16)
    out = ora.upscale_fp8(q, s, num_rows=13, out=canary.copy())
    assert (out[13:] == 0x1234).all()
    full = ora.upscale_fp8(q, s)
    assert np.array_equal(out[:13], full[:13])
    colmaj = ora.upscale_fp8(q, np.ascontiguousarray(s.T),
                             scales_col_major=True)
    assert np.array_equal(colmaj, full)

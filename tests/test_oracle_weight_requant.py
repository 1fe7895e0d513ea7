"""Pins for the oracle's weight-side UE8M0 block requant: block-scaled fp8
weights -> bf16 -> fp8 with one power-of-two (UE8M0) scale per 128 x 128
block."""
import numpy as np
import pytest
import torch

from test_oracle_upscale import nearest_bf16, torch_decode


def synthetic_weights(rng, B, N, K, bn=128, bk=128):
    """e4m3 weights quantized per block with an fp32 inverse scale
    amax/448 (the usual block-fp8 checkpoint convention): bytes of a
    Gaussian weight divided by its block scale."""
    nbn, nbk = -(-N // bn), -(-K // bk)
    w = rng.standard_normal((B, N, K)) * 0.02
    s = np.empty((B, nbn, nbk), np.float32)
    q = np.empty((B, N, K), np.uint8)
    for b in range(B):
        for i in range(nbn):
            for j in range(nbk):
                blk = w[b, i * bn:(i + 1) * bn, j * bk:(j + 1) * bk]
                s[b, i, j] = np.float32(np.abs(blk).max() / 448.0)
                y = torch.from_numpy((blk / s[b, i, j]).astype(np.float32))
                q[b, i * bn:(i + 1) * bn, j * bk:(j + 1) * bk] = y.clamp(
                    -448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return q, s


def reference(q, s, bn=128, bk=128):
    """Independent construction: torch decode, exact product, table rounding
    to bf16, the smallest power of two 2^e with amax <= 448 * 2^e found by
    search, torch's fp8 cast of w / 2^e."""
    B, N, K = q.shape
    nbn, nbk = s.shape[1:]
    sf = np.repeat(np.repeat(s.astype(np.float64), bn, 1), bk, 2)[:, :N, :K]
    wb = nearest_bf16(torch_decode(q) * sf)
    w = (wb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    q_out = np.empty_like(q)
    s_out = np.empty((B, nbn, nbk), np.uint8)
    for b in range(B):
        for i in range(nbn):
            for j in range(nbk):
                blk = w[b, i * bn:(i + 1) * bn, j * bk:(j + 1) * bk]
                amax = np.abs(blk).max()
                e = -127
                while e < 127 and amax > 448.0 * 2.0 ** e:
                    e += 1
                s_out[b, i, j] = e + 127
                y = torch.from_numpy((blk * 2.0 ** -e).astype(np.float32))
                q_out[b, i * bn:(i + 1) * bn, j * bk:(j + 1) * bk] = y.to(
                    torch.float8_e4m3fn).view(torch.uint8).numpy()
    return q_out, s_out


@pytest.mark.parametrize("B,N,K", [(2, 256, 384), (3, 200, 72), (1, 1, 16),
                                   (1, 129, 257)])
def test_against_independent_reference(ora, B, N, K):
    rng = np.random.default_rng(N * K + B)
    q, s = synthetic_weights(rng, B, N, K)
    # spread the block scales over many binades
    s = (s * np.exp2(rng.integers(-40, 40, s.shape))).astype(np.float32)
    got_q, got_s = ora.requant_weight_block_ue8m0(q, s)
    ref_q, ref_s = reference(q, s)
    assert np.array_equal(got_s, ref_s)
    assert np.array_equal(got_q, ref_q)


def test_power_of_two_blocks_are_fixed_points(ora):
    """A block already scaled by 2^k whose largest byte decodes above 224
    keeps its bytes and gets scale byte k + 127."""
    rng = np.random.default_rng(7)
    B, N, K = 2, 256, 256
    q = rng.integers(0, 0x7E, (B, N, K), dtype=np.uint8)
    q |= (rng.random((B, N, K)) < 0.5).astype(np.uint8) << 7
    q[:, ::128, ::128] = 0x7C                               # 320 in each block
    k = rng.integers(-30, 30, (B, 2, 2))
    s = np.exp2(k).astype(np.float32)
    got_q, got_s = ora.requant_weight_block_ue8m0(q, s)
    assert np.array_equal(got_q, q)
    assert np.array_equal(got_s.astype(int), k + 127)


def test_error_bound_and_scale_minimality(ora):
    rng = np.random.default_rng(8)
    q, s = synthetic_weights(rng, 2, 256, 256)
    got_q, got_s = ora.requant_weight_block_ue8m0(q, s)
    sf = np.repeat(np.repeat(s.astype(np.float64), 128, 1), 128, 2)
    w = torch_decode(q) * sf
    e = np.repeat(np.repeat(got_s.astype(np.int64) - 127, 128, 1), 128, 2)
    back = torch_decode(got_q) * np.exp2(e.astype(np.float64))
    # two roundings (bf16, then e4m3 at the block's power of two)
    tol = 2.0 ** -8 * np.abs(w) + (2.0 ** -4 * np.abs(w) + 2.0 ** -10 *
                                   np.exp2(e.astype(np.float64)))
    assert (np.abs(back - w) <= tol).all()
    for b in range(2):
        for i in range(2):
            for j in range(2):
                ex = int(got_s[b, i, j]) - 127
                blk = np.abs(w[b, i * 128:(i + 1) * 128, j * 128:(j + 1) * 128])
                amax = blk.max() * (1 + 2.0 ** -8)
                assert amax / 2.0 ** (ex - 1) > 448.0  # a smaller e clips
                wb = (nearest_bf16(blk).astype(np.uint32) << 16).view(
                    np.float32)
                assert wb.max() <= 448.0 * 2.0 ** ex     # nothing clipped
                assert (got_q[b, i * 128:(i + 1) * 128,
                              j * 128:(j + 1) * 128] & 0x7F).max() <= 0x7E


def test_all_zero_block(ora):
    q = np.zeros((1, 128, 128), np.uint8)
    q[0, 5, 5] = 0x80                                        # -0
    s = np.ones((1, 1, 1), np.float32)
    got_q, got_s = ora.requant_weight_block_ue8m0(q, s)
    assert got_s[0, 0, 0] == 0
    assert np.array_equal(got_q, q)

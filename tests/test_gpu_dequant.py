"""Receive-side upscale and weight-side UE8M0 block requant on the GPU
against the oracle: bf16 bits, fp8 bytes and scale bytes bit-exact; rows and
bytes a call should not write keep their canary."""
import numpy as np
import pytest
import torch

import fp8_mx_activation_amd as mxq
import synthetic_inputs as si
from gpu_util import CANARY, DEV, assert_equal, host, say
from test_oracle_upscale import double_rounding_traps

pytestmark = pytest.mark.gpu

CANARY16 = 0x1234


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def run_upscale(ora, q, s, n, G=128, col_major=False):
    rows, H = q.shape
    say("upscale", "rows=%d n=%d H=%d G=%d col_major=%s"
        % (rows, n, H, G, col_major))
    sd = torch.from_numpy(np.ascontiguousarray(s.T) if col_major else s).to(DEV)
    out = torch.full((rows, H), CANARY16, dtype=torch.int16,
                     device=DEV).view(torch.bfloat16)
    mxq.upscale_fp8_to_bf16(torch.from_numpy(q).to(DEV), sd, n, group=G,
                            scales_col_major=col_major, out=out)
    torch.cuda.synchronize()
    ref = ora.upscale_fp8(q, s, num_rows=n, G=G,
                          out=np.full((rows, H), CANARY16, np.uint16))
    assert_equal(bf16_bits(out), ref, "bf16 bits")


def test_every_byte_every_scale_kind(ora):
    """All 256 bytes against scales of every kind: powers of two, random
    values over many binades, scales below 2^-90 (the exact small-product
    path), subnormal scales, scales that overflow bf16, and the
    double-rounding cases where the fp32 product sits on a bf16 midpoint."""
    rng = np.random.default_rng(11)
    scales = np.concatenate([
        np.exp2(np.arange(-40, 41, dtype=np.float64)),
        rng.uniform(0.5, 2, 200) * np.exp2(rng.integers(-80, 80, 200)),
        rng.uniform(0.5, 2, 40) * np.exp2(rng.integers(-126, -88, 40)),
        np.array([2.0 ** -149, 2.0 ** -140, 1e-40, 1e-39, 2.0 ** -91,
                  2.0 ** -90, 2.0 ** -89, 1e36, 3e37, 1e38, 3.4e38]),
    ]).astype(np.float32)
    rows = len(scales)
    q = np.tile(np.arange(256, dtype=np.uint8), (rows, 1))
    s = np.repeat(scales[:, None], 2, axis=1)            # H=256, G=128
    run_upscale(ora, q, s, rows)
    traps = double_rounding_traps(rng, 128)
    qt = np.array([[t[0]] * 128 for t in traps], np.uint8)
    st = np.array([[t[1]] for t in traps], np.float32)
    run_upscale(ora, qt, st, len(traps))


@pytest.mark.parametrize("G,H,rows,n,col_major", [
    (128, 7168, 300, 257, False), (128, 7168, 300, 300, True),
    (32, 96, 70, 33, False), (32, 7168, 64, 64, True), (128, 128, 5, 0, False),
    (128, 16384 + 128, 9, 7, False)])
def test_upscale_shapes(ora, G, H, rows, n, col_major):
    rng = np.random.default_rng(H + rows)
    q = si.random_e4m3_bytes(rng, (rows, H))
    s = si.group_scales_f32(rng, (rows, H // G))
    run_upscale(ora, q, s, n, G, col_major)


def test_upscale_fp8_dispatch_full(ora):
    """The 3072 x 8 padded receive buffer (24576 x 7168) upscaled over its
    first 8192 rows, every element compared; the rest keep the canary."""
    b = si.fp8_dispatch()
    run_upscale(ora, b.q, b.scales, b.num_local_tokens)


def run_weights(ora, q, s, inplace=False):
    B, N, K = q.shape
    say("weight requant", "B=%d N=%d K=%d inplace=%s" % (B, N, K, inplace))
    qd = torch.from_numpy(q).to(DEV)
    sd = torch.from_numpy(s).to(DEV)
    nbn, nbk = s.shape[1:]
    so = torch.full((B, nbn, nbk), CANARY, dtype=torch.uint8, device=DEV)
    if inplace:
        qo, so = mxq.requant_weight_block_ue8m0(qd, sd, scales_out=so,
                                                inplace=True)
        assert qo.data_ptr() == qd.data_ptr()
    else:
        qo, so = mxq.requant_weight_block_ue8m0(qd, sd, scales_out=so)
    torch.cuda.synchronize()
    ref_q, ref_s = ora.requant_weight_block_ue8m0(q, s)
    assert_equal(host(so), ref_s, "block scale bytes")
    assert_equal(host(qo), ref_q, "fp8 weights")


@pytest.mark.parametrize("B,N,K", [(2, 256, 384), (3, 200, 272), (1, 1, 16),
                                   (1, 129, 144), (4, 128, 128),
                                   (2, 256, 1408), (1, 300, 2064)])
def test_weight_requant_shapes(ora, B, N, K):
    """Ragged rows and columns; 1408 and 2064 columns mix whole 1024-column
    tiles with a partial one (and 300 rows a partial row band)."""
    q, s = si.block_weights(N * K + B, B, N, K)
    run_weights(ora, q, s)


def test_weight_requant_scale_extremes_and_in_place(ora):
    """Block scales over many binades, below 2^-90 (exact small-product
    path) and subnormal, and all-zero blocks; computed in place."""
    rng = np.random.default_rng(12)
    q, s = si.block_weights(13, 2, 384, 512)
    s = (s * np.exp2(rng.integers(-60, 60, s.shape))).astype(np.float32)
    s[0, 0, 0] = 2.0 ** -100
    s[0, 0, 1] = 1e-40
    s[1, 2, 3] = 2.0 ** -90
    q[1, 128:256, 256:384] = 0
    q[1, 0:128, 0:128] = 0x80
    run_weights(ora, q, s, inplace=True)


def test_weight_requant_gate_up_sample(ora):
    """The gate/up weights of 32 local experts [32, 4096, 7168] on the
    GPU; the oracle checks the first and last expert in full."""
    B, N, K = 32, 4096, 7168
    say("weight requant gate/up full", (B, N, K))
    qd = si.random_e4m3_bytes_device(si.SEEDS["block_weights"], (B, N, K),
                                     DEV)
    s = si.group_scales_f32(np.random.default_rng(si.SEEDS["block_weights"]),
                            (B, N // 128, K // 128), 2.0 ** -16, 2.0 ** -8)
    sd = torch.from_numpy(s).to(DEV)
    qo, so = mxq.requant_weight_block_ue8m0(qd, sd)
    torch.cuda.synchronize()
    for e in (0, 31):
        ref_q, ref_s = ora.requant_weight_block_ue8m0(host(qd[e]), s[e])
        assert_equal(host(so[e]), ref_s, "scales expert %d" % e)
        assert_equal(host(qo[e]), ref_q, "weights expert %d" % e)

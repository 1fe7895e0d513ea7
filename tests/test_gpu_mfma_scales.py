"""The block-scaled MFMA scale placement on the GPU.

1. moe_scatter_quant_ex and mx_quant_live_rows_ex with scale_layout
   "mfma32" / "mfma16" against the oracle (fp8 bytes and placed scale bytes
   bit-exact; bytes no call writes keep their canary), with ragged rows and
   block counts and the full prefill workload.
2. The placement read by the hardware: a test-only consumer
   (tests/mfma_consumer.hip) multiplies the quantized rows by an identity
   matrix with v_mfma_scale_f32_32x32x64_f8f6f4 / 16x16x128_f8f6f4, taking
   the scales straight from the placed bytes.  The result must equal the
   oracle's dequantized rows dec(q) * 2^(s - 127) exactly, element by
   element."""
import ctypes
import os

import numpy as np
import pytest
import torch

import fp8_mx_activation_amd as mxq
import synthetic_inputs as si
from gpu_util import (CANARY, DEV, assert_equal, bf16_to_dev, host,
                      i32_to_dev, say)
from test_gpu_scales import clip_band_bf16

pytestmark = pytest.mark.gpu

FMT = {128: "ue8m0_g128", 32: "e8m0_g32"}
ORA_RULE = {"no_clip": "ceil", "ocp_floor": "ocp_floor"}
HERE = os.path.dirname(os.path.abspath(__file__))


def canary_scales(rows, H, tm):
    return torch.full(tuple(mxq.mfma_scales(rows, H, tm, "cpu").shape),
                      CANARY, dtype=torch.uint8, device=DEV)


def run_scatter(ora, x, src2dst, R, G, rule, tm):
    T, H = x.shape
    say("scatter mfma%d" % tm, rule, "T=%d H=%d G=%d rows=%d" % (T, H, G, R))
    q = torch.full((R, H), CANARY, dtype=torch.uint8, device=DEV)
    s = canary_scales(R, H, tm)
    mxq.moe_scatter_quant_ex(bf16_to_dev(x), i32_to_dev(src2dst), R, FMT[G],
                             rule=rule, scale_layout="mfma%d" % tm, q=q,
                             scales=s)
    torch.cuda.synchronize()
    q_ref, s_rows = ora.scatter_quant_ex(
        x, src2dst, G, R, ORA_RULE[rule], "rows",
        q=np.full((R, H), CANARY, np.uint8),
        s=np.full((R, H // G), CANARY, np.uint8))
    assert_equal(host(q), q_ref, "fp8 bytes")
    assert_equal(host(s), ora.mfma_scales(s_rows, H, G, tm, fill=CANARY),
                 "placed scales")
    return q, s, q_ref, s_rows


@pytest.mark.parametrize("tm", [32, 16])
@pytest.mark.parametrize("rule", ["no_clip", "ocp_floor"])
@pytest.mark.parametrize("G,H", [(32, 96), (128, 640), (32, 7200),
                                 (128, 7168)])
def test_scatter_mfma_placement(ora, tm, rule, G, H):
    """Block counts 3, 20, 225 and 224 (whole and partial word groups);
    208 rows, six and a half tiles of 32."""
    rng = np.random.default_rng(H + tm + G)
    T, E = 53, 7
    x = clip_band_bf16(rng, T, H, G)
    ids = si.uniform_topk(rng, T, E, 3)
    lay = ora.moe_layout(ids, 0, E, "compact", block_e=8)
    assert lay["num_rows"] == 208
    run_scatter(ora, x, lay["src2dst"], lay["num_rows"], G, rule, tm)


@pytest.mark.parametrize("tm", [32, 16])
def test_mfma_placement_lookahead(ora, tm):
    """More tokens than the scatter's lookahead distance with the MFMA
    placement's token order (each XCD takes a contiguous range; 300 tokens
    make a grid of 304 blocks, so the last range is short), and zero to
    eight local destinations per token (16 of 32 experts local)."""
    rng = np.random.default_rng(303 + tm)
    T, H, G = 300, 2048, 128
    x = clip_band_bf16(rng, T, H, G)
    ids = si.uniform_topk(rng, T, 32, 8)
    lay = ora.moe_layout(ids, 0, 16, "compact", block_e=32)
    run_scatter(ora, x, lay["src2dst"], lay["num_rows"], G, "no_clip", tm)


@pytest.mark.parametrize("tm", [32, 16])
def test_prefill_mfma_placement(ora, tm):
    """The full prefill workload (8192 x 7168, 65536 assignments into 98048
    rows, UE8M0 group 128)."""
    b = si.prefill_compact()
    lay = ora.moe_layout(b.topk_ids, 0, 256, "compact")
    run_scatter(ora, b.x, lay["src2dst"], lay["num_rows"], 128, "no_clip",
                tm)


@pytest.mark.parametrize("tm", [32, 16])
@pytest.mark.parametrize("G,H,segs,rps", [(32, 7168, 8, 64), (128, 640, 3, 5),
                                          (32, 96, 1, 9)])
def test_live_rows_mfma_placement(ora, tm, G, H, segs, rps):
    rng = np.random.default_rng(segs * 10 + H + tm)
    rows = segs * rps
    x = clip_band_bf16(rng, rows, H, G)
    live = rng.integers(0, rps + 1, segs).astype(np.int32)
    live[0] = rps
    if segs > 1:
        live[-1] = 0
    say("live_rows mfma%d" % tm, "H=%d G=%d live=%s" % (H, G, live.tolist()))
    d = np.full((rows, 1), -1, np.int32)
    for g in range(segs):
        d[g * rps:g * rps + live[g], 0] = np.arange(g * rps, g * rps + live[g])
    q = torch.full((rows, H), CANARY, dtype=torch.uint8, device=DEV)
    s = canary_scales(rows, H, tm)
    mxq.mx_quant_live_rows_ex(bf16_to_dev(x), segs, i32_to_dev(live), FMT[G],
                              scale_layout="mfma%d" % tm, q=q, scales=s)
    torch.cuda.synchronize()
    q_ref, s_rows = ora.scatter_quant_ex(
        x, d, G, rows, "ceil", "rows", q=np.full((rows, H), CANARY, np.uint8),
        s=np.full((rows, H // G), CANARY, np.uint8))
    assert_equal(host(q), q_ref, "fp8 bytes")
    assert_equal(host(s), ora.mfma_scales(s_rows, H, G, tm, fill=CANARY),
                 "placed scales")


# ------------------------------------------------------ the hardware reads it

@pytest.fixture(scope="module")
def consumer():
    path = os.path.join(HERE, "libmfma_consumer.so")
    if not os.path.exists(path):
        pytest.fail("tests/libmfma_consumer.so is not built "
                    "(__graft_entry__.build() builds it)")
    L = ctypes.CDLL(path)
    f = L.mfma_identity_dequant
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                  ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                  ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64,
                  ctypes.c_void_p]

    def run(q, s, tm):
        rows, H = q.shape
        assert q.is_contiguous() and q.dtype == torch.uint8
        assert s.is_contiguous() and s.numel() == \
            mxq.mxq_mfma_scale_bytes(rows, H, tm)
        out = torch.full((rows, H), float("nan"), dtype=torch.float32,
                         device=DEV)
        rc = f(q.data_ptr(), H, s.data_ptr(), s.shape[1], rows, H, tm,
               out.data_ptr(), H, torch.cuda.current_stream().cuda_stream)
        assert rc == 0, rc
        torch.cuda.synchronize()
        return host(out)
    return run


def dequant(ora, q, s_rows, G):
    """dec(q) * 2^(s - 127), exact in fp64, then fp32 (exact here: every
    value is a normal fp32 number or zero)."""
    v = ora.e4m3_decode(q.reshape(-1)).reshape(q.shape)
    e = np.repeat(s_rows.astype(np.int64) - 127, G, axis=1)
    return np.ldexp(v, e).astype(np.float32)


@pytest.mark.parametrize("tm", [32, 16])
@pytest.mark.parametrize("G", [32, 128])
def test_mfma_reads_the_live_rows_placement(ora, consumer, tm, G):
    """All rows live (96 rows, hidden 1024, exponents over 2^-12..2^12)."""
    rng = np.random.default_rng(900 + tm + G)
    rows, H = 96, 1024
    x = clip_band_bf16(rng, rows, H, G)
    say("mfma consumer live rows", tm, G)
    q, s = mxq.mx_quant_live_rows_ex(
        bf16_to_dev(x), 1, i32_to_dev([rows]), FMT[G],
        scale_layout="mfma%d" % tm)
    got = consumer(q, s, tm)
    d = np.arange(rows, dtype=np.int32).reshape(rows, 1)
    q_ref, s_rows = ora.scatter_quant_ex(x, d, G, rows, "ceil", "rows")
    want = dequant(ora, q_ref, s_rows, G)
    assert np.abs(want[want != 0]).min() >= np.float32(2.0 ** -126)
    assert_equal(got, want, "MFMA dequant")


@pytest.mark.parametrize("tm", [32, 16])
def test_mfma_reads_the_scatter_placement(ora, consumer, tm):
    """The compact layout written by the scatter (block 128, so the row
    bound is a whole number of tiles): every destination row, read by the
    MFMA with its placed scales, equals the oracle's dequantized row."""
    rng = np.random.default_rng(77 + tm)
    T, H, E, K, G = 150, 2048, 6, 2, 128
    x = clip_band_bf16(rng, T, H, G)
    ids = si.uniform_topk(rng, T, E, K)
    ref = ora.moe_layout(ids, 0, E, "compact")
    R = ref["num_rows"]
    assert R % tm == 0
    say("mfma consumer scatter", tm, R)
    lay = mxq.moe_layout(i32_to_dev(ids), 0, E, "compact", num_rows=R)
    q = torch.zeros((R, H), dtype=torch.uint8, device=DEV)
    s = torch.full(tuple(mxq.mfma_scales(R, H, tm, "cpu").shape), 127,
                   dtype=torch.uint8, device=DEV)
    mxq.moe_scatter_quant_ex(bf16_to_dev(x), lay["src2dst"], R, FMT[G],
                             scale_layout="mfma%d" % tm, q=q, scales=s)
    got = consumer(q, s, tm)
    q_ref, s_rows = ora.scatter_quant_ex(
        x, ref["src2dst"], G, R, "ceil", "rows",
        q=np.zeros((R, H), np.uint8), s=np.full((R, H // G), 127, np.uint8))
    live = ref["m_indices"] >= 0
    assert live.sum() == T * K
    assert_equal(got[live], dequant(ora, q_ref, s_rows, G)[live],
                 "MFMA dequant of destination rows")

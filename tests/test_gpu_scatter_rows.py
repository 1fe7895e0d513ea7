"""moe_scatter_rows (the psum prefill path: a dispatcher's quantized rows and
scales written into the contiguous layout) on the GPU against the oracle,
bit-exact, with canaries on rows that are no destination."""
import numpy as np
import pytest
import torch

import fp8_mx_activation_amd as mxq
import synthetic_inputs as si
from gpu_util import CANARY, DEV, assert_equal, host, i32_to_dev, say, u8_to_dev

pytestmark = pytest.mark.gpu


def run(ora, x, s2d, R, sc=None, in_cm=False, out_cm=False):
    T, rb = x.shape
    say("scatter_rows", "T=%d row_bytes=%d rows=%d scales=%s in_cm=%s out_cm=%s"
        % (T, rb, R, None if sc is None else sc.dtype, in_cm, out_cm))
    out = torch.full((R, rb), CANARY, dtype=torch.uint8, device=DEV)
    sd = osd = None
    if sc is not None:
        cols = sc.shape[1]
        sd = torch.from_numpy(np.ascontiguousarray(sc.T) if in_cm else sc).to(DEV)
        canary_s = np.full((cols, R) if out_cm else (R, cols), 77, sc.dtype)
        osd = torch.from_numpy(canary_s.copy()).to(DEV)
    mxq.moe_scatter_rows(u8_to_dev(x), i32_to_dev(s2d), R, scales=sd,
                         scales_col_major=in_cm, out=out, out_scales=osd,
                         out_scales_col_major=out_cm)
    torch.cuda.synchronize()
    q_ref, s_ref = ora.scatter_rows(
        x, s2d, R,
        scales=None if sc is None else (np.ascontiguousarray(sc.T) if in_cm
                                        else sc),
        scales_col_major=in_cm, out=np.full((R, rb), CANARY, np.uint8),
        out_scales=None if sc is None else canary_s.copy(),
        out_scales_col_major=out_cm)
    assert_equal(host(out), q_ref, "rows")
    if sc is not None:
        assert_equal(host(osd), s_ref, "scales")
    return out, osd


@pytest.mark.parametrize("rb,cols,dt,in_cm,out_cm", [
    (7168, 56, np.uint8, False, False), (7168, 56, np.float32, True, False),
    (448, 7, np.float32, False, True), (16, 1, np.uint8, True, True),
    (32768, 0, None, False, False)])
def test_shapes(ora, rb, cols, dt, in_cm, out_cm):
    rng = np.random.default_rng(rb + cols)
    T, K, E = 211, 6, 20
    ids = si.uniform_topk(rng, T, 24, K)           # experts 20..23 non-local
    lay = ora.moe_layout(ids, 0, E, "compact", block_e=128)
    x = si.random_e4m3_bytes(rng, (T, rb))
    sc = None
    if dt is not None:
        sc = rng.integers(1, 250, (T, cols)).astype(dt)
    run(ora, x, lay["src2dst"], lay["num_rows"], sc, in_cm, out_cm)


@pytest.mark.parametrize("rb,cols,dt,in_cm,out_cm", [
    (49168, 130, np.uint8, False, False), (65584, 70, np.float32, True, True)])
def test_rows_over_one_chunk_and_many_scale_entries(ora, rb, cols, dt, in_cm,
                                                    out_cm):
    """Rows that pass through LDS in two and three chunks (32 KB, then a
    ragged tail), and more than 64 scale entries per row (entries past the
    first 64 are fetched by the writing wavefront)."""
    rng = np.random.default_rng(rb)
    T, K, E = 40, 6, 20
    ids = si.uniform_topk(rng, T, 24, K)
    lay = ora.moe_layout(ids, 0, E, "compact", block_e=1)
    x = si.random_e4m3_bytes(rng, (T, rb))
    sc = rng.integers(1, 250, (T, cols)).astype(dt)
    run(ora, x, lay["src2dst"], lay["num_rows"], sc, in_cm, out_cm)


def test_more_destinations_than_wavefronts(ora):
    """Top-20 routing: a token's destinations outnumber the block's eight
    wavefronts, so wavefronts write several rows each."""
    rng = np.random.default_rng(35)
    T, K, E = 50, 20, 30
    ids = si.uniform_topk(rng, T, 32, K)
    lay = ora.moe_layout(ids, 0, E, "compact", block_e=16)
    x = si.random_e4m3_bytes(rng, (T, 1024))
    sc = rng.integers(1, 250, (T, 8)).astype(np.uint8)
    run(ora, x, lay["src2dst"], lay["num_rows"], sc)


def test_prefill_quantized_rows_equal_fused_scatter(ora):
    """The full prefill workload: quantizing every token row (the sender's
    job) and scattering the fp8 rows and scale bytes gives exactly what the
    fused scatter+quant writes, and both equal the oracle."""
    b = si.prefill_compact()
    x = torch.from_numpy(b.x.view(np.int16)).view(torch.bfloat16).to(DEV)
    lay = mxq.moe_layout(torch.from_numpy(b.topk_ids).to(DEV), 0, 256,
                         "compact")
    R = lay["num_rows"]
    say("scatter_rows prefill", R)
    q_tok, s_tok = mxq.mx_quant_live_rows(
        x, 1, torch.tensor([b.T], dtype=torch.int32, device=DEV),
        fmt="ue8m0_g128")
    out = torch.full((R, b.H), CANARY, dtype=torch.uint8, device=DEV)
    osc = torch.full((R, b.H // 128), CANARY, dtype=torch.uint8, device=DEV)
    mxq.moe_scatter_rows(q_tok, lay["src2dst"], R, scales=s_tok, out=out,
                         out_scales=osc)
    q_f = torch.full((R, b.H), CANARY, dtype=torch.uint8, device=DEV)
    s_f = torch.full((R, b.H // 128), CANARY, dtype=torch.uint8, device=DEV)
    mxq.moe_scatter_quant(x, lay["src2dst"], R, q=q_f, scales=s_f)
    torch.cuda.synchronize()
    assert torch.equal(out, q_f) and torch.equal(osc, s_f)
    ref = ora.moe_layout(b.topk_ids, 0, 256, "compact")
    q_ref, s_ref = ora.scatter_rows(host(q_tok), ref["src2dst"], R,
                                    scales=host(s_tok),
                                    out=np.full((R, b.H), CANARY, np.uint8),
                                    out_scales=np.full((R, b.H // 128), CANARY,
                                                       np.uint8))
    assert_equal(host(out), q_ref, "rows")
    assert_equal(host(osc), s_ref, "scales")


def test_skips_and_empty(ora):
    x = np.arange(3 * 32, dtype=np.uint8).reshape(3, 32)
    d = np.array([[0, 5], [-1, 2], [7, 1]], np.int32)
    run(ora, x, d, 4)
    out, _ = mxq.moe_scatter_rows(torch.zeros((0, 32), dtype=torch.uint8,
                                              device=DEV),
                                  torch.zeros((0, 2), dtype=torch.int32,
                                              device=DEV), 4)
    torch.cuda.synchronize()
    assert out.shape == (4, 32)

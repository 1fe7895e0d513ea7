"""Scale variants on the GPU against the oracle: the OCP Microscaling floor
exponent rule (with clipping to +-448) and the packed MN-major placement of
scale bytes, through moe_scatter_quant_ex and mx_quant_live_rows_ex.  fp8
bytes and scale bytes bit-exact; bytes no call should write keep their
canary."""
import numpy as np
import pytest
import torch

import fp8_mx_activation_amd as mxq
import synthetic_inputs as si
from gpu_util import (CANARY, DEV, assert_equal, bf16_to_dev, host,
                      i32_to_dev, say)

pytestmark = pytest.mark.gpu

FMT = {128: "ue8m0_g128", 32: "e8m0_g32"}
ORA_RULE = {"no_clip": "ceil", "ocp_floor": "ocp_floor"}
CANARY32 = 0xA5A5A5A5


def clip_band_bf16(rng, T, H, G):
    """Gaussian rows whose group maxima are pushed, in a third of the
    groups, to a significand in [1.75, 2): there the floor rule gives a
    payload in [448, 512) that must clip, while the no-clip rule picks the
    next exponent."""
    x = rng.standard_normal((T, H)).astype(np.float32)
    x *= np.exp2(rng.integers(-12, 12, (T, 1))).astype(np.float32)
    g = x.reshape(T, H // G, G)
    pick = rng.random((T, H // G)) < 1 / 3
    col = rng.integers(0, G, (T, H // G))
    amax = np.abs(g).max(axis=2)
    e = np.floor(np.log2(np.maximum(amax, 1e-30)))
    sig = 1.75 + rng.random((T, H // G)) * 0.25
    sign = np.where(rng.random((T, H // G)) < 0.5, -1.0, 1.0)
    ti, gi = np.nonzero(pick)
    g[ti, gi, col[ti, gi]] = (sign * sig * np.exp2(e + 1))[ti, gi]
    return si.to_bf16_bits(g.reshape(T, H))


def packed_canary(rows, ng):
    return np.full((-(-ng // 4), -(-rows // 4) * 4), CANARY32, np.uint32)


def run_scatter(ora, x_bits, src2dst, R, G, rule, layout):
    T, H = x_bits.shape
    ng = H // G
    say("scatter_ex", rule, layout, "T=%d H=%d G=%d rows=%d" % (T, H, G, R))
    q = torch.full((R, H), CANARY, dtype=torch.uint8, device=DEV)
    if layout == "rows":
        s0 = np.full((R, ng), CANARY, np.uint8)
        s = torch.from_numpy(s0).to(DEV)
    else:
        s0 = packed_canary(R, ng)
        s = torch.from_numpy(s0.view(np.int32)).to(DEV)
    mxq.moe_scatter_quant_ex(bf16_to_dev(x_bits), i32_to_dev(src2dst), R,
                             FMT[G], rule=rule, scale_layout=layout, q=q,
                             scales=s)
    torch.cuda.synchronize()
    q_ref = np.full((R, H), CANARY, np.uint8)
    q_ref, s_ref = ora.scatter_quant_ex(x_bits, src2dst, G, R, ORA_RULE[rule],
                                        layout, q=q_ref, s=s0.copy())
    assert_equal(host(q), q_ref, "fp8 bytes")
    sh = host(s)
    if layout == "packed_mn":
        sh = sh.view(np.uint32)
    assert_equal(sh, s_ref, "scale words" if layout != "rows" else "scales")
    return q_ref, s_ref


@pytest.mark.parametrize("layout", ["rows", "packed_mn"])
@pytest.mark.parametrize("rule", ["no_clip", "ocp_floor"])
@pytest.mark.parametrize("G,H", [(32, 96), (128, 640), (32, 7168),
                                 (128, 7168), (32, 32 * 5)])
def test_scatter_variants(ora, rule, layout, G, H):
    """Ragged scale counts (3, 5 and 5 groups leave part of the last packed
    word unused) and the full hidden size, under both rules."""
    rng = np.random.default_rng(H * 7 + G)
    T, E = 53, 7
    x = clip_band_bf16(rng, T, H, G)
    ids = si.uniform_topk(rng, T, E, 3)
    lay = ora.moe_layout(ids, 0, E, "compact", block_e=8)
    run_scatter(ora, x, lay["src2dst"], lay["num_rows"], G, rule, layout)


def test_floor_rule_clips_on_gpu(ora):
    """A group whose maximum is 460: the floor rule keeps exponent 0 and
    clips 460 to 448 (byte 0x7E); the no-clip rule takes exponent 1."""
    x = np.zeros((1, 32), np.float32)
    x[0, 3], x[0, 9] = 460.0, -1.0
    xb = si.to_bf16_bits(x)
    d = np.zeros((1, 1), np.int32)
    q, s = run_scatter(ora, xb, d, 1, 32, "ocp_floor", "rows")
    assert s[0, 0] == 127 and q[0, 3] == 0x7E
    q, s = run_scatter(ora, xb, d, 1, 32, "no_clip", "rows")
    assert s[0, 0] == 128 and q[0, 3] == 0x76


@pytest.mark.parametrize("layout", ["rows", "packed_mn"])
@pytest.mark.parametrize("rule", ["no_clip", "ocp_floor"])
def test_prefill_full_variants(ora, rule, layout):
    """The full prefill workload (8192 x 7168, 65536 assignments into 98048
    rows) in the group-128 format under each rule and placement."""
    b = si.prefill_compact()
    lay = ora.moe_layout(b.topk_ids, 0, 256, "compact")
    run_scatter(ora, b.x, lay["src2dst"], lay["num_rows"], 128, rule, layout)


def test_default_entry_point_is_the_no_clip_row_case(ora):
    """moe_scatter_quant equals moe_scatter_quant_ex(no_clip, rows)."""
    rng = np.random.default_rng(5)
    x = clip_band_bf16(rng, 40, 1024, 128)
    ids = si.uniform_topk(rng, 40, 5, 2)
    lay = mxq.moe_layout(i32_to_dev(ids), 0, 5, "compact", block_e=16)
    xd = bf16_to_dev(x)
    R = lay["num_rows"]
    say("scatter default vs ex", R)
    q1, s1 = mxq.moe_scatter_quant(xd, lay["src2dst"], R, "ue8m0_g128",
                                   q=torch.zeros((R, 1024), dtype=torch.uint8,
                                                 device=DEV),
                                   scales=torch.zeros((R, 8),
                                                      dtype=torch.uint8,
                                                      device=DEV))
    q2, s2 = mxq.moe_scatter_quant_ex(
        xd, lay["src2dst"], R, "ue8m0_g128", "no_clip", "rows",
        q=torch.zeros((R, 1024), dtype=torch.uint8, device=DEV),
        scales=torch.zeros((R, 8), dtype=torch.uint8, device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(q1, q2) and torch.equal(s1, s2)


@pytest.mark.parametrize("layout", ["rows", "packed_mn"])
@pytest.mark.parametrize("rule", ["no_clip", "ocp_floor"])
@pytest.mark.parametrize("G,H,segs,rps", [(32, 7168, 8, 64), (128, 640, 3, 5),
                                          (32, 96, 1, 9)])
def test_live_rows_variants(ora, rule, layout, G, H, segs, rps):
    """Live rows only: row r of segment g is quantized when r < live[g].
    The oracle side is the scatter of token r to row r (K = 1), with -1 for
    rows past a segment's live count."""
    rng = np.random.default_rng(segs * 100 + H)
    rows = segs * rps
    x = clip_band_bf16(rng, rows, H, G)
    live = rng.integers(0, rps + 1, segs).astype(np.int32)
    live[0] = rps
    if segs > 1:
        live[-1] = 0
    say("live_rows_ex", rule, layout, "H=%d G=%d live=%s"
        % (H, G, live.tolist()))
    d = np.full((rows, 1), -1, np.int32)
    for g in range(segs):
        d[g * rps:g * rps + live[g], 0] = np.arange(g * rps,
                                                    g * rps + live[g])
    ng = H // G
    q = torch.full((rows, H), CANARY, dtype=torch.uint8, device=DEV)
    if layout == "rows":
        s0 = np.full((rows, ng), CANARY, np.uint8)
        s = torch.from_numpy(s0).to(DEV)
    else:
        s0 = packed_canary(rows, ng)
        s = torch.from_numpy(s0.view(np.int32)).to(DEV)
    mxq.mx_quant_live_rows_ex(bf16_to_dev(x), segs, i32_to_dev(live),
                              FMT[G], rule=rule, scale_layout=layout, q=q,
                              scales=s)
    torch.cuda.synchronize()
    q_ref, s_ref = ora.scatter_quant_ex(
        x, d, G, rows, ORA_RULE[rule], layout,
        q=np.full((rows, H), CANARY, np.uint8), s=s0.copy())
    assert_equal(host(q), q_ref, "fp8 bytes")
    sh = host(s)
    if layout == "packed_mn":
        sh = sh.view(np.uint32)
    assert_equal(sh, s_ref, "scales")

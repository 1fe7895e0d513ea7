"""moe_scatter_quant and mx_quant_live_rows on the GPU against the oracle:
fp8 bytes and scale bytes bit-exact, untouched rows keep their canary."""
import numpy as np
import pytest
import torch

import fp8_mx_activation_amd as mxq
import synthetic_inputs as si
from gpu_util import (CANARY, DEV, assert_equal, bf16_to_dev, host,
                      i32_to_dev, say)

pytestmark = pytest.mark.gpu

FMT = {128: "ue8m0_g128", 32: "e8m0_g32"}


def scatter_both(ora, x_bits, ids, E, kind, G, cap=0, ld_pad=(0, 0, 0),
                 block_e=128):
    """Layout on the GPU (checked against the oracle elsewhere), then the
    scatter on both sides with canary-filled outputs and optional padded
    row strides (x, q, scales)."""
    T, H = x_bits.shape
    ref_l = ora.moe_layout(ids, 0, E, kind, block_e=block_e, capacity=cap)
    R = ref_l["num_rows"]
    say("scatter", kind, "T=%d H=%d G=%d rows=%d pad=%s"
        % (T, H, G, R, ld_pad))
    lay = mxq.moe_layout(i32_to_dev(ids), 0, E, kind, block_e=block_e,
                         capacity=cap, num_rows=R)
    assert_equal(host(lay["src2dst"]), ref_l["src2dst"], "src2dst")
    px, pq, ps = ld_pad
    xd_full = torch.zeros((T, H + px), dtype=torch.bfloat16, device=DEV)
    xd_full[:, :H] = bf16_to_dev(x_bits)
    xd = xd_full[:, :H]
    q_full = torch.full((R, H + pq), CANARY, dtype=torch.uint8, device=DEV)
    s_full = torch.full((R, H // G + ps), CANARY, dtype=torch.uint8,
                        device=DEV)
    mxq.moe_scatter_quant(xd, lay["src2dst"], R, FMT[G], q=q_full[:, :H],
                          scales=s_full[:, :H // G])
    torch.cuda.synchronize()
    q_ref = np.full((R, H), CANARY, np.uint8)
    s_ref = np.full((R, H // G), CANARY, np.uint8)
    ora.scatter_quant(x_bits, ref_l["src2dst"], G, R, q_ref, s_ref)
    qh, sh = host(q_full), host(s_full)
    assert_equal(qh[:, :H], q_ref, "fp8 bytes")
    assert_equal(sh[:, :H // G], s_ref, "scale bytes")
    assert (qh[:, H:] == CANARY).all() and (sh[:, H // G:] == CANARY).all()
    return ref_l


def test_tiny(ora):
    b = si.tiny()
    scatter_both(ora, b.x, b.topk_ids, 8, "compact", 128)


def test_decode_masked(ora):
    b = si.decode_masked()
    scatter_both(ora, b.x, b.topk_ids, 32, "masked", 128, cap=128)


def test_decode_masked_g32(ora):
    b = si.decode_masked()
    scatter_both(ora, b.x, b.topk_ids, 32, "masked", 32, cap=128)


def test_prefill_compact_full(ora):
    """The full prefill workload: 8192 x 7168, 65536 assignments into 98048
    rows, every byte of every row compared (padding rows keep the canary)."""
    b = si.prefill_compact()
    scatter_both(ora, b.x, b.topk_ids, 256, "compact", 128)


@pytest.mark.parametrize("G,H", [(32, 96), (128, 640), (32, 7168 + 32),
                                 (128, 16384 + 128), (32, 32)])
def test_ragged_widths(ora, G, H):
    rng = np.random.default_rng(H)
    x = si.gaussian_bf16(rng, (45, H))
    ids = si.uniform_topk(rng, 45, 12, 3)
    scatter_both(ora, x, ids, 9, "compact", G, block_e=16)


@pytest.mark.parametrize("H,G,pad", [(7168, 128, (0, 0, 0)),
                                     (12288, 32, (8, 16, 3)),
                                     (16384 + 128, 128, (0, 0, 0)),
                                     (640, 32, (24, 0, 1))])
def test_lookahead_mixed_destinations(ora, H, G, pad):
    """More tokens than the scatter's lookahead distance (96 blocks), zero
    to eight local destinations per token (16 of 32 experts local, so some
    blocks look ahead and some do not), and widths whose idle wavefronts
    cover the whole next row (7168, 640), part of it (12288) or none
    (16512).  The lookahead only loads, so every byte still matches."""
    rng = np.random.default_rng(H + G)
    T = 300
    x = si.gaussian_bf16(rng, (T, H))
    ids = si.uniform_topk(rng, T, 32, 8)
    scatter_both(ora, x, ids, 16, "compact", G, ld_pad=pad, block_e=16)


def test_padded_strides(ora):
    rng = np.random.default_rng(5)
    x = si.gaussian_bf16(rng, (70, 640))
    ids = si.uniform_topk(rng, 70, 8, 4)
    scatter_both(ora, x, ids, 8, "compact", 128, ld_pad=(8, 48, 3))
    scatter_both(ora, x, ids, 8, "masked", 32, cap=64, ld_pad=(24, 16, 7))


def test_extreme_values(ora):
    """Zero groups, signed zeros, bf16 subnormals, the largest finite bf16,
    exact powers 448 * 2^k, mixed magnitudes inside one group."""
    H = 512
    rows = []
    rows.append(np.zeros(H, np.uint16))
    r = np.zeros(H, np.uint16)
    r[::2] = 0x8000
    rows.append(r)
    rows.append(np.arange(1, H + 1, dtype=np.uint16) & 0x807F)  # subnormals
    r = np.full(H, 0x7F7F, np.uint16)
    r[1::3] = 0xFF7F
    rows.append(r)                                               # max bf16
    r = np.zeros(H, np.float32)
    r[::5] = 448.0
    r[1::7] = -448.0 * 2.0 ** -20
    r[3::11] = 1e-30
    rows.append(si.to_bf16_bits(r))
    rng = np.random.default_rng(3)
    v = (rng.standard_normal(H) * np.exp2(rng.uniform(-60, 60, H))).astype(
        np.float32)
    rows.append(si.to_bf16_bits(v))
    allbits = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    finite = allbits[(allbits & 0x7F80) != 0x7F80]
    for i in range(0, len(finite) - H + 1, H):
        rows.append(finite[i:i + H])
    x = np.stack(rows)
    T = x.shape[0]
    ids = (np.arange(T * 2).reshape(T, 2) % 4).astype(np.int32)
    for G in (32, 128):
        scatter_both(ora, x, ids, 4, "compact", G, block_e=8)


def test_row_column_fixture(ora):
    """Distinct value per token row, doubled on odd columns."""
    T, H = 200, 1024
    base = (np.arange(T) % 200 + 1).astype(np.float32)[:, None]
    gain = 1.0 + (np.arange(H) % 2).astype(np.float32)[None, :]
    x = si.to_bf16_bits(base * gain)
    ids = si.uniform_topk(np.random.default_rng(8), T, 16, 4)
    scatter_both(ora, x, ids, 16, "compact", 128)


def test_no_destination_rows_untouched(ora):
    rng = np.random.default_rng(4)
    x = si.gaussian_bf16(rng, (64, 256))
    ids = np.full((64, 2), 50, np.int32)   # nothing local
    scatter_both(ora, x, ids, 8, "compact", 128)


# --------------------------------------------------------------- live rows

def live_both(ora, lr, G=32, full_check=True):
    rows, H = lr.x.shape
    nseg = lr.num_segments
    say("live rows", "rows=%d H=%d seg=%d live=%s G=%d"
        % (rows, H, nseg, lr.live_counts.tolist(), G))
    xd = bf16_to_dev(lr.x)
    q = torch.full((rows, H), CANARY, dtype=torch.uint8, device=DEV)
    s = torch.full((rows, H // G), CANARY, dtype=torch.uint8, device=DEV)
    live_d = i32_to_dev(lr.live_counts)
    mxq.mx_quant_live_rows(xd, nseg, live_d, FMT[G], q=q, scales=s)
    torch.cuda.synchronize()
    q_ref = np.full((rows, H), CANARY, np.uint8)
    s_ref = np.full((rows, H // G), CANARY, np.uint8)
    ora.mx_quant_live_rows(lr.x, nseg, lr.live_counts, G, q_ref, s_ref)
    assert_equal(host(s), s_ref, "scale bytes")
    assert_equal(host(q), q_ref, "fp8 bytes")
    return q, s


def test_live_rows_send_side_config(ora):
    lr = si.live_rows(full_rows=False)
    q, s = live_both(ora, lr)
    qv, sv = mxq.live_rows_view(q, s, 8, lr.live_counts)
    assert tuple(sv.shape) == (112, 224) and tuple(qv.shape) == (112, 7168)


def test_live_rows_one_segment_and_empty(ora):
    lr = si.live_rows(live_counts=[112, 0, 0, 0, 0, 0, 0, 0],
                      full_rows=False)
    live_both(ora, lr)
    lr0 = si.live_rows(live_counts=[0] * 8, full_rows=False)
    q, s = live_both(ora, lr0)
    qv, sv = mxq.live_rows_view(q, s, 8, lr0.live_counts)
    assert tuple(sv.shape) == (0, 224)


def test_live_rows_clip_and_g128(ora):
    lr = si.live_rows(num_segments=3, rows_per_segment=40, H=640,
                      live_counts=[41, -2, 17])
    live_both(ora, lr, G=32)
    live_both(ora, lr, G=128)


def test_live_rows_many_segments_and_ragged_chunks(ora):
    """64 segments (the most the ballot path holds: one per lane), with
    empty segments, clipped and negative counts, a hidden size that ends
    inside a 1024-channel chunk, and every row of a small buffer live; then
    65 segments, which take the row-per-block path."""
    rng = np.random.default_rng(21)
    live = rng.integers(-3, 9, size=64)
    live[::7] = 0
    live[5] = 100                       # clipped to rows_per_segment
    lr = si.live_rows(num_segments=64, rows_per_segment=6, H=1152,
                      live_counts=live.tolist())
    live_both(ora, lr, G=32)
    live_both(ora, lr, G=128)
    lr = si.live_rows(num_segments=3, rows_per_segment=50, H=96,
                      live_counts=[50, 50, 50])
    live_both(ora, lr, G=32)
    live = rng.integers(0, 5, size=65)
    lr = si.live_rows(num_segments=65, rows_per_segment=4, H=256,
                      live_counts=live.tolist())
    live_both(ora, lr, G=32)
    live_both(ora, lr, G=128)

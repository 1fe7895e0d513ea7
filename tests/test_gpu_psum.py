"""psum (expanded) layout repack on the GPU against the oracle: m_indices
from psum, expanded -> masked slab (payload, scales by stride, masked_m,
flags) and slab -> expanded with fused weights, all bit-exact."""
import numpy as np
import pytest
import torch

import fp8_mx_activation_amd as mxq
import synthetic_inputs as si
from gpu_util import DEV, assert_equal, bf16_to_dev, bf16_to_host, host, say
from test_oracle_psum import build_layout

pytestmark = pytest.mark.gpu


def i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(DEV)


@pytest.mark.parametrize("counts,align", [([3, 0, 130, 1], 128),
                                          ([127, 129, 1, 255, 0, 2], 128),
                                          ([0, 0, 0], 16), ([5] * 40, 8),
                                          # 1024 experts, 1.1 M rows: several
                                          # passes of the whole grid
                                          (list(range(0, 2048, 2)), 128)])
def test_m_indices_from_psum(ora, counts, align):
    _, psum, _, total = build_layout(counts, align, 1)
    say("m_indices_from_psum counts=%s align=%d" % (counts[:6], align))
    for rows in (total, total + 300):
        got = host(mxq.moe_m_indices_from_psum(i32(psum), rows, align))
        assert_equal(got, ora.m_indices_from_psum(psum, align, rows),
                     "m_indices")


def test_m_indices_from_psum_matches_layout(ora):
    b = si.prefill_compact(H=128)
    lay = mxq.moe_layout(torch.from_numpy(b.topk_ids).to(DEV), 0, 256,
                         "compact")
    counts = host(lay["counts"]).tolist()
    _, psum, _, _ = build_layout(counts, 128, 1)
    say("m_indices_from_psum vs moe_layout, prefill routing")
    got = mxq.moe_m_indices_from_psum(i32(psum), lay["num_rows"], 128)
    assert torch.equal(got, lay["m_indices"])


def slab_case(ora, counts, align, max_m, H, payload="bf16", scales=None,
              col_major=False, src_rows=None):
    base, psum, starts, total = build_layout(counts, align, H)
    if payload == "bf16":
        xb = si.to_bf16_bits(base)
        x_host = xb.view(np.uint8)
        x_dev = bf16_to_dev(xb)
    else:
        x_host = np.random.default_rng(2).integers(0, 255, (total, H),
                                                   np.uint8)
        x_dev = torch.from_numpy(x_host).to(DEV)
    if src_rows is not None:
        x_host, x_dev = x_host[:src_rows], x_dev[:src_rows]
    sc_host = sc_dev = None
    if scales is not None:
        sc_host = scales(total)
        src = np.ascontiguousarray(sc_host.T) if col_major else sc_host
        sc_dev = torch.from_numpy(src).to(DEV)
        if src_rows is not None:
            sc_host = sc_host[:src_rows]
            sc_dev = sc_dev[:, :src_rows] if col_major else sc_dev[:src_rows]
    E = len(counts)
    say("expand_to_masked_slab counts=%s H=%d max_m=%d payload=%s scales=%s"
        % (counts[:6], H, max_m, payload, None if scales is None else
           sc_host.dtype))
    slab0 = torch.full((E * max_m, x_dev.shape[1]), 0x5A if payload != "bf16"
                       else 0, dtype=x_dev.dtype, device=DEV)
    if payload == "bf16":
        slab0.view(torch.int16).fill_(0x7FC0)
    ss0 = None
    if scales is not None:
        ss0 = torch.zeros((E * max_m, sc_host.shape[1]), dtype=sc_dev.dtype,
                          device=DEV)
    slab, ss, mm, flags = mxq.moe_expand_to_masked_slab(
        x_dev, i32(psum), max_m, align, scales=sc_dev,
        scales_col_major=col_major, slab=slab0, slab_scales=ss0)
    torch.cuda.synchronize()
    # rows that are not copied keep the canary the slab was filled with
    nbytes = (E * max_m, x_dev.shape[1] * x_dev.element_size())
    if payload == "bf16":
        ref_slab = np.tile(np.array([0xC0, 0x7F], np.uint8),
                           nbytes[0] * nbytes[1] // 2).reshape(nbytes)
    else:
        ref_slab = np.full(nbytes, 0x5A, np.uint8)
    ref_ss = None if scales is None else np.zeros((E * max_m,
                                                   sc_host.shape[1]),
                                                  sc_host.dtype)
    _, _, mm_ref, fl_ref = ora.expand_to_masked_slab(
        x_host, psum, align, max_m, scales=None if scales is None else (
            np.ascontiguousarray(sc_host.T) if col_major else sc_host),
        scales_col_major=col_major, slab=ref_slab, slab_scales=ref_ss)
    assert_equal(host(mm), mm_ref, "masked_m")
    assert int(host(flags)[0]) == fl_ref
    assert_equal(host(slab.view(torch.uint8)), ref_slab, "slab bytes")
    if scales is not None:
        assert_equal(host(ss), ref_ss, "slab scales")
    return slab, mm, psum, total


def test_expand_roundtrip_bf16(ora):
    counts, align, max_m, H = [5, 0, 17, 3, 64], 16, 64, 96
    slab, mm, psum, total = slab_case(ora, counts, align, max_m, H)
    out0 = np.full((total, H), 0x1234, np.uint16)
    got = mxq.moe_masked_slab_to_expand(slab, mm, i32(psum), max_m, align,
                                        out=bf16_to_dev(out0))
    ref = ora.masked_slab_to_expand(bf16_to_host(slab), host(mm), psum, align,
                                    max_m, out=out0.copy())
    assert_equal(bf16_to_host(got), ref, "round trip")


def test_slab_to_expand_weights(ora):
    counts, align, max_m, H = [7, 0, 12, 1], 8, 16, 640
    slab, mm, psum, total = slab_case(ora, counts, align, max_m, H)
    w = np.random.default_rng(4).uniform(0.01, 1, total).astype(np.float32)
    out0 = np.full((total, H), 0x1234, np.uint16)
    got = mxq.moe_masked_slab_to_expand(
        slab, mm, i32(psum), max_m, align,
        weights=torch.from_numpy(w).to(DEV), out=bf16_to_dev(out0))
    ref = ora.masked_slab_to_expand(bf16_to_host(slab), host(mm), psum, align,
                                    max_m, weights=w, out=out0.copy())
    assert_equal(bf16_to_host(got), ref, "weighted expand")


def test_fp8_rows_with_e8m0_scales_row_major(ora):
    def sc(total):
        return np.random.default_rng(5).integers(100, 140, (total, 56),
                                                 np.uint8)
    slab_case(ora, [9, 2, 0, 33], 128, 48, 7168, payload="fp8", scales=sc)


def test_fp32_scales_column_major_seven_columns(ora):
    def sc(total):
        a = np.zeros((total, 7), np.float32)
        a[:] = (np.arange(total) % 50 + 1)[:, None] * 0.5 + np.arange(7)
        return a
    slab_case(ora, [5, 9, 0, 2], 4, 16, 896, payload="fp8", scales=sc,
              col_major=True)


def test_overflow_and_source_flags(ora):
    slab_case(ora, [8, 3], 8, 8, 32)                    # at capacity
    slab_case(ora, [9, 3], 8, 8, 32)                    # over: bit 0
    slab_case(ora, [3, 20, 0], 8, 8, 32)
    slab_case(ora, [4, 12], 8, 64, 32, src_rows=18)     # past source: bit 1


def test_decode_shape(ora):
    """One GPU's 32 of 256 experts at decode: the counts of the decode
    routing, fp8 rows of 7168 with 56 UE8M0 bytes, slab capacity 128."""
    b = si.decode_masked(H=128)
    lay = ora.moe_layout(b.topk_ids, 0, 32, "masked", capacity=128)

    def sc(total):
        return np.random.default_rng(6).integers(110, 130, (total, 56),
                                                 np.uint8)
    slab_case(ora, lay["counts"].tolist(), 128, 128, 7168, payload="fp8",
              scales=sc)


def test_prefill_sized_slab(ora):
    """Slabs of more than 4M 16-byte vectors, so both copies take their
    large-slab launch shape (1024-thread blocks of about 3584 vectors):
    12 experts, capacity 1024, one empty expert and one over capacity."""
    rng = np.random.default_rng(21)
    counts = rng.integers(300, 1025, size=12).tolist()
    counts[3], counts[7] = 1100, 0
    align, max_m = 128, 1024

    def sc(total):
        return np.random.default_rng(22).integers(100, 140, (total, 56),
                                                  np.uint8)
    # fp8 rows of 7168: 12 * 1024 * 448 vectors
    slab_case(ora, counts, align, max_m, 7168, payload="fp8", scales=sc)
    # bf16 rows of 4096: 12 * 1024 * 512 vectors, then back with weights
    slab, mm, psum, total = slab_case(ora, counts, align, max_m, 4096)
    w = np.random.default_rng(23).uniform(0.01, 1, total).astype(np.float32)
    out0 = np.full((total, 4096), 0x1234, np.uint16)
    got = mxq.moe_masked_slab_to_expand(
        slab, mm, i32(psum), max_m, align,
        weights=torch.from_numpy(w).to(DEV), out=bf16_to_dev(out0))
    ref = ora.masked_slab_to_expand(bf16_to_host(slab), host(mm), psum, align,
                                    max_m, weights=w, out=out0.copy())
    assert_equal(bf16_to_host(got), ref, "weighted expand, large slab")


def test_small_slab_expert_limits(ora):
    """Small slabs with 64 experts (one per lane of the unit kernels), with
    empty experts, one over capacity and the source ending inside the last
    range; then 65 experts, which take the per-expert block grid; both
    directions, the bf16 one with weights."""
    rng = np.random.default_rng(31)
    for E in (64, 65):
        counts = rng.integers(0, 13, size=E).tolist()
        counts[1], counts[E - 2] = 0, 20            # max_m 16: bit 0
        align, max_m, H = 16, 16, 1040              # 130 vectors of bf16
        slab, mm, psum, total = slab_case(ora, counts, align, max_m, H,
                                          src_rows=None)
        w = np.random.default_rng(E).uniform(0.01, 1, total).astype(
            np.float32)
        out0 = np.full((total, H), 0x1234, np.uint16)
        say("slab_to_expand E=%d" % E)
        got = mxq.moe_masked_slab_to_expand(
            slab, mm, i32(psum), max_m, align,
            weights=torch.from_numpy(w).to(DEV), out=bf16_to_dev(out0))
        ref = ora.masked_slab_to_expand(bf16_to_host(slab), host(mm), psum,
                                        align, max_m, weights=w,
                                        out=out0.copy())
        assert_equal(bf16_to_host(got), ref, "weighted expand E=%d" % E)

        def sc(t):
            return np.random.default_rng(7).integers(100, 140, (t, 9),
                                                     np.uint8)
        slab_case(ora, counts, align, max_m, 4112, payload="fp8", scales=sc)
        # the source ends two rows into the last non-empty range: bit 1
        last = max(i for i, c in enumerate(counts) if c > 0)
        short = psum[last] - 2 if last >= 0 else 0
        slab_case(ora, counts, align, max_m, 64, src_rows=int(short))

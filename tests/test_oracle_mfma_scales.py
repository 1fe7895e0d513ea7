"""Pins of the oracle's block-scaled MFMA scale placement (reading R16).

No page fixes this layout: it is what gfx950's v_mfma_scale_f32_32x32x64 /
16x16x128 _f8f6f4 instructions read (lane l of instruction s supplies the
scale of block s*(64/tm) + l//tm of row l%tm from byte s%4 of its scale
register).  Here it is
pinned by its bijectivity, by positions worked out by hand from that operand
description, and by the group-128 replication; the GPU tests pin it to the
hardware itself by feeding it to those instructions."""
import numpy as np
import pytest

import oracle


def labels(rows, ng):
    return np.arange(rows * ng, dtype=np.int64).reshape(rows, ng)


@pytest.mark.parametrize("tm", [32, 16])
@pytest.mark.parametrize("rows,H", [(1, 32), (31, 224), (32, 7168),
                                    (33, 7200), (100, 96), (64, 4096)])
def test_every_block_once(tm, rows, H):
    """Each (row, block) lands on exactly one byte; nothing else is
    written; the size matches the library's host query."""
    nkb = H // 32
    out = oracle.mfma_scales(labels(rows, nkb), H, 32, tm, fill=-1)
    got = out[out >= 0]
    assert got.size == rows * nkb
    assert np.array_equal(np.sort(got), np.arange(rows * nkb))
    import fp8_mx_activation_amd as mxq
    if __import__("os").path.exists(mxq.LIB_PATH):
        assert out.size == mxq.mxq_mfma_scale_bytes(rows, H, tm)


def byte_at(out, offset):
    return out.reshape(-1)[offset]


def test_worked_positions_tile32():
    """32-row tiles (32x32x64: two 32-channel blocks per instruction, eight
    per register).  Worked from the operand description: lane r < 32 of
    instruction 0 supplies the scale of block 0 of row r, lane 32 + r that
    of block 1; instruction s reads byte s % 4 of the register of group
    s // 4."""
    H, rows = 512, 64                      # 16 blocks: 2 word groups
    L = labels(rows, H // 32)
    out = oracle.mfma_scales(L, H, 32, 32, fill=-1)
    assert out.shape == (2, 2, 64, 4)
    lab = lambda r, kb: r * (H // 32) + kb
    assert byte_at(out, 0) == lab(0, 0)            # instr 0, lane 0
    assert byte_at(out, 4) == lab(1, 0)            # instr 0, lane 1
    assert byte_at(out, 4 * 31) == lab(31, 0)      # instr 0, lane 31
    assert byte_at(out, 4 * 32) == lab(0, 1)       # instr 0, lane 32
    assert byte_at(out, 4 * 63) == lab(31, 1)      # instr 0, lane 63
    assert byte_at(out, 1) == lab(0, 2)            # instr 1, lane 0
    assert byte_at(out, 4 * 32 + 3) == lab(0, 7)   # instr 3, lane 32
    assert byte_at(out, 256) == lab(0, 8)          # instr 4, lane 0
    assert byte_at(out, 256 + 4 * 33 + 2) == lab(1, 13)  # instr 6, lane 33
    assert byte_at(out, 512) == lab(32, 0)         # second row tile
    assert byte_at(out, 1023) == lab(63, 15)       # last byte


def test_worked_positions_tile16():
    """16-row tiles (16x16x128: four blocks per instruction, sixteen per
    register): lane 16*h + r supplies the scale of block h of row r."""
    H, rows = 1024, 32                     # 32 blocks: 2 word groups
    L = labels(rows, H // 32)
    out = oracle.mfma_scales(L, H, 32, 16, fill=-1)
    assert out.shape == (2, 2, 64, 4)
    lab = lambda r, kb: r * (H // 32) + kb
    assert byte_at(out, 0) == lab(0, 0)
    assert byte_at(out, 4 * 15) == lab(15, 0)
    assert byte_at(out, 4 * 16) == lab(0, 1)
    assert byte_at(out, 4 * 48) == lab(0, 3)
    assert byte_at(out, 4 * 63) == lab(15, 3)
    assert byte_at(out, 1) == lab(0, 4)            # instr 1
    assert byte_at(out, 4 * 17 + 3) == lab(1, 13)  # instr 3, lane 17
    assert byte_at(out, 256) == lab(0, 16)         # instr 4
    assert byte_at(out, 512) == lab(16, 0)         # second row tile


def test_ragged_blocks_and_rows_untouched():
    """225 blocks (not a whole number of word groups) and 33 rows: the
    positions past the data keep the fill."""
    out = oracle.mfma_scales(labels(33, 225), 7200, 32, 32, fill=-1)
    assert out.shape == (2, 29, 64, 4)
    o = out.reshape(2, 29, 64, 4)
    assert (o[1, :, 1:32, :] == -1).all() and (o[1, :, 33:64, :] == -1).all()
    # block 224 is the only block of the last group: instruction 112
    # (byte 0), lanes 0..31
    assert (o[0, 28, :32, 0] == np.arange(32) * 225 + 224).all()
    assert (o[0, 28, 32:, 0] == -1).all() and (o[0, 28, :, 1:] == -1).all()


def test_group128_scale_on_its_four_blocks():
    rng = np.random.default_rng(16)
    S = rng.integers(0, 255, (40, 7), dtype=np.uint8)
    out = oracle.mfma_scales(S, 896, 128, 32)
    per_block = oracle.mfma_scales(np.repeat(S, 4, axis=1), 896, 32, 32)
    assert np.array_equal(out, per_block)

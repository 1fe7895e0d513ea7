"""C-ABI boundary checks that need no GPU: the library loads, exports every
function include/mxq.h declares, its host-only helpers agree with the oracle,
and argument validation rejects bad calls before anything is enqueued (no
compute call is made here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxq.h")

INVALID, UNSUPPORTED, WORKSPACE = 1, 2, 4


@pytest.fixture(scope="module")
def mxq():
    import fp8_mx_activation_amd as m
    if not os.path.exists(m.LIB_PATH):
        from fp8_mx_activation_amd import build
        build.build(verbose=False)
    m.lib()
    return m


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_path(mxq):
    names = declared_functions()
    for n in ("moe_layout", "moe_scatter_quant", "mx_quant_live_rows",
              "requant_per_token_to_per_tensor", "moe_combine",
              "moe_compact_row_bound", "moe_should_use_masked",
              "moe_read_overflow", "mxq_e4m3_encode_f32"):
        assert n in names


def test_every_declared_symbol_is_exported(mxq):
    L = ctypes.CDLL(mxq.LIB_PATH)
    for n in declared_functions():
        assert hasattr(L, n), n
    assert set(declared_functions()) <= set(mxq._SIGNATURES)


def test_abi_version_and_status_strings(mxq):
    assert mxq.mxq_abi_version() == 1
    L = mxq.lib()
    assert L.mxq_status_string(0) == b"ok"
    assert b"capacity" in L.mxq_status_string(3)


def test_host_helpers_match_oracle(mxq, ora):
    for A, E, b in [(128, 8, 128), (65536, 256, 128), (131072, 128, 128),
                    (0, 3, 128), (7, 9, 4), (1000, 1, 1)]:
        assert mxq.moe_compact_row_bound(A, E, b) == \
            ora.compact_row_bound(A, E, b)
    for g, l in [(256, 32), (256, 256), (256, 33), (8, 8), (64, 8)]:
        assert mxq.moe_should_use_masked(g, l) == ora.should_use_masked(g, l)
    assert mxq.lib().moe_compact_row_bound(-1, 8, 128) == -1
    assert mxq.lib().moe_compact_row_bound(8, 8, 0) == -1


def test_workspace_sizes(mxq):
    assert mxq.moe_layout_workspace_bytes(0, 8, 256) == 0
    assert mxq.moe_layout_workspace_bytes(512, 8, 256) == 0    # one launch
    # up to 2^14 assignments over at most 256 experts every block of the
    # slot kernel counts the routing itself: no workspace either
    assert mxq.moe_layout_workspace_bytes(513, 8, 256) == 0
    assert mxq.moe_layout_workspace_bytes(2048, 8, 256) == 0
    assert mxq.moe_layout_workspace_bytes(513, 8, 257) > 0
    assert mxq.moe_layout_workspace_bytes(2049, 8, 256) > 0
    w = mxq.moe_layout_workspace_bytes(8192, 8, 256)
    assert 0 < w <= 64 * 256 * 4
    assert mxq.requant_workspace_bytes(16384, 4096) >= 4


FAKE = 0x10000  # a 16-byte aligned non-null pointer value; never dereferenced


def test_scatter_quant_validation(mxq):
    L = mxq.lib()
    ok = dict(x=FAKE, ld_x=256, T=4, H=256, s2d=FAKE, K=2, fmt=0, q=FAKE,
              ld_q=256, s=FAKE, ld_s=2, rows=16)

    def call(**kw):
        a = dict(ok, **kw)
        return L.moe_scatter_quant(a["x"], a["ld_x"], a["T"], a["H"],
                                   a["s2d"], a["K"], a["fmt"], a["q"],
                                   a["ld_q"], a["s"], a["ld_s"], a["rows"],
                                   None)

    assert call(fmt=7) == UNSUPPORTED
    assert call(H=200) == INVALID              # not a multiple of 128
    assert call(H=96, fmt=1, ld_s=2) == INVALID  # 3 scales need ld_s >= 3
    assert call(ld_q=128) == INVALID
    assert call(ld_x=100) == INVALID
    assert call(s=None) == INVALID             # missing scales, rows > 0
    assert call(x=FAKE + 8) == INVALID         # misaligned rows
    assert call(ld_q=264) == INVALID           # fp8 stride not 16-byte
    assert call(T=-1) == INVALID
    assert call(K=65) == INVALID
    assert call(H=32768 + 128, ld_x=32768 + 128, ld_q=32768 + 128,
                ld_s=300) == UNSUPPORTED       # row does not fit in LDS
    assert call(T=0) == 0                      # empty batch: nothing to do
    assert call(rows=0, q=None, s=None) == 0


def test_scatter_quant_ex_validation(mxq):
    """Rule and scale placement checks of the variant entry points."""
    L = mxq.lib()
    ok = dict(x=FAKE, ld_x=256, T=4, H=640, s2d=FAKE, K=2, fmt=1, rule=0,
              q=FAKE, ld_q=640, s=FAKE, rs=20, c4=4, rows=18)

    def call(**kw):
        a = dict(ok, **kw)
        a["ld_x"] = max(a["ld_x"], a["H"])
        return L.moe_scatter_quant_ex(a["x"], a["ld_x"], a["T"], a["H"],
                                      a["s2d"], a["K"], a["fmt"], a["rule"],
                                      a["q"], a["ld_q"], a["s"], a["rs"],
                                      a["c4"], a["rows"], None)

    def live(**kw):
        a = dict(ok, **kw)
        a["ld_x"] = max(a["ld_x"], a["H"])
        return L.mx_quant_live_rows_ex(a["x"], a["ld_x"], 3, 6, FAKE, a["H"],
                                       a["fmt"], a["rule"], a["q"],
                                       a["ld_q"], a["s"], a["rs"], a["c4"],
                                       None)

    for f in (call, live):
        assert f(rule=2) == UNSUPPORTED
        assert f(rule=-1) == UNSUPPORTED
        assert f(rs=19) == INVALID            # 20 groups need rs >= 20
        assert f(rs=20, c4=8) == INVALID      # neither placement
        assert f(rs=4, c4=4 * 18 - 4) == INVALID  # packed: c4 < 4 * rows
        assert f(rs=4, c4=4 * 18 + 2) == INVALID  # packed: c4 not words
    # 20 groups of 32: packed needs 5 words per row
    assert call(T=0, rs=4, c4=4 * 20) == 0
    assert call(T=0, rule=1) == 0
    assert call(rows=0, q=None, s=None, rs=4, c4=0) == 0


def test_copy16_validation(mxq):
    L = mxq.lib()
    assert L.mxq_copy16(FAKE, FAKE + 4096, 0, 0, None) == 0
    assert L.mxq_copy16(FAKE, FAKE + 4096, 24, 0, None) == INVALID
    assert L.mxq_copy16(FAKE, FAKE + 4096, -16, 1, None) == INVALID
    assert L.mxq_copy16(None, FAKE, 32, 0, None) == INVALID
    assert L.mxq_copy16(FAKE + 8, FAKE + 4096, 32, 0, None) == INVALID
    assert L.mxq_copy16(FAKE, FAKE + 4096, 32, 4, None) == INVALID
    assert L.mxq_copy16(FAKE, FAKE + 4096, 32, -1, None) == INVALID
    # the gather-read and row-fill references
    g = L.mxq_gather_read16
    assert g(FAKE, 64, 10, FAKE, 0, 8, 64, FAKE, None) == 0      # no groups
    assert g(FAKE, 64, 10, FAKE, 4, 0, 64, FAKE, None) == INVALID
    assert g(FAKE, 64, 10, FAKE, 4, 65, 64, FAKE, None) == INVALID
    assert g(FAKE, 64, 10, FAKE, 4, 8, 72, FAKE, None) == INVALID  # ld < row
    assert g(FAKE, 64, 10, FAKE, 4, 8, 40, FAKE, None) == INVALID  # not 16
    assert g(FAKE + 8, 64, 10, FAKE, 4, 8, 64, FAKE, None) == INVALID
    assert g(FAKE, 64, 10, None, 4, 8, 64, FAKE, None) == INVALID
    f = L.mxq_fill_rows16
    assert f(FAKE, 64, 0, 64, 0, None) == 0
    assert f(FAKE, 48, 3, 64, 0, None) == INVALID
    assert f(FAKE + 8, 64, 3, 64, 0, None) == INVALID
    assert f(None, 64, 3, 64, 0, None) == INVALID


def test_mfma_placement_validation(mxq):
    """The block-scaled MFMA placement: size query and entry-point checks
    (every rejected call returns before anything is enqueued)."""
    L = mxq.lib()
    assert L.mxq_mfma_scale_bytes(98048, 7168, 32) == 98048 * 224
    assert L.mxq_mfma_scale_bytes(98048, 7168, 16) == 98048 * 224
    assert L.mxq_mfma_scale_bytes(33, 7200, 32) == 2 * 29 * 256
    assert L.mxq_mfma_scale_bytes(0, 7168, 32) == 0
    for bad in [(-1, 7168, 32), (4, 0, 32), (4, 7169, 32), (4, 7168, 8),
                (4, 7168, 64), (4, 96 + 16, 16)]:
        assert L.mxq_mfma_scale_bytes(*bad) == -1, bad
    ok = dict(x=FAKE, ld_x=640, T=4, H=640, s2d=FAKE, K=2, fmt=1, rule=0,
              q=FAKE, ld_q=640, s=FAKE, tm=32, rows=18)

    def call(**kw):
        a = dict(ok, **kw)
        return L.moe_scatter_quant_mfma(a["x"], a["ld_x"], a["T"], a["H"],
                                        a["s2d"], a["K"], a["fmt"], a["rule"],
                                        a["q"], a["ld_q"], a["s"], a["tm"],
                                        a["rows"], None)

    def live(**kw):
        a = dict(ok, **kw)
        return L.mx_quant_live_rows_mfma(a["x"], a["ld_x"], 3, 6, FAKE, a["H"],
                                         a["fmt"], a["rule"], a["q"],
                                         a["ld_q"], a["s"], a["tm"], None)

    for f in (call, live):
        assert f(tm=8) == INVALID
        assert f(tm=64) == INVALID
        assert f(rule=2) == UNSUPPORTED
        assert f(fmt=7) == UNSUPPORTED
        assert f(s=None) == INVALID
        assert f(ld_q=639) == INVALID
        assert f(H=650) == INVALID            # not a whole number of groups
    assert call(T=0) == 0
    assert call(rows=0, q=None, s=None) == 0
    assert live(H=640, x=None) == INVALID
    assert call(s=FAKE + 2) == INVALID          # scatter writes 32-bit words


def test_upscale_and_weight_requant_validation(mxq):
    L = mxq.lib()

    def up(q=FAKE, ld_q=256, s=FAKE, rs=2, cs=1, rows=4, H=256, G=128,
           o=FAKE, ld_o=256):
        return L.upscale_fp8_to_bf16(q, ld_q, s, rs, cs, rows, H, G, o, ld_o,
                                     None)

    assert up(G=64) == UNSUPPORTED
    assert up(H=200) == INVALID                # not a multiple of 128
    assert up(rows=-1) == INVALID
    assert up(ld_q=264 - 16 - 8) == INVALID    # ld_q < H
    assert up(ld_q=264) == INVALID             # not 16-byte rows
    assert up(ld_o=260) == INVALID             # bf16 rows not 16-byte
    assert up(o=FAKE + 2) == INVALID
    assert up(s=None) == INVALID
    assert up(rs=-1) == INVALID
    assert up(rows=0, q=None, s=None, o=None) == 0
    assert up(G=32, H=96, ld_q=96, ld_o=96, rows=0) == 0

    def wr(q=FAKE, ld=256, qbs=256 * 256, s=FAKE, sld=2, sbs=4, B=2, N=256,
           K=256, bn=128, bk=128, qo=FAKE, so=FAKE, old=2, obs=4):
        return L.requant_weight_block_ue8m0(q, ld, qbs, s, sld, sbs, B, N, K,
                                            bn, bk, qo, so, old, obs, None)

    assert wr(bn=64) == UNSUPPORTED
    assert wr(bk=256) == UNSUPPORTED
    assert wr(K=200, ld=208) == INVALID        # K % 16
    assert wr(ld=250) == INVALID               # ld < K
    assert wr(qbs=256 * 255) == INVALID        # matrices overlap
    assert wr(sld=1) == INVALID
    assert wr(sbs=3) == INVALID
    assert wr(old=1) == INVALID
    assert wr(obs=3) == INVALID
    assert wr(qo=FAKE + 4) == INVALID
    assert wr(so=None) == INVALID
    assert wr(B=-1) == INVALID
    assert wr(N=0) == 0
    assert wr(B=0, q=None, s=None, qo=None, so=None) == 0


def test_scatter_rows_validation(mxq):
    L = mxq.lib()

    def call(x=FAKE, ld_x=448, T=4, rb=448, xs=None, xrs=0, xcs=0, cols=0,
             elem=1, s2d=FAKE, K=2, rows=16, out=FAKE, ld_o=448, os=None,
             ors=0, ocs=0):
        return L.moe_scatter_rows(x, ld_x, T, rb, xs, xrs, xcs, cols, elem,
                                  s2d, K, rows, out, ld_o, os, ors, ocs, None)

    assert call(rb=440, ld_x=448) == UNSUPPORTED   # row bytes % 16
    assert call(K=65) == INVALID
    assert call(T=-1) == INVALID
    assert call(ld_x=432) == INVALID               # stride < row
    assert call(ld_o=456) == INVALID               # stride % 16
    assert call(x=FAKE + 4) == INVALID
    assert call(s2d=None) == INVALID
    assert call(xs=FAKE, os=None) == INVALID
    assert call(xs=FAKE, os=FAKE, cols=7, elem=2) == INVALID
    assert call(xs=FAKE, os=FAKE, cols=7, elem=4, xrs=30) == INVALID
    assert call(T=0, x=None, out=None) == 0
    assert call(rows=0, out=None) == 0


def test_layout_validation(mxq):
    L = mxq.lib()

    def call(T=8, K=2, E=4, kind=0, block=128, cap=0, rows=None, ws=FAKE,
             wsb=1 << 20, ids=FAKE):
        if rows is None:
            rows = mxq.moe_compact_row_bound(T * K, E, block)
        return L.moe_layout(ids, T, K, 0, E, kind, block, cap, rows, FAKE,
                            FAKE, FAKE, FAKE, FAKE, FAKE, ws, wsb, None)

    assert call(rows=100) == INVALID           # below the compact bound
    assert call(E=0) == INVALID
    assert call(E=1025) == INVALID
    assert call(K=0) == INVALID
    assert call(kind=5) == UNSUPPORTED
    assert call(kind=1, cap=0, rows=0) == INVALID
    assert call(kind=1, cap=16, rows=63) == INVALID  # E * cap = 64
    # the per-chunk count workspace: needed above 4096 assignments with more
    # than 256 experts, or above 2^14 assignments
    assert call(T=2048, K=8, E=300, ws=None) == WORKSPACE
    assert call(T=2048, K=8, E=300, wsb=4) == WORKSPACE
    assert call(T=20000, K=8, ws=None) == WORKSPACE
    assert call(ids=None) == INVALID
    assert call(block=0, rows=1024) == INVALID
    assert call(T=(1 << 21) + 1, K=8, rows=1 << 30) == UNSUPPORTED  # > 2^24


def test_layout_noalloc_validation(mxq):
    """The allocation-free layout checks what moe_layout checks and refuses
    a routing whose per-chunk counts exceed its static scratch, all before
    any HIP call."""
    L = mxq.lib()
    SCRATCH = 6

    def call(T=8, K=2, E=4, kind=0, block=128, cap=0, rows=None, ids=FAKE):
        if rows is None:
            rows = mxq.moe_compact_row_bound(T * K, E, block)
        return L.moe_layout_noalloc(ids, T, K, 0, E, kind, block, cap, rows,
                                    FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None)

    assert call(rows=100) == INVALID
    assert call(E=0) == INVALID
    assert call(kind=5) == UNSUPPORTED
    assert call(ids=None) == INVALID
    assert call(T=(1 << 21) + 1, K=8, rows=1 << 30) == UNSUPPORTED
    # 2^24 assignments over 1024 experts: 2048 chunks x 1024 counts = 8 MiB
    assert mxq.moe_layout_workspace_bytes(1 << 21, 8, 1024) == 8 << 20
    assert call(T=1 << 21, K=8, E=1024) == SCRATCH
    assert mxq.MXQ_ERR_SCRATCH_LIMIT == SCRATCH
    assert b"scratch" in L.mxq_status_string(SCRATCH)
    # a prefill-sized routing that uses the counts (8192 x top-8 over 384
    # experts) fits: 96 KiB
    assert 0 < mxq.moe_layout_workspace_bytes(8192, 8, 384) <= \
        mxq.LAYOUT_NOALLOC_SCRATCH_BYTES


def test_combine_requant_live_validation(mxq):
    L = mxq.lib()
    assert L.moe_combine(FAKE, 256, 16, FAKE, FAKE, 4, 2, 260, FAKE, 260, 0,
                         None) == INVALID     # H % 8
    assert L.moe_combine(FAKE, 256, 16, FAKE, FAKE, 4, 2, 256, FAKE, 256, 9,
                         None) == UNSUPPORTED
    assert L.moe_combine(FAKE, 256, 16, FAKE, FAKE, 0, 2, 256, FAKE, 256, 0,
                         None) == 0
    assert L.requant_per_token_to_per_tensor(FAKE, 256, FAKE, 4, 256, FAKE,
                                             256, FAKE, None, 0,
                                             None) == WORKSPACE
    assert L.requant_per_token_to_per_tensor(FAKE, 256, FAKE, 4, 256, FAKE,
                                             128, FAKE, FAKE, 4096,
                                             None) == INVALID
    assert L.requant_per_token_to_per_tensor(FAKE, 256, FAKE, 4, 256, FAKE,
                                             256, None, FAKE, 4096,
                                             None) == INVALID
    assert L.mx_quant_live_rows(FAKE, 256, 2, 8, FAKE, 250, 1, FAKE, 256,
                                FAKE, 8, None) == INVALID  # 250 % 32
    assert L.mx_quant_live_rows(FAKE, 256, 0, 8, FAKE, 256, 1, FAKE, 256,
                                FAKE, 8, None) == 0
    assert L.mxq_e4m3_encode_f32(FAKE, -1, FAKE, None) == INVALID


def test_product_path_never_touches_the_oracle():
    """The package imports neither the oracle nor the input generators."""
    pkg = os.path.join(ROOT, "fp8_mx_activation_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".h")):
                src = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+(oracle|"
                                     r"synthetic_inputs)\b", src, re.M), f


def test_psum_repack_validation(mxq):
    L = mxq.lib()
    assert L.moe_m_indices_from_psum(FAKE, 0, 128, 10, FAKE, None) == INVALID
    assert L.moe_m_indices_from_psum(FAKE, 4, 0, 10, FAKE, None) == INVALID
    assert L.moe_m_indices_from_psum(None, 4, 128, 0, None, None) == 0
    ok = dict(x=FAKE, ld_x=256, rows=64, rb=256, xs=None, xs_rs=0, xs_cs=0,
              sc=0, se=0, psum=FAKE, E=4, al=128, mm=8, slab=FAKE, ld_s=256,
              ss=None, ss_rs=0, ss_cs=0, masked=FAKE, flags=FAKE)

    def call(**kw):
        a = dict(ok, **kw)
        return L.moe_expand_to_masked_slab(
            a["x"], a["ld_x"], a["rows"], a["rb"], a["xs"], a["xs_rs"],
            a["xs_cs"], a["sc"], a["se"], a["psum"], a["E"], a["al"],
            a["mm"], a["slab"], a["ld_s"], a["ss"], a["ss_rs"], a["ss_cs"],
            a["masked"], a["flags"], None)

    assert call(rb=100, ld_x=112, ld_s=112) == UNSUPPORTED  # 16-byte rows
    assert call(ld_s=128) == INVALID            # slab stride below the row
    assert call(mm=0) == INVALID
    assert call(flags=None) == INVALID
    assert call(xs=FAKE, ss=FAKE, sc=7, se=2) == INVALID  # 1- or 4-byte only
    assert call(xs=FAKE, ss=FAKE, sc=7, se=4, xs_rs=30, xs_cs=4, ss_rs=28,
                ss_cs=4) == INVALID             # misaligned 4-byte stride
    assert L.moe_masked_slab_to_expand(FAKE, 64, 60, FAKE, FAKE, 4, 128, 8,
                                       None, FAKE, 64, 10, None) == INVALID
    assert L.moe_masked_slab_to_expand(FAKE, 64, 64, FAKE, FAKE, 4, 128, 8,
                                       None, FAKE, 64, 0, None) == 0

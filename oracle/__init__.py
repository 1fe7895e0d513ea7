"""CPU oracle for the MoE dispatch-preprocessing path (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: this package is the slow, plain reference the GPU
library is checked against.  Only the test suite, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import it; the product package
never does, and it is never a fallback for the GPU path.

The arithmetic lives in ``mxq_oracle.c`` (plain C, built with
``-O2 -ffp-contract=off -fopenmp``); see that file's header for the pages each
function follows and the readings taken where they are silent.  This module
only converts numpy arrays to pointers.

Arrays: bf16 data is carried as ``uint16`` (the upper half of a binary32
word), fp8 e4m3fn and scale bytes as ``uint8``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mxq_oracle.c")
# MXQ_ORACLE_LIB names a prebuilt copy to load instead (the sanitizer build
# of oracle/sanitize.py); it is never rebuilt here.
_LIB_ENV = os.environ.get("MXQ_ORACLE_LIB")
_LIB_PATH = _LIB_ENV or os.path.join(_HERE, "liboracle.so")

_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_u32 = ctypes.c_uint32
_p = ctypes.c_void_p


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (it is C, not part of the GPU library)."""
    if _LIB_ENV:
        if not os.path.exists(_LIB_ENV):
            raise RuntimeError("MXQ_ORACLE_LIB=%s does not exist" % _LIB_ENV)
        return _LIB_ENV
    if force or not os.path.exists(_LIB_PATH) or (
        os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)
    ):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
             "-fopenmp", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
        )
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        sig = {
            "ora_max_threads": (_i32, []),
            "ora_set_threads": (None, [_i32]),
            "ora_e4m3_decode": (ctypes.c_double, [ctypes.c_uint8]),
            "ora_e4m3_encode": (ctypes.c_uint8, [ctypes.c_double]),
            "ora_bf16_round": (ctypes.c_uint16, [ctypes.c_float]),
            "ora_bf16_round_array": (None, [_p, _i64, _p]),
            "ora_e4m3_encode_array_f32": (None, [_p, _i64, _p]),
            "ora_e4m3_decode_array": (None, [_p, _i64, _p]),
            "ora_e4m3_encode_bits_range": (None, [_u32, _i64, _p]),
            "ora_pow2_scale_exponent": (_i32, [ctypes.c_double]),
            "ora_quant_row": (None, [_p, _i32, _i32, _p, _p]),
            "ora_quant_row_rule": (None, [_p, _i32, _i32, _i32, _p, _p]),
            "ora_ocp_mx_exponent": (_i32, [ctypes.c_double]),
            "ora_scatter_quant_ex": (None, [_p, _i64, _i64, _i32, _p, _i32,
                                            _i32, _i32, _p, _i64, _p, _i64,
                                            _i64]),
            "ora_compact_row_bound": (_i64, [_i64, _i32, _i32]),
            "ora_should_use_masked": (_i32, [_i32, _i32]),
            "ora_moe_layout": (_i32, [_p, _i64, _i32, _i32, _i32, _i32, _i32,
                                      _i32, _i64, _p, _p, _p, _p, _p, _p]),
            "ora_scatter_quant": (None, [_p, _i64, _i64, _i32, _p, _i32, _i32,
                                         _p, _i64, _p, _i64]),
            "ora_mx_quant_live_rows": (None, [_p, _i64, _i32, _i64, _p, _i32,
                                              _i32, _p, _i64, _p, _i64]),
            "ora_requant_per_token_to_per_tensor": (
                None, [_p, _i64, _p, _i64, _i32, _p, _i64, _p]),
            "ora_combine_f32": (None, [_p, _i64, _p, _p, _i64, _i32, _i32, _p,
                                       _i64]),
            "ora_combine_f64": (None, [_p, _i64, _p, _p, _i64, _i32, _i32, _p,
                                       _p, _i64]),
            "ora_m_indices_from_psum": (None, [_p, _i32, _i32, _i64, _p]),
            "ora_expand_to_masked_slab": (
                _i32, [_p, _i64, _i64, _i64, _p, _i64, _i64, _i32, _i32, _p,
                       _i32, _i32, _i32, _p, _i64, _p, _i64, _i64, _p]),
            "ora_masked_slab_to_expand": (
                None, [_p, _i64, _i32, _p, _p, _i32, _i32, _i32, _p, _p, _i64,
                       _i64]),
            "ora_scatter_rows": (None, [_p, _i64, _i64, _i64, _p, _i64, _i64,
                                        _i32, _i32, _p, _i32, _i64, _p, _i64,
                                        _p, _i64, _i64]),
            "ora_bf16_round_f64": (ctypes.c_uint16, [ctypes.c_double]),
            "ora_bf16_round_f64_array": (None, [_p, _i64, _p]),
            "ora_upscale_fp8": (None, [_p, _i64, _p, _i64, _i64, _i64, _i32,
                                       _i32, _p, _i64]),
            "ora_requant_weight_block_ue8m0": (
                None, [_p, _i64, _i64, _p, _i64, _i64, _i32, _i32, _i32, _i32,
                       _i32, _p, _p, _i64, _i64]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data if a.size else 0


def _c(a, dtype) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def max_threads() -> int:
    return int(lib().ora_max_threads())


def set_threads(n: int) -> None:
    lib().ora_set_threads(int(n))


# ------------------------------------------------------------------ formats

def e4m3_decode(b) -> np.ndarray:
    b = _c(b, np.uint8)
    out = np.empty(b.shape, np.float64)
    lib().ora_e4m3_decode_array(_ptr(b), b.size, _ptr(out))
    return out


def e4m3_encode(y) -> np.ndarray:
    """Encode float32 values to e4m3fn bytes (nearest-even, saturating)."""
    y = _c(y, np.float32)
    out = np.empty(y.shape, np.uint8)
    lib().ora_e4m3_encode_array_f32(_ptr(y), y.size, _ptr(out))
    return out


def e4m3_encode_bits_range(w0: int, n: int) -> np.ndarray:
    out = np.empty(n, np.uint8)
    lib().ora_e4m3_encode_bits_range(w0, n, _ptr(out))
    return out


def bf16_round(x) -> np.ndarray:
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().ora_bf16_round_array(_ptr(x), x.size, _ptr(out))
    return out


def bf16_round_f64(x) -> np.ndarray:
    """Round float64 values to bf16 bits once (nearest-even; NaN -> 0x7FC0)."""
    x = _c(x, np.float64)
    out = np.empty(x.shape, np.uint16)
    lib().ora_bf16_round_f64_array(_ptr(x), x.size, _ptr(out))
    return out


def pow2_scale_exponent(amax: float) -> int:
    return int(lib().ora_pow2_scale_exponent(float(amax)))


RULES = {"ceil": 0, "ocp_floor": 1}


def quant_row(x_bf16, G: int, rule: str = "ceil"):
    x = _c(x_bf16, np.uint16)
    H = x.shape[-1]
    q = np.empty(H, np.uint8)
    s = np.empty(H // G, np.uint8)
    lib().ora_quant_row_rule(_ptr(x), H, G, RULES[rule], _ptr(q), _ptr(s))
    return q, s


def ocp_mx_exponent(amax: float) -> int:
    return int(lib().ora_ocp_mx_exponent(float(amax)))


# ------------------------------------------------------------------- layout

def compact_row_bound(num_assignments: int, num_experts: int,
                      block_e: int = 128) -> int:
    return int(lib().ora_compact_row_bound(num_assignments, num_experts,
                                           block_e))


def should_use_masked(num_experts: int, num_local_experts: int) -> bool:
    return bool(lib().ora_should_use_masked(num_experts, num_local_experts))


def moe_layout(topk_ids, expert_begin: int, num_local_experts: int,
               kind: str, block_e: int = 128, capacity: int = 0,
               num_rows: int | None = None):
    """Returns dict(counts, expert_offsets, m_indices, masked_m, src2dst,
    overflow, num_rows)."""
    ids = _c(topk_ids, np.int32)
    T, K = ids.shape
    E = num_local_experts
    k = {"compact": 0, "masked": 1}[kind]
    if num_rows is None:
        num_rows = (compact_row_bound(T * K, E, block_e) if k == 0
                    else E * capacity)
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    m_idx = np.empty(num_rows, np.int32)
    masked_m = np.empty(E, np.int32)
    src2dst = np.empty((T, K), np.int32)
    ovf = np.zeros(1, np.int32)
    rc = lib().ora_moe_layout(_ptr(ids), T, K, expert_begin, E, k, block_e,
                              capacity, num_rows, _ptr(counts),
                              _ptr(offsets), _ptr(m_idx), _ptr(masked_m),
                              _ptr(src2dst), _ptr(ovf))
    if rc != 0:
        raise ValueError("num_rows too small for this routing")
    return dict(counts=counts, expert_offsets=offsets, m_indices=m_idx,
                masked_m=masked_m, src2dst=src2dst, overflow=int(ovf[0]),
                num_rows=num_rows)


# ----------------------------------------------------------- quantization

def scatter_quant(x_bf16, src2dst, G: int, num_rows: int, q=None, s=None):
    """Quantize each token row once and copy it to its destination rows.
    ``q``/``s`` may be given pre-filled (untouched rows keep their bytes)."""
    x = _c(x_bf16, np.uint16)
    d = _c(src2dst, np.int32)
    T, H = x.shape
    K = d.shape[1] if d.ndim == 2 else 0
    if q is None:
        q = np.zeros((num_rows, H), np.uint8)
    if s is None:
        s = np.zeros((num_rows, H // G), np.uint8)
    assert q.flags.c_contiguous and s.flags.c_contiguous
    lib().ora_scatter_quant(_ptr(x), H, T, H, _ptr(d), K, G, _ptr(q),
                            q.shape[1], _ptr(s), s.shape[1])
    return q, s


def scatter_quant_ex(x_bf16, src2dst, G: int, num_rows: int, rule="ceil",
                     scale_layout="rows", q=None, s=None):
    """scatter_quant with an exponent rule and a scale placement:
    "rows" = uint8 [num_rows, H/G]; "packed_mn" = uint32 [ceil(H/G/4),
    align(num_rows, 4)] holding four scale bytes per word, rows contiguous."""
    x = _c(x_bf16, np.uint16)
    d = _c(src2dst, np.int32)
    T, H = x.shape
    K = d.shape[1]
    ng = H // G
    if q is None:
        q = np.zeros((num_rows, H), np.uint8)
    if scale_layout == "rows":
        if s is None:
            s = np.zeros((num_rows, ng), np.uint8)
        s_rs, s_c4 = s.shape[1], 4
    else:
        ld_mn = -(-num_rows // 4) * 4
        if s is None:
            s = np.zeros((-(-ng // 4), ld_mn), np.uint32)
        s_rs, s_c4 = 4, 4 * s.shape[1]
    lib().ora_scatter_quant_ex(_ptr(x), H, T, H, _ptr(d), K, G, RULES[rule],
                               _ptr(q), q.shape[1], _ptr(s), s_rs, s_c4)
    return q, s


def mfma_scales(scales_rows, H: int, G: int, tile_m: int, out=None,
                fill=0):
    """Reading R16: the scale placement read by gfx950's block-scaled MFMA
    (v_mfma_scale_f32_32x32x64_f8f6f4 for tile_m = 32,
    v_mfma_scale_f32_16x16x128_f8f6f4 for tile_m = 16) when the quantized
    rows are its A operand.  No page fixes this layout; it follows the
    instruction's operands (CDNA4 ISA, block-scaled matrix instructions):
    instruction s of a row tile covers channels [s*KW, (s+1)*KW), KW =
    64*32/tile_m; the scale of its block s*(64/tile_m) + l // tile_m of row
    l % tile_m is read from lane l, byte s % 4 (op_sel) of the lane's 32-bit
    scale register, one register per four instructions.  Stored as
    [row tile, s // 4, lane, s % 4].

    Built here from that instruction-side view: every (tile, word group,
    lane, byte) is filled with the scale of the (row, block) the lane reads,
    the group-G scale of block kb being scales_rows[row, kb*32 // G].
    Positions past the last row or past H/32 blocks keep ``fill`` (or what
    ``out`` holds).  Any dtype is accepted (the tests use labels)."""
    S = np.asarray(scales_rows)
    rows = S.shape[0]
    nkb = H // 32
    hh = 64 // tile_m                     # blocks per instruction
    nkg = -(-nkb // (4 * hh))             # word groups per row tile
    tiles = -(-rows // tile_m)
    if out is None:
        out = np.full((tiles, nkg, 64, 4), fill, S.dtype)
    step = 256
    for t0 in range(0, tiles, step):      # bounded index arrays
        nt = min(step, tiles - t0)
        mt, kg, lane, byte = np.indices((nt, nkg, 64, 4), dtype=np.int64)
        mt += t0
        instr = 4 * kg + byte
        row = mt * tile_m + lane % tile_m
        kb = instr * hh + lane // tile_m
        ok = (row < rows) & (kb < nkb)
        out[t0:t0 + nt][ok] = S[row[ok], (kb[ok] * 32) // G]
    return out


def unpack_mn_scales(packed: np.ndarray, rows: int, ng: int) -> np.ndarray:
    """[ceil(ng/4), ld_mn] uint32 words -> [rows, ng] scale bytes."""
    b = np.ascontiguousarray(packed).view(np.uint8).reshape(
        packed.shape[0], packed.shape[1], 4)
    return np.transpose(b, (1, 0, 2)).reshape(packed.shape[1], -1)[:rows, :ng]


def mx_quant_live_rows(x_bf16, num_segments: int, live_counts, G: int = 32,
                       q=None, s=None):
    x = _c(x_bf16, np.uint16)
    rows, H = x.shape
    rps = rows // num_segments if num_segments else 0
    live = _c(live_counts, np.int32)
    if q is None:
        q = np.zeros((rows, H), np.uint8)
    if s is None:
        s = np.zeros((rows, H // G), np.uint8)
    lib().ora_mx_quant_live_rows(_ptr(x), H, num_segments, rps, _ptr(live), H,
                                 G, _ptr(q), q.shape[1], _ptr(s), s.shape[1])
    return q, s


def requant_per_token_to_per_tensor(q_in, token_scales):
    q = _c(q_in, np.uint8)
    sc = _c(token_scales, np.float32)
    T, H = q.shape
    out = np.empty_like(q)
    S = np.zeros(1, np.float32)
    lib().ora_requant_per_token_to_per_tensor(_ptr(q), H, _ptr(sc), T, H,
                                              _ptr(out), H, _ptr(S))
    return out, float(S[0])


def combine_f32(y_bf16, src2dst, weights):
    """fp32 accumulator of the weighted combine, shape [T, H]."""
    y = _c(y_bf16, np.uint16)
    d = _c(src2dst, np.int32)
    w = _c(weights, np.float32)
    T, K = d.shape
    H = y.shape[1]
    acc = np.empty((T, H), np.float32)
    lib().ora_combine_f32(_ptr(y), H, _ptr(d), _ptr(w), T, K, H, _ptr(acc), H)
    return acc


def combine(y_bf16, src2dst, weights, out_dtype: str = "bf16"):
    acc = combine_f32(y_bf16, src2dst, weights)
    if out_dtype == "f32":
        return acc
    return bf16_round(acc)


def combine_f64(y_bf16, src2dst, weights):
    y = _c(y_bf16, np.uint16)
    d = _c(src2dst, np.int32)
    w = _c(weights, np.float32)
    T, K = d.shape
    H = y.shape[1]
    out = np.empty((T, H), np.float64)
    mag = np.empty((T, H), np.float64)
    lib().ora_combine_f64(_ptr(y), H, _ptr(d), _ptr(w), T, K, H, _ptr(out),
                          _ptr(mag), H)
    return out, mag


# ------------------------------------------------- psum (expanded) layouts

def m_indices_from_psum(psum, align: int, num_rows: int):
    p = _c(psum, np.int32)
    m = np.empty(num_rows, np.int32)
    lib().ora_m_indices_from_psum(_ptr(p), p.size, align, num_rows, _ptr(m))
    return m


def expand_to_masked_slab(x_rows: np.ndarray, psum, align: int, max_m: int,
                          scales: np.ndarray | None = None,
                          scales_col_major: bool = False, slab=None,
                          slab_scales=None):
    """x_rows: [rows, row_bytes] uint8 (any payload as bytes); scales:
    [rows, s_cols] array of 1- or 4-byte elements, stored row-major or (with
    scales_col_major) as the transpose [s_cols, rows].  Returns (slab
    [E, max_m, row_bytes], slab_scales [E, max_m, s_cols] or None, masked_m,
    flags)."""
    x = _c(x_rows, np.uint8)
    rows, rb = x.shape
    p = _c(psum, np.int32)
    E = p.size
    if slab is None:
        slab = np.zeros((E * max_m, rb), np.uint8)
    masked_m = np.empty(E, np.int32)
    xs_ptr = ss_ptr = 0
    xs_rs = xs_cs = ss_rs = ss_cs = s_cols = s_elem = 0
    if scales is not None:
        sc = np.ascontiguousarray(scales)
        s_elem = sc.dtype.itemsize
        if scales_col_major:
            s_cols = sc.shape[0]
            xs_rs, xs_cs = s_elem, sc.shape[1] * s_elem
        else:
            s_cols = sc.shape[1]
            xs_rs, xs_cs = s_cols * s_elem, s_elem
        if slab_scales is None:
            slab_scales = np.zeros((E * max_m, s_cols), sc.dtype)
        ss_rs, ss_cs = s_cols * s_elem, s_elem
        xs_ptr, ss_ptr = _ptr(sc), _ptr(slab_scales)
    flags = lib().ora_expand_to_masked_slab(
        _ptr(x), rb, rows, rb, xs_ptr, xs_rs, xs_cs, s_cols, s_elem, _ptr(p),
        E, align, max_m, _ptr(slab), rb, ss_ptr, ss_rs, ss_cs,
        _ptr(masked_m))
    return slab, slab_scales, masked_m, int(flags)


def masked_slab_to_expand(slab_bf16: np.ndarray, masked_m, psum, align: int,
                          max_m: int, weights=None, out=None,
                          out_rows: int | None = None):
    """slab_bf16: [E*max_m, H] bf16 bits.  out (bf16 bits) is updated in
    place on real rows only."""
    sl = _c(slab_bf16, np.uint16)
    H = sl.shape[1]
    p = _c(psum, np.int32)
    mm = _c(masked_m, np.int32)
    E = p.size
    if out is None:
        out = np.zeros((out_rows, H), np.uint16)
    assert out.flags.c_contiguous
    w = None if weights is None else _c(weights, np.float32)
    lib().ora_masked_slab_to_expand(_ptr(sl), H, H, _ptr(mm), _ptr(p), E,
                                    align, max_m, 0 if w is None else _ptr(w),
                                    _ptr(out), out.shape[1], out.shape[0])
    return out


# ------------------------------------------------ scatter of quantized rows

def scatter_rows(x_rows, src2dst, num_rows: int, scales=None,
                 scales_col_major: bool = False, out=None, out_scales=None,
                 out_scales_col_major: bool = False):
    """x_rows: uint8 [T, row_bytes] payload; scales: [T, cols] (or [cols, T]
    with scales_col_major) of 1- or 4-byte entries.  out / out_scales (same
    entry type, [num_rows, cols] or [cols, num_rows]) are updated in place on
    destination rows only."""
    x = _c(x_rows, np.uint8)
    T, rb = x.shape
    d = _c(src2dst, np.int32)
    K = d.shape[1] if d.ndim == 2 else 1
    if out is None:
        out = np.zeros((num_rows, rb), np.uint8)
    assert out.flags.c_contiguous and out.dtype == np.uint8
    xs_p, xs_rs, xs_cs, cols, elem = 0, 0, 0, 0, 1
    os_p, os_rs, os_cs = 0, 0, 0
    if scales is not None:
        sc = np.ascontiguousarray(scales)
        elem = sc.dtype.itemsize
        cols = sc.shape[0] if scales_col_major else sc.shape[1]
        xs_rs, xs_cs = ((elem, elem * T) if scales_col_major
                        else (elem * cols, elem))
        if out_scales is None:
            out_scales = np.zeros((cols, num_rows) if out_scales_col_major
                                  else (num_rows, cols), sc.dtype)
        assert out_scales.flags.c_contiguous
        os_rs, os_cs = ((elem, elem * num_rows) if out_scales_col_major
                        else (elem * cols, elem))
        xs_p, os_p = _ptr(sc), _ptr(out_scales)
    lib().ora_scatter_rows(_ptr(x), rb, T, rb, xs_p, xs_rs, xs_cs, cols, elem,
                           _ptr(d), K, num_rows, _ptr(out), out.shape[1],
                           os_p, os_rs, os_cs)
    return out, out_scales


# -------------------------------------------------------- receive-side upscale

def upscale_fp8(q, scales, num_rows: int | None = None, G: int = 128,
                scales_col_major: bool = False, out=None):
    """fp8 payload [rows, H] + fp32 group scales -> bf16 bits [rows, H] for
    the first ``num_rows`` rows.  Scales are [rows, H/G] or, with
    ``scales_col_major``, [H/G, rows].  ``out`` rows at or past ``num_rows``
    are left as they are."""
    qq = _c(q, np.uint8)
    rows, H = qq.shape
    n = rows if num_rows is None else num_rows
    sc = _c(scales, np.float32)
    if scales_col_major:
        s_rs, s_cs = 1, sc.shape[1]
    else:
        s_rs, s_cs = sc.shape[1], 1
    if out is None:
        out = np.zeros((rows, H), np.uint16)
    assert out.flags.c_contiguous and out.dtype == np.uint16
    lib().ora_upscale_fp8(_ptr(qq), H, _ptr(sc), s_rs, s_cs, n, H, G,
                          _ptr(out), out.shape[1])
    return out


# --------------------------------------------------- weight-side requant

def requant_weight_block_ue8m0(q, s_inv, block=(128, 128)):
    """q: e4m3 bytes [B, N, K] (or [N, K]); s_inv: fp32 [B, ceil(N/bn),
    ceil(K/bk)].  Returns (q_out bytes, UE8M0 scale bytes [B, nbn, nbk])."""
    qq = _c(q, np.uint8)
    squeeze = qq.ndim == 2
    if squeeze:
        qq = qq[None]
    si = _c(s_inv, np.float32)
    if si.ndim == 2:
        si = si[None]
    B, N, K = qq.shape
    bn, bk = block
    nbn, nbk = -(-N // bn), -(-K // bk)
    assert si.shape == (B, nbn, nbk), si.shape
    q_out = np.empty_like(qq)
    s_out = np.empty((B, nbn, nbk), np.uint8)
    lib().ora_requant_weight_block_ue8m0(
        _ptr(qq), K, N * K, _ptr(si), nbk, nbn * nbk, B, N, K, bn, bk,
        _ptr(q_out), _ptr(s_out), nbk, nbn * nbk)
    if squeeze:
        return q_out[0], s_out[0]
    return q_out, s_out

"""MoE expert-dispatch preprocessing with fp8 e4m3 activations and
power-of-two group scales, on MI355X (gfx950).

Thin Python binding over ``libmxq.so`` (declared in ``include/mxq.h``).  The
functions carry the C names; they check tensor dtypes, shapes and devices,
allocate missing outputs with ``torch.empty`` and pass raw pointers plus the
current HIP stream.  Every step of the path runs in the library's HIP
kernels; there is no CPU or PyTorch fallback: without the built library every
call raises.

Byte formats: fp8 payloads are ``torch.uint8`` tensors holding OCP e4m3fn
bytes (``.view(torch.float8_e4m3fn)`` reinterprets them); a scale byte b
means 2^(b - 127) (``.view(torch.float8_e8m0fnu)``).
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "MxqError", "lib", "SCALE_FORMATS",
    "moe_compact_row_bound", "moe_should_use_masked",
    "moe_layout_workspace_bytes", "requant_workspace_bytes",
    "moe_layout", "moe_read_overflow", "moe_scatter_quant",
    "mx_quant_live_rows", "live_rows_view", "SCALE_RULES",
    "moe_scatter_quant_ex", "mx_quant_live_rows_ex", "packed_mn_scales",
    "requant_per_token_to_per_tensor", "moe_combine", "mxq_e4m3_encode_f32",
    "mxq_abi_version", "moe_m_indices_from_psum", "moe_expand_to_masked_slab",
    "moe_masked_slab_to_expand", "moe_scatter_rows", "upscale_fp8_to_bf16",
    "requant_weight_block_ue8m0", "mxq_mfma_scale_bytes", "mfma_scales",
    "mxq_copy16", "moe_layout_scatter_quant", "moe_layout_noalloc",
    "mxq_gather_read16", "mxq_fill_rows16",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmxq.so")

MXQ_OK = 0
MXQ_ERR_CAPACITY_OVERFLOW = 3
MXQ_ERR_SCRATCH_LIMIT = 6
LAYOUT_NOALLOC_SCRATCH_BYTES = 1 << 20
LAYOUT_KINDS = {"compact": 0, "masked": 1}
SCALE_FORMATS = {"ue8m0_g128": (0, 128), "e8m0_g32": (1, 32)}
SCALE_RULES = {"no_clip": 0, "ocp_floor": 1}
SCALE_LAYOUTS = ("rows", "packed_mn", "mfma32", "mfma16")
OUT_DTYPES = {torch.bfloat16: 0, torch.float32: 1}

_i64, _i32, _p, _sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, \
    ctypes.c_size_t

_SIGNATURES = {
    "moe_compact_row_bound": (_i64, [_i64, _i32, _i32]),
    "moe_should_use_masked": (_i32, [_i32, _i32]),
    "moe_layout_workspace_bytes": (_sz, [_i64, _i32, _i32]),
    "requant_workspace_bytes": (_sz, [_i64, _i32]),
    "moe_layout": (_i32, [_p, _i64, _i32, _i32, _i32, _i32, _i32, _i32, _i64,
                          _p, _p, _p, _p, _p, _p, _p, _sz, _p]),
    "moe_read_overflow": (_i32, [_p, _p, _p]),
    "moe_layout_noalloc": (_i32, [_p, _i64, _i32, _i32, _i32, _i32, _i32,
                                  _i32, _i64, _p, _p, _p, _p, _p, _p, _p]),
    "moe_scatter_quant": (_i32, [_p, _i64, _i64, _i32, _p, _i32, _i32, _p,
                                 _i64, _p, _i64, _i64, _p]),
    "mx_quant_live_rows": (_i32, [_p, _i64, _i32, _i64, _p, _i32, _i32, _p,
                                  _i64, _p, _i64, _p]),
    "moe_scatter_quant_ex": (_i32, [_p, _i64, _i64, _i32, _p, _i32, _i32,
                                    _i32, _p, _i64, _p, _i64, _i64, _i64,
                                    _p]),
    "mx_quant_live_rows_ex": (_i32, [_p, _i64, _i32, _i64, _p, _i32, _i32,
                                     _i32, _p, _i64, _p, _i64, _i64, _p]),
    "requant_per_token_to_per_tensor": (_i32, [_p, _i64, _p, _i64, _i32, _p,
                                               _i64, _p, _p, _sz, _p]),
    "moe_combine": (_i32, [_p, _i64, _i64, _p, _p, _i64, _i32, _i32, _p, _i64,
                           _i32, _p]),
    "mxq_e4m3_encode_f32": (_i32, [_p, _i64, _p, _p]),
    "moe_m_indices_from_psum": (_i32, [_p, _i32, _i32, _i64, _p, _p]),
    "moe_expand_to_masked_slab": (_i32, [_p, _i64, _i64, _i64, _p, _i64, _i64,
                                         _i32, _i32, _p, _i32, _i32, _i32, _p,
                                         _i64, _p, _i64, _i64, _p, _p, _p]),
    "moe_masked_slab_to_expand": (_i32, [_p, _i64, _i32, _p, _p, _i32, _i32,
                                         _i32, _p, _p, _i64, _i64, _p]),
    "moe_scatter_rows": (_i32, [_p, _i64, _i64, _i64, _p, _i64, _i64, _i32,
                                _i32, _p, _i32, _i64, _p, _i64, _p, _i64,
                                _i64, _p]),
    "upscale_fp8_to_bf16": (_i32, [_p, _i64, _p, _i64, _i64, _i64, _i32,
                                   _i32, _p, _i64, _p]),
    "requant_weight_block_ue8m0": (_i32, [_p, _i64, _i64, _p, _i64, _i64,
                                          _i32, _i32, _i32, _i32, _i32, _p,
                                          _p, _i64, _i64, _p]),
    "mxq_mfma_scale_bytes": (_i64, [_i64, _i32, _i32]),
    "moe_scatter_quant_mfma": (_i32, [_p, _i64, _i64, _i32, _p, _i32, _i32,
                                      _i32, _p, _i64, _p, _i32, _i64, _p]),
    "mx_quant_live_rows_mfma": (_i32, [_p, _i64, _i32, _i64, _p, _i32, _i32,
                                       _i32, _p, _i64, _p, _i32, _p]),
    "mxq_copy16": (_i32, [_p, _p, _i64, _i32, _p]),
    "mxq_gather_read16": (_i32, [_p, _i64, _i64, _p, _i64, _i32, _i64, _p,
                                 _p]),
    "mxq_fill_rows16": (_i32, [_p, _i64, _i64, _i64, ctypes.c_uint32, _p]),
    "moe_layout_scatter_quant": (_i32, [_p, _i64, _i32, _i32, _i32, _i32, _i32,
                                        _i32, _i64, _p, _p, _p, _p, _p, _p, _p,
                                        _i64, _i32, _i32, _p, _i64, _p, _i64,
                                        _p]),
    "mxq_status_string": (ctypes.c_char_p, [_i32]),
    "mxq_abi_version": (_i32, []),
}

_lib = None


class MxqError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = lib().mxq_status_string(status).decode()
        super().__init__("%s failed: %s (status %d)" % (fn, msg, status))


def lib() -> ctypes.CDLL:
    """The loaded libmxq.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                "libmxq.so is not built (expected at %s); build it with "
                "`python -m fp8_mx_activation_amd.build`" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(fn: str, status: int) -> None:
    if status != MXQ_OK:
        raise MxqError(fn, status)


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t: torch.Tensor | None) -> int | None:
    if t is None or t.numel() == 0:
        return None
    return t.data_ptr()


def _dev(t: torch.Tensor | None, name: str,
         like: torch.Tensor | None = None) -> None:
    """Every tensor handed to the library must live on the GPU (a host
    pointer would fault the kernel), on the device of the call's inputs."""
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if like is not None and t.device != like.device:
        raise ValueError("%s is on %s, the inputs on %s"
                         % (name, t.device, like.device))


def _at_least(t: torch.Tensor, name: str, rows: int, cols: int) -> None:
    """A 2-D buffer the kernels index up to [rows, cols)."""
    if t.shape[0] < rows or t.shape[1] < cols:
        raise ValueError("%s must be at least [%d, %d], got %s"
                         % (name, rows, cols, tuple(t.shape)))


def _src2dst(src2dst: torch.Tensor, like: torch.Tensor, T: int | None):
    _dev(src2dst, "src2dst", like)
    if src2dst.dtype != torch.int32 or src2dst.dim() != 2 or \
            (T is not None and src2dst.shape[0] != T) or \
            not src2dst.is_contiguous():
        raise ValueError("src2dst must be contiguous int32 [T, K]")
    return src2dst.shape[1]


def _rows(t: torch.Tensor, name: str, dtypes) -> int:
    """Row stride (elements) of a 2-D tensor with unit column stride."""
    if t.dtype not in dtypes:
        raise TypeError("%s: dtype %s not in %s" % (name, t.dtype, dtypes))
    if t.dim() != 2:
        raise ValueError("%s must be 2-D" % name)
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError("%s must have unit column stride" % name)
    return t.stride(0) if t.shape[0] > 1 else max(t.shape[1], t.stride(0))


_FP8 = (torch.uint8, torch.float8_e4m3fn)
_SCALE = (torch.uint8,) + ((torch.float8_e8m0fnu,)
                           if hasattr(torch, "float8_e8m0fnu") else ())


def _u8(t: torch.Tensor) -> torch.Tensor:
    return t if t.dtype == torch.uint8 else t.view(torch.uint8)


def _empty_rows_u8(rows: int, cols: int, device) -> torch.Tensor:
    """[rows, cols] byte tensor whose rows start on 16-byte boundaries (the
    library's vector-row requirement): a view of a padded allocation when
    cols is not a multiple of 16."""
    ld = -(-cols // 16) * 16
    t = torch.empty((rows, ld), dtype=torch.uint8, device=device)
    return t if ld == cols else t[:, :cols]


# ---------------------------------------------------------------- host-only

def moe_compact_row_bound(num_assignments: int, num_local_experts: int,
                          block_e: int = 128) -> int:
    r = lib().moe_compact_row_bound(num_assignments, num_local_experts,
                                    block_e)
    if r < 0:
        raise ValueError("invalid arguments to moe_compact_row_bound")
    return int(r)


def moe_should_use_masked(num_experts: int, num_local_experts: int) -> bool:
    return bool(lib().moe_should_use_masked(num_experts, num_local_experts))


def moe_layout_workspace_bytes(T: int, K: int, E: int) -> int:
    return int(lib().moe_layout_workspace_bytes(T, K, E))


def requant_workspace_bytes(T: int, H: int) -> int:
    return int(lib().requant_workspace_bytes(T, H))


def mxq_abi_version() -> int:
    return int(lib().mxq_abi_version())


def mxq_copy16(src: torch.Tensor, dst: torch.Tensor,
               nontemporal: int = 0) -> torch.Tensor:
    """Bandwidth reference: copy src's bytes into dst with the library's
    16-byte vector copy kernel (see mxq.h).  Both contiguous, same size;
    ``nontemporal`` bit 0 = non-temporal stores, bit 1 = loads."""
    _dev(src, "src")
    _dev(dst, "dst", src)
    if not (src.is_contiguous() and dst.is_contiguous()) or \
            src.numel() * src.element_size() != dst.numel() * dst.element_size():
        raise ValueError("src and dst must be contiguous and the same size")
    st = lib().mxq_copy16(_ptr(src), _ptr(dst),
                          src.numel() * src.element_size(), int(nontemporal),
                          _stream(src))
    _check("mxq_copy16", st)
    return dst


def mxq_gather_read16(rows: torch.Tensor, idx: torch.Tensor,
                      sink: torch.Tensor | None = None) -> torch.Tensor:
    """Bandwidth reference: the combine's gather reads alone (see
    ``mxq_gather_read16`` in mxq.h).  ``rows`` is a 2-D device tensor,
    ``idx`` int32 [groups, group]; returns the per-group XOR words."""
    _dev(rows, "rows")
    _dev(idx, "idx", rows)
    if rows.dim() != 2 or rows.stride(1) != 1:
        raise ValueError("rows must be 2-D with contiguous rows")
    if idx.dtype != torch.int32 or idx.dim() != 2 or not idx.is_contiguous():
        raise ValueError("idx must be contiguous int32 [groups, group]")
    G, g = idx.shape
    es = rows.element_size()
    if sink is None:
        sink = torch.empty(G, dtype=torch.int32, device=rows.device)
    _dev(sink, "sink", rows)
    if sink.dtype != torch.int32 or sink.numel() < G or \
            not sink.is_contiguous():
        raise ValueError("sink must be contiguous int32 with >= groups entries")
    st = lib().mxq_gather_read16(_ptr(rows), rows.stride(0) * es,
                                 rows.shape[0], _ptr(idx), G, g,
                                 rows.shape[1] * es, _ptr(sink),
                                 _stream(rows))
    _check("mxq_gather_read16", st)
    return sink


def mxq_fill_rows16(dst: torch.Tensor, pattern: int = 0) -> torch.Tensor:
    """Bandwidth reference: the combine's row writes alone (see
    ``mxq_fill_rows16`` in mxq.h); fills the 2-D device tensor ``dst``."""
    _dev(dst, "dst")
    if dst.dim() != 2 or dst.stride(1) != 1:
        raise ValueError("dst must be 2-D with contiguous rows")
    es = dst.element_size()
    st = lib().mxq_fill_rows16(_ptr(dst), dst.stride(0) * es, dst.shape[0],
                               dst.shape[1] * es, pattern & 0xFFFFFFFF,
                               _stream(dst))
    _check("mxq_fill_rows16", st)
    return dst


def mxq_mfma_scale_bytes(rows: int, H: int, tile_m: int = 32) -> int:
    """Bytes of the block-scaled MFMA scale placement (see mxq.h)."""
    r = lib().mxq_mfma_scale_bytes(rows, H, tile_m)
    if r < 0:
        raise ValueError("invalid arguments to mxq_mfma_scale_bytes")
    return int(r)


# ------------------------------------------------------------------- layout

def _layout_outputs(ids: torch.Tensor, E: int, num_rows: int,
                    m_indices: bool, out: dict | None) -> dict:
    """The layout's output tensors: those given in ``out`` (checked) or new
    ones on the ids' device."""
    T, K = ids.shape
    o = dict(out or {})

    def get(key, shape):
        t = o.get(key)
        if t is None:
            t = torch.empty(shape, dtype=torch.int32, device=ids.device)
        else:
            _dev(t, "out[%r]" % key, ids)
            if t.dtype != torch.int32 or tuple(t.shape) != tuple(shape) or \
                    not t.is_contiguous():
                raise ValueError("out[%r] must be contiguous int32 %s"
                                 % (key, shape))
        return t

    return dict(counts=get("counts", (E,)),
                expert_offsets=get("expert_offsets", (E + 1,)),
                m_indices=get("m_indices", (num_rows,)) if m_indices else None,
                masked_m=get("masked_m", (E,)),
                src2dst=get("src2dst", (T, K)),
                overflow_flag=get("overflow_flag", (1,)),
                num_rows=num_rows)


def _layout_ids(topk_ids: torch.Tensor) -> torch.Tensor:
    _dev(topk_ids, "topk_ids")
    if topk_ids.dtype != torch.int32 or topk_ids.dim() != 2:
        raise TypeError("topk_ids must be int32 [T, K]")
    return topk_ids.contiguous()


def moe_layout(topk_ids: torch.Tensor, expert_begin: int,
               num_local_experts: int, kind: str = "compact",
               block_e: int = 128, capacity: int = 0,
               num_rows: int | None = None, m_indices: bool = True,
               out: dict | None = None,
               workspace: torch.Tensor | None = None) -> dict:
    """Expert-grouped layout of a top-k routing (see ``moe_layout`` in
    mxq.h).  Returns a dict with ``counts``, ``expert_offsets``,
    ``m_indices`` (or None), ``masked_m``, ``src2dst``, ``overflow_flag``
    (device tensors) and ``num_rows``.  ``out`` may hold preallocated tensors
    under the same keys."""
    ids = _layout_ids(topk_ids)
    T, K = ids.shape
    E = num_local_experts
    k = LAYOUT_KINDS[kind]
    if num_rows is None:
        num_rows = (moe_compact_row_bound(T * K, E, block_e) if k == 0
                    else E * capacity)
    lay = _layout_outputs(ids, E, num_rows, m_indices, out)
    need = moe_layout_workspace_bytes(T, K, E)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8,
                                device=ids.device)
    else:
        _dev(workspace, "workspace", ids)
        if workspace.dtype != torch.uint8 or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous uint8 tensor")
    st = lib().moe_layout(_ptr(ids), T, K, expert_begin, E, k, block_e,
                          capacity, num_rows, _ptr(lay["counts"]),
                          _ptr(lay["expert_offsets"]), _ptr(lay["m_indices"]),
                          _ptr(lay["masked_m"]), _ptr(lay["src2dst"]),
                          _ptr(lay["overflow_flag"]), _ptr(workspace),
                          workspace.numel(), _stream(ids))
    _check("moe_layout", st)
    return lay


def moe_layout_noalloc(topk_ids: torch.Tensor, expert_begin: int,
                       num_local_experts: int, kind: str = "compact",
                       block_e: int = 128, capacity: int = 0,
                       num_rows: int | None = None, m_indices: bool = True,
                       out: dict | None = None) -> dict:
    """``moe_layout`` without a workspace: the library keeps the per-chunk
    counts in its own static device array (see ``moe_layout_noalloc`` in
    mxq.h), so with every output given in ``out`` nothing is allocated.
    Routings that need more than ``LAYOUT_NOALLOC_SCRATCH_BYTES`` of counts
    raise ``MxqError`` (status ``MXQ_ERR_SCRATCH_LIMIT``).  Calls on one
    device share that array: overlapping calls race."""
    ids = _layout_ids(topk_ids)
    T, K = ids.shape
    E = num_local_experts
    k = LAYOUT_KINDS[kind]
    if num_rows is None:
        num_rows = (moe_compact_row_bound(T * K, E, block_e) if k == 0
                    else E * capacity)
    lay = _layout_outputs(ids, E, num_rows, m_indices, out)
    st = lib().moe_layout_noalloc(
        _ptr(ids), T, K, expert_begin, E, k, block_e, capacity, num_rows,
        _ptr(lay["counts"]), _ptr(lay["expert_offsets"]),
        _ptr(lay["m_indices"]), _ptr(lay["masked_m"]), _ptr(lay["src2dst"]),
        _ptr(lay["overflow_flag"]), _stream(ids))
    _check("moe_layout_noalloc", st)
    return lay


def moe_layout_scatter_quant(topk_ids: torch.Tensor, x: torch.Tensor,
                             expert_begin: int, num_local_experts: int,
                             kind: str = "compact", block_e: int = 128,
                             capacity: int = 0, num_rows: int | None = None,
                             fmt: str = "ue8m0_g128", m_indices: bool = True,
                             out: dict | None = None,
                             q: torch.Tensor | None = None,
                             scales: torch.Tensor | None = None):
    """``moe_layout`` and ``moe_scatter_quant`` in one launch, for routings
    of at most 4096 assignments.  Returns ``(layout dict, q, scales)`` with
    the same contents as the two calls."""
    ids = _layout_ids(topk_ids)
    T, K = ids.shape
    E = num_local_experts
    k = LAYOUT_KINDS[kind]
    if num_rows is None:
        num_rows = (moe_compact_row_bound(T * K, E, block_e) if k == 0
                    else E * capacity)
    lay = _layout_outputs(ids, E, num_rows, m_indices, out)
    _dev(x, "x", ids)
    code, G = SCALE_FORMATS[fmt]
    ld_x = _rows(x, "x", (torch.bfloat16,))
    if x.shape[0] != T:
        raise ValueError("x must have one row per token of topk_ids")
    H = x.shape[1]
    if q is None:
        q = _empty_rows_u8(num_rows, H, x.device)
    if scales is None:
        scales = torch.empty((num_rows, H // G), dtype=torch.uint8,
                             device=x.device)
    _dev(q, "q", x)
    _dev(scales, "scales", x)
    qq, ss = _u8(q), _u8(scales)
    ld_q = _rows(qq, "q", (torch.uint8,))
    ld_s = _rows(ss, "scales", (torch.uint8,))
    _at_least(qq, "q", num_rows, H)
    _at_least(ss, "scales", num_rows, H // G)
    st = lib().moe_layout_scatter_quant(
        _ptr(ids), T, K, expert_begin, E, k, block_e, capacity, num_rows,
        _ptr(lay["counts"]), _ptr(lay["expert_offsets"]),
        _ptr(lay["m_indices"]), _ptr(lay["masked_m"]), _ptr(lay["src2dst"]),
        _ptr(lay["overflow_flag"]), _ptr(x), ld_x, H, code, _ptr(qq), ld_q,
        _ptr(ss), ld_s, _stream(ids))
    _check("moe_layout_scatter_quant", st)
    return lay, q, scales


def moe_read_overflow(overflow_flag: torch.Tensor) -> int:
    """Waits for the current stream and returns the flag (0 or 1)."""
    _dev(overflow_flag, "overflow_flag")
    v = ctypes.c_int32(0)
    st = lib().moe_read_overflow(_ptr(overflow_flag), ctypes.addressof(v),
                                 _stream(overflow_flag))
    if st not in (MXQ_OK, MXQ_ERR_CAPACITY_OVERFLOW):
        _check("moe_read_overflow", st)
    return int(v.value)


# ------------------------------------------------------------ quantization

def moe_scatter_quant(x: torch.Tensor, src2dst: torch.Tensor, num_rows: int,
                      fmt: str = "ue8m0_g128", q: torch.Tensor | None = None,
                      scales: torch.Tensor | None = None):
    """Quantize each bf16 token row once and write it to its destination
    rows.  Returns ``(q [num_rows, H] uint8, scales [num_rows, H/G] uint8)``;
    rows that are no destination keep the contents of a given ``q``/
    ``scales`` (uninitialised if allocated here)."""
    _dev(x, "x")
    code, G = SCALE_FORMATS[fmt]
    ld_x = _rows(x, "x", (torch.bfloat16,))
    T, H = x.shape
    K = _src2dst(src2dst, x, T)
    if q is None:
        q = _empty_rows_u8(num_rows, H, x.device)
    if scales is None:
        scales = torch.empty((num_rows, H // G), dtype=torch.uint8,
                             device=x.device)
    _dev(q, "q", x)
    _dev(scales, "scales", x)
    qq, ss = _u8(q), _u8(scales)
    ld_q = _rows(qq, "q", (torch.uint8,))
    ld_s = _rows(ss, "scales", (torch.uint8,))
    _at_least(qq, "q", num_rows, H)
    _at_least(ss, "scales", num_rows, H // G)
    st = lib().moe_scatter_quant(_ptr(x), ld_x, T, H, _ptr(src2dst), K, code,
                                 _ptr(qq), ld_q, _ptr(ss), ld_s, num_rows,
                                 _stream(x))
    _check("moe_scatter_quant", st)
    return q, scales


def mx_quant_live_rows(x: torch.Tensor, num_segments: int,
                       live_counts: torch.Tensor, fmt: str = "e8m0_g32",
                       q: torch.Tensor | None = None,
                       scales: torch.Tensor | None = None):
    """Send-side quant of the live rows of a padded buffer of
    ``num_segments`` equal segments (live rows at the head of each).
    Returns the padded ``(q, scales)``; only live rows are written."""
    _dev(x, "x")
    _dev(live_counts, "live_counts", x)
    code, G = SCALE_FORMATS[fmt]
    ld_x = _rows(x, "x", (torch.bfloat16,))
    rows, H = x.shape
    if num_segments <= 0 or rows % num_segments:
        raise ValueError("rows must split into num_segments equal segments")
    if live_counts.dtype != torch.int32 or live_counts.numel() != \
            num_segments or not live_counts.is_contiguous():
        raise ValueError("live_counts must be contiguous int32 [segments]")
    if q is None:
        q = _empty_rows_u8(rows, H, x.device)
    if scales is None:
        scales = torch.empty((rows, H // G), dtype=torch.uint8,
                             device=x.device)
    _dev(q, "q", x)
    _dev(scales, "scales", x)
    qq, ss = _u8(q), _u8(scales)
    ld_q = _rows(qq, "q", (torch.uint8,))
    ld_s = _rows(ss, "scales", (torch.uint8,))
    _at_least(qq, "q", rows, H)
    _at_least(ss, "scales", rows, H // G)
    st = lib().mx_quant_live_rows(_ptr(x), ld_x, num_segments,
                                  rows // num_segments, _ptr(live_counts), H,
                                  code, _ptr(qq), ld_q, _ptr(ss), ld_s,
                                  _stream(x))
    _check("mx_quant_live_rows", st)
    return q, scales


def packed_mn_scales(rows: int, groups: int, device) -> torch.Tensor:
    """Empty packed MN-major scale tensor: int32 ``[ceil(groups/4),
    align(rows, 4)]``, four scale bytes per word (group g of row r in byte
    g % 4 of word ``[g // 4, r]``), rows contiguous."""
    return torch.empty((-(-groups // 4), -(-rows // 4) * 4),
                       dtype=torch.int32, device=device)


def mfma_scales(rows: int, H: int, tile_m: int, device) -> torch.Tensor:
    """Empty scale buffer in the block-scaled MFMA placement: uint8
    ``[ceil(rows/tile_m), nkg, 64, 4]`` = (row tile, group of four
    instructions, lane, op_sel byte); see ``mxq_mfma_scale_bytes``."""
    n = mxq_mfma_scale_bytes(rows, H, tile_m)
    tiles = -(-rows // tile_m)
    nkg = n // (256 * tiles) if tiles else -(-(H // 32) // (4 * 64 // tile_m))
    return torch.empty((tiles, nkg, 64, 4), dtype=torch.uint8, device=device)


def _mfma_place(scales: torch.Tensor | None, layout: str, rows: int, H: int,
                like: torch.Tensor):
    """(tensor, tile_m) for an MFMA placement; allocates when none given."""
    tm = int(layout[4:])
    if scales is None:
        return mfma_scales(rows, H, tm, like.device), tm
    _dev(scales, "scales", like)
    need = mxq_mfma_scale_bytes(rows, H, tm)
    if scales.dtype != torch.uint8 or not scales.is_contiguous() or \
            scales.numel() < need:
        raise ValueError("MFMA-placed scales must be contiguous uint8 with "
                         ">= %d bytes" % need)
    return scales, tm


def _scale_place(scales: torch.Tensor | None, layout: str, rows: int,
                 groups: int, like: torch.Tensor):
    """(tensor, byte pointer tensor, row stride, quad stride) for a scale
    placement; allocates the tensor on ``like``'s device when none is
    given."""
    _dev(scales, "scales", like)
    device = like.device
    if layout == "rows":
        if scales is None:
            scales = torch.empty((rows, groups), dtype=torch.uint8,
                                 device=device)
        ss = _u8(scales)
        ld = _rows(ss, "scales", (torch.uint8,))
        if ss.shape[0] < rows or ss.shape[1] < groups:
            raise ValueError("scales must be at least [%d, %d]"
                             % (rows, groups))
        return scales, ss, ld, 4
    if layout != "packed_mn":
        raise ValueError("scale_layout must be one of %s" % (SCALE_LAYOUTS,))
    if scales is None:
        scales = packed_mn_scales(rows, groups, device)
    if scales.dtype != torch.int32 or scales.dim() != 2 or \
            scales.shape[0] < -(-groups // 4) or scales.shape[1] < rows or \
            (scales.shape[0] > 1 and scales.stride(1) != 1):
        raise ValueError("packed scales must be int32 [ceil(groups/4), >= "
                         "rows] with rows contiguous")
    return scales, scales, 4, 4 * scales.stride(0)


def moe_scatter_quant_ex(x: torch.Tensor, src2dst: torch.Tensor,
                         num_rows: int, fmt: str = "ue8m0_g128",
                         rule: str = "no_clip", scale_layout: str = "rows",
                         q: torch.Tensor | None = None,
                         scales: torch.Tensor | None = None):
    """``moe_scatter_quant`` with an exponent ``rule`` (``"no_clip"`` or
    ``"ocp_floor"``) and a ``scale_layout``: ``"rows"`` (uint8 [rows,
    groups]), ``"packed_mn"`` (see ``packed_mn_scales``) or ``"mfma32"`` /
    ``"mfma16"``, the block-scaled MFMA operand order (see
    ``mfma_scales``)."""
    _dev(x, "x")
    code, G = SCALE_FORMATS[fmt]
    ld_x = _rows(x, "x", (torch.bfloat16,))
    T, H = x.shape
    K = _src2dst(src2dst, x, T)
    if q is None:
        q = _empty_rows_u8(num_rows, H, x.device)
    _dev(q, "q", x)
    qq = _u8(q)
    ld_q = _rows(qq, "q", (torch.uint8,))
    _at_least(qq, "q", num_rows, H)
    if scale_layout in ("mfma32", "mfma16"):
        scales, tm = _mfma_place(scales, scale_layout, num_rows, H, x)
        st = lib().moe_scatter_quant_mfma(
            _ptr(x), ld_x, T, H, _ptr(src2dst), K, code, SCALE_RULES[rule],
            _ptr(qq), ld_q, _ptr(scales), tm, num_rows, _stream(x))
        _check("moe_scatter_quant_mfma", st)
        return q, scales
    scales, sp, rs, c4 = _scale_place(scales, scale_layout, num_rows, H // G,
                                      x)
    st = lib().moe_scatter_quant_ex(_ptr(x), ld_x, T, H, _ptr(src2dst), K,
                                    code, SCALE_RULES[rule], _ptr(qq), ld_q,
                                    _ptr(sp), rs, c4, num_rows, _stream(x))
    _check("moe_scatter_quant_ex", st)
    return q, scales


def mx_quant_live_rows_ex(x: torch.Tensor, num_segments: int,
                          live_counts: torch.Tensor, fmt: str = "e8m0_g32",
                          rule: str = "no_clip", scale_layout: str = "rows",
                          q: torch.Tensor | None = None,
                          scales: torch.Tensor | None = None):
    """``mx_quant_live_rows`` with an exponent rule and scale layout as in
    ``moe_scatter_quant_ex``."""
    _dev(x, "x")
    _dev(live_counts, "live_counts", x)
    code, G = SCALE_FORMATS[fmt]
    ld_x = _rows(x, "x", (torch.bfloat16,))
    rows, H = x.shape
    if num_segments <= 0 or rows % num_segments:
        raise ValueError("rows must split into num_segments equal segments")
    if live_counts.dtype != torch.int32 or live_counts.numel() != \
            num_segments or not live_counts.is_contiguous():
        raise ValueError("live_counts must be contiguous int32 [segments]")
    if q is None:
        q = _empty_rows_u8(rows, H, x.device)
    _dev(q, "q", x)
    qq = _u8(q)
    ld_q = _rows(qq, "q", (torch.uint8,))
    _at_least(qq, "q", rows, H)
    if scale_layout in ("mfma32", "mfma16"):
        scales, tm = _mfma_place(scales, scale_layout, rows, H, x)
        st = lib().mx_quant_live_rows_mfma(
            _ptr(x), ld_x, num_segments, rows // num_segments,
            _ptr(live_counts), H, code, SCALE_RULES[rule], _ptr(qq), ld_q,
            _ptr(scales), tm, _stream(x))
        _check("mx_quant_live_rows_mfma", st)
        return q, scales
    scales, sp, rs, c4 = _scale_place(scales, scale_layout, rows, H // G,
                                      x)
    st = lib().mx_quant_live_rows_ex(_ptr(x), ld_x, num_segments,
                                     rows // num_segments, _ptr(live_counts),
                                     H, code, SCALE_RULES[rule], _ptr(qq),
                                     ld_q, _ptr(sp), rs, c4, _stream(x))
    _check("mx_quant_live_rows_ex", st)
    return q, scales


def live_rows_view(q: torch.Tensor, scales: torch.Tensor, num_segments: int,
                   live_counts_host):
    """Host-side view of the live rows only: ``(q[n_live, H],
    scales[n_live, H/G])``, which is ``(0, H/G)`` for an empty batch."""
    rows = q.shape[0]
    rps = rows // num_segments
    sel = []
    for g, n in enumerate(list(live_counts_host)):
        n = max(0, min(int(n), rps))
        sel.append((g * rps, g * rps + n))
    if len(sel) == 1 or sum(b - a > 0 for a, b in sel) <= 1:
        a, b = next(((a, b) for a, b in sel if b > a), (0, 0))
        return q[a:b], scales[a:b]
    return (torch.cat([q[a:b] for a, b in sel]),
            torch.cat([scales[a:b] for a, b in sel]))


def requant_per_token_to_per_tensor(q_in: torch.Tensor,
                                    token_scales: torch.Tensor,
                                    q_out: torch.Tensor | None = None,
                                    tensor_scale: torch.Tensor | None = None,
                                    workspace: torch.Tensor | None = None):
    """fp8 rows with per-token fp32 scales -> fp8 rows with one fp32 scale.
    Returns ``(q_out uint8 [T, H], tensor_scale float32 [1])``."""
    _dev(q_in, "q_in")
    qi = _u8(q_in)
    ld_in = _rows(qi, "q_in", (torch.uint8,))
    T, H = qi.shape
    _dev(token_scales, "token_scales", qi)
    if token_scales.dtype != torch.float32 or token_scales.numel() != T or \
            not token_scales.is_contiguous():
        raise ValueError("token_scales must be contiguous float32 [T]")
    if q_out is None:
        q_out = _empty_rows_u8(T, H, qi.device)
    _dev(q_out, "q_out", qi)
    qo = _u8(q_out)
    ld_out = _rows(qo, "q_out", (torch.uint8,))
    _at_least(qo, "q_out", T, H)
    if tensor_scale is None:
        tensor_scale = torch.empty(1, dtype=torch.float32, device=qi.device)
    _dev(tensor_scale, "tensor_scale", qi)
    if tensor_scale.dtype != torch.float32 or tensor_scale.numel() < 1:
        raise ValueError("tensor_scale must be float32 with one element")
    need = requant_workspace_bytes(T, H)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=qi.device)
    else:
        _dev(workspace, "workspace", qi)
        if workspace.dtype != torch.uint8 or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous uint8 tensor")
    st = lib().requant_per_token_to_per_tensor(
        _ptr(qi), ld_in, _ptr(token_scales), T, H, _ptr(qo), ld_out,
        tensor_scale.data_ptr(), _ptr(workspace), workspace.numel(),
        _stream(qi))
    _check("requant_per_token_to_per_tensor", st)
    return q_out, tensor_scale


def moe_combine(y: torch.Tensor, src2dst: torch.Tensor,
                topk_weights: torch.Tensor,
                out_dtype: torch.dtype = torch.bfloat16,
                out: torch.Tensor | None = None) -> torch.Tensor:
    """Weighted un-permute of expert outputs ``y [num_rows, H]`` (bf16) back
    to tokens: ``out [T, H]`` in bf16 or float32."""
    _dev(y, "y")
    ld_y = _rows(y, "y", (torch.bfloat16,))
    num_rows, H = y.shape
    K = _src2dst(src2dst, y, None)
    T = src2dst.shape[0]
    _dev(topk_weights, "topk_weights", y)
    if topk_weights.dtype != torch.float32 or \
            tuple(topk_weights.shape) != (T, K) or \
            not topk_weights.is_contiguous():
        raise ValueError("topk_weights must be contiguous float32 [T, K]")
    if out is None:
        out = torch.empty((T, H), dtype=out_dtype, device=y.device)
    _dev(out, "out", y)
    if out.dtype not in OUT_DTYPES:
        raise TypeError("out dtype must be one of %s" % list(OUT_DTYPES))
    code = OUT_DTYPES[out.dtype]
    ld_out = _rows(out, "out", (out.dtype,))
    _at_least(out, "out", T, H)
    st = lib().moe_combine(_ptr(y), ld_y, num_rows, _ptr(src2dst),
                           _ptr(topk_weights), T, K, H, _ptr(out), ld_out,
                           code, _stream(y))
    _check("moe_combine", st)
    return out


def mxq_e4m3_encode_f32(x: torch.Tensor) -> torch.Tensor:
    """The kernels' fp32 -> e4m3fn conversion, element by element."""
    _dev(x, "x")
    if x.dtype != torch.float32:
        raise TypeError("x must be float32")
    xc = x.contiguous()
    out = torch.empty(xc.shape, dtype=torch.uint8, device=x.device)
    st = lib().mxq_e4m3_encode_f32(_ptr(xc), xc.numel(), _ptr(out),
                                   _stream(xc))
    _check("mxq_e4m3_encode_f32", st)
    return out


# ---------------------------------------------------- psum (expanded) layout

def _psum(psum: torch.Tensor) -> torch.Tensor:
    _dev(psum, "psum")
    if psum.dtype != torch.int32 or psum.dim() != 1 or \
            not psum.is_contiguous():
        raise ValueError("psum must be contiguous int32 [E]")
    return psum


def moe_m_indices_from_psum(psum: torch.Tensor, num_rows: int,
                            align: int = 128,
                            out: torch.Tensor | None = None) -> torch.Tensor:
    """m_indices [num_rows] of the contiguous GEMM from a dispatcher's
    psum: e on rows [align(psum[e-1]), psum[e]), -1 elsewhere."""
    p = _psum(psum)
    if out is None:
        out = torch.empty(num_rows, dtype=torch.int32, device=p.device)
    _dev(out, "out", p)
    if out.dtype != torch.int32 or out.numel() < num_rows or \
            not out.is_contiguous():
        raise ValueError("out must be contiguous int32 with >= num_rows "
                         "entries")
    st = lib().moe_m_indices_from_psum(_ptr(p), p.numel(), align, num_rows,
                                       _ptr(out), _stream(p))
    _check("moe_m_indices_from_psum", st)
    return out


def moe_expand_to_masked_slab(x: torch.Tensor, psum: torch.Tensor,
                              max_m: int, align: int = 128,
                              scales: torch.Tensor | None = None,
                              scales_col_major: bool = False,
                              slab: torch.Tensor | None = None,
                              slab_scales: torch.Tensor | None = None):
    """Expanded rows ``x [rows, cols]`` (any element type) -> masked slab
    ``[E * max_m, cols]``.  ``scales`` is ``[rows, s_cols]``, or its
    transpose stored as ``[s_cols, rows]`` when ``scales_col_major``.
    Returns ``(slab, slab_scales, masked_m, flags)`` (device tensors)."""
    _dev(x, "x")
    p = _psum(psum)
    _dev(p, "psum", x)
    E = p.numel()
    if x.dim() != 2 or (x.shape[1] > 1 and x.stride(1) != 1):
        raise ValueError("x must be 2-D with unit column stride")
    esz = x.element_size()
    rows, cols = x.shape
    ld_x = (x.stride(0) if rows > 1 else cols) * esz
    if slab is None:
        slab = torch.empty((E * max_m, cols), dtype=x.dtype, device=x.device)
    _dev(slab, "slab", x)
    if slab.dim() != 2 or slab.element_size() != esz or \
            (slab.shape[1] > 1 and slab.stride(1) != 1):
        raise ValueError("slab must be 2-D, unit column stride, with x's "
                         "element size")
    _at_least(slab, "slab", E * max_m, cols)
    ld_slab = (slab.stride(0) if slab.shape[0] > 1 else cols) * esz
    masked_m = torch.empty(E, dtype=torch.int32, device=x.device)
    flags = torch.empty(1, dtype=torch.int32, device=x.device)
    xs_rs = xs_cs = ss_rs = ss_cs = s_cols = s_elem = 0
    if scales is not None:
        _dev(scales, "scales", x)
        s_elem = scales.element_size()
        if scales.dim() != 2:
            raise ValueError("scales must be 2-D")
        if scales_col_major:
            s_cols = scales.shape[0]
            if scales.shape[1] < rows:
                raise ValueError("column-major scales need >= %d columns"
                                 % rows)
            xs_rs, xs_cs = scales.stride(1) * s_elem, scales.stride(0) * s_elem
        else:
            s_cols = scales.shape[1]
            if scales.shape[0] < rows:
                raise ValueError("scales need >= %d rows" % rows)
            xs_rs, xs_cs = scales.stride(0) * s_elem, scales.stride(1) * s_elem
        if slab_scales is None:
            slab_scales = torch.empty((E * max_m, s_cols), dtype=scales.dtype,
                                      device=x.device)
        _dev(slab_scales, "slab_scales", x)
        if slab_scales.dim() != 2 or slab_scales.element_size() != s_elem:
            raise ValueError("slab_scales must be 2-D with the scales' "
                             "entry size")
        _at_least(slab_scales, "slab_scales", E * max_m, s_cols)
        ss_rs = slab_scales.stride(0) * s_elem
        ss_cs = slab_scales.stride(1) * s_elem
    st = lib().moe_expand_to_masked_slab(
        _ptr(x), ld_x, rows, cols * esz, _ptr(scales), xs_rs, xs_cs, s_cols,
        s_elem, _ptr(p), E, align, max_m, _ptr(slab), ld_slab,
        _ptr(slab_scales), ss_rs, ss_cs, _ptr(masked_m), _ptr(flags),
        _stream(x))
    _check("moe_expand_to_masked_slab", st)
    return slab, slab_scales, masked_m, flags


def moe_masked_slab_to_expand(slab: torch.Tensor, masked_m: torch.Tensor,
                              psum: torch.Tensor, max_m: int,
                              align: int = 128,
                              weights: torch.Tensor | None = None,
                              out: torch.Tensor | None = None,
                              out_rows: int | None = None) -> torch.Tensor:
    """bf16 slab ``[E * max_m, H]`` -> expanded rows of ``out [rows, H]``
    (real rows only), multiplied by ``weights [rows]`` when given."""
    _dev(slab, "slab")
    p = _psum(psum)
    _dev(p, "psum", slab)
    E = p.numel()
    _dev(masked_m, "masked_m", slab)
    if masked_m.dtype != torch.int32 or masked_m.numel() < E or \
            not masked_m.is_contiguous():
        raise ValueError("masked_m must be contiguous int32 [E]")
    ld_slab = _rows(slab, "slab", (torch.bfloat16,))
    H = slab.shape[1]
    _at_least(slab, "slab", E * max_m, H)
    if out is None:
        if out_rows is None:
            raise ValueError("give out or out_rows")
        out = torch.zeros((out_rows, H), dtype=torch.bfloat16,
                          device=slab.device)
    _dev(out, "out", slab)
    ld_out = _rows(out, "out", (torch.bfloat16,))
    _at_least(out, "out", 0, H)
    _dev(weights, "weights", slab)
    if weights is not None and (weights.dtype != torch.float32 or
                                not weights.is_contiguous() or
                                weights.numel() < out.shape[0]):
        raise ValueError("weights must be contiguous float32 [rows]")
    st = lib().moe_masked_slab_to_expand(
        _ptr(slab), ld_slab, H, _ptr(masked_m), _ptr(p), p.numel(), align,
        max_m, _ptr(weights), _ptr(out), ld_out, out.shape[0], _stream(slab))
    _check("moe_masked_slab_to_expand", st)
    return out


# ------------------------------------------------ scatter of quantized rows

def _scale_strides(t: torch.Tensor, col_major: bool, rows: int, name: str):
    """(row stride, column stride) in bytes and column count of a 2-D scale
    tensor stored [rows, cols] or, when col_major, [cols, rows]."""
    if t.dim() != 2:
        raise ValueError("%s must be 2-D" % name)
    e = t.element_size()
    if col_major:
        cols = t.shape[0]
        if t.shape[1] < rows or (t.shape[1] > 1 and t.stride(1) != 1):
            raise ValueError("%s must be [cols, >= %d] with unit row stride"
                             % (name, rows))
        return e, e * t.stride(0), cols
    cols = t.shape[1]
    if t.shape[0] < rows or (cols > 1 and t.stride(1) != 1):
        raise ValueError("%s must be [>= %d, cols] with unit column stride"
                         % (name, rows))
    return e * t.stride(0), e, cols


def moe_scatter_rows(x: torch.Tensor, src2dst: torch.Tensor, num_rows: int,
                     scales: torch.Tensor | None = None,
                     scales_col_major: bool = False,
                     out: torch.Tensor | None = None,
                     out_scales: torch.Tensor | None = None,
                     out_scales_col_major: bool = False):
    """Already-quantized rows (any 1-byte payload, e.g. fp8) and optional
    scales (1- or 4-byte entries) copied to their destination rows in
    ``src2dst``.  Returns ``(out, out_scales)``; rows that are no
    destination keep the contents of a given ``out``."""
    _dev(x, "x")
    xx = _u8(x)
    ld_x = _rows(xx, "x", (torch.uint8,))
    T, rb = xx.shape
    K = _src2dst(src2dst, x, T)
    if out is None:
        out = _empty_rows_u8(num_rows, rb, x.device)
    _dev(out, "out", x)
    oo = _u8(out)
    ld_o = _rows(oo, "out", (torch.uint8,))
    if oo.shape[0] < num_rows or oo.shape[1] < rb:
        raise ValueError("out must be at least [num_rows, row bytes]")
    xs_rs = xs_cs = os_rs = os_cs = 0
    cols, elem = 0, 1
    if scales is not None:
        _dev(scales, "scales", x)
        elem = scales.element_size()
        xs_rs, xs_cs, cols = _scale_strides(scales, scales_col_major, T,
                                            "scales")
        if out_scales is None:
            shape = (cols, num_rows) if out_scales_col_major else \
                (num_rows, cols)
            out_scales = torch.empty(shape, dtype=scales.dtype,
                                     device=x.device)
        _dev(out_scales, "out_scales", x)
        if out_scales.element_size() != elem:
            raise TypeError("out_scales must have the scales' entry size")
        os_rs, os_cs, ocols = _scale_strides(out_scales, out_scales_col_major,
                                             num_rows, "out_scales")
        if ocols < cols:
            raise ValueError("out_scales has fewer columns than scales")
    st = lib().moe_scatter_rows(_ptr(xx), ld_x, T, rb, _ptr(scales), xs_rs,
                                xs_cs, cols, elem, _ptr(src2dst), K, num_rows,
                                _ptr(oo), ld_o, _ptr(out_scales), os_rs,
                                os_cs, _stream(x))
    _check("moe_scatter_rows", st)
    return out, out_scales


# ---------------------------------------------------- receive-side upscale

def upscale_fp8_to_bf16(q: torch.Tensor, scales: torch.Tensor,
                        num_rows: int | None = None, group: int = 128,
                        scales_col_major: bool = False,
                        out: torch.Tensor | None = None) -> torch.Tensor:
    """fp8 rows + fp32 group scales -> bf16 rows for the first ``num_rows``
    rows.  ``scales`` is [rows, H/group], or [H/group, rows] with
    ``scales_col_major``.  Rows of ``out`` at or past ``num_rows`` keep
    their contents."""
    _dev(q, "q")
    _dev(scales, "scales", q)
    qq = _u8(q)
    ld_q = _rows(qq, "q", (torch.uint8,))
    rows, H = qq.shape
    n = rows if num_rows is None else int(num_rows)
    if not 0 <= n <= rows:
        raise ValueError("num_rows out of range")
    if scales.dtype != torch.float32 or scales.dim() != 2:
        raise TypeError("scales must be fp32 2-D")
    ng = H // group if group else 0
    if scales_col_major:
        if scales.shape[0] < ng or scales.shape[1] < n or \
                (scales.shape[0] > 1 and scales.stride(1) != 1):
            raise ValueError("column-major scales must be [H/group, >= rows]")
        s_rs, s_cs = 1, scales.stride(0)
    else:
        if scales.shape[0] < n or scales.shape[1] < ng or \
                (scales.shape[1] > 1 and scales.stride(1) != 1):
            raise ValueError("scales must be [>= rows, H/group]")
        s_rs, s_cs = scales.stride(0), 1
    if out is None:
        out = torch.empty((rows, H), dtype=torch.bfloat16, device=q.device)
    _dev(out, "out", q)
    ld_o = _rows(out, "out", (torch.bfloat16,))
    _at_least(out, "out", n, H)
    st = lib().upscale_fp8_to_bf16(_ptr(qq), ld_q, _ptr(scales), s_rs, s_cs,
                                   n, H, group, _ptr(out), ld_o, _stream(q))
    _check("upscale_fp8_to_bf16", st)
    return out


# --------------------------------------------------- weight-side requant

def requant_weight_block_ue8m0(q: torch.Tensor, s_inv: torch.Tensor,
                               block=(128, 128), q_out: torch.Tensor | None =
                               None, scales_out: torch.Tensor | None = None,
                               inplace: bool = False):
    """Block-scaled fp8 weights [B, N, K] (or [N, K]) with fp32 inverse
    scales [B, ceil(N/128), ceil(K/128)] -> (fp8 weights, UE8M0 scale bytes
    [B, nbn, nbk]).  ``inplace`` writes the weights over ``q``."""
    _dev(q, "q")
    _dev(s_inv, "s_inv", q)
    _dev(q_out, "q_out", q)
    _dev(scales_out, "scales_out", q)
    qq = _u8(q)
    squeeze = qq.dim() == 2
    q3 = qq.unsqueeze(0) if squeeze else qq
    s3 = s_inv.unsqueeze(0) if s_inv.dim() == 2 else s_inv
    if q3.dim() != 3 or not q3.is_contiguous():
        raise ValueError("q must be contiguous [B, N, K] or [N, K]")
    if s3.dtype != torch.float32 or s3.dim() != 3 or not s3.is_contiguous():
        raise ValueError("s_inv must be contiguous fp32 [B, nbn, nbk]")
    B, N, K = q3.shape
    bn, bk = block
    nbn, nbk = -(-N // bn) if bn else 0, -(-K // bk) if bk else 0
    if tuple(s3.shape) != (B, nbn, nbk):
        raise ValueError("s_inv must be [%d, %d, %d]" % (B, nbn, nbk))
    if inplace:
        qo = q3
    elif q_out is None:
        qo = torch.empty_like(q3)
    else:
        qo = _u8(q_out)
        qo = qo.unsqueeze(0) if qo.dim() == 2 else qo
        if tuple(qo.shape) != (B, N, K) or not qo.is_contiguous():
            raise ValueError("q_out must match q")
    if scales_out is None:
        so = torch.empty((B, nbn, nbk), dtype=torch.uint8, device=q.device)
    else:
        so = _u8(scales_out)
        so = so.unsqueeze(0) if so.dim() == 2 else so
        if tuple(so.shape) != (B, nbn, nbk) or not so.is_contiguous():
            raise ValueError("scales_out must be [%d, %d, %d]" % (B, nbn, nbk))
    st = lib().requant_weight_block_ue8m0(
        _ptr(q3), K, N * K, _ptr(s3), nbk, nbn * nbk, B, N, K, bn, bk,
        _ptr(qo), _ptr(so), nbk, nbn * nbk, _stream(q))
    _check("requant_weight_block_ue8m0", st)
    if squeeze:
        return qo[0], so[0]
    return qo, so

"""The binding refuses, before anything is launched, a host tensor in any
argument of a call whose inputs are on the GPU, and an output buffer smaller
than what the kernels write: a host pointer or a short buffer would make the
kernel fault instead of failing with an error."""
import pytest
import torch

import fp8_mx_activation_amd as mxq
from gpu_util import DEV

pytestmark = pytest.mark.gpu

T, K, H, R = 4, 2, 256, 8

# entry points that launch nothing; every other one is replaced below
HOST_ONLY = {"moe_compact_row_bound", "moe_should_use_masked",
             "moe_layout_workspace_bytes", "requant_workspace_bytes",
             "mxq_status_string", "mxq_abi_version", "mxq_mfma_scale_bytes"}


class NoLaunch:
    """Stands in for the library: a refusal the binding misses fails the
    test here instead of reaching a kernel."""

    def __init__(self, real):
        self._real = real

    def __getattr__(self, name):
        if name in HOST_ONLY:
            return getattr(self._real, name)

        def reached(*args):
            raise AssertionError("%s reached the library" % name)
        return reached


@pytest.fixture(autouse=True)
def no_launch(monkeypatch):
    monkeypatch.setattr(mxq, "_lib", NoLaunch(mxq.lib()))


# The case tables take the factory of the tensors that should be on the GPU;
# they are built with the host factory only to list the case names.


def gpu(*shape, dtype=torch.uint8):
    return torch.zeros(shape, dtype=dtype, device=DEV)


def h(*shape, dtype=torch.uint8):
    return torch.zeros(shape, dtype=dtype)


def host_argument_calls(g):
    x = g(T, H, dtype=torch.bfloat16)
    ids = g(T, K, dtype=torch.int32)
    w = g(T, K, dtype=torch.float32)
    q = g(T, H)
    lc = g(2, dtype=torch.int32)
    ps = g(4, dtype=torch.int32)
    return {
        "layout out": lambda: mxq.moe_layout(
            ids, 0, 4, out={"counts": h(4, dtype=torch.int32)}),
        "layout workspace": lambda: mxq.moe_layout(
            g(2048, K, dtype=torch.int32), 0, 4, workspace=h(1 << 20)),
        "scatter src2dst": lambda: mxq.moe_scatter_quant(
            x, h(T, K, dtype=torch.int32), R),
        "scatter q": lambda: mxq.moe_scatter_quant(x, ids, R, q=h(R, H)),
        "scatter scales": lambda: mxq.moe_scatter_quant(
            x, ids, R, scales=h(R, H // 128)),
        "scatter_ex src2dst": lambda: mxq.moe_scatter_quant_ex(
            x, h(T, K, dtype=torch.int32), R),
        "scatter_ex packed scales": lambda: mxq.moe_scatter_quant_ex(
            x, ids, R, scale_layout="packed_mn",
            scales=h(1, R, dtype=torch.int32)),  # packed [ceil(2/4), 8]
        "scatter_ex mfma scales": lambda: mxq.moe_scatter_quant_ex(
            x, ids, R, scale_layout="mfma32", scales=h(1, 1, 64, 4)),
        "live counts": lambda: mxq.mx_quant_live_rows(
            x, 2, h(2, dtype=torch.int32)),
        "live q": lambda: mxq.mx_quant_live_rows(x, 2, lc, q=h(T, H)),
        "live_ex scales": lambda: mxq.mx_quant_live_rows_ex(
            x, 2, lc, scales=h(T, H // 32)),
        "requant token scales": lambda: mxq.requant_per_token_to_per_tensor(
            q, h(T, dtype=torch.float32)),
        "requant tensor scale": lambda: mxq.requant_per_token_to_per_tensor(
            q, g(T, dtype=torch.float32), tensor_scale=h(1, dtype=torch.float32)),
        "combine src2dst": lambda: mxq.moe_combine(
            x, h(T, K, dtype=torch.int32), w),
        "combine weights": lambda: mxq.moe_combine(
            x, ids, h(T, K, dtype=torch.float32)),
        "combine out": lambda: mxq.moe_combine(
            x, ids, w, out=h(T, H, dtype=torch.bfloat16)),
        "m_indices out": lambda: mxq.moe_m_indices_from_psum(
            ps, 16, out=h(16, dtype=torch.int32)),
        "expand psum": lambda: mxq.moe_expand_to_masked_slab(
            q, h(4, dtype=torch.int32), 16),
        "expand slab": lambda: mxq.moe_expand_to_masked_slab(
            q, ps, 16, slab=h(64, H)),
        "expand scales": lambda: mxq.moe_expand_to_masked_slab(
            q, ps, 16, scales=h(T, 2)),
        "slab masked_m": lambda: mxq.moe_masked_slab_to_expand(
            g(64, H, dtype=torch.bfloat16), h(4, dtype=torch.int32), ps, 16,
            out_rows=8),
        "slab weights": lambda: mxq.moe_masked_slab_to_expand(
            g(64, H, dtype=torch.bfloat16), ps, ps, 16, out_rows=8,
            weights=h(8, dtype=torch.float32)),
        "scatter_rows src2dst": lambda: mxq.moe_scatter_rows(
            q, h(T, K, dtype=torch.int32), R),
        "scatter_rows out": lambda: mxq.moe_scatter_rows(q, ids, R,
                                                         out=h(R, H)),
        "scatter_rows out_scales": lambda: mxq.moe_scatter_rows(
            q, ids, R, scales=g(T, 2), out_scales=h(R, 2)),
        "upscale scales": lambda: mxq.upscale_fp8_to_bf16(
            q, h(T, 2, dtype=torch.float32)),
        "upscale out": lambda: mxq.upscale_fp8_to_bf16(
            q, g(T, 2, dtype=torch.float32),
            out=h(T, H, dtype=torch.bfloat16)),
        "copy16 dst": lambda: mxq.mxq_copy16(q, h(T, H)),
        "weight s_inv": lambda: mxq.requant_weight_block_ue8m0(
            g(128, 128), h(1, 1, dtype=torch.float32)),
        "weight q_out": lambda: mxq.requant_weight_block_ue8m0(
            g(128, 128), g(1, 1, dtype=torch.float32), q_out=h(128, 128)),
        "fused x": lambda: mxq.moe_layout_scatter_quant(
            ids, h(T, H, dtype=torch.bfloat16), 0, 4, "masked", capacity=2),
        "fused q": lambda: mxq.moe_layout_scatter_quant(
            ids, x, 0, 4, "masked", capacity=2, q=h(R, H)),
        "fused out": lambda: mxq.moe_layout_scatter_quant(
            ids, x, 0, 4, "masked", capacity=2,
            out={"src2dst": h(T, K, dtype=torch.int32)}),
    }


@pytest.mark.parametrize("case", sorted(host_argument_calls(h)))
def test_host_tensor_refused(case):
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        host_argument_calls(gpu)[case]()


def short_output_calls(g):
    x = g(T, H, dtype=torch.bfloat16)
    ids = g(T, K, dtype=torch.int32)
    w = g(T, K, dtype=torch.float32)
    q = g(T, H)
    lc = g(2, dtype=torch.int32)
    ps = g(4, dtype=torch.int32)
    return {
        "scatter q narrow": lambda: mxq.moe_scatter_quant(
            x, ids, R, q=g(R, H - 16)),
        "scatter scales short": lambda: mxq.moe_scatter_quant(
            x, ids, R, scales=g(R - 1, H // 128)),
        "scatter_ex q short": lambda: mxq.moe_scatter_quant_ex(
            x, ids, R, q=g(R - 1, H)),
        "scatter_ex mfma scales short": lambda: mxq.moe_scatter_quant_ex(
            x, ids, R, scale_layout="mfma16", scales=g(255)),
        "live_ex mfma scales short": lambda: mxq.mx_quant_live_rows_ex(
            x, 2, lc, scale_layout="mfma32", scales=g(1, 1, 63, 4)),
        "live q narrow": lambda: mxq.mx_quant_live_rows(
            x, 2, lc, q=g(T, H - 16)),
        "live scales narrow": lambda: mxq.mx_quant_live_rows(
            x, 2, lc, scales=g(T, H // 32 - 1)),
        "requant q_out short": lambda: mxq.requant_per_token_to_per_tensor(
            q, g(T, dtype=torch.float32), q_out=g(T - 1, H)),
        "combine out narrow": lambda: mxq.moe_combine(
            x, ids, w, out=g(T, H - 8, dtype=torch.bfloat16)),
        "m_indices out short": lambda: mxq.moe_m_indices_from_psum(
            ps, 16, out=g(15, dtype=torch.int32)),
        "expand slab short": lambda: mxq.moe_expand_to_masked_slab(
            q, ps, 16, slab=g(63, H)),
        "expand scales short": lambda: mxq.moe_expand_to_masked_slab(
            q, ps, 16, scales=g(T - 1, 2)),
        "expand slab_scales short": lambda: mxq.moe_expand_to_masked_slab(
            q, ps, 16, scales=g(T, 2), slab_scales=g(63, 2)),
        "slab short": lambda: mxq.moe_masked_slab_to_expand(
            g(63, H, dtype=torch.bfloat16), ps, ps, 16, out_rows=8),
        "slab masked_m short": lambda: mxq.moe_masked_slab_to_expand(
            g(64, H, dtype=torch.bfloat16), g(3, dtype=torch.int32), ps, 16,
            out_rows=8),
        "scatter_rows out short": lambda: mxq.moe_scatter_rows(
            q, ids, R, out=g(R - 1, H)),
        "upscale out short": lambda: mxq.upscale_fp8_to_bf16(
            q, g(T, 2, dtype=torch.float32),
            out=g(T - 1, H, dtype=torch.bfloat16)),
        "fused q short": lambda: mxq.moe_layout_scatter_quant(
            ids, x, 0, 4, "masked", capacity=2, q=g(R - 1, H)),
        "fused scales narrow": lambda: mxq.moe_layout_scatter_quant(
            ids, x, 0, 4, "masked", capacity=2, scales=g(R, H // 128 - 1)),
        "fused x rows": lambda: mxq.moe_layout_scatter_quant(
            ids, g(T - 1, H, dtype=torch.bfloat16), 0, 4, "masked",
            capacity=2),
    }


@pytest.mark.parametrize("case", sorted(short_output_calls(h)))
def test_short_output_refused(case):
    with pytest.raises(ValueError):
        short_output_calls(gpu)[case]()

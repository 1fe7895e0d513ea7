"""Seeded synthetic inputs for the MoE dispatch-preprocessing path.

Shared by the tests (both the oracle side and the GPU side) and the
benchmark.  It holds no step of the method itself: it only draws random
activations, routings and weights with the shapes and distributions of the
workloads below, using numpy's ``default_rng`` and torch's own dtype casts.

Workloads (shapes follow the pages' DeepSeek-class models: hidden 7168, a
3072 x 8 padded receive buffer, top-8 routing):

  tiny            T=64, H=256, 8 experts all local, top-2 uniform, block 128,
                  group 128                                         seed 101
  decode_masked   T=128, H=7168, 256 experts, local [0, 32), top-8 uniform,
                  slab capacity 128, group 128                      seed 202
  prefill_compact T=8192, H=7168, 256 experts all local, top-8 from a Zipf(1.1)
                  popularity with the 8 least popular experts at zero, 0.1% of
                  channels scaled x100, block 128, group 128       seed 303
  live_rows       24576 x 7168 padded rows = 8 segments of 3072, live counts
                  [14]*8, group 32 (e8m0)                           seed 404
  requant_combine T=16384, H=4096: fp8 rows (bytes drawn field by field,
                  one +-448 per row) with per-token scales 2^U,
                  U ~ U[-8, 4]; 128 experts top-8 uniform, block 128  seed 505
  fp8_dispatch    24576 x 7168 e4m3 rows (3072 x 8 padded receive buffer)
                  with group-128 fp32 scales, upscaled over the first
                  num_local_tokens rows                             seed 606
  block_weights   e4m3 expert weights [32, 4096, 7168] (gate/up) and
                  [32, 7168, 2048] (down), one fp32 inverse scale per
                  128 x 128 block                                   seed 707
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

SEEDS = {
    "fp8_dispatch": 606,
    "block_weights": 707,
    "tiny": 101,
    "decode_masked": 202,
    "prefill_compact": 303,
    "live_rows": 404,
    "requant_combine": 505,
}


# ------------------------------------------------------------- primitives

def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 array -> bf16 bit patterns (uint16), rounded by torch's cast."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def gaussian_bf16(rng: np.random.Generator, shape, outlier_channels=None,
                  outlier_gain: float = 100.0) -> np.ndarray:
    """N(0,1) activations as bf16 bits; optional channels scaled before the
    bf16 rounding."""
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if outlier_channels is not None and len(outlier_channels):
        a[..., outlier_channels] *= np.float32(outlier_gain)
    return to_bf16_bits(a)


def gaussian_bf16_device(seed: int, shape, device) -> torch.Tensor:
    """N(0,1) bf16 tensor drawn directly on a device (for buffers too large
    to draw on the host); deterministic for a given seed and device type."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=device,
                       dtype=torch.float32).to(torch.bfloat16)


def uniform_topk(rng: np.random.Generator, T: int, n_experts: int,
                 K: int) -> np.ndarray:
    """K distinct experts per token, every K-subset equally likely, in random
    order (int32 [T, K])."""
    if T == 0:
        return np.zeros((0, K), np.int32)
    keys = rng.random((T, n_experts))
    return np.argsort(keys, axis=1)[:, :K].astype(np.int32)


def zipf_topk(rng: np.random.Generator, T: int, n_experts: int, K: int,
              s: float = 1.1, n_zero: int = 8) -> np.ndarray:
    """Top-K without replacement from a Zipf(s) expert popularity over a random
    permutation of the experts, the n_zero least popular forced to zero
    (Gumbel-top-k sampling).  Returns int32 [T, K], highest score first."""
    ranks = np.arange(1, n_experts + 1, dtype=np.float64)
    p = ranks ** (-s)
    p[n_experts - n_zero:] = 0.0
    perm = rng.permutation(n_experts)
    pop = np.empty(n_experts)
    pop[perm] = p
    with np.errstate(divide="ignore"):
        logp = np.log(pop)
    g = rng.gumbel(size=(T, n_experts))
    score = logp[None, :] + g
    top = np.argsort(-score, axis=1, kind="stable")[:, :K]
    return top.astype(np.int32)


def strided_topk(rng: np.random.Generator, T: int, n_experts: int, K: int,
                 stride: int = 131) -> np.ndarray:
    """Top-K for very large T without a [T, n_experts] draw: a skewed base
    expert b_t = floor(n_experts * u^3) per token, then experts (b_t + j *
    stride) mod n_experts, distinct for j < K when stride * K stays below
    n_experts or stride is odd and n_experts a power of two."""
    b = np.floor(n_experts * rng.random(T) ** 3).astype(np.int64)
    ids = (b[:, None] + np.arange(K, dtype=np.int64) * stride) % n_experts
    return ids.astype(np.int32)


def softmax_weights(rng: np.random.Generator, T: int, K: int) -> np.ndarray:
    """Routing weights: softmax over K standard-normal logits per token."""
    z = rng.standard_normal((T, K))
    z = z - z.max(axis=1, keepdims=True) if T else z
    e = np.exp(z)
    return (e / e.sum(axis=1, keepdims=True)).astype(np.float32)


def per_token_fp8(rng: np.random.Generator, T: int, H: int,
                  log2_lo: float = -8.0, log2_hi: float = 4.0):
    """fp8 e4m3fn rows whose largest magnitude is 448, as a per-token absmax
    quantizer leaves them, with per-token fp32 scales 2^U,
    U ~ U[log2_lo, log2_hi].  The bytes are drawn field by field
    (random_e4m3_bytes), and one random position per row is set to +-448
    (byte 0x7E with a random sign); no finite e4m3 byte is larger."""
    q = random_e4m3_bytes(rng, (T, H))
    if H > 0 and T > 0:
        pos = rng.integers(0, H, T)
        sign = (rng.random(T) < 0.5).astype(np.uint8) << 7
        q[np.arange(T), pos] = np.uint8(0x7E) | sign
    u = rng.uniform(log2_lo, log2_hi, size=T)
    scales = np.exp2(u).astype(np.float32)
    return q, scales


# --------------------------------------------------------------- workloads

@dataclass
class RoutedBatch:
    name: str
    x: np.ndarray            # bf16 bits [T, H]
    topk_ids: np.ndarray     # int32 [T, K]
    topk_weights: np.ndarray  # float32 [T, K]
    n_experts: int           # global experts
    expert_begin: int        # first local expert
    n_local: int             # local experts
    layout: str              # "compact" | "masked"
    block_e: int = 128
    capacity: int = 0
    group: int = 128
    extra: dict = field(default_factory=dict)

    @property
    def T(self):
        return self.x.shape[0]

    @property
    def H(self):
        return self.x.shape[1]

    @property
    def K(self):
        return self.topk_ids.shape[1]


def tiny(seed: int = SEEDS["tiny"], T: int = 64, H: int = 256) -> RoutedBatch:
    rng = np.random.default_rng(seed)
    x = gaussian_bf16(rng, (T, H))
    ids = uniform_topk(rng, T, 8, 2)
    w = softmax_weights(rng, T, 2)
    return RoutedBatch("tiny", x, ids, w, 8, 0, 8, "compact", 128, 0, 128)


def decode_masked(seed: int = SEEDS["decode_masked"], T: int = 128,
                  H: int = 7168) -> RoutedBatch:
    rng = np.random.default_rng(seed)
    x = gaussian_bf16(rng, (T, H))
    ids = uniform_topk(rng, T, 256, 8)
    w = softmax_weights(rng, T, 8)
    return RoutedBatch("decode_masked", x, ids, w, 256, 0, 32, "masked", 128,
                       128, 128)


def prefill_compact(seed: int = SEEDS["prefill_compact"], T: int = 8192,
                    H: int = 7168, n_experts: int = 256) -> RoutedBatch:
    rng = np.random.default_rng(seed)
    n_out = max(1, round(0.001 * H))
    channels = rng.choice(H, n_out, replace=False)
    x = gaussian_bf16(rng, (T, H), outlier_channels=channels)
    ids = zipf_topk(rng, T, n_experts, 8)
    w = softmax_weights(rng, T, 8)
    return RoutedBatch("prefill_compact", x, ids, w, n_experts, 0, n_experts,
                       "compact", 128, 0, 128,
                       extra={"outlier_channels": channels})


@dataclass
class LiveRows:
    x: np.ndarray          # bf16 bits [segments * rows_per_segment, H]
    num_segments: int
    live_counts: np.ndarray  # int32 [segments]
    group: int = 32


def live_rows(seed: int = SEEDS["live_rows"], num_segments: int = 8,
              rows_per_segment: int = 3072, H: int = 7168,
              live_counts=None, full_rows: bool = True) -> LiveRows:
    """Padded send buffer.  With ``full_rows=False`` only the live rows are
    drawn and the other rows are zero (they are never read)."""
    rng = np.random.default_rng(seed)
    if live_counts is None:
        live_counts = [14] * num_segments
    live = np.asarray(live_counts, np.int32)
    rows = num_segments * rows_per_segment
    if full_rows:
        x = gaussian_bf16(rng, (rows, H))
    else:
        x = np.zeros((rows, H), np.uint16)
        for s in range(num_segments):
            n = int(min(live[s], rows_per_segment))
            r0 = s * rows_per_segment
            x[r0:r0 + n] = gaussian_bf16(rng, (n, H))
    return LiveRows(x, num_segments, live, 32)


@dataclass
class RequantBatch:
    q: np.ndarray        # uint8 e4m3fn [T, H]
    scales: np.ndarray   # float32 [T]


def requant_input(seed: int = SEEDS["requant_combine"], T: int = 16384,
                  H: int = 4096) -> RequantBatch:
    rng = np.random.default_rng(seed)
    q, s = per_token_fp8(rng, T, H)
    return RequantBatch(q, s)


def large_combine_routing(seed: int = SEEDS["requant_combine"] + 1,
                          T: int = 16384, n_experts: int = 128, K: int = 8):
    """Routing and weights for the large combine (all experts local)."""
    rng = np.random.default_rng(seed)
    ids = uniform_topk(rng, T, n_experts, K)
    w = softmax_weights(rng, T, K)
    return ids, w


def expert_outputs_bf16(seed: int, num_rows: int, H: int) -> np.ndarray:
    """Expert-output rows (bf16 bits) drawn on the host."""
    rng = np.random.default_rng(seed)
    return gaussian_bf16(rng, (num_rows, H))


def poison_padding_rows(y_bits: np.ndarray, m_indices: np.ndarray):
    """Set every padding row (m_indices == -1) to NaN (bf16 0x7FC0)."""
    y_bits[np.asarray(m_indices) < 0] = np.uint16(0x7FC0)
    return y_bits


def random_e4m3_bytes(rng: np.random.Generator, shape,
                      exp_mean: float = 11.0, exp_sd: float = 2.0):
    """Finite e4m3fn bytes drawn field by field: random sign, exponent field
    ~ round(N(exp_mean, exp_sd)) clipped to [0, 15], uniform mantissa; the
    NaN pattern (exponent 15, mantissa 7) is redrawn as mantissa 6.  A
    block of a few thousand bytes almost surely holds exponent 15 (values
    256..448), like a block quantized to the full e4m3 range."""
    ef = np.clip(np.rint(rng.normal(exp_mean, exp_sd, shape)), 0, 15).astype(
        np.uint8)
    m = rng.integers(0, 8, shape, dtype=np.uint8)
    m = np.where((ef == 15) & (m == 7), np.uint8(6), m)
    sign = (rng.random(shape) < 0.5).astype(np.uint8) << 7
    return (sign | (ef << 3) | m).astype(np.uint8)


def random_e4m3_bytes_device(seed: int, shape, device) -> torch.Tensor:
    """Finite e4m3fn bytes drawn uniformly on a device (torch generator):
    0..253 with 0x7F..0xFD moved up by one, so 0x7F and 0xFF never occur."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    v = torch.randint(0, 254, shape, dtype=torch.int16, device=device,
                      generator=g)
    return (v + (v >= 0x7F).to(torch.int16)).to(torch.uint8)


def group_scales_f32(rng: np.random.Generator, shape, lo: float = 2.0 ** -14,
                     hi: float = 2.0 ** -6) -> np.ndarray:
    """Positive fp32 scales, log-uniform in [lo, hi) (an amax / 448 range
    for bf16 activations or weights)."""
    return np.exp(rng.uniform(np.log(lo), np.log(hi), shape)).astype(
        np.float32)


@dataclass
class Fp8Dispatch:
    q: np.ndarray          # uint8 [rows, H]
    scales: np.ndarray     # float32 [rows, H / 128]
    num_local_tokens: int


def fp8_dispatch(seed: int = SEEDS["fp8_dispatch"], rows: int = 24576,
                 H: int = 7168, num_local_tokens: int = 8192) -> Fp8Dispatch:
    rng = np.random.default_rng(seed)
    return Fp8Dispatch(random_e4m3_bytes(rng, (rows, H)),
                       group_scales_f32(rng, (rows, H // 128)),
                       num_local_tokens)


def block_weights(seed: int, B: int, N: int, K: int, block: int = 128):
    """(q bytes [B, N, K], s_inv fp32 [B, ceil(N/128), ceil(K/128)])."""
    rng = np.random.default_rng(seed)
    q = random_e4m3_bytes(rng, (B, N, K))
    s = group_scales_f32(rng, (B, -(-N // block), -(-K // block)),
                         2.0 ** -16, 2.0 ** -8)
    return q, s

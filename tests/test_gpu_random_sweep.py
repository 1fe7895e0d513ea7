"""Seeded random configurations of the whole dispatch path on the GPU against
the oracle: moe_layout, moe_scatter_quant, moe_layout_scatter_quant (when the
routing has at most 4096 assignments), moe_combine and moe_scatter_rows.

Each case draws its token count (1 to 6000, so the per-token, the one-launch
and the two-launch layouts all occur), top-k, the global expert count, the
local window (possibly with no local expert at all), the layout kind and its
block_e / capacity (masked capacities may overflow), the group size, the
hidden size (a multiple of the group, sized so the case stays small), and the
routing: distinct experts per token, repeated experts, or some ids set to -1.
Every output is compared bit for bit; rows that are no destination keep their
canary."""
import numpy as np
import pytest
import torch

import fp8_mx_activation_amd as mxq
import synthetic_inputs as si
from gpu_util import (CANARY, DEV, assert_equal, bf16_to_dev, f32_to_dev,
                      host, i32_to_dev, say, u8_to_dev)

pytestmark = pytest.mark.gpu

N_CASES = 128
FUSED_MAX = 4096
FMT = {128: "ue8m0_g128", 32: "e8m0_g32"}
ROW_BYTES_BUDGET = 48 << 20     # destination rows x H, per case
TOKEN_BUDGET = 6 << 20          # T x H elements, per case


def make_case(i):
    rng = np.random.default_rng(9000 + i)
    size = rng.choice(["tiny", "decode", "mid", "large"],
                      p=[0.15, 0.35, 0.3, 0.2])
    lo, hi = {"tiny": (1, 9), "decode": (9, 257), "mid": (257, 2049),
              "large": (2049, 6001)}[size]
    T = int(rng.integers(lo, hi))
    K = int(rng.integers(1, 17))
    n_glob = int(rng.integers(max(K, 2), 1100))
    E = int(rng.integers(1, min(n_glob, 1024) + 1))
    begin = int(rng.integers(0, n_glob - E + 1))
    kind = "masked" if rng.random() < 0.35 else "compact"
    block_e = int(rng.choice([1, 8, 32, 128]))
    G = int(rng.choice([32, 128]))
    style = rng.choice(["distinct", "repeats", "dropped"], p=[0.6, 0.2, 0.2])
    if style == "repeats":
        ids = rng.integers(0, n_glob, (T, K)).astype(np.int32)
    else:
        ids = si.uniform_topk(rng, T, n_glob, K)
        if style == "dropped":
            ids[rng.random((T, K)) < 0.05] = -1
    if kind == "masked":
        fair = max(1, (T * K) // E)
        cap = int(rng.integers(1, 2 * fair + 2))
        R = E * cap
    else:
        cap = 0
        R = mxq.moe_compact_row_bound(T * K, E, block_e)
    n_max = max(1, min(64, TOKEN_BUDGET // (T * G),
                       ROW_BYTES_BUDGET // (max(R, 1) * G)))
    H = G * int(rng.integers(1, n_max + 1))
    x = si.gaussian_bf16(rng, (T, H))
    w = si.softmax_weights(rng, T, K)
    return dict(rng=rng, T=T, K=K, n_glob=n_glob, E=E, begin=begin,
                kind=kind, block_e=block_e, cap=cap, R=R, G=G, H=H,
                style=str(style), ids=ids, x=x, w=w)


def check_layout(lay, ref, what):
    for key in ("counts", "expert_offsets", "masked_m", "src2dst",
                "m_indices"):
        assert_equal(host(lay[key]), ref[key], "%s %s" % (what, key))
    assert mxq.moe_read_overflow(lay["overflow_flag"]) == ref["overflow"], \
        what + " overflow flag"


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(ora, i):
    c = make_case(i)
    T, K, E, H, G, R = c["T"], c["K"], c["E"], c["H"], c["G"], c["R"]
    kind, cap, block_e, begin = c["kind"], c["cap"], c["block_e"], c["begin"]
    rng = c["rng"]
    say("random sweep case %d:" % i, "T=%d K=%d experts [%d,%d) of %d %s "
        "block_e=%d cap=%d rows=%d H=%d G=%d ids=%s"
        % (T, K, begin, begin + E, c["n_glob"], kind, block_e, cap, R, H, G,
           c["style"]))
    ref = ora.moe_layout(c["ids"], begin, E, kind, block_e=block_e,
                         capacity=cap, num_rows=R)
    d = ref["src2dst"]
    idd, xd = i32_to_dev(c["ids"]), bf16_to_dev(c["x"])

    # layout, then scatter+quant
    lay = mxq.moe_layout(idd, begin, E, kind, block_e=block_e, capacity=cap,
                         num_rows=R)
    torch.cuda.synchronize()
    check_layout(lay, ref, "layout")
    q = torch.full((R, H), CANARY, dtype=torch.uint8, device=DEV)
    s = torch.full((R, H // G), CANARY, dtype=torch.uint8, device=DEV)
    mxq.moe_scatter_quant(xd, lay["src2dst"], R, FMT[G], q=q, scales=s)
    torch.cuda.synchronize()
    q_ref = np.full((R, H), CANARY, np.uint8)
    s_ref = np.full((R, H // G), CANARY, np.uint8)
    ora.scatter_quant(c["x"], d, G, R, q_ref, s_ref)
    assert_equal(host(q), q_ref, "scatter fp8 bytes")
    assert_equal(host(s), s_ref, "scatter scale bytes")

    # the same in one launch
    if T * K <= FUSED_MAX:
        q.fill_(CANARY)
        s.fill_(CANARY)
        lay2, _, _ = mxq.moe_layout_scatter_quant(
            idd, xd, begin, E, kind, block_e=block_e, capacity=cap,
            num_rows=R, fmt=FMT[G], q=q, scales=s)
        torch.cuda.synchronize()
        check_layout(lay2, ref, "fused")
        assert_equal(host(q), q_ref, "fused fp8 bytes")
        assert_equal(host(s), s_ref, "fused scale bytes")
    del q, s

    # combine of random expert outputs, bf16 or fp32 out
    y = si.gaussian_bf16(rng, (R, H))
    out_dtype = torch.float32 if rng.random() < 0.3 else torch.bfloat16
    out = mxq.moe_combine(bf16_to_dev(y), lay["src2dst"], f32_to_dev(c["w"]),
                          out_dtype=out_dtype)
    torch.cuda.synchronize()
    acc = ora.combine_f32(y, d, c["w"])
    if out_dtype == torch.float32:
        assert_equal(host(out).view(np.uint32), acc.view(np.uint32),
                     "combine fp32 bits")
    else:
        assert_equal(host(out.view(torch.int16)).view(np.uint16),
                     ora.bf16_round(acc), "combine bf16 bits")
    del out

    # already-quantized rows and their scale bytes
    xr = si.random_e4m3_bytes(rng, (T, H))
    xs = rng.integers(0, 256, (T, H // G)).astype(np.uint8)
    o = torch.full((R, H), CANARY, dtype=torch.uint8, device=DEV)
    os_ = torch.full((R, H // G), CANARY, dtype=torch.uint8, device=DEV)
    mxq.moe_scatter_rows(u8_to_dev(xr), lay["src2dst"], R,
                         scales=u8_to_dev(xs), out=o, out_scales=os_)
    torch.cuda.synchronize()
    o_ref, os_ref = ora.scatter_rows(
        xr, d, R, scales=xs, out=np.full((R, H), CANARY, np.uint8),
        out_scales=np.full((R, H // G), CANARY, np.uint8))
    assert_equal(host(o), o_ref, "scatter_rows bytes")
    assert_equal(host(os_), os_ref, "scatter_rows scale bytes")

"""Masked and compact layouts at a point of the layout sweep (48 local of 384
experts, T = 1024, masked capacity T): the same fp8 rows and scales reach
each assignment's destination in either layout, and the combine gives
bit-identical tokens from either; the compact side is checked against the
oracle."""
import numpy as np
import pytest
import torch

import fp8_mx_activation_amd as mxq
import synthetic_inputs as si
from gpu_util import (DEV, assert_equal, bf16_to_dev, bf16_to_host, f32_to_dev,
                      host, i32_to_dev, say)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("e_loc,e_glob,T", [(48, 384, 1024), (128, 128, 256)])
def test_masked_and_compact_agree(ora, e_loc, e_glob, T):
    H, K = 7168, 8
    rng = np.random.default_rng(e_loc + T)
    ids = si.uniform_topk(rng, T, e_glob, K)
    w = si.softmax_weights(rng, T, K)
    x = si.gaussian_bf16(rng, (T, H))
    xd, idd = bf16_to_dev(x), i32_to_dev(ids)
    res = {}
    for kind, cap in (("compact", 0), ("masked", T)):
        rows = (mxq.moe_compact_row_bound(T * K, e_loc, 128)
                if kind == "compact" else e_loc * cap)
        say("crossover", kind, "E=%d/%d T=%d rows=%d" % (e_loc, e_glob, T,
                                                        rows))
        lay = mxq.moe_layout(idd, 0, e_loc, kind, capacity=cap,
                             num_rows=rows)
        q, s = mxq.moe_scatter_quant(x=xd, src2dst=lay["src2dst"],
                                     num_rows=rows)
        torch.cuda.synchronize()
        res[kind] = (host(lay["src2dst"]), lay, q, s, rows)
        ref = ora.moe_layout(ids, 0, e_loc, kind, capacity=cap)
        assert_equal(res[kind][0], ref["src2dst"], "%s src2dst" % kind)
        assert mxq.moe_read_overflow(lay["overflow_flag"]) == 0

    d_c, _, q_c, s_c, _ = res["compact"]
    d_m, _, q_m, s_m, _ = res["masked"]
    assert np.array_equal(d_c >= 0, d_m >= 0)
    sel = d_c >= 0
    qc, qm = host(q_c), host(q_m)
    assert_equal(qm[d_m[sel]], qc[d_c[sel]], "fp8 rows by assignment")
    assert_equal(host(s_m)[d_m[sel]], host(s_c)[d_c[sel]],
                 "scales by assignment")
    q_ref, s_ref = ora.scatter_quant(x, d_c, 128, res["compact"][4])
    assert_equal(qc[d_c[sel]], q_ref[d_c[sel]], "compact fp8 vs oracle")
    assert_equal(host(s_c)[d_c[sel]], s_ref[d_c[sel]], "compact scales")

    # per-assignment expert outputs placed into each layout
    ya = si.gaussian_bf16(rng, (T, K, H))
    outs = []
    for d, rows in ((d_c, res["compact"][4]), (d_m, res["masked"][4])):
        y = np.full((rows, H), 0x7FC0, np.uint16)
        y[d[sel]] = ya[sel]
        o = mxq.moe_combine(bf16_to_dev(y), i32_to_dev(d), f32_to_dev(w))
        torch.cuda.synchronize()
        outs.append(bf16_to_host(o))
        del y
    assert_equal(outs[0], outs[1], "masked vs compact combine")
    acc = ora.combine_f32(
        np.ascontiguousarray(ya.reshape(T * K, H)),
        np.where(sel, np.arange(T * K).reshape(T, K), -1).astype(np.int32),
        w)
    assert_equal(outs[0], ora.bf16_round(acc), "combine vs oracle")

"""The whole path (layout -> scatter+quant -> combine, plus the send-side
and requant calls) captured once in a hipGraph and replayed with new inputs
copied into the static buffers between replays; every replay is checked
against the oracle."""
import numpy as np
import pytest
import torch

import fp8_mx_activation_amd as mxq
import synthetic_inputs as si
from gpu_util import (DEV, assert_equal, bf16_to_dev, bf16_to_host, host,
                      i32_to_dev, say, f32_to_dev, u8_to_dev)

pytestmark = pytest.mark.gpu


def test_graph_replay_full_path(ora):
    T, H, E, K = 96, 512, 16, 4
    R = ora.compact_row_bound(T * K, E, 128)
    ids_s = torch.zeros((T, K), dtype=torch.int32, device=DEV)
    x_s = torch.zeros((T, H), dtype=torch.bfloat16, device=DEV)
    w_s = torch.zeros((T, K), dtype=torch.float32, device=DEV)
    y_s = torch.zeros((R, H), dtype=torch.bfloat16, device=DEV)
    lay_out = {k: torch.empty(shape, dtype=torch.int32, device=DEV)
               for k, shape in (("counts", (E,)), ("expert_offsets", (E + 1,)),
                                ("m_indices", (R,)), ("masked_m", (E,)),
                                ("src2dst", (T, K)), ("overflow_flag", (1,)))}
    ws = torch.empty(max(1, mxq.moe_layout_workspace_bytes(T, K, E)),
                     dtype=torch.uint8, device=DEV)
    q_s = torch.empty((R, H), dtype=torch.uint8, device=DEV)
    sc_s = torch.empty((R, H // 128), dtype=torch.uint8, device=DEV)
    out_s = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    live_s = torch.zeros(2, dtype=torch.int32, device=DEV)
    qmx_s = torch.empty((T, H), dtype=torch.uint8, device=DEV)
    smx_s = torch.empty((T, H // 32), dtype=torch.uint8, device=DEV)
    rq_in = torch.zeros((T, H), dtype=torch.uint8, device=DEV)
    rs_in = torch.ones(T, dtype=torch.float32, device=DEV)
    rq_out = torch.empty((T, H), dtype=torch.uint8, device=DEV)
    S_s = torch.empty(1, dtype=torch.float32, device=DEV)
    rws = torch.empty(mxq.requant_workspace_bytes(T, H), dtype=torch.uint8,
                      device=DEV)
    # psum repack: a 4-expert expanded layout of R rows
    psum_s = torch.zeros(4, dtype=torch.int32, device=DEV)
    slab_s = torch.empty((4 * 64, H), dtype=torch.bfloat16, device=DEV)
    mm_s = torch.empty(4, dtype=torch.int32, device=DEV)
    fl_s = torch.empty(1, dtype=torch.int32, device=DEV)
    pm_s = torch.empty(R, dtype=torch.int32, device=DEV)
    back_s = torch.empty((R, H), dtype=torch.bfloat16, device=DEV)

    def step():
        lay = mxq.moe_layout(ids_s, 0, E, "compact", num_rows=R, out=lay_out,
                             workspace=ws)
        mxq.moe_scatter_quant(x_s, lay["src2dst"], R, q=q_s, scales=sc_s)
        mxq.moe_combine(y_s, lay["src2dst"], w_s, out=out_s)
        mxq.mx_quant_live_rows(x_s, 2, live_s, q=qmx_s, scales=smx_s)
        mxq.requant_per_token_to_per_tensor(rq_in, rs_in, q_out=rq_out,
                                            tensor_scale=S_s, workspace=rws)
        lib = mxq.lib()
        st = torch.cuda.current_stream().cuda_stream
        assert lib.moe_expand_to_masked_slab(
            y_s.data_ptr(), H * 2, R, H * 2, None, 0, 0, 0, 0,
            psum_s.data_ptr(), 4, 16, 64, slab_s.data_ptr(), H * 2, None, 0,
            0, mm_s.data_ptr(), fl_s.data_ptr(), st) == 0
        mxq.moe_masked_slab_to_expand(slab_s, mm_s, psum_s, 64, 16,
                                      out=back_s)
        mxq.moe_m_indices_from_psum(psum_s, R, 16, out=pm_s)

    say("graph: warm-up on a side stream")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    say("graph: capture")
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for rep in range(4):
        rng = np.random.default_rng(1000 + rep)
        ids = si.uniform_topk(rng, T, 24, K)      # experts 16..23 non-local
        x = si.gaussian_bf16(rng, (T, H))
        w = si.softmax_weights(rng, T, K)
        y = si.gaussian_bf16(rng, (R, H))
        live = np.array([rep * 11 % 48, 48 - rep * 7], np.int32)
        rq, rs = si.per_token_fp8(rng, T, H)
        counts = [int(c) for c in rng.integers(0, 65, 4)]
        from test_oracle_psum import build_layout
        _, psum_h, _, _ = build_layout(counts, 16, 1)
        ids_s.copy_(i32_to_dev(ids))
        x_s.copy_(bf16_to_dev(x))
        w_s.copy_(f32_to_dev(w))
        y_s.copy_(bf16_to_dev(y))
        live_s.copy_(i32_to_dev(live))
        rq_in.copy_(u8_to_dev(rq))
        rs_in.copy_(f32_to_dev(rs))
        psum_s.copy_(torch.from_numpy(psum_h).to(DEV))
        back_s.view(torch.int16).fill_(0x1234)
        q_s.fill_(0xA5)
        sc_s.fill_(0xA5)
        qmx_s.fill_(0xA5)
        smx_s.fill_(0xA5)
        torch.cuda.synchronize()
        say("graph: replay", rep)
        g.replay()
        torch.cuda.synchronize()

        ref = ora.moe_layout(ids, 0, E, "compact", num_rows=R)
        assert_equal(host(lay_out["src2dst"]), ref["src2dst"], "src2dst")
        assert_equal(host(lay_out["m_indices"]), ref["m_indices"], "m_idx")
        q_ref = np.full((R, H), 0xA5, np.uint8)
        s_ref = np.full((R, H // 128), 0xA5, np.uint8)
        ora.scatter_quant(x, ref["src2dst"], 128, R, q_ref, s_ref)
        assert_equal(host(q_s), q_ref, "fp8 bytes")
        assert_equal(host(sc_s), s_ref, "scales")
        out_ref = ora.combine(y, ref["src2dst"], w)
        assert_equal(bf16_to_host(out_s), out_ref, "combine")
        qm_ref = np.full((T, H), 0xA5, np.uint8)
        sm_ref = np.full((T, H // 32), 0xA5, np.uint8)
        ora.mx_quant_live_rows(x, 2, live, 32, qm_ref, sm_ref)
        assert_equal(host(qmx_s), qm_ref, "live fp8")
        assert_equal(host(smx_s), sm_ref, "live scales")
        rq_ref, S_ref = ora.requant_per_token_to_per_tensor(rq, rs)
        assert_equal(host(rq_out), rq_ref, "requant")
        assert np.float32(host(S_s)[0]) == np.float32(S_ref)
        y8 = y.view(np.uint8).reshape(R, H * 2)
        ref_slab = np.zeros((4 * 64, H * 2), np.uint8)
        _, _, mm_ref, fl_ref = ora.expand_to_masked_slab(y8, psum_h, 16, 64,
                                                         slab=ref_slab)
        assert_equal(host(mm_s), mm_ref, "psum masked_m")
        assert int(host(fl_s)[0]) == fl_ref
        back_ref = ora.masked_slab_to_expand(
            ref_slab.view(np.uint16), mm_ref, psum_h, 16, 64,
            out=np.full((R, H), 0x1234, np.uint16))
        assert_equal(bf16_to_host(back_s), back_ref, "psum round trip")
        assert_equal(host(pm_s), ora.m_indices_from_psum(psum_h, 16, R),
                     "psum m_indices")
        # eager work between replays
        _ = (x_s.float() * 2).sum().item()

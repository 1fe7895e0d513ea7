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


def test_graph_replay_variants_upscale_weights(ora):
    """The scale variants, the upscale, the weight requant and the layout in
    both of its launch forms above 4096 assignments (8800 over 40 experts:
    one launch that counts the routing in every block; the same ids over
    300 experts: histogram launch + slot launch with the per-chunk
    workspace) captured once and replayed three times with new inputs and
    eager work between replays; every replay is checked."""
    T, H, E, K, G = 1100, 256, 40, 8, 32
    R = ora.compact_row_bound(T * K, E, 128)
    E2 = 300
    R2 = ora.compact_row_bound(T * K, E2, 128)
    lay_out2 = {k: torch.empty(shape, dtype=torch.int32, device=DEV)
                for k, shape in (("counts", (E2,)),
                                 ("expert_offsets", (E2 + 1,)),
                                 ("m_indices", (R2,)), ("masked_m", (E2,)),
                                 ("src2dst", (T, K)),
                                 ("overflow_flag", (1,)))}
    assert mxq.moe_layout_workspace_bytes(T, K, E) == 0
    assert mxq.moe_layout_workspace_bytes(T, K, E2) > 0
    ws2 = torch.empty(mxq.moe_layout_workspace_bytes(T, K, E2),
                      dtype=torch.uint8, device=DEV)
    ng = H // G
    ids_s = torch.zeros((T, K), dtype=torch.int32, device=DEV)
    x_s = torch.zeros((T, H), dtype=torch.bfloat16, device=DEV)
    lay_out = {k: torch.empty(shape, dtype=torch.int32, device=DEV)
               for k, shape in (("counts", (E,)), ("expert_offsets", (E + 1,)),
                                ("m_indices", (R,)), ("masked_m", (E,)),
                                ("src2dst", (T, K)), ("overflow_flag", (1,)))}
    ws = torch.empty(max(1, mxq.moe_layout_workspace_bytes(T, K, E)),
                     dtype=torch.uint8, device=DEV)
    q_s = torch.empty((R, H), dtype=torch.uint8, device=DEV)
    pk_s = mxq.packed_mn_scales(R, ng, DEV)
    live_s = torch.zeros(4, dtype=torch.int32, device=DEV)
    ql_s = torch.empty((T, H), dtype=torch.uint8, device=DEV)
    sl_s = torch.empty((T, ng), dtype=torch.uint8, device=DEV)
    uq_s = torch.zeros((T, H), dtype=torch.uint8, device=DEV)
    us_s = torch.ones((T, H // 128), dtype=torch.float32, device=DEV)
    uo_s = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    wq_s = torch.zeros((2, 256, 384), dtype=torch.uint8, device=DEV)
    wsi_s = torch.ones((2, 2, 3), dtype=torch.float32, device=DEV)
    wo_s = torch.empty_like(wq_s)
    wso_s = torch.empty((2, 2, 3), dtype=torch.uint8, device=DEV)

    def step():
        lay = mxq.moe_layout(ids_s, 0, E, "compact", num_rows=R, out=lay_out,
                             workspace=ws)
        mxq.moe_layout(ids_s, 0, E2, "compact", num_rows=R2, out=lay_out2,
                       workspace=ws2)
        mxq.moe_scatter_quant_ex(x_s, lay["src2dst"], R, "e8m0_g32",
                                 "ocp_floor", "packed_mn", q=q_s,
                                 scales=pk_s)
        mxq.mx_quant_live_rows_ex(x_s[:1100 // 4 * 4], 4, live_s,
                                  "e8m0_g32", "ocp_floor", "rows",
                                  q=ql_s[:1100 // 4 * 4],
                                  scales=sl_s[:1100 // 4 * 4])
        mxq.upscale_fp8_to_bf16(uq_s, us_s, T - 7, out=uo_s)
        mxq.requant_weight_block_ue8m0(wq_s, wsi_s, q_out=wo_s,
                                       scales_out=wso_s)

    say("graph variants: warm-up on a side stream")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    say("graph variants: capture")
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for rep in range(3):
        rng = np.random.default_rng(2000 + rep)
        ids = si.zipf_topk(rng, T, E, K, n_zero=3)
        x = si.gaussian_bf16(rng, (T, H))
        live = np.array([rep * 37 % 275, 275, 0, 100 + rep], np.int32)
        uq = si.random_e4m3_bytes(rng, (T, H))
        usc = si.group_scales_f32(rng, (T, H // 128))
        wq, wsi = si.block_weights(3000 + rep, 2, 256, 384)
        ids_s.copy_(i32_to_dev(ids))
        x_s.copy_(bf16_to_dev(x))
        live_s.copy_(i32_to_dev(live))
        uq_s.copy_(u8_to_dev(uq))
        us_s.copy_(f32_to_dev(usc))
        wq_s.copy_(u8_to_dev(wq))
        wsi_s.copy_(f32_to_dev(wsi))
        q_s.fill_(0xA5)
        pk_s.fill_(-1)
        ql_s.fill_(0xA5)
        sl_s.fill_(0xA5)
        uo_s.view(torch.int16).fill_(0x1234)
        torch.cuda.synchronize()
        say("graph variants: replay", rep)
        g.replay()
        torch.cuda.synchronize()

        ref = ora.moe_layout(ids, 0, E, "compact", num_rows=R)
        assert_equal(host(lay_out["src2dst"]), ref["src2dst"], "src2dst")
        assert_equal(host(lay_out["m_indices"]), ref["m_indices"],
                     "m_indices")
        ref2 = ora.moe_layout(ids, 0, E2, "compact", num_rows=R2)
        assert_equal(host(lay_out2["src2dst"]), ref2["src2dst"],
                     "src2dst (two launches)")
        assert_equal(host(lay_out2["m_indices"]), ref2["m_indices"],
                     "m_indices (two launches)")
        q_ref, pk_ref = ora.scatter_quant_ex(
            x, ref["src2dst"], G, R, "ocp_floor", "packed_mn",
            q=np.full((R, H), 0xA5, np.uint8),
            s=np.full(pk_s.shape, 0xFFFFFFFF, np.uint32))
        assert_equal(host(q_s), q_ref, "scatter_ex fp8")
        assert_equal(host(pk_s).view(np.uint32), pk_ref, "packed scales")
        n4 = 1100 // 4 * 4
        d = np.full((n4, 1), -1, np.int32)
        rps = n4 // 4
        for gi in range(4):
            nl = min(int(live[gi]), rps)
            d[gi * rps:gi * rps + nl, 0] = np.arange(gi * rps, gi * rps + nl)
        ql_ref, sl_ref = ora.scatter_quant_ex(
            x[:n4], d, G, n4, "ocp_floor", "rows",
            q=np.full((n4, H), 0xA5, np.uint8),
            s=np.full((n4, ng), 0xA5, np.uint8))
        assert_equal(host(ql_s)[:n4], ql_ref, "live_ex fp8")
        assert_equal(host(sl_s)[:n4], sl_ref, "live_ex scales")
        uo_ref = ora.upscale_fp8(uq, usc, num_rows=T - 7,
                                 out=np.full((T, H), 0x1234, np.uint16))
        assert_equal(bf16_to_host(uo_s), uo_ref, "upscale")
        wo_ref, wso_ref = ora.requant_weight_block_ue8m0(wq, wsi)
        assert_equal(host(wo_s), wo_ref, "weights")
        assert_equal(host(wso_s), wso_ref, "weight scales")
        # eager work between replays
        _ = (x_s.float() * 2).sum().item()


def test_graph_replay_psum_repack_and_placements(ora):
    """The psum repack (m_indices from psum, expanded rows -> masked slab
    with 4-byte scales, slab -> expanded rows with weights), the scatter of
    quantized rows and the scatter with MFMA-placed scales, captured once
    and replayed three times with new routings and psum counts (some over
    the slab capacity); every replay is checked."""
    from test_oracle_psum import build_layout
    T, H, E, K, G = 300, 256, 12, 3, 32
    R = ora.compact_row_bound(T * K, E, 128)
    PE, align, max_m = 6, 128, 64
    rows_cap = PE * align           # counts stay below align
    ng = H // G
    C = 0xA5
    ids_s = torch.zeros((T, K), dtype=torch.int32, device=DEV)
    x_s = torch.zeros((T, H), dtype=torch.bfloat16, device=DEV)
    lay_out = {k: torch.empty(shape, dtype=torch.int32, device=DEV)
               for k, shape in (("counts", (E,)), ("expert_offsets", (E + 1,)),
                                ("m_indices", (R,)), ("masked_m", (E,)),
                                ("src2dst", (T, K)), ("overflow_flag", (1,)))}
    ws = torch.empty(max(1, mxq.moe_layout_workspace_bytes(T, K, E)),
                     dtype=torch.uint8, device=DEV)
    q_s = torch.empty((R, H), dtype=torch.uint8, device=DEV)
    sm_s = mxq.mfma_scales(R, H, 16, DEV)
    qt_s = torch.zeros((T, H), dtype=torch.uint8, device=DEV)
    st_s = torch.zeros((T, ng), dtype=torch.uint8, device=DEV)
    qr_s = torch.empty((R, H), dtype=torch.uint8, device=DEV)
    sr_s = torch.empty((R, ng), dtype=torch.uint8, device=DEV)
    psum_s = torch.zeros(PE, dtype=torch.int32, device=DEV)
    mi_s = torch.empty(rows_cap, dtype=torch.int32, device=DEV)
    xe_s = torch.zeros((rows_cap, H), dtype=torch.bfloat16, device=DEV)
    xsc_s = torch.zeros((rows_cap, 2), dtype=torch.float32, device=DEV)
    slab_s = torch.empty((PE * max_m, H), dtype=torch.bfloat16, device=DEV)
    slabsc_s = torch.empty((PE * max_m, 2), dtype=torch.float32, device=DEV)
    w_s = torch.zeros(rows_cap, dtype=torch.float32, device=DEV)
    eo_s = torch.empty((rows_cap, H), dtype=torch.bfloat16, device=DEV)

    def step():
        lay = mxq.moe_layout(ids_s, 0, E, "compact", num_rows=R, out=lay_out,
                             workspace=ws)
        mxq.moe_scatter_quant_ex(x_s, lay["src2dst"], R, "e8m0_g32",
                                 "no_clip", "mfma16", q=q_s, scales=sm_s)
        mxq.moe_scatter_rows(qt_s, lay["src2dst"], R, scales=st_s, out=qr_s,
                             out_scales=sr_s)
        mxq.moe_m_indices_from_psum(psum_s, rows_cap, align, out=mi_s)
        res = mxq.moe_expand_to_masked_slab(xe_s, psum_s, max_m, align,
                                            scales=xsc_s, slab=slab_s,
                                            slab_scales=slabsc_s)
        mxq.moe_masked_slab_to_expand(slab_s, res[2], psum_s, max_m, align,
                                      weights=w_s, out=eo_s)
        return res

    say("graph psum: warm-up on a side stream")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    say("graph psum: capture")
    with torch.cuda.graph(g):
        _, _, mm_s, flags_s = step()
    torch.cuda.synchronize()

    for rep in range(3):
        rng = np.random.default_rng(4000 + rep)
        ids = si.uniform_topk(rng, T, E + 4, K)      # some ids non-local
        x = si.gaussian_bf16(rng, (T, H))
        qt = si.random_e4m3_bytes(rng, (T, H))
        st = rng.integers(0, 255, (T, ng)).astype(np.uint8)
        counts = rng.integers(0, 100, PE)
        counts[rep] = 0
        _, psum, _, _ = build_layout(counts.tolist(), align, 1)
        xe = si.gaussian_bf16(rng, (rows_cap, H))
        xsc = rng.standard_normal((rows_cap, 2)).astype(np.float32)
        w = rng.random(rows_cap).astype(np.float32)
        ids_s.copy_(i32_to_dev(ids))
        x_s.copy_(bf16_to_dev(x))
        qt_s.copy_(u8_to_dev(qt))
        st_s.copy_(u8_to_dev(st))
        psum_s.copy_(i32_to_dev(psum))
        xe_s.copy_(bf16_to_dev(xe))
        xsc_s.copy_(f32_to_dev(xsc))
        w_s.copy_(f32_to_dev(w))
        for t in (q_s, sm_s, qr_s, sr_s, slab_s.view(torch.uint8),
                  slabsc_s.view(torch.uint8), eo_s.view(torch.uint8)):
            t.fill_(C)
        mi_s.fill_(-7)
        torch.cuda.synchronize()
        say("graph psum: replay", rep, "counts", counts.tolist())
        g.replay()
        torch.cuda.synchronize()

        ref = ora.moe_layout(ids, 0, E, "compact", num_rows=R)
        s2d = ref["src2dst"]
        assert_equal(host(lay_out["src2dst"]), s2d, "src2dst")
        q_ref, s_rows = ora.scatter_quant_ex(
            x, s2d, G, R, "ceil", "rows", q=np.full((R, H), C, np.uint8),
            s=np.full((R, ng), C, np.uint8))
        assert_equal(host(q_s), q_ref, "scatter fp8")
        assert_equal(host(sm_s), ora.mfma_scales(s_rows, H, G, 16, fill=C),
                     "MFMA-placed scales")
        qr_ref, sr_ref = ora.scatter_rows(
            qt, s2d, R, scales=st, out=np.full((R, H), C, np.uint8),
            out_scales=np.full((R, ng), C, np.uint8))
        assert_equal(host(qr_s), qr_ref, "scatter_rows")
        assert_equal(host(sr_s), sr_ref, "scatter_rows scales")
        assert_equal(host(mi_s), ora.m_indices_from_psum(psum, align,
                                                         rows_cap),
                     "m_indices")
        slab_ref, slabsc_ref, mm_ref, fl_ref = ora.expand_to_masked_slab(
            xe.view(np.uint8), psum, align, max_m, scales=xsc,
            slab=np.full((PE * max_m, 2 * H), C, np.uint8),
            slab_scales=np.full((PE * max_m, 2), C, np.uint8).view(
                np.uint8).repeat(4, axis=1).view(np.float32))
        assert_equal(host(slab_s.view(torch.uint8)), slab_ref, "slab")
        assert_equal(host(slabsc_s).view(np.uint32),
                     slabsc_ref.view(np.uint32), "slab scales")
        assert_equal(host(mm_s), mm_ref, "masked_m")
        assert int(host(flags_s)[0]) == fl_ref
        eo_ref = ora.masked_slab_to_expand(
            slab_ref.view(np.uint16), mm_ref, psum, align, max_m, weights=w,
            out=np.full((rows_cap, H), C * 257, np.uint16))
        assert_equal(bf16_to_host(eo_s), eo_ref, "slab to expanded")
        # eager work between replays
        _ = (x_s.float() * 2).sum().item()

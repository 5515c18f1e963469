"""A decode step captured as a HIP graph: every replay, with eager work and synchronisation in
between, returns exactly the eager call's bits (the calls are deterministic and allocate
nothing, so the captured launches are the eager ones)."""
import numpy as np
import pytest

import synth
from _pools import bf16_queries, oracle_pool, to_device

pytestmark = pytest.mark.gpu


def test_decode_append_step_graph_replays_match_eager():
    import torch
    import compressed_kv_attention_kvexec_amd as tq4
    layers = []
    for layer, lens in enumerate([(1000, 3000), (2500, 77)]):
        w = synth.Workload(110, "graph", "decode", 2, 64, 120, seq_lens=lens)
        pool, table = oracle_pool(w, layer=layer)
        q_t, _ = bf16_queries(w, layer, w.batch)
        rng = np.random.default_rng(110 + layer)
        new = torch.from_numpy(rng.standard_normal((2, w.batch, w.n_kv, 256)).astype(np.float32)).cuda()
        last = [int(table[b, (L - 1) // 64]) * 64 + (L - 1) % 64 for b, L in enumerate(lens)]
        layers.append(dict(pool=to_device(pool), q=q_t.cuda(), table=torch.from_numpy(table).cuda(),
                           seq=torch.tensor(lens, dtype=torch.int32).cuda(), max_len=max(lens),
                           k_new=new[0].contiguous(), v_new=new[1].contiguous(),
                           slots=torch.tensor(last, dtype=torch.int32).cuda()))
    ws = tq4.new_workspace(tq4.tq4_attn_decode_workspace_size(2, 3000, 24, 4, 64))
    ref = [tq4.tq4_attn_decode_append(L["pool"], L["k_new"], L["v_new"], L["slots"], L["q"], L["table"], L["seq"],
                                      L["max_len"], synth.SCALE, workspace=ws) for L in layers]
    torch.cuda.synchronize()

    s = torch.cuda.Stream()
    outs = [torch.empty_like(L["q"]) for L in layers]
    ws_g = tq4.new_workspace(tq4.tq4_attn_decode_workspace_size(2, 3000, 24, 4, 64))
    calls = [tq4.prepare_decode_append(L["pool"], L["k_new"], L["v_new"], L["slots"], L["q"], L["table"], L["seq"],
                                       L["max_len"], synth.SCALE, outs[i], ws_g, s) for i, L in enumerate(layers)]
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for c in calls:
            c()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for c in calls:
            c()
    x = torch.randn(512, 512, device="cuda")
    for rep in range(4):
        for o in outs:
            o.fill_(0)
        y = x @ x  # eager work on the default stream between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, o in enumerate(outs):
            assert torch.equal(o, ref[i]), f"replay {rep} layer {i}"
        assert torch.isfinite(y).all()


def test_other_entry_points_graph_replays_match_eager():
    """Verify, prefill, the unfused pair, the decode variants, decode without a workspace and the INT8
    encode, decode and decode-with-append captured in one graph: every replay equals the eager
    results bit for bit."""
    import torch
    import compressed_kv_attention_kvexec_amd as tq4
    from _pools import int8_to_device, oracle_int8_pool
    w = synth.Workload(111, "graph2", "decode", 1, 64, 120, seq_lens=(2000, 700))
    pool, table = oracle_pool(w)
    dpool = to_device(pool)
    pool8, _ = oracle_int8_pool(w, table=table)
    dpool8 = int8_to_device(pool8)
    tab = torch.from_numpy(table).cuda()
    seq = torch.tensor(w.seq_lens, dtype=torch.int32).cuda()
    qv, _ = bf16_queries(w, 0, w.batch * 4)
    qv = qv.reshape(w.batch, 4, w.n_q, 256).contiguous().cuda()
    qd, _ = bf16_queries(w, 1, w.batch)
    qd = qd.cuda()
    pf = synth.Workload(112, "graph_pf", "prefill", 1, 64, 20, prior_len=900, chunk_len=50)
    ppool, ptable = oracle_pool(pf)
    dppool = to_device(ppool)
    ptab = torch.from_numpy(ptable[0]).cuda()
    qp, _ = bf16_queries(pf, 0, 50)
    qp = qp.cuda()
    rng = np.random.default_rng(112)
    knew = torch.from_numpy(rng.standard_normal((3, w.n_kv, 256)).astype(np.float32)).cuda()
    new_slots = torch.tensor([int(table[1, 12]) * 64 + 5, int(table[1, 12]) * 64 + 6, int(table[1, 12]) * 64 + 7],
                             dtype=torch.int32).cuda()
    kv_app = torch.from_numpy(rng.standard_normal((2, 2, w.n_kv, 256)).astype(np.float32)).to(torch.bfloat16).cuda()
    app_slots = torch.tensor([int(table[b, (L - 1) // 64]) * 64 + (L - 1) % 64 for b, L in enumerate(w.seq_lens)],
                             dtype=torch.int32).cuda()

    s = torch.cuda.Stream()
    ws_v = tq4.new_workspace(tq4.tq4_attn_verify_workspace_size(2, 2000, 4, 24, 4, 64))
    ws_d = tq4.new_workspace(tq4.tq4_int8_attn_decode_workspace_size(2, 2000, 24, 4, 64))
    ws_p = tq4.new_workspace(tq4.tq4_attn_prefill_workspace_size(900, 50, 24, 4, 64))
    ws_s = tq4.new_workspace(tq4.tq4_sdpa_decode_workspace_size(2, 2000, 24, 4))
    out_v = torch.empty_like(qv)
    out_d = torch.empty_like(qd)
    out_p = torch.empty_like(qp)
    out_s = torch.empty_like(qd)
    out_a = torch.empty_like(qd)
    ws_a = tq4.new_workspace(tq4.tq4_int8_attn_decode_workspace_size(2, 2000, 24, 4, 64))
    ws_r = tq4.new_workspace(tq4.tq4_attn_decode_workspace_size(2, 2000, 24, 4, 64))
    ws_l = tq4.new_workspace(tq4.tq4_attn_decode_workspace_size(2, 2000, 24, 4, 64))
    out_r = torch.empty_like(qd)
    out_l = torch.empty_like(qd)
    out_n = torch.empty_like(qd)
    k_dense = torch.zeros((2, w.n_kv, 2000, 256), dtype=torch.bfloat16, device="cuda")
    v_dense = torch.zeros_like(k_dense)
    calls = [
        tq4.prepare_verify(dpool, qv, tab, seq, 2000, synth.SCALE, out_v, ws_v, s),
        tq4.prepare_prefill(dppool, qp, ptab, 900, synth.SCALE, out_p, ws_p, s),
        tq4.prepare_reconstruct(dpool, tab, seq, 2000, k_dense, v_dense, s),
        tq4.prepare_sdpa_decode(qd, k_dense, v_dense, seq, synth.SCALE, out_s, ws_s, s),
        tq4.prepare_decode_variant(dpool, qd, tab, seq, 2000, synth.SCALE, "valu_rotated", out_r, ws_r, s),
        tq4.prepare_decode_variant(dpool, qd, tab, seq, 2000, synth.SCALE, "valu_literal", out_l, ws_l, s),
        lambda: tq4.tq4_attn_decode_noalloc(dpool, qd, tab, seq, 2000, synth.SCALE, out_n, stream=s),
    ]

    def int8_calls():
        tq4.tq4_int8_encode_pages(dpool8, knew, knew, new_slots, stream=s)
        # the append first: it rewrites the last records the same way on every replay
        tq4.tq4_int8_attn_decode_append(dpool8, kv_app[0], kv_app[1], app_slots, qd, tab, seq, 2000, synth.SCALE,
                                        out=out_a, workspace=ws_a, stream=s)
        tq4.tq4_int8_attn_decode(dpool8, qd, tab, seq, 2000, synth.SCALE, out=out_d, workspace=ws_d, stream=s)

    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for c in calls:
            c()
        int8_calls()
    torch.cuda.synchronize()
    outs = (out_v, out_p, out_s, out_d, out_a, out_r, out_l, out_n)
    ref = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for c in calls:
            c()
        int8_calls()
    x = torch.randn(512, 512, device="cuda")
    for rep in range(4):
        for o in outs:
            o.fill_(0)
        y = x @ x
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, o, r in zip(("verify", "prefill", "sdpa", "int8", "int8 append", "valu rotated", "valu literal",
                               "noalloc"), outs, ref):
            assert torch.equal(o, r), f"replay {rep}: {name}"
        assert torch.isfinite(y).all()

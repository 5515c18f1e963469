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

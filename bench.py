"""Benchmark: TQ4 decode attention over a paged 4-bit KV cache on one MI355X.

A step is one decode step of all 16 full-attention layers at 212,992 cached
positions (196,608 prompt + 16,384 generated; 4 KV heads x 256 dims, 24 bf16
query heads, 256-token pages shuffled in a 229,376-position pool, one pool per
layer): per layer, one tq4_attn_decode_append call encodes the current token's
K and V into its slot and attends all cached positions in the same launch.
Inputs are resident in HBM before timing starts.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "TQ4 decode-attn cached positions/s & HBM GB/s (% peak) at 212,992 ctx"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 matrix
TQ4_BYTES_PER_POS_LAYER = 4 * 2 * 130  # 4 KV heads x (K, V) x (128 B words + 2 B norm)
EVENT_EVERY = 4  # time every 4th layer's call with events (fewer markers in the timed stream)


DECODE_PROFILE = os.path.join(ROOT, "profiles", "tq4_attn_split_kernel_decode_212k_16l.md")
DECODE_SOURCES = ["compressed_kv_attention_kvexec_amd/csrc/tq4_decode.hip",
                  "compressed_kv_attention_kvexec_amd/csrc/tq4_tile.h",
                  "compressed_kv_attention_kvexec_amd/csrc/tq4_device.h"]


def measured_traffic():
    """HBM bytes per decode launch from the committed PMC summary (FETCH_SIZE + WRITE_SIZE, each
    scaled by a 1 GiB copy), or None when the decode sources changed since it was taken."""
    import hashlib
    try:
        text = open(DECODE_PROFILE).read()
    except OSError:
        return None
    fields = dict(line.split(": ", 1) for line in text.splitlines() if line.startswith(("traffic_bytes", "source_sha")))
    h = hashlib.sha256()
    for f in DECODE_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    if fields.get("source_sha256", "").strip() != h.hexdigest()[:16]:
        return None
    return float(fields["traffic_bytes_per_launch"])


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def decode_algorithmic_bytes(seq_lens, page_size: int, n_q: int) -> int:
    """Bytes one decode launch must move: TQ4 records of every attended position,
    the queries, the output and the page-table entries (and lengths) it reads."""
    pages = sum(-(-L // page_size) for L in seq_lens)
    return (sum(seq_lens) * TQ4_BYTES_PER_POS_LAYER + len(seq_lens) * n_q * 256 * 2 * 2
            + pages * 4 + len(seq_lens) * 4)


def append_bytes(batch: int, n_kv: int) -> int:
    """Bytes the fused append adds to a decode call: the new token's fp32 K and V in, the two
    130 B records out, and the slot index, per request and KV head."""
    return batch * n_kv * 2 * (1024 + 130) + batch * 4


def build_layers(w, device, stats=None):
    """Per layer: pool, page table, lengths, query, current-token K/V and slot (GPU-encoded).
    stats (dict) receives the encode throughput measured on layer 0's pool build."""
    import torch
    import compressed_kv_attention_kvexec_amd as tq4
    import synth
    layers = []
    chunk = 32768
    for layer in range(w.n_layers):
        table = synth.placement(w, layer)
        slots = synth.used_slots(w, table)
        pool = tq4.Tq4LayerPool.empty(w.pool_pages, w.n_kv, w.page_size, device=device)
        slots_d = torch.from_numpy(slots).to(device)
        for which, seed_t in ((0, synth.T_K), (1, synth.T_V)):
            src = synth.torch_normal(synth.seed_of(w.wid, layer, seed_t), (len(slots), w.n_kv, 256), device)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for c0 in range(0, len(slots), chunk):
                part = src[c0:c0 + chunk]
                if which == 0:
                    tq4.tq4_encode_pages(pool, part, None, slots_d[c0:c0 + chunk])
                else:
                    tq4.tq4_encode_pages(pool, None, part, slots_d[c0:c0 + chunk])
            e1.record()
            if stats is not None and layer == 0:
                torch.cuda.synchronize()
                vecs = len(slots) * w.n_kv
                sec = e0.elapsed_time(e1) / 1e3
                stats.setdefault("encode_vectors", 0)
                stats.setdefault("encode_seconds", 0.0)
                stats["encode_vectors"] += vecs
                stats["encode_seconds"] += sec
            del src
        # the current token (last position of every request) is re-encoded inside each step
        last = []
        for b, L in enumerate(w.seq_lens):
            p = L - 1
            last.append(int(table[b, p // w.page_size]) * w.page_size + p % w.page_size)
        gen = torch.Generator(device=device)
        gen.manual_seed(synth.seed_of(w.wid, layer, 7))
        k_new = torch.randn((len(last), w.n_kv, 256), generator=gen, device=device)
        v_new = torch.randn((len(last), w.n_kv, 256), generator=gen, device=device)
        q = synth.torch_normal(synth.seed_of(w.wid, layer, synth.T_Q), (w.batch, w.n_q, 256), device)
        layers.append(dict(pool=pool, table=torch.from_numpy(table).to(device),
                           seq=torch.tensor(w.seq_lens, dtype=torch.int32, device=device),
                           q=q.to(torch.bfloat16).contiguous(), k_new=k_new, v_new=v_new,
                           slot_new=torch.tensor(last, dtype=torch.int32, device=device)))
        torch.cuda.synchronize()
        log(f"layer {layer}: pool built ({len(slots)} positions encoded)")
    return layers


def encode_leg(layer, w, device, tokens: int = 32768, reps: int = 10, groups: int = 5):
    """Encode throughput: back-to-back launches writing K and V of `tokens` tokens into layer 0's
    pool (its first used slots, rewritten with the same records), timed with events after 200
    untimed launches; the median over `groups` groups of `reps` launches."""
    import numpy as np
    import torch
    import compressed_kv_attention_kvexec_amd as tq4
    import synth
    slots = torch.from_numpy(synth.used_slots(w, synth.placement(w, 0))[:tokens]).to(device)
    k = synth.torch_normal(synth.seed_of(w.wid, 0, synth.T_K), (tokens, w.n_kv, 256), device)
    v = synth.torch_normal(synth.seed_of(w.wid, 0, synth.T_V), (tokens, w.n_kv, 256), device)
    call = tq4.prepare_encode(layer["pool"], k, v, slots)
    # ~15 ms of untimed launches first: the first milliseconds of launches run slower (a median of
    # 72 us over the first 200 against 63 us afterwards in a profiled run)
    for _ in range(200):
        call()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    times = []
    for _ in range(groups):
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            call()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / 1e3 / reps)
    sec = float(np.median(times))
    vecs = 2 * tokens * w.n_kv
    vps = vecs / sec
    # fp32 source in (1,024 B), one 130 B record out and the slot index per vector
    gbs = vps * (1024 + 130) / 1e9
    return {"vectors_per_s": vps, "gb_per_s": gbs, "frac_of_hbm_peak": gbs / HBM_PEAK_GBS,
            "us_per_launch": sec * 1e6,
            "sample": f"median of {groups} x {reps} launches of K and V for {tokens} tokens x {w.n_kv} heads "
                      "(fp32 source)"}


def decode_config_leg(name: str, device, reps: int = 20, n_queries: int = 1, variants=()) -> dict:
    """One layer of a decode workload timed cold: a read of 768 MiB evicts the 256 MB Infinity
    Cache before every call (a read, so no dirty lines are written back during the call).
    Reports the median call time, position-layers/s and GB/s of algorithmic bytes.  With
    n_queries > 1 the call is the packed verifier: the last n_queries positions of each request
    attend causally in one pass over its pages.  variants: decode variants ("valu_rotated",
    "valu_literal") timed the same way on the same pool, reported under "variants"."""
    import torch
    import compressed_kv_attention_kvexec_amd as tq4
    import synth
    w = synth.WORKLOADS[name]
    table = synth.placement(w, 0)
    slots = synth.used_slots(w, table)
    pool = tq4.Tq4LayerPool.empty(w.pool_pages, w.n_kv, w.page_size, device=device)
    sd = torch.from_numpy(slots).to(device)
    for which, st in ((0, synth.T_K), (1, synth.T_V)):
        src = synth.torch_normal(synth.seed_of(w.wid, 0, st), (len(slots), w.n_kv, 256), device)
        for c in range(0, len(slots), 65536):
            part = src[c:c + 65536]
            tq4.tq4_encode_pages(pool, part if which == 0 else None, part if which == 1 else None,
                                 sd[c:c + 65536])
        del src
    k = n_queries
    q = synth.torch_normal(synth.seed_of(w.wid, 0, synth.T_Q), (w.batch * k, w.n_q, 256), device).to(torch.bfloat16)
    tab = torch.from_numpy(table).to(device)
    seq = torch.tensor(w.seq_lens, dtype=torch.int32, device=device)
    ws = tq4.new_workspace(tq4.tq4_attn_verify_workspace_size(w.batch, max(w.seq_lens), k, w.n_q, w.n_kv,
                                                              w.page_size), device)
    if k == 1:
        out = torch.empty_like(q)
        call = tq4.prepare_decode(pool, q, tab, seq, max(w.seq_lens), synth.SCALE, out, ws)
        vcalls = {v: tq4.prepare_decode_variant(pool, q, tab, seq, max(w.seq_lens), synth.SCALE, v, out, ws)
                  for v in variants}
    else:
        q = q.reshape(w.batch, k, w.n_q, 256)
        out = torch.empty_like(q)
        call = tq4.prepare_verify(pool, q, tab, seq, max(w.seq_lens), synth.SCALE, out, ws)
    flush = torch.ones(192 << 20, dtype=torch.float32, device=device)

    def cold_median(fn):
        for _ in range(3):
            fn()
        times = []
        for _ in range(reps):
            flush.sum()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) / 1e3)
        if not torch.isfinite(out.float()).all():
            raise RuntimeError(f"non-finite output ({name}, {k} queries)")
        return sorted(times)[reps // 2]

    vt = {v: cold_median(fn) for v, fn in (vcalls.items() if k == 1 else ())}
    t = cold_median(call)
    positions = sum(w.seq_lens)
    nbytes = decode_algorithmic_bytes(w.seq_lens, w.page_size, w.n_q) + (k - 1) * w.batch * w.n_q * 256 * 2 * 2
    unique = len(slots) * TQ4_BYTES_PER_POS_LAYER
    # q.k and p.v products over the keys each query row attends
    flops = 4 * w.n_q * 256 * sum(max(L - k + i + 1, 0) for L in w.seq_lens for i in range(k))
    del pool, flush
    torch.cuda.empty_cache()
    r = {"workload": name, "batch": w.batch, "cached_positions": list(w.seq_lens), "page_size": w.page_size,
         "us_per_call": t * 1e6, "position_layers_per_s": positions / t, "gb_per_s": nbytes / t / 1e9,
         "frac_of_hbm_peak": nbytes / t / 1e9 / HBM_PEAK_GBS, "unique_tq4_bytes": unique,
         "timing": f"median of {reps} cold calls (768 MiB read between calls)"}
    if k > 1:
        r.update({"n_queries": k, "query_tokens_per_s": w.batch * k / t, "tflops": flops / t / 1e12})
    if vt:
        r["variants"] = {v: {"us_per_call": tv * 1e6, "gb_per_s": nbytes / tv / 1e9,
                             "frac_of_hbm_peak": nbytes / tv / 1e9 / HBM_PEAK_GBS, "vs_fused": tv / t}
                         for v, tv in vt.items()}
    return r


def unfused_leg(device, reps: int = 10) -> dict:
    """The unfused path on one layer of the 212,992-position workload, timed cold: reconstruct the
    pages into bf16 K/V (tq4_reconstruct_pages), then dense decode attention over them
    (tq4_sdpa_decode).  Reports each call, the sum, and the bytes the reconstruction materialises."""
    import torch
    import compressed_kv_attention_kvexec_amd as tq4
    import synth
    w = synth.WORKLOADS["decode_212k_16l"]
    table = synth.placement(w, 0)
    slots = synth.used_slots(w, table)
    pool = tq4.Tq4LayerPool.empty(w.pool_pages, w.n_kv, w.page_size, device=device)
    sd = torch.from_numpy(slots).to(device)
    for which, st in ((0, synth.T_K), (1, synth.T_V)):
        src = synth.torch_normal(synth.seed_of(w.wid, 0, st), (len(slots), w.n_kv, 256), device)
        for c in range(0, len(slots), 65536):
            part = src[c:c + 65536]
            tq4.tq4_encode_pages(pool, part if which == 0 else None, part if which == 1 else None,
                                 sd[c:c + 65536])
        del src
    L = w.seq_lens[0]
    q = synth.torch_normal(synth.seed_of(w.wid, 0, synth.T_Q), (1, w.n_q, 256), device).to(torch.bfloat16)
    tab = torch.from_numpy(table).to(device)
    seq = torch.tensor([L], dtype=torch.int32, device=device)
    k = torch.empty((1, w.n_kv, L, 256), dtype=torch.bfloat16, device=device)
    v = torch.empty_like(k)
    out = torch.empty_like(q)
    ws = tq4.new_workspace(tq4.tq4_sdpa_decode_workspace_size(1, L, w.n_q, w.n_kv), device)
    rec = tq4.prepare_reconstruct(pool, tab, seq, L, k, v)
    att = tq4.prepare_sdpa_decode(q, k, v, seq, synth.SCALE, out, ws)
    flush = torch.ones(192 << 20, dtype=torch.float32, device=device)
    for _ in range(2):
        rec()
        att()
    t_rec, t_att = [], []
    for _ in range(reps):
        flush.sum()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record()
        rec()
        e[1].record()
        att()
        e[2].record()
        torch.cuda.synchronize()
        t_rec.append(e[0].elapsed_time(e[1]) / 1e3)
        t_att.append(e[1].elapsed_time(e[2]) / 1e3)
    if not torch.isfinite(out.float()).all():
        raise RuntimeError("non-finite unfused output")
    tr, ta = sorted(t_rec)[reps // 2], sorted(t_att)[reps // 2]
    kv_bytes = 2 * w.n_kv * L * 256 * 2
    tq4_bytes = L * TQ4_BYTES_PER_POS_LAYER
    del pool, k, v, flush
    torch.cuda.empty_cache()
    return {"workload": w.name, "layers": 1, "cached_positions": L,
            "reconstruct_us": tr * 1e6, "sdpa_us": ta * 1e6, "total_us": (tr + ta) * 1e6,
            "materialized_bf16_kv_bytes": kv_bytes,
            "reconstruct_gb_per_s": (tq4_bytes + kv_bytes) / tr / 1e9,
            "sdpa_gb_per_s": (kv_bytes + 2 * w.n_q * 256 * 2) / ta / 1e9,
            "timing": f"median of {reps} cold calls (768 MiB read before each pair)"}


INT8_BYTES_PER_POS_LAYER = 4 * 2 * 258  # 4 KV heads x (K, V) x (256 codes + 2 B scale)


def int8_leg(name: str, device, reps: int = 20) -> dict:
    """The uniform INT8 arm on one layer of a decode workload, timed cold like the TQ4 configs:
    records written by tq4_int8_encode_pages, one tq4_int8_attn_decode call per timing.  Also
    times the INT8 encoder over 32,768 tokens."""
    import torch
    import compressed_kv_attention_kvexec_amd as tq4
    import synth
    w = synth.WORKLOADS[name]
    table = synth.placement(w, 0)
    slots = synth.used_slots(w, table)
    pool = tq4.Int8LayerPool.empty(w.pool_pages, w.n_kv, w.page_size, device=device)
    sd = torch.from_numpy(slots).to(device)
    for which, st in ((0, synth.T_K), (1, synth.T_V)):
        src = synth.torch_normal(synth.seed_of(w.wid, 0, st), (len(slots), w.n_kv, 256), device)
        for c in range(0, len(slots), 65536):
            part = src[c:c + 65536]
            tq4.tq4_int8_encode_pages(pool, part if which == 0 else None, part if which == 1 else None,
                                      sd[c:c + 65536])
        del src
    q = synth.torch_normal(synth.seed_of(w.wid, 0, synth.T_Q), (w.batch, w.n_q, 256), device).to(torch.bfloat16)
    tab = torch.from_numpy(table).to(device)
    seq = torch.tensor(w.seq_lens, dtype=torch.int32, device=device)
    ws = tq4.new_workspace(tq4.tq4_int8_attn_decode_workspace_size(w.batch, max(w.seq_lens), w.n_q, w.n_kv,
                                                                   w.page_size), device)
    out = torch.empty_like(q)
    call = tq4.prepare_int8_decode(pool, q, tab, seq, max(w.seq_lens), synth.SCALE, out, ws)
    flush = torch.ones(192 << 20, dtype=torch.float32, device=device)
    for _ in range(3):
        call()
    times = []
    for _ in range(reps):
        flush.sum()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        call()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / 1e3)
    if not torch.isfinite(out.float()).all():
        raise RuntimeError(f"non-finite INT8 output ({name})")
    t = sorted(times)[reps // 2]
    pages = sum(-(-L // w.page_size) for L in w.seq_lens)
    positions = sum(w.seq_lens)
    nbytes = positions * INT8_BYTES_PER_POS_LAYER + w.batch * w.n_q * 256 * 2 * 2 + pages * 4 + w.batch * 4
    # the same call with the fused append: the new token's fp32 K and V written as the records of
    # position seq_len - 1 of each request inside the launch
    new_kv = synth.torch_normal(synth.seed_of(w.wid, 2, synth.T_K), (2, w.batch, w.n_kv, 256), device)
    last = torch.tensor([int(table[b, (L - 1) // w.page_size]) * w.page_size + (L - 1) % w.page_size
                         for b, L in enumerate(w.seq_lens)], dtype=torch.int32, device=device)
    acall = tq4.prepare_int8_decode_append(pool, new_kv[0], new_kv[1], last, q, tab, seq, max(w.seq_lens),
                                           synth.SCALE, out, ws)
    for _ in range(2):
        acall()
    at = []
    for _ in range(reps):
        flush.sum()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        acall()
        e1.record()
        torch.cuda.synchronize()
        at.append(e0.elapsed_time(e1) / 1e3)
    t_append = sorted(at)[reps // 2]
    # the packed verifier over the same INT8 pages: the last k positions of each request
    verify = []
    for k in (2, 4, 8):
        qv = synth.torch_normal(synth.seed_of(w.wid, 0, synth.T_Q), (w.batch, k, w.n_q, 256), device).to(torch.bfloat16)
        outv = torch.empty_like(qv)
        wsv = tq4.new_workspace(tq4.tq4_int8_attn_verify_workspace_size(w.batch, max(w.seq_lens), k, w.n_q, w.n_kv,
                                                                        w.page_size), device)
        vcall = tq4.prepare_int8_verify(pool, qv, tab, seq, max(w.seq_lens), synth.SCALE, outv, wsv)
        for _ in range(2):
            vcall()
        vt = []
        for _ in range(reps // 2):
            flush.sum()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            vcall()
            e1.record()
            torch.cuda.synchronize()
            vt.append(e0.elapsed_time(e1) / 1e3)
        tv = sorted(vt)[len(vt) // 2]
        verify.append({"n_queries": k, "us_per_call": tv * 1e6, "query_tokens_per_s": w.batch * k / tv})
    # encoder: 32,768 tokens of fp32 K and V
    tokens = 32768
    k = synth.torch_normal(synth.seed_of(w.wid, 1, synth.T_K), (tokens, w.n_kv, 256), device)
    v = synth.torch_normal(synth.seed_of(w.wid, 1, synth.T_V), (tokens, w.n_kv, 256), device)
    es = sd[:tokens]
    for _ in range(2):
        tq4.tq4_int8_encode_pages(pool, k, v, es)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        tq4.tq4_int8_encode_pages(pool, k, v, es)
    e1.record()
    torch.cuda.synchronize()
    te = e0.elapsed_time(e1) / 1e3 / 10
    enc_bytes = tokens * w.n_kv * 2 * (1024 + 258) + tokens * 4
    del pool, flush, k, v
    torch.cuda.empty_cache()
    return {"workload": name, "cached_positions": list(w.seq_lens), "us_per_call": t * 1e6,
            "position_layers_per_s": positions / t, "gb_per_s": nbytes / t / 1e9,
            "frac_of_hbm_peak": nbytes / t / 1e9 / HBM_PEAK_GBS,
            "int8_bytes_per_position_layer": INT8_BYTES_PER_POS_LAYER,
            "encode_vectors_per_s": tokens * w.n_kv * 2 / te, "encode_gb_per_s": enc_bytes / te / 1e9,
            "append_us_per_call": t_append * 1e6,
            "verify": verify,
            "timing": f"median of {reps} cold calls (768 MiB read between calls)"}


def prefill_leg(device, reps: int = 3, int8: bool = False):
    """The chunked-prefill workload: 2,048 bf16 query tokens x 24 heads over 194,560 cached
    positions plus the chunk itself (causal inside the chunk), one layer, over TQ4 pages (or the
    INT8 arm's pages).  Reports the call time and useful matrix-core throughput
    (4 * heads * 256 * attended pairs)."""
    import torch
    import compressed_kv_attention_kvexec_amd as tq4
    import synth
    w = synth.WORKLOADS["prefill_2k_over_194k"]
    table = synth.placement(w, 0)
    slots = synth.used_slots(w, table)
    if int8:
        pool = tq4.Int8LayerPool.empty(w.pool_pages, w.n_kv, w.page_size, device=device)
        encode = tq4.tq4_int8_encode_pages
    else:
        pool = tq4.Tq4LayerPool.empty(w.pool_pages, w.n_kv, w.page_size, device=device)
        encode = tq4.tq4_encode_pages
    sd = torch.from_numpy(slots).to(device)
    for which, st in ((0, synth.T_K), (1, synth.T_V)):
        src = synth.torch_normal(synth.seed_of(w.wid, 0, st), (len(slots), w.n_kv, 256), device)
        for c in range(0, len(slots), 65536):
            kv = (src[c:c + 65536], None) if which == 0 else (None, src[c:c + 65536])
            encode(pool, *kv, sd[c:c + 65536])
        del src
    q = synth.torch_normal(synth.seed_of(w.wid, 0, synth.T_Q), (w.chunk_len, w.n_q, 256), device)
    q = q.to(torch.bfloat16).contiguous()
    tb = torch.from_numpy(table[0]).to(device)
    ws = tq4.new_workspace(tq4.tq4_attn_prefill_workspace_size(w.prior_len, w.chunk_len, w.n_q, w.n_kv,
                                                               w.page_size), device)
    out = torch.empty_like(q)
    prepare = tq4.prepare_int8_prefill if int8 else tq4.prepare_prefill
    call = prepare(pool, q, tb, w.prior_len, synth.SCALE, out, ws)
    call()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in ev:
        e0.record()
        call()
        e1.record()
    torch.cuda.synchronize()
    ms = sorted(e0.elapsed_time(e1) for e0, e1 in ev)[reps // 2]
    pairs = sum(w.prior_len + t + 1 for t in range(w.chunk_len))
    flop = 4 * w.n_q * 256 * pairs
    if not torch.isfinite(out.float()).all():
        raise RuntimeError("non-finite prefill output")
    tflops = flop / (ms / 1e3) / 1e12
    return {"workload": w.name, "ms_per_call": ms, "tflop_per_call": flop / 1e12, "achieved_tflops": tflops,
            "peak_tflops": MFMA_F16_PEAK_TFLOPS, "frac": tflops / MFMA_F16_PEAK_TFLOPS,
            "query_tokens_per_s": w.chunk_len / (ms / 1e3), "calls_timed": reps}


def torch_sum_read(device, gib: int = 4, reps: int = 5) -> float:
    """Read rate of torch's fp32 sum over `gib` GiB (far beyond the 256 MB Infinity Cache), GB/s,
    best of `reps`: what a library reduction kernel reads (a reference point)."""
    import torch
    x = torch.ones(gib * (1 << 30) // 4, dtype=torch.float32, device=device)
    x.sum()
    torch.cuda.synchronize()
    best = 0.0
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        x.sum()
        e1.record()
        torch.cuda.synchronize()
        best = max(best, x.numel() * 4 / (e0.elapsed_time(e1) / 1e3) / 1e9)
    del x
    torch.cuda.empty_cache()
    return best


def stream_read_probe(device, gib: int = 4, reps: int = 5, call_bytes: int = 0) -> dict:
    """Read rate of the streaming-read probe (libtq4probe.so, compressed_kv_attention_kvexec_amd/csrc/tq4_probe.h)
    over `gib` GiB: the best over grid sizes, loads in flight per thread and `reps` repetitions,
    i.e. what a plain streaming-read kernel reaches on this device; with call_bytes, also the best
    configuration's cold time over that many bytes."""
    import ctypes
    import torch
    from compressed_kv_attention_kvexec_amd import build as hipbuild
    lib = ctypes.CDLL(hipbuild.PROBE_LIB)
    lib.tq4_probe_sink_words.argtypes = [ctypes.c_int32]
    lib.tq4_probe_sink_words.restype = ctypes.c_size_t
    lib.tq4_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int32,
                                          ctypes.c_int32, ctypes.c_void_p]
    lib.tq4_probe_stream_read.restype = ctypes.c_int
    nbytes = gib << 30
    x = torch.ones(nbytes // 4, dtype=torch.float32, device=device)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    best = {"gb_per_s": 0.0}
    sweep = []
    for u in (4, 8, 16):
        for wgs in (256, 512, 1024, 2048, 4096):
            sink = torch.empty(lib.tq4_probe_sink_words(wgs), dtype=torch.int32, device=device)
            args = (ctypes.c_void_p(x.data_ptr()), nbytes, ctypes.c_void_p(sink.data_ptr()), wgs, u, stream)
            if lib.tq4_probe_stream_read(*args) != 0:
                raise RuntimeError("stream-read probe launch failed")
            top = 0.0
            for _ in range(reps):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                lib.tq4_probe_stream_read(*args)
                e1.record()
                torch.cuda.synchronize()
                top = max(top, nbytes / (e0.elapsed_time(e1) / 1e3) / 1e9)
            sweep.append({"loads_in_flight": u, "workgroups": wgs, "gb_per_s": top})
            if top > best["gb_per_s"]:
                best = {"gb_per_s": top, "workgroups": wgs, "loads_in_flight": u}
            del sink
    best["bytes"] = nbytes
    best["threads_per_workgroup"] = 512
    best["sweep"] = sweep
    if call_bytes:
        # the best configuration over one decode call's byte count, timed like the one-layer decode
        # legs (768 MiB read before every call): a plain read's time for those bytes, launch included
        nb = call_bytes // 16 * 16
        sink = torch.empty(lib.tq4_probe_sink_words(best["workgroups"]), dtype=torch.int32, device=device)
        args = (ctypes.c_void_p(x.data_ptr()), nb, ctypes.c_void_p(sink.data_ptr()), best["workgroups"],
                best["loads_in_flight"], stream)
        flush = torch.ones(192 << 20, dtype=torch.float32, device=device)
        times = []
        for i in range(23):
            flush.sum()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            lib.tq4_probe_stream_read(*args)
            e1.record()
            torch.cuda.synchronize()
            if i >= 3:
                times.append(e0.elapsed_time(e1) * 1e3)
        t = sorted(times)[len(times) // 2]
        best["call_bytes"] = {"bytes": nb, "us": t, "gb_per_s": nb / t / 1e3,
                              "timing": "median of 20 cold reads (768 MiB read before each)"}
        del flush, sink
    del x
    torch.cuda.empty_cache()
    return best


def cpu_model_name() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            return next((line.split(":", 1)[1].strip() for line in f if line.startswith("model name")), "")
    except OSError:
        return ""


def cpu_threads() -> int:
    """Threads the CPU oracle runs on: the cores this process may use, at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def oracle_pool_for(w, layer: int = 0):
    """The oracle's TQ4 pool of a workload's cached positions (seeded synth sources), encoded with
    the oracle's encoder on all threads (disjoint slots per thread).  Not timed."""
    import numpy as np
    import oracle
    import synth
    from concurrent.futures import ThreadPoolExecutor
    table = synth.placement(w, layer)
    slots = synth.used_slots(w, table)
    pool = oracle.Pool.empty(w.pool_pages, w.n_kv, w.page_size)
    k = synth.kv_source(w, layer, len(slots), synth.T_K)
    v = synth.kv_source(w, layer, len(slots), synth.T_V)
    bounds = np.linspace(0, len(slots), cpu_threads() + 1).astype(int)
    with ThreadPoolExecutor(max_workers=cpu_threads()) as ex:
        list(ex.map(lambda ab: oracle.encode_to_pool(pool, k[ab[0]:ab[1]], v[ab[0]:ab[1]], slots[ab[0]:ab[1]]),
                    zip(bounds[:-1], bounds[1:])))
    return pool, table


def _queries64(w, layer: int, rows: int):
    import numpy as np
    import synth
    return synth.bf16_round(synth.queries_f32(w, layer, rows)).astype(np.float64)


def cpu_decode_config(name: str) -> dict:
    """The oracle (plain C, fp64) on a one-layer decode workload in full: the whole call on one
    core, then the same call split over KV heads (the oracle's natural unit: one thread per KV head
    with its query heads) on all threads."""
    import oracle
    import synth
    from concurrent.futures import ThreadPoolExecutor
    w = synth.WORKLOADS[name]
    pool, table = oracle_pool_for(w)
    q = _queries64(w, 0, w.batch)
    t0 = time.perf_counter()
    oracle.attn_decode(pool, q, table, w.seq_lens, synth.SCALE)
    t1 = time.perf_counter() - t0
    G = w.n_q // w.n_kv
    threads = min(cpu_threads(), w.n_kv)
    with ThreadPoolExecutor(max_workers=threads) as ex:
        t0 = time.perf_counter()
        list(ex.map(lambda g: oracle.attn_decode(pool, q, table, w.seq_lens, synth.SCALE, heads=(g * G, (g + 1) * G)),
                    range(w.n_kv)))
        tn = time.perf_counter() - t0
    pos = sum(w.seq_lens)
    return {"value": pos / tn, "unit": "position-layers/s", "cores": threads, "kind": "oracle",
            "sample": f"full call ({pos} cached positions x {w.n_q} query heads), one thread per KV head",
            "seconds": tn, "single_core_value": pos / t1, "single_core_seconds": t1, "cpu_model": cpu_model_name()}


def cpu_decode_step(name: str, single_core_layer: bool) -> dict:
    """The oracle on a 16-layer decode step in full: 16 decode calls (one per layer, each with its
    own queries over the workload's pool, every cached position of every request), one layer per
    thread on all threads.  With single_core_layer, one layer's call is also timed on one core and
    scaled by the layer count (labelled as extrapolated)."""
    import oracle
    import synth
    from concurrent.futures import ThreadPoolExecutor
    w = synth.WORKLOADS[name]
    pool, table = oracle_pool_for(w)
    qs = [_queries64(w, layer, w.batch) for layer in range(w.n_layers)]
    threads = min(cpu_threads(), w.n_layers)
    with ThreadPoolExecutor(max_workers=threads) as ex:
        t0 = time.perf_counter()
        list(ex.map(lambda ql: oracle.attn_decode(pool, ql, table, w.seq_lens, synth.SCALE), qs))
        tn = time.perf_counter() - t0
    pos = sum(w.seq_lens)
    r = {"value": pos / tn, "unit": "positions/s", "cores": threads, "kind": "oracle",
         "sample": (f"full step: {w.n_layers} layers x {list(w.seq_lens)} cached positions x {w.n_q} query heads, "
                    f"one layer per thread over one oracle pool of the workload"),
         "seconds": tn, "cpu_model": cpu_model_name(), "host_cores_available": len(os.sched_getaffinity(0))}
    if single_core_layer:
        t0 = time.perf_counter()
        oracle.attn_decode(pool, qs[0], table, w.seq_lens, synth.SCALE)
        t1 = time.perf_counter() - t0
        r.update({"single_core_value": pos / (t1 * w.n_layers), "single_core_seconds_one_layer": t1,
                  "single_core_note": f"one layer on one core, scaled by {w.n_layers} layers (extrapolated)"})
    return r


def cpu_prefill_sample(n_rows: int = 32) -> dict:
    """The oracle on the 2,048-token prefill chunk over 194,560 positions: n_rows sampled query rows
    (t = 0 and t = 2047 among them) x 24 heads, one thread per (row, KV head); the full chunk's time
    is extrapolated by attended (query, key) pairs and labelled as such."""
    import numpy as np
    import oracle
    import synth
    from concurrent.futures import ThreadPoolExecutor
    w = synth.WORKLOADS["prefill_2k_over_194k"]
    pool, table = oracle_pool_for(w)
    rows = np.unique(np.linspace(0, w.chunk_len - 1, n_rows).round().astype(np.int32))
    q = _queries64(w, 0, w.chunk_len)[rows]
    G = w.n_q // w.n_kv
    units = [(i, g) for i in range(len(rows)) for g in range(w.n_kv)]
    threads = cpu_threads()
    with ThreadPoolExecutor(max_workers=threads) as ex:
        t0 = time.perf_counter()
        list(ex.map(lambda u: oracle.attn_prefill_rows(pool, q[u[0]:u[0] + 1], rows[u[0]:u[0] + 1], table[0],
                                                       w.prior_len, synth.SCALE, heads=(u[1] * G, (u[1] + 1) * G)),
                    units))
        tn = time.perf_counter() - t0
    pairs_sampled = int(sum(w.prior_len + int(t) + 1 for t in rows))
    pairs_all = int(sum(w.prior_len + t + 1 for t in range(w.chunk_len)))
    t_full = tn * pairs_all / pairs_sampled
    return {"value": w.chunk_len / t_full, "unit": "query tokens/s", "cores": threads, "kind": "oracle",
            "sample": (f"{len(rows)} of {w.chunk_len} query rows (t = 0 .. {w.chunk_len - 1}, evenly spaced) x {w.n_q} "
                       f"heads, one thread per (row, KV head); the chunk's time extrapolated by attended pairs"),
            "extrapolated": True, "sample_seconds": tn, "extrapolated_seconds": t_full,
            "cpu_model": cpu_model_name()}


def cpu_encode_baseline(tokens: int = 32768) -> dict:
    """The oracle's encoder (plain C, fp32 as the encoding rule fixes it) on K and V of `tokens`
    tokens x 4 KV heads (about 1% of one 212,992-position pool build): once on one core, then with
    the tokens split over T threads (each its own slots, so the records written are disjoint)."""
    import numpy as np
    import oracle
    import synth
    from concurrent.futures import ThreadPoolExecutor
    w0 = synth.WORKLOADS["decode_212k_16l"]
    w = synth.Workload(w0.wid, "enc_sample", "decode", 1, w0.page_size, w0.pool_pages, seq_lens=(tokens,))
    slots = synth.used_slots(w, synth.placement(w, 0))
    k = synth.kv_source(w, 0, tokens, synth.T_K)
    v = synth.kv_source(w, 0, tokens, synth.T_V)
    pool = oracle.Pool.empty(w.pool_pages, w.n_kv, w.page_size)
    t0 = time.perf_counter()
    oracle.encode_to_pool(pool, k, v, slots)
    dt1 = time.perf_counter() - t0
    n_threads = max(1, min(16, len(os.sched_getaffinity(0))))
    bounds = np.linspace(0, tokens, n_threads + 1).astype(int)
    parts = [(k[a:b], v[a:b], slots[a:b]) for a, b in zip(bounds[:-1], bounds[1:])]
    with ThreadPoolExecutor(max_workers=n_threads) as ex:
        t0 = time.perf_counter()
        list(ex.map(lambda kvs: oracle.encode_to_pool(pool, *kvs), parts))
        dtn = time.perf_counter() - t0
    vecs = 2 * tokens * w.n_kv
    return {"vectors_per_s": vecs / dtn, "cores": n_threads, "single_core_vectors_per_s": vecs / dt1,
            "kind": "oracle", "sample": f"K and V of {tokens} tokens x {w.n_kv} heads (fp32 source)"}


def calibration_copy(mib: int, dev) -> None:
    """One device copy of `mib` MiB: the reference dispatch for scaling the PMC byte counters."""
    import torch
    a = torch.ones(mib * (1 << 20) // 4, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    del a, b
    log(f"calibration copy of {mib} MiB done")


def run_decode_step(w, dev, steps: int, warmup: int, use_graph: bool = True, calibrate_mib: int = 0,
                    keep_layers: bool = False):
    """Time the decode step of a workload: w.n_layers fused calls (encode the new token, attend),
    one per layer, in order on one stream, as one HIP graph (and eagerly with events around every
    EVENT_EVERY-th call for the per-call duration).  Returns (result dict, layers or None)."""
    import torch
    import compressed_kv_attention_kvexec_amd as tq4
    import synth
    build_stats = {}
    layers = build_layers(w, dev, build_stats)
    ws_bytes = tq4.tq4_attn_decode_workspace_size(w.batch, max(w.seq_lens), w.n_q, w.n_kv, w.page_size)
    workspace = tq4.new_workspace(ws_bytes, dev)
    outs = [torch.empty_like(L["q"]) for L in layers]
    stream = torch.cuda.current_stream()
    # one fused call per layer: encode the step's new token into the layer's pages, then attend
    calls = [tq4.prepare_decode_append(L["pool"], L["k_new"], L["v_new"], L["slot_new"], L["q"], L["table"],
                                       L["seq"], max(w.seq_lens), synth.SCALE, outs[i], workspace, stream)
             for i, L in enumerate(layers)]
    timed_layers = list(range(0, w.n_layers, EVENT_EVERY))
    if calibrate_mib > 0:
        calibration_copy(calibrate_mib, dev)

    def step(events=None):
        for i in range(w.n_layers):
            timed = events is not None and i % EVENT_EVERY == 0
            if timed:
                events[i // EVENT_EVERY][0].record(stream)
            calls[i]()
            if timed:
                events[i // EVENT_EVERY][1].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    log(f"{w.name}: warmup {warmup} steps done")

    # The step as one HIP graph: the same calls captured on a side stream and replayed, which
    # removes the host launch gaps between them.
    graph = None
    if use_graph:
        gstream = torch.cuda.Stream()
        gcalls = [tq4.prepare_decode_append(L["pool"], L["k_new"], L["v_new"], L["slot_new"], L["q"], L["table"],
                                            L["seq"], max(w.seq_lens), synth.SCALE, outs[i], workspace, gstream)
                  for i, L in enumerate(layers)]
        try:
            gstream.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(gstream):
                for c in gcalls:  # one eager pass on the capture stream first
                    c()
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=gstream):
                for c in gcalls:
                    c()
            for _ in range(warmup):
                graph.replay()
            torch.cuda.synchronize()
            log(f"{w.name}: captured the step as a HIP graph; {warmup} warmup replays done")
        except Exception as exc:  # capture unsupported: fall back to the eager step
            log(f"graph capture failed ({exc}); timing the eager step")
            graph = None

    def timed_steps(run_step):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(steps):
            run_step(k)
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    # The graph replays run on the current stream; two HIP events on it bracket the timed replays,
    # so the per-call duration there is the events' time over steps x layers calls (the gaps
    # between the kernels included).
    graph_ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))

    def replay(k):
        if k == 0:
            graph_ev[0].record(stream)
        graph.replay()
        if k == steps - 1:
            graph_ev[1].record(stream)

    elapsed_graph = timed_steps(replay) if graph is not None else None
    graph_call_s = (graph_ev[0].elapsed_time(graph_ev[1]) / 1e3 / (steps * w.n_layers)
                    if graph is not None else None)
    # eager steps with per-call events on every EVENT_EVERY-th layer (each call bracketed alone)
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in timed_layers] for _ in range(steps)]
    elapsed_eager = timed_steps(lambda k: step(ev[k]))
    dec_ms = [e0.elapsed_time(e1) for row in ev for (e0, e1) in row]
    eager_call_s = sum(dec_ms) / len(dec_ms) / 1e3
    avg_dec_s = graph_call_s if graph_call_s is not None else eager_call_s
    elapsed = elapsed_graph if elapsed_graph is not None else elapsed_eager
    log(f"{w.name}: timed {steps} steps: {elapsed * 1e3 / steps:.3f} ms/step"
        f"{' (graph)' if elapsed_graph is not None else ''}, eager {elapsed_eager * 1e3 / steps:.3f} ms/step, "
        f"decode call avg {avg_dec_s * 1e6:.1f} us"
        f"{' in the graph' if graph_call_s is not None else ''} (eager, bracketed alone: {eager_call_s * 1e6:.1f} us)")
    for o in outs:  # a cheap guard that the timed work produced results
        if not torch.isfinite(o.float()).all():
            raise RuntimeError(f"non-finite decode output ({w.name})")
    positions = sum(w.seq_lens)  # cached positions per step, each across all layers
    bytes_launch = decode_algorithmic_bytes(w.seq_lens, w.page_size, w.n_q) + append_bytes(w.batch, w.n_kv)
    unique = len(synth.used_slots(w, synth.placement(w, 0))) * TQ4_BYTES_PER_POS_LAYER
    r = {"workload": w.name, "layers": w.n_layers, "batch": w.batch, "cached_positions": list(w.seq_lens),
         "ms_per_step": elapsed * 1e3 / steps, "positions_per_s": positions / (elapsed / steps),
         "execution": "hip graph of the step's calls" if elapsed_graph is not None else "eager launches",
         "eager_ms_per_step": elapsed_eager * 1e3 / steps,
         "eager_positions_per_s": positions / (elapsed_eager / steps),
         "avg_launch_us": avg_dec_s * 1e6, "bytes_per_launch": bytes_launch,
         "launch_timing": ("HIP events on the launch stream around the timed graph replays: their time over "
                           "steps x layers calls" if graph_call_s is not None else
                           "HIP events around single eager calls"),
         "eager_call_us": eager_call_s * 1e6,
         "achieved_gb_per_s": bytes_launch / avg_dec_s / 1e9,
         "frac_of_hbm_peak": bytes_launch / avg_dec_s / 1e9 / HBM_PEAK_GBS,
         "step_gb_per_s": bytes_launch * w.n_layers / (elapsed / steps) / 1e9,
         "step_frac_of_peak": bytes_launch * w.n_layers / (elapsed / steps) / 1e9 / HBM_PEAK_GBS,
         "unique_tq4_bytes_per_layer": unique,
         "eager_calls_timed": len(dec_ms),
         "eager_timed_calls": f"layers {timed_layers} of every eager timed step (events bracket each)",
         "encode_build": build_stats}
    del calls, workspace, graph
    if not keep_layers:
        del layers
        torch.cuda.empty_cache()
        return r, None
    return r, layers


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode_212k_16l")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="skip the chunked-prefill leg")
    ap.add_argument("--no-ablation", action="store_true",
                    help="skip the decode variants without matrix cores (rotated and literal, on the vector ALUs)")
    ap.add_argument("--variants", default="",
                    help="with --only-config: also time these decode variants (comma-separated)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other benchmark workloads (1k and 32k layers, the two-request step)")
    ap.add_argument("--no-verify", action="store_true",
                    help="skip the one-layer cold timings of the packed multi-query verifier")
    ap.add_argument("--no-unfused", action="store_true",
                    help="skip the reconstruct-then-dense-attention timing")
    ap.add_argument("--no-int8", action="store_true",
                    help="skip the uniform INT8 arm timing")
    ap.add_argument("--no-probe", action="store_true", help="skip the read-bandwidth reference points")
    ap.add_argument("--only-config", default="",
                    help="run only the cold one-layer timing of this decode workload (profiler runs)")
    ap.add_argument("--queries", type=int, default=1,
                    help="with --only-config: time the packed verifier with this many query tokens per request")
    ap.add_argument("--only-step", default="",
                    help="run only the timed decode step of this workload, no other leg (profiler runs)")
    ap.add_argument("--only-prefill", action="store_true",
                    help="run only the TQ4 chunked-prefill timing (profiler runs)")
    ap.add_argument("--only-encode", action="store_true",
                    help="run only the encode timing, into an empty pool of the workload's size (profiler runs)")
    ap.add_argument("--int8-only", action="store_true",
                    help="run only the uniform INT8 arm timing (profiler runs)")
    ap.add_argument("--no-graph", action="store_true",
                    help="time the eager per-layer launches instead of a HIP graph of the step")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="run one device copy of this many MiB first (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        return 2

    import torch
    import compressed_kv_attention_kvexec_amd as tq4
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tq4.load_library()
    if args.only_config:  # one cold one-layer decode workload alone, for profiler runs
        if args.calibrate_copy_mib > 0:
            calibration_copy(args.calibrate_copy_mib, dev)
        variants = tuple(v for v in args.variants.split(",") if v)
        print(json.dumps({"decode_config": decode_config_leg(args.only_config, dev, n_queries=args.queries,
                                                             variants=variants)}), flush=True)
        return 0
    if args.int8_only:  # the INT8 arm alone, for profiler runs
        if args.calibrate_copy_mib > 0:
            calibration_copy(args.calibrate_copy_mib, dev)
        print(json.dumps({"int8": int8_leg(args.workload, dev)}), flush=True)
        return 0
    if args.only_encode:  # the encoder alone, for profiler runs
        if args.calibrate_copy_mib > 0:
            calibration_copy(args.calibrate_copy_mib, dev)
        w = synth.WORKLOADS[args.workload]
        pool = tq4.Tq4LayerPool.empty(w.pool_pages, w.n_kv, w.page_size, device=dev)
        print(json.dumps({"encode": encode_leg({"pool": pool}, w, dev)}), flush=True)
        return 0
    if args.only_prefill:  # the TQ4 prefill chunk alone, for profiler runs
        print(json.dumps({"prefill": prefill_leg(dev)}), flush=True)
        return 0
    if args.only_step:  # one timed decode step workload alone, for profiler runs
        r, _ = run_decode_step(synth.WORKLOADS[args.only_step], dev, args.steps, args.warmup, not args.no_graph,
                               args.calibrate_copy_mib)
        print(json.dumps({"step": r}), flush=True)
        return 0

    w = synth.WORKLOADS[args.workload]
    assert w.kind == "decode"
    log(f"workload {w.name}: {w.n_layers} layers, seq_lens {w.seq_lens}")
    head, layers = run_decode_step(w, dev, args.steps, args.warmup, not args.no_graph, args.calibrate_copy_mib,
                                   keep_layers=True)
    positions = sum(w.seq_lens)
    result = {
        "metric": METRIC, "value": head["positions_per_s"], "unit": "positions/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": w.name, "layers": w.n_layers, "batch": w.batch,
                   "cached_positions": list(w.seq_lens), "n_q_heads": w.n_q, "n_kv_heads": w.n_kv,
                   "head_dim": 256, "page_size": w.page_size, "pool_pages": w.pool_pages,
                   "query_dtype": "bf16"},
        "roofline": {"bound": "hbm", "achieved": head["achieved_gb_per_s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": head["achieved_gb_per_s"] / HBM_PEAK_GBS, "traffic": measured_traffic(),
                     "kernel": "tq4_attn_decode_append call = tq4_attn_split_kernel<1, 8> + tq4_decode_combine_kernel",
                     "bytes_per_launch": head["bytes_per_launch"], "avg_launch_us": head["avg_launch_us"]},
        "extra": {"step": head, "step_hbm_gb_per_s": head["step_gb_per_s"],
                  "step_frac_of_peak": head["step_frac_of_peak"]},
    }
    result["extra"]["encode"] = encode_leg(layers[0], w, dev)
    log(f"encode: {result['extra']['encode']['vectors_per_s'] / 1e9:.2f} G vectors/s, "
        f"{result['extra']['encode']['gb_per_s']:.0f} GB/s")
    del layers
    torch.cuda.empty_cache()
    if not args.no_probe:
        # plain streaming reads over 4 GiB: torch's reduction and the probe's sweep (a measured ceiling)
        result["extra"]["torch_sum_read_gb_per_s"] = torch_sum_read(dev)
        probe = result["extra"]["stream_read_probe"] = stream_read_probe(dev, call_bytes=head["bytes_per_launch"])
        # the decode call's rate as a fraction of the best plain streaming read measured here
        result["extra"]["decode_frac_of_stream_read_probe"] = result["roofline"]["achieved"] / probe["gb_per_s"]
        log(f"torch.sum over 4 GiB fp32: {result['extra']['torch_sum_read_gb_per_s']:.0f} GB/s; stream-read probe "
            f"{probe['gb_per_s']:.0f} GB/s ({probe['loads_in_flight']} loads in flight, {probe['workgroups']} "
            f"workgroups); decode call at {result['extra']['decode_frac_of_stream_read_probe']:.3f} of it; "
            f"the probe over one call's {probe['call_bytes']['bytes'] / 1e6:.1f} MB: {probe['call_bytes']['us']:.1f} us cold")
    configs = result["extra"]["configs"] = {}
    if not args.no_configs:
        for name in ("decode_1k_p64", "decode_32k"):
            r = decode_config_leg(name, dev)
            configs[name] = {"gpu": r}
            log(f"{name}: {r['us_per_call']:.1f} us/call, {r['gb_per_s']:.0f} GB/s (cold)")
        w3 = synth.WORKLOADS["decode_2req_shared"]
        r3, _ = run_decode_step(w3, dev, args.steps, args.warmup, not args.no_graph)
        configs[w3.name] = {"gpu_step": r3, "gpu_one_layer_cold": decode_config_leg(w3.name, dev)}
        log(f"{w3.name}: {r3['ms_per_step']:.3f} ms/step, {r3['positions_per_s'] / 1e6:.1f} M positions/s, "
            f"{r3['step_gb_per_s']:.0f} GB/s logical")
    if not args.no_verify:
        result["extra"]["verify"] = []
        for k in (2, 4, 8):
            r = decode_config_leg(w.name, dev, n_queries=k)
            result["extra"]["verify"].append(r)
            log(f"verify k={k} at {w.seq_lens}: {r['us_per_call']:.1f} us/call, {r['gb_per_s']:.0f} GB/s, "
                f"{r['tflops']:.1f} TFLOP/s (cold)")
    if not args.no_ablation:
        r = decode_config_leg(w.name, dev, variants=("valu_rotated", "valu_literal"))
        result["extra"]["ablation"] = r
        log(f"decode ablation at {w.seq_lens}: fused {r['us_per_call']:.1f} us, " + ", ".join(
            f"{v} {x['us_per_call']:.1f} us ({x['vs_fused']:.2f}x)" for v, x in r["variants"].items()))
    tq4_cold_cache = {}

    def tq4_cold_us():  # the fused call timed like the unfused and INT8 legs: one cold layer
        if "us" not in tq4_cold_cache:
            tq4_cold_cache["us"] = decode_config_leg(w.name, dev)["us_per_call"]
        return tq4_cold_cache["us"]

    if not args.no_unfused:
        r = unfused_leg(dev)
        r["fused_call_us"] = tq4_cold_us()
        r["fused_call_timing"] = "one cold layer, median of 20 calls (768 MiB read between calls)"
        r["unfused_over_fused"] = r["total_us"] / r["fused_call_us"]
        result["extra"]["unfused"] = r
        log(f"unfused: reconstruct {r['reconstruct_us']:.1f} us + dense attention {r['sdpa_us']:.1f} us "
            f"= {r['total_us']:.1f} us ({r['unfused_over_fused']:.1f}x the fused call), "
            f"{r['materialized_bf16_kv_bytes'] / 2**20:.0f} MiB of bf16 K/V")
    if not args.no_int8:
        r = int8_leg(w.name, dev)
        r["tq4_cold_us_per_call"] = tq4_cold_us()
        r["int8_over_tq4"] = r["us_per_call"] / r["tq4_cold_us_per_call"]
        result["extra"]["int8"] = r
        log(f"int8 arm: {r['us_per_call']:.1f} us/call, {r['gb_per_s']:.0f} GB/s (cold); TQ4 cold "
            f"{r['tq4_cold_us_per_call']:.1f} us ({r['int8_over_tq4']:.2f}x); encode {r['encode_gb_per_s']:.0f} GB/s; "
            f"verify k=2/4/8 " + " / ".join(f"{v['us_per_call']:.1f}" for v in r["verify"]) + " us")
    if not args.no_prefill:
        log("prefill leg ...")
        pf = prefill_leg(dev)
        result["extra"]["prefill"] = pf
        configs["prefill_2k_over_194k"] = {"gpu": pf}
        log(f"prefill: {pf['ms_per_call']:.3f} ms/call, {pf['achieved_tflops']:.1f} TFLOP/s")
        if not args.no_int8:
            r = prefill_leg(dev, int8=True)
            result["extra"]["int8"]["prefill"] = r
            log(f"int8 prefill: {r['ms_per_call']:.3f} ms/call, {r['achieved_tflops']:.1f} TFLOP/s")
    if not args.no_cpu_baseline:
        log("cpu baseline: the oracle on the full 16-layer step ...")
        result["cpu_baseline"] = cb = cpu_decode_step(w.name, single_core_layer=True)
        log(f"cpu baseline: {cb['value']:.0f} positions/s on {cb['cores']} threads in {cb['seconds']:.1f} s "
            f"({cb['single_core_value']:.0f} on one core, extrapolated from one layer)")
        if "encode" in result.get("extra", {}):
            ce = result["extra"]["encode"]["cpu_oracle"] = cpu_encode_baseline()
            log(f"cpu oracle encode: {ce['vectors_per_s'] / 1e6:.2f} M vectors/s on {ce['cores']} threads "
                f"({ce['single_core_vectors_per_s'] / 1e6:.3f} M on one core)")
        if not args.no_configs:
            for name in ("decode_1k_p64", "decode_32k"):
                configs[name]["cpu_baseline"] = c = cpu_decode_config(name)
                log(f"cpu baseline {name}: {c['value']:.0f} position-layers/s on {c['cores']} threads "
                    f"({c['single_core_value']:.0f} on one core)")
            configs["decode_2req_shared"]["cpu_baseline"] = c = cpu_decode_step("decode_2req_shared", False)
            log(f"cpu baseline decode_2req_shared: {c['value']:.0f} positions/s on {c['cores']} threads "
                f"in {c['seconds']:.1f} s")
        if not args.no_prefill:
            configs["prefill_2k_over_194k"]["cpu_baseline"] = c = cpu_prefill_sample()
            log(f"cpu baseline prefill: {c['value']:.2f} query tokens/s (extrapolated from {c['sample_seconds']:.1f} s "
                f"on {c['cores']} threads)")
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

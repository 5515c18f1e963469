"""Seeded synthetic inputs for the TQ4 paged-attention workloads.

This module is shared by the oracle side and the GPU side of the tests and by
the benchmark.  It draws random numbers and page placements only; it holds none
of the codec's or attention's arithmetic.

Workload shapes follow the JustFit pages: 4 KV heads of dimension 256 per
full-attention layer and 16 such layers ("Fitting a 27B-Parameter LLM into
24 GiB of Laptop Memory", section "The Memory Budget Equation"), 256-token pages
(section "KVExec: Fused Reconstruction with Layer-Scoped Lifetime"), a
229,376-position page pool and 196,608 + 16,384 = 212,992 retained positions
(section "Results: 212K Positions, Three for Three").  The 24 bf16 query heads,
N(0,1) sources and the 1/16 softmax scale are readings stated with each
workload below.

Seeds: 20260915 + 1000 * workload_id + 10 * layer + tensor, where tensor is
0 = K source, 1 = V source, 2 = queries, 3 = page placement, 5 / 6 = per-position
K / V scale factors (mixed-norm pools).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

BASE_SEED = 20260915
T_K, T_V, T_Q, T_PLACE = 0, 1, 2, 3
T_KSCALE, T_VSCALE = 5, 6

HEAD_DIM = 256
N_KV = 4
N_Q = 24
SCALE = 1.0 / 16.0


def seed_of(workload_id: int, layer: int, tensor: int) -> int:
    return BASE_SEED + 1000 * workload_id + 10 * layer + tensor


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: a decode step or a prefill chunk."""
    wid: int
    name: str
    kind: str                      # "decode" or "prefill"
    n_layers: int
    page_size: int
    pool_pages: int
    seq_lens: tuple = ()           # decode: cached positions per request (incl. current token)
    shared_prefix_pages: int = 0   # decode: leading pages shared by all requests
    prior_len: int = 0             # prefill: positions already cached
    chunk_len: int = 0             # prefill: query tokens in the chunk
    n_kv: int = N_KV
    n_q: int = N_Q
    note: str = field(default="", compare=False)

    @property
    def batch(self) -> int:
        return len(self.seq_lens) if self.kind == "decode" else 1

    def pages_of(self, length: int) -> int:
        return -(-length // self.page_size)

    @property
    def table_stride(self) -> int:
        if self.kind == "decode":
            return max(self.pages_of(L) for L in self.seq_lens)
        return self.pages_of(self.prior_len + self.chunk_len)

    @property
    def positions(self) -> int:
        """Cached positions attended per layer (decode: summed over requests)."""
        if self.kind == "decode":
            return int(sum(self.seq_lens))
        return self.prior_len + self.chunk_len


WORKLOADS = {
    w.name: w for w in [
        Workload(0, "decode_1k_p64", "decode", 1, 64, 32, seq_lens=(1024,),
                 note="1 layer, 1 request, 1,024 positions in 16 pages of 64 at random slots of a 32-page pool"),
        Workload(1, "decode_32k", "decode", 1, 256, 896, seq_lens=(32768,),
                 note="1 layer, 1 request, 32,768 positions, 256-token pages shuffled in a 229,376-position pool"),
        Workload(2, "decode_212k_16l", "decode", 16, 256, 896, seq_lens=(212992,),
                 note="16 layers, 1 request, 212,992 positions (196,608 prompt + 16,384 generated)"),
        Workload(3, "decode_2req_shared", "decode", 16, 256, 896, seq_lens=(131072, 98304),
                 shared_prefix_pages=128,
                 note="16 layers, 2 requests (131,072 and 98,304 positions) sharing a 32,768-position prefix"),
        Workload(4, "prefill_2k_over_194k", "prefill", 1, 256, 896, prior_len=194560, chunk_len=2048,
                 note="1 layer, a 2,048-token chunk over 194,560 cached positions, causal inside the chunk"),
    ]
}


def placement(workload: Workload, layer: int = 0) -> np.ndarray:
    """Page tables int32 [batch][table_stride] for a workload.

    Pages are drawn without replacement from a seeded permutation of the pool.
    With a shared prefix, every request's first `shared_prefix_pages` entries
    name the same pages; the rest are distinct.  Unused table entries are 0."""
    rng = np.random.Generator(np.random.PCG64(seed_of(workload.wid, layer, T_PLACE)))
    perm = rng.permutation(workload.pool_pages).astype(np.int32)
    stride = workload.table_stride
    if workload.kind == "prefill":
        n = workload.pages_of(workload.prior_len + workload.chunk_len)
        assert n <= workload.pool_pages
        return perm[:n].reshape(1, n).copy()
    table = np.zeros((workload.batch, stride), np.int32)
    shared = workload.shared_prefix_pages
    table[:, :shared] = perm[:shared]
    cursor = shared
    for b, L in enumerate(workload.seq_lens):
        n = workload.pages_of(L)
        own = n - shared
        assert cursor + own <= workload.pool_pages, "pool too small for the workload"
        table[b, shared:n] = perm[cursor:cursor + own]
        cursor += own
    return table


def used_slots(workload: Workload, table: np.ndarray) -> np.ndarray:
    """Distinct pool slots (page * P + offset) holding cached positions, in first-use order."""
    P = workload.page_size
    seen, out = set(), []
    lens = workload.seq_lens if workload.kind == "decode" else (workload.prior_len + workload.chunk_len,)
    for b, L in enumerate(lens):
        for p in range(workload.pages_of(L)):
            page = int(table[b, p])
            if page in seen:
                continue
            seen.add(page)
            n = min(P, L - p * P)
            out.append(page * P + np.arange(n, dtype=np.int64))
    return np.concatenate(out).astype(np.int32)


def normal_f32(seed: int, shape) -> np.ndarray:
    """N(0,1) fp32 from numpy PCG64."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.standard_normal(shape, dtype=np.float32)


def kv_source(workload: Workload, layer: int, n_tokens: int, which: int) -> np.ndarray:
    """Source K (which=T_K) or V (which=T_V) vectors [n_tokens][n_kv][256], N(0,1) fp32."""
    return normal_f32(seed_of(workload.wid, layer, which), (n_tokens, workload.n_kv, HEAD_DIM))


def queries_f32(workload: Workload, layer: int, rows: int) -> np.ndarray:
    """N(0,1) fp32 queries [rows][n_q][256]; callers round them to bf16."""
    return normal_f32(seed_of(workload.wid, layer, T_Q), (rows, workload.n_q, HEAD_DIM))


def log_uniform_f32(seed: int, n: int, lo: float, hi: float) -> np.ndarray:
    """n factors drawn log-uniformly from [lo, hi] (numpy PCG64), fp32: per-position scales of the
    source vectors for pools whose norms span several orders of magnitude."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return np.exp(rng.uniform(np.log(lo), np.log(hi), n)).astype(np.float32)


def bf16_round(x) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even) via torch; returns the values as fp32."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def torch_normal(seed: int, shape, device, dtype=None):
    """N(0,1) fp32 torch tensor from a seeded torch.Generator on `device` (large pools)."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    return torch.randn(shape, generator=gen, device=device, dtype=dtype or torch.float32)

"""Test helpers: build TQ4 pools with the oracle from seeded inputs and copy them
to the GPU, and the parity criterion for attention outputs."""
from __future__ import annotations

import numpy as np

import oracle
import synth

MAX_ABS = 2e-2      # max |gpu - oracle| over an output tensor
REL_L2 = 5e-3       # ||gpu - oracle||_2 / ||oracle||_2


def oracle_pool(workload: synth.Workload, layer: int = 0, heads=None, table=None, fill=None,
                kscale=1.0, vscale=1.0):
    """Encode the workload's cached positions with the oracle (heads: KV heads to fill).  fill: an
    optional numpy Generator that first fills every record with random bits (unwritten records
    then hold arbitrary words and norms, NaN and infinity among them).  kscale / vscale: a factor,
    or one factor per cached position (in used-slot order), applied to the N(0,1) sources."""
    table = synth.placement(workload, layer) if table is None else table
    pool = oracle.Pool.empty(workload.pool_pages, workload.n_kv, workload.page_size)
    if fill is not None:
        for a in (pool.k_words, pool.v_words):
            a[...] = fill.integers(0, 1 << 32, a.shape, dtype=np.uint32)
        for a in (pool.k_norms, pool.v_norms):
            a[...] = fill.integers(0, 1 << 16, a.shape, dtype=np.uint16)
    slots = synth.used_slots(workload, table)
    k = synth.kv_source(workload, layer, len(slots), synth.T_K)
    v = synth.kv_source(workload, layer, len(slots), synth.T_V)
    k *= np.asarray(kscale, np.float32).reshape(-1, 1, 1)
    v *= np.asarray(vscale, np.float32).reshape(-1, 1, 1)
    if heads is not None:
        mask = np.zeros(workload.n_kv, bool)
        mask[list(heads)] = True
        k[:, ~mask] = 0.0
        v[:, ~mask] = 0.0
    oracle.encode_to_pool(pool, k, v, slots)
    return pool, table


def to_device(pool: "oracle.Pool", device="cuda"):
    import torch
    from compressed_kv_attention_kvexec_amd import Tq4LayerPool
    cv = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a).view(dt)).to(device)
    return Tq4LayerPool(cv(pool.k_words, np.int32), cv(pool.v_words, np.int32),
                        cv(pool.k_norms, np.int16), cv(pool.v_norms, np.int16))


def from_device(dpool) -> "oracle.Pool":
    cv = lambda t, dt: t.cpu().numpy().view(dt)
    return oracle.Pool(cv(dpool.k_words, np.uint32), cv(dpool.k_norms, np.uint16),
                       cv(dpool.v_words, np.uint32), cv(dpool.v_norms, np.uint16))


def bf16_queries(workload: synth.Workload, layer: int, rows: int, scale: float = 1.0):
    """Seeded N(0,1) queries rounded to bf16: (torch bf16 CPU tensor, fp64 numpy copy)."""
    import torch
    q = synth.queries_f32(workload, layer, rows) * np.float32(scale)
    qt = torch.from_numpy(q).to(torch.bfloat16)
    return qt, qt.to(torch.float64).numpy()


def parity(gpu_out, ref: np.ndarray, what: str = "", value_scale: float = 1.0):
    """The attention bar: max |gpu - oracle| <= 2e-2 and relative L2 <= 5e-3.  For values drawn
    with a scale s (value_scale) the outputs scale by s, bf16 rounding included, so the absolute
    bound is taken in those units (2e-2 s); the relative bound does not change."""
    got = gpu_out.to(__import__("torch").float64).cpu().numpy() if hasattr(gpu_out, "cpu") else gpu_out
    diff = got - ref
    max_abs = float(np.max(np.abs(diff)))
    rel = float(np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-300))
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert max_abs <= MAX_ABS * value_scale and rel <= REL_L2, f"{what}: max_abs={max_abs:.3e} rel_l2={rel:.3e}"
    return max_abs, rel


def oracle_int8_pool(workload: synth.Workload, layer: int = 0, table=None, fill=None):
    """INT8 records of the workload's cached positions, encoded by the oracle.  fill: an optional
    numpy Generator that first fills every record with random bytes (unwritten records then hold
    arbitrary bits, NaN and infinite scales included)."""
    table = synth.placement(workload, layer) if table is None else table
    pool = oracle.Int8Pool.empty(workload.pool_pages, workload.n_kv, workload.page_size)
    if fill is not None:
        for a in (pool.k_codes, pool.v_codes):
            a[...] = fill.integers(-128, 128, a.shape, dtype=np.int8)
        for a in (pool.k_scales, pool.v_scales):
            a[...] = fill.integers(0, 1 << 16, a.shape, dtype=np.uint16)
    slots = synth.used_slots(workload, table)
    k = synth.kv_source(workload, layer, len(slots), synth.T_K)
    v = synth.kv_source(workload, layer, len(slots), synth.T_V)
    oracle.int8_encode_to_pool(pool, k, v, slots)
    return pool, table


def int8_to_device(pool: "oracle.Int8Pool", device="cuda"):
    import torch
    from compressed_kv_attention_kvexec_amd import Int8LayerPool
    cv = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a).view(dt)).to(device)
    return Int8LayerPool(cv(pool.k_codes, np.int8), cv(pool.v_codes, np.int8),
                         cv(pool.k_scales, np.int16), cv(pool.v_scales, np.int16))

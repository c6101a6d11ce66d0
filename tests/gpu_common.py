"""Shared helpers for the GPU parity tests: run the HIP path and the oracle on the same
seeded workload.

The oracle side builds its pools on the CPU (the bf16/f16 source pool, or the fp8 pool the
oracle's own quantiser produces) and applies the step's KV write with the oracle scatter.
The HIP side uploads the same source pool and applies paged_kv_write on the GPU (for fp8 it
first quantises every slot with paged_kv_write too).  Nothing the HIP path produces is ever an
oracle input.
"""
import functools

import numpy as np
import torch

import oracle
import paged_kv_cache_224_amd as pk
from paged_kv_cache_224_amd import inputs as I

DEV = torch.device("cuda")


def tolerance(cfg) -> float:
    """Max-abs bounds: 2e-3 for fp16 output, 1e-2 for bf16 output, 3e-2 with an fp8 cache."""
    if cfg.kv_dtype == "fp8":
        return 3e-2
    return 2e-3 if cfg.q_dtype == "f16" else 1e-2


def oracle_pools(w):
    """CPU pools after the step's write, as the oracle sees them."""
    if w.cfg.kv_dtype == "fp8":
        kc = oracle.quantize_pool(w.k_pool, w.k_scale)
        vc = oracle.quantize_pool(w.v_pool, w.v_scale)
    else:
        kc, vc = w.k_pool.clone(), w.v_pool.clone()
    oracle.kv_write(w.k_new, w.v_new, kc, vc, w.slot_mapping, w.k_scale, w.v_scale)
    return kc, vc


def gpu_pools(w, write_step=True):
    """GPU pools after the step's write, built by paged_kv_write."""
    cfg = w.cfg
    if cfg.kv_dtype == "fp8":
        NB, BS = w.num_blocks, cfg.block_size
        kc = torch.empty((NB, BS, cfg.Hkv, cfg.D), dtype=torch.uint8, device=DEV)
        vc = torch.empty_like(kc)
        all_slots = torch.arange(NB * BS, dtype=torch.int64, device=DEV)
        ksrc = w.k_pool.to(DEV).view(NB * BS, cfg.Hkv, cfg.D)
        vsrc = w.v_pool.to(DEV).view(NB * BS, cfg.Hkv, cfg.D)
        pk.paged_kv_write(ksrc, vsrc, kc, vc, all_slots, w.k_scale, w.v_scale)
        del ksrc, vsrc
    else:
        kc, vc = w.k_pool.to(DEV), w.v_pool.to(DEV)
    if write_step:
        pk.paged_kv_write(w.k_new.to(DEV), w.v_new.to(DEV), kc, vc,
                          torch.from_numpy(w.slot_mapping).to(DEV), w.k_scale, w.v_scale)
    return kc, vc


def gpu_decode(w, kc, vc, partition_size, max_context_len=None, shared_blocks=None):
    """Decode through the C ABI.  shared_blocks defaults to whether the workload's tables share
    physical blocks (a common prefix)."""
    cfg = w.cfg
    maxlen = int(max_context_len if max_context_len is not None else max(1, int(w.context_lens.max(initial=0))))
    out = torch.full((cfg.B, cfg.Hq, cfg.D), float("nan"), dtype=I.DTYPES[cfg.q_dtype], device=DEV)
    ws = pk.DecodeWorkspace(cfg.B, cfg.Hq, cfg.D, maxlen, partition_size, device=DEV)
    if shared_blocks is None:
        shared_blocks = bool(w.prefix_blocks.size)
    pk.decode(out, w.q.to(DEV), kc, vc, torch.from_numpy(w.block_tables).to(DEV),
              torch.from_numpy(w.context_lens).to(DEV), w.scale, ws, w.k_scale, w.v_scale,
              shared_blocks=shared_blocks)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


def oracle_decode(w, kc, vc):
    kvdt = "fp8" if w.cfg.kv_dtype == "fp8" else None
    return oracle.attn(w.q, kc, vc, w.block_tables, w.context_lens, w.scale, w.k_scale, w.v_scale, kvdt)


@functools.lru_cache(maxsize=8)
def full_case(name):
    """(workload, oracle pools, oracle output) for one full-size workload, cached."""
    w = I.make_workload(I.CONFIGS[name])
    kc, vc = oracle_pools(w)
    ref = oracle_decode(w, kc, vc)
    return w, kc, vc, ref


def max_err(got, ref):
    assert not np.isnan(got).any(), "NaN in output"
    return float(np.max(np.abs(got - ref)))

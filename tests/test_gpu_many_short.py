"""GPU parity of the balanced split on batches of many short sequences, against the fp64 oracle.

The balanced split counts one unit in front of every sequence's first tile (the cost of starting
a segment) besides one unit per tile, and a workgroup's table of sequences holds 64 of them at a
time.  Batches of hundreds of sequences of a few tiles put many sequence starts into every
range, move table refills into the middle of ranges and leave ranges with a single short
sequence; mixed batches put a few long sequences among them.  Each case runs the decode at the
device's balanced width and at small and large explicit widths, plus multi-query, and compares
every output row with the oracle (empty rows must be exactly zero).
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_224_amd as pk
from gpu_common import DEV, gpu_decode, gpu_pools, max_err, tolerance
from paged_kv_cache_224_amd import inputs as I

pytestmark = pytest.mark.gpu

# (name, B, Hkv, G, D, block_size, q dtype, cache dtype, max length, kind)
CASES = [
    ("short300_bf16", 300, 8, 4, 128, 16, "bf16", "bf16", 40, "short"),
    ("short300_fp8", 300, 8, 8, 128, 32, "bf16", "fp8", 64, "short"),
    ("short200_f16_d64", 200, 2, 4, 64, 16, "f16", "f16", 33, "short"),
    ("mixed150_bf16", 150, 8, 4, 128, 16, "bf16", "bf16", 5000, "mixed"),
    ("mixed130_fp8_g16", 130, 1, 16, 128, 64, "bf16", "fp8", 3000, "mixed"),
]


def _lens(kind, B, maxL, rng):
    if kind == "short":
        lens = rng.integers(0, maxL + 1, size=B)
        lens[rng.random(B) < 0.2] = 1                  # one-token sequences: one tile, one row
        lens[rng.random(B) < 0.1] = 0
    else:
        lens = rng.integers(1, 33, size=B)
        lens[rng.choice(B, size=10, replace=False)] = rng.integers(maxL // 2, maxL + 1, size=10)
    return np.clip(lens, 0, maxL).astype(np.int32)


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_many_short_sequences(case):
    name, B, Hkv, G, D, BS, qdt, kvdt, maxL, kind = case
    rng = np.random.default_rng(900 + CASES.index(case))
    cfg = I.Config(name, 700 + CASES.index(case), B=B, Hq=G * Hkv, Hkv=Hkv, D=D, block_size=BS, q_dtype=qdt,
                   kv_dtype=kvdt, lens=("uniform", maxL, maxL), pool=("factor", 1.25), max_len=maxL,
                   partition_size=2 * BS)
    w = I.make_workload(cfg)
    lens = _lens(kind, B, maxL, rng)
    w = dataclasses.replace(w, context_lens=lens)
    kvt = torch.uint8 if kvdt == "fp8" else I.DTYPES[kvdt]
    W = pk.balanced_split(Hkv, D, I.DTYPES[qdt], kvt)
    kv_ref = (oracle.quantize_pool(w.k_pool, w.k_scale), oracle.quantize_pool(w.v_pool, w.v_scale)) \
        if kvdt == "fp8" else (w.k_pool, w.v_pool)
    kvo = "fp8" if kvdt == "fp8" else None
    ref = oracle.attn(w.q, kv_ref[0], kv_ref[1], w.block_tables, lens, w.scale, w.k_scale, w.v_scale, kvo)
    kc, vc = gpu_pools(w, write_step=False)
    for PS in (W, -7, -61, -1000):
        print(f"[many-short] {name} PS={PS}", flush=True)
        got = gpu_decode(w, kc, vc, PS, max_context_len=maxL, shared_blocks=False)
        assert max_err(got, ref) <= tolerance(cfg), PS
        assert np.all(got[lens == 0] == 0), PS
    L = 2 if G * 2 <= 16 else 1
    if L > 1:
        q = I.multi_query_q(cfg, L, seed=3)
        mref = oracle.attn_multi_query(q, kv_ref[0], kv_ref[1], w.block_tables, lens, w.scale, w.k_scale,
                                       w.v_scale, kvo)
        ws = pk.DecodeWorkspace(B, L * cfg.Hq, D, maxL, W, device=DEV)
        out = torch.full((B, L, cfg.Hq, D), float("nan"), dtype=I.DTYPES[qdt], device=DEV)
        pk.multi_query(out, q.to(DEV), kc, vc, torch.from_numpy(w.block_tables).to(DEV),
                       torch.from_numpy(lens).to(DEV), w.scale, ws, w.k_scale, w.v_scale)
        torch.cuda.synchronize()
        assert max_err(out.float().cpu().numpy(), mref) <= tolerance(cfg)

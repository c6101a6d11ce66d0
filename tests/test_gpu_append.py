"""GPU parity of paged_attn_decode_append (the step's KV write and the decode in one call) for
16-bit caches.

The fused call must leave the pools byte for byte as paged_kv_write leaves them, and give the
output of paged_kv_write followed by paged_attn_decode bit for bit (the attention sees the same
row bits, through the same arithmetic), in every schedule; and it must match the fp64 oracle
(write, then attention) within the usual tolerance.  The new-token slots are filled with NaN
beforehand, so a kernel that read the stale pool row instead of the new one would fail.
"""
import dataclasses

import numpy as np
import pytest
import torch

import paged_kv_cache_224_amd as pk
from gpu_common import DEV, max_err, oracle_decode, oracle_pools, tolerance
from paged_kv_cache_224_amd import inputs as I

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


CASES = [("tiny", {}), ("llama3_8b", dict(B=7, len_div=4)), ("long_ctx", dict(B=2, len_div=32)),
         ("shared_prefix", dict(B=9, len_div=4)), ("hkv16_g1", None), ("hkv1_g16_bs64", None)]


def _small(name, **kw):
    if name == "hkv16_g1":          # two KV-head groups per workgroup grid, one query head each
        cfg = dataclasses.replace(I.CONFIGS["llama3_8b"], name=name, seed=71, B=5, Hq=16, Hkv=16,
                                  lens=("uniform", 1, 700), max_len=700)
        return I.make_workload(cfg)
    if name == "hkv1_g16_bs64":     # one KV head for 16 query heads, 64-token blocks
        cfg = dataclasses.replace(I.CONFIGS["tiny"], name=name, seed=72, B=6, Hq=16, Hkv=1, block_size=64,
                                  lens=("uniform", 1, 600), max_len=640, partition_size=128)
        return I.make_workload(cfg)
    return I.make_workload(I.shrink(I.CONFIGS[name], **kw))


def _nan_new_slots(kc, vc, w):
    """Stale NaN in the slots the step writes (in a real pool they hold an old token's bytes)."""
    BS = w.cfg.block_size
    for s in w.slot_mapping.tolist():
        if s >= 0:
            kc[s // BS, s % BS] = float("nan")
            vc[s // BS, s % BS] = float("nan")


def _schedules(w):
    cfg = w.cfg
    W = pk.balanced_split(cfg.Hkv, cfg.D, I.DTYPES[cfg.q_dtype], I.DTYPES[cfg.kv_dtype])
    return [W, -3, 0, cfg.partition_size]


def _run_pair(w, PS):
    """(fused out, fused pools, two-call out, two-call pools) on the same inputs."""
    cfg = w.cfg
    shared = bool(w.prefix_blocks.size)
    maxlen = max(1, int(w.context_lens.max()))
    q = w.q.to(DEV)
    kn, vn = w.k_new.to(DEV), w.v_new.to(DEV)
    bt = torch.from_numpy(w.block_tables).to(DEV)
    lens = torch.from_numpy(w.context_lens).to(DEV)
    res = []
    for fused in (True, False):
        kc, vc = w.k_pool.to(DEV), w.v_pool.to(DEV)
        _nan_new_slots(kc, vc, w)
        ws = pk.DecodeWorkspace(cfg.B, cfg.Hq, cfg.D, maxlen, PS, device=DEV)
        out = torch.full((cfg.B, cfg.Hq, cfg.D), float("nan"), dtype=I.DTYPES[cfg.q_dtype], device=DEV)
        if fused:
            pk.decode_append(out, q, kn, vn, kc, vc, bt, lens, w.scale, ws, shared_blocks=shared)
        else:
            pk.paged_kv_write(kn, vn, kc, vc, torch.from_numpy(w.slot_mapping).to(DEV))
            pk.decode(out, q, kc, vc, bt, lens, w.scale, ws, shared_blocks=shared)
        torch.cuda.synchronize()
        res += [out.cpu(), kc.cpu(), vc.cpu()]
    return res


def _same_bytes(a, b):
    return torch.equal(a.contiguous().view(torch.uint8).flatten(), b.contiguous().view(torch.uint8).flatten())


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_append_equals_write_then_decode(case):
    name, kw = case
    w = _small(name, **(kw or {}))
    kc_ref, vc_ref = oracle_pools(w)
    ref = oracle_decode(w, kc_ref, vc_ref)
    for PS in _schedules(w):
        _say(f"[append] {name} {kw} partition_size={PS}")
        fo, fk, fv, to, tk, tv = _run_pair(w, PS)
        assert _same_bytes(fk, tk) and _same_bytes(fv, tv), "pools differ from paged_kv_write's"
        assert _same_bytes(fk, kc_ref) and _same_bytes(fv, vc_ref), "pools differ from the oracle's write"
        assert torch.equal(fo, to), "fused output differs from write + decode"
        assert max_err(fo.float().numpy(), ref) <= tolerance(w.cfg)


def test_append_full_llama_workload():
    w = I.make_workload(I.CONFIGS["llama3_8b"])
    _say("[append] llama3_8b full size, balanced")
    W = pk.balanced_split(8, 128, torch.bfloat16, torch.bfloat16)
    fo, fk, fv, to, tk, tv = _run_pair(w, W)
    assert _same_bytes(fk, tk) and _same_bytes(fv, tv)
    assert torch.equal(fo, to)


def test_append_empty_rows_store_nothing():
    """Rows with n = 0 have no new token: a zero output row and no store."""
    w = _small("llama3_8b", B=6, len_div=8)
    lens = w.context_lens.copy()
    lens[[0, 3]] = 0
    sm = w.slot_mapping.copy()
    sm[[0, 3]] = -1
    w = dataclasses.replace(w, context_lens=lens, slot_mapping=sm)
    for PS in _schedules(w):
        _say(f"[append] empty rows, partition_size={PS}")
        fo, fk, fv, to, tk, tv = _run_pair(w, PS)
        assert _same_bytes(fk, tk) and _same_bytes(fv, tv)
        assert torch.equal(fo, to)
        assert torch.all(fo[[0, 3]] == 0)

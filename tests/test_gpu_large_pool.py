"""GPU parity with pools larger than 4 GiB.

A pool of MI355X size holds far more than 2**32 bytes, so every pool address must be formed in
64 bits.  Here a small seeded workload is moved into a pool of 140,000 blocks of 32 KiB
(4.27 GiB per pool): its compact block i goes to a distinct big id, half of them past the
4 GiB mark and half below.  Block tables and slots are renamed the same way, so the expected
values are the oracle's on the compact pool.  Covered: the write, the decode in all three
schedules, multi-query, the shared-prefix decode, the fused append and whole-block copies.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_224_amd as pk
from gpu_common import DEV, max_err, oracle_decode, oracle_pools, tolerance
from paged_kv_cache_224_amd import inputs as I

pytestmark = pytest.mark.gpu

NB_BIG = 140_000
FOUR_GIB = 2 ** 32


def _say(msg):
    print(msg, flush=True)


def _block_bytes(cfg):
    return cfg.block_size * cfg.Hkv * cfg.D * (1 if cfg.kv_dtype == "fp8" else 2)


def _big_ids(cfg, nb_small, seed):
    """Distinct big ids for the compact blocks: even blocks past 4 GiB, odd blocks below."""
    first_high = -(-FOUR_GIB // _block_bytes(cfg))
    assert first_high + nb_small <= NB_BIG and nb_small <= first_high
    rng = np.random.default_rng(seed)
    high = rng.choice(np.arange(first_high, NB_BIG), size=nb_small, replace=False)
    low = rng.choice(np.arange(0, first_high), size=nb_small, replace=False)
    ids = np.where(np.arange(nb_small) % 2 == 0, high, low).astype(np.int64)
    assert (ids * _block_bytes(cfg) >= FOUR_GIB).sum() >= nb_small // 2
    return ids


def _relabel(w, ids):
    """The workload's tables and slots with compact block ids replaced by big ones."""
    BS = w.cfg.block_size
    bt = ids[w.block_tables].astype(np.int32)
    sm = w.slot_mapping
    big_sm = np.where(sm >= 0, ids[np.maximum(sm, 0) // BS] * BS + np.maximum(sm, 0) % BS, -1).astype(np.int64)
    return bt, big_sm


def _big_pools(w, ids):
    """Device pools of NB_BIG blocks holding the compact pools' blocks at `ids` (fp8 pools are
    quantised by paged_kv_write first); the other blocks are zero."""
    cfg = w.cfg
    NB, BS = w.num_blocks, cfg.block_size
    if cfg.kv_dtype == "fp8":
        kq = torch.empty((NB, BS, cfg.Hkv, cfg.D), dtype=torch.uint8, device=DEV)
        vq = torch.empty_like(kq)
        pk.paged_kv_write(w.k_pool.to(DEV).view(NB * BS, cfg.Hkv, cfg.D), w.v_pool.to(DEV).view(NB * BS, cfg.Hkv, cfg.D),
                          kq, vq, torch.arange(NB * BS, dtype=torch.int64, device=DEV), w.k_scale, w.v_scale)
        dt = torch.uint8
    else:
        kq, vq = w.k_pool.to(DEV), w.v_pool.to(DEV)
        dt = I.DTYPES[cfg.kv_dtype]
    kb = torch.zeros((NB_BIG, BS, cfg.Hkv, cfg.D), dtype=dt, device=DEV)
    vb = torch.zeros_like(kb)
    idx = torch.from_numpy(ids).to(DEV)
    kb[idx] = kq
    vb[idx] = vq
    torch.cuda.synchronize()
    return kb, vb


def _bytes(t):
    return t.contiguous().view(torch.uint8).cpu()


def _check_written_rows(w, kb, vb, kc_ref, vc_ref, ids):
    BS = w.cfg.block_size
    for s in w.slot_mapping.tolist():
        if s < 0:
            continue
        blk, off = s // BS, s % BS
        big = int(ids[blk])
        assert torch.equal(_bytes(kb[big, off]), kc_ref[blk, off].contiguous().view(torch.uint8)), (blk, big)
        assert torch.equal(_bytes(vb[big, off]), vc_ref[blk, off].contiguous().view(torch.uint8)), (blk, big)


CASES = [("llama3_8b", dict(B=8, len_div=4)), ("llama3_70b_fp8", dict(B=6, len_div=8))]


@pytest.mark.parametrize("name,kw", CASES, ids=[c[0] for c in CASES])
def test_write_and_decode_past_4gib(name, kw):
    w = I.make_workload(I.shrink(I.CONFIGS[name], **kw))
    cfg = w.cfg
    ids = _big_ids(cfg, w.num_blocks, seed=5)
    bt, big_sm = _relabel(w, ids)
    kc_ref, vc_ref = oracle_pools(w)
    ref = oracle_decode(w, kc_ref, vc_ref)
    _say(f"[large pool] {name}: {NB_BIG} blocks of {_block_bytes(cfg)} B per pool, {w.num_blocks} used")
    kb, vb = _big_pools(w, ids)
    pk.paged_kv_write(w.k_new.to(DEV), w.v_new.to(DEV), kb, vb, torch.from_numpy(big_sm).to(DEV),
                      w.k_scale, w.v_scale)
    torch.cuda.synchronize()
    _check_written_rows(w, kb, vb, kc_ref, vc_ref, ids)
    kvt = torch.uint8 if cfg.kv_dtype == "fp8" else I.DTYPES[cfg.kv_dtype]
    maxlen = max(1, int(w.context_lens.max()))
    q = w.q.to(DEV)
    btd = torch.from_numpy(bt).to(DEV)
    lens = torch.from_numpy(w.context_lens).to(DEV)
    for PS in (0, cfg.partition_size, pk.balanced_split(cfg.Hkv, cfg.D, I.DTYPES[cfg.q_dtype], kvt)):
        _say(f"  decode partition_size={PS}")
        out = torch.full((cfg.B, cfg.Hq, cfg.D), float("nan"), dtype=I.DTYPES[cfg.q_dtype], device=DEV)
        ws = pk.DecodeWorkspace(cfg.B, cfg.Hq, cfg.D, maxlen, PS, device=DEV)
        pk.decode(out, q, kb, vb, btd, lens, w.scale, ws, w.k_scale, w.v_scale)
        torch.cuda.synchronize()
        assert max_err(out.float().cpu().numpy(), ref) <= tolerance(cfg), PS
    # multi-query over the same big pools
    L = 2
    qm = I.multi_query_q(cfg, L, seed=3)
    kvdt = "fp8" if cfg.kv_dtype == "fp8" else None
    mref = oracle.attn_multi_query(qm, kc_ref, vc_ref, w.block_tables, w.context_lens, w.scale, w.k_scale,
                                   w.v_scale, kvdt)
    PS = pk.balanced_split(cfg.Hkv, cfg.D, I.DTYPES[cfg.q_dtype], kvt)
    ws = pk.DecodeWorkspace(cfg.B, L * cfg.Hq, cfg.D, maxlen, PS, device=DEV)
    out = torch.full((cfg.B, L, cfg.Hq, cfg.D), float("nan"), dtype=I.DTYPES[cfg.q_dtype], device=DEV)
    _say("  multi-query L=2")
    pk.multi_query(out, qm.to(DEV), kb, vb, btd, lens, w.scale, ws, w.k_scale, w.v_scale)
    torch.cuda.synchronize()
    assert max_err(out.float().cpu().numpy(), mref) <= tolerance(cfg)
    del kb, vb
    torch.cuda.empty_cache()


def test_shared_prefix_decode_past_4gib():
    cfg = dataclasses.replace(I.CONFIGS["shared_prefix"], name="sp_big", B=24, lens=("prefix", 256, 1, 120),
                              max_len=256 + 120, pool=("factor", 1.25), seed=91)
    w = I.make_workload(cfg)
    P = int(w.prefix_blocks.size) * cfg.block_size
    ids = _big_ids(cfg, w.num_blocks, seed=6)
    bt, _ = _relabel(w, ids)
    kc_ref, vc_ref = oracle_pools(w)
    ref = oracle_decode(w, kc_ref, vc_ref)
    kb, vb = _big_pools(w, ids)
    pk.paged_kv_write(w.k_new.to(DEV), w.v_new.to(DEV), kb, vb, torch.from_numpy(_relabel(w, ids)[1]).to(DEV))
    PS = pk.balanced_split(cfg.Hkv, cfg.D, torch.bfloat16, torch.bfloat16)
    ws = pk.SharedPrefixWorkspace(cfg.B, cfg.Hq, cfg.Hkv, cfg.D, cfg.max_len, P, PS, 64, device=DEV)
    out = torch.full((cfg.B, cfg.Hq, cfg.D), float("nan"), dtype=torch.bfloat16, device=DEV)
    _say(f"[large pool] shared prefix of {P} tokens, prefix blocks at big ids {ids[w.prefix_blocks].tolist()}")
    pk.decode_shared_prefix(out, w.q.to(DEV), kb, vb, torch.from_numpy(bt).to(DEV),
                            torch.from_numpy(w.context_lens).to(DEV), w.scale, ws)
    torch.cuda.synchronize()
    assert max_err(out.float().cpu().numpy(), ref) <= tolerance(cfg)
    del kb, vb
    torch.cuda.empty_cache()


def test_append_past_4gib():
    w = I.make_workload(I.shrink(I.CONFIGS["llama3_8b"], B=6, len_div=8, seed=92))
    cfg = w.cfg
    ids = _big_ids(cfg, w.num_blocks, seed=7)
    bt, _ = _relabel(w, ids)
    kc_ref, vc_ref = oracle_pools(w)
    ref = oracle_decode(w, kc_ref, vc_ref)
    kb, vb = _big_pools(w, ids)
    maxlen = max(1, int(w.context_lens.max()))
    _say("[large pool] decode_append, balanced and single pass")
    for PS in (pk.balanced_split(cfg.Hkv, cfg.D, torch.bfloat16, torch.bfloat16), 0):
        ws = pk.DecodeWorkspace(cfg.B, cfg.Hq, cfg.D, maxlen, PS, device=DEV)
        out = torch.full((cfg.B, cfg.Hq, cfg.D), float("nan"), dtype=torch.bfloat16, device=DEV)
        pk.decode_append(out, w.q.to(DEV), w.k_new.to(DEV), w.v_new.to(DEV), kb, vb, torch.from_numpy(bt).to(DEV),
                         torch.from_numpy(w.context_lens).to(DEV), w.scale, ws)
        torch.cuda.synchronize()
        _check_written_rows(w, kb, vb, kc_ref, vc_ref, ids)
        assert max_err(out.float().cpu().numpy(), ref) <= tolerance(cfg), PS
    del kb, vb
    torch.cuda.empty_cache()


def test_copy_blocks_across_4gib():
    cfg = I.CONFIGS["llama3_8b"]
    bb = _block_bytes(cfg)
    first_high = -(-FOUR_GIB // bb)
    kb = torch.zeros((NB_BIG, cfg.block_size, cfg.Hkv, cfg.D), dtype=torch.bfloat16, device=DEV)
    vb = torch.zeros_like(kb)
    rng = np.random.default_rng(8)
    high = rng.choice(np.arange(first_high, NB_BIG), 32, replace=False)      # past 4 GiB
    src = np.concatenate([high[:16], rng.choice(np.arange(0, first_high // 2), 16, replace=False)]).astype(np.int32)
    dst = np.concatenate([rng.choice(np.arange(first_high // 2, first_high), 16, replace=False),
                          high[16:]]).astype(np.int32)            # high -> low and low -> high
    assert not set(src.tolist()) & set(dst.tolist())
    g = torch.Generator().manual_seed(9)
    vals_k = torch.randn((src.size, cfg.block_size, cfg.Hkv, cfg.D), generator=g).to(torch.bfloat16)
    vals_v = torch.randn((src.size, cfg.block_size, cfg.Hkv, cfg.D), generator=g).to(torch.bfloat16)
    kb[torch.from_numpy(src).long().to(DEV)] = vals_k.to(DEV)
    vb[torch.from_numpy(src).long().to(DEV)] = vals_v.to(DEV)
    _say("[large pool] copy_blocks between ids below and above 4 GiB")
    pk.paged_kv_copy_blocks(kb, vb, torch.from_numpy(src).to(DEV), torch.from_numpy(dst).to(DEV))
    torch.cuda.synchronize()
    d = torch.from_numpy(dst).long().to(DEV)
    assert torch.equal(_bytes(kb[d]), vals_k.view(torch.uint8))
    assert torch.equal(_bytes(vb[d]), vals_v.view(torch.uint8))
    del kb, vb
    torch.cuda.empty_cache()


def test_swap_blocks_past_4gib():
    """Swap out device blocks that lie past 4 GiB to a small pinned host pool, then swap them
    back into other device blocks, half of them past 4 GiB."""
    cfg = I.CONFIGS["llama3_8b"]
    first_high = -(-FOUR_GIB // _block_bytes(cfg))
    kb = torch.zeros((NB_BIG, cfg.block_size, cfg.Hkv, cfg.D), dtype=torch.bfloat16, device=DEV)
    vb = torch.zeros_like(kb)
    rng = np.random.default_rng(10)
    high = rng.choice(np.arange(first_high, NB_BIG), 24, replace=False)
    out_ids = high[:16].astype(np.int32)
    in_ids = np.concatenate([high[16:], rng.choice(np.arange(0, first_high), 8, replace=False)]).astype(np.int32)
    host_ids = rng.permutation(32)[:16].astype(np.int32)
    g = torch.Generator().manual_seed(11)
    vals_k = torch.randn((16, cfg.block_size, cfg.Hkv, cfg.D), generator=g).to(torch.bfloat16)
    vals_v = torch.randn((16, cfg.block_size, cfg.Hkv, cfg.D), generator=g).to(torch.bfloat16)
    kb[torch.from_numpy(out_ids).long().to(DEV)] = vals_k.to(DEV)
    vb[torch.from_numpy(out_ids).long().to(DEV)] = vals_v.to(DEV)
    hk = torch.zeros((32, cfg.block_size, cfg.Hkv, cfg.D), dtype=torch.bfloat16, pin_memory=True)
    hv = torch.zeros_like(hk, pin_memory=True)
    _say("[large pool] swap out from ids past 4 GiB, swap in to ids on both sides")
    hids = torch.from_numpy(host_ids).to(DEV)
    pk.paged_kv_swap_blocks(kb, vb, hk, hv, torch.from_numpy(out_ids).to(DEV), hids, to_host=True)
    torch.cuda.synchronize()
    hsel = torch.from_numpy(host_ids).long()
    assert torch.equal(hk[hsel].view(torch.uint8), vals_k.view(torch.uint8))
    assert torch.equal(hv[hsel].view(torch.uint8), vals_v.view(torch.uint8))
    pk.paged_kv_swap_blocks(kb, vb, hk, hv, torch.from_numpy(in_ids).to(DEV), hids, to_host=False)
    torch.cuda.synchronize()
    d = torch.from_numpy(in_ids).long().to(DEV)
    assert torch.equal(_bytes(kb[d]), vals_k.view(torch.uint8))
    assert torch.equal(_bytes(vb[d]), vals_v.view(torch.uint8))
    del kb, vb
    torch.cuda.empty_cache()

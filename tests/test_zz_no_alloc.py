"""paged_attn_decode_noalloc: the decode + merge whose split-K partials live in the library's
fixed device scratch.  Through the C ABI it must give the same output bits as the existing pair
paged_attn_decode + paged_attn_reduce (with a caller workspace), and stay within the oracle's
tolerance, on two calls in a row, the second with a smaller batch (the scratch keeps the first
call's partials, which the second must never read).
"""
import dataclasses

import numpy as np
import pytest
import torch

import paged_kv_cache_224_amd as pk
from gpu_common import DEV, full_case, gpu_decode, gpu_pools, max_err, oracle_decode, oracle_pools, tolerance
from paged_kv_cache_224_amd import inputs as I

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _noalloc(w, kc, vc, PS, maxlen):
    cfg = w.cfg
    out = torch.full((cfg.B, cfg.Hq, cfg.D), float("nan"), dtype=I.DTYPES[cfg.q_dtype], device=DEV)
    pk.paged_attn_decode_noalloc(out, w.q.to(DEV), kc, vc, torch.from_numpy(w.block_tables).to(DEV),
                                 torch.from_numpy(w.context_lens).to(DEV), w.scale, maxlen, PS, w.k_scale,
                                 w.v_scale)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


def _balanced(cfg):
    return pk.balanced_split(cfg.Hkv, cfg.D, I.DTYPES[cfg.q_dtype],
                             torch.uint8 if cfg.kv_dtype == "fp8" else I.DTYPES[cfg.kv_dtype])


@pytest.mark.parametrize("big,small", [("llama3_8b", ("llama3_8b", 16, 4)),
                                       ("llama3_70b_fp8", ("llama3_70b_fp8", 24, 8))])
def test_noalloc_matches_decode_and_reduce_on_two_calls(big, small):
    """First call: the full workload; second call: a smaller batch with shorter contexts."""
    w1, _, _, ref1 = full_case(big)
    name, B2, div = small
    w2 = I.make_workload(I.shrink(I.CONFIGS[name], B=B2, len_div=div, seed=I.CONFIGS[name].seed + 100))
    kc2_ref, vc2_ref = oracle_pools(w2)
    ref2 = oracle_decode(w2, kc2_ref, vc2_ref)
    for w, ref in ((w1, ref1), (w2, ref2)):
        cfg = w.cfg
        PS = _balanced(cfg)
        _say(f"[noalloc] {cfg.name} B={cfg.B} PS={PS}")
        kc, vc = gpu_pools(w)
        got = _noalloc(w, kc, vc, PS, cfg.max_len)
        want = gpu_decode(w, kc, vc, PS, max_context_len=cfg.max_len)
        assert np.array_equal(got, want), "noalloc differs from paged_attn_decode + paged_attn_reduce"
        err = max_err(got, ref)
        _say(f"    bit-equal to decode + reduce; max-abs err vs oracle {err:.3e}")
        assert err <= tolerance(cfg)
        del kc, vc


def test_noalloc_single_pass_and_empty_rows():
    """partition_size 0 (no scratch) equals the single-pass decode; rows of length 0 are zeros in
    both schedules, and a balanced call after it with other lengths is unaffected."""
    cfg = I.shrink(I.CONFIGS["tiny"], B=6, name="noalloc_tiny")
    w = I.make_workload(cfg)
    lens = w.context_lens.copy()
    lens[[1, 4]] = 0
    w = dataclasses.replace(w, context_lens=lens)
    kc_ref, vc_ref = oracle_pools(w)
    ref = oracle_decode(w, kc_ref, vc_ref)
    kc, vc = gpu_pools(w)
    for PS in (0, _balanced(cfg), -3):
        got = _noalloc(w, kc, vc, PS, cfg.max_len)
        want = gpu_decode(w, kc, vc, PS, max_context_len=cfg.max_len)
        assert np.array_equal(got, want)
        assert np.all(got[[1, 4]] == 0)
        assert max_err(got, ref) <= tolerance(cfg)


def test_noalloc_rejects_calls_beyond_the_scratch():
    """A balanced call whose partials would exceed the 32 MiB buffer fails before any launch."""
    cfg = I.CONFIGS["llama3_8b"]
    B, Hq, D = 4096, 32, 128
    q = torch.zeros((B, Hq, D), dtype=torch.bfloat16, device=DEV)
    out = torch.zeros_like(q)
    kc = torch.zeros((16, 16, 8, D), dtype=torch.bfloat16, device=DEV)
    bt = torch.zeros((B, 8), dtype=torch.int32, device=DEV)
    lens = torch.zeros((B,), dtype=torch.int32, device=DEV)
    with pytest.raises(pk.PagedKVError) as e:
        pk.paged_attn_decode_noalloc(out, q, kc, kc, bt, lens, 0.1, 128, -256)
    assert e.value.status == -12
    assert cfg.Hkv == 8


@pytest.mark.parametrize("seed", range(20))
def test_noalloc_random_draws(seed):
    """Random shapes, dtype pairs, lengths and widths (the draws of the randomized decode tests):
    bit-equal to decode + reduce with a caller workspace, and within the oracle's tolerance."""
    import oracle
    from test_gpu_random import _draw, _oracle_pools
    cfg, lens, share, _, W, _ = _draw(900 + seed)
    w = I.make_workload(cfg)
    bt = w.block_tables.copy()
    if share:
        bt[1:, :share] = bt[0, :share]
    w = dataclasses.replace(w, context_lens=lens, block_tables=bt)
    kvt = torch.uint8 if cfg.kv_dtype == "fp8" else I.DTYPES[cfg.kv_dtype]
    PS = pk.balanced_split(cfg.Hkv, cfg.D, I.DTYPES[cfg.q_dtype], kvt) if seed % 2 else -W
    _say(f"[noalloc random {seed}] Hq={cfg.Hq} Hkv={cfg.Hkv} D={cfg.D} BS={cfg.block_size} "
         f"{cfg.q_dtype}/{cfg.kv_dtype} B={cfg.B} max={cfg.max_len} PS={PS}")
    kc_ref, vc_ref = _oracle_pools(w)
    kvdt = "fp8" if cfg.kv_dtype == "fp8" else None
    ref = oracle.attn(w.q, kc_ref, vc_ref, bt, lens, w.scale, w.k_scale, w.v_scale, kvdt)
    kc, vc = gpu_pools(w, write_step=False)
    got = _noalloc(w, kc, vc, PS, cfg.max_len)
    want = gpu_decode(w, kc, vc, PS, max_context_len=cfg.max_len, shared_blocks=bool(share))
    assert np.array_equal(got, want)
    assert max_err(got, ref) <= tolerance(cfg)

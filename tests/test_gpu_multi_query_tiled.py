"""GPU parity of paged_attn_multi_query past one MFMA tile of (head, new token) columns
(G * L > 16: chunked prefill, long draft verification) against the fp64 oracle: up to 32 columns
the decode wave carries two tiles, beyond that the tiled kernel runs.  All three schedules, the Llama-3-8B (G = 4, bf16) and Llama-3-70B (G = 8, fp8
cache) shapes at L = 8, 16 and 64, contexts shorter than L, odd L, G = 1 and G = 16, and
sampled rows of the full-size batches in the configuration the benchmark times."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_224_amd as pk
from gpu_common import DEV, full_case, gpu_pools, max_err, oracle_pools, tolerance
from paged_kv_cache_224_amd import inputs as I

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _kvdt(cfg):
    return torch.uint8 if cfg.kv_dtype == "fp8" else I.DTYPES[cfg.kv_dtype]


def _mq_split(cfg, L):
    return pk.multi_query_split(cfg.Hq, cfg.Hkv, cfg.D, L, I.DTYPES[cfg.q_dtype], _kvdt(cfg))


def _run(w, q, PS, maxlen, kc=None, vc=None):
    B, L, Hq, D = q.shape
    if kc is None:
        kc, vc = gpu_pools(w)
    out = torch.full((B, L, Hq, D), float("nan"), dtype=q.dtype, device=DEV)
    ws = pk.DecodeWorkspace(B, L * Hq, D, maxlen, PS, device=DEV)
    pk.multi_query(out, q.to(DEV), kc, vc, torch.from_numpy(w.block_tables).to(DEV),
                   torch.from_numpy(w.context_lens).to(DEV), w.scale, ws, w.k_scale, w.v_scale)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


def _oracle(w, q, kc_ref, vc_ref, rows=None):
    kvdt = "fp8" if w.cfg.kv_dtype == "fp8" else None
    bt, lens = w.block_tables, w.context_lens
    if rows is not None:
        q, bt, lens = q[rows].contiguous(), bt[rows], lens[rows]
    return oracle.attn_multi_query(q, kc_ref, vc_ref, bt, lens, w.scale, w.k_scale, w.v_scale, kvdt)


CASES = [("llama3_8b", dict(B=6, len_div=8), 8), ("llama3_8b", dict(B=5, len_div=8), 16),
         ("llama3_8b", dict(B=3, len_div=8), 64), ("llama3_70b_fp8", dict(B=6, len_div=8), 8),
         ("llama3_70b_fp8", dict(B=4, len_div=8), 16), ("llama3_70b_fp8", dict(B=3, len_div=16), 64),
         ("tiny", {}, 8), ("long_ctx", dict(B=2, len_div=64), 16)]


@pytest.mark.parametrize("name,kw,L", CASES, ids=lambda x: str(x) if not isinstance(x, dict) else "")
def test_tiled_multi_query_parity(name, kw, L):
    w = I.make_workload(I.shrink(I.CONFIGS[name], **kw))
    cfg = w.cfg
    q = I.multi_query_q(cfg, L, seed=L + 1)
    kc_ref, vc_ref = oracle_pools(w)
    ref = _oracle(w, q, kc_ref, vc_ref)
    maxlen = int(w.context_lens.max())
    kc, vc = gpu_pools(w)
    for PS in (0, cfg.partition_size, -37, _mq_split(cfg, L),
               pk.balanced_split(cfg.Hkv, cfg.D, I.DTYPES[cfg.q_dtype], _kvdt(cfg))):
        _say(f"[mq-tiled] {name} L={L} PS={PS}")
        got = _run(w, q, PS, maxlen, kc, vc)
        err = max_err(got, ref)
        _say(f"    max-abs err {err:.3e}")
        assert err <= tolerance(cfg), (PS, err)


@pytest.mark.parametrize("Hq,Hkv,L", [(8, 2, 24), (4, 4, 32), (32, 2, 2), (16, 2, 17)])
def test_tiled_multi_query_short_contexts(Hq, Hkv, L):
    """Contexts of 0..L+2 tokens and longer ones: new token i of a sequence with n < L - i
    visible tokens gets a zero row; odd L and group sizes 1 and 16 split columns unevenly over
    the waves and column blocks."""
    cfg = I.Config("mqt", 41, B=8, Hq=Hq, Hkv=Hkv, D=128, block_size=32, q_dtype="bf16", kv_dtype="bf16",
                   lens=("uniform", 1, 1), pool=("factor", 1.25), max_len=700, partition_size=64)
    lens = [0, 1, 3, L - 1, L, L + 2, 300, 700]
    w = I.permute_blocks(I.dense_workload(cfg, lens, seed=6), seed=7)
    q = I.multi_query_q(cfg, L, seed=8)
    kc_ref, vc_ref = oracle_pools(w)
    ref = _oracle(w, q, kc_ref, vc_ref)
    kc, vc = gpu_pools(w)
    for PS in (0, 64, -3, -300):
        _say(f"[mq-tiled short] Hq={Hq} Hkv={Hkv} L={L} PS={PS}")
        got = _run(w, q, PS, 700, kc, vc)
        assert max_err(got, ref) <= 1e-2, PS
        assert np.all(got[0] == 0)
        for b, n in enumerate(lens):
            hidden = max(0, L - n)             # new tokens 0 .. L - n - 1 see nothing
            assert np.all(got[b, :hidden] == 0), (b, n)


@pytest.mark.parametrize("name,L", [("llama3_8b", 16), ("llama3_8b", 64), ("llama3_70b_fp8", 8)])
def test_tiled_multi_query_full_batch_sampled(name, L):
    """The full-size batch in the configuration bench.py --op multi_query times (balanced split
    of paged_attn_multi_query_split); every output of four sampled sequences (the shortest,
    the longest and two others) against the oracle, and no NaN anywhere."""
    w, kc_ref, vc_ref, _ = full_case(name)
    cfg = w.cfg
    q = I.multi_query_q(cfg, L, seed=0)
    rows = sorted({int(np.argmin(w.context_lens)), int(np.argmax(w.context_lens)), 1, cfg.B // 2})
    ref = _oracle(w, q, kc_ref, vc_ref, rows)
    PS = _mq_split(cfg, L)
    _say(f"[mq-tiled full] {name} L={L} PS={PS} rows={rows}")
    got = _run(w, q, PS, cfg.max_len)
    assert not np.isnan(got).any()
    err = max_err(got[rows], ref)
    _say(f"    max-abs err {err:.3e}")
    assert err <= tolerance(cfg)


def test_tiled_multi_query_is_deterministic_and_block_order_free():
    """Two runs, and a run over physically permuted blocks, give the same bits."""
    w = I.make_workload(I.shrink(I.CONFIGS["llama3_8b"], B=5, len_div=8))
    q = I.multi_query_q(w.cfg, 16, seed=3)
    PS = _mq_split(w.cfg, 16)
    a = _run(w, q, PS, w.cfg.max_len)
    b = _run(w, q, PS, w.cfg.max_len)
    c = _run(I.permute_blocks(w, seed=11), q, PS, w.cfg.max_len)
    assert np.array_equal(a, b) and np.array_equal(a, c)
    assert dataclasses.is_dataclass(w)


def test_many_rows_merge_straddling_sequences():
    """800 sequences x 7 new tokens x 3 query heads = 16800 output rows, 21 per sequence: the
    merge serves four rows per wave, and a wave's rows often straddle two sequences, whose
    balanced-split partial counts differ (G * L = 21: the two-tile decode writes the partials)."""
    cfg = I.Config("mq_rows", 51, B=800, Hq=3, Hkv=1, D=128, block_size=16, q_dtype="bf16", kv_dtype="bf16",
                   lens=("uniform", 1, 200), pool=("factor", 1.25), max_len=200, partition_size=64)
    w = I.make_workload(cfg)
    L = 7
    q = I.multi_query_q(cfg, L, seed=12)
    kc_ref, vc_ref = oracle_pools(w)
    ref = _oracle(w, q, kc_ref, vc_ref)
    kc, vc = gpu_pools(w)
    for PS in (_mq_split(cfg, L), -37, 64):
        _say(f"[mq many rows] PS={PS}")
        got = _run(w, q, PS, cfg.max_len, kc, vc)
        assert max_err(got, ref) <= tolerance(cfg), PS


@pytest.mark.parametrize("L", [1024, 4096])
def test_prefill_chunk_lengths(L):
    """q_len up to the 4096 the header allows (a prefill chunk): 4096 (head, new token) columns per
    KV group, i.e. 32 column blocks.  Contexts longer than L, a few tokens shorter (its first new
    tokens see nothing: zero rows) and much shorter, in the balanced, fixed and single-pass
    schedules."""
    cfg = I.Config("mq_chunk", 61, B=3, Hq=4, Hkv=1, D=128, block_size=16, q_dtype="bf16", kv_dtype="bf16",
                   lens=("uniform", 1, 1), pool=("factor", 1.25), max_len=L + 100, partition_size=512)
    lens = [L + 100, L - 7, 300]
    w = I.permute_blocks(I.dense_workload(cfg, lens, seed=62), seed=63)
    q = I.multi_query_q(cfg, L, seed=64)
    kc_ref, vc_ref = oracle_pools(w)
    ref = _oracle(w, q, kc_ref, vc_ref)
    kc, vc = gpu_pools(w)
    for PS in (_mq_split(cfg, L), 512, 0):
        _say(f"[mq-tiled chunk] L={L} PS={PS}")
        got = _run(w, q, PS, cfg.max_len, kc, vc)
        assert max_err(got, ref) <= tolerance(cfg), PS
        for b, n in enumerate(lens):
            assert np.all(got[b, :max(0, L - n)] == 0), (b, n)

"""Pins for the fp64 oracle: each check ties it to something other than itself.

* Dense attention by library routines (numpy einsum/softmax, torch SDPA in fp64) on tables
  that are the identity map, so the gather must reproduce plain attention.
* Invariances the pages fix: a block table is pure indirection, so permuting physical blocks
  changes nothing, and copy-on-write sharing of prefix blocks gives the same result as
  private copies ("vllm-project-vllm -- L2", section 3 Q2, section 9, section 11 step 5).
* Closed forms (one token, zero query, constant values, two tokens, needles, partition
  indicators) and a scalar brute force on tiny inputs.
* Stale data in unused table entries and tail slots is never read.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from brute import brute_attn
from paged_kv_cache_224_amd import inputs as I

SMALL_SHAPES = {
    # name: (cfg, lens) with identity tables
    "tiny_f16": (I.CONFIGS["tiny"], [1, 17, 100, 256]),
    "gqa4_bf16": (I.shrink(I.CONFIGS["llama3_8b"], len_div=16), [32, 1, 255, 100, 77]),
    "gqa8_bs32_fp8": (I.shrink(I.CONFIGS["llama3_70b_fp8"], len_div=64), [16, 31, 64, 511, 3]),
}


def _pool_as_fp8(w):
    kq = oracle.quantize_pool(w.k_pool, w.k_scale)
    vq = oracle.quantize_pool(w.v_pool, w.v_scale)
    return kq, vq


def _cache_values(w):
    """(k_cache, v_cache, kv_dtype, fp64 K values, fp64 V values) as the oracle reads them."""
    if w.cfg.kv_dtype == "fp8":
        kc, vc = _pool_as_fp8(w)
        kval = oracle.fp8_decode(kc.numpy()) * w.k_scale
        vval = oracle.fp8_decode(vc.numpy()) * w.v_scale
        return kc, vc, "fp8", kval, vval
    return w.k_pool, w.v_pool, None, w.k_pool.double().numpy(), w.v_pool.double().numpy()


def _dense_numpy(q, kval, vval, lens, MB, BS, Hkv, scale):
    """Plain attention over the contiguous [B, MB*BS, Hkv, D] view of an identity-mapped pool."""
    B, Hq, D = q.shape
    G = Hq // Hkv
    out = np.zeros((B, Hq, D))
    for b in range(B):
        n = int(lens[b])
        if n == 0:
            continue
        K = kval[b * MB:(b + 1) * MB].reshape(MB * BS, Hkv, D)[:n]
        V = vval[b * MB:(b + 1) * MB].reshape(MB * BS, Hkv, D)[:n]
        K = np.repeat(K, G, axis=1)               # query head h reads KV head h // G
        V = np.repeat(V, G, axis=1)
        s = np.einsum("hd,thd->ht", q[b], K) * scale
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        out[b] = np.einsum("ht,thd->hd", p, V)
    return out


@pytest.mark.parametrize("name", list(SMALL_SHAPES))
def test_identity_table_equals_dense_numpy(name):
    cfg, lens = SMALL_SHAPES[name]
    w = I.dense_workload(cfg, lens, seed=11)
    kc, vc, kvdt, kval, vval = _cache_values(w)
    got = oracle.attn(w.q, kc, vc, w.block_tables, w.context_lens, w.scale, w.k_scale, w.v_scale, kvdt)
    ref = _dense_numpy(w.q.double().numpy(), kval, vval, w.context_lens, cfg.max_blocks, cfg.block_size,
                       cfg.Hkv, w.scale)
    assert np.max(np.abs(got - ref)) <= 1e-12


@pytest.mark.parametrize("name", list(SMALL_SHAPES))
def test_identity_table_equals_torch_sdpa(name):
    cfg, lens = SMALL_SHAPES[name]
    w = I.dense_workload(cfg, lens, seed=12)
    kc, vc, kvdt, kval, vval = _cache_values(w)
    got = oracle.attn(w.q, kc, vc, w.block_tables, w.context_lens, w.scale, w.k_scale, w.v_scale, kvdt)
    MB, BS, G = cfg.max_blocks, cfg.block_size, cfg.group
    for b, n in enumerate(w.context_lens.tolist()):
        K = torch.from_numpy(kval[b * MB:(b + 1) * MB].reshape(MB * BS, cfg.Hkv, cfg.D)[:n])
        V = torch.from_numpy(vval[b * MB:(b + 1) * MB].reshape(MB * BS, cfg.Hkv, cfg.D)[:n])
        K = K.repeat_interleave(G, dim=1).transpose(0, 1)      # [Hq, n, D]
        V = V.repeat_interleave(G, dim=1).transpose(0, 1)
        qb = w.q[b].double().unsqueeze(1)                        # [Hq, 1, D]
        ref = torch.nn.functional.scaled_dot_product_attention(qb, K, V, scale=w.scale)[:, 0, :]
        assert np.max(np.abs(got[b] - ref.numpy())) <= 1e-12


def test_brute_force_tiny_random_tables():
    cfg = I.Config("brute", 5, B=2, Hq=4, Hkv=2, D=8, block_size=4, q_dtype="bf16", kv_dtype="bf16",
                   lens=("uniform", 1, 40), pool=("factor", 1.25), max_len=40, partition_size=8)
    for seed in range(3):
        w = I.make_workload(I.shrink(cfg, seed=seed))
        got = oracle.attn(w.q, w.k_pool, w.v_pool, w.block_tables, w.context_lens, w.scale)
        ref = brute_attn(w.q.double().tolist(), w.k_pool.double().tolist(), w.v_pool.double().tolist(),
                         w.block_tables.tolist(), w.context_lens.tolist(), w.scale)
        assert np.max(np.abs(got - np.array(ref))) <= 1e-13


def test_brute_force_fp8_tiny():
    cfg = I.Config("brute8", 6, B=2, Hq=8, Hkv=1, D=8, block_size=8, q_dtype="bf16", kv_dtype="fp8",
                   lens=("uniform", 1, 40), pool=("factor", 1.25), max_len=40, partition_size=16)
    w = I.make_workload(cfg)
    kc, vc = _pool_as_fp8(w)
    got = oracle.attn(w.q, kc, vc, w.block_tables, w.context_lens, w.scale, w.k_scale, w.v_scale, "fp8")
    kv = oracle.fp8_decode(kc.numpy()).tolist()
    vv = oracle.fp8_decode(vc.numpy()).tolist()
    ref = brute_attn(w.q.double().tolist(), kv, vv, w.block_tables.tolist(), w.context_lens.tolist(),
                     w.scale, w.k_scale, w.v_scale)
    assert np.max(np.abs(got - np.array(ref))) <= 1e-13


def _small(name, **kw):
    return I.make_workload(I.shrink(I.CONFIGS[name], **kw))


@pytest.mark.parametrize("name,kw", [("tiny", {}), ("llama3_8b", dict(B=6, len_div=8)),
                                     ("llama3_70b_fp8", dict(B=6, len_div=16))])
def test_block_permutation_invariance_bitwise(name, kw):
    w = _small(name, **kw)
    w2 = I.permute_blocks(w, seed=99)
    assert not np.array_equal(w.block_tables, w2.block_tables)
    outs = []
    for x in (w, w2):
        kc, vc, kvdt, _, _ = _cache_values(x)
        outs.append(oracle.attn(x.q, kc, vc, x.block_tables, x.context_lens, x.scale, x.k_scale, x.v_scale,
                                kvdt))
    assert np.array_equal(outs[0], outs[1])


def test_shared_prefix_equals_private_copies_bitwise():
    w = _small("shared_prefix", B=8, len_div=8)
    assert w.prefix_blocks.size > 0
    assert np.all(w.refcount[w.prefix_blocks] == w.cfg.B)
    w2 = I.unshare_prefix(w)
    assert np.all(w2.refcount <= 1)
    a = oracle.attn(w.q, w.k_pool, w.v_pool, w.block_tables, w.context_lens, w.scale)
    b = oracle.attn(w2.q, w2.k_pool, w2.v_pool, w2.block_tables, w2.context_lens, w2.scale)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("name,kw", [("tiny", {}), ("llama3_8b", dict(B=4, len_div=8)),
                                     ("llama3_70b_fp8", dict(B=6, len_div=16))])
def test_stale_slots_never_read(name, kw):
    w = _small(name, **kw)
    kc, vc, kvdt, _, _ = _cache_values(w)
    a = oracle.attn(w.q, kc, vc, w.block_tables, w.context_lens, w.scale, w.k_scale, w.v_scale, kvdt)
    stale = torch.from_numpy(w.stale_slots())
    BS = w.cfg.block_size
    kc2, vc2 = kc.clone(), vc.clone()
    nan = 0x7F if kvdt == "fp8" else float("nan")
    for c in (kc2, vc2):
        flat = c.view(-1, BS, *c.shape[2:]).reshape(-1, *c.shape[2:])
        flat[stale] = nan
    b = oracle.attn(w.q, kc2, vc2, w.block_tables, w.context_lens, w.scale, w.k_scale, w.v_scale, kvdt)
    assert np.array_equal(a, b)


# ---------------------------------------------------------------- closed forms

def _one_seq(n, D=16, Hq=4, Hkv=2, BS=4, seed=3, q=None, v_fill=None):
    cfg = I.Config("cf", seed, B=1, Hq=Hq, Hkv=Hkv, D=D, block_size=BS, q_dtype="bf16", kv_dtype="bf16",
                   lens=("uniform", n, n), pool=("factor", 1.25), max_len=max(n, 1), partition_size=BS)
    w = I.make_workload(cfg)
    if q is not None:
        w.q[:] = q
    if v_fill is not None:
        w.v_pool[:] = v_fill
    return w


def _gather_rows(w, b, pool):
    BS = w.cfg.block_size
    n = int(w.context_lens[b])
    idx = [int(w.block_tables[b, t // BS]) * BS + t % BS for t in range(n)]
    return pool.reshape(-1, *pool.shape[2:])[idx].double().numpy()   # [n, Hkv, D]


def test_single_token_returns_its_value_row_exactly():
    w = _one_seq(1)
    got = oracle.attn(w.q, w.k_pool, w.v_pool, w.block_tables, w.context_lens, w.scale)
    V = _gather_rows(w, 0, w.v_pool)
    G = w.cfg.group
    for h in range(w.cfg.Hq):
        assert np.array_equal(got[0, h], V[0, h // G])


def test_zero_query_gives_mean_of_values():
    w = _one_seq(37, q=0.0)
    got = oracle.attn(w.q, w.k_pool, w.v_pool, w.block_tables, w.context_lens, w.scale)
    V = _gather_rows(w, 0, w.v_pool)
    G = w.cfg.group
    for h in range(w.cfg.Hq):
        assert np.max(np.abs(got[0, h] - V[:, h // G].mean(axis=0))) <= 1e-14


def test_constant_values_give_the_constant():
    w = _one_seq(29, v_fill=0.625)
    got = oracle.attn(w.q, w.k_pool, w.v_pool, w.block_tables, w.context_lens, w.scale)
    assert np.max(np.abs(got - 0.625)) <= 1e-15


def test_two_tokens_logistic_weights():
    w = _one_seq(2)
    got = oracle.attn(w.q, w.k_pool, w.v_pool, w.block_tables, w.context_lens, w.scale)
    K = _gather_rows(w, 0, w.k_pool)
    V = _gather_rows(w, 0, w.v_pool)
    G = w.cfg.group
    for h in range(w.cfg.Hq):
        qh = [float(x) for x in w.q[0, h].double()]
        s0 = w.scale * math.fsum(a * b for a, b in zip(qh, K[0, h // G]))
        s1 = w.scale * math.fsum(a * b for a, b in zip(qh, K[1, h // G]))
        w0 = 1.0 / (1.0 + math.exp(s1 - s0))
        ref = w0 * V[0, h // G] + (1.0 - w0) * V[1, h // G]
        assert np.max(np.abs(got[0, h] - ref)) <= 1e-14


def test_query_head_groups_read_their_kv_head():
    # V of KV head g is the constant g+1: output of head h must be h // G + 1 (not h % Hkv + 1)
    w = _one_seq(21, Hq=8, Hkv=2)
    for g in range(2):
        w.v_pool[:, :, g, :] = float(g + 1)
    got = oracle.attn(w.q, w.k_pool, w.v_pool, w.block_tables, w.context_lens, w.scale)
    for h in range(8):
        assert np.max(np.abs(got[0, h] - (h // 4 + 1))) <= 1e-15


def test_needle_dominates():
    # A key aligned with q and large enough carries ~all the weight at any position.
    w = _one_seq(70, D=16, Hq=2, Hkv=1, BS=8)
    BS = w.cfg.block_size
    q = w.q[0, 0].float()
    for pos in (0, 7, 8, 35, 69):
        w2 = _one_seq(70, D=16, Hq=2, Hkv=1, BS=8)
        w2.q[0, 1] = w2.q[0, 0]
        slot = int(w2.block_tables[0, pos // BS]) * BS + pos % BS
        kv = w2.k_pool.view(-1, 1, 16)
        vv = w2.v_pool.view(-1, 1, 16)
        kv[slot, 0] = (q / q.norm() * 64.0).to(torch.bfloat16)
        vv[slot, 0] = 3.0
        got = oracle.attn(w2.q, w2.k_pool, w2.v_pool, w2.block_tables, w2.context_lens, w2.scale)
        assert np.max(np.abs(got[0] - 3.0)) <= 1e-6


def test_partition_indicator_closed_form():
    # q = 0 and V_t = a_{t // PS}: out = sum_p a_p |P_p| / n exactly (up to fp64 rounding)
    n, PS = 150, 32
    w = _one_seq(n, D=8, Hq=2, Hkv=1, BS=8, q=0.0)
    BS = w.cfg.block_size
    a = [1.0, -2.0, 4.0, 0.5, 8.0]
    vv = w.v_pool.view(-1, 1, 8)
    for t in range(n):
        vv[int(w.block_tables[0, t // BS]) * BS + t % BS, 0] = a[t // PS]
    got = oracle.attn(w.q, w.k_pool, w.v_pool, w.block_tables, w.context_lens, w.scale)
    sizes = [min(PS, n - p * PS) for p in range(-(-n // PS))]
    ref = sum(x * s for x, s in zip(a, sizes)) / n
    assert np.max(np.abs(got - ref)) <= 1e-14


def test_empty_sequence_gives_zeros():
    w = _small("tiny")
    lens = w.context_lens.copy()
    lens[1] = 0
    got = oracle.attn(w.q, w.k_pool, w.v_pool, w.block_tables, lens, w.scale)
    assert np.all(got[1] == 0.0) and np.all(np.isfinite(got))


# ---------------------------------------------------------------- split-K partials + merge

@pytest.mark.parametrize("name,kw", [("tiny", {}), ("llama3_8b", dict(B=4, len_div=4)),
                                     ("llama3_70b_fp8", dict(B=5, len_div=8))])
def test_lse_merge_of_any_partitioning_equals_unsplit(name, kw):
    w = _small(name, **kw)
    kc, vc, kvdt, _, _ = _cache_values(w)
    full = oracle.attn(w.q, kc, vc, w.block_tables, w.context_lens, w.scale, w.k_scale, w.v_scale, kvdt)
    BS = w.cfg.block_size
    for PS in (BS, 2 * BS, 512, int(w.context_lens.max())):
        m, l, o = oracle.attn_partials(w.q, kc, vc, w.block_tables, w.context_lens, w.scale, PS,
                                       w.k_scale, w.v_scale, kvdt)
        B, Hq, Pmax = m.shape
        nparts = np.repeat(-(-w.context_lens.astype(np.int64) // PS), Hq)
        merged = oracle.lse_merge(m.reshape(B * Hq, Pmax), l.reshape(B * Hq, Pmax),
                                  o.reshape(B * Hq, Pmax, -1), nparts).reshape(full.shape)
        assert np.max(np.abs(merged - full)) <= 1e-12


def test_lse_merge_closed_form_two_partials():
    # two partials with m = (0, ln 2), l = (1, 1): weights 1 : 2
    m = np.array([[0.0, math.log(2.0)]])
    l = np.array([[1.0, 1.0]])
    o = np.array([[[3.0, 0.0], [0.0, 3.0]]])
    out = oracle.lse_merge(m, l, o, np.array([2]))
    assert np.allclose(out, [[1.0, 2.0]], rtol=0, atol=1e-15)
    assert np.all(oracle.lse_merge(m, l, o, np.array([0])) == 0.0)

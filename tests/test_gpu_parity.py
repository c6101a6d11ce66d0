"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

KV write: every byte of both pools equal.  Attention: max |GPU - oracle| within 2e-3 (fp16
output), 1e-2 (bf16) or 3e-2 (fp8 cache), and no NaN.  Full-size workloads are compared on
every output element, in the launch configuration the benchmark times (split-K with the
workload's partition size) and single pass.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_224_amd as pk
from gpu_common import (DEV, full_case, gpu_decode, gpu_pools, max_err, oracle_decode, oracle_pools,
                        tolerance)
from paged_kv_cache_224_amd import inputs as I

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


# ---------------------------------------------------------------- full-size workloads

@pytest.mark.parametrize("name", I.CONFIG_ORDER)
def test_full_write_bitexact(name):
    _say(f"[write] {name}")
    w, kc_ref, vc_ref, _ = full_case(name)
    kc, vc = gpu_pools(w)
    torch.cuda.synchronize()
    assert torch.equal(kc.cpu().view(torch.uint8).flatten(), kc_ref.view(torch.uint8).flatten())
    assert torch.equal(vc.cpu().view(torch.uint8).flatten(), vc_ref.view(torch.uint8).flatten())


def _partition(w, mode):
    if mode == "split":
        return w.cfg.partition_size
    if mode == "balanced":
        return pk.balanced_split(w.cfg.Hkv, w.cfg.D, I.DTYPES[w.cfg.q_dtype],
                                 torch.uint8 if w.cfg.kv_dtype == "fp8" else I.DTYPES[w.cfg.kv_dtype])
    return 0


@pytest.mark.parametrize("name,mode", [(n, m) for n in I.CONFIG_ORDER for m in ("balanced", "split", "single")])
def test_full_decode_parity(name, mode):
    _say(f"[decode] {name} {mode}")
    w, _, _, ref = full_case(name)
    kc, vc = gpu_pools(w)
    PS = _partition(w, mode)
    got = gpu_decode(w, kc, vc, PS, max_context_len=w.cfg.max_len)
    err = max_err(got, ref)
    _say(f"    max-abs err {err:.3e} (tol {tolerance(w.cfg)})")
    assert err <= tolerance(w.cfg)


# ---------------------------------------------------------------- smaller cases, many shapes

def _small(name, **kw):
    return I.make_workload(I.shrink(I.CONFIGS[name], **kw))


SMALL = [("tiny", {}), ("llama3_8b", dict(B=6, len_div=4)), ("long_ctx", dict(B=2, len_div=32)),
         ("shared_prefix", dict(B=6, len_div=4)), ("llama3_70b_fp8", dict(B=8, len_div=4))]


def _case_id(x):
    return x[0] if isinstance(x, tuple) else str(x)


@pytest.mark.parametrize("case", SMALL, ids=_case_id)
def test_stale_nan_slots_do_not_leak(case):
    name, kw = case
    _say(f"[poison] {name}")
    w = _small(name, **kw)
    kc_ref, vc_ref = oracle_pools(w)
    ref = oracle_decode(w, kc_ref, vc_ref)
    kc, vc = gpu_pools(w)
    clean = gpu_decode(w, kc, vc, w.cfg.partition_size)
    stale = torch.from_numpy(w.stale_slots()).to(DEV)
    nan = 0x7F if w.cfg.kv_dtype == "fp8" else float("nan")
    for c in (kc, vc):
        c.view(-1, *c.shape[2:])[stale] = nan
    for PS in (w.cfg.partition_size, 0, -64):
        got = gpu_decode(w, kc, vc, PS)
        assert max_err(got, ref) <= tolerance(w.cfg)
        if PS == w.cfg.partition_size:
            assert np.array_equal(got, clean)


@pytest.mark.parametrize("case", SMALL, ids=_case_id)
def test_deterministic_and_block_permutation_invariant(case):
    name, kw = case
    _say(f"[determinism] {name}")
    w = _small(name, **kw)
    kc, vc = gpu_pools(w)
    a = gpu_decode(w, kc, vc, w.cfg.partition_size)
    b = gpu_decode(w, kc, vc, w.cfg.partition_size)
    assert np.array_equal(a, b)
    w2 = I.permute_blocks(w, seed=7)
    kc2, vc2 = gpu_pools(w2)
    c = gpu_decode(w2, kc2, vc2, w.cfg.partition_size)
    assert np.array_equal(a, c)
    d = gpu_decode(w, kc, vc, -64)
    e = gpu_decode(w2, kc2, vc2, -64)
    assert np.array_equal(d, e)


@pytest.mark.parametrize("W", [1, 3, 37, 512, 100000])
def test_balanced_split_any_workgroup_count(W):
    """Balanced schedules cut sequences at arbitrary tile boundaries; every W must give the
    oracle's answer, including empty, one-token and single-tile sequences."""
    _say(f"[balanced] W={W}")
    cfg = I.Config("bal", 33, B=11, Hq=16, Hkv=4, D=128, block_size=32, q_dtype="bf16", kv_dtype="bf16",
                   lens=("uniform", 1, 1), pool=("factor", 1.25), max_len=3000, partition_size=512)
    lens = [0, 1, 16, 17, 2999, 512, 0, 33, 1500, 7, 3000]
    w = I.permute_blocks(I.dense_workload(cfg, lens, seed=5), seed=6)
    kc_ref, vc_ref = oracle_pools(w)
    ref = oracle_decode(w, kc_ref, vc_ref)
    kc, vc = gpu_pools(w)
    got = gpu_decode(w, kc, vc, -W, max_context_len=3000)
    assert max_err(got, ref) <= 1e-2
    assert np.all(got[0] == 0) and np.all(got[6] == 0)


def test_shared_prefix_equals_private_copies_on_gpu():
    _say("[cow] shared_prefix")
    w = _small("shared_prefix", B=16, len_div=2)
    w2 = I.unshare_prefix(w)
    for PS in (512, 0, -200):
        kc, vc = gpu_pools(w)
        a = gpu_decode(w, kc, vc, PS)
        kc2, vc2 = gpu_pools(w2)
        b = gpu_decode(w2, kc2, vc2, PS)
        assert np.array_equal(a, b)


@pytest.mark.parametrize("case", SMALL, ids=_case_id)
def test_load_policy_flag_changes_no_result(case):
    """The shared-blocks flag only picks the cache policy of the K/V loads: both settings give
    the same bits in every schedule."""
    name, kw = case
    _say(f"[policy] {name} {kw}")
    w = _small(name, **kw)
    kc, vc = gpu_pools(w)
    for PS in (0, 512, -64):
        a = gpu_decode(w, kc, vc, PS, shared_blocks=False)
        b = gpu_decode(w, kc, vc, PS, shared_blocks=True)
        assert np.array_equal(a, b, equal_nan=True), PS


@pytest.mark.parametrize("case", SMALL, ids=_case_id)
def test_split_partials_match_oracle(case):
    name, kw = case
    _say(f"[partials] {name}")
    w = _small(name, **kw)
    cfg = w.cfg
    kc_ref, vc_ref = oracle_pools(w)
    kvdt = "fp8" if cfg.kv_dtype == "fp8" else None
    PS = cfg.partition_size
    maxlen = int(w.context_lens.max())
    m, l, o = oracle.attn_partials(w.q, kc_ref, vc_ref, w.block_tables, w.context_lens, w.scale, PS,
                                   w.k_scale, w.v_scale, kvdt)
    kc, vc = gpu_pools(w)
    ws = pk.DecodeWorkspace(cfg.B, cfg.Hq, cfg.D, maxlen, PS, device=DEV)
    pk.paged_attn_decode(None, w.q.to(DEV), kc, vc, torch.from_numpy(w.block_tables).to(DEV),
                         torch.from_numpy(w.context_lens).to(DEV), w.scale, maxlen, PS, ws.tmp_out,
                         ws.max_logits, ws.exp_sums, w.k_scale, w.v_scale)
    torch.cuda.synchronize()
    P = -(-w.context_lens.astype(np.int64) // PS)
    gm, gl, go = (x.cpu().numpy() for x in (ws.max_logits, ws.exp_sums, ws.tmp_out))
    for b in range(cfg.B):
        for p in range(P[b]):
            assert np.max(np.abs(gm[b, :, p] - m[b, :, p])) <= 2e-3
            assert np.max(np.abs(gl[b, :, p] / l[b, :, p] - 1.0)) <= 1e-2
            assert np.max(np.abs(go[b, :, p] - o[b, :, p])) <= tolerance(cfg)


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("D", [64, 128])
def test_reduce_alone_on_injected_partials(D, out_dtype):
    _say(f"[reduce] D={D} {out_dtype}")
    rng = np.random.default_rng(5)
    B, Hq, PS = 7, 5, 64
    lens = np.array([0, 1, 64, 65, 300, 1000, 4096], dtype=np.int32)
    maxlen = int(lens.max())
    Pmax = -(-maxlen // PS)
    m = rng.normal(0, 3, size=(B, Hq, Pmax)).astype(np.float32)
    l = rng.uniform(1, 100, size=(B, Hq, Pmax)).astype(np.float32)
    o = rng.normal(0, 1, size=(B, Hq, Pmax, D)).astype(np.float32)
    P = -(-lens.astype(np.int64) // PS)
    # partials past P hold garbage that must never be read
    for b in range(B):
        m[b, :, P[b]:] = np.nan
        l[b, :, P[b]:] = np.nan
        o[b, :, P[b]:] = np.nan
    ref = oracle.lse_merge(m.reshape(B * Hq, Pmax), l.reshape(B * Hq, Pmax), o.reshape(B * Hq, Pmax, D),
                           np.repeat(P, Hq)).reshape(B, Hq, D)
    out = torch.full((B, Hq, D), float("nan"), dtype=out_dtype, device=DEV)
    pk.paged_attn_reduce(out, torch.from_numpy(o).to(DEV), torch.from_numpy(m).to(DEV),
                         torch.from_numpy(l).to(DEV), torch.from_numpy(lens).to(DEV), maxlen, PS)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    tol = 1e-2 if out_dtype == torch.bfloat16 else 2e-3
    assert max_err(got, ref) <= tol
    assert np.all(got[0] == 0.0)


# ---------------------------------------------------------------- closed forms on long contexts

def test_needles_at_partition_boundaries():
    """One key aligned with q carries ~all weight: output = that token's V (any position)."""
    _say("[needle]")
    cfg = I.Config("needle", 21, B=1, Hq=4, Hkv=1, D=128, block_size=16, q_dtype="bf16", kv_dtype="bf16",
                   lens=("uniform", 5000, 5000), pool=("factor", 1.25), max_len=5000, partition_size=512)
    base = I.make_workload(cfg)
    BS = cfg.block_size
    q = base.q[0, 0].float()
    base.q[0, :] = base.q[0, 0]
    for pos in (0, 15, 16, 511, 512, 1023, 2048, 4990, 4999):
        w = I.make_workload(cfg)
        w.q[0, :] = base.q[0, 0]
        slot = int(w.block_tables[0, pos // BS]) * BS + pos % BS
        kview = w.k_pool.view(-1, 1, 128)
        vview = w.v_pool.view(-1, 1, 128)
        kview[slot, 0] = (q / q.norm() * 96.0).to(torch.bfloat16)
        vview[slot, 0] = torch.linspace(-2, 2, 128).to(torch.bfloat16)
        w.slot_mapping[:] = -1                     # no write this step
        kc, vc = gpu_pools(w)
        for PS in (512, 0, -3):
            got = gpu_decode(w, kc, vc, PS)
            want = vview[slot, 0].float().numpy()
            assert np.max(np.abs(got[0] - want[None, :])) <= 1e-2, (pos, PS)


def test_partition_indicator_exact_weights():
    """q = 0 and V_t = a_{t // 512}: out = sum_p a_p |P_p| / n, catching dropped or doubled
    partitions that a 1e-2 tolerance would otherwise hide at long context."""
    _say("[indicator]")
    n, PS = 40000, 512
    cfg = I.Config("indic", 22, B=1, Hq=8, Hkv=2, D=128, block_size=16, q_dtype="bf16", kv_dtype="bf16",
                   lens=("uniform", n, n), pool=("factor", 1.25), max_len=n, partition_size=PS)
    w = I.make_workload(cfg)
    w.q.zero_()
    BS = cfg.block_size
    nparts = -(-n // PS)
    a = (np.arange(nparts) % 7 - 3).astype(np.float32)          # small integers, bf16-exact
    t = np.arange(n)
    slots = w.block_tables[0, t // BS].astype(np.int64) * BS + t % BS
    vflat = w.v_pool.view(-1, cfg.Hkv, cfg.D)
    vflat[torch.from_numpy(slots)] = torch.from_numpy(a[t // PS]).to(torch.bfloat16)[:, None, None].expand(
        n, cfg.Hkv, cfg.D)
    w.slot_mapping[:] = -1
    sizes = np.minimum(PS, n - PS * np.arange(nparts))
    want = float((a * sizes).sum() / n)
    kc, vc = gpu_pools(w)
    for P in (PS, 0, -7, -1000):
        got = gpu_decode(w, kc, vc, P)
        assert np.max(np.abs(got - want)) <= 2e-3 + abs(want) * 2 ** -8, P


# ---------------------------------------------------------------- fp8 encode, exhaustively

@pytest.mark.parametrize("scale", [1.0, 2.0 ** -4, 0.0137, 3.0])
def test_fp8_write_all_bf16_patterns(scale):
    _say(f"[fp8 encode] scale {scale}")
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    src = bits.view(torch.bfloat16).view(512, 1, 128)
    want = oracle.fp8_encode(src.float(), scale).view(512, 1, 128)
    kc = torch.zeros((32, 16, 1, 128), dtype=torch.uint8, device=DEV)
    vc = torch.zeros_like(kc)
    slots = torch.arange(512, dtype=torch.int64, device=DEV)
    pk.paged_kv_write(src.to(DEV), src.to(DEV), kc, vc, slots, scale, scale)
    torch.cuda.synchronize()
    got = kc.cpu().view(512, 1, 128)
    assert torch.equal(got, want)
    assert torch.equal(vc.cpu().view(512, 1, 128), want)


def test_write_skips_negative_slots_and_keeps_other_bytes():
    _say("[write skip]")
    w = _small("llama3_8b", B=8, len_div=8)
    sm = w.slot_mapping.copy()
    sm[::3] = -1
    kc_ref, vc_ref = w.k_pool.clone(), w.v_pool.clone()
    oracle.kv_write(w.k_new, w.v_new, kc_ref, vc_ref, sm)
    kc, vc = w.k_pool.to(DEV), w.v_pool.to(DEV)
    pk.paged_kv_write(w.k_new.to(DEV), w.v_new.to(DEV), kc, vc, torch.from_numpy(sm).to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(kc.cpu().view(torch.int16), kc_ref.view(torch.int16))
    assert torch.equal(vc.cpu().view(torch.int16), vc_ref.view(torch.int16))


# ---------------------------------------------------------------- shapes and edges

SHAPES = [
    # (Hq, Hkv, D, BS, q dtype, kv dtype)
    (8, 8, 128, 16, "bf16", "bf16"),
    (16, 8, 128, 32, "bf16", "bf16"),
    (32, 2, 128, 64, "bf16", "bf16"),
    (16, 1, 64, 16, "f16", "f16"),
    (4, 2, 64, 32, "bf16", "bf16"),
    (8, 1, 128, 16, "bf16", "fp8"),
    (16, 2, 64, 32, "f16", "fp8"),
    (12, 4, 128, 256, "f16", "f16"),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "-".join(map(str, s)))
def test_shapes_and_ragged_lengths(shape):
    Hq, Hkv, D, BS, qdt, kvdt = shape
    _say(f"[shape] {shape}")
    lens = [1, 2, 15, 16, 17, BS - 1, BS, BS + 1, 255, 256, 257, 511, 512, 513, 1000, 1537]
    cfg = I.Config("shape", 31, B=len(lens), Hq=Hq, Hkv=Hkv, D=D, block_size=BS, q_dtype=qdt, kv_dtype=kvdt,
                   lens=("uniform", 1, 1), pool=("factor", 1.25), max_len=2048, partition_size=256)
    w = I.dense_workload(cfg, lens, seed=3)
    w = I.permute_blocks(w, seed=4)
    kc_ref, vc_ref = oracle_pools(w)
    ref = oracle_decode(w, kc_ref, vc_ref)
    kc, vc = gpu_pools(w)
    assert torch.equal(kc.cpu().view(torch.uint8).flatten(), kc_ref.view(torch.uint8).flatten())
    for PS in (0, 256, max(BS, 64) if BS <= 64 else BS, -5, -300):
        got = gpu_decode(w, kc, vc, PS, max_context_len=2048)
        assert max_err(got, ref) <= tolerance(cfg), PS


def test_empty_and_full_length_sequences():
    _say("[edges]")
    cfg = I.Config("edge", 32, B=5, Hq=8, Hkv=2, D=128, block_size=16, q_dtype="bf16", kv_dtype="bf16",
                   lens=("uniform", 1, 1), pool=("factor", 1.25), max_len=1024, partition_size=128)
    lens = [0, 1024, 0, 7, 1024]
    w = I.dense_workload(cfg, lens, seed=9)
    kc_ref, vc_ref = oracle_pools(w)
    ref = oracle_decode(w, kc_ref, vc_ref)
    kc, vc = gpu_pools(w)
    for PS in (128, 0, -2):
        got = gpu_decode(w, kc, vc, PS, max_context_len=1024)
        assert max_err(got, ref) <= 1e-2
        assert np.all(got[0] == 0) and np.all(got[2] == 0)


def test_checked_mode_rejects_bad_device_values(monkeypatch):
    _say("[checked mode]")
    w = _small("tiny")
    cfg = w.cfg
    kc, vc = gpu_pools(w)
    bt = w.block_tables.copy()
    bt[1, 0] = w.num_blocks + 5                    # out-of-range block id (kernel clamps it)
    out = torch.empty((cfg.B, cfg.Hq, cfg.D), dtype=torch.float16, device=DEV)
    args = (out, w.q.to(DEV), kc, vc, torch.from_numpy(bt).to(DEV), torch.from_numpy(w.context_lens).to(DEV),
            w.scale, cfg.max_len, 0)
    monkeypatch.setenv("PKV_CHECK", "1")
    with pytest.raises(pk.PagedKVError) as ei:
        pk.paged_attn_decode(*args)
    assert ei.value.status == -7
    dup = np.repeat(w.slot_mapping[:1], 2)
    with pytest.raises(pk.PagedKVError):
        pk.paged_kv_write(w.k_new[:2].to(DEV), w.v_new[:2].to(DEV), kc, vc, torch.from_numpy(dup).to(DEV))
    monkeypatch.delenv("PKV_CHECK")
    pk.paged_attn_decode(*args)                    # fast path: clamped id, no fault
    torch.cuda.synchronize()


# ---------------------------------------------------------------- a caller error stays in its row

@pytest.mark.parametrize("mode", ["balanced", "split", "single"])
def test_length_past_the_table_spoils_only_its_row(mode):
    """One context length above max_blocks * block_size (a caller error; PKV_CHECK=1 reports it)
    must leave every other row correct: the decode and the reduce clamp lengths to the same
    max_context_len, so they count the same split units, and the decode clamps the table index
    to the row, so the bad row only re-reads its own last entry."""
    cfg = I.shrink(I.CONFIGS["llama3_8b"], B=24, len_div=8, name="overlong")
    _say(f"[overlong] {mode}")
    w = I.make_workload(cfg)
    kc_ref, vc_ref = oracle_pools(w)
    ref = oracle_decode(w, kc_ref, vc_ref)
    kc, vc = gpu_pools(w)
    bad = 5
    lens = w.context_lens.copy()
    lens[bad] = cfg.max_blocks * cfg.block_size + 200
    maxlen = int(lens.max())
    PS = _partition(w, mode)
    out = torch.full((cfg.B, cfg.Hq, cfg.D), float("nan"), dtype=torch.bfloat16, device=DEV)
    ws = pk.DecodeWorkspace(cfg.B, cfg.Hq, cfg.D, maxlen, PS, device=DEV)
    pk.decode(out, w.q.to(DEV), kc, vc, torch.from_numpy(w.block_tables).to(DEV), torch.from_numpy(lens).to(DEV),
              w.scale, ws)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    keep = np.arange(cfg.B) != bad
    err = max_err(got[keep], ref[keep])
    _say(f"    other rows max-abs err {err:.3e}")
    assert err <= tolerance(cfg)


@pytest.mark.parametrize("B,Hq", [(40, 512), (3300, 5)])
def test_reduce_alone_many_rows(B, Hq):
    """A merge with more than 16384 output rows runs one row per 16-lane group (four rows per
    wave); with 5 rows per sequence a wave's rows straddle two sequences.  Injected partials,
    NaN garbage past each row's count, against the fp64 merge."""
    _say(f"[reduce many rows] B={B} Hq={Hq}")
    rng = np.random.default_rng(9)
    D, PS = 128, 64
    lens = rng.integers(0, 300, size=B).astype(np.int32)
    lens[:3] = [0, 1, 299]
    maxlen = int(lens.max())
    Pmax = -(-maxlen // PS)
    m = rng.normal(0, 3, size=(B, Hq, Pmax)).astype(np.float32)
    l = rng.uniform(1, 100, size=(B, Hq, Pmax)).astype(np.float32)
    o = rng.normal(0, 1, size=(B, Hq, Pmax, D)).astype(np.float32)
    P = -(-lens.astype(np.int64) // PS)
    for b in range(B):
        m[b, :, P[b]:] = np.nan
        l[b, :, P[b]:] = np.nan
        o[b, :, P[b]:] = np.nan
    ref = oracle.lse_merge(m.reshape(B * Hq, Pmax), l.reshape(B * Hq, Pmax), o.reshape(B * Hq, Pmax, D),
                           np.repeat(P, Hq)).reshape(B, Hq, D)
    out = torch.full((B, Hq, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    pk.paged_attn_reduce(out, torch.from_numpy(o).to(DEV), torch.from_numpy(m).to(DEV),
                         torch.from_numpy(l).to(DEV), torch.from_numpy(lens).to(DEV), maxlen, PS)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    # bf16 keeps 8 significant bits: rounding is at most 2^-8 of the value (single-partition rows
    # pass normal(0, 1) values through, and a few of 2.6M reach 4 and beyond)
    assert not np.isnan(got).any()
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-3)
    assert np.all(got[lens == 0] == 0)

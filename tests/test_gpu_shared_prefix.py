"""GPU parity of paged_attn_decode_shared_prefix: the prefix pass (every row's queries against
the shared prefix on MFMA), the balanced suffix decode and the merge must give what the fp64
oracle's plain decode gives for the same batch -- the same definition of attention, computed
in a different order -- within the usual tolerance.

Cases: the full shared-prefix workload; smaller batches over every dtype pair and head size,
with prefix partitions that end mid-stage, a prefix of one partition, no prefix, rows shorter
than the prefix (down to empty), partial query-column groups, NaN in prefix slots that no row
can see, determinism, and the checked mode's test of the sharing contract.
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


def _prefix_len(w):
    return int(w.prefix_blocks.size) * w.cfg.block_size


def _run(w, kc, vc, prefix_len, pps=None, PS=None, maxlen=None):
    cfg = w.cfg
    maxlen = maxlen or max(1, int(w.context_lens.max()))
    if PS is None:
        PS = pk.balanced_split(cfg.Hkv, cfg.D, I.DTYPES[cfg.q_dtype],
                               torch.uint8 if cfg.kv_dtype == "fp8" else I.DTYPES[cfg.kv_dtype])
    ws = pk.SharedPrefixWorkspace(cfg.B, cfg.Hq, cfg.Hkv, cfg.D, maxlen, prefix_len, PS, pps, device=DEV)
    ws.tmp_out.fill_(float("nan"))                  # every slot the merge reads must be written
    ws.max_logits.fill_(float("nan"))
    ws.exp_sums.fill_(float("nan"))
    out = torch.full((cfg.B, cfg.Hq, cfg.D), float("nan"), dtype=I.DTYPES[cfg.q_dtype], device=DEV)
    pk.decode_shared_prefix(out, w.q.to(DEV), kc, vc, torch.from_numpy(w.block_tables).to(DEV),
                            torch.from_numpy(w.context_lens).to(DEV), w.scale, ws, w.k_scale, w.v_scale)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


def test_full_shared_prefix_workload():
    w, kc_ref, vc_ref, ref = full_case("shared_prefix")
    P = _prefix_len(w)
    _say(f"[shared prefix] full workload, prefix {P}")
    kc, vc = gpu_pools(w)
    got = _run(w, kc, vc, P)
    err = max_err(got, ref)
    _say(f"  max-abs err vs oracle {err:.2e}")
    assert err <= tolerance(w.cfg)
    plain = gpu_decode(w, kc, vc, pk.balanced_split(8, 128, torch.bfloat16, torch.bfloat16))
    assert max_err(got, plain) <= tolerance(w.cfg)


def _prefix_cfg(base, name, B, P, lo, hi, **kw):
    cfg = dataclasses.replace(I.CONFIGS[base], name=name, B=B, lens=("prefix", P, lo, hi), max_len=P + hi,
                              pool=("factor", 1.25), **kw)
    return cfg


CASES = [
    # name, config, prefix partition sizes to try
    ("bf16_g4_d128", _prefix_cfg("shared_prefix", "sp_a", 37, 256, 1, 100, seed=21), (64, 48, 256, 16)),
    ("f16_g4_d64_bs32", _prefix_cfg("tiny", "sp_b", 9, 96, 0, 70, seed=22, block_size=32), (32, 96)),
    ("fp8_g8_d128_bs32", _prefix_cfg("llama3_70b_fp8", "sp_c", 20, 320, 5, 200, seed=23), (64, 112)),
    ("bf16_g4_d128_bs64", _prefix_cfg("shared_prefix", "sp_d", 33, 192, 16, 300, seed=24, block_size=64), (128,)),
    ("f16_fp8_d64", _prefix_cfg("tiny", "sp_e", 3, 48, 1, 40, seed=25, kv_dtype="fp8"), (16, 48)),
    ("bf16_g16_hkv1_d64", _prefix_cfg("tiny", "sp_f", 11, 80, 1, 60, seed=26, Hq=16, Hkv=1, q_dtype="bf16",
                                      kv_dtype="bf16"), (32, 80)),
    ("bf16_g1_hkv16", _prefix_cfg("shared_prefix", "sp_g", 5, 64, 1, 50, seed=27, Hq=16, Hkv=16), (64, 16)),
]


@pytest.mark.parametrize("name,cfg,ppss", CASES, ids=[c[0] for c in CASES])
def test_shared_prefix_small(name, cfg, ppss):
    w = I.make_workload(cfg)
    P = _prefix_len(w)
    kc_ref, vc_ref = oracle_pools(w)
    ref = oracle_decode(w, kc_ref, vc_ref)
    kc, vc = gpu_pools(w)
    for pps in ppss:
        _say(f"[shared prefix] {name} B={cfg.B} prefix {P} partition {pps}")
        got = _run(w, kc, vc, P, pps)
        assert max_err(got, ref) <= tolerance(cfg), pps
    # a balanced split over very few workgroups (several suffix segments per workgroup)
    got = _run(w, kc, vc, P, ppss[0], PS=-3)
    assert max_err(got, ref) <= tolerance(cfg)


def test_no_prefix_equals_balanced_decode():
    _say("[shared prefix] prefix_len 0")
    w = I.make_workload(I.shrink(I.CONFIGS["llama3_8b"], B=10, len_div=8))
    kc, vc = gpu_pools(w)
    PS = pk.balanced_split(8, 128, torch.bfloat16, torch.bfloat16)
    got = _run(w, kc, vc, 0, PS=PS)
    plain = gpu_decode(w, kc, vc, PS)
    assert np.array_equal(got, plain)              # same kernels, same partials, same merge


def test_rows_shorter_than_prefix_and_invisible_nan():
    """Rows of length 0, 1, P - 1, P and P + k.  Then every row is cut below the prefix end and
    the prefix slots no row can see are filled with NaN: no NaN may reach the output."""
    cfg = _prefix_cfg("shared_prefix", "sp_short", 12, 128, 1, 60, seed=31)
    w = I.make_workload(cfg)
    P = _prefix_len(w)
    lens = w.context_lens.copy()
    lens[:6] = [0, 1, P - 1, P, 17, P - 16]
    w = dataclasses.replace(w, context_lens=lens)
    kc_ref, vc_ref = oracle_pools(w)
    ref = oracle_decode(w, kc_ref, vc_ref)
    kc, vc = gpu_pools(w)
    _say(f"[shared prefix] short rows {lens.tolist()}")
    got = _run(w, kc, vc, P, 64, maxlen=int(cfg.max_len))
    assert max_err(got, ref) <= tolerance(cfg)
    assert np.all(got[0] == 0)

    cut = np.minimum(lens, P - 40)                 # nobody sees prefix tokens >= P - 40
    cut[1] = 0
    w2 = dataclasses.replace(w, context_lens=cut.astype(np.int32))
    BS = cfg.block_size
    kc2, vc2 = kc.clone(), vc.clone()
    for t in range(int(cut.max()), P):             # stale bytes in shared blocks past every row
        blk = int(w.prefix_blocks[t // BS])
        kc2[blk, t % BS] = float("nan")
        vc2[blk, t % BS] = float("nan")
    ref2 = oracle_decode(w2, kc_ref, vc_ref)
    got2 = _run(w2, kc2, vc2, P, 64, maxlen=int(cfg.max_len))
    assert max_err(got2, ref2) <= tolerance(cfg)


def test_partial_column_groups():
    """B * G = 12 (one wave of 16 columns, 4 idle) and B * G = 132 (a second workgroup with one
    active wave)."""
    for B in (3, 33):
        cfg = _prefix_cfg("shared_prefix", f"sp_cols{B}", B, 64, 1, 40, seed=40 + B)
        w = I.make_workload(cfg)
        kc_ref, vc_ref = oracle_pools(w)
        ref = oracle_decode(w, kc_ref, vc_ref)
        kc, vc = gpu_pools(w)
        _say(f"[shared prefix] B={B}")
        assert max_err(_run(w, kc, vc, 64, 32), ref) <= tolerance(cfg)


def test_deterministic():
    cfg = _prefix_cfg("shared_prefix", "sp_det", 40, 512, 1, 300, seed=51)
    w = I.make_workload(cfg)
    kc, vc = gpu_pools(w)
    _say("[shared prefix] determinism")
    a = _run(w, kc, vc, 512, 128)
    b = _run(w, kc, vc, 512, 128)
    assert np.array_equal(a, b)


def test_checked_mode_rejects_unshared_prefix(monkeypatch):
    cfg = _prefix_cfg("shared_prefix", "sp_chk", 4, 64, 1, 40, seed=61)
    w = I.make_workload(cfg)
    kc, vc = gpu_pools(w)
    bt = w.block_tables.copy()
    bt[2, 1] = w.trap_block                        # row 2 names another block inside the prefix
    w2 = dataclasses.replace(w, block_tables=bt)
    _say("[shared prefix] checked mode")
    monkeypatch.setenv("PKV_CHECK", "1")
    with pytest.raises(pk.PagedKVError) as ei:
        _run(w2, kc, vc, 64, 32)
    assert ei.value.status == -7
    _run(w, kc, vc, 64, 32)                        # the intact table passes the check
    monkeypatch.delenv("PKV_CHECK")


def test_many_rows_merge_with_prefix_slots():
    """1100 rows x 16 query heads = 17600 output rows: the merge takes one row per 16-lane group
    and reads the prefix pass's slots before the suffix slots (slot0 > 0), over a default and a
    narrow balanced split."""
    cfg = _prefix_cfg("tiny", "sp_rows", 1100, 64, 1, 40, seed=29, Hq=16, Hkv=4, q_dtype="bf16", kv_dtype="bf16")
    w = I.make_workload(cfg)
    P = _prefix_len(w)
    kc_ref, vc_ref = oracle_pools(w)
    ref = oracle_decode(w, kc_ref, vc_ref)
    kc, vc = gpu_pools(w)
    for pps, PS in ((32, None), (64, -5)):
        _say(f"[shared prefix] many rows B={cfg.B} prefix {P} partition {pps} PS={PS}")
        got = _run(w, kc, vc, P, pps, PS=PS)
        assert max_err(got, ref) <= tolerance(cfg), (pps, PS)

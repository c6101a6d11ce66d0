"""HIP-graph capture of the decode step (write -> decode -> reduce), replayed.

A captured step must reproduce the eager step bit for bit on every replay, with eager work
and device synchronisation between the replays (the kernels allocate nothing, enqueue no
memset and keep no state between launches, so a replay is the same launch sequence).
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_224_amd as pk
from gpu_common import DEV, gpu_pools, max_err, oracle_decode, oracle_pools, tolerance
from paged_kv_cache_224_amd import inputs as I

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("name,kw,PS", [("tiny", {}, 0), ("tiny", {}, -64), ("llama3_8b", dict(B=12, len_div=4), -64),
                                        ("llama3_70b_fp8", dict(B=10, len_div=4), 512)])
def test_graph_replay_matches_eager(name, kw, PS):
    _say(f"[graph] {name} PS={PS}")
    w = I.make_workload(I.shrink(I.CONFIGS[name], **kw))
    cfg = w.cfg
    kc, vc = gpu_pools(w, write_step=False)
    q = w.q.to(DEV)
    k_new, v_new = w.k_new.to(DEV), w.v_new.to(DEV)
    slots = torch.from_numpy(w.slot_mapping).to(DEV)
    bt = torch.from_numpy(w.block_tables).to(DEV)
    lens = torch.from_numpy(w.context_lens).to(DEV)
    maxlen = int(w.context_lens.max())
    ws = pk.DecodeWorkspace(cfg.B, cfg.Hq, cfg.D, maxlen, PS, device=DEV)
    out = torch.empty((cfg.B, cfg.Hq, cfg.D), dtype=I.DTYPES[cfg.q_dtype], device=DEV)

    def step():
        pk.paged_kv_write(k_new, v_new, kc, vc, slots, w.k_scale, w.v_scale)
        pk.decode(out, q, kc, vc, bt, lens, w.scale, ws, w.k_scale, w.v_scale)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    kc_ref, vc_ref = oracle_pools(w)
    assert max_err(eager.float().cpu().numpy(), oracle_decode(w, kc_ref, vc_ref)) <= tolerance(cfg)

    g = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        step()                                         # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=stream):
        step()
    scratch = torch.randn(1 << 20, device=DEV)
    for rep in range(4):
        out.fill_(float("nan"))
        scratch.mul_(1.0001)                           # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep} differs from the eager step"
    # the replayed KV write stores the same rows at the same slots: pools still equal the oracle's
    assert torch.equal(kc.cpu().view(torch.uint8).flatten(), kc_ref.view(torch.uint8).flatten())
    assert torch.equal(vc.cpu().view(torch.uint8).flatten(), vc_ref.view(torch.uint8).flatten())


def test_step_graphs_for_a_set_of_batch_sizes():
    """Graphs captured for sizes 1, 4, 16, 64; batches of 3, 16, 40, 1 and 40 rows replay the
    smallest size that fits (padding rows have no tokens and no slot) and give the eager step's
    output bit for bit; the pools end as the eager writes leave them."""
    from paged_kv_cache_224_amd.graphs import StepGraphs
    w = I.make_workload(I.shrink(I.CONFIGS["llama3_8b"], B=40, len_div=8))
    cfg = w.cfg
    kc, vc = w.k_pool.to(DEV), w.v_pool.to(DEV)
    kc_e, vc_e = kc.clone(), vc.clone()
    maxlen = cfg.max_len
    g = StepGraphs(kc, vc, cfg.Hq, cfg.max_blocks, maxlen, torch.bfloat16, sizes=(1, 4, 16, 64))
    PS = g.partition_size
    ws = pk.DecodeWorkspace(cfg.B, cfg.Hq, cfg.D, maxlen, PS, device=DEV)
    for B in (3, 16, 40, 1, 40):
        _say(f"[graphs] batch {B} -> size {g.size_for(B)}")
        q, kn, vn, sl, bt, ln = g.inputs(B)
        q.copy_(w.q[:B])
        kn.copy_(w.k_new[:B])
        vn.copy_(w.v_new[:B])
        sl.copy_(torch.from_numpy(w.slot_mapping[:B]))
        bt.copy_(torch.from_numpy(w.block_tables[:B]))
        ln.copy_(torch.from_numpy(w.context_lens[:B]))
        got = g.replay(B).clone()
        torch.cuda.synchronize()
        out = torch.empty((B, cfg.Hq, cfg.D), dtype=torch.bfloat16, device=DEV)
        pk.paged_kv_write(w.k_new[:B].to(DEV), w.v_new[:B].to(DEV), kc_e, vc_e,
                          torch.from_numpy(w.slot_mapping[:B]).to(DEV))
        pk.decode(out, w.q[:B].to(DEV), kc_e, vc_e, torch.from_numpy(w.block_tables[:B]).to(DEV),
                  torch.from_numpy(w.context_lens[:B]).to(DEV), w.scale, ws)
        torch.cuda.synchronize()
        assert torch.equal(got, out), B
    assert torch.equal(kc.view(torch.uint8), kc_e.view(torch.uint8))
    assert torch.equal(vc.view(torch.uint8), vc_e.view(torch.uint8))


@pytest.mark.parametrize("path", ["shared_prefix", "append"])
def test_graph_replay_of_the_newer_entry_points(path):
    """The shared-prefix decode and the append decode allocate nothing either: captured once,
    replayed four times with eager work in between, equal to the eager call."""
    _say(f"[graph] {path}")
    if path == "shared_prefix":
        w = I.make_workload(I.shrink(I.CONFIGS["shared_prefix"], B=24, len_div=4))
    else:
        w = I.make_workload(I.shrink(I.CONFIGS["llama3_8b"], B=12, len_div=4))
    cfg = w.cfg
    kc, vc = w.k_pool.to(DEV), w.v_pool.to(DEV)
    q, kn, vn = w.q.to(DEV), w.k_new.to(DEV), w.v_new.to(DEV)
    bt = torch.from_numpy(w.block_tables).to(DEV)
    lens = torch.from_numpy(w.context_lens).to(DEV)
    maxlen = int(w.context_lens.max())
    PS = pk.balanced_split(cfg.Hkv, cfg.D, torch.bfloat16, torch.bfloat16)
    out = torch.empty((cfg.B, cfg.Hq, cfg.D), dtype=torch.bfloat16, device=DEV)
    if path == "shared_prefix":
        P = int(w.prefix_blocks.size) * cfg.block_size
        ws = pk.SharedPrefixWorkspace(cfg.B, cfg.Hq, cfg.Hkv, cfg.D, maxlen, P, PS, 64, device=DEV)

        def call():
            pk.decode_shared_prefix(out, q, kc, vc, bt, lens, w.scale, ws)
    else:
        ws = pk.DecodeWorkspace(cfg.B, cfg.Hq, cfg.D, maxlen, PS, device=DEV)

        def call():
            pk.decode_append(out, q, kn, vn, kc, vc, bt, lens, w.scale, ws)

    call()
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        call()
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=stream):
        call()
    scratch = torch.randn(1 << 20, device=DEV)
    for rep in range(4):
        out.fill_(float("nan"))
        scratch.mul_(1.0001)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), rep

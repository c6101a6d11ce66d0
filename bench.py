#!/usr/bin/env python3
"""Benchmark one paged-attention decode step on one MI355X.

A step is the whole hot path over one batch: paged_kv_write of the step's new K/V rows, then
paged_attn_decode (split-K), then paged_attn_reduce.  Inputs are seeded synthetic tensors
already resident in HBM.  To keep steps honest about HBM (the 256 MB Infinity Cache would
otherwise hold part of a 0.6 GB cache between steps), the step rotates over several copies of
the KV pools, so each step reads pools the previous steps did not touch.

Prints one JSON line: whole-step KV GB/s as `value`, plus decode tokens/s, the decode
kernel's roofline (algorithmic bytes per launch / its mean duration, from HIP events bound to
the kernel's own dispatch on every timed step) and the fp64 CPU oracle timed on this host's
cores (all of them, and one thread).
"""
import argparse
import ctypes
import dataclasses
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import paged_kv_cache_224_amd as pk  # noqa: E402
from paged_kv_cache_224_amd import inputs as I  # noqa: E402

METRIC = "paged decode KV GB/s and % of HBM peak; decode tokens/s, 1 MI355X"
HBM_PEAK_GBPS = 8000.0          # MI355X published HBM3E bandwidth


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama3_8b", choices=I.CONFIG_ORDER)
    ap.add_argument("--schedule", default="balanced", choices=["balanced", "fixed", "single", "shared_prefix"],
                    help="balanced split-K (default), fixed 512-token partitions, single pass, or the "
                         "shared-prefix decode (prefix pass + balanced suffix + merge in one call)")
    ap.add_argument("--partition-size", type=int, default=None,
                    help="explicit partition_size (overrides --schedule; <0 = balanced over -N workgroups)")
    ap.add_argument("--prefix-partition-size", type=int, default=None,
                    help="shared_prefix schedule: prefix tokens per partition (default: one workgroup per CU)")
    ap.add_argument("--kv-dtype", default=None, choices=["bf16", "f16", "fp8"],
                    help="run the workload's shapes with this cache dtype instead of its own (the query "
                         "dtype stays); the workload is then named <workload>:kv=<dtype>")
    ap.add_argument("--copies", type=int, default=None, help="pool copies to rotate over")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--append", action="store_true",
                    help="16-bit caches, balanced schedule: run the step's KV write inside the decode launch "
                         "(paged_attn_decode_append) instead of paged_kv_write + paged_attn_decode")
    ap.add_argument("--event-every", type=int, default=1,
                    help="time the decode launch with HIP events on every N-th timed step (default: all)")
    ap.add_argument("--event-mode", default="kernel", choices=["kernel", "marker"],
                    help="kernel: timing-only events bound to the call's kernels (pkv_time_next_call, no "
                         "packet between kernels); marker: default events recorded on the stream around the call")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="minimum oracle time to measure")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step replayed from HIP graphs (one per pool copy)")
    ap.add_argument("--op", default="decode", choices=["decode", "copy_blocks", "swap", "multi_query", "graphs"],
                    help="decode: the decode step (default); copy_blocks / swap: the whole-block operations "
                         "on a pool of the workload's block shape")
    ap.add_argument("--pairs", type=int, default=4096, help="block pairs per copy_blocks / swap call")
    ap.add_argument("--q-len", type=int, default=4, help="new tokens per sequence for --op multi_query")
    ap.add_argument("--copy-reference", type=int, default=0, metavar="MiB",
                    help="only copy a buffer of this size 5 times (reference for HBM traffic counters)")
    return ap.parse_args()


class HipEvents:
    """Timing-only HIP events created with hipEventDisableSystemFence: recording one skips the
    system-scope cache write-back a default event performs, so timing every launch does not
    slow the work that follows (a default event costs ~5 us per timed decode launch here)."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.pairs = []
        for _ in range(n):
            pair = []
            for _ in range(2):
                h = ctypes.c_void_p()
                rc = self.hip.hipEventCreateWithFlags(ctypes.byref(h), self.DISABLE_SYSTEM_FENCE)
                if rc != 0:
                    raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
                pair.append(h.value)
            self.pairs.append(tuple(pair))

    def elapsed_ms(self, pair):
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(pair[0]), ctypes.c_void_p(pair[1]))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def close(self):
        for pair in self.pairs:
            for h in pair:
                self.hip.hipEventDestroy(ctypes.c_void_p(h))
        self.pairs = []


def workload_cfg(args):
    """The workload's configuration, with the cache dtype of --kv-dtype if given."""
    cfg = I.CONFIGS[args.workload]
    if args.kv_dtype and args.kv_dtype != cfg.kv_dtype:
        cfg = dataclasses.replace(cfg, kv_dtype=args.kv_dtype, name=f"{cfg.name}:kv={args.kv_dtype}")
    return cfg


def copy_gbps(mib=1024, reps=10):
    """Read + write GB/s of a plain device-to-device copy of mib MiB (HIP events around the
    copies): a second yardstick beside the 8 TB/s peak, measured on the same GPU."""
    n = mib * 2 ** 20 // 4
    a = torch.ones(n, dtype=torch.int32, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    dt = e0.elapsed_time(e1) * 1e-3 / reps
    del a, b
    return 2 * mib * 2 ** 20 / dt / 1e9


def copy_reference(mib):
    """Plain device-to-device copies of a known size: the HBM counters of this kernel calibrate
    FETCH_SIZE / WRITE_SIZE (each copy reads and writes exactly mib MiB)."""
    n = mib * 2 ** 20 // 4
    a = torch.ones(n, dtype=torch.int32, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / 5
    print(json.dumps({"copy_reference_mib": mib, "ms": round(dt * 1e3, 4),
                      "read_plus_write_gbps": round(2 * mib * 2 ** 20 / dt / 1e9, 1)}), flush=True)


def measured_traffic(workload, schedule):
    """HBM bytes per decode launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE summary of
    this workload, or None if there is none or the kernel code changed since it was taken."""
    from paged_kv_cache_224_amd.profile_summary import source_hash
    path = os.path.join(ROOT, "profiles", f"pa_decode_{workload}_traffic.json")
    if schedule != "balanced" or not os.path.exists(path):
        return None
    rec = json.load(open(path))
    return int(rec["decode_traffic_bytes"]) if rec.get("kernel_source_sha256_16") == source_hash() else None


def decode_bytes(w):
    """Algorithmic bytes of one decode call: KV rows of every (sequence, token) once, the query
    and output rows, the used block-table entries and the context lengths (logical and
    unique-block counts).  The output row is counted although in the split-K schedules the
    merge launch, not the decode launch, writes it; the difference is 0.09% on the Llama-3-8B
    layer."""
    nb = I.algorithmic_bytes(w)
    return nb["decode_logical"], nb["decode_unique"], nb


def cpu_baseline(w, min_seconds, threads=None, max_reps=50):
    """fp64 oracle (KV write + attention over the whole batch) on this host's cores (all of
    them unless `threads` is given)."""
    import oracle
    threads = threads or len(os.sched_getaffinity(0))
    kvdt = "fp8" if w.cfg.kv_dtype == "fp8" else None
    if kvdt:
        kc = oracle.quantize_pool(w.k_pool, w.k_scale)
        vc = oracle.quantize_pool(w.v_pool, w.v_scale)
    else:
        kc, vc = w.k_pool.clone(), w.v_pool.clone()
    reps, t_total = 0, 0.0
    while t_total < min_seconds or reps == 0:
        t0 = time.perf_counter()
        oracle.kv_write(w.k_new, w.v_new, kc, vc, w.slot_mapping, w.k_scale, w.v_scale)
        oracle.attn(w.q, kc, vc, w.block_tables, w.context_lens, w.scale, w.k_scale, w.v_scale, kvdt,
                    nthreads=threads)
        t_total += time.perf_counter() - t0
        reps += 1
        if reps >= max_reps:
            break
    t = t_total / reps
    return t, threads, reps


def block_ops(args):
    """Whole-block operations on pools of the workload's block shape: copy-on-write copies
    (HBM, read + write) or swap out to / in from pinned host memory (host link)."""
    cfg = workload_cfg(args)
    dev = torch.device("cuda:0")
    fp8 = cfg.kv_dtype == "fp8"
    dt = torch.uint8 if fp8 else I.DTYPES[cfg.kv_dtype]
    n = args.pairs
    NB = 2 * n + 16
    shape = (NB, cfg.block_size, cfg.Hkv, cfg.D)
    kc = torch.zeros(shape, dtype=dt, device=dev)
    vc = torch.zeros_like(kc)
    block_bytes = cfg.block_size * cfg.Hkv * cfg.D * (1 if fp8 else 2)
    rng = np.random.default_rng(0)
    perm = rng.permutation(NB).astype(np.int32)
    a = torch.from_numpy(perm[:n].copy()).to(dev)
    b = torch.from_numpy(perm[n:2 * n].copy()).to(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    res = {"n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "fp8" if fp8 else cfg.kv_dtype, "data": "synthetic",
           "config": {"workload": f"{cfg.name} block shape", "op": args.op, "pairs": n, "block_bytes": block_bytes,
                      "pools": 2}}
    if args.op == "copy_blocks":
        def run():
            pk.paged_kv_copy_blocks(kc, vc, a, b)
        moved = 2 * 2 * n * block_bytes                 # read + write, K and V
        for _ in range(args.warmup):
            run()
        torch.cuda.synchronize()
        for e in ev:
            e[0].record()
            run()
            e[1].record()
        torch.cuda.synchronize()
        t = float(np.mean([e[0].elapsed_time(e[1]) for e in ev])) * 1e-3
        gbps = moved / t / 1e9
        res.update({"metric": "copy_blocks HBM GB/s (read + write)", "value": round(gbps, 1), "unit": "GB/s",
                    "ms_per_step": round(t * 1e3, 4),
                    "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                 "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                                 "kernel": "copy_blocks_kernel", "bytes_per_launch": moved}})
    else:
        NH = n + 16
        hk = torch.zeros((NH,) + shape[1:], dtype=dt, pin_memory=True)
        hv = torch.zeros((NH,) + shape[1:], dtype=dt, pin_memory=True)
        hid = torch.from_numpy(rng.permutation(NH)[:n].astype(np.int32)).to(dev)
        moved = 2 * n * block_bytes                     # K and V blocks across the link, one way
        out = {}
        for direction in ("out", "in"):
            def run():
                pk.paged_kv_swap_blocks(kc, vc, hk, hv, a, hid, to_host=direction == "out")
            for _ in range(args.warmup):
                run()
            torch.cuda.synchronize()
            for e in ev:
                e[0].record()
                run()
                e[1].record()
            torch.cuda.synchronize()
            out[direction] = float(np.mean([e[0].elapsed_time(e[1]) for e in ev])) * 1e-3
        # reference: one contiguous pinned <-> device copy of the same bytes (DMA engines)
        flat_d = torch.empty(moved, dtype=torch.uint8, device=dev)
        flat_h = torch.empty(moved, dtype=torch.uint8, pin_memory=True)
        ref = {}
        for direction in ("out", "in"):
            for _ in range(2):
                (flat_h.copy_(flat_d, non_blocking=True) if direction == "out" else flat_d.copy_(flat_h, non_blocking=True))
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(5):
                (flat_h.copy_(flat_d, non_blocking=True) if direction == "out" else flat_d.copy_(flat_h, non_blocking=True))
            torch.cuda.synchronize()
            ref[direction] = (time.perf_counter() - t0) / 5
        g_out, g_in = moved / out["out"] / 1e9, moved / out["in"] / 1e9
        r_out, r_in = moved / ref["out"] / 1e9, moved / ref["in"] / 1e9
        res.update({"metric": "block swap GB/s over the host link (out = device to host)",
                    "value": round(min(g_out, g_in), 2), "unit": "GB/s",
                    "ms_per_step": round((out["out"] + out["in"]) * 1e3, 4),
                    "swap_out_gbps": round(g_out, 2), "swap_in_gbps": round(g_in, 2),
                    "contiguous_dma_copy_gbps": {"out": round(r_out, 2), "in": round(r_in, 2)},
                    "roofline": {"bound": "host link", "achieved": round(min(g_out, g_in), 2),
                                 "peak": round(min(r_out, r_in), 2), "unit": "GB/s",
                                 "frac": round(min(g_out / r_out, g_in / r_in), 4), "traffic": None,
                                 "kernel": "swap_blocks_kernel", "bytes_per_launch": moved,
                                 "peak_is": "contiguous pinned<->device copy of the same bytes, measured"}})
    print(json.dumps(res), flush=True)


def device_pools(w, dev, copies=None):
    """Copies of the workload's pools on the device (fp8 pools quantised by paged_kv_write),
    enough of them that a rotation over them never finds its pool in the 256 MB Infinity Cache."""
    cfg = w.cfg
    fp8 = cfg.kv_dtype == "fp8"
    NB, BS, D = w.num_blocks, cfg.block_size, cfg.D
    pool_bytes = 2 * NB * BS * cfg.Hkv * D * (1 if fp8 else 2)
    copies = copies or max(2, math.ceil(1.5 * 2 ** 30 / pool_bytes) + 1)
    pools = []
    ksrc = w.k_pool.to(dev)
    vsrc = w.v_pool.to(dev)
    for _ in range(copies):
        if fp8:
            kc = torch.empty((NB, BS, cfg.Hkv, D), dtype=torch.uint8, device=dev)
            vc = torch.empty_like(kc)
            slots = torch.arange(NB * BS, dtype=torch.int64, device=dev)
            pk.paged_kv_write(ksrc.view(NB * BS, cfg.Hkv, D), vsrc.view(NB * BS, cfg.Hkv, D), kc, vc, slots,
                              w.k_scale, w.v_scale)
        else:
            kc, vc = ksrc.clone(), vsrc.clone()
        pools.append((kc, vc))
    return pools, copies


def multi_query_op(args):
    """L new tokens per sequence (speculative verification / chunked prefill) on the workload's
    batch, balanced split of paged_attn_multi_query_split(): the attention call timed by
    kernel-bound events on every step, the whole step (attention + merge) by wall clock.
    Algorithmic bytes: the KV rows once (shared by the L tokens), L query rows and L output rows
    per (sequence, head), the used table entries and lengths.  Flops: 4 * D per (query row,
    visible token), QK^T and PV; new token i of a sequence sees n - L + 1 + i tokens."""
    dev = torch.device("cuda:0")
    cfg = workload_cfg(args)
    L = args.q_len
    w = I.make_workload(cfg)
    fp8 = cfg.kv_dtype == "fp8"
    pools, copies = device_pools(w, dev, args.copies)
    q = I.multi_query_q(cfg, L, 0).to(dev)
    bt = torch.from_numpy(w.block_tables).to(dev)
    lens = torch.from_numpy(w.context_lens).to(dev)
    kvdt = torch.uint8 if fp8 else I.DTYPES[cfg.kv_dtype]
    PS = args.partition_size if args.partition_size is not None else \
        pk.multi_query_split(cfg.Hq, cfg.Hkv, cfg.D, L, I.DTYPES[cfg.q_dtype], kvdt)
    ws = pk.DecodeWorkspace(cfg.B, L * cfg.Hq, cfg.D, cfg.max_len, PS, device=dev)
    out = torch.empty((cfg.B, L, cfg.Hq, cfg.D), dtype=I.DTYPES[cfg.q_dtype], device=dev)
    shared = bool(w.prefix_blocks.size)                 # tables share a common prefix's blocks
    calls = [pk.paged_attn_multi_query(None if PS else out, q, kc, vc, bt, lens, w.scale, cfg.max_len, PS,
                                       ws.tmp_out, ws.max_logits, ws.exp_sums, w.k_scale, w.v_scale,
                                       shared_blocks=shared, bind=True) for kc, vc in pools]
    merge = pk.paged_attn_reduce(out.view(cfg.B, L * cfg.Hq, cfg.D), ws.tmp_out, ws.max_logits, ws.exp_sums,
                                 lens, cfg.max_len, PS, bind=True) if PS else None
    hev = HipEvents(args.steps)

    def run(i, e=None):
        if e is not None:
            pk.time_next_call(e[0], e[1])
        calls[i % copies]()
        if merge is not None:
            merge()

    for i in range(args.warmup):
        run(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        run(i, hev.pairs[i])
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps
    kern_ms = [hev.elapsed_ms(p) for p in hev.pairs]
    hev.close()
    kern = float(np.mean(kern_ms)) * 1e-3
    nb = I.algorithmic_bytes(w)
    e_q = 2
    moved = nb["kv_unique"] + 2 * L * cfg.B * cfg.Hq * cfg.D * e_q + 4 * int(w.blocks_used.sum()) + 4 * cfg.B
    n = w.context_lens.astype(np.int64)
    visible = sum(int(np.clip(n - L + 1 + i, 0, None).sum()) for i in range(L))
    flops = 4 * cfg.D * cfg.Hq * visible
    gbps = moved / kern / 1e9
    tflops = flops / kern / 1e12
    mfma_peak = 2500.0                                  # dense bf16 / f16 MFMA, TFLOP/s
    hbm_frac, mfma_frac = gbps / HBM_PEAK_GBPS, tflops / mfma_peak
    tiled = cfg.group * L > 32
    res = {"metric": "multi-query paged attention KV GB/s and query tokens/s", "value": round(gbps, 1),
           "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(wall * 1e3, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "fp8" if fp8 else cfg.kv_dtype, "data": "synthetic",
           "config": {"workload": cfg.name, "q_len": L, "num_seqs": cfg.B, "num_heads": cfg.Hq,
                      "num_kv_heads": cfg.Hkv, "head_dim": cfg.D, "partition_size": PS},
           "query_tokens_per_s": round(cfg.B * L / wall, 1), "kernel_ms_mean": round(kern * 1e3, 5),
           "kernel_ms_median": round(float(np.median(kern_ms)), 5), "kernel_samples": len(kern_ms),
           "tflops": round(tflops, 1), "flops_per_launch": flops,
           "roofline": {"bound": "hbm" if hbm_frac >= mfma_frac else "mfma",
                        "achieved": round(gbps if hbm_frac >= mfma_frac else tflops, 1),
                        "peak": HBM_PEAK_GBPS if hbm_frac >= mfma_frac else mfma_peak,
                        "unit": "GB/s" if hbm_frac >= mfma_frac else "TFLOP/s",
                        "frac": round(max(hbm_frac, mfma_frac), 4), "hbm_frac": round(hbm_frac, 4),
                        "mfma_frac": round(mfma_frac, 4), "traffic": None,
                        "kernel": "pa_mq_tiled_kernel" if tiled else ("pa_decode_kernel, two column tiles per wave" if cfg.group * L > 16 else "pa_decode_kernel"),
                        "bytes_per_launch": moved}}
    print(json.dumps(res), flush=True)


def graphs_op(args):
    """Step time (write -> decode -> reduce) eager and as the replay of the smallest captured HIP
    graph that fits, for several batch sizes of the workload's shapes (the first B sequences)."""
    from paged_kv_cache_224_amd.graphs import StepGraphs
    dev = torch.device("cuda:0")
    cfg = workload_cfg(args)
    w = I.make_workload(cfg)
    fp8 = cfg.kv_dtype == "fp8"
    pools, _ = device_pools(w, dev, 1)
    kc, vc = pools[0]
    sizes = [1 << i for i in range(0, 12) if (1 << (i - 1) if i else 0) < cfg.B]
    g = StepGraphs(kc, vc, cfg.Hq, cfg.max_blocks, cfg.max_len, I.DTYPES[cfg.q_dtype], sizes,
                   k_scale=w.k_scale, v_scale=w.v_scale)
    rows = []
    for B in sorted({1, 4, 16, cfg.B} & set(range(1, cfg.B + 1))):
        q, kn, vn, sl, bt, ln = g.inputs(B)
        q.copy_(w.q[:B])
        kn.copy_(w.k_new[:B])
        vn.copy_(w.v_new[:B])
        sl.copy_(torch.from_numpy(w.slot_mapping[:B]))
        bt.copy_(torch.from_numpy(w.block_tables[:B]))
        ln.copy_(torch.from_numpy(w.context_lens[:B]))
        times = {}
        for mode in ("eager", "graph"):
            run = (lambda: g._step(B)) if mode == "eager" else (lambda: g.replay(B))
            for _ in range(args.warmup):
                run()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(args.steps):
                run()
            torch.cuda.synchronize()
            times[mode] = 1e6 * (time.perf_counter() - t0) / args.steps
        rows.append({"batch": B, "captured_size": g.size_for(B), "eager_us": round(times["eager"], 2),
                     "graph_us": round(times["graph"], 2),
                     "step_time_saved": round(1 - times["graph"] / times["eager"], 4)})
        print(f"[bench] graphs B={B}: eager {times['eager']:.1f} us, graph {times['graph']:.1f} us",
              file=sys.stderr, flush=True)
    print(json.dumps({"metric": "decode step time, eager calls vs replay of the smallest captured HIP graph",
                      "unit": "us", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                      "higher_is_better": False, "data": "synthetic", "dtype": "fp8" if fp8 else cfg.kv_dtype,
                      "config": {"workload": cfg.name, "captured_sizes": sizes,
                                 "partition_size": g.partition_size}, "rows": rows}), flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} (WORLD_SIZE={world}) is not supported: "
              "the paged decode path here has no multi-GPU mode.", file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_reference:
        copy_reference(args.copy_reference)
        return
    if args.op == "multi_query":
        multi_query_op(args)
        return
    if args.op == "graphs":
        graphs_op(args)
        return
    if args.op != "decode":
        block_ops(args)
        return
    dev = torch.device("cuda:0")
    cfg = workload_cfg(args)
    if args.partition_size is not None:
        PS = args.partition_size
    elif args.schedule in ("balanced", "shared_prefix"):
        PS = pk.balanced_split(cfg.Hkv, cfg.D, I.DTYPES[cfg.q_dtype],
                               torch.uint8 if cfg.kv_dtype == "fp8" else I.DTYPES[cfg.kv_dtype])
    elif args.schedule == "fixed":
        PS = cfg.partition_size
    else:
        PS = 0
    schedule = "single" if PS == 0 else ("fixed" if PS > 0 else "balanced")
    cascade = args.schedule == "shared_prefix"
    if cascade:
        schedule = "shared_prefix"
    print(f"[bench] generating {cfg.name}", file=sys.stderr, flush=True)
    w = I.make_workload(cfg)
    B, Hq, D = cfg.B, cfg.Hq, cfg.D
    fp8 = cfg.kv_dtype == "fp8"

    # ---- device-resident inputs
    NB, BS = w.num_blocks, cfg.block_size
    pools, copies = device_pools(w, dev, args.copies)
    q = w.q.to(dev)
    k_new, v_new = w.k_new.to(dev), w.v_new.to(dev)
    slots = torch.from_numpy(w.slot_mapping).to(dev)
    bt = torch.from_numpy(w.block_tables).to(dev)
    lens = torch.from_numpy(w.context_lens).to(dev)
    maxlen = cfg.max_len
    ws = pk.DecodeWorkspace(B, Hq, D, maxlen, PS, device=dev)
    out = torch.empty((B, Hq, D), dtype=I.DTYPES[cfg.q_dtype], device=dev)
    shared = bool(w.prefix_blocks.size)                 # tables share a common prefix's blocks
    prefix_len = int(w.prefix_blocks.size) * BS
    # --append (16-bit caches, balanced schedule): the step's KV write rides in the decode launch
    append = args.append and not fp8 and schedule == "balanced" and args.partition_size is None
    if cascade:
        # the prefix pass reads the shared blocks; the suffix pass streams private blocks
        sws = pk.SharedPrefixWorkspace(B, Hq, cfg.Hkv, D, maxlen, prefix_len, PS, args.prefix_partition_size,
                                       device=dev)
        shared = False
    torch.cuda.synchronize()

    marker = args.event_mode == "marker"
    # Every call of the step is prepared once per pool copy (arguments validated and converted
    # to C values by the binding), so the timed loop only makes the library calls.
    def make_calls(kc, vc):
        """The step's calls on one pool copy, prepared for the current stream."""
        c = {}
        if append:                                      # write + decode in one launch, then the merge
            c["attn"] = pk.paged_attn_decode_append(None, q, k_new, v_new, kc, vc, bt, lens, w.scale, maxlen, PS,
                                                    ws.tmp_out, ws.max_logits, ws.exp_sums, shared_blocks=shared,
                                                    bind=True)
        else:
            c["write"] = pk.paged_kv_write(k_new, v_new, kc, vc, slots, w.k_scale, w.v_scale, bind=True)
            if cascade:                                 # three kernels: prefix, suffix, merge
                c["attn"] = pk.decode_shared_prefix(out, q, kc, vc, bt, lens, w.scale, sws, w.k_scale, w.v_scale,
                                                    bind=True)
            else:
                c["attn"] = pk.paged_attn_decode(out if PS == 0 else None, q, kc, vc, bt, lens, w.scale, maxlen, PS,
                                                 ws.tmp_out, ws.max_logits, ws.exp_sums, w.k_scale, w.v_scale,
                                                 shared_blocks=shared, bind=True)
        if PS != 0 and not cascade:
            c["reduce"] = pk.paged_attn_reduce(out, ws.tmp_out, ws.max_logits, ws.exp_sums, lens, maxlen, PS,
                                               bind=True)
        return c

    calls = [make_calls(kc, vc) for kc, vc in pools]

    def run_calls(c, ev=None):
        if "write" in c:
            c["write"]()
        if ev is not None:
            if marker:
                ev[0].record()
            else:
                pk.time_next_call(ev[0], ev[1])
        c["attn"]()
        if ev is not None and marker:
            ev[1].record()
        if "reduce" in c:
            c["reduce"]()

    def step(i, ev=None):
        run_calls(calls[i % copies], ev)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # ---- timed region: exactly K steps, synchronised on both sides
    # HIP events time the decode call on every event_every-th timed step.  By default they are
    # bound to the call's kernels (recorded at the first kernel's start and the last kernel's
    # end), so no marker packet sits between two kernels of the step and the step rate is not
    # disturbed; --event-mode marker records them on the stream around the call instead.
    every = max(1, args.event_every)
    nsamp = (args.steps + every - 1) // every
    if marker:
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) if i % every == 0
               else None for i in range(args.steps)]
        elapsed = lambda e: e[0].elapsed_time(e[1])     # noqa: E731
    else:
        hip_events = HipEvents(nsamp)
        it = iter(hip_events.pairs)
        evs = [next(it) if i % every == 0 else None for i in range(args.steps)]
        elapsed = hip_events.elapsed_ms
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    decode_ms = [elapsed(e) for e in evs if e is not None]
    if not marker:
        hip_events.close()

    ms_per_step = 1e3 * wall / args.steps

    ms_graph = None
    if args.graph:
        # capture one step per pool copy; replay them in the same rotation
        graphs = []
        cap_stream = torch.cuda.Stream()
        for c in range(copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap_stream):
                run_calls(make_calls(*pools[c]))
            graphs.append(g)
        for i in range(args.warmup):
            graphs[i % copies].replay()
        torch.cuda.synchronize()
        tg = time.perf_counter()
        for i in range(args.steps):
            graphs[i % copies].replay()
        torch.cuda.synchronize()
        ms_graph = 1e3 * (time.perf_counter() - tg) / args.steps

    dec_logical, dec_unique, nb = decode_bytes(w)
    step_bytes_unique = nb["decode_unique"] + nb["write"]
    step_bytes_logical = nb["decode_logical"] + nb["write"]
    value = step_bytes_unique / (ms_per_step * 1e-3) / 1e9
    dec_mean_ms = float(np.mean(decode_ms))
    dec_median_ms = float(np.median(decode_ms))
    if append:                                          # the timed launch also moves the new rows
        dec_unique += nb["write"]
    achieved = dec_unique / (dec_mean_ms * 1e-3) / 1e9
    tokens_per_s = B / (ms_per_step * 1e-3)

    res = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8" if fp8 else cfg.kv_dtype,
        "data": "synthetic",
        "config": {
            "workload": cfg.name, "num_seqs": B, "num_heads": Hq, "num_kv_heads": cfg.Hkv, "head_dim": D,
            "block_size": BS, "context_lens": list(cfg.lens), "sum_context": int(w.context_lens.sum()),
            "kv_dtype": cfg.kv_dtype, "q_dtype": cfg.q_dtype, "schedule": schedule, "partition_size": PS,
            "new_tokens": B, "kv_load_policy": "cached" if shared else "streaming",
            "kv_write": "in the decode launch" if append else "separate launch",
            **({"prefix_len": prefix_len, "prefix_partition_size": sws.prefix_partition_size} if cascade else {}),
            "num_blocks": NB, "pool_copies_rotated": copies,
        },
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBPS, 2),
        "ms_per_step_graph": None if ms_graph is None else round(ms_graph, 4),
        "tokens_per_s": round(tokens_per_s, 1),
        "decode_kernel_ms_mean": round(dec_mean_ms, 5),
        "decode_kernel_ms_median": round(dec_median_ms, 5),
        "decode_event_samples": len(decode_ms),
        "decode_event_mode": ("timing-only events bound to the kernels (hipExtLaunchKernel)" if not marker
                              else "default events recorded around the call"),
        "decode_kernel_ms_p10_p50_p90": [round(float(x), 5) for x in np.percentile(decode_ms, [10, 50, 90])],
        "step_bytes": {"logical": step_bytes_logical, "unique": step_bytes_unique},
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "frac_at_median": round(dec_unique / (dec_median_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "samples": len(decode_ms),
            "traffic": measured_traffic(cfg.name, schedule),
            "kernel": ("pa_prefix_kernel + pa_decode_kernel + pa_reduce_kernel (one call, timed together)"
                       if cascade else ("pa_decode_kernel with the step's KV write appended" if append
                                        else "pa_decode_kernel")),
            "bytes_per_launch": dec_unique,
        },
    }
    if w.prefix_blocks.size:
        res["logical_gbps"] = round(step_bytes_logical / (ms_per_step * 1e-3) / 1e9, 1)
    # second yardstick: a plain 1 GiB device copy measured on the same GPU (after the timed region)
    cg = copy_gbps()
    res["copy_reference"] = {"copy_read_plus_write_gbps": round(cg, 1), "decode_frac_of_copy": round(achieved / cg, 4)}

    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        t_cpu, threads, reps = cpu_baseline(w, args.cpu_seconds)
        res["cpu_baseline"] = {
            "value": round(step_bytes_unique / t_cpu / 1e9, 3),
            "unit": "GB/s",
            "cores": threads,
            "kind": "oracle",
            "sample": f"whole {cfg.name} batch ({B} sequences): fp64 KV write + attention, mean of {reps} runs "
                      f"({t_cpu:.3f} s each)",
            "tokens_per_s": round(B / t_cpu, 2),
        }
        # the same oracle on one thread: this workload (one pass) and the tiny workload
        one = {}
        for wl in (w, I.make_workload(I.CONFIGS["tiny"])):
            t1, _, r1 = cpu_baseline(wl, 0.0 if wl is w else 1.0, threads=1, max_reps=1 if wl is w else 50)
            ab = I.algorithmic_bytes(wl)
            one[wl.cfg.name] = {"seconds": round(t1, 4), "runs": r1, "tokens_per_s": round(wl.cfg.B / t1, 2),
                                "gbps": round((ab["decode_unique"] + ab["write"]) / t1 / 1e9, 4)}
        res["cpu_baseline"]["one_thread"] = {"cores": 1, **one}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

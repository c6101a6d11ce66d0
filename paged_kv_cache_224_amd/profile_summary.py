"""Turn rocprofv3 output of the benchmark into the short summaries kept under profiles/.

Usage (from the repository root, after the commands that ``commands()`` lists have written
their CSV files under OUT on an MI355X):

    python -m paged_kv_cache_224_amd.profile_summary OUT WORKLOAD [SCHEDULE]

writes profiles/pa_decode_<WORKLOAD>.md (kernel statistics, HBM counters scaled by a plain
device copy of known size, the benchmark line) and profiles/pa_decode_<WORKLOAD>_traffic.json
(measured HBM bytes per decode launch, keyed by the kernel source hash; bench.py reports it as
``roofline.traffic`` while the source is unchanged).  With SCHEDULE shared_prefix it writes
profiles/pa_shared_prefix_<WORKLOAD>.md instead (the prefix pass, the suffix decode and the
merge of one call).  Reads CSV and JSON text only.
"""
from __future__ import annotations

import collections
import csv
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "paged_kv_cache_224_amd", "csrc", "pagedkv.hip")
COPY_MIB = 1024


def source_hash(path: str = SRC) -> str:
    """sha256[:16] of the kernel source's code: // comments, trailing blanks and empty lines
    are dropped first, so editing a comment keeps the recorded measurements."""
    code = []
    for line in open(path, encoding="utf-8").read().splitlines():
        cut = line.find("//")
        if cut >= 0:
            line = line[:cut]
        line = line.rstrip()
        if line:
            code.append(line)
    return hashlib.sha256("\n".join(code).encode()).hexdigest()[:16]


def commands(workload: str, schedule: str, out: str = "OUT") -> list:
    """The profiling commands whose output summarize() reads (run from the repository root)."""
    b = f"python -u bench.py --workload {workload} --schedule {schedule} --no-cpu-baseline"
    return [
        f"python -u bench.py --workload {workload} --schedule {schedule} --no-cpu-baseline > {out}/bench.json",
        f"rocprofv3 --kernel-trace --stats --output-format csv -d {out}/kt -o run -- {b}",
        f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {out}/fetch -o run -- {b} --steps 10 --warmup 3",
        f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {out}/write -o run -- {b} --steps 10 --warmup 3",
        f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {out}/copyf -o run -- python -u bench.py "
        f"--copy-reference {COPY_MIB}",
        f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {out}/copyw -o run -- python -u bench.py "
        f"--copy-reference {COPY_MIB}",
    ]


def _counter(path: str, name: str) -> dict:
    acc = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == name:
            acc[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def summarize(out: str, workload: str, schedule: str = "balanced") -> str:
    ks = list(csv.DictReader(open(os.path.join(out, "kt", "run_kernel_stats.csv"))))
    fetch = _counter(os.path.join(out, "fetch", "run_counter_collection.csv"), "FETCH_SIZE")
    write = _counter(os.path.join(out, "write", "run_counter_collection.csv"), "WRITE_SIZE")
    cf = _counter(os.path.join(out, "copyf", "run_counter_collection.csv"), "FETCH_SIZE")
    cw = _counter(os.path.join(out, "copyw", "run_counter_collection.csv"), "WRITE_SIZE")
    copy_name = [k for k in cf if "copyBuffer" in k][0]
    true_kib = COPY_MIB * 1024
    ff, wf = true_kib / cf[copy_name], true_kib / cw[copy_name]
    bench = json.loads(open(os.path.join(out, "bench.json")).read().strip().splitlines()[-1])
    h = source_hash()

    lines = [f"# {workload}: rocprofv3 summary of the benchmark step ({schedule} schedule)", "",
             f"Kernel source sha256[:16] = `{h}` (paged_kv_cache_224_amd/csrc/pagedkv.hip without comments)", "",
             "## Commands (run from the repository root on one MI355X; OUT is any scratch folder)", "",
             "```"] + commands(workload, schedule) + [
             f"python -m paged_kv_cache_224_amd.profile_summary OUT {workload} {schedule}", "```", "",
             "## Kernel statistics (--kernel-trace --stats)", "",
             "| kernel | calls | average ns | min ns | max ns |", "|---|---|---|---|---|"]
    for r in ks:
        lines.append(f"| {r['Name'][:90]} | {r['Calls']} | {float(r['AverageNs']):.0f} | {r['MinNs']} | "
                     f"{r['MaxNs']} |")
    lines += ["", "## HBM counters (KiB per dispatch, mean over dispatches)", "",
              f"Calibration: a {COPY_MIB} MiB device copy reads {cf[copy_name]:.0f} KiB by FETCH_SIZE and writes "
              f"{cw[copy_name]:.0f} KiB by WRITE_SIZE, so FETCH_SIZE is scaled by {ff:.3f} and WRITE_SIZE by "
              f"{wf:.3f}.", "",
              "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | read bytes (scaled) | written bytes (scaled) |",
              "|---|---|---|---|---|"]
    scaled = {}
    for k in sorted(set(fetch) | set(write)):
        if "copyBuffer" in k or "elementwise" in k or "fill" in k:
            continue
        f, w = fetch.get(k, 0.0), write.get(k, 0.0)
        rb, wb = f * ff * 1024, w * wf * 1024
        scaled[k] = (rb, wb)
        lines.append(f"| {k[:90]} | {f:.1f} | {w:.1f} | {rb / 1e6:.2f} MB | {wb / 1e6:.2f} MB |")
    alg = bench["roofline"]["bytes_per_launch"]
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    if schedule == "shared_prefix":
        # three kernels per call: prefix pass, suffix decode, merge
        parts, tr = [], 0.0
        tot = 0.0
        for tag in ("prefix", "decode", "reduce"):
            k = [x for x in scaled if tag in x][0]
            t = [float(r["AverageNs"]) for r in ks if tag in r["Name"]][0]
            rb, wb = scaled[k]
            tot += rb + wb
            tr += t
            parts.append(f"{tag} {(rb + wb) / 1e6:.2f} MB in {t / 1e3:.1f} us")
        lines += ["", f"Shared-prefix call: {', '.join(parts)}; together {tot / 1e6:.2f} MB of HBM traffic "
                      f"against {alg / 1e6:.2f} MB algorithmic (unique) bytes.  Kernel-trace sum {tr / 1e3:.1f} us "
                      f"= {alg / tr:.0f} GB/s algorithmic; the benchmark's HIP events around the call give "
                      f"{bench['decode_kernel_ms_mean'] * 1e3:.1f} us.", "",
                  "## Benchmark line of the same build", "", "```json", json.dumps(bench), "```", ""]
        text = "\n".join(lines)
        with open(os.path.join(ROOT, "profiles", f"pa_shared_prefix_{workload}.md"), "w") as fh:
            fh.write(text)
        return text
    dk = [k for k in scaled if "decode" in k][0]
    rb, wb = scaled[dk]
    trace_avg = [float(r["AverageNs"]) for r in ks if "decode" in r["Name"]][0]
    lines += ["", f"Decode kernel: HBM traffic {(rb + wb) / 1e6:.2f} MB per launch (read {rb / 1e6:.2f} + "
                  f"written {wb / 1e6:.2f}) against {alg / 1e6:.2f} MB algorithmic bytes "
                  f"({(rb + wb) / alg:.3f}x).  Kernel-trace average {trace_avg / 1e3:.1f} us = "
                  f"{alg / trace_avg:.0f} GB/s algorithmic; the benchmark's HIP events give "
                  f"{bench['decode_kernel_ms_mean'] * 1e3:.1f} us.", "",
              "## Benchmark line of the same build", "", "```json", json.dumps(bench), "```", ""]
    text = "\n".join(lines)
    with open(os.path.join(ROOT, "profiles", f"pa_decode_{workload}.md"), "w") as fh:
        fh.write(text)
    with open(os.path.join(ROOT, "profiles", f"pa_decode_{workload}_traffic.json"), "w") as fh:
        json.dump({"kernel_source_sha256_16": h, "workload": workload, "schedule": schedule,
                   "decode_traffic_bytes": rb + wb, "decode_read_bytes": rb, "decode_write_bytes": wb,
                   "fetch_scale": ff, "write_scale": wf, "trace_average_ns": trace_avg}, fh, indent=1)
    return text


# Core counters of one pass (at most 8 SQ and 2 GRBM counters fit in one rocprofv3 pass).
SQ_COUNTERS = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES", "SQ_INSTS_MFMA", "SQ_INSTS_VALU", "SQ_INSTS_LDS",
               "SQ_LDS_BANK_CONFLICT", "SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES", "GRBM_GUI_ACTIVE"]


OUR_KERNELS = ("pa_decode", "pa_prefix", "pa_reduce", "kv_write", "pa_mq_tiled")


def _bench_args(workload: str, schedule: str, bench_args: str = "") -> str:
    return bench_args or f"--workload {workload} --schedule {schedule} --no-cpu-baseline"


# A second pass: VALU activity, MFMA/VALU co-execution, waits of any cause, LDS activity.
SQ_COUNTERS2 = ["SQ_ACTIVE_INST_VALU", "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_WAIT_ANY",
                "SQ_WAVE_CYCLES", "SQ_ACTIVE_INST_LDS", "SQ_INSTS_VALU_TRANS_F32", "SQ_BUSY_CU_CYCLES",
                "GRBM_GUI_ACTIVE"]


def sq_commands(workload: str, schedule: str, out: str = "OUT", bench_args: str = "") -> list:
    """The two counter passes that sq_summary() reads."""
    run = f"python -u bench.py {_bench_args(workload, schedule, bench_args)} --steps 5 --warmup 2"
    return [f"rocprofv3 --pmc {' '.join(SQ_COUNTERS)} --output-format csv -d {out}/sq -o run -- {run}",
            f"rocprofv3 --pmc {' '.join(SQ_COUNTERS2)} --output-format csv -d {out}/sq2 -o run -- {run}"]


def _per_kernel(path: str):
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    meta = {}
    for r in csv.DictReader(open(path)):
        k = r["Kernel_Name"]
        if not any(t in k for t in OUR_KERNELS):
            continue
        vals[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
        meta[k] = int(r["Grid_Size"])
    return vals, meta


def sq_summary(out: str, workload: str, schedule: str = "balanced", bench_args: str = "", name: str = "") -> str:
    """profiles/counters_<name or schedule_workload>.md: per kernel of the step, instructions per
    wave, the MFMA pipe's and the VALU's busy shares per SIMD, MFMA/VALU co-execution, the shares
    of wave cycles spent waiting, LDS bank conflicts."""
    vals, meta = _per_kernel(os.path.join(out, "sq", "run_counter_collection.csv"))
    p2 = os.path.join(out, "sq2", "run_counter_collection.csv")
    vals2 = _per_kernel(p2)[0] if os.path.exists(p2) else {}
    name = name or f"{schedule}_{workload}"
    lines = [f"# {workload}: core counters of the benchmark step ({bench_args or schedule + ' schedule'})", "",
             f"Kernel source sha256[:16] = `{source_hash()}` (paged_kv_cache_224_amd/csrc/pagedkv.hip without "
             "comments)", "", "## Commands (run from the repository root on one MI355X; OUT is any scratch folder)",
             "", "```"] + sq_commands(workload, schedule, bench_args=bench_args) + [
             f"python -c \"from paged_kv_cache_224_amd.profile_summary import sq_summary; "
             f"sq_summary('OUT', '{workload}', '{schedule}', '{bench_args}', '{name}')\"", "```", "",
             "Means over the dispatches of the run.  Counters are summed over the whole GPU.  Definitions:",
             "- per wave: an instruction count / (grid threads / 64);",
             "- MFMA busy per SIMD: SQ_VALU_MFMA_BUSY_CYCLES / (4 x SQ_BUSY_CU_CYCLES), the share of the CUs' busy "
             "cycles in which a SIMD's matrix pipe works (SQ_BUSY_CU_CYCLES counts CU-cycles; one "
             "v_mfma_f32_16x16x32 occupies the pipe for 16 cycles);",
             "- VALU busy per SIMD: SQ_ACTIVE_INST_VALU / SQ_BUSY_CU_CYCLES (quad-cycles that waves spend on VALU "
             "instructions, x 4, per SIMD-cycle; waves sharing a SIMD are counted separately, so the share can pass "
             "100%);",
             "- MFMA/VALU co-exec: SQ_VALU_MFMA_COEXEC_CYCLES / SQ_VALU_MFMA_BUSY_CYCLES, the share of the matrix "
             "pipe's busy cycles in which a vector instruction issued beside it;",
             "- waiting to issue: SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES, the share of wave cycles spent waiting for an "
             "instruction to issue; waiting (any): SQ_WAIT_ANY / SQ_WAVE_CYCLES, waiting for anything (issue, "
             "memory counters, barriers);",
             "- LDS bank conflicts: SQ_LDS_BANK_CONFLICT, cycles stalled on conflicts (whole GPU).",
             "- The second group of columns comes from a second pass (the second command); a kernel's rows in the "
             "two passes are separate runs of the same step.", "",
             "| kernel | waves | MFMA / wave | VALU / wave | LDS / wave | MFMA busy per SIMD | VALU busy per SIMD | "
             "MFMA/VALU co-exec | waiting to issue | waiting (any) | LDS bank-conflict cycles |",
             "|---|---|---|---|---|---|---|---|---|---|---|"]
    for k in sorted(vals):
        m = {c: sum(v) / len(v) for c, v in vals[k].items()}
        waves = max(1, meta[k] // 64)
        busy = m.get("SQ_BUSY_CU_CYCLES", 0.0)
        mfma_busy = m.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (4 * busy) if busy else 0.0
        wc = m.get("SQ_WAVE_CYCLES", 0.0)
        wait = m.get("SQ_WAIT_INST_ANY", 0.0) / wc if wc else 0.0
        m2 = {c: sum(v) / len(v) for c, v in vals2.get(k, {}).items()}
        busy2, wc2, mb2 = m2.get("SQ_BUSY_CU_CYCLES", 0.0), m2.get("SQ_WAVE_CYCLES", 0.0), m2.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
        valu = f"{100 * m2['SQ_ACTIVE_INST_VALU'] / busy2:.1f}%" if busy2 and "SQ_ACTIVE_INST_VALU" in m2 else "-"
        coex = f"{100 * m2.get('SQ_VALU_MFMA_COEXEC_CYCLES', 0.0) / mb2:.1f}%" if mb2 else "-"
        wany = f"{100 * m2.get('SQ_WAIT_ANY', 0.0) / wc2:.1f}%" if wc2 else "-"
        lines.append(f"| {k[:80]} | {waves} | {m.get('SQ_INSTS_MFMA', 0) / waves:.0f} | "
                     f"{m.get('SQ_INSTS_VALU', 0) / waves:.0f} | {m.get('SQ_INSTS_LDS', 0) / waves:.0f} | "
                     f"{100 * mfma_busy:.1f}% | {valu} | {coex} | {100 * wait:.1f}% | {wany} | "
                     f"{m.get('SQ_LDS_BANK_CONFLICT', 0):.0f} |")
    lines.append("")
    text = "\n".join(lines)
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", f"counters_{name}.md"), "w") as fh:
        fh.write(text)
    return text


# L2 (TCC) hits and misses and the mean resident waves per CU, one pass.
CACHE_COUNTERS = ["TCC_HIT_sum", "TCC_MISS_sum", "MeanOccupancyPerCU"]


def cache_commands(workload: str, schedule: str, out: str = "OUT", bench_args: str = "") -> list:
    """The one counter pass that cache_summary() reads."""
    return [f"rocprofv3 --pmc {' '.join(CACHE_COUNTERS)} --output-format csv -d {out}/cache -o run -- python -u "
            f"bench.py {_bench_args(workload, schedule, bench_args)} --steps 5 --warmup 2"]


def cache_summary(out: str, workload: str, schedule: str = "balanced", bench_args: str = "", name: str = "",
                  waves_per_cu: str = "") -> str:
    """profiles/cache_<name or schedule_workload>.md: per kernel, the L2 hit rate TCC_HIT / (TCC_HIT +
    TCC_MISS) and the mean number of waves resident per CU while the GPU is busy."""
    vals, meta = _per_kernel(os.path.join(out, "cache", "run_counter_collection.csv"))
    name = name or f"{schedule}_{workload}"
    lines = [f"# {workload}: L2 hit rate and occupancy of the benchmark step "
             f"({bench_args or schedule + ' schedule'})", "",
             f"Kernel source sha256[:16] = `{source_hash()}` (paged_kv_cache_224_amd/csrc/pagedkv.hip without "
             "comments)", "", "## Commands (run from the repository root on one MI355X; OUT is any scratch folder)",
             "", "```"] + cache_commands(workload, schedule, bench_args=bench_args) + [
             f"python -c \"from paged_kv_cache_224_amd.profile_summary import cache_summary; "
             f"cache_summary('OUT', '{workload}', '{schedule}', '{bench_args}', '{name}')\"", "```", "",
             "Means over the dispatches of the run.  L2 hit rate = TCC_HIT_sum / (TCC_HIT_sum + TCC_MISS_sum) "
             "over all L2 channels (uncached reads count as misses).  MeanOccupancyPerCU = accumulated "
             "SQ_LEVEL_WAVES / GRBM_GUI_ACTIVE / CUs: waves resident per CU, averaged over the kernel's busy time "
             "(a CU holds at most 32 waves; the resident limit of each kernel follows from its workgroup size, "
             "registers and LDS).", "",
             "| kernel | waves in the grid | L2 hits | L2 misses | L2 hit rate | mean waves per CU |",
             "|---|---|---|---|---|---|"]
    for k in sorted(vals):
        m = {c: sum(v) / len(v) for c, v in vals[k].items()}
        hit, miss = m.get("TCC_HIT_sum", 0.0), m.get("TCC_MISS_sum", 0.0)
        rate = hit / (hit + miss) if hit + miss else 0.0
        lines.append(f"| {k[:80]} | {max(1, meta[k] // 64)} | {hit:.0f} | {miss:.0f} | {100 * rate:.1f}% | "
                     f"{m.get('MeanOccupancyPerCU', 0.0):.2f} |")
    lines.append("")
    text = "\n".join(lines)
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", f"cache_{name}.md"), "w") as fh:
        fh.write(text)
    return text


if __name__ == "__main__":
    if len(sys.argv) < 3:
        sys.exit(__doc__)
    print(summarize(sys.argv[1], sys.argv[2], sys.argv[3] if len(sys.argv) > 3 else "balanced"))

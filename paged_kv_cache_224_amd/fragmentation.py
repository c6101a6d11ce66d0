"""KV-memory waste of paged versus static allocation on a synthetic request trace (host only).

The pages claim that paging keeps KV fragmentation under 4% where static allocation wastes
60% and more, because a paged sequence leaves at most block_size - 1 slots unused while a
static one reserves the maximum length up front ("vllm-project-vllm -- L2", section 3 Q3,
section 9 "Memory Management", section 11 steps 1-3).  This module replays a seeded trace of
requests through a continuous-batching loop under both policies with the same slot budget:

  paged   the native block manager: a request is admitted when its prompt's blocks are free,
          one token is appended per running sequence per step (a new block only when the last
          one is full); a sequence that cannot get a block is preempted (freed and requeued
          with the tokens it has, to be re-admitted later);
  static  every admitted request reserves max_len slots for its whole life.

Per step it records allocated slots and used slots (tokens held); waste = 1 - used/allocated,
averaged over steps weighted by allocated slots.  It also reports the mean number of running
sequences and the steps needed to drain the trace.  Synthetic lengths stand in for a real
request mix; nothing here reads a dataset.
"""
from __future__ import annotations

import argparse
import json
from collections import deque
from dataclasses import dataclass
from typing import List

import numpy as np

from ._lib import BlockManager, PagedKVError


@dataclass
class Request:
    prompt: int
    output: int


def make_trace(num_requests: int, seed: int = 0, prompt_mu: float = 6.0, prompt_sigma: float = 1.0,
               output_mu: float = 5.0, output_sigma: float = 1.0, max_len: int = 8192) -> List[Request]:
    """Lognormal prompt and output lengths, clipped so that prompt + output <= max_len."""
    rng = np.random.default_rng(seed)
    p = np.clip(np.rint(np.exp(rng.normal(prompt_mu, prompt_sigma, num_requests))), 1, max_len - 1).astype(int)
    o = np.clip(np.rint(np.exp(rng.normal(output_mu, output_sigma, num_requests))), 1, None).astype(int)
    o = np.minimum(o, max_len - p)
    return [Request(int(a), int(b)) for a, b in zip(p, o)]


def simulate(trace: List[Request], budget_slots: int, block_size: int = 16, max_len: int = 8192,
             policy: str = "paged", max_batch: int = 1024, check_every: int = 0) -> dict:
    if policy not in ("paged", "static"):
        raise ValueError(policy)
    waiting = deque((i, r.prompt, r.output) for i, r in enumerate(trace))   # (id, tokens now, tokens to go)
    running = {}                                                            # id -> [tokens, to go]
    bm = BlockManager(budget_slots // block_size, block_size) if policy == "paged" else None
    steps = preemptions = 0
    alloc_sum = used_sum = batch_sum = 0
    max_waste_bound_excess = 0
    while waiting or running:
        # admit in arrival order while memory and the batch limit allow
        while waiting and len(running) < max_batch:
            rid, n, togo = waiting[0]
            if policy == "paged":
                try:
                    bm.add(rid, n)
                except PagedKVError:
                    break
            elif (len(running) + 1) * max_len > budget_slots:
                break
            waiting.popleft()
            running[rid] = [n, togo]
        if not running:
            raise RuntimeError("a single request does not fit the budget")
        # one decode step: every running sequence appends a token
        finished = []
        for rid in list(running):
            n, togo = running[rid]
            if policy == "paged":
                try:
                    bm.append(rid)
                except PagedKVError:                 # out of blocks: preempt and requeue
                    bm.free(rid)
                    del running[rid]
                    waiting.appendleft((rid, n, togo))
                    preemptions += 1
                    continue
            running[rid] = [n + 1, togo - 1]
            if togo - 1 == 0:
                finished.append(rid)
        used = sum(v[0] for v in running.values())
        if policy == "paged":
            alloc = (bm.num_blocks - bm.num_free()) * block_size
            bound = (block_size - 1) * len(running)             # at most block_size - 1 idle slots each
            max_waste_bound_excess = max(max_waste_bound_excess, (alloc - used) - bound)
            if check_every and steps % check_every == 0:
                assert bm.check()
        else:
            alloc = len(running) * max_len
        alloc_sum += alloc
        used_sum += used
        batch_sum += len(running)
        steps += 1
        for rid in finished:
            del running[rid]
            if policy == "paged":
                bm.free(rid)
    return {"policy": policy, "steps": steps, "mean_running": batch_sum / steps,
            "waste": 1.0 - used_sum / alloc_sum, "preemptions": preemptions,
            "paged_waste_bound_excess": max_waste_bound_excess if policy == "paged" else None}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--requests", type=int, default=2000)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--budget-slots", type=int, default=1 << 20)
    ap.add_argument("--block-size", type=int, default=16)
    ap.add_argument("--max-len", type=int, default=8192)
    a = ap.parse_args(argv)
    trace = make_trace(a.requests, a.seed, max_len=a.max_len)
    out = {p: simulate(trace, a.budget_slots, a.block_size, a.max_len, p) for p in ("paged", "static")}
    out["trace"] = {"requests": a.requests, "seed": a.seed, "mean_prompt": float(np.mean([r.prompt for r in trace])),
                    "mean_output": float(np.mean([r.output for r in trace])), "max_len": a.max_len,
                    "budget_slots": a.budget_slots, "block_size": a.block_size}
    print(json.dumps(out))
    return out


if __name__ == "__main__":
    main()

"""HIP graphs of the decode step for a set of batch sizes.

The pages capture the decode step as CUDA/HIP graphs for several batch sizes and replay, for
each step, the smallest captured graph that fits the batch ("vllm-project-vllm -- L2",
section 10, the CUDA/HIP-graphs row of the "Key Performance Mechanisms" table, and the graph
dispatcher the same page names).  Here the step is paged_kv_write -> paged_attn_decode ->
paged_attn_reduce, captured once per size over persistent device buffers:

* the caller fills the input views that ``inputs(B)`` returns (query, new K/V rows, slots,
  block tables, context lengths of B sequences) and calls ``replay(B)``;
* rows B .. size-1 of the chosen graph are padding: context length 0 (no tiles, a zero output
  row) and slot -1 (nothing written), so they cost no bandwidth and change nothing;
* the balanced split only sees the tiles of real rows, so a padded replay computes exactly
  what the eager step on the B rows computes, bit for bit.

Capture happens once in the constructor; a replay enqueues no allocation, memset or host
synchronisation (the kernels keep no state between launches).  Host-side bookkeeping only:
every step runs the library's kernels.
"""
from __future__ import annotations

import bisect
from typing import Dict, Sequence

import torch

from . import _lib as L


class StepGraphs:
    def __init__(self, key_cache: torch.Tensor, value_cache: torch.Tensor, num_heads: int, max_blocks: int,
                 max_context_len: int, q_dtype: torch.dtype, sizes: Sequence[int] = (1, 2, 4, 8, 16, 32, 64, 128, 256),
                 partition_size: int | None = None, scale: float | None = None, k_scale: float = 1.0,
                 v_scale: float = 1.0):
        NB, BS, Hkv, D = key_cache.shape
        self.kc, self.vc = key_cache, value_cache
        self.sizes = sorted(set(int(s) for s in sizes))
        self.Hq, self.Hkv, self.D, self.max_blocks = num_heads, Hkv, D, max_blocks
        self.max_context_len = max_context_len
        self.scale = D ** -0.5 if scale is None else scale
        self.k_scale, self.v_scale = k_scale, v_scale
        dev = key_cache.device
        src_dt = q_dtype if key_cache.dtype in (torch.float16, torch.bfloat16) else torch.bfloat16
        if partition_size is None:
            partition_size = L.balanced_split(Hkv, D, q_dtype, key_cache.dtype)
        self.partition_size = partition_size
        Bmax = self.sizes[-1]
        self.q = torch.zeros((Bmax, num_heads, D), dtype=q_dtype, device=dev)
        self.k_new = torch.zeros((Bmax, Hkv, D), dtype=src_dt, device=dev)
        self.v_new = torch.zeros_like(self.k_new)
        self.slots = torch.full((Bmax,), -1, dtype=torch.int64, device=dev)
        self.block_tables = torch.zeros((Bmax, max_blocks), dtype=torch.int32, device=dev)
        self.context_lens = torch.zeros((Bmax,), dtype=torch.int32, device=dev)
        self.out = torch.zeros((Bmax, num_heads, D), dtype=q_dtype, device=dev)
        self.ws = L.DecodeWorkspace(Bmax, num_heads, D, max_context_len, partition_size, device=dev)
        self._live = 0                       # rows of the last batch (rows past it hold padding)
        self.graphs: Dict[int, torch.cuda.CUDAGraph] = {}
        stream = torch.cuda.Stream()
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            for s in self.sizes:             # warm-up launches outside the capture
                self._step(s)
        torch.cuda.current_stream().wait_stream(stream)
        torch.cuda.synchronize()
        for s in self.sizes:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                self._step(s)
            self.graphs[s] = g
        torch.cuda.synchronize()

    def _step(self, s: int) -> None:
        """The captured step on rows [0, s) of the persistent buffers."""
        ws = self.ws
        L.paged_kv_write(self.k_new[:s], self.v_new[:s], self.kc, self.vc, self.slots[:s], self.k_scale,
                         self.v_scale)
        L.paged_attn_decode(None, self.q[:s], self.kc, self.vc, self.block_tables[:s], self.context_lens[:s],
                            self.scale, self.max_context_len, self.partition_size, ws.tmp_out, ws.max_logits,
                            ws.exp_sums, self.k_scale, self.v_scale)
        L.paged_attn_reduce(self.out[:s], ws.tmp_out, ws.max_logits, ws.exp_sums, self.context_lens[:s],
                            self.max_context_len, self.partition_size)

    def size_for(self, B: int) -> int:
        """The smallest captured batch size that holds B rows."""
        i = bisect.bisect_left(self.sizes, B)
        if i == len(self.sizes):
            raise ValueError(f"batch of {B} exceeds the largest captured size {self.sizes[-1]}")
        return self.sizes[i]

    def inputs(self, B: int):
        """Views (q, k_new, v_new, slots, block_tables, context_lens) of the first B rows, for the
        caller to fill before replay(B).  Rows the previous batch used beyond B are reset to
        padding here."""
        if B < self._live:
            self.context_lens[B:self._live].zero_()
            self.slots[B:self._live].fill_(-1)
        self._live = B
        return (self.q[:B], self.k_new[:B], self.v_new[:B], self.slots[:B], self.block_tables[:B],
                self.context_lens[:B])

    def replay(self, B: int) -> torch.Tensor:
        """Replay the graph of size_for(B); returns the view out[:B] (valid after the stream
        reaches it)."""
        if B != self._live:
            raise ValueError("call inputs(B) for this batch before replay(B)")
        self.graphs[self.size_for(B)].replay()
        return self.out[:B]

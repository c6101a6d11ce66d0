"""Seeded synthetic workloads for one paged-attention decode step.

This module only *builds inputs*: context lengths, a shuffled block pool, block tables,
slot mappings and N(0,1) tensors.  It holds none of the attention arithmetic, so both the
fp64 oracle (tests) and the HIP path (tests, benchmark) can draw from it.

The data structures follow the pages' description of PagedAttention:

* KV storage is a pool of fixed-size blocks that need not be contiguous per sequence
  ("vllm-project-vllm — L2", §3 Q2 and §9 Memory Management).
* A block table is a 2-D integer tensor mapping (sequence, logical block) to a physical
  block id, read-only on the GPU (same page, §6 "KV Cache Block Tables").
* Blocks may be shared copy-on-write between sequences that have a common prefix
  (same page, §9 and §11 step 5).
* The block-table invariant: every physical block is free, owned by exactly one logical
  block, or shared with a positive reference count (same page, §8).
* Per-sequence waste is below one block (same page, §11 step 2).

Recipe (fixed; every draw is seeded):

1. ``numpy.random.default_rng(seed)`` (PCG64) draws, in this order, the context lengths
   and then one permutation of the physical block ids.  Physical blocks are handed out in
   permutation order.
2. ``torch.Generator().manual_seed(seed)`` (CPU) draws float32 N(0,1) values for q, the K
   pool, the V pool, the new K rows and the new V rows, in that order.  Each tensor is drawn
   in chunks of ``_CHUNK`` elements and rounded to its storage dtype with
   round-to-nearest-even.
3. Table entries past a sequence's last used block point to a "trap" block that no
   sequence uses.  They are never meant to be read.
4. For an fp8 KV cache, the pools are produced in bf16.  The per-tensor scale is
   fp32(max|x|) / 448, taken over the whole bf16 pool plus the new rows, with the division
   done in fp32.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np
import torch

_CHUNK = 1 << 24

DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16}
E4M3_MAX = 448.0


@dataclass(frozen=True)
class Config:
    """One decode-step workload: shapes, dtypes and how lengths and pools are drawn."""

    name: str
    seed: int
    B: int
    Hq: int
    Hkv: int
    D: int
    block_size: int
    q_dtype: str            # "f16" | "bf16"; also the output dtype
    kv_dtype: str           # "f16" | "bf16" | "fp8"
    lens: Tuple             # ("uniform", lo, hi) | ("lognormal", mu, sigma, lo, hi) | ("prefix", P, lo, hi)
    pool: Tuple             # ("fixed", nblocks) | ("factor", f)
    max_len: int            # upper bound on a context length; sizes the block table
    partition_size: int     # split-K partition (tokens) the benchmark and tests use; 0 = single pass

    @property
    def group(self) -> int:
        return self.Hq // self.Hkv

    @property
    def max_blocks(self) -> int:
        return -(-self.max_len // self.block_size)

    @property
    def src_dtype(self) -> str:
        """dtype of the rows handed to the KV write (the cache dtype unless it is fp8)."""
        return "bf16" if self.kv_dtype == "fp8" else self.kv_dtype


# The five workloads.  Shapes: Llama-3-8B and Llama-3-70B attention layers, a long-context
# split-K case and a shared-prefix (copy-on-write) batch, plus a tiny case.
CONFIGS: Dict[str, Config] = {
    "tiny": Config("tiny", 0, B=4, Hq=8, Hkv=2, D=64, block_size=16, q_dtype="f16", kv_dtype="f16",
                   lens=("uniform", 1, 256), pool=("fixed", 80), max_len=256, partition_size=64),
    "llama3_8b": Config("llama3_8b", 1, B=64, Hq=32, Hkv=8, D=128, block_size=16, q_dtype="bf16",
                        kv_dtype="bf16", lens=("uniform", 512, 4096), pool=("factor", 1.25),
                        max_len=4096, partition_size=512),
    "long_ctx": Config("long_ctx", 2, B=8, Hq=32, Hkv=8, D=128, block_size=16, q_dtype="bf16",
                       kv_dtype="bf16", lens=("uniform", 32768, 131072), pool=("factor", 1.25),
                       max_len=131072, partition_size=512),
    "shared_prefix": Config("shared_prefix", 3, B=256, Hq=32, Hkv=8, D=128, block_size=16,
                            q_dtype="bf16", kv_dtype="bf16", lens=("prefix", 2048, 64, 512),
                            pool=("factor", 1.25), max_len=2048 + 512, partition_size=512),
    "llama3_70b_fp8": Config("llama3_70b_fp8", 4, B=128, Hq=64, Hkv=8, D=128, block_size=32,
                             q_dtype="bf16", kv_dtype="fp8", lens=("lognormal", 7.5, 1.0, 16, 32768),
                             pool=("factor", 1.25), max_len=32768, partition_size=512),
}
CONFIG_ORDER = ["tiny", "llama3_8b", "long_ctx", "shared_prefix", "llama3_70b_fp8"]


def shrink(cfg: Config, B: Optional[int] = None, len_div: int = 1, name: Optional[str] = None,
           seed: Optional[int] = None) -> Config:
    """Same workload shape with fewer sequences and/or shorter contexts (for CPU-sized tests)."""
    lens = cfg.lens
    if len_div != 1:
        if lens[0] == "uniform":
            lens = ("uniform", max(1, lens[1] // len_div), max(1, lens[2] // len_div))
        elif lens[0] == "lognormal":
            lens = ("lognormal", lens[1] - math.log(len_div), lens[2], max(1, lens[3] // len_div),
                    max(1, lens[4] // len_div))
        elif lens[0] == "prefix":
            lens = ("prefix", max(cfg.block_size, lens[1] // len_div // cfg.block_size * cfg.block_size),
                    max(1, lens[2] // len_div), max(1, lens[3] // len_div))
    max_len = max(1, cfg.max_len // len_div)
    if lens[0] == "prefix":
        max_len = lens[1] + lens[3]
    pool = cfg.pool
    return dataclasses.replace(cfg, name=name or f"{cfg.name}_small", B=B or cfg.B, lens=lens,
                               max_len=max_len, pool=pool, seed=cfg.seed if seed is None else seed)


@dataclass
class Workload:
    """Host (CPU) tensors of one decode step.  Pools hold the *source* dtype (f16/bf16)."""

    cfg: Config
    context_lens: np.ndarray          # [B] int32
    block_tables: np.ndarray          # [B, max_blocks] int32
    num_blocks: int
    trap_block: int
    prefix_blocks: np.ndarray         # physical ids shared by every row (empty unless prefix-shared)
    q: torch.Tensor                   # [B, Hq, D] q dtype
    k_pool: torch.Tensor              # [NB, BS, Hkv, D] source dtype
    v_pool: torch.Tensor
    k_new: torch.Tensor               # [T, Hkv, D] source dtype
    v_new: torch.Tensor
    slot_mapping: np.ndarray          # [T] int64; slot = block * BS + offset
    k_scale: float = 1.0              # per-tensor fp8 scales (1.0 unless the cache is fp8)
    v_scale: float = 1.0
    refcount: np.ndarray = field(default=None)  # [NB] references from the used part of the tables

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.cfg.D)

    @property
    def blocks_used(self) -> np.ndarray:
        return -(-self.context_lens.astype(np.int64) // self.cfg.block_size)

    def stale_slots(self) -> np.ndarray:
        """Pool slots no sequence reads: tail slots past n in each last block, and the trap block.

        Filling them with NaN must not change any output (blocks are reused across requests,
        so real pools hold stale bytes there).
        """
        BS = self.cfg.block_size
        slots: List[np.ndarray] = [self.trap_block * BS + np.arange(BS, dtype=np.int64)]
        for b, n in enumerate(self.context_lens.tolist()):
            if n % BS:
                last = int(self.block_tables[b, (n - 1) // BS])
                slots.append(last * BS + np.arange(n % BS, BS, dtype=np.int64))
        return np.unique(np.concatenate(slots))


def _draw_lengths(cfg: Config, rng: np.random.Generator) -> Tuple[np.ndarray, int]:
    kind = cfg.lens[0]
    if kind == "uniform":
        lens = rng.integers(cfg.lens[1], cfg.lens[2] + 1, size=cfg.B)
        return lens.astype(np.int64), 0
    if kind == "lognormal":
        _, mu, sigma, lo, hi = cfg.lens
        lens = np.clip(np.rint(np.exp(rng.normal(mu, sigma, size=cfg.B))), lo, hi)
        return lens.astype(np.int64), 0
    if kind == "prefix":
        _, P, lo, hi = cfg.lens
        assert P % cfg.block_size == 0, "shared prefix must fill whole blocks"
        suffix = rng.integers(lo, hi + 1, size=cfg.B).astype(np.int64)
        return P + suffix, P
    raise ValueError(kind)


def _normals(gen: torch.Generator, shape, dtype: torch.dtype) -> torch.Tensor:
    n = int(np.prod(shape))
    out = torch.empty(n, dtype=dtype)
    for lo in range(0, n, _CHUNK):
        hi = min(n, lo + _CHUNK)
        out[lo:hi] = torch.randn(hi - lo, generator=gen, dtype=torch.float32).to(dtype)
    return out.view(*shape)


def make_workload(cfg: Config, tensors: bool = True) -> Workload:
    """Draw one seeded decode-step workload (see the module docstring for the recipe).

    With ``tensors=False`` only lengths, tables and slots are drawn (q and the pools are
    empty placeholders); the structure is identical to the full draw."""
    BS = cfg.block_size
    assert cfg.Hq % cfg.Hkv == 0
    rng = np.random.default_rng(cfg.seed)
    lens, prefix_len = _draw_lengths(cfg, rng)
    assert lens.max() <= cfg.max_len
    nb_used = -(-lens // BS)
    prefix_nb = prefix_len // BS
    unique_needed = int((nb_used - prefix_nb).sum()) + prefix_nb
    if cfg.pool[0] == "fixed":
        NB = int(cfg.pool[1])
    else:
        NB = int(math.ceil(cfg.pool[1] * unique_needed))
    NB = max(NB, unique_needed + 1)          # room for the trap block
    perm = rng.permutation(NB).astype(np.int64)

    bt = np.empty((cfg.B, cfg.max_blocks), dtype=np.int64)
    cursor = 0
    prefix_blocks = perm[cursor:cursor + prefix_nb]
    cursor += prefix_nb
    for b in range(cfg.B):
        own = int(nb_used[b]) - prefix_nb
        row = np.concatenate([prefix_blocks, perm[cursor:cursor + own]])
        cursor += own
        bt[b, :row.size] = row
        bt[b, row.size:] = -1
    trap = int(perm[cursor])                 # first block nobody owns
    bt[bt < 0] = trap
    assert cursor < NB

    # refcounts over the used part of every row (block-table invariant, checked by tests)
    refcount = np.zeros(NB, dtype=np.int64)
    for b in range(cfg.B):
        np.add.at(refcount, bt[b, :nb_used[b]], 1)

    # one new token per sequence, at logical position n - 1
    pos = lens - 1
    slot_mapping = bt[np.arange(cfg.B), pos // BS] * BS + pos % BS

    gen = torch.Generator().manual_seed(cfg.seed)
    qdt = DTYPES[cfg.q_dtype]
    sdt = DTYPES[cfg.src_dtype]
    if not tensors:
        e = torch.empty(0)
        return Workload(cfg=cfg, context_lens=lens.astype(np.int32), block_tables=bt.astype(np.int32),
                        num_blocks=NB, trap_block=trap, prefix_blocks=prefix_blocks, q=e, k_pool=e,
                        v_pool=e, k_new=e, v_new=e, slot_mapping=slot_mapping.astype(np.int64),
                        refcount=refcount)
    q = _normals(gen, (cfg.B, cfg.Hq, cfg.D), qdt)
    k_pool = _normals(gen, (NB, BS, cfg.Hkv, cfg.D), sdt)
    v_pool = _normals(gen, (NB, BS, cfg.Hkv, cfg.D), sdt)
    k_new = _normals(gen, (cfg.B, cfg.Hkv, cfg.D), sdt)
    v_new = _normals(gen, (cfg.B, cfg.Hkv, cfg.D), sdt)

    k_scale = v_scale = 1.0
    if cfg.kv_dtype == "fp8":
        k_scale = per_tensor_fp8_scale(k_pool, k_new)
        v_scale = per_tensor_fp8_scale(v_pool, v_new)

    return Workload(cfg=cfg, context_lens=lens.astype(np.int32), block_tables=bt.astype(np.int32),
                    num_blocks=NB, trap_block=trap, prefix_blocks=prefix_blocks, q=q, k_pool=k_pool,
                    v_pool=v_pool, k_new=k_new, v_new=v_new, slot_mapping=slot_mapping.astype(np.int64),
                    k_scale=k_scale, v_scale=v_scale, refcount=refcount)


def per_tensor_fp8_scale(*tensors: torch.Tensor) -> float:
    """fp32(max |x|) / 448 in fp32 arithmetic, over all given tensors."""
    amax = max(float(t.abs().max().float()) for t in tensors)
    return float(np.float32(amax) / np.float32(E4M3_MAX))


def identity_tables(w: Workload) -> np.ndarray:
    """Row-contiguous tables over the same pool: row b owns blocks [b*max_blocks, ...).

    Only meaningful when the pool was built for it (see ``dense_workload``)."""
    B, MB = w.block_tables.shape
    return (np.arange(B)[:, None] * MB + np.arange(MB)[None, :]).astype(np.int32)


def permute_blocks(w: Workload, seed: int) -> Workload:
    """Move every physical block to a new random id, remapping the tables to match.

    The logical content of every sequence is unchanged."""
    rng = np.random.default_rng(seed)
    NB = w.num_blocks
    newid = rng.permutation(NB)                  # block i moves to newid[i]
    inv = np.argsort(newid)                      # new slot j holds old block inv[j]
    k_pool = w.k_pool[torch.from_numpy(inv)].contiguous()
    v_pool = w.v_pool[torch.from_numpy(inv)].contiguous()
    bt = newid[w.block_tables.astype(np.int64)].astype(np.int32)
    BS = w.cfg.block_size
    sm = w.slot_mapping.copy()
    ok = sm >= 0
    sm[ok] = newid[sm[ok] // BS] * BS + sm[ok] % BS
    refcount = np.zeros_like(w.refcount)
    refcount[newid] = w.refcount
    return dataclasses.replace(w, block_tables=bt, k_pool=k_pool, v_pool=v_pool, slot_mapping=sm,
                               trap_block=int(newid[w.trap_block]),
                               prefix_blocks=newid[w.prefix_blocks], refcount=refcount)


def unshare_prefix(w: Workload) -> Workload:
    """Give every row a private copy of the shared prefix blocks (same logical content)."""
    P = w.prefix_blocks.size
    if P == 0:
        return w
    B = w.cfg.B
    extra = B * P
    NB2 = w.num_blocks + extra
    k_pool = torch.cat([w.k_pool, w.k_pool[torch.from_numpy(np.tile(w.prefix_blocks, B))]])
    v_pool = torch.cat([w.v_pool, w.v_pool[torch.from_numpy(np.tile(w.prefix_blocks, B))]])
    bt = w.block_tables.copy()
    for b in range(B):
        bt[b, :P] = w.num_blocks + b * P + np.arange(P)
    refcount = np.concatenate([w.refcount, np.ones(extra, dtype=np.int64)])
    refcount[w.prefix_blocks] = 0
    return dataclasses.replace(w, num_blocks=NB2, block_tables=bt, k_pool=k_pool, v_pool=v_pool,
                               prefix_blocks=np.zeros(0, dtype=np.int64), refcount=refcount)


def dense_workload(cfg: Config, lens: List[int], seed: int = 0) -> Workload:
    """A workload whose tables are the identity map: row b uses blocks b*MB .. b*MB+MB-1.

    Its pool, read in table order, is a contiguous [B, MB*BS, Hkv, D] tensor, so dense
    attention over that tensor is an independent check of the block-table gather."""
    BS, MB = cfg.block_size, cfg.max_blocks
    B = len(lens)
    NB = B * MB + 1
    gen = torch.Generator().manual_seed(seed)
    qdt, sdt = DTYPES[cfg.q_dtype], DTYPES[cfg.src_dtype]
    q = _normals(gen, (B, cfg.Hq, cfg.D), qdt)
    k_pool = _normals(gen, (NB, BS, cfg.Hkv, cfg.D), sdt)
    v_pool = _normals(gen, (NB, BS, cfg.Hkv, cfg.D), sdt)
    k_new = _normals(gen, (B, cfg.Hkv, cfg.D), sdt)
    v_new = _normals(gen, (B, cfg.Hkv, cfg.D), sdt)
    bt = (np.arange(B)[:, None] * MB + np.arange(MB)[None, :]).astype(np.int32)
    lens_a = np.asarray(lens, dtype=np.int32)
    pos = np.maximum(lens_a.astype(np.int64) - 1, 0)
    slot = bt[np.arange(B), pos // BS].astype(np.int64) * BS + pos % BS
    slot[lens_a == 0] = -1
    refcount = np.zeros(NB, dtype=np.int64)
    for b in range(B):
        refcount[bt[b, :-(-int(lens_a[b]) // BS)]] += 1
    k_scale = v_scale = 1.0
    if cfg.kv_dtype == "fp8":
        k_scale = per_tensor_fp8_scale(k_pool, k_new)
        v_scale = per_tensor_fp8_scale(v_pool, v_new)
    cfg2 = dataclasses.replace(cfg, B=B)
    return Workload(cfg=cfg2, context_lens=lens_a, block_tables=bt, num_blocks=NB, trap_block=NB - 1,
                    prefix_blocks=np.zeros(0, dtype=np.int64), q=q, k_pool=k_pool, v_pool=v_pool,
                    k_new=k_new, v_new=v_new, slot_mapping=slot, k_scale=k_scale, v_scale=v_scale,
                    refcount=refcount)


def algorithmic_bytes(w: Workload) -> Dict[str, int]:
    """Bytes one decode step must move at minimum (KV read once per logical token).

    kv_logical counts every (sequence, token) once; kv_unique counts each physical block's
    used rows once, which is what HBM has to deliver when shared prefix blocks are cached."""
    cfg = w.cfg
    e_kv = 1 if cfg.kv_dtype == "fp8" else 2
    e_q = 2
    n = w.context_lens.astype(np.int64)
    row = cfg.Hkv * cfg.D * e_kv * 2                      # K and V bytes per token
    kv_logical = int(n.sum()) * row
    P = w.prefix_blocks.size * cfg.block_size
    kv_unique = kv_logical - max(0, cfg.B - 1) * P * row if P else kv_logical
    other = cfg.B * cfg.Hq * cfg.D * (e_q + e_q) + 4 * int(w.blocks_used.sum()) + 4 * cfg.B
    e_src = 2
    T = int((w.slot_mapping >= 0).sum())
    write = T * cfg.Hkv * cfg.D * 2 * (e_src + e_kv) + 8 * T
    return {"kv_logical": kv_logical, "kv_unique": kv_unique, "other": other,
            "decode_logical": kv_logical + other, "decode_unique": kv_unique + other, "write": write}


def multi_query_q(cfg: Config, q_len: int, seed: int) -> torch.Tensor:
    """Seeded queries [B, q_len, Hq, D] for L new tokens per sequence: N(0,1) drawn in fp32,
    rounded to the query dtype (nearest even), like the decode query."""
    gen = torch.Generator().manual_seed(10_000 + seed)
    return _normals(gen, (cfg.B, q_len, cfg.Hq, cfg.D), DTYPES[cfg.q_dtype])

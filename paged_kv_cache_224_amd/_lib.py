"""ctypes binding of libpagedkv.so (C ABI in include/pagedkv.h).

Argument marshalling only: shapes become ints, tensors become device pointers, the stream is
torch's current HIP stream.  Every computation runs in the library's HIP kernels.  If the
library has not been built, every call raises ``PagedKVError``; there is no fallback.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# PAGEDKV_LIB may name another build of the same library (same ABI); default: the in-tree one.
LIB_PATH = os.environ.get("PAGEDKV_LIB") or os.path.join(_HERE, "libpagedkv.so")

PKV_F16, PKV_BF16, PKV_FP8_E4M3 = 0, 1, 2
PKV_ERR_SHAPE = -2
PKV_ERR_SCRATCH = -12
PKV_FLAG_SHARED_BLOCKS = 1
_DT = {torch.float16: PKV_F16, torch.bfloat16: PKV_BF16, torch.uint8: PKV_FP8_E4M3,
       torch.float8_e4m3fn: PKV_FP8_E4M3}

_lib: Optional[ctypes.CDLL] = None


class PagedKVError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed: {text} (status {status})")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded library; raises PagedKVError if libpagedkv.so is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise PagedKVError("load", -100, f"{LIB_PATH} is not built (run __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        P, I, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        L.paged_kv_write.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, F, F, P]
        L.paged_kv_write.restype = I
        L.paged_attn_decode.argtypes = [P, P, P, P, P, I, P, I, I, I, I, I, I, F, I, I, F, F, I, I, P, P,
                                        P, I, P]
        L.paged_attn_decode.restype = I
        L.paged_attn_multi_query.argtypes = [P, P, P, P, P, I, P, I, I, I, I, I, I, I, F, I, I, F, F, I, I, P, P,
                                             P, I, P]
        L.paged_attn_multi_query.restype = I
        L.paged_attn_decode_noalloc.argtypes = [P, P, P, P, P, I, P, I, I, I, I, I, I, F, I, I, F, F, I, I, I, P]
        L.paged_attn_decode_noalloc.restype = I
        L.paged_attn_reduce.argtypes = [P, P, P, P, P, I, I, I, I, I, I, P]
        L.paged_attn_reduce.restype = I
        L.paged_attn_decode_append.argtypes = [P, P, P, P, P, P, P, I, P, I, I, I, I, I, I, F, I, I, I, P, P, P,
                                               I, P]
        L.paged_attn_decode_append.restype = I
        L.paged_attn_decode_shared_prefix.argtypes = [P, P, P, P, P, I, P, I, I, I, I, I, I, F, I, I, F, F, I, I,
                                                      I, I, P, P, P, I, P]
        L.paged_attn_decode_shared_prefix.restype = I
        L.paged_attn_shared_prefix_slots.argtypes = [I, I, I, I]
        L.paged_attn_shared_prefix_slots.restype = I
        L.paged_attn_prefix_split.argtypes = [I, I, I, I]
        L.paged_attn_prefix_split.restype = I
        L.paged_attn_workspace_bytes.argtypes = [I, I, I, I, I]
        L.paged_attn_workspace_bytes.restype = ctypes.c_size_t
        L.paged_attn_partial_slots.argtypes = [I, I]
        L.paged_attn_partial_slots.restype = I
        L.paged_attn_multi_query_split.argtypes = [I, I, I, I, I, I]
        L.paged_attn_multi_query_split.restype = I
        L.paged_attn_balanced_split.argtypes = [I, I, I, I]
        L.paged_attn_balanced_split.restype = I
        L.pkv_time_next_call.argtypes = [P, P]
        L.pkv_time_next_call.restype = I
        L.pkv_status_string.argtypes = [I]
        L.pkv_status_string.restype = ctypes.c_char_p
        L.paged_kv_copy_blocks.argtypes = [P, P, P, P, I, I, I, I, I, I, P]
        L.paged_kv_copy_blocks.restype = I
        L.paged_kv_swap_blocks.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I, I, P]
        L.paged_kv_swap_blocks.restype = I
        I64, PI64, PI32 = ctypes.c_int64, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int32)
        L.pkv_bm_create.argtypes = [I, I, I]
        L.pkv_bm_create.restype = P
        L.pkv_bm_destroy.argtypes = [P]
        L.pkv_bm_destroy.restype = None
        for fn in ("pkv_bm_num_free", "pkv_bm_num_free_host", "pkv_bm_check"):
            getattr(L, fn).argtypes = [P]
            getattr(L, fn).restype = I
        L.pkv_bm_add.argtypes = [P, I64, I64]
        L.pkv_bm_append.argtypes = [P, I64, PI64, PI32, PI32]
        L.pkv_bm_fork.argtypes = [P, I64, I64, I64]
        L.pkv_bm_free.argtypes = [P, I64]
        L.pkv_bm_swap_out.argtypes = [P, I64, PI32, PI32, I]
        L.pkv_bm_swap_in.argtypes = [P, I64, PI32, PI32, I]
        L.pkv_bm_num_tokens.argtypes = [P, I64, PI64]
        L.pkv_bm_table.argtypes = [P, PI64, I, PI32, I, PI32]
        for fn in ("pkv_bm_add", "pkv_bm_append", "pkv_bm_fork", "pkv_bm_free", "pkv_bm_swap_out",
                   "pkv_bm_swap_in", "pkv_bm_num_tokens", "pkv_bm_table"):
            getattr(L, fn).restype = I
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().pkv_status_string(int(status)).decode()


def time_next_call(start, stop) -> None:
    """Bind two timing events (raw hipEvent_t handles as ints, or torch.cuda.Events that have
    been recorded once so that their HIP events exist) to the next attention call's kernels on
    this thread (pkv_time_next_call): the elapsed time between them is that call's GPU time."""
    h = [e if isinstance(e, int) else e.cuda_event for e in (start, stop)]
    lib().pkv_time_next_call(ctypes.c_void_p(h[0]), ctypes.c_void_p(h[1]))


class BoundCall:
    """A library call with its arguments validated and converted to C values once; calling it
    repeats exactly that call (same tensors, same stream) with no per-call Python checks.  For
    tight loops such as a benchmark's timed region."""

    __slots__ = ("name", "fn", "args")

    def __init__(self, name: str, args: tuple):
        self.name = name
        self.fn = getattr(lib(), name)
        self.args = tuple(None if a is None else t(a) for t, a in zip(self.fn.argtypes, args))

    def __call__(self) -> None:
        rc = self.fn(*self.args)
        if rc != 0:
            _check(self.name, rc)


def _call(name: str, args: tuple, bind: bool):
    """Call the library now, or (bind=True) return the prepared call."""
    if bind:
        return BoundCall(name, args)
    _check(name, getattr(lib(), name)(*args))


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise PagedKVError(fn, status, status_string(status))


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


# ---- argument validation (before any call into the library).  The C ABI receives raw pointers
# and trusts the sizes it is given; these checks make sure the tensors really have the shapes
# the kernels index with.  Shapes and dtypes are checked first and the device last, so that
# every check can run on a machine without a GPU.

_KV16 = (torch.float16, torch.bfloat16)
_KV8 = (torch.uint8, torch.float8_e4m3fn)


def _shape(name: str, t: torch.Tensor, shape, dtype=None) -> None:
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(int(x) for x in shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")


def _pools(query_dtype, key_cache: torch.Tensor, value_cache: torch.Tensor):
    """(NB, BS, Hkv, D) of a K/V pool pair of the cache dtype a query dtype allows."""
    if key_cache.dim() != 4 or value_cache.shape != key_cache.shape or value_cache.dtype != key_cache.dtype:
        raise ValueError("key_cache and value_cache must both be [num_blocks, block_size, num_kv_heads, head_dim] "
                         "of one dtype")
    if query_dtype not in _KV16:
        raise ValueError(f"query dtype must be float16 or bfloat16, not {query_dtype}")
    if key_cache.dtype != query_dtype and key_cache.dtype not in _KV8:
        raise ValueError(f"a {key_cache.dtype} cache cannot be read with {query_dtype} queries")
    return tuple(key_cache.shape)


def _tables(block_tables: torch.Tensor, context_lens: torch.Tensor, B: int) -> None:
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise ValueError("block_tables and context_lens must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError(f"block_tables must be [{B}, max_blocks], got {tuple(block_tables.shape)}")
    if context_lens.dim() != 1 or context_lens.shape[0] != B:
        raise ValueError(f"context_lens must be [{B}], got {tuple(context_lens.shape)}")


def _workspace(tmp_out, max_logits, exp_sums, B: int, rows: int, P: int, D: int) -> None:
    """Split-K partials: tmp_out fp32 [B', rows, P, D], max_logits / exp_sums fp32 [B', rows, P]
    with B' >= B (the kernels index sequences b < B only, so a workspace sized for a larger
    batch serves a smaller one); rows may be given as two dims (q_len, num_heads)."""
    P = max(P, 1)
    for name, t, tail in (("tmp_out", tmp_out, (P, D)), ("max_logits", max_logits, (P,)),
                          ("exp_sums", exp_sums, (P,))):
        if t is None:
            raise ValueError(f"{name} is required for split-K")
        if t.dtype != torch.float32:
            raise ValueError(f"{name} must be float32")
        want = (B, rows) + tail
        lead = tuple(t.shape[:t.dim() - len(tail)])
        if tuple(t.shape[t.dim() - len(tail):]) != tail or len(lead) < 2 or lead[0] < B or \
                math.prod(lead[1:]) != rows:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {want}")


def _on_gpu(**tensors) -> None:
    dev = None
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor (it is on {t.device})")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the other tensors on {dev}")


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def paged_kv_write(key: torch.Tensor, value: torch.Tensor, key_cache: torch.Tensor,
                   value_cache: torch.Tensor, slot_mapping: torch.Tensor, k_scale: float = 1.0,
                   v_scale: float = 1.0, stream=None, bind: bool = False):
    """Scatter key/value [T, Hkv, D] into caches [NB, BS, Hkv, D] at slot_mapping [T] (int64).

    A uint8 / float8_e4m3fn cache is written as E4M3FN codes of x / scale."""
    if key.dim() != 3 or key.dtype not in _KV16:
        raise ValueError("key must be float16/bfloat16 [num_tokens, num_kv_heads, head_dim]")
    T, Hkv, D = key.shape
    NB, BS, Hkv2, D2 = _pools(key.dtype, key_cache, value_cache)
    if (Hkv2, D2) != (Hkv, D):
        raise ValueError("key rows and cache rows differ in num_kv_heads or head_dim")
    _shape("value", value, key.shape, key.dtype)
    _shape("slot_mapping", slot_mapping, (T,), torch.int64)
    _on_gpu(key=key, value=value, key_cache=key_cache, value_cache=value_cache, slot_mapping=slot_mapping)
    return _call("paged_kv_write", (_ptr(key), _ptr(value), _ptr(key_cache), _ptr(value_cache),
                              _ptr(slot_mapping), T, NB, BS, Hkv, D, _DT[key.dtype], _DT[key_cache.dtype],
                              float(k_scale), float(v_scale), _stream(stream)), bind)


def partial_slots(max_context_len: int, partition_size: int) -> int:
    """Partial slots per (sequence, row) of a split-K schedule (paged_attn_partial_slots)."""
    return int(lib().paged_attn_partial_slots(int(max_context_len), int(partition_size)))


def workspace_shapes(num_seqs: int, num_heads: int, head_dim: int, max_context_len: int,
                     partition_size: int):
    """(tmp_out, max_logits/exp_sums) shapes for a split-K schedule (partition_size != 0)."""
    P = max(1, partial_slots(max_context_len, partition_size))
    return (num_seqs, num_heads, P, head_dim), (num_seqs, num_heads, P)


def balanced_split(num_kv_heads: int, head_dim: int, q_dtype: torch.dtype, kv_dtype: torch.dtype) -> int:
    """partition_size value (< 0) for the balanced split that fills the current device once."""
    v = int(lib().paged_attn_balanced_split(num_kv_heads, head_dim, _DT[q_dtype], _DT[kv_dtype]))
    if v >= 0:
        raise PagedKVError("paged_attn_balanced_split", v, "no device / unsupported shape")
    return v


def multi_query_split(num_heads: int, num_kv_heads: int, head_dim: int, q_len: int, q_dtype: torch.dtype,
                      kv_dtype: torch.dtype) -> int:
    """partition_size value (< 0) of the balanced split that fills the current device for
    paged_attn_multi_query with q_len new tokens per sequence."""
    v = int(lib().paged_attn_multi_query_split(num_heads, num_kv_heads, head_dim, q_len, _DT[q_dtype],
                                               _DT[kv_dtype]))
    if v >= 0:
        raise PagedKVError("paged_attn_multi_query_split", v, "no device / unsupported shape")
    return v


def paged_attn_decode(out: Optional[torch.Tensor], query: torch.Tensor, key_cache: torch.Tensor,
                      value_cache: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor,
                      scale: float, max_context_len: int, partition_size: int = 0,
                      tmp_out: Optional[torch.Tensor] = None, max_logits: Optional[torch.Tensor] = None,
                      exp_sums: Optional[torch.Tensor] = None, k_scale: float = 1.0, v_scale: float = 1.0,
                      stream=None, shared_blocks: bool = False, bind: bool = False):
    """Decode attention; see include/pagedkv.h.  partition_size != 0 writes split-K partials.
    shared_blocks: some physical blocks appear in several table rows (keeps them cached)."""
    if query.dim() != 3:
        raise ValueError("query must be [num_seqs, num_heads, head_dim]")
    B, Hq, D = query.shape
    NB, BS, Hkv, D2 = _pools(query.dtype, key_cache, value_cache)
    if D2 != D:
        raise ValueError("query and cache head_dim differ")
    _tables(block_tables, context_lens, B)
    if out is not None:
        _shape("out", out, query.shape, query.dtype)
    if partition_size != 0:
        _workspace(tmp_out, max_logits, exp_sums, B, Hq, partial_slots(max_context_len, partition_size), D)
    _on_gpu(out=out, query=query, key_cache=key_cache, value_cache=value_cache, block_tables=block_tables,
            context_lens=context_lens, tmp_out=tmp_out, max_logits=max_logits, exp_sums=exp_sums)
    return _call("paged_attn_decode", (_ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache),
                                 _ptr(block_tables), block_tables.shape[1], _ptr(context_lens), B, Hq, Hkv,
                                 D, BS, NB, float(scale), _DT[query.dtype], _DT[key_cache.dtype],
                                 float(k_scale), float(v_scale), int(max_context_len), int(partition_size),
                                 _ptr(tmp_out), _ptr(max_logits), _ptr(exp_sums),
                                 PKV_FLAG_SHARED_BLOCKS if shared_blocks else 0, _stream(stream)), bind)


def paged_attn_multi_query(out: Optional[torch.Tensor], query: torch.Tensor, key_cache: torch.Tensor,
                           value_cache: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor,
                           scale: float, max_context_len: int, partition_size: int = 0,
                           tmp_out: Optional[torch.Tensor] = None, max_logits: Optional[torch.Tensor] = None,
                           exp_sums: Optional[torch.Tensor] = None, k_scale: float = 1.0, v_scale: float = 1.0,
                           stream=None, shared_blocks: bool = False, bind: bool = False):
    """query [B, L, Hq, D]: L new tokens per sequence, causal among themselves (include/pagedkv.h).
    Split-K partials have L * Hq rows per sequence: tmp_out [B, L * Hq, P, D]."""
    if query.dim() != 4:
        raise ValueError("query must be [num_seqs, q_len, num_heads, head_dim]")
    B, Lq, Hq, D = query.shape
    NB, BS, Hkv, D2 = _pools(query.dtype, key_cache, value_cache)
    if D2 != D:
        raise ValueError("query and cache head_dim differ")
    _tables(block_tables, context_lens, B)
    if out is not None:
        _shape("out", out, query.shape, query.dtype)
    if partition_size != 0:
        _workspace(tmp_out, max_logits, exp_sums, B, Lq * Hq, partial_slots(max_context_len, partition_size), D)
    _on_gpu(out=out, query=query, key_cache=key_cache, value_cache=value_cache, block_tables=block_tables,
            context_lens=context_lens, tmp_out=tmp_out, max_logits=max_logits, exp_sums=exp_sums)
    return _call("paged_attn_multi_query", (_ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache),
                                      _ptr(block_tables), block_tables.shape[1], _ptr(context_lens), B, Lq, Hq,
                                      Hkv, D, BS, NB, float(scale), _DT[query.dtype], _DT[key_cache.dtype],
                                      float(k_scale), float(v_scale), int(max_context_len), int(partition_size),
                                      _ptr(tmp_out), _ptr(max_logits), _ptr(exp_sums),
                                      PKV_FLAG_SHARED_BLOCKS if shared_blocks else 0, _stream(stream)), bind)


def multi_query(out: torch.Tensor, query, key_cache, value_cache, block_tables, context_lens, scale,
                ws: "DecodeWorkspace", k_scale=1.0, v_scale=1.0, stream=None, shared_blocks: bool = False) -> None:
    """paged_attn_multi_query, then paged_attn_reduce over q_len * Hq rows when split-K.

    ws must be a DecodeWorkspace for (num_seqs, q_len * num_heads, ...)."""
    PS = ws.partition_size
    B, Lq, Hq, D = query.shape
    paged_attn_multi_query(out if PS == 0 else None, query, key_cache, value_cache, block_tables, context_lens,
                           scale, ws.max_context_len, PS, ws.tmp_out, ws.max_logits, ws.exp_sums, k_scale, v_scale,
                           stream, shared_blocks)
    if PS != 0:
        paged_attn_reduce(out.view(B, Lq * Hq, D), ws.tmp_out, ws.max_logits, ws.exp_sums, context_lens,
                          ws.max_context_len, PS, stream)


def paged_attn_decode_noalloc(out: torch.Tensor, query: torch.Tensor, key_cache: torch.Tensor,
                              value_cache: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor,
                              scale: float, max_context_len: int, partition_size: int = 0, k_scale: float = 1.0,
                              v_scale: float = 1.0, stream=None, shared_blocks: bool = False, bind: bool = False):
    """Decode (and, for partition_size < 0, the merge) with the split-K partials in the
    library's fixed device scratch: no workspace, no allocation (include/pagedkv.h).  Calls that
    overlap on one GPU race on that scratch."""
    if query.dim() != 3:
        raise ValueError("query must be [num_seqs, num_heads, head_dim]")
    B, Hq, D = query.shape
    NB, BS, Hkv, D2 = _pools(query.dtype, key_cache, value_cache)
    if D2 != D:
        raise ValueError("query and cache head_dim differ")
    _tables(block_tables, context_lens, B)
    _shape("out", out, query.shape, query.dtype)
    _on_gpu(out=out, query=query, key_cache=key_cache, value_cache=value_cache, block_tables=block_tables,
            context_lens=context_lens)
    return _call("paged_attn_decode_noalloc", (
        _ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables), block_tables.shape[1],
        _ptr(context_lens), B, Hq, Hkv, D, BS, NB, float(scale), _DT[query.dtype], _DT[key_cache.dtype],
        float(k_scale), float(v_scale), int(max_context_len), int(partition_size),
        PKV_FLAG_SHARED_BLOCKS if shared_blocks else 0, _stream(stream)), bind)


def paged_attn_decode_append(out: Optional[torch.Tensor], query: torch.Tensor, key: torch.Tensor,
                             value: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
                             block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                             max_context_len: int, partition_size: int = 0,
                             tmp_out: Optional[torch.Tensor] = None, max_logits: Optional[torch.Tensor] = None,
                             exp_sums: Optional[torch.Tensor] = None, stream=None,
                             shared_blocks: bool = False, bind: bool = False):
    """Store key/value [B, Hkv, D] at position n - 1 of every sequence and decode, in one call
    (16-bit caches; include/pagedkv.h).  partition_size != 0 writes split-K partials."""
    if query.dim() != 3:
        raise ValueError("query must be [num_seqs, num_heads, head_dim]")
    B, Hq, D = query.shape
    NB, BS, Hkv, D2 = _pools(query.dtype, key_cache, value_cache)
    if D2 != D or key_cache.dtype != query.dtype:
        raise ValueError("paged_attn_decode_append needs 16-bit caches of the query dtype and head_dim")
    _shape("key", key, (B, Hkv, D), query.dtype)
    _shape("value", value, (B, Hkv, D), query.dtype)
    _tables(block_tables, context_lens, B)
    if out is not None:
        _shape("out", out, query.shape, query.dtype)
    if partition_size != 0:
        _workspace(tmp_out, max_logits, exp_sums, B, Hq, partial_slots(max_context_len, partition_size), D)
    _on_gpu(out=out, query=query, key=key, value=value, key_cache=key_cache, value_cache=value_cache,
            block_tables=block_tables, context_lens=context_lens, tmp_out=tmp_out, max_logits=max_logits,
            exp_sums=exp_sums)
    return _call("paged_attn_decode_append", (
        _ptr(out), _ptr(query), _ptr(key), _ptr(value), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables),
        block_tables.shape[1], _ptr(context_lens), B, Hq, Hkv, D, BS, NB, float(scale), _DT[query.dtype],
        int(max_context_len), int(partition_size), _ptr(tmp_out), _ptr(max_logits), _ptr(exp_sums),
        PKV_FLAG_SHARED_BLOCKS if shared_blocks else 0, _stream(stream)), bind)


def decode_append(out: torch.Tensor, query, key, value, key_cache, value_cache, block_tables, context_lens, scale,
                  ws: "DecodeWorkspace", stream=None, shared_blocks: bool = False) -> None:
    """paged_attn_decode_append, followed by paged_attn_reduce when the workspace is split-K."""
    PS = ws.partition_size
    paged_attn_decode_append(out if PS == 0 else None, query, key, value, key_cache, value_cache, block_tables,
                             context_lens, scale, ws.max_context_len, PS, ws.tmp_out, ws.max_logits, ws.exp_sums,
                             stream, shared_blocks)
    if PS != 0:
        paged_attn_reduce(out, ws.tmp_out, ws.max_logits, ws.exp_sums, context_lens, ws.max_context_len, PS,
                          stream)


def paged_attn_decode_shared_prefix(out: torch.Tensor, query: torch.Tensor, key_cache: torch.Tensor,
                                    value_cache: torch.Tensor, block_tables: torch.Tensor,
                                    context_lens: torch.Tensor, scale: float, max_context_len: int,
                                    prefix_len: int, prefix_partition_size: int, partition_size: int,
                                    tmp_out: torch.Tensor, max_logits: torch.Tensor, exp_sums: torch.Tensor,
                                    k_scale: float = 1.0, v_scale: float = 1.0, stream=None,
                                    shared_blocks: bool = False, bind: bool = False):
    """Decode of a batch whose rows share their first prefix_len tokens' blocks: prefix pass,
    suffix pass and merge in one call; writes out [B, Hq, D] (include/pagedkv.h)."""
    if query.dim() != 3:
        raise ValueError("query must be [num_seqs, num_heads, head_dim]")
    B, Hq, D = query.shape
    NB, BS, Hkv, D2 = _pools(query.dtype, key_cache, value_cache)
    if D2 != D:
        raise ValueError("query and cache head_dim differ")
    _tables(block_tables, context_lens, B)
    _shape("out", out, query.shape, query.dtype)
    P = int(lib().paged_attn_shared_prefix_slots(int(max_context_len), int(prefix_len), int(prefix_partition_size),
                                                 int(partition_size)))
    if P >= 0:                                          # invalid arguments: the library reports them
        _workspace(tmp_out, max_logits, exp_sums, B, Hq, P, D)
    _on_gpu(out=out, query=query, key_cache=key_cache, value_cache=value_cache, block_tables=block_tables,
            context_lens=context_lens, tmp_out=tmp_out, max_logits=max_logits, exp_sums=exp_sums)
    return _call("paged_attn_decode_shared_prefix", (
        _ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(block_tables), block_tables.shape[1],
        _ptr(context_lens), B, Hq, Hkv, D, BS, NB, float(scale), _DT[query.dtype], _DT[key_cache.dtype],
        float(k_scale), float(v_scale), int(max_context_len), int(prefix_len), int(prefix_partition_size),
        int(partition_size), _ptr(tmp_out), _ptr(max_logits), _ptr(exp_sums),
        PKV_FLAG_SHARED_BLOCKS if shared_blocks else 0, _stream(stream)), bind)


def prefix_split(num_seqs: int, num_heads: int, num_kv_heads: int, prefix_len: int) -> int:
    """prefix_partition_size that gives the prefix pass about one workgroup per compute unit."""
    v = int(lib().paged_attn_prefix_split(num_seqs, num_heads, num_kv_heads, prefix_len))
    if v <= 0:
        raise PagedKVError("paged_attn_prefix_split", v, "no device / invalid arguments")
    return v


class SharedPrefixWorkspace:
    """Partial buffers of paged_attn_decode_shared_prefix for a fixed shape and split."""

    def __init__(self, num_seqs, num_heads, num_kv_heads, head_dim, max_context_len, prefix_len, partition_size,
                 prefix_partition_size=None, device="cuda"):
        if prefix_partition_size is None:
            prefix_partition_size = prefix_split(num_seqs, num_heads, num_kv_heads, prefix_len) if prefix_len else 64
        self.max_context_len = max_context_len
        self.prefix_len = prefix_len
        self.partition_size = partition_size
        self.prefix_partition_size = prefix_partition_size
        P = int(lib().paged_attn_shared_prefix_slots(max_context_len, prefix_len, prefix_partition_size,
                                                     partition_size))
        if P < 0:
            raise PagedKVError("paged_attn_shared_prefix_slots", P, "invalid arguments")
        self.slots = P
        P = max(P, 1)
        self.tmp_out = torch.empty((num_seqs, num_heads, P, head_dim), dtype=torch.float32, device=device)
        self.max_logits = torch.empty((num_seqs, num_heads, P), dtype=torch.float32, device=device)
        self.exp_sums = torch.empty((num_seqs, num_heads, P), dtype=torch.float32, device=device)


def decode_shared_prefix(out: torch.Tensor, query, key_cache, value_cache, block_tables, context_lens, scale,
                         ws: SharedPrefixWorkspace, k_scale=1.0, v_scale=1.0, stream=None,
                         shared_blocks: bool = False, bind: bool = False):
    return paged_attn_decode_shared_prefix(out, query, key_cache, value_cache, block_tables, context_lens, scale,
                                           ws.max_context_len, ws.prefix_len, ws.prefix_partition_size,
                                           ws.partition_size, ws.tmp_out, ws.max_logits, ws.exp_sums, k_scale,
                                           v_scale, stream, shared_blocks, bind)


def paged_attn_reduce(out: torch.Tensor, tmp_out: torch.Tensor, max_logits: torch.Tensor,
                      exp_sums: torch.Tensor, context_lens: torch.Tensor, max_context_len: int,
                      partition_size: int, stream=None, bind: bool = False):
    """Log-sum-exp merge of split-K partials into out [B, Hq, D]."""
    if out.dim() != 3 or out.dtype not in _KV16:
        raise ValueError("out must be float16/bfloat16 [num_seqs, num_heads, head_dim]")
    B, Hq, D = out.shape
    if context_lens.dtype != torch.int32 or context_lens.dim() != 1 or context_lens.shape[0] != B:
        raise ValueError(f"context_lens must be int32 [{B}]")
    _workspace(tmp_out, max_logits, exp_sums, B, Hq, partial_slots(max_context_len, partition_size), D)
    _on_gpu(out=out, tmp_out=tmp_out, max_logits=max_logits, exp_sums=exp_sums, context_lens=context_lens)
    return _call("paged_attn_reduce", (_ptr(out), _ptr(tmp_out), _ptr(max_logits), _ptr(exp_sums),
                                 _ptr(context_lens), B, Hq, D, int(max_context_len), int(partition_size),
                                 _DT[out.dtype], _stream(stream)), bind)


def paged_attn_workspace_bytes(num_seqs: int, num_heads: int, head_dim: int, max_context_len: int,
                               partition_size: int) -> int:
    return int(lib().paged_attn_workspace_bytes(num_seqs, num_heads, head_dim, max_context_len,
                                                partition_size))


class DecodeWorkspace:
    """Preallocated split-K buffers for a fixed (B, Hq, D, max_context_len, partition_size)."""

    def __init__(self, num_seqs, num_heads, head_dim, max_context_len, partition_size, device="cuda"):
        self.partition_size = partition_size
        self.max_context_len = max_context_len
        if partition_size != 0:
            so, sm = workspace_shapes(num_seqs, num_heads, head_dim, max_context_len, partition_size)
            self.tmp_out = torch.empty(so, dtype=torch.float32, device=device)
            self.max_logits = torch.empty(sm, dtype=torch.float32, device=device)
            self.exp_sums = torch.empty(sm, dtype=torch.float32, device=device)
        else:
            self.tmp_out = self.max_logits = self.exp_sums = None


def decode(out: torch.Tensor, query, key_cache, value_cache, block_tables, context_lens, scale,
           ws: DecodeWorkspace, k_scale=1.0, v_scale=1.0, stream=None, shared_blocks: bool = False) -> None:
    """paged_attn_decode, followed by paged_attn_reduce when the workspace is split-K."""
    PS = ws.partition_size
    paged_attn_decode(out if PS == 0 else None, query, key_cache, value_cache, block_tables, context_lens,
                      scale, ws.max_context_len, PS, ws.tmp_out, ws.max_logits, ws.exp_sums, k_scale, v_scale,
                      stream, shared_blocks)
    if PS != 0:
        paged_attn_reduce(out, ws.tmp_out, ws.max_logits, ws.exp_sums, context_lens, ws.max_context_len, PS,
                          stream)


def paged_kv_copy_blocks(key_cache: torch.Tensor, value_cache: torch.Tensor, src_blocks: torch.Tensor,
                         dst_blocks: torch.Tensor, stream=None) -> None:
    """Copy whole blocks inside both pools (copy-on-write); src/dst are int32 device tensors."""
    if key_cache.dim() != 4 or value_cache.shape != key_cache.shape or value_cache.dtype != key_cache.dtype:
        raise ValueError("key_cache and value_cache must be [num_blocks, block_size, num_kv_heads, head_dim]")
    NB, BS, Hkv, D = key_cache.shape
    if src_blocks.dim() != 1 or src_blocks.shape != dst_blocks.shape:
        raise ValueError("src_blocks and dst_blocks must be 1-D of one length")
    if src_blocks.dtype != torch.int32 or dst_blocks.dtype != torch.int32:
        raise ValueError("block ids must be int32")
    _on_gpu(key_cache=key_cache, value_cache=value_cache, src_blocks=src_blocks, dst_blocks=dst_blocks)
    rc = lib().paged_kv_copy_blocks(_ptr(key_cache), _ptr(value_cache), _ptr(src_blocks), _ptr(dst_blocks),
                                    src_blocks.numel(), NB, BS, Hkv, D, _DT[key_cache.dtype], _stream(stream))
    _check("paged_kv_copy_blocks", rc)


def paged_kv_swap_blocks(key_cache: torch.Tensor, value_cache: torch.Tensor, host_key: torch.Tensor,
                         host_value: torch.Tensor, dev_blocks: torch.Tensor, host_blocks: torch.Tensor,
                         to_host: bool, stream=None) -> None:
    """Move whole blocks between the device pools and pinned host pools (same block shape).

    host_key / host_value must be pinned CPU tensors (pin_memory=True); ids are int32 device
    tensors."""
    if key_cache.dim() != 4 or value_cache.shape != key_cache.shape or value_cache.dtype != key_cache.dtype:
        raise ValueError("key_cache and value_cache must be [num_blocks, block_size, num_kv_heads, head_dim]")
    NB, BS, Hkv, D = key_cache.shape
    NH = host_key.shape[0]
    if host_key.shape[1:] != key_cache.shape[1:] or host_value.shape != host_key.shape:
        raise ValueError("host pools must have the device pools' block shape")
    if dev_blocks.dim() != 1 or dev_blocks.shape != host_blocks.shape or dev_blocks.dtype != torch.int32 or \
            host_blocks.dtype != torch.int32:
        raise ValueError("dev_blocks and host_blocks must be int32, 1-D of one length")
    if host_key.dtype != key_cache.dtype or host_value.dtype != key_cache.dtype or host_key.is_cuda or \
            host_value.is_cuda:
        raise ValueError("host pools must be CPU tensors of the cache dtype")
    _on_gpu(key_cache=key_cache, value_cache=value_cache, dev_blocks=dev_blocks, host_blocks=host_blocks)
    if not (host_key.is_pinned() and host_value.is_pinned()):
        raise ValueError("host pools must be pinned (pin_memory=True)")
    rc = lib().paged_kv_swap_blocks(_ptr(key_cache), _ptr(value_cache), _ptr(host_key), _ptr(host_value),
                                    _ptr(dev_blocks), _ptr(host_blocks), dev_blocks.numel(), NB, NH, BS, Hkv, D,
                                    _DT[key_cache.dtype], 1 if to_host else 0, _stream(stream))
    _check("paged_kv_swap_blocks", rc)


class BlockManager:
    """Host block manager of the native library (see include/pagedkv.h: refcounted blocks,
    copy-on-write forks, swap bookkeeping, lowest-free-block-first allocation)."""

    def __init__(self, num_blocks: int, block_size: int, num_host_blocks: int = 0):
        self._h = lib().pkv_bm_create(num_blocks, block_size, num_host_blocks)
        if not self._h:
            raise PagedKVError("pkv_bm_create", PKV_ERR_SHAPE, "bad sizes or out of memory")
        self.num_blocks, self.block_size, self.num_host_blocks = num_blocks, block_size, num_host_blocks

    def __del__(self):
        h = getattr(self, "_h", None)
        if h and _lib is not None:
            _lib.pkv_bm_destroy(h)
            self._h = None

    def _call(self, fn, *args):
        rc = getattr(lib(), fn)(self._h, *args)
        if rc < 0:
            raise PagedKVError(fn, rc, status_string(rc))
        return rc

    def num_free(self) -> int:
        return self._call("pkv_bm_num_free")

    def num_free_host(self) -> int:
        return self._call("pkv_bm_num_free_host")

    def add(self, seq_id: int, num_tokens: int) -> None:
        self._call("pkv_bm_add", seq_id, num_tokens)

    def append(self, seq_id: int):
        """-> (slot, copy_src, copy_dst); copy ids are -1 when no copy-on-write was needed."""
        slot, cs, cd = ctypes.c_int64(), ctypes.c_int32(), ctypes.c_int32()
        self._call("pkv_bm_append", seq_id, ctypes.byref(slot), ctypes.byref(cs), ctypes.byref(cd))
        return slot.value, cs.value, cd.value

    def fork(self, parent: int, child: int, num_tokens: int = -1) -> None:
        self._call("pkv_bm_fork", parent, child, num_tokens)

    def free(self, seq_id: int) -> None:
        self._call("pkv_bm_free", seq_id)

    def num_tokens(self, seq_id: int) -> int:
        n = ctypes.c_int64()
        self._call("pkv_bm_num_tokens", seq_id, ctypes.byref(n))
        return n.value

    def _swap(self, fn, seq_id, capacity):
        a = (ctypes.c_int32 * max(1, capacity))()
        b = (ctypes.c_int32 * max(1, capacity))()
        n = self._call(fn, seq_id, a, b, capacity)
        return list(a[:n]), list(b[:n])

    def swap_out(self, seq_id: int, capacity: int = 1 << 16):
        """-> (device blocks, host blocks) to copy device -> host."""
        return self._swap("pkv_bm_swap_out", seq_id, capacity)

    def swap_in(self, seq_id: int, capacity: int = 1 << 16):
        """-> (host blocks, device blocks) to copy host -> device."""
        return self._swap("pkv_bm_swap_in", seq_id, capacity)

    def table(self, seq_ids, max_blocks: int):
        """-> (block_tables int32 [n, max_blocks], context_lens int32 [n]) as numpy arrays."""
        import numpy as np
        ids = np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int64))
        bt = np.zeros((len(ids), max_blocks), dtype=np.int32)
        lens = np.zeros(len(ids), dtype=np.int32)
        self._call("pkv_bm_table", ids.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), len(ids),
                   bt.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), max_blocks,
                   lens.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)))
        return bt, lens

    def check(self) -> bool:
        """True if the reference-count invariant and the per-sequence block bound hold."""
        rc = lib().pkv_bm_check(self._h)
        return rc == 0

"""ctypes binding of libpagedkv.so (C ABI in include/pagedkv.h).

Argument marshalling only: shapes become ints, tensors become device pointers, the stream is
torch's current HIP stream.  Every computation runs in the library's HIP kernels.  If the
library has not been built, every call raises ``PagedKVError``; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# PAGEDKV_LIB may name another build of the same library (same ABI); default: the in-tree one.
LIB_PATH = os.environ.get("PAGEDKV_LIB") or os.path.join(_HERE, "libpagedkv.so")

PKV_F16, PKV_BF16, PKV_FP8_E4M3 = 0, 1, 2
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
                                        P, P]
        L.paged_attn_decode.restype = I
        L.paged_attn_reduce.argtypes = [P, P, P, P, P, I, I, I, I, I, I, P]
        L.paged_attn_reduce.restype = I
        L.paged_attn_workspace_bytes.argtypes = [I, I, I, I, I]
        L.paged_attn_workspace_bytes.restype = ctypes.c_size_t
        L.paged_attn_partial_slots.argtypes = [I, I]
        L.paged_attn_partial_slots.restype = I
        L.paged_attn_balanced_split.argtypes = [I, I, I, I]
        L.paged_attn_balanced_split.restype = I
        L.pkv_status_string.argtypes = [I]
        L.pkv_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().pkv_status_string(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise PagedKVError(fn, status, status_string(status))


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def paged_kv_write(key: torch.Tensor, value: torch.Tensor, key_cache: torch.Tensor,
                   value_cache: torch.Tensor, slot_mapping: torch.Tensor, k_scale: float = 1.0,
                   v_scale: float = 1.0, stream=None) -> None:
    """Scatter key/value [T, Hkv, D] into caches [NB, BS, Hkv, D] at slot_mapping [T] (int64).

    A uint8 / float8_e4m3fn cache is written as E4M3FN codes of x / scale."""
    T, Hkv, D = key.shape
    NB, BS, Hkv2, D2 = key_cache.shape
    if (Hkv2, D2) != (Hkv, D) or value.shape != key.shape or value_cache.shape != key_cache.shape:
        raise ValueError("shape mismatch")
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (T,):
        raise ValueError("slot_mapping must be int64 [T]")
    rc = lib().paged_kv_write(_ptr(key), _ptr(value), _ptr(key_cache), _ptr(value_cache),
                              _ptr(slot_mapping), T, NB, BS, Hkv, D, _DT[key.dtype], _DT[key_cache.dtype],
                              float(k_scale), float(v_scale), _stream(stream))
    _check("paged_kv_write", rc)


def workspace_shapes(num_seqs: int, num_heads: int, head_dim: int, max_context_len: int,
                     partition_size: int):
    """(tmp_out, max_logits/exp_sums) shapes for a split-K schedule (partition_size != 0)."""
    P = max(1, int(lib().paged_attn_partial_slots(int(max_context_len), int(partition_size))))
    return (num_seqs, num_heads, P, head_dim), (num_seqs, num_heads, P)


def balanced_split(num_kv_heads: int, head_dim: int, q_dtype: torch.dtype, kv_dtype: torch.dtype) -> int:
    """partition_size value (< 0) for the balanced split that fills the current device once."""
    v = int(lib().paged_attn_balanced_split(num_kv_heads, head_dim, _DT[q_dtype], _DT[kv_dtype]))
    if v >= 0:
        raise PagedKVError("paged_attn_balanced_split", v, "no device / unsupported shape")
    return v


def paged_attn_decode(out: Optional[torch.Tensor], query: torch.Tensor, key_cache: torch.Tensor,
                      value_cache: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor,
                      scale: float, max_context_len: int, partition_size: int = 0,
                      tmp_out: Optional[torch.Tensor] = None, max_logits: Optional[torch.Tensor] = None,
                      exp_sums: Optional[torch.Tensor] = None, k_scale: float = 1.0, v_scale: float = 1.0,
                      stream=None) -> None:
    """Decode attention; see include/pagedkv.h.  partition_size > 0 writes split-K partials."""
    B, Hq, D = query.shape
    NB, BS, Hkv, D2 = key_cache.shape
    if D2 != D or value_cache.shape != key_cache.shape:
        raise ValueError("shape mismatch")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise ValueError("block_tables and context_lens must be int32")
    rc = lib().paged_attn_decode(_ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache),
                                 _ptr(block_tables), block_tables.shape[1], _ptr(context_lens), B, Hq, Hkv,
                                 D, BS, NB, float(scale), _DT[query.dtype], _DT[key_cache.dtype],
                                 float(k_scale), float(v_scale), int(max_context_len), int(partition_size),
                                 _ptr(tmp_out), _ptr(max_logits), _ptr(exp_sums), _stream(stream))
    _check("paged_attn_decode", rc)


def paged_attn_reduce(out: torch.Tensor, tmp_out: torch.Tensor, max_logits: torch.Tensor,
                      exp_sums: torch.Tensor, context_lens: torch.Tensor, max_context_len: int,
                      partition_size: int, stream=None) -> None:
    """Log-sum-exp merge of split-K partials into out [B, Hq, D]."""
    B, Hq, D = out.shape
    rc = lib().paged_attn_reduce(_ptr(out), _ptr(tmp_out), _ptr(max_logits), _ptr(exp_sums),
                                 _ptr(context_lens), B, Hq, D, int(max_context_len), int(partition_size),
                                 _DT[out.dtype], _stream(stream))
    _check("paged_attn_reduce", rc)


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
           ws: DecodeWorkspace, k_scale=1.0, v_scale=1.0, stream=None) -> None:
    """paged_attn_decode, followed by paged_attn_reduce when the workspace is split-K."""
    PS = ws.partition_size
    paged_attn_decode(out if PS == 0 else None, query, key_cache, value_cache, block_tables, context_lens,
                      scale, ws.max_context_len, PS, ws.tmp_out, ws.max_logits, ws.exp_sums, k_scale, v_scale,
                      stream)
    if PS != 0:
        paged_attn_reduce(out, ws.tmp_out, ws.max_logits, ws.exp_sums, context_lens, ws.max_context_len, PS,
                          stream)

"""fp64 CPU oracle for paged-attention decode -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline leg may import
this package.  The product library never links, includes or calls it, and it shares no
code with the HIP kernels.

The arithmetic lives in ``pagedkv_oracle.c`` (plain C, fp64, OpenMP over (sequence, head)).
This module builds it with gcc and marshals numpy/torch CPU arrays through ctypes.

Functions:
  attn(...)            softmax(scale * q K^T) V through the block table, fp64
  attn_partials(...)   the same per token partition: (m, l, o) partials
  lse_merge(...)       log-sum-exp merge of partials
  kv_write(...)        byte-exact scatter of new K/V rows into pool slots (fp8 quantising)
  fp8_encode / fp8_decode   OCP E4M3FN codec (fp32 division, nearest-even, saturating)
  quantize_pool(...)   a whole pool through the codec
  attn_multi_query(...)  L new tokens per sequence, causal among themselves (loops over attn)
  copy_blocks(...)     whole-block copies (copy-on-write), reading the pools as before the call
  swap_blocks(...)     whole blocks between the device pools and host pools, either direction
The host block manager's reference model is ``oracle/block_manager.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pagedkv_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle_pagedkv.so")
_lib: Optional[ctypes.CDLL] = None

DT_CODE = {"f16": 0, "bf16": 1, "fp8": 2}
TORCH_DT = {torch.float16: 0, torch.bfloat16: 1, torch.uint8: 2}


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
               "-std=c99", "-Wall", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        P, I, I64, D_ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        lib.oracle_attn.argtypes = [P, I, P, P, I, P, I, P, I, I, I, I, I, D_, D_, D_, P, I]
        lib.oracle_attn.restype = I
        lib.oracle_attn_partials.argtypes = [P, I, P, P, I, P, I, P, I, I, I, I, I, D_, D_, D_, I, I,
                                             P, P, P, I]
        lib.oracle_attn_partials.restype = I
        lib.oracle_lse_merge.argtypes = [P, P, P, P, I64, I, I, P]
        lib.oracle_lse_merge.restype = None
        lib.oracle_kv_write.argtypes = [P, P, P, P, P, I64, I64, I, I, I, I, I, ctypes.c_float,
                                        ctypes.c_float]
        lib.oracle_kv_write.restype = I
        lib.oracle_fp8_encode_array.argtypes = [P, I64, ctypes.c_float, P]
        lib.oracle_fp8_encode_array.restype = None
        lib.oracle_fp8_decode_array.argtypes = [P, I64, P]
        lib.oracle_fp8_decode_array.restype = None
        _lib = lib
    return _lib


def default_threads() -> int:
    return len(os.sched_getaffinity(0))


def _ptr(x) -> int:
    if isinstance(x, torch.Tensor):
        assert x.device.type == "cpu" and x.is_contiguous()
        return x.data_ptr()
    assert isinstance(x, np.ndarray) and x.flags["C_CONTIGUOUS"]
    return x.ctypes.data


def _dt(x, kv_dtype: Optional[str] = None) -> int:
    if kv_dtype is not None:
        return DT_CODE[kv_dtype]
    return TORCH_DT[x.dtype]


def attn(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_tables: np.ndarray,
         context_lens: np.ndarray, scale: float, k_scale: float = 1.0, v_scale: float = 1.0,
         kv_dtype: Optional[str] = None, nthreads: Optional[int] = None) -> np.ndarray:
    """fp64 [B, Hq, D] = softmax(scale * q K^T) V per (sequence, head), K/V via the table.

    Pools are [NB, BS, Hkv, D] (fp16/bf16 tensors, or uint8 holding E4M3FN codes)."""
    lib = _load()
    B, Hq, D = q.shape
    NB, BS, Hkv, D2 = k_cache.shape
    assert D2 == D and v_cache.shape == k_cache.shape
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    assert bt.shape[0] == B and lens.shape == (B,)
    used = -(-lens.astype(np.int64) // BS)
    for b in range(B):
        assert np.all((bt[b, :used[b]] >= 0) & (bt[b, :used[b]] < NB)), "block id out of range"
    out = np.zeros((B, Hq, D), dtype=np.float64)
    rc = lib.oracle_attn(_ptr(q), _dt(q), _ptr(k_cache), _ptr(v_cache), _dt(k_cache, kv_dtype), _ptr(bt),
                         bt.shape[1], _ptr(lens), B, Hq, Hkv, D, BS, float(scale), float(k_scale),
                         float(v_scale), out.ctypes.data, nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle_attn rejected its arguments ({rc})")
    return out


def attn_partials(q, k_cache, v_cache, block_tables, context_lens, scale, partition_size,
                  k_scale=1.0, v_scale=1.0, kv_dtype=None, nthreads=None, Pmax=None):
    """Per-partition partials (m [B,Hq,Pmax], l [B,Hq,Pmax], o [B,Hq,Pmax,D]); unused = NaN."""
    lib = _load()
    B, Hq, D = q.shape
    NB, BS, Hkv, _ = k_cache.shape
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    if Pmax is None:
        Pmax = max(1, int(-(-lens.max() // partition_size))) if B else 1
    m = np.full((B, Hq, Pmax), np.nan)
    l = np.full((B, Hq, Pmax), np.nan)
    o = np.full((B, Hq, Pmax, D), np.nan)
    rc = lib.oracle_attn_partials(_ptr(q), _dt(q), _ptr(k_cache), _ptr(v_cache), _dt(k_cache, kv_dtype),
                                  _ptr(bt), bt.shape[1], _ptr(lens), B, Hq, Hkv, D, BS, float(scale),
                                  float(k_scale), float(v_scale), int(partition_size), int(Pmax),
                                  m.ctypes.data, l.ctypes.data, o.ctypes.data,
                                  nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle_attn_partials rejected its arguments ({rc})")
    return m, l, o


def lse_merge(m: np.ndarray, l: np.ndarray, o: np.ndarray, nparts: np.ndarray) -> np.ndarray:
    """Merge partials [R, Pmax], [R, Pmax], [R, Pmax, D] over the first nparts[r] entries."""
    lib = _load()
    m = np.ascontiguousarray(m, dtype=np.float64)
    l = np.ascontiguousarray(l, dtype=np.float64)
    o = np.ascontiguousarray(o, dtype=np.float64)
    R, Pmax = m.shape
    D = o.shape[-1]
    npar = np.ascontiguousarray(nparts, dtype=np.int32).reshape(R)
    out = np.zeros((R, D), dtype=np.float64)
    lib.oracle_lse_merge(m.ctypes.data, l.ctypes.data, o.ctypes.data, npar.ctypes.data, R, Pmax, D,
                         out.ctypes.data)
    return out


def kv_write(key: torch.Tensor, value: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
             slot_mapping: np.ndarray, k_scale: float = 1.0, v_scale: float = 1.0) -> None:
    """In-place scatter of key/value [T, Hkv, D] into caches [NB, BS, Hkv, D] (uint8 = fp8)."""
    lib = _load()
    T, Hkv, D = key.shape
    NB, BS, Hkv2, D2 = key_cache.shape
    assert (Hkv2, D2) == (Hkv, D) and value.shape == key.shape and value_cache.shape == key_cache.shape
    sm = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    assert sm.shape == (T,)
    rc = lib.oracle_kv_write(_ptr(key), _ptr(value), _ptr(key_cache), _ptr(value_cache), sm.ctypes.data,
                             T, NB, BS, Hkv, D, _dt(key), _dt(key_cache), float(k_scale), float(v_scale))
    if rc != 0:
        raise ValueError("oracle_kv_write: slot outside the pool")


def fp8_encode(x: torch.Tensor, scale: float) -> torch.Tensor:
    """E4M3FN codes (uint8) of fp32(x) / fp32(scale), nearest-even, saturating at +-448."""
    lib = _load()
    xf = x.detach().to(torch.float32).contiguous().cpu()
    out = torch.empty(xf.shape, dtype=torch.uint8)
    lib.oracle_fp8_encode_array(xf.data_ptr(), xf.numel(), float(scale), out.data_ptr())
    return out


def fp8_decode(codes) -> np.ndarray:
    """fp64 values of E4M3FN codes (NaN for S.1111.111)."""
    lib = _load()
    c = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8))
    out = np.empty(c.shape, dtype=np.float64)
    lib.oracle_fp8_decode_array(c.ctypes.data, c.size, out.ctypes.data)
    return out


def quantize_pool(pool: torch.Tensor, scale: float) -> torch.Tensor:
    """Whole-pool fp8 quantisation, element by element through fp8_encode."""
    return fp8_encode(pool, scale).view(pool.shape)


def copy_blocks(k_cache: torch.Tensor, v_cache: torch.Tensor, src, dst) -> None:
    """Copy-on-write data copies ("vllm-project-vllm -- L2", section 9, COW sharing): block
    dst[i] of each pool becomes block src[i] as the pools were before the call.  In place on
    CPU pools [num_blocks, block_size, Hkv, D] of any dtype (bytes are moved unchanged)."""
    k0, v0 = k_cache.clone(), v_cache.clone()
    for s, d in zip(np.asarray(src).tolist(), np.asarray(dst).tolist()):
        k_cache[d] = k0[s]
        v_cache[d] = v0[s]


def swap_blocks(k_cache: torch.Tensor, v_cache: torch.Tensor, host_k: torch.Tensor, host_v: torch.Tensor,
                dev_blocks, host_blocks, to_host: bool) -> None:
    """Swapping blocks to host memory and back ("vllm-project-vllm -- L2", section 9):
    to_host copies device block dev_blocks[i] into host block host_blocks[i], else the reverse.
    In place on CPU tensors of the same block shape."""
    for d, h in zip(np.asarray(dev_blocks).tolist(), np.asarray(host_blocks).tolist()):
        if to_host:
            host_k[h] = k_cache[d]
            host_v[h] = v_cache[d]
        else:
            k_cache[d] = host_k[h]
            v_cache[d] = host_v[h]


def attn_multi_query(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_tables: np.ndarray,
                     context_lens: np.ndarray, scale: float, k_scale: float = 1.0, v_scale: float = 1.0,
                     kv_dtype: Optional[str] = None, nthreads: Optional[int] = None) -> np.ndarray:
    """fp64 [B, L, Hq, D] for L new query tokens per sequence, causal among themselves.

    Speculative verification scores k draft tokens in one pass ("vLLM vs vllm", speculative
    decoding) and chunked prefill feeds several new tokens of a sequence at once ("L2", the
    mechanisms table): the L new tokens are the last L of the sequence's n cached tokens, and
    new token i (position n - L + i) sees exactly the tokens up to and including itself.  So
    query i is a one-token decode over the first clip(n - L + 1 + i, 0, n) tokens."""
    B, L, Hq, D = q.shape
    lens = np.asarray(context_lens, dtype=np.int64)
    out = np.zeros((B, L, Hq, D), dtype=np.float64)
    for i in range(L):
        vis = np.clip(lens - L + 1 + i, 0, lens).astype(np.int32)
        out[:, i] = attn(q[:, i].contiguous(), k_cache, v_cache, block_tables, vis, scale, k_scale, v_scale,
                         kv_dtype, nthreads)
    return out

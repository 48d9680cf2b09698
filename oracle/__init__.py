"""Paged-attention oracle: a slow, plain fp64 CPU implementation.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this package. The product library
(`paged_kv_cache_slot_amd`) never imports, loads or calls it; the two share no
code.

The arithmetic lives in `oracle.cpp` (built into `liboracle.so` by `build.py`).
This module only marshals numpy arrays into that library's C entry points.
bf16 tensors travel as uint16 arrays holding the raw bf16 bits.

What each function computes, and the passages it follows, is stated beside the
C entry points in `oracle.cpp`:
  store_kvcache  -- "nano-vllm 深度分析报告", table 可复用的模式与技巧,
                    row "slot_mapping -1 padding"
  decode         -- "DeepSeek研究员1200行代码复刻vLLM…", section "vLLM是什么？"
  prefill        -- the same section, plus prefix caching from the feature
                    lists of both pages
"""
import ctypes
import os

import numpy as np

from .build import LIB, build_oracle

_lib = None

_ERRORS = {1: "bad argument", 2: "metadata out of range"}


def load(path=None):
    """Loads liboracle.so (building it first if it is missing)."""
    global _lib
    if path is None:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB):
            build_oracle()
        path = LIB
    lib = ctypes.CDLL(path)
    p = ctypes.c_void_p
    i32 = ctypes.c_int32
    i64 = ctypes.c_int64
    lib.oracle_store_kvcache.argtypes = [p, p, i64, p, p, p, i32, i32, i32, i32, i32]
    lib.oracle_store_kvcache.restype = ctypes.c_int
    lib.oracle_decode.argtypes = [p, p, p, p, p, i32, p, i32, i32, i32, i32, i32,
                                  i32, ctypes.c_double, p, i32, i32]
    lib.oracle_decode.restype = ctypes.c_int
    lib.oracle_prefill.argtypes = [p, p, p, p, p, p, p, i32, i32, i32, i32, i32,
                                   i32, i32, i32, ctypes.c_double, p, i32, i32]
    lib.oracle_prefill.restype = ctypes.c_int
    lib.oracle_hardware_threads.argtypes = []
    lib.oracle_hardware_threads.restype = ctypes.c_int32
    if path == LIB:
        _lib = lib
    return lib


def _u16(a):
    """Raw bf16 bits as a C-contiguous uint16 array (accepts torch CPU tensors)."""
    if hasattr(a, "detach"):
        import torch
        a = a.detach().contiguous().view(torch.int16).numpy()
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        a = a.view(np.uint16)
    return a


def _u16_rows(a):
    """2-D uint16 view whose rows may be strided (elements contiguous within a row).

    Returns (array, row_stride_in_elements) without copying strided rows, so a
    row slice of a wider fused buffer is passed as it lies in memory.
    """
    if hasattr(a, "detach"):
        import torch
        a = a.detach().view(torch.int16).numpy()
    a = a.view(np.uint16) if a.dtype != np.uint16 else a
    a = a.reshape(a.shape[0], -1) if a.ndim != 2 else a
    if a.strides[1] != 2 or a.strides[0] % 2:
        a = np.ascontiguousarray(a)
    return a, a.strides[0] // 2


def _i32(a):
    if hasattr(a, "detach"):
        a = a.detach().cpu().numpy()
    return np.ascontiguousarray(a, dtype=np.int32)


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what}: {_ERRORS.get(rc, rc)}")


def hardware_threads(lib=None):
    return int((lib or load()).oracle_hardware_threads())


def store_kvcache(k, v, k_cache, v_cache, slot_mapping, block_size, lib=None, inplace=False):
    """Returns (k_cache, v_cache) uint16 pools after the store.

    k, v: [T, Hkv, D] (or [T, >= Hkv*D] rows: the token stride is taken from the
    array); pools: [num_blocks, block_size, Hkv, D]. The inputs are not changed,
    unless inplace=True and the pools are C-contiguous uint16 numpy arrays, which
    are then written in place and returned.
    """
    lib = lib or load()
    if inplace:
        kc, vc = k_cache, v_cache
        assert kc.dtype == np.uint16 and kc.flags.c_contiguous and vc.flags.c_contiguous
    else:
        kc = _u16(k_cache).copy()
        vc = _u16(v_cache).copy()
    num_blocks, bs, hkv, d = kc.shape
    assert bs == block_size
    k, k_stride = _u16_rows(k)
    v, v_stride = _u16_rows(v)
    assert k.shape == v.shape and k.shape[1] >= hkv * d and k_stride == v_stride
    sm = _i32(slot_mapping)
    _check(lib.oracle_store_kvcache(_ptr(k), _ptr(v), k_stride, _ptr(kc), _ptr(vc),
                                    _ptr(sm), len(sm), num_blocks, block_size, hkv, d),
           "store_kvcache")
    return kc, vc


def decode(q, k_cache, v_cache, block_table, context_lens, scale, rows=None,
           nthreads=1, lib=None):
    """fp64 output [B, Hq, D] of paged decode (rows not in `rows` stay 0)."""
    lib = lib or load()
    q = _u16(q)
    kc, vc = _u16(k_cache), _u16(v_cache)
    bt, cl = _i32(block_table), _i32(context_lens)
    B, hq, d = q.shape
    num_blocks, bs, hkv, d2 = kc.shape
    assert d == d2 and bt.shape[0] == B and cl.shape == (B,)
    out = np.zeros((B, hq, d), dtype=np.float64)
    r = _i32(rows) if rows is not None else None
    _check(lib.oracle_decode(_ptr(out), _ptr(q), _ptr(kc), _ptr(vc), _ptr(bt), bt.shape[1],
                             _ptr(cl), B, hq, hkv, d, bs, num_blocks, float(scale), _ptr(r),
                             0 if r is None else len(r), nthreads),
           "decode")
    return out


def prefill(q, k_cache, v_cache, cu_seqlens_q, context_lens, block_table, scale,
            tokens=None, nthreads=1, lib=None):
    """fp64 output [total_q, Hq, D] of causal varlen prefill with cached prefix."""
    lib = lib or load()
    q = _u16(q)
    kc, vc = _u16(k_cache), _u16(v_cache)
    cu, cl, bt = _i32(cu_seqlens_q), _i32(context_lens), _i32(block_table)
    total_q, hq, d = q.shape
    num_blocks, bs, hkv, d2 = kc.shape
    B = len(cl)
    assert d == d2 and len(cu) == B + 1 and bt.shape[0] == B
    out = np.zeros((total_q, hq, d), dtype=np.float64)
    t = _i32(tokens) if tokens is not None else None
    _check(lib.oracle_prefill(_ptr(out), _ptr(q), _ptr(kc), _ptr(vc), _ptr(cu), _ptr(cl),
                              _ptr(bt), bt.shape[1], B, total_q, hq, hkv, d, bs, num_blocks,
                              float(scale), _ptr(t), 0 if t is None else len(t), nthreads),
           "prefill")
    return out

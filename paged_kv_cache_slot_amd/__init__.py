"""Paged KV-cache attention for AMD Instinct MI355X (gfx950).

A thin ctypes binding over libpa.so (C ABI in include/pa.h). Each function has
the name of the C entry point it calls and only marshals arguments: torch
tensors become device pointers and sizes, and the stream defaults to torch's
current stream. Every step of the computation runs in the HIP kernels of
libpa.so; there is no fallback. If libpa.so has not been built, every call
raises.

  pa_store_kvcache   write new tokens' K/V into the paged pools (slot -1 skipped)
  pa_decode          one query token per sequence over its paged context
  pa_prefill_varlen  causal varlen prefill over a cached prefix plus new tokens
  pa_sample_gumbel   Gumbel-max token sampling from per-row probabilities
  pa_decode_graphs_create  HIP graphs of the whole decode step (store + decode)
                     at a few batch-size buckets, replayed with one launch

The host-side block manager that produces their metadata (block tables, slot
mappings, lengths) with chained-hash prefix caching is bound in
`paged_kv_cache_slot_amd.block_manager`.
"""
import ctypes
import os

__all__ = ["PAError", "library", "lib_path", "pa_store_kvcache", "pa_decode", "pa_decode_store",
           "pa_decode_store_noalloc",
           "pa_decode_workspace_bytes", "pa_prefill_varlen", "pa_validate_metadata",
           "pa_status_string", "pa_sample_workspace_bytes", "pa_sample_gumbel",
           "pa_decode_graphs_create", "DecodeGraphs", "DEFAULT_BUCKETS",
           "EXPORTED_SYMBOLS"]

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libpa.so")

EXPORTED_SYMBOLS = ("pa_status_string", "pa_store_kvcache", "pa_decode_workspace_bytes",
                    "pa_decode", "pa_decode_store", "pa_decode_store_noalloc", "pa_prefill_varlen",
                    "pa_validate_metadata",
                    # block manager (include/pa_block_manager.h, block_manager.py)
                    "pa_xxh64", "pa_block_hash", "pa_bm_create", "pa_bm_destroy",
                    "pa_bm_num_free_blocks", "pa_bm_can_allocate", "pa_bm_allocate",
                    "pa_bm_can_append", "pa_bm_append", "pa_bm_append_batch", "pa_bm_deallocate", "pa_bm_seq_info",
                    "pa_bm_block_table", "pa_bm_block_info", "pa_bm_stats",
                    "pa_bm_batch_info", "pa_bm_prefill_metadata", "pa_bm_decode_metadata",
                    "pa_kv_cache_num_blocks",
                    # sampler
                    "pa_sample_workspace_bytes", "pa_sample_gumbel",
                    # decode-step graphs
                    "pa_decode_graphs_create", "pa_decode_graphs_bucket",
                    "pa_decode_graphs_launch", "pa_decode_graphs_destroy")

_lib = None


class _StepBuffers(ctypes.Structure):
    """pa_decode_step_buffers (include/pa.h), field for field."""
    _fields_ = [("out", ctypes.c_void_p), ("q", ctypes.c_void_p), ("k_new", ctypes.c_void_p),
                ("v_new", ctypes.c_void_p), ("kv_token_stride", ctypes.c_int64),
                ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
                ("slot_mapping", ctypes.c_void_p), ("context_lens", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("block_table_stride", ctypes.c_int32),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("max_context_len", ctypes.c_int32),
                ("scale", ctypes.c_float)]


class PAError(RuntimeError):
    """A libpa.so call returned a non-zero status."""

    def __init__(self, name, status, detail=""):
        self.status = status
        msg = f"{name}: {pa_status_string(status)} (status {status})"
        super().__init__(msg + (f": {detail}" if detail else ""))


def library():
    """The loaded libpa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(lib_path):
            raise RuntimeError(f"{lib_path} is missing: build it with "
                               "`python -m paged_kv_cache_slot_amd.build` (hipcc, gfx950)")
        lib = ctypes.CDLL(lib_path)
        p, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        lib.pa_status_string.argtypes = [ctypes.c_int]
        lib.pa_status_string.restype = ctypes.c_char_p
        lib.pa_store_kvcache.argtypes = [p, p, i64, p, p, p, i32, i32, i32, i32, i32, p]
        lib.pa_store_kvcache.restype = ctypes.c_int
        lib.pa_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
        lib.pa_decode_workspace_bytes.restype = sz
        lib.pa_decode.argtypes = [p, p, p, p, p, i32, p, i32, i32, i32, i32, i32, i32,
                                  ctypes.c_float, p, sz, p]
        lib.pa_decode.restype = ctypes.c_int
        lib.pa_decode_store.argtypes = [p, p, p, p, i64, p, p, p, p, i32, p, i32, i32, i32,
                                        i32, i32, i32, i32, ctypes.c_float, p, sz, p]
        lib.pa_decode_store.restype = ctypes.c_int
        lib.pa_decode_store_noalloc.argtypes = [p, p, p, p, i64, p, p, p, p, i32, p, i32, i32,
                                                i32, i32, i32, i32, i32, ctypes.c_float, p]
        lib.pa_decode_store_noalloc.restype = ctypes.c_int
        lib.pa_prefill_varlen.argtypes = [p, p, p, p, p, p, p, i32, i32, i32, i32, i32, i32,
                                          i32, i32, ctypes.c_float, p]
        lib.pa_prefill_varlen.restype = ctypes.c_int
        lib.pa_validate_metadata.argtypes = [p, i32, p, i32, p, p, i32, i32, i32, i32,
                                             ctypes.c_char_p, sz]
        lib.pa_validate_metadata.restype = ctypes.c_int
        lib.pa_sample_workspace_bytes.argtypes = [i32, i32]
        lib.pa_sample_workspace_bytes.restype = sz
        lib.pa_sample_gumbel.argtypes = [p, p, i64, i32, i32, ctypes.c_uint64, ctypes.c_uint64,
                                         p, sz, p]
        lib.pa_sample_gumbel.restype = ctypes.c_int
        lib.pa_decode_graphs_create.argtypes = [ctypes.POINTER(_StepBuffers), p, i32,
                                                ctypes.POINTER(ctypes.c_void_p)]
        lib.pa_decode_graphs_create.restype = ctypes.c_int
        lib.pa_decode_graphs_bucket.argtypes = [p, i32, ctypes.POINTER(i32)]
        lib.pa_decode_graphs_bucket.restype = ctypes.c_int
        lib.pa_decode_graphs_launch.argtypes = [p, i32, p]
        lib.pa_decode_graphs_launch.restype = ctypes.c_int
        lib.pa_decode_graphs_destroy.argtypes = [p]
        lib.pa_decode_graphs_destroy.restype = None
        _lib = lib
    return _lib


def pa_status_string(status):
    return library().pa_status_string(int(status)).decode()


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(int(stream))
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t, name, dtype=None):
    """Device pointer of a tensor (None -> NULL), after checking where it lives."""
    if t is None:
        return None
    import torch
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _check(name, rc):
    if rc != 0:
        raise PAError(name, rc)


def _pool_shape(k_cache, v_cache):
    if k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache must both be [num_blocks, block_size, Hkv, D]")
    if not (k_cache.is_contiguous() and v_cache.is_contiguous()):
        raise ValueError("pools must be contiguous")
    return tuple(int(x) for x in k_cache.shape)


def pa_store_kvcache(k, v, k_cache, v_cache, slot_mapping, stream=None):
    """k, v: [T, Hkv, D] or [T, >= Hkv*D] bf16 with unit stride inside a row
    (row slices of a fused QKV buffer are fine); pools [NB, bs, Hkv, D];
    slot_mapping [T] int32 (-1 = skip)."""
    import torch
    num_blocks, bs, hkv, d = _pool_shape(k_cache, v_cache)
    T = int(k.shape[0])
    k2 = k.flatten(1) if k.dim() == 3 else k
    v2 = v.flatten(1) if v.dim() == 3 else v
    if k2.dim() != 2 or k2.stride(1) != 1 or v2.stride(1) != 1 or k2.stride(0) != v2.stride(0):
        raise ValueError("k and v rows must have unit element stride and equal row strides")
    if slot_mapping.numel() != T:
        raise ValueError("slot_mapping must have one entry per token")
    rc = library().pa_store_kvcache(
        _dev(k2, "k", torch.bfloat16), _dev(v2, "v", torch.bfloat16), int(k2.stride(0)),
        _dev(k_cache, "k_cache", torch.bfloat16), _dev(v_cache, "v_cache", torch.bfloat16),
        _dev(slot_mapping, "slot_mapping", torch.int32), T, num_blocks, bs, hkv, d,
        _stream(stream))
    _check("pa_store_kvcache", rc)


def pa_decode_workspace_bytes(batch, num_q_heads, head_dim, max_context_len, block_size):
    return int(library().pa_decode_workspace_bytes(batch, num_q_heads, head_dim,
                                                   max_context_len, block_size))


def pa_decode(out, q, k_cache, v_cache, block_table, context_lens, max_context_len, scale,
              workspace, stream=None):
    """out, q: [B, Hq, D] bf16; block_table [B, stride] int32; context_lens [B] int32;
    workspace: a uint8 GPU tensor of at least pa_decode_workspace_bytes(...) bytes."""
    import torch
    num_blocks, bs, hkv, d = _pool_shape(k_cache, v_cache)
    B, hq, dq = (int(x) for x in q.shape)
    if out.shape != q.shape or not (q.is_contiguous() and out.is_contiguous()):
        raise ValueError("out and q must be contiguous [B, Hq, D]")
    if not block_table.is_contiguous() or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be a contiguous [B, stride] int32 tensor")
    rc = library().pa_decode(
        _dev(out, "out", torch.bfloat16), _dev(q, "q", torch.bfloat16),
        _dev(k_cache, "k_cache", torch.bfloat16), _dev(v_cache, "v_cache", torch.bfloat16),
        _dev(block_table, "block_table", torch.int32), int(block_table.shape[1]),
        _dev(context_lens, "context_lens", torch.int32), B, hq, hkv, dq, bs,
        int(max_context_len), float(scale), _dev(workspace, "workspace"),
        workspace.numel() * workspace.element_size() if workspace is not None else 0,
        _stream(stream))
    _check("pa_decode", rc)


def pa_decode_store(out, q, k_new, v_new, k_cache, v_cache, slot_mapping, block_table,
                    context_lens, max_context_len, scale, workspace, stream=None):
    """The decode step in one call: pa_store_kvcache(k_new, v_new, ..., slot_mapping)
    fused into pa_decode. k_new, v_new: [B, Hkv, D] or [B, >= Hkv*D] bf16 rows;
    slot_mapping [B] int32 in the decode-step layout (a live row's new-token slot or
    -1; -1 for padding rows); the rest as for pa_decode."""
    import torch
    num_blocks, bs, hkv, d = _pool_shape(k_cache, v_cache)
    B, hq, dq = (int(x) for x in q.shape)
    if out.shape != q.shape or not (q.is_contiguous() and out.is_contiguous()):
        raise ValueError("out and q must be contiguous [B, Hq, D]")
    if not block_table.is_contiguous() or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be a contiguous [B, stride] int32 tensor")
    k2 = k_new.flatten(1) if k_new.dim() == 3 else k_new
    v2 = v_new.flatten(1) if v_new.dim() == 3 else v_new
    if k2.dim() != 2 or k2.stride(1) != 1 or v2.stride(1) != 1 or k2.stride(0) != v2.stride(0):
        raise ValueError("k_new and v_new rows must have unit element stride and equal row "
                         "strides")
    if int(k2.shape[0]) != B or slot_mapping.numel() != B:
        raise ValueError("k_new, v_new and slot_mapping must have one row per sequence")
    rc = library().pa_decode_store(
        _dev(out, "out", torch.bfloat16), _dev(q, "q", torch.bfloat16),
        _dev(k2, "k_new", torch.bfloat16), _dev(v2, "v_new", torch.bfloat16), int(k2.stride(0)),
        _dev(k_cache, "k_cache", torch.bfloat16), _dev(v_cache, "v_cache", torch.bfloat16),
        _dev(slot_mapping, "slot_mapping", torch.int32),
        _dev(block_table, "block_table", torch.int32), int(block_table.shape[1]),
        _dev(context_lens, "context_lens", torch.int32), B, num_blocks, hq, hkv, dq, bs,
        int(max_context_len), float(scale), _dev(workspace, "workspace"),
        workspace.numel() * workspace.element_size() if workspace is not None else 0,
        _stream(stream))
    _check("pa_decode_store", rc)


def pa_decode_store_noalloc(out, q, k_new, v_new, k_cache, v_cache, slot_mapping, block_table,
                            context_lens, max_context_len, scale, stream=None):
    """pa_decode_store with the library's fixed device scratch instead of a
    workspace: the call allocates no device memory. Calls that overlap on one
    GPU share that scratch and race; calls ordered on one stream do not."""
    import torch
    num_blocks, bs, hkv, d = _pool_shape(k_cache, v_cache)
    B, hq, dq = (int(x) for x in q.shape)
    if out.shape != q.shape or not (q.is_contiguous() and out.is_contiguous()):
        raise ValueError("out and q must be contiguous [B, Hq, D]")
    if not block_table.is_contiguous() or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be a contiguous [B, stride] int32 tensor")
    k2 = k_new.flatten(1) if k_new.dim() == 3 else k_new
    v2 = v_new.flatten(1) if v_new.dim() == 3 else v_new
    if k2.dim() != 2 or k2.stride(1) != 1 or v2.stride(1) != 1 or k2.stride(0) != v2.stride(0):
        raise ValueError("k_new and v_new rows must have unit element stride and equal row "
                         "strides")
    if int(k2.shape[0]) != B or slot_mapping.numel() != B:
        raise ValueError("k_new, v_new and slot_mapping must have one row per sequence")
    rc = library().pa_decode_store_noalloc(
        _dev(out, "out", torch.bfloat16), _dev(q, "q", torch.bfloat16),
        _dev(k2, "k_new", torch.bfloat16), _dev(v2, "v_new", torch.bfloat16), int(k2.stride(0)),
        _dev(k_cache, "k_cache", torch.bfloat16), _dev(v_cache, "v_cache", torch.bfloat16),
        _dev(slot_mapping, "slot_mapping", torch.int32),
        _dev(block_table, "block_table", torch.int32), int(block_table.shape[1]),
        _dev(context_lens, "context_lens", torch.int32), B, num_blocks, hq, hkv, dq, bs,
        int(max_context_len), float(scale), _stream(stream))
    _check("pa_decode_store_noalloc", rc)


def pa_prefill_varlen(out, q, k_cache, v_cache, cu_seqlens_q, context_lens, block_table,
                      max_seqlen_q, scale, stream=None):
    """out, q: [total_q, Hq, D] bf16; cu_seqlens_q [B+1], context_lens [B],
    block_table [B, stride] int32."""
    import torch
    num_blocks, bs, hkv, d = _pool_shape(k_cache, v_cache)
    T, hq, dq = (int(x) for x in q.shape)
    B = int(context_lens.shape[0])
    if out.shape != q.shape or not (q.is_contiguous() and out.is_contiguous()):
        raise ValueError("out and q must be contiguous [total_q, Hq, D]")
    if cu_seqlens_q.numel() != B + 1 or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("cu_seqlens_q must be [B+1] and block_table [B, stride]")
    if not block_table.is_contiguous():
        raise ValueError("block_table must be contiguous")
    rc = library().pa_prefill_varlen(
        _dev(out, "out", torch.bfloat16), _dev(q, "q", torch.bfloat16),
        _dev(k_cache, "k_cache", torch.bfloat16), _dev(v_cache, "v_cache", torch.bfloat16),
        _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32),
        _dev(context_lens, "context_lens", torch.int32),
        _dev(block_table, "block_table", torch.int32), int(block_table.shape[1]), B, T,
        int(max_seqlen_q), hq, hkv, dq, bs, float(scale), _stream(stream))
    _check("pa_prefill_varlen", rc)


def pa_validate_metadata(block_table, context_lens, num_blocks, block_size, cu_seqlens_q=None,
                         slot_mapping=None, max_context_len=-1):
    """Host-side metadata check (numpy or CPU tensors). Raises PAError with the
    library's message on the first violation."""
    import numpy as np

    def arr(a):
        if a is None:
            return None
        if hasattr(a, "detach"):
            a = a.detach().cpu().numpy()
        return np.ascontiguousarray(a, dtype=np.int32)

    bt, cl, cu, sm = arr(block_table), arr(context_lens), arr(cu_seqlens_q), arr(slot_mapping)
    ptr = lambda a: a.ctypes.data_as(ctypes.c_void_p) if a is not None else None
    msg = ctypes.create_string_buffer(256)
    rc = library().pa_validate_metadata(
        ptr(bt), int(bt.shape[1]) if bt is not None and bt.ndim == 2 else 0, ptr(cl),
        int(len(cl)), ptr(cu), ptr(sm), 0 if sm is None else int(len(sm)), int(num_blocks),
        int(block_size), int(max_context_len), msg, 256)
    if rc != 0:
        raise PAError("pa_validate_metadata", rc, msg.value.decode())


def pa_sample_workspace_bytes(batch, vocab):
    return int(library().pa_sample_workspace_bytes(int(batch), int(vocab)))


def pa_sample_gumbel(tokens, probs, seed, offset, workspace=None, stream=None):
    """tokens: [B] int32; probs: [B, V] fp32 with unit stride inside a row.
    Draws tokens[b] = argmax_i probs[b, i] / E[b, i], E ~ Exp(1) from Philox
    at (seed, offset). workspace: uint8 tensor of pa_sample_workspace_bytes
    bytes (allocated here if None)."""
    import torch
    if probs.dim() != 2 or probs.stride(1) != 1:
        raise ValueError("probs must be [B, V] with unit stride inside a row")
    B, V = int(probs.shape[0]), int(probs.shape[1])
    if tokens.numel() != B:
        raise ValueError("one token per row")
    if workspace is None:
        workspace = torch.empty(max(pa_sample_workspace_bytes(B, V), 8), dtype=torch.uint8,
                                device=probs.device)
    rc = library().pa_sample_gumbel(
        _dev(tokens, "tokens", torch.int32), _dev(probs, "probs", torch.float32),
        int(probs.stride(0)), B, V, int(seed) & (2**64 - 1), int(offset) & (2**64 - 1),
        _dev(workspace, "workspace"), int(workspace.numel() * workspace.element_size()),
        _stream(stream))
    _check("pa_sample_gumbel", rc)


DEFAULT_BUCKETS = (1, 2, 4, 8, 16, 32, 64, 128, 256, 512)


class DecodeGraphs:
    """Handle of pa_decode_graphs_create: keeps the step buffers alive while
    the graphs that read them exist. bucket() and launch() call
    pa_decode_graphs_bucket and pa_decode_graphs_launch; close() calls
    pa_decode_graphs_destroy."""

    def __init__(self, handle, buckets, tensors):
        self._h = handle
        self.buckets = tuple(buckets)
        self._tensors = tensors

    def bucket(self, batch):
        b = ctypes.c_int32()
        _check("pa_decode_graphs_bucket",
               library().pa_decode_graphs_bucket(self._h, int(batch), ctypes.byref(b)))
        return b.value

    def launch(self, batch, stream=None):
        _check("pa_decode_graphs_launch",
               library().pa_decode_graphs_launch(self._h, int(batch), _stream(stream)))

    def close(self):
        if getattr(self, "_h", None):
            library().pa_decode_graphs_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()


def pa_decode_graphs_create(out, q, k_new, v_new, k_cache, v_cache, slot_mapping, context_lens,
                            block_table, workspace, max_context_len, scale, buckets=None):
    """Captures the decode step at each bucket (default 1, 2, 4, ..., 512).

    Static device buffers sized for the largest bucket B: out, q [B, Hq, D];
    k_new, v_new [B, Hkv, D] (or [B, >= Hkv*D] rows with unit stride inside a
    row); pools [NB, bs, Hkv, D]; slot_mapping, context_lens [B] int32;
    block_table [B, stride] int32; workspace uint8 of at least
    pa_decode_workspace_bytes(B, Hq, D, max_context_len, bs) bytes. Before
    launch(batch) the caller fills rows [0, bucket(batch)) of the inputs,
    padding rows with context length 0 and slot -1."""
    import torch
    bk = list(DEFAULT_BUCKETS if buckets is None else buckets)
    B = bk[-1] if bk else 0
    num_blocks, bs, hkv, d = _pool_shape(k_cache, v_cache)
    hq = int(q.shape[1])
    k2 = k_new.flatten(1) if k_new.dim() == 3 else k_new
    v2 = v_new.flatten(1) if v_new.dim() == 3 else v_new
    if k2.stride(1) != 1 or v2.stride(1) != 1 or k2.stride(0) != v2.stride(0):
        raise ValueError("k_new and v_new rows must have unit element stride and equal strides")
    for name, t, rows in (("out", out, B), ("q", q, B), ("k_new", k2, B), ("v_new", v2, B),
                          ("slot_mapping", slot_mapping, B), ("context_lens", context_lens, B),
                          ("block_table", block_table, B)):
        if t.shape[0] < rows:
            raise ValueError(f"{name} has {t.shape[0]} rows, the largest bucket needs {rows}")
    if not (out.is_contiguous() and q.is_contiguous() and block_table.is_contiguous()):
        raise ValueError("out, q and block_table must be contiguous")
    sb = _StepBuffers(
        out=_dev(out, "out", torch.bfloat16).value, q=_dev(q, "q", torch.bfloat16).value,
        k_new=_dev(k2, "k_new", torch.bfloat16).value, v_new=_dev(v2, "v_new", torch.bfloat16).value,
        kv_token_stride=int(k2.stride(0)),
        k_cache=_dev(k_cache, "k_cache", torch.bfloat16).value,
        v_cache=_dev(v_cache, "v_cache", torch.bfloat16).value,
        slot_mapping=_dev(slot_mapping, "slot_mapping", torch.int32).value,
        context_lens=_dev(context_lens, "context_lens", torch.int32).value,
        block_table=_dev(block_table, "block_table", torch.int32).value,
        block_table_stride=int(block_table.shape[1]),
        workspace=_dev(workspace, "workspace").value,
        workspace_bytes=int(workspace.numel() * workspace.element_size()),
        num_blocks=num_blocks, block_size=bs, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
        max_context_len=int(max_context_len), scale=float(scale))
    arr = (ctypes.c_int32 * len(bk))(*bk) if bk else None
    handle = ctypes.c_void_p()
    rc = library().pa_decode_graphs_create(ctypes.byref(sb), arr, len(bk), ctypes.byref(handle))
    _check("pa_decode_graphs_create", rc)
    return DecodeGraphs(handle.value, bk, (out, q, k2, v2, k_cache, v_cache, slot_mapping,
                                           context_lens, block_table, workspace))

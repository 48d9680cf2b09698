"""ctypes binding of libpa.so's block manager (C ABI in
include/pa_block_manager.h): paged KV block allocation with chained-hash
prefix caching, producing the metadata arrays the attention calls take.

Argument marshalling only: every rule runs in the C++ code of libpa.so.
Arrays are numpy int32/int64 on the host; copy them to the GPU with torch.
"""
import ctypes

import numpy as np

from . import PAError, library

__all__ = ["BlockManager", "xxh64", "block_hash", "kv_cache_num_blocks",
           "kv_cache_num_blocks_on_device"]

_configured = False


def _lib():
    global _configured
    lib = library()
    if not _configured:
        p, i32, i64, u64, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                ctypes.c_uint64, ctypes.c_size_t)
        sigs = {
            "pa_xxh64": ([p, sz, u64], u64),
            "pa_block_hash": ([u64, i32, p, i32], u64),
            "pa_bm_create": ([i32, i32], p),
            "pa_bm_destroy": ([p], None),
            "pa_bm_num_free_blocks": ([p], i32),
            "pa_bm_can_allocate": ([p, p, i32, p], ctypes.c_int),
            "pa_bm_allocate": ([p, i64, p, i32, p], ctypes.c_int),
            "pa_bm_can_append": ([p, i64, p], ctypes.c_int),
            "pa_bm_append": ([p, i64, i32], ctypes.c_int),
            "pa_bm_append_batch": ([p, p, p, i32], ctypes.c_int),
            "pa_bm_deallocate": ([p, i64], ctypes.c_int),
            "pa_bm_seq_info": ([p, i64, p, p, p], ctypes.c_int),
            "pa_bm_block_table": ([p, i64, p, i32], ctypes.c_int),
            "pa_bm_block_info": ([p, i32, p, p, p], ctypes.c_int),
            "pa_bm_stats": ([p, p], ctypes.c_int),
            "pa_bm_batch_info": ([p, p, i32, p, p, p, p], ctypes.c_int),
            "pa_bm_prefill_metadata": ([p, p, i32, p, p, p, i32, p, i32, p, p], ctypes.c_int),
            "pa_bm_decode_metadata": ([p, p, i32, i32, p, p, p, i32, p], ctypes.c_int),
            "pa_kv_cache_num_blocks": ([u64, u64, u64, u64, ctypes.c_double, i32, i32, i32, i32,
                                        i32], i64),
        }
        for name, (args, res) in sigs.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        _configured = True
    return lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _i32(a):
    """C-contiguous int32 array (no copy when `a` already is one)."""
    if isinstance(a, np.ndarray) and a.dtype == np.int32 and a.flags.c_contiguous:
        return a
    return np.ascontiguousarray(np.asarray(a, dtype=np.int64).astype(np.int32))


def _ids(a):
    return np.ascontiguousarray(a, dtype=np.int64)


def _out(arr, shape, name):
    """A caller-provided int32 output array of exactly `shape`, or a new one."""
    if arr is None:
        return np.empty(shape, np.int32)
    if (not isinstance(arr, np.ndarray) or arr.dtype != np.int32 or arr.shape != tuple(shape)
            or not arr.flags.c_contiguous):
        raise ValueError(f"{name} must be a C-contiguous int32 array of shape {tuple(shape)}")
    return arr


def _check(name, rc):
    if rc != 0:
        raise PAError(name, rc)


def xxh64(data, seed=0):
    """XXH64 of a bytes object (pa_xxh64)."""
    buf = ctypes.create_string_buffer(bytes(data), len(data))
    return int(_lib().pa_xxh64(ctypes.cast(buf, ctypes.c_void_p), len(data), seed))


def block_hash(tokens, parent=None):
    """Chained hash of one full block of token ids (pa_block_hash)."""
    t = _i32(tokens)
    return int(_lib().pa_block_hash(0 if parent is None else int(parent),
                                    0 if parent is None else 1, _ptr(t), len(t)))


def kv_cache_num_blocks(total_bytes, used_bytes, peak_bytes, current_bytes, num_layers,
                        block_size, num_kv_heads, head_dim, dtype_bytes=2, utilization=0.9):
    """Blocks that fit in (total * utilization - used - peak + current) bytes
    (pa_kv_cache_num_blocks)."""
    n = _lib().pa_kv_cache_num_blocks(int(total_bytes), int(used_bytes), int(peak_bytes),
                                      int(current_bytes), float(utilization), int(num_layers),
                                      int(block_size), int(num_kv_heads), int(head_dim),
                                      int(dtype_bytes))
    if n < 0:
        raise ValueError("pa_kv_cache_num_blocks: bad arguments")
    return int(n)


def kv_cache_num_blocks_on_device(num_layers, block_size, num_kv_heads, head_dim,
                                  dtype_bytes=2, utilization=0.9, device=None):
    """The same budget from the current device after a warm-up: total and free
    memory from the runtime, peak and current from torch's allocator."""
    import torch
    free, total = torch.cuda.mem_get_info(device)
    peak = torch.cuda.max_memory_allocated(device)
    current = torch.cuda.memory_allocated(device)
    return kv_cache_num_blocks(total, total - free, peak, current, num_layers, block_size,
                               num_kv_heads, head_dim, dtype_bytes, utilization)


class BlockManager:
    """One pool of num_blocks blocks of block_size tokens (pa_bm_create)."""

    STAT_NAMES = ("shared", "taken_back", "fresh_alloc", "fresh_append", "evicted")

    def __init__(self, num_blocks, block_size):
        self._lib = _lib()
        self._h = self._lib.pa_bm_create(int(num_blocks), int(block_size))
        if not self._h:
            raise ValueError("pa_bm_create failed (bad sizes or out of memory)")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)

    def close(self):
        if getattr(self, "_h", None):
            self._lib.pa_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    @property
    def num_free_blocks(self):
        return int(self._lib.pa_bm_num_free_blocks(self._h))

    def can_allocate(self, tokens):
        t = _i32(tokens)
        ok = ctypes.c_int32()
        _check("pa_bm_can_allocate",
               self._lib.pa_bm_can_allocate(self._h, _ptr(t), len(t), ctypes.byref(ok)))
        return bool(ok.value)

    def allocate(self, seq_id, tokens):
        """Returns the number of cached leading tokens."""
        t = _i32(tokens)
        cached = ctypes.c_int32()
        _check("pa_bm_allocate", self._lib.pa_bm_allocate(self._h, int(seq_id), _ptr(t), len(t),
                                                          ctypes.byref(cached)))
        return cached.value

    def can_append(self, seq_id):
        ok = ctypes.c_int32()
        _check("pa_bm_can_append", self._lib.pa_bm_can_append(self._h, int(seq_id),
                                                              ctypes.byref(ok)))
        return bool(ok.value)

    def append(self, seq_id, token):
        _check("pa_bm_append", self._lib.pa_bm_append(self._h, int(seq_id), int(token)))

    def append_batch(self, seq_ids, tokens):
        """One token per sequence, all or nothing (pa_bm_append_batch)."""
        ids = _ids(seq_ids)
        t = _i32(tokens)
        if len(ids) != len(t):
            raise ValueError("one token per sequence id")
        _check("pa_bm_append_batch",
               self._lib.pa_bm_append_batch(self._h, _ptr(ids), _ptr(t), len(ids)))

    def deallocate(self, seq_id):
        _check("pa_bm_deallocate", self._lib.pa_bm_deallocate(self._h, int(seq_id)))

    def seq_info(self, seq_id):
        """(num_tokens, num_cached_tokens, num_blocks)."""
        n, c, b = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        _check("pa_bm_seq_info", self._lib.pa_bm_seq_info(self._h, int(seq_id), ctypes.byref(n),
                                                          ctypes.byref(c), ctypes.byref(b)))
        return n.value, c.value, b.value

    def block_table(self, seq_id):
        nblk = self.seq_info(seq_id)[2]
        out = np.zeros(max(nblk, 1), np.int32)
        _check("pa_bm_block_table",
               self._lib.pa_bm_block_table(self._h, int(seq_id), _ptr(out), len(out)))
        return out[:nblk]

    def block_info(self, block):
        """(ref_count, cached, hash)."""
        r, c, h = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_uint64()
        _check("pa_bm_block_info", self._lib.pa_bm_block_info(self._h, int(block), ctypes.byref(r),
                                                              ctypes.byref(c), ctypes.byref(h)))
        return r.value, c.value, h.value

    def stats(self):
        out = np.zeros(5, np.int64)
        _check("pa_bm_stats", self._lib.pa_bm_stats(self._h, _ptr(out)))
        return dict(zip(self.STAT_NAMES, (int(x) for x in out)))

    def batch_info(self, seq_ids):
        """(new_tokens, max_new_tokens, max_len, max_blocks) of live sequences."""
        ids = _ids(seq_ids)
        nt, mq, ml, mb = ctypes.c_int64(), ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        _check("pa_bm_batch_info", self._lib.pa_bm_batch_info(
            self._h, _ptr(ids), len(ids), ctypes.byref(nt), ctypes.byref(mq), ctypes.byref(ml),
            ctypes.byref(mb)))
        return nt.value, mq.value, ml.value, mb.value

    def prefill_metadata(self, seq_ids, block_table_stride, slot_capacity=None):
        """(cu_seqlens_q, context_lens, slot_mapping, block_table, total_q,
        max_seqlen_q) as numpy int32 arrays and ints. slot_capacity defaults to
        the exact total."""
        ids = _ids(seq_ids)
        B = len(ids)
        if slot_capacity is None:
            slot_capacity = self.batch_info(ids)[0]
        cu = np.zeros(B + 1, np.int32)
        ctx = np.zeros(max(B, 1), np.int32)
        slots = np.zeros(max(int(slot_capacity), 1), np.int32)
        bt = np.zeros((max(B, 1), max(int(block_table_stride), 1)), np.int32)
        tq, mq = ctypes.c_int32(), ctypes.c_int32()
        _check("pa_bm_prefill_metadata", self._lib.pa_bm_prefill_metadata(
            self._h, _ptr(ids), B, _ptr(cu), _ptr(ctx), _ptr(slots), int(slot_capacity),
            _ptr(bt), int(block_table_stride), ctypes.byref(tq), ctypes.byref(mq)))
        return (cu, ctx[:B], slots[:int(slot_capacity)], bt[:B, :int(block_table_stride)],
                tq.value, mq.value)

    def decode_metadata(self, seq_ids, padded_batch, block_table_stride, out=None):
        """(context_lens, slot_mapping, block_table, max_context_len).

        `out` may hold three int32 arrays ([P], [P], [P, stride]) to fill in
        place, so a decode loop allocates nothing per step."""
        ids = _ids(seq_ids)
        B, P, S = len(ids), int(padded_batch), int(block_table_stride)
        o = out or (None, None, None)
        ctx = _out(o[0], (P,), "context_lens")
        slots = _out(o[1], (P,), "slot_mapping")
        bt = _out(o[2], (P, S), "block_table")
        mx = ctypes.c_int32()
        _check("pa_bm_decode_metadata", self._lib.pa_bm_decode_metadata(
            self._h, _ptr(ids), B, P, _ptr(ctx), _ptr(slots), _ptr(bt), S, ctypes.byref(mx)))
        return ctx, slots, bt, mx.value

"""The block manager driving the HIP path: its block tables, slot mappings and
lengths go straight into pa_store_kvcache, pa_prefill_varlen and pa_decode,
through prefix hits inside one batch, decode steps that fill and register
blocks, padded decode batches, and freed cached blocks taken back.

The reference never looks at the manager's layout: token t's Q/K/V are drawn
from a generator seeded by the hash of the token prefix ending at t (K/V of a
position depends on everything before it, as in a real model), and each row is
checked against the oracle's attention over the sequence's own contiguous K/V.
A prefix block read from the cache therefore matches only if it holds exactly
what the sequence would have computed itself."""
import math

import numpy as np
import pytest
import torch
import xxhash

import oracle
import paged_kv_cache_slot_amd as pa
from paged_kv_cache_slot_amd.block_manager import BlockManager
from tests.gpu_common import DEV, compare, require_gpu, say

pytestmark = pytest.mark.gpu

BS, HQ, HKV, D, NB = 16, 8, 2, 128, 96
SCALE = 1.0 / math.sqrt(D)
STRIDE = 12          # block-table row width (up to 192 tokens)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


_memo = {}


def qkv_of(prefix):
    """bf16 (q [HQ, D], k [HKV, D], v [HKV, D]) of the last token of `prefix`."""
    key = tuple(prefix)
    if key not in _memo:
        seed = xxhash.xxh64_intdigest(np.asarray(key, dtype="<i4").tobytes(), 99)
        x = np.random.default_rng(seed).standard_normal((HQ + 2 * HKV, D)).astype(np.float32)
        t = torch.from_numpy(x).to(torch.bfloat16)
        _memo[key] = (t[:HQ], t[HQ:HQ + HKV], t[HQ + HKV:])
    return _memo[key]


def rows_of(tokens, positions, which):
    idx = {"q": 0, "k": 1, "v": 2}[which]
    return torch.stack([qkv_of(tokens[:p + 1])[idx] for p in positions])


def reference(tokens, positions):
    """fp64 attention outputs [len(positions), HQ, D] of the given positions,
    each over its own causal prefix, with the sequence laid out contiguously."""
    n = len(tokens)
    nblk = -(-n // BS)
    kpool = torch.zeros(nblk * BS, HKV, D, dtype=torch.bfloat16)
    vpool = torch.zeros(nblk * BS, HKV, D, dtype=torch.bfloat16)
    kpool[:n] = rows_of(tokens, range(n), "k")
    vpool[:n] = rows_of(tokens, range(n), "v")
    kpool = kpool.view(nblk, BS, HKV, D)
    vpool = vpool.view(nblk, BS, HKV, D)
    q = rows_of(tokens, range(n), "q")
    out = oracle.prefill(q, kpool, vpool, np.array([0, n]), np.array([n]),
                         np.arange(nblk, dtype=np.int32)[None, :], SCALE)
    return out[list(positions)]


class Engine:
    """A minimal caller: the manager plus the GPU pools."""

    def __init__(self, seed):
        self.bm = BlockManager(NB, BS)
        gen = torch.Generator(device=DEV).manual_seed(seed)
        # Stale, finite data in every slot, as a reused pool would hold.
        self.kc = (4 * torch.randn(NB, BS, HKV, D, generator=gen, device=DEV)).to(torch.bfloat16)
        self.vc = (4 * torch.randn(NB, BS, HKV, D, generator=gen, device=DEV)).to(torch.bfloat16)
        self.tokens = {}

    def prefill(self, batch):
        """batch: {seq_id: prompt}; allocates, stores, runs prefill and checks
        every computed row. Returns the cached token counts."""
        cached = {}
        for sid, toks in batch.items():
            cached[sid] = self.bm.allocate(sid, toks)
            self.tokens[sid] = list(toks)
        ids = list(batch)
        cu, ctx, slots, bt, total_q, max_q = self.bm.prefill_metadata(ids, STRIDE)
        pa.pa_validate_metadata(bt, ctx, NB, BS, cu_seqlens_q=cu, slot_mapping=slots)
        pos = [(sid, p) for sid in ids for p in range(cached[sid], len(batch[sid]))]
        q = torch.stack([qkv_of(self.tokens[s][:p + 1])[0] for s, p in pos])
        k = torch.stack([qkv_of(self.tokens[s][:p + 1])[1] for s, p in pos])
        v = torch.stack([qkv_of(self.tokens[s][:p + 1])[2] for s, p in pos])
        say(f"[case] manager prefill ids {ids} cached {cached} total_q {total_q}")
        pa.pa_store_kvcache(k.to(DEV), v.to(DEV), self.kc, self.vc,
                            torch.from_numpy(slots).to(DEV))
        out = torch.empty(total_q, HQ, D, dtype=torch.bfloat16, device=DEV)
        pa.pa_prefill_varlen(out, q.to(DEV), self.kc, self.vc, torch.from_numpy(cu).to(DEV),
                             torch.from_numpy(ctx).to(DEV), torch.from_numpy(bt).to(DEV),
                             max_q, SCALE)
        torch.cuda.synchronize()
        for b, sid in enumerate(ids):
            want = reference(self.tokens[sid], range(cached[sid], len(batch[sid])))
            compare(out[cu[b]:cu[b + 1]], want, f"prefill seq {sid} (cached {cached[sid]})")
        return cached

    def decode_step(self, ids, padded, rng):
        for sid in ids:
            assert self.bm.can_append(sid)
            t = int(rng.integers(0, 1000))
            self.bm.append(sid, t)
            self.tokens[sid].append(t)
        ctx, slots, bt, max_len = self.bm.decode_metadata(ids, padded, STRIDE)
        pa.pa_validate_metadata(bt, ctx, NB, BS, slot_mapping=slots, max_context_len=max_len)
        last = [qkv_of(self.tokens[s]) for s in ids]
        zero_q = torch.zeros(HQ, D, dtype=torch.bfloat16)
        zero_kv = torch.zeros(HKV, D, dtype=torch.bfloat16)
        pad = padded - len(ids)
        q = torch.stack([x[0] for x in last] + [zero_q] * pad).to(DEV)
        k = torch.stack([x[1] for x in last] + [zero_kv] * pad).to(DEV)
        v = torch.stack([x[2] for x in last] + [zero_kv] * pad).to(DEV)
        pa.pa_store_kvcache(k, v, self.kc, self.vc, torch.from_numpy(slots).to(DEV))
        out = torch.full((padded, HQ, D), float("nan"), dtype=torch.bfloat16, device=DEV)
        nbytes = pa.pa_decode_workspace_bytes(padded, HQ, D, max_len, BS)
        ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=DEV)
        pa.pa_decode(out, q, self.kc, self.vc, torch.from_numpy(bt).to(DEV),
                     torch.from_numpy(ctx).to(DEV), max_len, SCALE, ws)
        torch.cuda.synchronize()
        for b, sid in enumerate(ids):
            n = len(self.tokens[sid])
            compare(out[b:b + 1], reference(self.tokens[sid], [n - 1]),
                    f"decode seq {sid} len {n}")
        if pad:
            assert int(out[len(ids):].float().abs().sum()) == 0, "padding rows must be zero"


def test_manager_driven_prefill_decode_and_reuse():
    rng = np.random.default_rng(2024)
    tok = lambda n: [int(x) for x in rng.integers(0, 1000, size=n)]
    stem1, stem2 = tok(3 * BS + 5), tok(2 * BS)
    eng = Engine(seed=31)
    A, B, C, E, F = 1, 2, 3, 4, 5
    prompts = {A: stem1 + tok(20), B: stem1[:3 * BS] + tok(9), C: stem2 + tok(40),
               E: stem1[:2 * BS]}
    cached = eng.prefill(prompts)
    # B hits A's three full prefix blocks inside the same batch; E (exactly two
    # blocks) shares one and recomputes the block that holds its last token.
    assert cached == {A: 0, B: 3 * BS, C: 0, E: BS}
    st = eng.bm.stats()
    assert st["shared"] == 4 and st["taken_back"] == 0

    # Decode 20 steps over the four sequences, padded to a batch of 8; A passes
    # the 80-token boundary, which registers its fifth block.
    for step in range(20):
        say(f"[case] manager decode step {step}")
        eng.decode_step([A, B, C, E], 8, rng)

    # A finishes: its own blocks go back to the free queue, still cached.
    free_before = eng.bm.num_free_blocks
    eng.bm.deallocate(A)
    assert eng.bm.num_free_blocks > free_before
    # F repeats A's first 88 tokens (prompt and generated): three blocks shared
    # with B, two taken back from the free queue (one registered by decode).
    cached = eng.prefill({F: eng.tokens[A][:88] + tok(10)})
    assert cached == {F: 5 * BS}
    st = eng.bm.stats()
    assert st["taken_back"] == 2, st
    for step in range(3):
        say(f"[case] manager decode after reuse, step {step}")
        eng.decode_step([B, C, E, F], 4, rng)


def test_kv_budget_on_device():
    """After a warm-up, the budget from the device's own figures matches the
    oracle on the same figures, and a KV cache of that many blocks (all 28
    layers of a Qwen3-0.6B shape, at 5% of the device) can be allocated."""
    import oracle.kv_budget as okb
    from paged_kv_cache_slot_amd.block_manager import (kv_cache_num_blocks,
                                                       kv_cache_num_blocks_on_device)
    eng = Engine(seed=5)
    eng.prefill({1: list(range(40))})                   # warm-up step
    torch.cuda.synchronize()
    free, total = torch.cuda.mem_get_info()
    peak, cur = torch.cuda.max_memory_allocated(), torch.cuda.memory_allocated()
    shape = dict(num_layers=28, block_size=256, num_kv_heads=8, head_dim=128)
    n = kv_cache_num_blocks(total, total - free, peak, cur, utilization=0.05, **shape)
    assert n == okb.num_blocks(total, total - free, peak, cur, 28, 256, 8, 128, 2, 0.05)
    assert n > 0
    n_dev = kv_cache_num_blocks_on_device(utilization=0.05, **shape)
    assert abs(n_dev - n) <= 1 + n // 100             # the device figures move a little
    block_bytes = 2 * 28 * 256 * 8 * 128 * 2
    say(f"[case] kv budget: {n} blocks of {block_bytes} bytes at 5% of {total} bytes")
    kv = torch.empty(n * block_bytes, dtype=torch.uint8, device=DEV)
    kv[-1] = 1
    torch.cuda.synchronize()
    assert kv.numel() <= 0.05 * total
    del kv

"""Seeded synthetic inputs shaped like the pages' workloads.

This module only draws inputs: lengths, physical block assignments, pool and
activation values, and the metadata a scheduler would hand to the attention
path (block tables, context lengths, slot mappings, cu_seqlens). It computes
no attention, no softmax and no KV store. Both the CPU oracle and the GPU
library consume what it returns; neither is imported here.

Recipe (the same for every caller):
  * metadata from numpy's PCG64 `default_rng(seed)`, drawn in a fixed order:
    lengths, padding rows, prefix choices, block permutation;
  * values from a torch generator seeded with `seed`, on the requested
    device, drawn in a fixed order: K pool, V pool, q, new K, new V. Every
    value is N(0,1) drawn in fp32 and rounded to bf16 (round to nearest even);
  * lengths are integers uniform over the inclusive range;
  * the whole pool is filled with noise first, so slots no sequence owns, the
    tail of each sequence's last block, and the slot a new token is about to
    be written to all hold data that would change a result if read;
  * physical blocks are a random permutation of [0, num_blocks), handed out
    in logical order.
Values drawn on the CPU and on the GPU differ (different generators); every
check feeds the same bytes to both sides.
"""
import hashlib
import math

import numpy as np
import torch

# The five workloads, by name. Shapes follow the pages' benchmarks: Qwen3-0.6B
# with 256 sequences and lengths of 100..1024 tokens, Qwen3-8B with random
# lengths, and the two block sizes the pages contrast (256 in nano-vLLM, 16 in
# vLLM). Each has a fixed seed.
WORKLOADS = {
    "tiny_decode": dict(seed=1001, kind="decode", batch=4, len_range=(100, 300),
            num_q_heads=16, num_kv_heads=8, head_dim=128, block_size=256,
            num_blocks=16, pad=0, pad_at="tail"),
    "qwen3_0.6b_decode": dict(seed=1002, kind="decode", batch=256, len_range=(100, 2048),
            num_q_heads=16, num_kv_heads=8, head_dim=128, block_size=256,
            num_blocks=None, pad=0, pad_at="tail"),
    "qwen3_8b_decode": dict(seed=1003, kind="decode", batch=512, len_range=(200, 2048),
            num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=256,
            num_blocks=None, pad=41, pad_at="tail"),
    "qwen3_8b_prefill_prefix": dict(seed=1004, kind="prefill", batch=64, new_range=(100, 1024),
            num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=256,
            chains=8, chain_blocks=3),
    "bs16_stress_decode": dict(seed=1005, kind="decode", batch=1024, len_range=(100, 2048),
            num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
            num_blocks=None, pad=102, pad_at="random"),
}


def seed_of(name):
    return WORKLOADS[name]["seed"]


def softmax_scale(head_dim):
    """1/sqrt(head_dim) rounded to fp32, as a Python float (both sides use it)."""
    return float(np.float32(1.0 / math.sqrt(head_dim)))


def _randn_bf16(shape, gen, device, chunk=1 << 26):
    """N(0,1) drawn in fp32, rounded to bf16; drawn in chunks to bound memory."""
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(-1)
    for s in range(0, flat.numel(), chunk):
        n = min(chunk, flat.numel() - s)
        flat[s:s + n] = torch.randn(n, generator=gen, device=device,
                                    dtype=torch.float32).to(torch.bfloat16)
    return out


def _generator(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def decode_case(batch, len_range, num_q_heads, num_kv_heads, head_dim, block_size,
                seed, device="cpu", num_blocks=None, pad=0, pad_at="tail",
                spare_blocks=0, lens=None):
    """One decode batch: one new token per sequence, already counted in its length.

    Returns a dict of tensors on `device`:
      q [B, Hq, D], k_new/v_new [B, Hkv, D] bf16; k_cache/v_cache
      [num_blocks, bs, Hkv, D] bf16; block_table [B, max_blocks] int32 (-1 past
      each row's blocks); context_lens [B] int32 (0 on padding rows);
      slot_mapping [B] int32 (-1 on padding rows; else the slot of position L-1),
    plus scalars (scale, max_context_len, ...).
    """
    rng = np.random.default_rng(seed)
    lo, hi = len_range
    if lens is None:
        lens = rng.integers(lo, hi + 1, size=batch).astype(np.int64)
    else:
        lens = np.asarray(lens, dtype=np.int64).copy()
        assert len(lens) == batch
    if pad:
        if pad_at == "tail":
            pad_rows = np.arange(batch - pad, batch)
        else:
            pad_rows = np.sort(rng.choice(batch, size=pad, replace=False))
        lens[pad_rows] = 0
    nblk = (lens + block_size - 1) // block_size
    needed = int(nblk.sum())
    if num_blocks is None:
        num_blocks = needed + spare_blocks
    assert num_blocks >= needed, "pool too small for the batch"
    perm = rng.permutation(num_blocks)
    max_blocks = max(1, -(-max(hi, int(lens.max()) if batch else 0) // block_size))
    table = np.full((batch, max_blocks), -1, dtype=np.int32)
    slots = np.full(batch, -1, dtype=np.int32)
    off = 0
    for b in range(batch):
        n = int(nblk[b])
        table[b, :n] = perm[off:off + n]
        off += n
        if lens[b] > 0:
            pos = int(lens[b]) - 1
            slots[b] = table[b, pos // block_size] * block_size + pos % block_size
    gen = _generator(seed, device)
    pool_shape = (num_blocks, block_size, num_kv_heads, head_dim)
    case = dict(
        kind="decode",
        k_cache=_randn_bf16(pool_shape, gen, device),
        v_cache=_randn_bf16(pool_shape, gen, device),
        q=_randn_bf16((batch, num_q_heads, head_dim), gen, device),
        k_new=_randn_bf16((batch, num_kv_heads, head_dim), gen, device),
        v_new=_randn_bf16((batch, num_kv_heads, head_dim), gen, device),
        block_table=torch.from_numpy(table).to(device),
        context_lens=torch.from_numpy(lens.astype(np.int32)).to(device),
        slot_mapping=torch.from_numpy(slots).to(device),
        batch=batch, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
        head_dim=head_dim, block_size=block_size, num_blocks=num_blocks,
        max_context_len=int(lens.max()) if batch else 0,
        scale=softmax_scale(head_dim), seed=seed,
        lens=lens, num_real=int((lens > 0).sum()),
    )
    return case


def prefill_case(batch, new_range, num_q_heads, num_kv_heads, head_dim, block_size,
                 seed, device="cpu", chains=8, chain_blocks=3, max_prefix_blocks=None,
                 new_lens=None, prefix_blocks=None, prefix_chain=None):
    """One varlen prefill batch whose sequences may reuse cached prefix blocks.

    Sequence b takes k_b ~ U{0..max_prefix_blocks} full blocks from shared chain
    c_b ~ U{0..chains-1} (so P_b = k_b * block_size cached tokens, shared with
    every other sequence on the same chain), then N_b ~ U[new_range] new tokens
    in freshly assigned blocks. Returns tensors on `device`:
      q [T, Hq, D], k_new/v_new [T, Hkv, D] bf16 (T = sum N_b); pools;
      block_table [B, max_blocks]; cu_seqlens_q [B+1]; context_lens [B] = P+N;
      slot_mapping [T] (the slot of position P_b + i for new row i).
    """
    rng = np.random.default_rng(seed)
    lo, hi = new_range
    if max_prefix_blocks is None:
        max_prefix_blocks = chain_blocks
    N = (rng.integers(lo, hi + 1, size=batch) if new_lens is None
         else np.asarray(new_lens)).astype(np.int64)
    k = (rng.integers(0, max_prefix_blocks + 1, size=batch) if prefix_blocks is None
         else np.asarray(prefix_blocks)).astype(np.int64)
    c = (rng.integers(0, chains, size=batch) if prefix_chain is None
         else np.asarray(prefix_chain)).astype(np.int64)
    assert (k <= chain_blocks).all()
    P = k * block_size
    L = P + N
    total_blocks = -(-L // block_size)
    fresh = total_blocks - k
    num_shared = chains * chain_blocks
    num_blocks = num_shared + int(fresh.sum())
    perm = rng.permutation(num_blocks)
    chain_ids = perm[:num_shared].reshape(chains, chain_blocks)
    max_blocks = max(1, int(total_blocks.max()) if batch else 1)
    table = np.full((batch, max_blocks), -1, dtype=np.int32)
    off = num_shared
    for b in range(batch):
        kb = int(k[b])
        table[b, :kb] = chain_ids[c[b], :kb]
        n = int(fresh[b])
        table[b, kb:kb + n] = perm[off:off + n]
        off += n
    cu = np.zeros(batch + 1, dtype=np.int32)
    cu[1:] = np.cumsum(N)
    T = int(cu[-1])
    slots = np.empty(T, dtype=np.int32)
    for b in range(batch):
        for i in range(int(N[b])):
            pos = int(P[b]) + i
            slots[cu[b] + i] = table[b, pos // block_size] * block_size + pos % block_size
    gen = _generator(seed, device)
    pool_shape = (num_blocks, block_size, num_kv_heads, head_dim)
    return dict(
        kind="prefill",
        k_cache=_randn_bf16(pool_shape, gen, device),
        v_cache=_randn_bf16(pool_shape, gen, device),
        q=_randn_bf16((T, num_q_heads, head_dim), gen, device),
        k_new=_randn_bf16((T, num_kv_heads, head_dim), gen, device),
        v_new=_randn_bf16((T, num_kv_heads, head_dim), gen, device),
        block_table=torch.from_numpy(table).to(device),
        cu_seqlens_q=torch.from_numpy(cu).to(device),
        context_lens=torch.from_numpy(L.astype(np.int32)).to(device),
        slot_mapping=torch.from_numpy(slots).to(device),
        batch=batch, total_q=T, max_seqlen_q=int(N.max()) if batch else 0,
        num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
        block_size=block_size, num_blocks=num_blocks,
        scale=softmax_scale(head_dim), seed=seed,
        new_lens=N, prefix_lens=P, prefix_blocks=k, prefix_chain=c,
    )


def workload_case(name, device="cpu", seed=None, **overrides):
    """The inputs of the named workload, optionally with fields overridden."""
    cfg = dict(WORKLOADS[name])
    cfg.update(overrides)
    seed = cfg["seed"] if seed is None else seed
    if cfg["kind"] == "decode":
        return decode_case(cfg["batch"], cfg["len_range"], cfg["num_q_heads"],
                           cfg["num_kv_heads"], cfg["head_dim"], cfg["block_size"],
                           seed, device=device, num_blocks=cfg.get("num_blocks"),
                           pad=cfg.get("pad", 0), pad_at=cfg.get("pad_at", "tail"))
    return prefill_case(cfg["batch"], cfg["new_range"], cfg["num_q_heads"],
                        cfg["num_kv_heads"], cfg["head_dim"], cfg["block_size"], seed,
                        device=device, chains=cfg["chains"], chain_blocks=cfg["chain_blocks"])


def digest(t):
    """64-bit hash of a tensor's bytes, so two runs can show they shared inputs."""
    a = t.detach().contiguous().cpu()
    if a.dtype == torch.bfloat16:
        a = a.view(torch.int16)
    return hashlib.blake2b(a.numpy().tobytes(), digest_size=8).hexdigest()

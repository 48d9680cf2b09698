"""Seeded random shapes against the oracle: head groupings G = 1..8, kv head
counts 1..8, block sizes 16..256, batch sizes (up to 200 rows), lengths (up to
8000 tokens) with empty rows mixed in, cached prefixes of up to 6 blocks, and
softmax scales between 0.02 and 1, drawn once from fixed seeds (the test ids
name each draw). Decode: the fused step (pa_decode_store) on every
row against the oracle, both pools bit for bit against the oracle's store,
and the separate store + decode bit for bit against the fused step. Prefill:
store + prefill over cached prefixes, every row against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_slot_amd as pa
import workloads
from tests.gpu_common import (DEV, ORACLE_THREADS, compare, gpu_decode, gpu_prefill, gpu_store,
                              host_copy, oracle_after_store, require_gpu, say, to_device)

pytestmark = pytest.mark.gpu

BLOCK_SIZES = [16, 32, 64, 128, 256]


def _heads(rng):
    while True:
        g = int(rng.choice([1, 2, 4, 8]))
        hkv = int(rng.choice([1, 2, 4, 8]))
        if g * hkv <= 64:
            return g * hkv, hkv


def _decode_draws(n, seed, data_seed, max_batch=48, max_len=3000, tag="d"):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        hq, hkv = _heads(rng)
        bs = int(rng.choice(BLOCK_SIZES))
        batch = int(rng.integers(1, max_batch + 1))
        lens = rng.integers(1, max_len + 1, size=batch)
        lens[rng.random(batch) < 0.1] = 0
        scale = float(np.float32(np.exp(rng.uniform(np.log(0.02), 0.0))))
        extra = int(rng.choice([0, 0, 7, 300]))  # max_context_len above the longest row
        out.append((f"{tag}{i}-hq{hq}-hkv{hkv}-bs{bs}-b{batch}", hq, hkv, bs,
                    [int(x) for x in lens], scale, extra, data_seed + i))
    return out


def _prefill_draws(n, seed, data_seed, max_new=300, max_pre=3, tag="p"):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        hq, hkv = _heads(rng)
        bs = int(rng.choice(BLOCK_SIZES))
        batch = int(rng.integers(1, 7))
        new = rng.integers(1, max_new + 1, size=batch)
        new[rng.random(batch) < 0.15] = 0
        if new.sum() == 0:  # at least one row to check
            new[0] = int(rng.integers(1, max_new + 1))
        pre = rng.integers(0, max_pre + 1, size=batch)
        scale = float(np.float32(np.exp(rng.uniform(np.log(0.02), 0.0))))
        out.append((f"{tag}{i}-hq{hq}-hkv{hkv}-bs{bs}-b{batch}", hq, hkv, bs,
                    [int(x) for x in new], [int(x) for x in pre], scale, data_seed + i))
    return out


# Two sets each: short contexts and small batches, then longer contexts (up to
# 8000 tokens), larger batches (up to 200 rows) and longer prefixes.
DECODE_DRAWS = (_decode_draws(8, 71, 2000)
                + _decode_draws(8, 73, 4000, max_batch=200, max_len=8000, tag="D"))
PREFILL_DRAWS = (_prefill_draws(6, 72, 3000)
                 + _prefill_draws(6, 74, 5000, max_new=600, max_pre=6, tag="P"))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _pool_bits(t):
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("cid,hq,hkv,bs,lens,scale,extra,seed", DECODE_DRAWS,
                         ids=[d[0] for d in DECODE_DRAWS])
def test_decode_step_random(cid, hq, hkv, bs, lens, scale, extra, seed):
    say(f"[case] random decode {cid}: lens={lens} scale={scale} extra={extra} seed={seed}")
    h = workloads.decode_case(len(lens), (1, 3000), hq, hkv, 128, bs, seed=seed, device="cpu",
                              lens=lens, spare_blocks=2)
    h["scale"] = scale
    h["max_context_len"] = int(h["max_context_len"]) + extra
    # The block table must cover max_context_len (-1 past each row's blocks).
    width = -(-h["max_context_len"] // bs)
    bt = h["block_table"]
    if bt.shape[1] < width:
        pad = torch.full((bt.shape[0], width - bt.shape[1]), -1, dtype=bt.dtype)
        h["block_table"] = torch.cat([bt, pad], 1).contiguous()
    case = to_device(host_copy(h))
    B = len(lens)
    ws = torch.empty(max(16, pa.pa_decode_workspace_bytes(B, hq, 128, case["max_context_len"],
                                                          bs)), dtype=torch.uint8, device=DEV)
    fused = torch.full_like(case["q"], float("nan"))
    pa.pa_decode_store(fused, case["q"], case["k_new"], case["v_new"], case["k_cache"],
                       case["v_cache"], case["slot_mapping"], case["block_table"],
                       case["context_lens"], case["max_context_len"], scale, ws)
    torch.cuda.synchronize()
    kc, vc = oracle_after_store(h)
    assert np.array_equal(_pool_bits(case["k_cache"]), kc), "K pool differs from the oracle"
    assert np.array_equal(_pool_bits(case["v_cache"]), vc), "V pool differs from the oracle"
    ref = oracle.decode(h["q"], kc, vc, h["block_table"], h["context_lens"], scale,
                        nthreads=ORACLE_THREADS)
    compare(fused, ref, f"random decode {cid}")
    # The separate calls from the pre-store pools: the same bits.
    case["k_cache"].copy_(h["k_cache"])
    case["v_cache"].copy_(h["v_cache"])
    gpu_store(case)
    sep = gpu_decode(case)
    torch.cuda.synchronize()
    assert torch.equal(sep, fused), "fused and separate decode steps differ"


@pytest.mark.parametrize("cid,hq,hkv,bs,new,pre,scale,seed", PREFILL_DRAWS,
                         ids=[d[0] for d in PREFILL_DRAWS])
def test_prefill_random(cid, hq, hkv, bs, new, pre, scale, seed):
    say(f"[case] random prefill {cid}: new={new} prefix_blocks={pre} scale={scale} seed={seed}")
    h = workloads.prefill_case(len(new), (1, 300), hq, hkv, 128, bs, seed=seed, device="cpu",
                               chains=3, chain_blocks=max(3, max(pre)), new_lens=new,
                               prefix_blocks=pre)
    h["scale"] = scale
    case = to_device(host_copy(h))
    gpu_store(case)
    out = gpu_prefill(case)
    torch.cuda.synchronize()
    kc, vc = oracle_after_store(h)
    assert np.array_equal(_pool_bits(case["k_cache"]), kc), "K pool differs from the oracle"
    ref = oracle.prefill(h["q"], kc, vc, h["cu_seqlens_q"], h["context_lens"], h["block_table"],
                         scale, nthreads=ORACLE_THREADS)
    compare(out, ref, f"random prefill {cid}")

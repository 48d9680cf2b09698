"""Pools larger than 4 GiB. Every K/V row a call touches lies past byte 2^32
(element 2^31) of its pool, so a 32-bit offset anywhere in the store, the
decode step or the prefill would read or write the wrong rows.

Each case is generated with a compact pool. It then runs once on that pool
and once on pools whose first 4.5 GiB are left unused, with block i of the
compact pool copied to block OFF + i and the block table and slot mapping
shifted to match. The two runs must give the same bits: the outputs, and the
pools' rows at and above OFF. The outputs must also match the oracle, and
the written rows must match the oracle's store bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_slot_amd as pa
import workloads
from tests.gpu_common import (DEV, ORACLE_THREADS, compare, gpu_prefill, gpu_store, host_copy,
                              oracle_after_store, require_gpu, say, to_device)

pytestmark = pytest.mark.gpu

LOW_BYTES = 9 << 29  # 4.5 GiB of each pool below the first block any call uses


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _pool_bits(t):
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def _high(h):
    """Device copy of case h with its pools moved above LOW_BYTES."""
    bs, hkv, d = h["k_cache"].shape[1:]
    block_bytes = bs * hkv * d * 2
    off = -(-LOW_BYTES // block_bytes)
    nb = h["k_cache"].shape[0]
    case = to_device(host_copy(h))
    for name in ("k_cache", "v_cache"):
        big = torch.empty((off + nb, bs, hkv, d), dtype=torch.bfloat16, device=DEV)
        big[off:].copy_(case[name])
        case[name] = big
    bt = case["block_table"]
    case["block_table"] = torch.where(bt >= 0, bt + off, bt).contiguous()
    sm = case["slot_mapping"]
    case["slot_mapping"] = torch.where(sm >= 0, sm + off * bs, sm).contiguous()
    assert off * block_bytes >= 1 << 32
    say(f"  pools of {(off + nb) * block_bytes / 2**30:.2f} GiB each, first used block {off}")
    return case, off


def _decode_store(case, scale):
    B, hq, d = case["q"].shape
    ws = torch.empty(max(16, pa.pa_decode_workspace_bytes(B, hq, d, case["max_context_len"],
                                                          case["block_size"])),
                     dtype=torch.uint8, device=DEV)
    out = torch.full_like(case["q"], float("nan"))
    pa.pa_decode_store(out, case["q"], case["k_new"], case["v_new"], case["k_cache"],
                       case["v_cache"], case["slot_mapping"], case["block_table"],
                       case["context_lens"], case["max_context_len"], scale, ws)
    return out


@pytest.mark.parametrize("bs", [256, 16])
def test_decode_step_large_pool(bs):
    say(f"[case] large-pool decode step, block_size {bs}, seed 4101")
    h = workloads.decode_case(48, (1, 3000), 16, 8, 128, bs, seed=4101, device="cpu",
                              spare_blocks=3)
    scale = h["scale"]
    small = to_device(host_copy(h))
    out_small = _decode_store(small, scale)
    big, off = _high(h)
    out_big = _decode_store(big, scale)
    torch.cuda.synchronize()
    assert torch.equal(out_big, out_small), "decode step differs above 4 GiB"
    for name in ("k_cache", "v_cache"):
        assert torch.equal(big[name][off:], small[name]), f"{name} rows differ above 4 GiB"
    kc, vc = oracle_after_store(h)
    assert np.array_equal(_pool_bits(small["k_cache"]), kc), "K pool differs from the oracle"
    assert np.array_equal(_pool_bits(small["v_cache"]), vc), "V pool differs from the oracle"
    ref = oracle.decode(h["q"], kc, vc, h["block_table"], h["context_lens"], scale,
                        nthreads=ORACLE_THREADS)
    compare(out_big, ref, f"large-pool decode step bs{bs}")
    del big, small
    torch.cuda.empty_cache()


def test_prefill_large_pool():
    say("[case] large-pool store + prefill, block_size 256, seed 4102")
    h = workloads.prefill_case(6, (1, 600), 32, 8, 128, 256, seed=4102, device="cpu",
                               chains=3, chain_blocks=3, prefix_blocks=[0, 1, 2, 3, 1, 2])
    small = to_device(host_copy(h))
    gpu_store(small)
    out_small = gpu_prefill(small)
    big, off = _high(h)
    gpu_store(big)
    out_big = gpu_prefill(big)
    torch.cuda.synchronize()
    assert torch.equal(out_big, out_small), "prefill differs above 4 GiB"
    for name in ("k_cache", "v_cache"):
        assert torch.equal(big[name][off:], small[name]), f"{name} rows differ above 4 GiB"
    kc, vc = oracle_after_store(h)
    assert np.array_equal(_pool_bits(small["k_cache"]), kc), "K pool differs from the oracle"
    ref = oracle.prefill(h["q"], kc, vc, h["cu_seqlens_q"], h["context_lens"], h["block_table"],
                         h["scale"], nthreads=ORACLE_THREADS)
    compare(out_big, ref, "large-pool prefill")
    del big, small
    torch.cuda.empty_cache()

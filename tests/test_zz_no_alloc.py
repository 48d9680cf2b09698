"""GPU test of pa_decode_store_noalloc, the decode step that allocates nothing
(its split-K records live in the library's fixed device scratch): through the
C ABI its output and pools equal pa_decode_store's (caller workspace) bit for
bit, on two calls in a row, the second with a smaller input of other head
counts, so the second call runs on scratch the first one left behind."""
import numpy as np
import pytest
import torch

import paged_kv_cache_slot_amd as pa
import workloads
from tests.gpu_common import DEV, require_gpu, say

pytestmark = pytest.mark.gpu

CALLS = [
    # (batch, len range, Hq, Hkv, block_size, explicit lengths or None)
    (300, (100, 2048), 32, 8, 16, None),
    (6, (1, 5000), 16, 8, 256, [5000, 1, 0, 257, 40, 2049]),
]


def _step(fn, case, ws=None):
    out = torch.full_like(case["q"], float("nan"))
    args = (out, case["q"], case["k_new"], case["v_new"], case["k_cache"], case["v_cache"],
            case["slot_mapping"], case["block_table"], case["context_lens"],
            case["max_context_len"], case["scale"])
    if ws is None:
        fn(*args)
    else:
        fn(*args, ws)
    return out


def test_noalloc_matches_workspace_call_twice():
    require_gpu()
    for i, (B, rng, hq, hkv, bs, lens) in enumerate(CALLS):
        say(f"[case] no-alloc decode step, call {i + 1}: B={B} Hq={hq} Hkv={hkv} bs={bs}")
        case = workloads.decode_case(B, rng, hq, hkv, 128, bs, seed=4100 + i, device=DEV,
                                     lens=lens, spare_blocks=2)
        kc0, vc0 = case["k_cache"].clone(), case["v_cache"].clone()
        ws = torch.empty(max(16, pa.pa_decode_workspace_bytes(B, hq, 128, case["max_context_len"],
                                                              bs)), dtype=torch.uint8,
                         device=DEV)
        ref = _step(pa.pa_decode_store, case, ws)
        kc_ref, vc_ref = case["k_cache"].clone(), case["v_cache"].clone()
        case["k_cache"].copy_(kc0)
        case["v_cache"].copy_(vc0)
        got = _step(pa.pa_decode_store_noalloc, case)
        torch.cuda.synchronize()
        assert torch.isfinite(got.float()).all()
        assert torch.equal(got, ref), f"call {i + 1}: outputs differ"
        assert torch.equal(case["k_cache"], kc_ref) and torch.equal(case["v_cache"], vc_ref), \
            f"call {i + 1}: pools differ"
        pad = np.flatnonzero(np.asarray(case["lens"]) == 0)
        if len(pad):
            assert int(got[torch.from_numpy(pad).to(DEV)].float().abs().sum()) == 0
        say(f"  call {i + 1}: output and pools equal pa_decode_store's")

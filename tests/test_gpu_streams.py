"""Calls on two streams at once share nothing. The fused decode step (each
with its own workspace), the prefill and the sampler (each with its own
workspace) are enqueued on two default-priority streams in an interleaved
order, several times over, and every result must equal, bit for bit, the
same call made alone on the current stream. This guards against hidden
global state in the library: the no-allocation entry point, whose shared
scratch is documented, is the only one that has any.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_slot_amd as pa
import workloads
from tests.gpu_common import DEV, host_copy, require_gpu, say, to_device

pytestmark = pytest.mark.gpu

REPEATS = 3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _decode_case(seed, batch, hq, hkv, bs):
    h = workloads.decode_case(batch, (100, 2048), hq, hkv, 128, bs, seed=seed, device="cpu")
    ws_bytes = max(16, pa.pa_decode_workspace_bytes(batch, hq, 128, h["max_context_len"], bs))
    return h, ws_bytes


def _decode_call(case, ws, stream=None):
    out = case.setdefault("out", torch.empty_like(case["q"]))
    pa.pa_decode_store(out, case["q"], case["k_new"], case["v_new"], case["k_cache"],
                       case["v_cache"], case["slot_mapping"], case["block_table"],
                       case["context_lens"], case["max_context_len"], case["scale"], ws,
                       stream=stream)


def _prefill_call(case, stream=None):
    out = case.setdefault("out", torch.empty_like(case["q"]))
    pa.pa_prefill_varlen(out, case["q"], case["k_cache"], case["v_cache"], case["cu_seqlens_q"],
                         case["context_lens"], case["block_table"], case["max_seqlen_q"],
                         case["scale"], stream=stream)


def _sample_call(job, stream=None):
    pa.pa_sample_gumbel(job["tokens"], job["probs"], job["seed"], 0, workspace=job["ws"],
                        stream=stream)


def test_two_streams_share_nothing():
    say("[case] two streams: decode steps (seeds 8101, 8102), prefills (8103, 8104), "
        "samplers (8105, 8106)")
    dec_h = [_decode_case(8101, 64, 16, 8, 256), _decode_case(8102, 48, 32, 8, 16)]
    pre_h = [workloads.prefill_case(4, (50, 400), 32, 8, 128, 256, seed=8103, device="cpu",
                                    chains=2, chain_blocks=2),
             workloads.prefill_case(3, (50, 300), 16, 8, 128, 64, seed=8104, device="cpu",
                                    chains=2, chain_blocks=2)]
    gen = torch.Generator().manual_seed(8105)
    probs = [torch.softmax(torch.randn(r, 32000, generator=gen), dim=1) for r in (16, 24)]

    def fresh():
        """Device copies of every input (the fused step writes its pools)."""
        decs = [(to_device(host_copy(h)),
                 torch.empty(n, dtype=torch.uint8, device=DEV)) for h, n in dec_h]
        pres = [to_device(host_copy(h)) for h in pre_h]
        for c in pres:
            pa.pa_store_kvcache(c["k_new"], c["v_new"], c["k_cache"], c["v_cache"],
                                c["slot_mapping"])
        samps = [dict(probs=p.to(DEV), tokens=torch.empty(p.shape[0], dtype=torch.int32,
                                                           device=DEV),
                      ws=torch.empty(max(8, pa.pa_sample_workspace_bytes(*p.shape)),
                                     dtype=torch.uint8, device=DEV), seed=8105 + i)
                 for i, p in enumerate(probs)]
        torch.cuda.synchronize()
        return decs, pres, samps

    # Each call alone, in turn, on the current stream.
    decs, pres, samps = fresh()
    for c, ws in decs:
        _decode_call(c, ws)
        torch.cuda.synchronize()
    for c in pres:
        _prefill_call(c)
        torch.cuda.synchronize()
    for j in samps:
        _sample_call(j)
        torch.cuda.synchronize()
    ref_dec = [(c["out"].clone(), c["k_cache"].clone(), c["v_cache"].clone()) for c, _ in decs]
    ref_pre = [c["out"].clone() for c in pres]
    ref_smp = [j["tokens"].clone() for j in samps]

    # The same calls, interleaved on two streams, several times over.
    decs, pres, samps = fresh()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for _ in range(REPEATS):
        for i in range(2):
            s = streams[i]
            with torch.cuda.stream(s):
                _decode_call(decs[i][0], decs[i][1], stream=s.cuda_stream)
            s2 = streams[1 - i]
            with torch.cuda.stream(s2):
                _prefill_call(pres[i], stream=s2.cuda_stream)
                _sample_call(samps[i], stream=s2.cuda_stream)
    torch.cuda.synchronize()

    for i, ((c, _), (o, kc, vc)) in enumerate(zip(decs, ref_dec)):
        assert torch.equal(c["out"], o), f"decode step {i} differs on two streams"
        assert torch.equal(c["k_cache"], kc) and torch.equal(c["v_cache"], vc), \
            f"decode step {i}: pools differ on two streams"
    for i, (c, o) in enumerate(zip(pres, ref_pre)):
        assert torch.equal(c["out"], o), f"prefill {i} differs on two streams"
    for i, (j, t) in enumerate(zip(samps, ref_smp)):
        assert torch.equal(j["tokens"], t), f"sampler {i} differs on two streams"
    say(f"  {REPEATS} rounds on two streams: every result equal to the call alone")

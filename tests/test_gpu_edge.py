"""GPU parity on the method's numeric edge cases: softmax scales other than
1/sqrt(128), sharp attention, scores that keep rising along the context (the
online softmax must raise its reference and rescale, chunk after chunk and
tile after tile), one late key that dominates (o -> its value row), and
scores far beyond fp32's exponent range. Every case is checked against the
fp64 oracle, element by element, and each test asserts on the host, from the
inputs alone, that its scores really cross the kernels' rescale thresholds.

Thresholds the inputs must cross (in log2 units of the scaled score):
  decode:  a later 16-token chunk's maximum above the first chunk's by more
           than 8 (the decode kernel's reference headroom);
  prefill: a later 64-key tile's maximum above the first tile's by more than
           8 (a single exponential then exceeds 256, the per-lane row-sum
           bound that triggers a rescale), and for the overflow case by more
           than 128 (2^(s - m) is then infinite in fp32).
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_slot_amd as pa
import workloads
from tests import edge_inputs as ei
from tests.gpu_common import (DEV, ORACLE_THREADS, compare, gpu_prefill, gpu_store,
                              oracle_after_store, require_gpu, say, to_device)

pytestmark = pytest.mark.gpu

DECODE_CHUNK = 16    # tokens per decode chunk (4 groups of 4) at these head counts
PREFILL_TILE = 64    # keys per prefill tile
HEADROOM = 8.0       # log2 units


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _pool_bits(t):
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def _f32(x):
    return float(np.float32(x))


# ----------------------------------------------------------------- decode --

DECODE_EDGE = [
    # id, block_size, Hq, Hkv, lengths, scale, query multiplier per row, shaping
    ("ramp60-s0.3-40k", 16, 32, 8, [40000, 2048, 1000, 17, 0, 300], 0.3,
     [1, 8, 1, 8, 1, 8], ("ramp", 60.0)),
    ("ramp40-s1.0", 256, 16, 8, [5000, 1100, 257, 0, 64], 1.0, [1, 1, 8, 1, 1], ("ramp", 40.0)),
    ("ramp60-s0.02-q8", 64, 8, 8, [12345, 700, 3], 0.02, [8, 8, 8], ("ramp", 60.0)),
    ("dominant30-s1.0", 16, 32, 8, [3000, 513, 40, 2], 1.0, [1, 1, 1, 1], ("dominant", 3, 30.0)),
    ("dominant30-newtoken-s0.3", 128, 64, 8, [1500, 100, 0, 1], 0.3, [8, 1, 1, 1],
     ("dominant", 0, 30.0)),
    ("plain-s1.0-q8", 16, 32, 8, [2049, 333, 0, 1, 700], 1.0, [8, 8, 8, 8, 8], None),
    ("plain-s0.02", 256, 16, 8, [1024, 1, 4097], 0.02, [1, 1, 1], None),
]


@pytest.mark.parametrize("cid,bs,hq,hkv,lens,scale,qmul,shape", DECODE_EDGE,
                         ids=[c[0] for c in DECODE_EDGE])
def test_decode_store_edge(cid, bs, hq, hkv, lens, scale, qmul, shape):
    """pa_decode_store (the benchmarked call) on sharp / rising / dominated
    scores at non-default scales: every row against the oracle, both pools
    bit for bit."""
    scale = _f32(scale)
    say(f"[case] decode edge {cid}: bs={bs} Hq={hq} Hkv={hkv} lens={lens} scale={scale}")
    h = workloads.decode_case(len(lens), (1, 2048), hq, hkv, 128, bs, seed=1200 + bs + hq,
                              device="cpu", lens=lens, spare_blocks=3)
    h["scale"] = scale
    h["q"] = ei.scale_queries(h["q"], qmul)
    G = hq // hkv
    longest = int(np.argmax(lens))
    if shape and shape[0] == "ramp":
        ei.decode_ramp(h, shape[1], scale)
        s = ei.decode_scores(h, longest, 0, scale)
        rise = ei.max_rise_over_first_chunk(s, DECODE_CHUNK)
        say(f"  longest row: later chunk max above the first by {rise:.1f} log2 units")
        assert rise > HEADROOM, "inputs do not take the decode rescale path"
    elif shape and shape[0] == "dominant":
        ei.decode_dominant_key(h, shape[1], shape[2], scale)
        s = ei.decode_scores(h, longest, 0, scale)
        j = lens[longest] - 1 - shape[1]
        margin = s[j] - np.delete(s, j).max()
        say(f"  dominant key at {j}: {margin:.1f} log2 units above the rest")
        assert margin > 20.0
        if j >= DECODE_CHUNK:
            assert s[j] - s[:DECODE_CHUNK].max() > HEADROOM
    else:
        s = ei.decode_scores(h, longest, 0, scale)
        say(f"  score spread {s.max() - s.min():.1f} log2 units")
    case = to_device(h)
    B = len(lens)
    out = torch.full_like(case["q"], float("nan"))
    ws = torch.empty(max(16, pa.pa_decode_workspace_bytes(B, hq, 128, case["max_context_len"],
                                                          bs)), dtype=torch.uint8, device=DEV)
    pa.pa_decode_store(out, case["q"], case["k_new"], case["v_new"], case["k_cache"],
                       case["v_cache"], case["slot_mapping"], case["block_table"],
                       case["context_lens"], case["max_context_len"], scale, ws)
    torch.cuda.synchronize()
    kc, vc = oracle_after_store(h)
    assert np.array_equal(_pool_bits(case["k_cache"]), kc), "K pool differs from the oracle"
    assert np.array_equal(_pool_bits(case["v_cache"]), vc), "V pool differs from the oracle"
    ref = oracle.decode(h["q"], kc, vc, h["block_table"], h["context_lens"], scale,
                        nthreads=ORACLE_THREADS)
    compare(out, ref, f"decode edge {cid}")
    if shape and shape[0] == "dominant":
        # o -> v of the dominant key for the heads it was built for.
        for b, L in enumerate(lens):
            j = L - 1 - shape[1]
            if j < 0:
                continue
            for g in range(hkv):
                if j == L - 1:
                    vj = h["v_new"][b, g].double().numpy()
                else:
                    slot = int(h["block_table"][b, j // bs]) * bs + j % bs
                    vj = vc.reshape(-1, hkv, 128)[slot, g].view(np.uint16)
                    vj = torch.from_numpy(vj.astype(np.int32) << 16).view(torch.float32)
                    vj = vj.double().numpy()
                assert np.abs(ref[b, g * G] - vj).max() < 1e-3
                assert np.abs(out[b, g * G].double().cpu().numpy() - vj).max() <= 1e-2


# ---------------------------------------------------------------- prefill --

PREFILL_EDGE = [
    # id, block_size, Hq, Hkv, new lengths, prefix blocks, scale, query multiplier, shaping
    ("ramp60-s0.3", 256, 32, 8, [300, 64, 1, 700], [3, 1, 2, 0], 0.3, 1.0, ("ramp", 60.0)),
    ("ramp40-s1.0", 16, 16, 16, [200, 129, 5], [1, 2, 0], 1.0, 1.0, ("ramp", 40.0)),
    ("ramp60-s0.02", 64, 16, 8, [70, 300, 2], [2, 0, 1], 0.02, 1.0, ("ramp", 60.0)),
    ("dominant150-overflow-s0.3", 256, 32, 8, [300, 100, 64], [1, 0, 3], 0.3, 1.0,
     ("dominant", 2, 150.0)),
    ("dominant30-s1.0", 32, 64, 8, [40, 90, 17], [1, 3, 0], 1.0, 1.0, ("dominant", 0, 30.0)),
    ("plain-s1.0-q8", 16, 32, 8, [100, 257], [1, 0], 1.0, 8.0, None),
    ("plain-s0.02-q8", 256, 32, 8, [500, 33], [2, 1], 0.02, 8.0, None),
]


def _tile_rise(s):
    first = s[:PREFILL_TILE].max()
    later = [s[t:t + PREFILL_TILE].max() for t in range(PREFILL_TILE, len(s), PREFILL_TILE)]
    return float(max(later) - first) if later else 0.0


@pytest.mark.parametrize("cid,bs,hq,hkv,new,pre,scale,qmul,shape", PREFILL_EDGE,
                         ids=[c[0] for c in PREFILL_EDGE])
def test_prefill_edge(cid, bs, hq, hkv, new, pre, scale, qmul, shape):
    """Store + prefill over cached prefixes with sharp / rising / dominated
    scores at non-default scales: every row against the oracle."""
    scale = _f32(scale)
    say(f"[case] prefill edge {cid}: bs={bs} Hq={hq} Hkv={hkv} new={new} prefix_blocks={pre} "
        f"scale={scale}")
    h = workloads.prefill_case(len(new), (1, 1024), hq, hkv, 128, bs, seed=1300 + bs + hq,
                               device="cpu", chains=len(new), chain_blocks=3, new_lens=new,
                               prefix_blocks=pre, prefix_chain=list(range(len(new))))
    h["scale"] = scale
    if qmul != 1.0:
        h["q"] = ei.scale_queries(h["q"], [qmul] * h["q"].shape[0])
    cu = h["cu_seqlens_q"].numpy()
    L = h["context_lens"].numpy()
    longest = int(np.argmax(L))
    t_last = int(cu[longest + 1]) - 1
    if shape and shape[0] == "ramp":
        # Every sequence has a prefix chain of its own here, so no sequence's
        # ramp is written over by another's in a shared block.
        ei.prefill_ramp(h, shape[1], scale)
        s = ei.prefill_scores(h, t_last, 0, scale)
        rise = _tile_rise(s)
        say(f"  longest sequence, last row: later tile max above the first by {rise:.1f}")
        assert rise > HEADROOM, "inputs do not take the prefill rescale path"
    elif shape and shape[0] == "dominant":
        ei.prefill_dominant_key(h, shape[1], shape[2], scale)
        s = ei.prefill_scores(h, t_last, 0, scale)
        j = int(L[longest]) - 1 - shape[1]
        margin = s[j] - np.delete(s, j).max()
        say(f"  dominant key at {j}: {margin:.1f} log2 units above the rest, "
            f"{s[j] - s[:PREFILL_TILE].max():.1f} above the first tile")
        assert margin > 20.0
        if shape[2] > 128:
            assert s[j] - s[:PREFILL_TILE].max() > 128.0, "no fp32 overflow of 2^(s - m)"
    else:
        s = ei.prefill_scores(h, t_last, 0, scale)
        say(f"  score spread {s.max() - s.min():.1f} log2 units, later tile rise "
            f"{_tile_rise(s):.1f}")
    case = to_device(h)
    gpu_store(case)
    out = gpu_prefill(case)
    torch.cuda.synchronize()
    kc, vc = oracle_after_store(h)
    ref = oracle.prefill(h["q"], kc, vc, h["cu_seqlens_q"], h["context_lens"], h["block_table"],
                         scale, nthreads=ORACLE_THREADS)
    compare(out, ref, f"prefill edge {cid}")

"""GPU parity: the HIP path through the C ABI against the CPU oracle.

KV stores must be bit-exact over the whole pool. Attention must satisfy
|gpu - oracle| <= 1e-2 + 1e-2 |oracle| element-wise, with the oracle in fp64.
Full-size workloads are checked on sampled rows the oracle computes one by one;
small cases that still span several tiles and ragged tails are checked on
every row.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_slot_amd as pa
import workloads
from tests.gpu_common import (DEV, compare, gpu_decode, gpu_prefill, gpu_store, host_copy,
                              make_case, oracle_after_store, require_gpu, say,
                              ORACLE_THREADS)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _pool_bits(t):
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


# ------------------------------------------------------------------ store --

@pytest.mark.parametrize("name", ["tiny_decode", "qwen3_8b_decode", "bs16_stress_decode",
                                  "qwen3_8b_prefill_prefix"])
def test_store_bit_exact_full_pool(name):
    """Whole-pool memcmp after the store, -1 rows included (the Qwen3-8B and
    block-16 decode workloads pad)."""
    case, h = make_case(name)
    say(f"  pa_store_kvcache T={case['slot_mapping'].numel()} "
        f"(-1 rows: {int((h['slot_mapping'] < 0).sum())})")
    gpu_store(case)
    torch.cuda.synchronize()
    kc, vc = oracle_after_store(h)
    assert np.array_equal(_pool_bits(case["k_cache"]), kc), "K pool differs from the oracle"
    assert np.array_equal(_pool_bits(case["v_cache"]), vc), "V pool differs from the oracle"
    # The store must have changed every named slot (the pool held other data).
    named = h["slot_mapping"][h["slot_mapping"] >= 0].numpy()
    before = _pool_bits(h["k_cache"]).reshape(-1, h["num_kv_heads"] * 128)
    assert not np.array_equal(before[named], kc.reshape(-1, h["num_kv_heads"] * 128)[named])


def test_store_fused_qkv_rows():
    """k and v as row slices of a fused [T, (Hq + 2 Hkv) * D] projection output."""
    T, hq, hkv, d, nb, bs = 300, 32, 8, 128, 24, 16
    gen = torch.Generator(device=DEV).manual_seed(5)
    fused = torch.randn(T, (hq + 2 * hkv) * d, generator=gen, device=DEV).to(torch.bfloat16)
    kc = torch.randn(nb, bs, hkv, d, generator=gen, device=DEV).to(torch.bfloat16)
    vc = torch.randn(nb, bs, hkv, d, generator=gen, device=DEV).to(torch.bfloat16)
    rng = np.random.default_rng(5)
    slots = rng.choice(nb * bs, size=T, replace=False).astype(np.int32)
    slots[rng.choice(T, size=30, replace=False)] = -1
    k = fused[:, hq * d:(hq + hkv) * d]
    v = fused[:, (hq + hkv) * d:]
    h = dict(k=k.cpu(), v=v.cpu(), kc=kc.cpu(), vc=vc.cpu())
    say("  pa_store_kvcache fused rows, T=300, bs=16")
    pa.pa_store_kvcache(k, v, kc, vc, torch.from_numpy(slots).to(DEV))
    torch.cuda.synchronize()
    ek, ev = oracle.store_kvcache(h["k"], h["v"], h["kc"], h["vc"], slots, bs)
    assert np.array_equal(_pool_bits(kc), ek) and np.array_equal(_pool_bits(vc), ev)


def test_store_empty_is_noop():
    kc = torch.zeros(2, 16, 8, 128, dtype=torch.bfloat16, device=DEV)
    e = torch.empty(0, 8, 128, dtype=torch.bfloat16, device=DEV)
    pa.pa_store_kvcache(e, e, kc, kc.clone(), torch.empty(0, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    assert int(kc.abs().sum()) == 0


# ----------------------------------------------------------------- decode --

@pytest.mark.parametrize("name", ["tiny_decode", "qwen3_0.6b_decode", "qwen3_8b_decode",
                                  "bs16_stress_decode"])
def test_decode_step_full_size(name):
    """The decode step on the full workload, both ways it can be called: the
    fused pa_decode_store (the call the benchmark times) and pa_store_kvcache
    followed by pa_decode. Every row of both outputs against the oracle, both
    pools bit for bit against the oracle's store after each, and the two
    outputs bit for bit against each other."""
    case, h = make_case(name)
    B, hq, d = case["q"].shape
    say(f"  pa_decode_store B={case['batch']} Hq={case['num_q_heads']} "
        f"Hkv={case['num_kv_heads']} bs={case['block_size']} max_len={case['max_context_len']} "
        f"(-1 slots: {int((h['slot_mapping'] < 0).sum())})")
    ws = torch.empty(max(16, pa.pa_decode_workspace_bytes(B, hq, d, case["max_context_len"],
                                                          case["block_size"])),
                     dtype=torch.uint8, device=DEV)
    fused = torch.full_like(case["q"], float("nan"))
    pa.pa_decode_store(fused, case["q"], case["k_new"], case["v_new"], case["k_cache"],
                       case["v_cache"], case["slot_mapping"], case["block_table"],
                       case["context_lens"], case["max_context_len"], case["scale"], ws)
    torch.cuda.synchronize()
    kc, vc = oracle_after_store(h)
    assert np.array_equal(_pool_bits(case["k_cache"]), kc), "fused: K pool differs from the oracle"
    assert np.array_equal(_pool_bits(case["v_cache"]), vc), "fused: V pool differs from the oracle"
    ref = oracle.decode(h["q"], kc, vc, h["block_table"], h["context_lens"], h["scale"],
                        nthreads=ORACLE_THREADS)
    compare(fused, ref, f"{name} pa_decode_store, every row")
    pad = np.flatnonzero(h["lens"] == 0)
    if len(pad):
        assert int(fused[torch.from_numpy(pad).to(DEV)].float().abs().sum()) == 0

    # The same step as two calls, from the pre-store pools.
    case["k_cache"].copy_(h["k_cache"])
    case["v_cache"].copy_(h["v_cache"])
    say("  pa_store_kvcache + pa_decode")
    gpu_store(case)
    sep = gpu_decode(case)
    torch.cuda.synchronize()
    assert np.array_equal(_pool_bits(case["k_cache"]), kc), "store: K pool differs from the oracle"
    assert np.array_equal(_pool_bits(case["v_cache"]), vc), "store: V pool differs from the oracle"
    compare(sep, ref, f"{name} pa_store_kvcache + pa_decode, every row")
    assert torch.equal(sep, fused), "fused and separate decode steps differ"


DECODE_GRID = [
    # (block_size, Hq, Hkv, lengths)
    (16, 32, 8, [1, 15, 16, 17, 255, 256, 257, 600, 1023, 0, 2048, 333]),
    (256, 16, 8, [1, 255, 256, 257, 511, 512, 513, 0, 1100, 77]),
    (32, 8, 8, [3, 64, 700, 129, 1, 256]),
    (64, 16, 2, [5, 300, 1000, 0, 640]),
    (128, 32, 4, [100, 1500, 260, 1]),
    (16, 64, 8, [1, 17, 290, 513, 40]),
]


@pytest.mark.parametrize("bs,hq,hkv,lens", DECODE_GRID,
                         ids=[f"bs{a}-hq{b}-hkv{c}" for a, b, c, _ in DECODE_GRID])
def test_decode_grid_all_rows(bs, hq, hkv, lens):
    """Pairs cut by the work split, ragged chunk and block tails, padding rows,
    every GQA ratio."""
    say(f"[case] decode grid bs={bs} Hq={hq} Hkv={hkv} lens={lens}")
    case = workloads.decode_case(len(lens), (1, 2048), hq, hkv, 128, bs, seed=77 + bs + hq,
                                 device=DEV, lens=lens, spare_blocks=5)
    h = host_copy(case)
    gpu_store(case)
    out = gpu_decode(case)
    torch.cuda.synchronize()
    kc, vc = oracle_after_store(h)
    ref = oracle.decode(h["q"], kc, vc, h["block_table"], h["context_lens"], h["scale"],
                        nthreads=ORACLE_THREADS)
    compare(out, ref, "decode grid")
    for b, L in enumerate(lens):
        if L == 0:
            assert int(out[b].float().abs().sum()) == 0


def test_decode_large_batch_long_pieces():
    """520 rows x 8 kv heads (4160 pairs, most of them cut between wavefronts),
    lengths on and around chunk, block and 1024-token boundaries, padding rows:
    every row."""
    rng = np.random.default_rng(41)
    lens = rng.integers(1, 2100, size=520)
    lens[:12] = [1, 1023, 1024, 1025, 2047, 2048, 2049, 0, 511, 512, 513, 2099]
    say("[case] decode 520 rows, bs=32, Hq=16, Hkv=8, lengths U[1,2100) + boundaries")
    case = workloads.decode_case(520, (1, 2100), 16, 8, 128, 32, seed=41, device=DEV,
                                 lens=lens)
    h = host_copy(case)
    gpu_store(case)
    out = gpu_decode(case)
    torch.cuda.synchronize()
    kc, vc = oracle_after_store(h)
    ref = oracle.decode(h["q"], kc, vc, h["block_table"], h["context_lens"], h["scale"],
                        nthreads=ORACLE_THREADS)
    compare(out, ref, "decode 520 rows")
    assert int(out[7].float().abs().sum()) == 0


LONG_ROWS = [
    # (block_size, Hq, Hkv, lengths)
    (256, 16, 8, [40000, 5, 0, 3000]),
    (128, 32, 8, [25000, 1]),
    (64, 8, 8, [12345]),
]


@pytest.mark.parametrize("bs,hq,hkv,lens", LONG_ROWS,
                         ids=[f"bs{a}-hq{b}-hkv{c}" for a, b, c, _ in LONG_ROWS])
def test_decode_long_rows_many_pieces(bs, hq, hkv, lens):
    """Few very long rows: each (sequence, kv head) pair is cut between tens to
    hundreds of wavefronts, so the merge folds many pieces per pair."""
    say(f"[case] decode long rows bs={bs} Hq={hq} Hkv={hkv} lens={lens}")
    case = workloads.decode_case(len(lens), (1, 2048), hq, hkv, 128, bs, seed=5 + bs,
                                 device=DEV, lens=lens, spare_blocks=2)
    h = host_copy(case)
    gpu_store(case)
    out = gpu_decode(case)
    torch.cuda.synchronize()
    kc, vc = oracle_after_store(h)
    ref = oracle.decode(h["q"], kc, vc, h["block_table"], h["context_lens"], h["scale"],
                        nthreads=ORACLE_THREADS)
    compare(out, ref, "decode long rows")
    for b, L in enumerate(lens):
        if L == 0:
            assert int(out[b].float().abs().sum()) == 0


# Batches on both sides of the two points where the decode's wavefront count
# changes regime. With 16 q / 8 kv heads, contexts U[900, 1100] and chunks of
# 16 tokens, a (sequence, kv head) pair costs about 64.5 units, so the cost
# line holds C ~ 516 B units: near B = 16, C / 4 reaches 2048 (below it every
# wavefront takes 4 units); near B = 64, C / 16 does (above it 16 units each).
CROSSOVER_BATCHES = [15, 16, 17, 62, 63, 64, 65]


@pytest.mark.parametrize("batch", CROSSOVER_BATCHES)
def test_decode_wave_count_crossovers(batch):
    """Decode parity at batch sizes around both changes of the work share per
    wavefront (4 units, then 2048 wavefronts, then 16 units)."""
    say(f"[case] decode crossover batch={batch}")
    case = workloads.decode_case(batch, (900, 1100), 16, 8, 128, 256, seed=700 + batch,
                                 device=DEV)
    h = host_copy(case)
    gpu_store(case)
    out = gpu_decode(case)
    torch.cuda.synchronize()
    kc, vc = oracle_after_store(h)
    ref = oracle.decode(h["q"], kc, vc, h["block_table"], h["context_lens"], h["scale"],
                        nthreads=ORACLE_THREADS)
    compare(out, ref, f"decode crossover batch {batch}")


FUSED_CASES = [
    # (block_size, Hq, Hkv, lengths): ragged tails, padding rows, pairs cut many times
    (16, 32, 8, [1, 15, 16, 17, 255, 256, 257, 600, 1023, 0, 2048, 333]),
    (256, 16, 8, [1, 255, 256, 257, 0, 1100, 77, 40000]),
    (64, 8, 8, [12345, 2, 0, 64]),
    (128, 64, 8, [100, 1500, 0, 1]),
]


def _fused_vs_separate(case, say_what):
    """Runs the decode step twice on copies of the pools: pa_store_kvcache then
    pa_decode, and pa_decode_store. Returns (separate out, fused out, pools...)."""
    kc0, vc0 = case["k_cache"].clone(), case["v_cache"].clone()
    gpu_store(case)
    sep = gpu_decode(case)
    kc_sep, vc_sep = case["k_cache"].clone(), case["v_cache"].clone()
    case["k_cache"].copy_(kc0)
    case["v_cache"].copy_(vc0)
    B, hq, d = case["q"].shape
    out = torch.full_like(case["q"], float("nan"))
    ws = torch.empty(max(16, pa.pa_decode_workspace_bytes(B, hq, d, case["max_context_len"],
                                                          case["block_size"])),
                     dtype=torch.uint8, device=DEV)
    say(f"[case] {say_what}")
    pa.pa_decode_store(out, case["q"], case["k_new"], case["v_new"], case["k_cache"],
                       case["v_cache"], case["slot_mapping"], case["block_table"],
                       case["context_lens"], case["max_context_len"], case["scale"], ws)
    torch.cuda.synchronize()
    return sep, out, kc_sep, vc_sep


@pytest.mark.parametrize("bs,hq,hkv,lens", FUSED_CASES,
                         ids=[f"bs{a}-hq{b}-hkv{c}" for a, b, c, _ in FUSED_CASES])
def test_decode_store_fused_equals_separate(bs, hq, hkv, lens):
    """pa_decode_store gives the output and pools of pa_store_kvcache + pa_decode,
    bit for bit, and the output matches the oracle."""
    case = workloads.decode_case(len(lens), (1, 2048), hq, hkv, 128, bs, seed=900 + bs + hq,
                                 device=DEV, lens=lens, spare_blocks=3)
    h = host_copy(case)
    sep, fused, kc_sep, vc_sep = _fused_vs_separate(
        case, f"fused decode store bs={bs} Hq={hq} Hkv={hkv} lens={lens}")
    assert torch.equal(case["k_cache"], kc_sep) and torch.equal(case["v_cache"], vc_sep)
    assert torch.equal(fused, sep)
    kc, vc = oracle_after_store(h)
    ref = oracle.decode(h["q"], kc, vc, h["block_table"], h["context_lens"], h["scale"],
                        nthreads=ORACLE_THREADS)
    compare(fused, ref, "fused decode store")


def test_decode_store_fused_large_batch_and_prestored_rows():
    """More rows than one launch covers (the fused store follows each slice), and
    live rows whose new token is already in the pool (slot -1): every row and
    both pools equal the separate calls."""
    rng = np.random.default_rng(8)
    lens = rng.integers(1, 600, size=1500)
    lens[rng.choice(1500, size=60, replace=False)] = 0
    case = workloads.decode_case(1500, (1, 600), 16, 8, 128, 16, seed=8, device=DEV, lens=lens)
    # Rows 0..99 have their new token stored up front and pass slot -1.
    pre = torch.arange(100, device=DEV)
    live = case["slot_mapping"][pre] >= 0
    pa.pa_store_kvcache(case["k_new"][pre], case["v_new"][pre], case["k_cache"], case["v_cache"],
                        case["slot_mapping"][pre].contiguous())
    slots = case["slot_mapping"].clone()
    slots[pre] = -1
    case = dict(case, slot_mapping=slots)
    torch.cuda.synchronize()
    assert int(live.sum()) > 90
    sep, fused, kc_sep, vc_sep = _fused_vs_separate(case, "fused decode store, 1500 rows")
    assert torch.equal(case["k_cache"], kc_sep) and torch.equal(case["v_cache"], vc_sep)
    assert torch.equal(fused, sep)


def test_decode_more_rows_than_one_scan_window():
    """2600 rows (more than the 1024 rows of context lengths a work-group holds in
    LDS at once), mixed lengths and padding: every row against the oracle."""
    rng = np.random.default_rng(31)
    lens = rng.integers(1, 700, size=2600)
    lens[rng.choice(2600, size=150, replace=False)] = 0
    say("[case] decode 2600 rows, bs=16, Hq=16, Hkv=8, lengths U[1,700) + 150 padding")
    case = workloads.decode_case(2600, (1, 700), 16, 8, 128, 16, seed=31, device=DEV,
                                 lens=lens)
    h = host_copy(case)
    gpu_store(case)
    out = gpu_decode(case)
    torch.cuda.synchronize()
    kc, vc = oracle_after_store(h)
    ref = oracle.decode(h["q"], kc, vc, h["block_table"], h["context_lens"], h["scale"],
                        nthreads=ORACLE_THREADS)
    compare(out, ref, "decode 2600 rows")
    assert int(out[torch.from_numpy(np.flatnonzero(lens == 0)).to(DEV)].float().abs().sum()) == 0


def test_decode_max_context_len_above_all_rows():
    """A loose max_context_len (a larger workspace bound and grid cap than the rows
    need) changes neither the work split nor any output bit."""
    lens = [40, 300, 0, 513]
    case = workloads.decode_case(4, (1, 2048), 16, 8, 128, 16, seed=3, device=DEV, lens=lens)
    tight = gpu_decode(case)
    loose = gpu_decode(case, max_context_len=2048)
    torch.cuda.synchronize()
    assert torch.equal(tight, loose)


def test_decode_all_padding_and_empty_batch():
    case = workloads.decode_case(3, (1, 10), 16, 8, 128, 256, seed=4, device=DEV, lens=[0, 0, 0],
                                 spare_blocks=1)
    out = gpu_decode(case)
    torch.cuda.synchronize()
    assert int(out.float().abs().sum()) == 0
    e = torch.empty(0, 16, 128, dtype=torch.bfloat16, device=DEV)
    pa.pa_decode(e, e, case["k_cache"], case["v_cache"],
                 torch.empty(0, 1, dtype=torch.int32, device=DEV),
                 torch.empty(0, dtype=torch.int32, device=DEV), 0, 0.1, None)


def test_decode_block_permutation_bitwise():
    """Relabelling physical blocks (pool and table together) changes no output bit."""
    lens = [1000, 17, 256, 2048, 513]
    for bs in (16, 256):
        case = workloads.decode_case(5, (1, 2048), 32, 8, 128, bs, seed=9, device=DEV, lens=lens,
                                     spare_blocks=7)
        out1 = gpu_decode(case)
        nb = case["num_blocks"]
        perm = torch.from_numpy(np.random.default_rng(9).permutation(nb)).to(DEV)
        kc2 = torch.empty_like(case["k_cache"]); kc2[perm] = case["k_cache"]
        vc2 = torch.empty_like(case["v_cache"]); vc2[perm] = case["v_cache"]
        bt = case["block_table"]
        bt2 = torch.where(bt >= 0, perm.to(torch.int32)[bt.clamp(min=0).long()], bt)
        out2 = gpu_decode(dict(case, k_cache=kc2, v_cache=vc2, block_table=bt2.contiguous()))
        torch.cuda.synchronize()
        assert torch.equal(out1, out2), f"bs={bs}: permutation changed bits"


def test_decode_deterministic():
    case = workloads.workload_case("tiny_decode", device=DEV)
    a = gpu_decode(case)
    b = gpu_decode(case)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# ---------------------------------------------------------------- prefill --

def _whole_sequences(h, extra, seed):
    """Sequences to check in full: the longest, the longest of each prefix
    length (0 .. 3 blocks), and `extra` more drawn at random."""
    N = np.asarray(h["new_lens"])
    k = np.asarray(h["prefix_blocks"])
    pick = {int(np.argmax(N))}
    for kb in range(int(k.max()) + 1):
        cand = np.flatnonzero(k == kb)
        if len(cand):
            pick.add(int(cand[np.argmax(N[cand])]))
    rng = np.random.default_rng(seed)
    rest = [b for b in range(len(N)) if b not in pick]
    pick |= set(int(b) for b in rng.choice(rest, size=min(extra, len(rest)), replace=False))
    return sorted(pick)


def test_prefill_full_size():
    """The Qwen3-8B prefill workload (64 sequences, cached prefixes from 8
    shared chains): store the new tokens, run prefill, then check every row and
    head of whole sequences -- the longest, the longest with each prefix length
    0..3 blocks, two more -- so that every query tile and key tile of those
    sequences is compared, plus 120 rows drawn from the whole batch and the
    first and last row of 10 more sequences."""
    case, h = make_case("qwen3_8b_prefill_prefix")
    say(f"  pa_store_kvcache + pa_prefill_varlen T={case['total_q']} "
        f"max_seqlen_q={case['max_seqlen_q']}")
    gpu_store(case)
    out = gpu_prefill(case)
    torch.cuda.synchronize()
    kc, vc = oracle_after_store(h)
    cu = h["cu_seqlens_q"].numpy()
    seqs = _whole_sequences(h, 2, seed=45)
    toks = set()
    for b in seqs:
        toks |= set(range(int(cu[b]), int(cu[b + 1])))
    say(f"  whole sequences {seqs}: new lengths {[int(h['new_lens'][b]) for b in seqs]}, "
        f"prefix blocks {[int(h['prefix_blocks'][b]) for b in seqs]}")
    rng = np.random.default_rng(44)
    toks |= set(int(x) for x in rng.choice(case["total_q"], size=120, replace=False))
    for b in rng.choice(case["batch"], size=10, replace=False):   # first and last rows
        toks |= {int(cu[b]), int(cu[b + 1] - 1)}
    toks = np.array(sorted(toks), dtype=np.int32)
    say(f"  {len(toks)} query rows of {case['total_q']} checked, all {case['num_q_heads']} heads")
    ref = oracle.prefill(h["q"], kc, vc, h["cu_seqlens_q"], h["context_lens"], h["block_table"],
                         h["scale"], tokens=toks, nthreads=ORACLE_THREADS)
    compare(out, ref, "qwen3_8b_prefill_prefix prefill (whole sequences + sample)", rows=toks)


PREFILL_GRID = [
    # (block_size, Hq, Hkv, new lengths, prefix blocks)
    (256, 32, 8, [100, 1, 33, 64, 257, 31], [0, 1, 3, 2, 1, 0]),
    (16, 32, 8, [50, 1, 128, 97], [3, 0, 1, 2]),
    (16, 16, 16, [200, 5, 129], [1, 2, 0]),
    (64, 16, 8, [70, 300, 2], [2, 0, 1]),
    (32, 64, 8, [40, 17, 90], [1, 3, 0]),
    (16, 8, 4, [1, 1, 2, 3], [0, 3, 1, 2]),
]


@pytest.mark.parametrize("bs,hq,hkv,new,pre", PREFILL_GRID,
                         ids=[f"bs{a}-hq{b}-hkv{c}" for a, b, c, _, _ in PREFILL_GRID])
def test_prefill_grid_all_rows(bs, hq, hkv, new, pre):
    """Every GQA ratio, prefixes that end mid key-tile, ragged query tiles, N = 1."""
    say(f"[case] prefill grid bs={bs} Hq={hq} Hkv={hkv} new={new} prefix_blocks={pre}")
    case = workloads.prefill_case(len(new), (1, 1024), hq, hkv, 128, bs, seed=500 + bs + hq,
                                  device=DEV, chains=2, chain_blocks=3, new_lens=new,
                                  prefix_blocks=pre, prefix_chain=[i % 2 for i in range(len(new))])
    h = host_copy(case)
    gpu_store(case)
    out = gpu_prefill(case)
    torch.cuda.synchronize()
    kc, vc = oracle_after_store(h)
    ref = oracle.prefill(h["q"], kc, vc, h["cu_seqlens_q"], h["context_lens"], h["block_table"],
                         h["scale"], nthreads=ORACLE_THREADS)
    compare(out, ref, "prefill grid")


def test_prefill_sequences_without_new_tokens():
    """Batch members with no new tokens (N = 0, cached prefix only) contribute no
    rows and leave their neighbours' rows exact; a batch with no new token at
    all is a no-op."""
    new, pre = [0, 50, 0, 3, 0], [2, 1, 0, 3, 3]
    say(f"[case] prefill with empty sequences new={new} prefix_blocks={pre}")
    case = workloads.prefill_case(len(new), (1, 64), 32, 8, 128, 16, seed=71, device=DEV,
                                  chains=2, chain_blocks=3, new_lens=new, prefix_blocks=pre,
                                  prefix_chain=[0, 1, 0, 1, 1])
    h = host_copy(case)
    gpu_store(case)
    out = gpu_prefill(case)
    torch.cuda.synchronize()
    kc, vc = oracle_after_store(h)
    ref = oracle.prefill(h["q"], kc, vc, h["cu_seqlens_q"], h["context_lens"], h["block_table"],
                         h["scale"], nthreads=ORACLE_THREADS)
    assert out.shape[0] == 53
    compare(out, ref, "prefill with empty sequences")
    empty = workloads.prefill_case(3, (1, 64), 32, 8, 128, 16, seed=72, device=DEV, chains=2,
                                   chain_blocks=3, new_lens=[0, 0, 0], prefix_blocks=[1, 2, 0],
                                   prefix_chain=[0, 1, 0])
    assert empty["q"].shape[0] == 0
    gpu_store(empty)
    out = gpu_prefill(empty)
    torch.cuda.synchronize()
    assert out.shape[0] == 0


def test_prefill_row_matches_decode():
    """Prefill row i of a sequence with prefix P and decode with L = P + i + 1
    over the same pool compute the same attention: both against the oracle's
    decode for those lengths, and the oracle's prefill and decode agree."""
    case = workloads.prefill_case(1, (1, 1024), 32, 8, 128, 16, seed=61, device=DEV, chains=1,
                                  chain_blocks=3, new_lens=[150], prefix_blocks=[3],
                                  prefix_chain=[0])
    h = host_copy(case)
    gpu_store(case)
    pre = gpu_prefill(case)
    P = 48
    rows = [0, 1, 15, 16, 63, 64, 100, 149]
    dec_case = dict(case, q=case["q"][rows].contiguous(),
                    block_table=case["block_table"].expand(len(rows), -1).contiguous(),
                    context_lens=torch.tensor([P + i + 1 for i in rows], dtype=torch.int32,
                                              device=DEV),
                    max_context_len=P + 150)
    dec = gpu_decode(dec_case)
    torch.cuda.synchronize()
    kc, vc = oracle_after_store(h)
    ref_dec = oracle.decode(h["q"][rows], kc, vc,
                            np.repeat(h["block_table"].numpy(), len(rows), axis=0),
                            np.array([P + i + 1 for i in rows], dtype=np.int32), h["scale"],
                            nthreads=ORACLE_THREADS)
    ref_pre = oracle.prefill(h["q"], kc, vc, h["cu_seqlens_q"], h["context_lens"],
                             h["block_table"], h["scale"], tokens=np.array(rows, np.int32),
                             nthreads=ORACLE_THREADS)[rows]
    assert np.array_equal(ref_pre, ref_dec)
    compare(pre[rows], ref_dec, "prefill rows against the oracle's decode")
    compare(dec, ref_dec, "decode at L = P + i + 1 against the oracle")


def test_prefill_shared_prefix_rows_identical():
    """Two sequences on the same 2 physical prefix blocks, recomputed in full
    (P = 0) with identical query rows there: identical output bits there."""
    bs, hq, hkv = 16, 32, 8
    case = workloads.prefill_case(2, (1, 1024), hq, hkv, 128, bs, seed=62, device=DEV, chains=1,
                                  chain_blocks=2, new_lens=[70, 90], prefix_blocks=[0, 0],
                                  prefix_chain=[0, 0])
    # Point both sequences' first two blocks at the same physical blocks and
    # give them the same keys/values/queries on those 32 positions.
    bt = case["block_table"].clone()
    bt[1, :2] = bt[0, :2]
    q = case["q"].clone()
    q[70:102] = q[0:32]
    kn, vn = case["k_new"].clone(), case["v_new"].clone()
    kn[70:102] = kn[0:32]
    vn[70:102] = vn[0:32]
    slots = case["slot_mapping"].clone()
    slots[70:102] = -1          # the shared rows are stored once, by sequence 0
    c2 = dict(case, block_table=bt, q=q, k_new=kn, v_new=vn, slot_mapping=slots)
    gpu_store(c2)
    out = gpu_prefill(c2)
    torch.cuda.synchronize()
    assert torch.equal(out[0:32], out[70:102])

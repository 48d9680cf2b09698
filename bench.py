#!/usr/bin/env python3
"""Benchmark of the paged-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-secondary] [--no-cpu-baseline]

One step = one pass of the hot path over one synthetic batch of the
Qwen3-0.6B-shaped decode workload (256 sequences, context lengths uniform in
[100, 2048], 16 query / 8 KV heads, head_dim 128, block_size 256, physical
blocks randomly permuted): one pa_decode_store call, which writes the 256 new
tokens' K/V into the pools and attends over the paged contexts. Inputs are
resident in HBM before timing starts. The headline `value` is algorithmic
bytes moved per step / step time (GB/s).

The same JSON line carries:
  roofline      for pa_decode_store (the stream-K attention kernel + its
                merge pass, which also writes the new tokens into the pools),
                timed with HIP events around each call on the launch stream;
  cpu_baseline  the CPU oracle (fp64) on the same step, on the host cores;
  secondary     the other workloads of the pages: Qwen3-8B-shaped decode
                (512 rows, 41 padding), block-16 stress decode (1024 rows),
                and Qwen3-8B-shaped varlen prefill with cached prefixes
                (TFLOP/s against the bf16 MFMA peak);
  block_manager host cost of the C++ block manager per decode step (batched
                append + decode metadata for 256 sequences) and per
                allocation, beside the oracle's Python manager;
  sampler       Gumbel-max sampling of 256 tokens from a 151936-entry
                vocabulary (GB/s of probabilities against HBM peak);
  decode_graphs wall time per decode step replayed from HIP graphs against
                the eager launches, at batches 1 .. 256, for dependent
                (wait after every step) and pipelined steps;
  mfma_ceiling  a library bf16 GEMM (torch.mm, 8192^3) on random and on
                zero operands: what the matrix cores sustain at the clock
                the chip holds under real data, beside the prefill figure.
Progress goes to stderr; stdout holds only the JSON line.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
MFMA_BF16_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 MFMA (2.5 PFLOP/s)
METRIC = "paged decode KV GB/s (% HBM peak); paged prefill TFLOP/s (% MFMA peak)"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_digest(*names):
    """Digest of the code of the named sources: comments and whitespace are
    removed first, so that only a change to the code itself invalidates the
    counter record taken on it."""
    import re
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "paged_kv_cache_slot_amd", "csrc", n), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)   # block comments
        text = re.sub(r"//[^\n]*", " ", text)                 # line comments
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel, digest):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they
    were taken on the current source of the kernel; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(kernel)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_digest") != digest:
        return None
    return rec["hbm_bytes_per_launch"]


# ------------------------------------------------------------- byte counts --

def decode_bytes(case):
    """Algorithmic HBM bytes of one pa_decode call: every K and V row of every
    context read once, q read for live rows, out written for all rows."""
    import numpy as np
    lens = np.asarray(case["lens"], dtype=np.int64)
    hkv, hq, d = case["num_kv_heads"], case["num_q_heads"], case["head_dim"]
    kv = int(lens.sum()) * hkv * d * 2 * 2
    q = int((lens > 0).sum()) * hq * d * 2
    out = len(lens) * hq * d * 2
    return kv + q + out


def store_bytes(case, fused=False):
    """pa_store_kvcache: read k and v of every stored new token, write them into
    the pools. Fused into the decode (pa_decode_store), the read is the decode's
    own read of the new token (already in decode_bytes): only the writes."""
    live = int((case["slot_mapping"] >= 0).sum())
    return live * case["num_kv_heads"] * case["head_dim"] * 2 * 2 * (1 if fused else 2)


def prefill_flops(case):
    """4 * Hq * D per causal (query, key) pair: N*P + N(N+1)/2 pairs per sequence."""
    import numpy as np
    N = np.asarray(case["new_lens"], dtype=np.int64)
    P = np.asarray(case["prefix_lens"], dtype=np.int64)
    pairs = int((N * P + N * (N + 1) // 2).sum())
    return 4 * case["num_q_heads"] * case["head_dim"] * pairs


# ----------------------------------------------------------------- timing --

# Warm-up of the secondary legs: at least this many steps and this many
# seconds of them. Measured in a fresh process, the Qwen3-8B decode steps get
# faster over the first seconds of GPU work (389 -> 363 us over four 20-step
# runs), so a few warm-up steps leave those legs below their steady state.
ORACLE_SECONDS = 10.0  # host time the decode oracle baseline runs for
SECONDARY_WARMUP = 10
SECONDARY_WARM_S = 0.5


class _no_gc:
    """Pauses Python's garbage collector (without running it) inside a timed
    region: a full collection can stall the launching thread for tens of
    milliseconds, and the GPU idle it causes lowers its clocks (measured: a
    50 ms idle gap before a warm-up slows the next Qwen3-8B decode steps by
    about 10%)."""

    def __enter__(self):
        import gc
        self.was_enabled = gc.isenabled()
        gc.disable()

    def __exit__(self, *exc):
        import gc
        if self.was_enabled:
            gc.enable()


def run_timed(step, warmup, steps, warm_s=0.0):
    """Warm up, then time exactly `steps` calls of step(i) between two device
    synchronisations, with the garbage collector paused (see _no_gc). Returns
    (ms per step, [per-step kernel ms])."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    with _no_gc():
        t_w = time.perf_counter()
        i = 0
        while i < warmup or time.perf_counter() - t_w < warm_s:
            step(i, None)
            i += 1
            if i % 64 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            step(i, evs[i])
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
    return ms, [a.elapsed_time(b) for a, b in evs]


def decode_bench(name, warmup, steps, fused=True, warm_s=0.0, flushed_only=False):
    import torch
    import numpy as np
    import paged_kv_cache_slot_amd as pa
    import workloads
    case = workloads.workload_case(name, device="cuda")
    B, hq, d = case["q"].shape
    out = torch.empty_like(case["q"])
    ws = torch.empty(pa.pa_decode_workspace_bytes(B, hq, d, case["max_context_len"],
                                                  case["block_size"]),
                     dtype=torch.uint8, device="cuda")
    # The buffer that evicts the 256 MB last-level cache (MALL) before each
    # call of the flushed protocol, allocated before anything is timed.
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()

    def step(i, ev):
        if fused:  # the store fused into the decode call
            if ev:
                ev[0].record()
            pa.pa_decode_store(out, case["q"], case["k_new"], case["v_new"], case["k_cache"],
                               case["v_cache"], case["slot_mapping"], case["block_table"],
                               case["context_lens"], case["max_context_len"], case["scale"], ws)
            if ev:
                ev[1].record()
            return
        pa.pa_store_kvcache(case["k_new"], case["v_new"], case["k_cache"], case["v_cache"],
                            case["slot_mapping"])
        if ev:
            ev[0].record()
        pa.pa_decode(out, case["q"], case["k_cache"], case["v_cache"], case["block_table"],
                     case["context_lens"], case["max_context_len"], case["scale"], ws)
        if ev:
            ev[1].record()

    def flushed_step(i, ev):
        # The survey's protocol: a 512 MiB write before every call (outside
        # its events), so no part of the pool is served from the MALL.
        scratch.fill_(i & 0xFF)
        step(i, ev)

    if flushed_only:  # the flushed loop alone (for a kernel trace of it)
        _, fk = run_timed(flushed_step, warmup, steps, warm_s)
        return dict(flushed_ms=float(np.median(fk)), flushed_all_ms=fk)
    ms, kms = run_timed(step, warmup, steps, warm_s)
    # The same call under the flushed protocol, warmed up the same way and
    # with the garbage collector paused: median of the decode calls.
    _, fk = run_timed(flushed_step, warmup, steps, warm_s)
    flushed_ms = float(np.median(fk))
    del scratch
    # Bytes of the timed call: the decode's, plus the fused store's writes.
    dbytes = decode_bytes(case) + (store_bytes(case, fused=True) if fused else 0)
    sbytes = 0 if fused else store_bytes(case)
    kern_ms = float(np.mean(kms))
    res = dict(case=case, ms_per_step=ms, step_bytes=dbytes + sbytes, decode_bytes=dbytes,
               decode_ms=kern_ms, gbs=(dbytes + sbytes) / (ms * 1e-3) / 1e9,
               decode_gbs=dbytes / (kern_ms * 1e-3) / 1e9, flushed_ms=flushed_ms,
               decode_ms_min=float(np.min(kms)), decode_ms_median=float(np.median(kms)),
               decode_ms_max=float(np.max(kms)),
               flushed_gbs=dbytes / (flushed_ms * 1e-3) / 1e9,
               flushed_ms_min=float(np.min(fk)), flushed_ms_max=float(np.max(fk)))
    return res


def prefill_bench(warmup, steps, warm_s=0.0):
    import torch
    import numpy as np
    import paged_kv_cache_slot_amd as pa
    import workloads
    case = workloads.workload_case("qwen3_8b_prefill_prefix", device="cuda")
    out = torch.empty_like(case["q"])
    torch.cuda.synchronize()

    def step(i, ev):
        pa.pa_store_kvcache(case["k_new"], case["v_new"], case["k_cache"], case["v_cache"],
                            case["slot_mapping"])
        if ev:
            ev[0].record()
        pa.pa_prefill_varlen(out, case["q"], case["k_cache"], case["v_cache"],
                             case["cu_seqlens_q"], case["context_lens"], case["block_table"],
                             case["max_seqlen_q"], case["scale"])
        if ev:
            ev[1].record()

    ms, kms = run_timed(step, warmup, steps, warm_s)
    flops = prefill_flops(case)
    kern_ms = float(np.mean(kms))
    return dict(ms_per_step=ms, flops=flops, prefill_ms=kern_ms,
                tflops=flops / (kern_ms * 1e-3) / 1e12, total_q=case["total_q"], case=case)


def prefill_lengths_bench(warmup, steps, warm_s=0.0,
                          lengths=(512, 1024, 2048, 4096, 8192, 16384), tokens=32768):
    """pa_prefill_varlen against prompt length: for each N, tokens // N
    sequences of N new tokens and no cached prefix (32 q / 8 kv heads,
    head_dim 128, block_size 256), algorithmic TFLOP/s. Beside it, torch's
    flash attention (forced flash backend, dense causal, K/V heads expanded)
    on the same shapes, for context; it is not part of the hot path."""
    import torch
    import numpy as np
    import paged_kv_cache_slot_amd as pa
    import workloads
    import torch.nn.functional as F
    rows = []
    for n in lengths:
        b = max(1, tokens // n)
        case = workloads.prefill_case(b, (n, n), 32, 8, 128, 256, seed=500 + n, device="cuda",
                                      chains=1, chain_blocks=1, new_lens=[n] * b,
                                      prefix_blocks=[0] * b, prefix_chain=[0] * b)
        pa.pa_store_kvcache(case["k_new"], case["v_new"], case["k_cache"], case["v_cache"],
                            case["slot_mapping"])
        out = torch.empty_like(case["q"])
        torch.cuda.synchronize()

        def step(i, ev):
            if ev:
                ev[0].record()
            pa.pa_prefill_varlen(out, case["q"], case["k_cache"], case["v_cache"],
                                 case["cu_seqlens_q"], case["context_lens"], case["block_table"],
                                 case["max_seqlen_q"], case["scale"])
            if ev:
                ev[1].record()

        _, kms = run_timed(step, warmup, steps, warm_s)
        flops = 4 * 32 * 128 * b * n * (n + 1) // 2
        us = float(np.median(kms)) * 1e3
        row = {"new_tokens": n, "sequences": b, "prefill_us": round(us, 1),
               "prefill_TFLOPs": round(flops / us / 1e6, 1),
               "prefill_frac_mfma": round(flops / us / 1e6 / MFMA_BF16_PEAK_TFLOPS, 4)}
        try:
            from torch.nn.attention import sdpa_kernel, SDPBackend
            q = case["q"].view(b, n, 32, 128).transpose(1, 2).contiguous()
            k = case["k_new"].view(b, n, 8, 128).transpose(1, 2).repeat_interleave(4, 1).contiguous()
            v = case["v_new"].view(b, n, 8, 128).transpose(1, 2).repeat_interleave(4, 1).contiguous()
            with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
                def tstep(i, ev):
                    if ev:
                        ev[0].record()
                    F.scaled_dot_product_attention(q, k, v, is_causal=True, scale=case["scale"])
                    if ev:
                        ev[1].record()
                _, tms = run_timed(tstep, warmup, steps, warm_s)
            tus = float(np.median(tms)) * 1e3
            row["torch_flash_us"] = round(tus, 1)
            row["torch_flash_TFLOPs"] = round(flops / tus / 1e6, 1)
            del q, k, v
        except (RuntimeError, ImportError) as e:  # no flash backend in this torch build
            row["torch_flash_us"] = None
            row["torch_flash_note"] = str(e)[:120]
        log(f"[bench] prefill {b} x {n}: {row}")
        rows.append(row)
        del case, out
        torch.cuda.empty_cache()
    return {"shape": "32 q / 8 kv heads, head_dim 128, block_size 256, no cached prefix",
            "rows": rows}


def mfma_ceiling_bench(warmup, steps, n=8192, warm_s=0.0):
    """A plain bf16 GEMM from the vendor library (torch.mm, C = A B with
    contiguous n x n operands), timed like the prefill leg, once on N(0,1)
    operands and once on zeros. Not part of the hot path: it shows the MFMA
    rate the chip sustains at the clock it holds under real data (zero
    operands draw less power, so the chip clocks higher), the practical
    ceiling beside the nominal peak."""
    import torch
    import numpy as np
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16, generator=gen)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16, generator=gen)
    c = torch.empty(n, n, device="cuda", dtype=torch.bfloat16)
    flops = 2.0 * n ** 3
    res = {"shape": f"bf16 [{n},{n}] x [{n},{n}]"}
    for kind in ("random", "zeros"):
        if kind == "zeros":
            a.zero_()
            b.zero_()
        torch.cuda.synchronize()

        def step(i, ev):
            if ev:
                ev[0].record()
            torch.mm(a, b, out=c)
            if ev:
                ev[1].record()

        _, kms = run_timed(step, warmup, steps, warm_s)
        med = float(np.median(kms))
        res[f"{kind}_us"] = round(med * 1e3, 2)
        res[f"{kind}_TFLOPs"] = round(flops / (med * 1e-3) / 1e12, 2)
        res[f"{kind}_frac_mfma"] = round(flops / (med * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)
    del a, b, c
    torch.cuda.empty_cache()
    return res


def block_manager_bench(decode_steps=256, oracle_steps=8):
    """Host cost of the block manager on the Qwen3-0.6B decode shape: 256
    sequences, block_size 256, prompts of U[100,1024] tokens of which 0..3
    leading blocks come from one of 8 shared prefix chains.

    native   the C++ calls timed by the `bm_bench` executable (no Python in
             the loop): allocation, decode steps of one batched append plus
             the step's decode metadata, prefill metadata, XXH64 throughput;
    binding  the same decode step through the Python binding, reusing its
             output arrays (what a Python scheduler pays per step);
    oracle   the oracle's plain Python manager: allocation of the batch and
             `oracle_steps` decode steps."""
    import subprocess
    import numpy as np
    from paged_kv_cache_slot_amd.block_manager import BlockManager
    from paged_kv_cache_slot_amd.build import BM_BENCH
    if not os.path.exists(BM_BENCH):
        raise RuntimeError(f"{BM_BENCH} is missing: run __graft_entry__.build()")
    native = json.loads(subprocess.run([BM_BENCH, "256", "256", str(decode_steps)],
                                       check=True, capture_output=True, text=True).stdout)
    B, bs, vocab = 256, 256, 151936
    rng = np.random.default_rng(4242)
    chains = rng.integers(0, vocab, size=(8, 3 * bs))
    prompts = []
    for _ in range(B):
        n = int(rng.integers(100, 1025))
        k = min(int(rng.integers(0, 4)), n // bs)
        head = chains[int(rng.integers(0, 8))][:k * bs]
        prompts.append(np.concatenate([head, rng.integers(0, vocab, size=n - k * bs)])
                       .astype(np.int32))
    gen = rng.integers(0, vocab, size=(decode_steps, B)).astype(np.int32)
    stride = -(-(max(len(p) for p in prompts) + decode_steps) // bs)
    num_blocks = sum(-(-(len(p) + decode_steps) // bs) for p in prompts) + 64
    ids = np.arange(B, dtype=np.int64)

    bm = BlockManager(num_blocks, bs)
    for i, p in enumerate(prompts):
        bm.allocate(i, p)
    out = (np.empty(B, np.int32), np.empty(B, np.int32), np.empty((B, stride), np.int32))
    t0 = time.perf_counter()
    for s in range(decode_steps):
        bm.append_batch(ids, gen[s])
        bm.decode_metadata(ids, B, stride, out=out)
    t_step = (time.perf_counter() - t0) / decode_steps

    import oracle.block_manager as obm
    ob = obm.BlockManager(num_blocks, bs)
    t0 = time.perf_counter()
    for i, p in enumerate(prompts):
        ob.allocate(i, p.tolist())
    o_alloc = time.perf_counter() - t0
    t0 = time.perf_counter()
    for s in range(oracle_steps):
        ob.append_batch(list(range(B)), gen[s].tolist())
        ob.decode_metadata(list(range(B)), B, stride)
    o_step = (time.perf_counter() - t0) / oracle_steps
    return {"native": native,
            "binding": {"decode_step_us": round(t_step * 1e6, 2), "steps": decode_steps},
            "oracle": {"allocate_us_per_seq": round(o_alloc / B * 1e6, 1),
                       "decode_step_us": round(o_step * 1e6, 1), "steps": oracle_steps}}


def graph_bench(batches=(1, 4, 16, 64, 256), steps=200, warmup=10):
    """Decode step replayed from HIP graphs against the same step launched
    eagerly, per batch size, on the Qwen3-0.6B decode shape (16 q / 8 kv
    heads, block_size 256, context lengths U[100,2048], permuted blocks).
    Both paths are driven from Python the way a serving loop would: eager =
    one pa_decode_store call per step (its two kernel launches), graph = one
    pa_decode_graphs_launch per step (the same launches captured). Two patterns, wall-clock microseconds per step over `steps`
    steps: dependent (the host waits for every step, as a decode loop that
    samples from each step must) and pipelined (steps enqueued back to back,
    one wait at the end)."""
    import numpy as np
    import torch
    import paged_kv_cache_slot_amd as pa
    B, hq, hkv, d, bs, max_len = 512, 16, 8, 128, 256, 2048
    stride = max_len // bs
    nb = B * stride + 8
    g = torch.Generator(device="cuda").manual_seed(5150)
    rnd = lambda *shape: torch.randn(*shape, generator=g, device="cuda").to(torch.bfloat16)
    kc, vc = rnd(nb, bs, hkv, d), rnd(nb, bs, hkv, d)
    q, kn, vn = rnd(B, hq, d), rnd(B, hkv, d), rnd(B, hkv, d)
    out = torch.empty(B, hq, d, dtype=torch.bfloat16, device="cuda")
    slots = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    lens = torch.zeros(B, dtype=torch.int32, device="cuda")
    table = torch.full((B, stride), -1, dtype=torch.int32, device="cuda")
    ws = torch.empty(pa.pa_decode_workspace_bytes(B, hq, d, max_len, bs), dtype=torch.uint8,
                     device="cuda")
    scale = 1.0 / np.sqrt(d)
    graphs = pa.pa_decode_graphs_create(out, q, kn, vn, kc, vc, slots, lens, table, ws, max_len,
                                        scale)
    rng = np.random.default_rng(5150)
    res = []
    for batch in batches:
        bucket = graphs.bucket(batch)
        L = np.zeros(bucket, np.int32)
        L[:batch] = rng.integers(100, max_len + 1, size=batch)
        perm = rng.permutation(nb)
        t = np.full((bucket, stride), -1, np.int32)
        sm = np.full(bucket, -1, np.int32)
        used = 0
        for b in range(batch):
            n = -(-int(L[b]) // bs)
            t[b, :n] = perm[used:used + n]
            used += n
            sm[b] = t[b, (L[b] - 1) // bs] * bs + (L[b] - 1) % bs
        lens[:bucket].copy_(torch.from_numpy(L))
        slots[:bucket].copy_(torch.from_numpy(sm))
        table[:bucket].copy_(torch.from_numpy(t))

        def eager():
            pa.pa_decode_store(out[:batch], q[:batch], kn[:batch], vn[:batch], kc, vc,
                               slots[:batch], table[:batch], lens[:batch], max_len, scale, ws)

        def graph():
            graphs.launch(batch)

        row = {"batch": batch, "bucket": bucket}
        for name, fn in (("eager", eager), ("graph", graph)):
            with _no_gc():
                for _ in range(warmup):
                    fn()
                torch.cuda.synchronize()
                # Dependent steps: the host waits for each step before the next, as
                # a serving loop must (the next step's tokens come from this one).
                t0 = time.perf_counter()
                for _ in range(steps):
                    fn()
                    torch.cuda.synchronize()
                row[f"{name}_dependent_us"] = round((time.perf_counter() - t0) / steps * 1e6, 2)
                # Pipelined steps: enqueued back to back, one wait at the end.
                t0 = time.perf_counter()
                for _ in range(steps):
                    fn()
                torch.cuda.synchronize()
                row[f"{name}_pipelined_us"] = round((time.perf_counter() - t0) / steps * 1e6, 2)
        row["dependent_speedup"] = round(row["eager_dependent_us"] / row["graph_dependent_us"], 3)
        row["pipelined_speedup"] = round(row["eager_pipelined_us"] / row["graph_pipelined_us"], 3)
        res.append(row)
    graphs.close()
    del kc, vc
    torch.cuda.empty_cache()
    return {"shape": "16 q / 8 kv heads, head_dim 128, block_size 256, context U[100,2048], "
                     "buckets 1..512 (powers of two), captured max_context_len 2048",
            "steps": steps, "per_batch": res}


def sampler_bench(warmup, steps, B=256, V=151936):
    """Gumbel-max sampling of one token per row from fp32 probabilities:
    256 rows of a Qwen3-sized vocabulary (151936), softmax of N(0,1) logits.
    Algorithmic bytes: every probability read once and one int32 token written
    per row. The oracle (numpy Philox + fp32 keys) is timed on 8 rows."""
    import numpy as np
    import torch
    import oracle.sampler as osm
    import paged_kv_cache_slot_amd as pa
    g = torch.Generator(device="cuda").manual_seed(404)
    probs = torch.softmax(torch.randn(B, V, generator=g, device="cuda"), dim=1).contiguous()
    tok = torch.empty(B, dtype=torch.int32, device="cuda")
    ws = torch.empty(pa.pa_sample_workspace_bytes(B, V), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    with _no_gc():
        for i in range(warmup):
            pa.pa_sample_gumbel(tok, probs, 1, i, ws)
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(evs):
            a.record(stream)
            pa.pa_sample_gumbel(tok, probs, 1, warmup + i, ws)
            b.record(stream)
        torch.cuda.synchronize()
    us = float(np.mean([a.elapsed_time(b) for a, b in evs])) * 1e3
    nbytes = B * V * 4 + B * 4
    sample_rows = 8
    pc = probs[:sample_rows].cpu().numpy()
    t0 = time.perf_counter()
    osm.sample(pc, 1, 0, rows=np.arange(sample_rows))
    dt = time.perf_counter() - t0
    return {"workload": f"gumbel-max sampling, {B} rows x vocab {V}, fp32 probabilities",
            "us": round(us, 2), "GBps": round(nbytes / (us * 1e-6) / 1e9, 2),
            "frac_hbm": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "algorithmic_bytes": nbytes,
            "Gelem_per_s": round(B * V / (us * 1e-6) / 1e9, 2),
            "oracle": {"Gelem_per_s": round(sample_rows * V / dt / 1e9, 5), "rows": sample_rows,
                       "cores": 1}}


def cpu_baseline(case):
    """The oracle (plain fp64 C++) on the same decode step, on the host cores:
    the KV store of the new tokens, then attention for every row."""
    import numpy as np
    import torch
    import oracle
    hw = oracle.hardware_threads()
    affinity = len(os.sched_getaffinity(0))
    nthreads = min(hw, affinity, 16)
    u16 = lambda t: t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    kc, vc = u16(case["k_cache"]), u16(case["v_cache"])
    kn, vn = u16(case["k_new"]), u16(case["v_new"])
    slots = case["slot_mapping"].cpu().numpy()
    bt, cl = case["block_table"].cpu().numpy(), case["context_lens"].cpu().numpy()
    q = u16(case["q"])
    # The whole step, repeated until about 10 s of host time have passed (the
    # store rewrites the same rows each time).
    reps = 0
    t0 = time.perf_counter()
    while reps < 1 or (time.perf_counter() - t0 < ORACLE_SECONDS and reps < 256):
        oracle.store_kvcache(kn, vn, kc, vc, slots, case["block_size"], inplace=True)
        oracle.decode(q, kc, vc, bt, cl, case["scale"], nthreads=nthreads)
        reps += 1
    dt = time.perf_counter() - t0
    nbytes = decode_bytes(case) + store_bytes(case)
    return {"value": round(nbytes * reps / dt / 1e9, 4), "unit": "GB/s", "cores": nthreads,
            "kind": "oracle", "seconds": round(dt, 3), "steps": reps,
            "host": {"nproc": os.cpu_count(), "hardware_concurrency": hw,
                     "affinity_cpus": affinity,
                     "threads_used": f"min(hardware_concurrency, affinity, 16) = {nthreads}"},
            "sample": f"the whole step, {reps} times back to back: store of {case['batch']} new "
                      f"tokens + fp64 attention for all {case['batch']} rows x "
                      f"{case['num_q_heads']} heads (qwen3_0.6b_decode, "
                      f"{int(np.asarray(case['lens']).sum())} context tokens)"}


def cpu_prefill_baseline(case, sequences=8):
    """The oracle (plain fp64 C++) on the first `sequences` sequences of the
    prefill workload (store of their new tokens, then causal attention over
    prefix + new tokens), on the host cores: TFLOP/s of algorithmic flops."""
    import numpy as np
    import torch
    import oracle
    nthreads = min(oracle.hardware_threads(), len(os.sched_getaffinity(0)), 16)
    u16 = lambda t: t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    cu = case["cu_seqlens_q"].cpu().numpy()
    n = min(sequences, len(cu) - 1)
    rows = int(cu[n])
    kc, vc = u16(case["k_cache"]), u16(case["v_cache"])
    kn, vn = u16(case["k_new"])[:rows], u16(case["v_new"])[:rows]
    slots = case["slot_mapping"].cpu().numpy()[:rows]
    q = u16(case["q"])[:rows]
    cl = case["context_lens"].cpu().numpy()[:n]
    bt = case["block_table"].cpu().numpy()[:n]
    N = np.diff(cu[:n + 1]).astype(np.int64)
    P = cl.astype(np.int64) - N
    flops = 4 * case["num_q_heads"] * case["head_dim"] * int((N * P + N * (N + 1) // 2).sum())
    t0 = time.perf_counter()
    oracle.store_kvcache(kn, vn, kc, vc, slots, case["block_size"], inplace=True)
    oracle.prefill(q, kc, vc, cu[:n + 1], cl, bt, case["scale"], nthreads=nthreads)
    dt = time.perf_counter() - t0
    return {"TFLOPs": round(flops / dt / 1e12, 5), "cores": nthreads, "kind": "oracle",
            "seconds": round(dt, 3), "algorithmic_flops": flops,
            "sample": f"sequences 0..{n - 1} of qwen3_8b_prefill_prefix ({rows} new tokens "
                      f"after {int(P.sum())} cached), store + fp64 causal attention, once"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-leg", choices=["prefill", "sampler", "decode", "decode-flushed",
                                              "graphs", "mfma-ceiling", "prefill-lengths"],
                    default=None,
                    help="only run this leg and print its own result (for counter runs and "
                         "kernel traces under rocprofv3); the benchmark line is not printed")
    ap.add_argument("--workload", default="qwen3_0.6b_decode",
                    help="decode workload of --profile-leg decode / decode-flushed")
    ap.add_argument("--batch", type=int, default=256,
                    help="batch of --profile-leg graphs (eager and graph steps at that batch)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (a known "
                         "byte count for scaling the HBM counters of rocprofv3)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the paged-attention path is built and timed on a "
              f"single MI355X; --gpus {args.gpus} is not supported.", file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_kv_cache_slot_amd as pa
    import workloads
    assert torch.cuda.is_available(), "bench.py needs the GPU"
    pa.library()
    if args.calibrate_copy:
        src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] copied 1 GiB 5 times")
        return
    if args.profile_leg:
        fn = {"prefill": lambda: prefill_bench(max(args.warmup, SECONDARY_WARMUP), args.steps,
                                               warm_s=SECONDARY_WARM_S),
              "sampler": lambda: sampler_bench(args.warmup, args.steps),
              "decode": lambda: decode_bench(args.workload, max(args.warmup, SECONDARY_WARMUP),
                                             args.steps, warm_s=SECONDARY_WARM_S),
              "decode-flushed": lambda: decode_bench(args.workload,
                                                     max(args.warmup, SECONDARY_WARMUP),
                                                     args.steps, warm_s=SECONDARY_WARM_S,
                                                     flushed_only=True),
              "graphs": lambda: graph_bench(batches=(args.batch,)),
              "mfma-ceiling": lambda: mfma_ceiling_bench(max(args.warmup, SECONDARY_WARMUP),
                                                         args.steps, warm_s=SECONDARY_WARM_S),
              "prefill-lengths": lambda: prefill_lengths_bench(
                  max(args.warmup, SECONDARY_WARMUP), args.steps, warm_s=SECONDARY_WARM_S),
              }[args.profile_leg]
        res = fn()
        print(json.dumps({k: v for k, v in res.items() if k != "case"},
                         default=lambda x: x.tolist() if hasattr(x, "tolist") else str(x)),
              flush=True)
        return
    log(f"device: {torch.cuda.get_device_name(0)} "
        f"({torch.cuda.get_device_properties(0).gcnArchName})")

    log("[bench] qwen3_0.6b_decode: decode step (store fused into the decode call)")
    main_res = decode_bench("qwen3_0.6b_decode", args.warmup, args.steps)
    case = main_res["case"]
    digest = source_digest("decode.hip", "pa_internal.h")
    traffic = measured_traffic("pa_decode_store", digest)
    roofline = {"kernel": "pa_decode_store (decode_kernel<2, 4> + decode_merge_kernel<2>, "
                          "the store fused into them)",
                "bound": "hbm", "achieved": round(main_res["decode_gbs"], 2),
                "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(main_res["decode_gbs"] / HBM_PEAK_GBS, 4),
                "traffic": traffic, "algorithmic_bytes": main_res["decode_bytes"],
                "avg_launch_us": round(main_res["decode_ms"] * 1e3, 2),
                "median_launch_us": round(main_res["decode_ms_median"] * 1e3, 2),
                "mall_flushed_median_us": round(main_res["flushed_ms"] * 1e3, 2),
                "mall_flushed_frac": round(main_res["flushed_gbs"] / HBM_PEAK_GBS, 4),
                "protocol": "frac: mean of back-to-back calls (HIP events); mall_flushed_*: "
                            "median with a 512 MiB write before every call (the survey's "
                            "protocol)",
                "source_digest": digest}

    secondary = []
    if not args.no_secondary:
        for name in ("qwen3_8b_decode", "bs16_stress_decode"):
            log(f"[bench] {name}: decode step (store fused into the decode call)")
            r = decode_bench(name, max(args.warmup, SECONDARY_WARMUP), args.steps,
                             warm_s=SECONDARY_WARM_S)
            secondary.append({
                "workload": name, "ms_per_step": round(r["ms_per_step"], 4),
                "step_GBps": round(r["gbs"], 2),
                "decode_us": round(r["decode_ms"] * 1e3, 2),
                "decode_GBps": round(r["decode_gbs"], 2),
                "decode_frac_hbm": round(r["decode_gbs"] / HBM_PEAK_GBS, 4),
                "decode_median_us": round(r["decode_ms_median"] * 1e3, 2),
                "mall_flushed_median_us": round(r["flushed_ms"] * 1e3, 2),
                "mall_flushed_frac": round(r["flushed_gbs"] / HBM_PEAK_GBS, 4)})
            del r
            torch.cuda.empty_cache()
        log("[bench] qwen3_8b_prefill_prefix: store + prefill")
        r = prefill_bench(max(args.warmup, SECONDARY_WARMUP), args.steps,
                          warm_s=SECONDARY_WARM_S)
        secondary.append({
            "workload": "qwen3_8b_prefill_prefix",
            "ms_per_step": round(r["ms_per_step"], 4), "prefill_us": round(r["prefill_ms"] * 1e3, 2),
            "prefill_TFLOPs": round(r["tflops"], 2),
            "prefill_frac_mfma": round(r["tflops"] / MFMA_BF16_PEAK_TFLOPS, 4),
            "algorithmic_flops": r["flops"], "total_q": r["total_q"]})
        if not args.no_cpu_baseline:
            log("[bench] prefill oracle on a sample of the sequences")
            po = cpu_prefill_baseline(r["case"])
            po["gpu_over_oracle"] = round(r["tflops"] / po["TFLOPs"], 1)
            secondary[-1]["oracle"] = po
        del r
        torch.cuda.empty_cache()

    graphs = sampler = ceiling = None
    if not args.no_secondary:
        log("[bench] gumbel-max sampler")
        sampler = sampler_bench(args.warmup, args.steps)
        log("[bench] decode-step graphs vs eager")
        graphs = graph_bench()
        log("[bench] library bf16 GEMM (MFMA ceiling under real data)")
        ceiling = mfma_ceiling_bench(max(args.warmup, SECONDARY_WARMUP), args.steps,
                                     warm_s=SECONDARY_WARM_S)
        pf = next(x for x in secondary if x["workload"] == "qwen3_8b_prefill_prefix")
        ceiling["prefill_over_gemm_random"] = round(pf["prefill_TFLOPs"]
                                                    / ceiling["random_TFLOPs"], 4)

    log("[bench] block manager (host)")
    bmr = block_manager_bench()
    bmr["native_step_frac_of_gpu_step"] = round(bmr["native"]["decode_step_us"] * 1e-3
                                                / main_res["ms_per_step"], 4)

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        cpu = cpu_baseline(case)
        cpu["gpu_over_oracle"] = round(main_res["gbs"] / cpu["value"], 1)

    line = {
        "metric": METRIC, "value": round(main_res["gbs"], 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(main_res["ms_per_step"], 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "qwen3_0.6b_decode: pa_decode_store (the new tokens' K/V store "
                               "fused into the decode), 256 sequences, "
                               "context lengths U[100,2048], 16 q / 8 kv heads, head_dim 128, "
                               "block_size 256, permuted physical blocks",
                   "batch": case["batch"], "max_context_len": case["max_context_len"],
                   "context_tokens": int(sum(case["lens"])), "block_size": case["block_size"],
                   "num_q_heads": case["num_q_heads"], "num_kv_heads": case["num_kv_heads"],
                   "head_dim": case["head_dim"], "seed": case["seed"],
                   "step_bytes": main_res["step_bytes"]},
        "roofline": roofline, "cpu_baseline": cpu, "secondary": secondary,
        "block_manager": bmr, "decode_graphs": graphs, "sampler": sampler,
        "mfma_ceiling": ceiling,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

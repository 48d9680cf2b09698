"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI,
run the oracle on host copies of the same inputs, compare."""
import json
import os
import sys

import numpy as np
import torch

import oracle
import paged_kv_cache_slot_amd as pa
import workloads

DEV = "cuda"
# Attention outputs (bf16 in, bf16 out) must match the fp64 oracle within
# 1e-2 absolute and 1e-2 relative, element by element.
ATOL = 1e-2
RTOL = 1e-2
ORACLE_THREADS = 16
# Every comparison appends its error margins (test, case, element count, max
# abs error, max abs error over max |ref|, max relative error over |ref| >=
# 1e-2) to this JSON-lines file, so a GPU run leaves a record of how close
# each case came to the tolerance.
MARGINS_FILE = os.environ.get(
    "PA_MARGINS_FILE",
    os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "gpurun_out",
                 "parity_margins.jsonl"))


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()


def require_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    name = torch.cuda.get_device_properties(0).gcnArchName
    assert name.startswith("gfx950"), f"built for gfx950, found {name}"
    pa.library()  # fails loudly if libpa.so is missing


def host_copy(case):
    """CPU copies of every tensor input (taken before any GPU call mutates them)."""
    return {k: (v.detach().cpu().clone() if torch.is_tensor(v) else v) for k, v in case.items()}


def to_device(case):
    return {k: (v.to(DEV) if torch.is_tensor(v) else v) for k, v in case.items()}


def gpu_store(case):
    pa.pa_store_kvcache(case["k_new"], case["v_new"], case["k_cache"], case["v_cache"],
                        case["slot_mapping"])


def gpu_decode(case, max_context_len=None):
    B, hq, d = case["q"].shape
    mcl = case["max_context_len"] if max_context_len is None else max_context_len
    out = torch.full((B, hq, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    nbytes = pa.pa_decode_workspace_bytes(B, hq, d, mcl, case["block_size"])
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=DEV)
    pa.pa_decode(out, case["q"], case["k_cache"], case["v_cache"], case["block_table"],
                 case["context_lens"], mcl, case["scale"], ws)
    return out


def gpu_prefill(case):
    T, hq, d = case["q"].shape
    out = torch.full((T, hq, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    pa.pa_prefill_varlen(out, case["q"], case["k_cache"], case["v_cache"], case["cu_seqlens_q"],
                         case["context_lens"], case["block_table"], case["max_seqlen_q"],
                         case["scale"])
    return out


def oracle_after_store(h):
    """Oracle pools after the store, from host copies of the pre-store pools."""
    return oracle.store_kvcache(h["k_new"], h["v_new"], h["k_cache"], h["v_cache"],
                                h["slot_mapping"], h["block_size"])


def compare(gpu_out, ref, what, rows=None):
    """Element-wise |g - r| <= ATOL + RTOL |r| and max|g - r| / max|r| <= 1e-2."""
    g = gpu_out.float().cpu().double().numpy()
    r = ref
    if rows is not None:
        g, r = g[rows], r[rows]
    assert np.isfinite(g).all(), f"{what}: non-finite GPU output"
    err = np.abs(g - r)
    bound = ATOL + RTOL * np.abs(r)
    bad = err > bound
    max_abs = float(err.max()) if err.size else 0.0
    scale = float(np.abs(r).max()) if r.size else 0.0
    stats = dict(max_abs=max_abs, norm_rel=max_abs / scale if scale else 0.0,
                 max_rel=float((err / np.maximum(np.abs(r), 1e-2)).max()) if err.size else 0.0)
    _record_margins(what, g.size, stats, bool(bad.any()))
    if bad.any():
        idx = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} elements out of tolerance; worst at "
                             f"{idx}: gpu {g[idx]:.6f} oracle {r[idx]:.6f} ({stats})")
    assert stats["norm_rel"] <= 1e-2 or scale == 0.0, f"{what}: {stats}"
    say(f"  {what}: max|err| {max_abs:.2e}, max|err|/max|ref| {stats['norm_rel']:.2e}")
    return stats


def _record_margins(what, n, stats, failed):
    try:
        os.makedirs(os.path.dirname(MARGINS_FILE), exist_ok=True)
        rec = dict(test=os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0], case=what,
                   elements=int(n), failed=failed,
                   **{k: float(f"{v:.4g}") for k, v in stats.items()})
        with open(MARGINS_FILE, "a") as f:
            f.write(json.dumps(rec) + "\n")
    except OSError:
        pass  # the record is a convenience; the assertions decide


def make_case(name, **over):
    """Full-size (or overridden) case generated on the GPU, plus host copies."""
    say(f"[case] workload {name} seed {workloads.seed_of(name)} "
        f"overrides {over}")
    case = workloads.workload_case(name, device=DEV, **over)
    torch.cuda.synchronize()
    return case, host_copy(case)

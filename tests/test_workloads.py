"""The seeded input generator: determinism and the structure of each workload."""
import numpy as np
import pytest

import workloads


def test_same_seed_same_bytes():
    a = workloads.workload_case("tiny_decode")
    b = workloads.workload_case("tiny_decode")
    for key in ("k_cache", "v_cache", "q", "k_new", "v_new", "block_table", "slot_mapping"):
        assert workloads.digest(a[key]) == workloads.digest(b[key]), key
    c = workloads.workload_case("tiny_decode", seed=99)
    assert workloads.digest(a["q"]) != workloads.digest(c["q"])


@pytest.mark.parametrize("name", ["tiny_decode", "qwen3_8b_decode", "bs16_stress_decode"])
def test_decode_metadata(name):
    cfg = workloads.WORKLOADS[name]
    # Small stand-ins keep the pool tiny on the CPU; the metadata rules are the same.
    over = {} if name == "tiny_decode" else dict(batch=40, pad=4)
    case = workloads.workload_case(name, **over)
    bs = case["block_size"]
    lens = case["context_lens"].numpy()
    table = case["block_table"].numpy()
    slots = case["slot_mapping"].numpy()
    lo, hi = cfg["len_range"]
    real = lens > 0
    assert (lens[real] >= lo).all() and (lens[real] <= hi).all()
    assert int((~real).sum()) == (over.get("pad", cfg["pad"]))
    used = []
    for b in range(case["batch"]):
        n = -(-int(lens[b]) // bs)
        assert (table[b, :n] >= 0).all() and (table[b, n:] == -1).all()
        used += list(table[b, :n])
        if lens[b] == 0:
            assert slots[b] == -1
        else:
            pos = int(lens[b]) - 1
            assert slots[b] == table[b, pos // bs] * bs + pos % bs
    assert len(set(used)) == len(used), "a physical block is owned twice"
    assert max(used) < case["num_blocks"]


def test_prefill_prefix_sharing():
    case = workloads.workload_case("qwen3_8b_prefill_prefix", batch=24)
    bs = case["block_size"]
    table = case["block_table"].numpy()
    k = case["prefix_blocks"]
    c = case["prefix_chain"]
    N = case["new_lens"]
    cu = case["cu_seqlens_q"].numpy()
    assert (np.diff(cu) == N).all()
    assert (case["context_lens"].numpy() == k * bs + N).all()
    # Sequences on the same chain share their first min(k) physical blocks.
    for a in range(len(k)):
        for b in range(len(k)):
            m = min(k[a], k[b])
            if c[a] == c[b] and m > 0:
                assert (table[a, :m] == table[b, :m]).all()
    # New tokens go to fresh blocks, never to a shared prefix block.
    shared = set(table[b, j] for b in range(len(k)) for j in range(k[b]))
    slots = case["slot_mapping"].numpy()
    assert not (set(slots // bs) & shared)
    assert len(set(slots)) == len(slots)

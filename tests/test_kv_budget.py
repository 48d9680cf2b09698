"""KV-cache budget: the oracle against hand-worked cases, the library against
the oracle. Host only."""
import json
import os
import random

import pytest

from oracle.kv_budget import num_blocks as oracle_blocks
from paged_kv_cache_slot_amd.block_manager import kv_cache_num_blocks

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "kv_budget.json")


def _cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("impl", ["oracle", "native"])
def test_hand_worked_cases(impl):
    f = oracle_blocks if impl == "oracle" else kv_cache_num_blocks
    for c in _cases():
        got = f(c["total"], c["used"], c["peak"], c["current"], c["layers"], c["block_size"],
                c["kv_heads"], c["head_dim"])
        assert got == c["blocks"], c["what"]


def test_native_matches_oracle_random():
    rng = random.Random(12)
    for _ in range(2000):
        total = rng.randrange(1 << 30, 300 << 30)
        used = rng.randrange(0, total // 4)
        peak = rng.randrange(0, total // 3)
        current = rng.randrange(0, peak + 1)
        args = (total, used, peak, current, rng.randrange(1, 100), rng.choice([16, 32, 256]),
                rng.choice([1, 2, 4, 8]), 128, rng.choice([1, 2, 4]), rng.choice([0.5, 0.9, 1.0]))
        assert kv_cache_num_blocks(*args) == oracle_blocks(*args), args


def test_more_warmup_memory_means_fewer_blocks():
    base = dict(total_bytes=100 << 30, used_bytes=10 << 30, num_layers=28, block_size=256,
                num_kv_heads=8, head_dim=128)
    a = kv_cache_num_blocks(peak_bytes=8 << 30, current_bytes=2 << 30, **base)
    b = kv_cache_num_blocks(peak_bytes=12 << 30, current_bytes=2 << 30, **base)
    c = kv_cache_num_blocks(peak_bytes=12 << 30, current_bytes=6 << 30, **base)
    assert a > b and c == a                        # -peak + current: only the temporaries count


def test_bad_arguments():
    with pytest.raises(ValueError):
        kv_cache_num_blocks(1 << 30, 0, 0, 0, 0, 16, 8, 128)
    with pytest.raises(ValueError):
        kv_cache_num_blocks(1 << 30, 0, 0, 0, 1, 16, 8, 128, utilization=0.0)
    with pytest.raises(ValueError):
        kv_cache_num_blocks(1 << 30, 0, 0, 0, 1, 16, 8, 128, utilization=1.5)

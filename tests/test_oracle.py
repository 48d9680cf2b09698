"""The CPU oracle against its pins, and the pins against planted mistakes."""
import os
import re
import subprocess
import sys

import pytest

import oracle
from oracle.build import SRC, build_oracle
from tests import oracle_pins

PIN_IDS = [p.__name__ for p in oracle_pins.ALL_PINS]


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=PIN_IDS)
def test_oracle_pin(pin, oracle_lib):
    pin(oracle_lib)


# Plausible mistakes, planted in a copy of the oracle's source. Each must make
# at least one pin fail. (old text, new text, what the mistake is)
MUTATIONS = {
    "gqa_modulo": (r"int32_t g = h / group;", "int32_t g = h % num_kv_heads;",
                   "query head h read kv head h mod Hkv"),
    "causal_off_by_one": (r"int32_t visible = P \+ i \+ 1;", "int32_t visible = P + i;",
                          "new row i misses its own key"),
    "scale_dropped": (r"s\[j\] = scale \* acc;", "s[j] = acc;", "softmax scale ignored"),
    "slot_not_scaled": (r"return static_cast<int64_t>\(physical\) \* block_size \+ offset;",
                        "return static_cast<int64_t>(physical) + offset;",
                        "physical block id not multiplied by block_size"),
    "block_offset_swapped": (r"int32_t logical_block = j / block_size;\n  int32_t offset = j % block_size;",
                             "int32_t logical_block = j % block_size;\n  int32_t offset = j / block_size;",
                             "logical block and offset swapped"),
    "values_from_k": (r"gather\(v_cache, table_row, L,", "gather(k_cache, table_row, L,",
                      "decode reads V from the K pool"),
    "decode_drops_new_token": (r"attend\(qv, K, V, L, D, scale,", "attend(qv, K, V, L - 1, D, scale,",
                               "decode ignores the newest token"),
    "partition_skips_first": (r"for \(int32_t j = 0; j < L; \+\+j\) \{\n    s\[j\] = std::exp",
                              "for (int32_t j = 1; j < L; ++j) {\n    s[j] = std::exp",
                              "softmax denominator misses the first key"),
    "prefill_wrong_query_row": (r"q \+ \(static_cast<int64_t>\(t\) \* num_q_heads \+ h\) \* D",
                                "q + (static_cast<int64_t>(i) * num_q_heads + h) * D",
                                "prefill reads the query row of the sequence-local index"),
    "head_dim_transposed": (r"const uint16_t\* src = cache \+ \(slot \* Hkv \+ g\) \* D;",
                            "const uint16_t* src = cache + slot * Hkv * D + g;",
                            "kv head and head_dim offsets exchanged"),
    "store_ignores_stride": (r"k\[i \* kv_token_stride \+ e\]", "k[i * row + e]",
                             "store assumes packed k rows"),
    "store_skips_slot_zero": (r"if \(s == -1\) continue;", "if (s <= 0) continue;",
                              "store treats slot 0 as padding"),
    "prefix_ignored": (r"int32_t P = context_lens\[b\] - N;", "int32_t P = 0;",
                       "prefill ignores the cached prefix"),
}


_RUN_PINS = """
import sys
sys.path.insert(0, {root!r})
import oracle
from tests import oracle_pins
lib = oracle.load({lib!r})
for pin in oracle_pins.ALL_PINS:
    try:
        pin(lib)
    except (AssertionError, ValueError) as e:
        print("CAUGHT", pin.__name__, str(e).splitlines()[0] if str(e) else "")
"""


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    pattern, repl, _ = MUTATIONS[name]
    with open(SRC) as f:
        src = f.read()
    mutated, n = re.subn(pattern, repl, src)
    assert n >= 1, f"mutation {name} did not apply"
    path = tmp_path / "mutant.cpp"
    path.write_text(mutated)
    lib = build_oracle(str(path), str(tmp_path / "libmutant.so"))
    # The mutant runs in a child process: a planted mistake may also crash it,
    # which counts as caught (the mistake cannot pass unnoticed).
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    proc = subprocess.run([sys.executable, "-c", _RUN_PINS.format(root=root, lib=lib)],
                          capture_output=True, text=True, timeout=300)
    caught = [l for l in proc.stdout.splitlines() if l.startswith("CAUGHT")]
    assert caught or proc.returncode != 0, \
        f"no pin caught the planted mistake '{name}'\n{proc.stdout}\n{proc.stderr}"

"""KV-cache budget oracle: how many blocks fit after a warm-up run.

TEST INFRASTRUCTURE ONLY (tests, the smoke check and the benchmark's CPU
leg). It shares no code with the product library.

[Report] "nano-vllm 深度分析报告", section "创新之处" (dynamic KV-cache sizing)
and table "可复用的模式与技巧", row "warmup → peak → 分配": after one warm-up
step the budget is total * 0.9 - used - peak + current bytes. Reading: one
block holds K and V of block_size tokens in every layer, so it costs
2 * layers * block_size * kv_heads * head_dim * dtype_bytes bytes, and the
count is the floor of budget / block bytes (0 when the budget is not
positive). Computed with exact rational arithmetic.
"""
from fractions import Fraction


def num_blocks(total, used, peak, current, num_layers, block_size, num_kv_heads, head_dim,
               dtype_bytes=2, utilization=0.9):
    budget = Fraction(total) * Fraction(utilization) - used - peak + current
    block = 2 * num_layers * block_size * num_kv_heads * head_dim * dtype_bytes
    if budget <= 0:
        return 0
    return int(budget // block)

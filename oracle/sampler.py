"""Sampler oracle: Gumbel-max (exponential race) sampling from per-row
probabilities, with the random numbers from the Philox counter-based
generator.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this module. It shares no code with the
product library's sampler kernel.

What it follows:
  [Report] "nano-vllm 深度分析报告" (nightvoyager), section "创新之处" (the
  Gumbel-Max item) and table "可复用的模式与技巧", row "Gumbel-Max 采样": a
  token is drawn as the index of the largest p_i / E_i with E_i ~ Exp(1)
  independent, which replaces a multinomial draw. (With E_i ~ Exp(1), the
  smallest E_i / p_i is the winner of an exponential race with rates p_i, so
  index i wins with probability p_i / sum(p).)

Random numbers (the pages do not fix a generator): Philox4x32 with 10 rounds,
as defined in J. K. Salmon, M. A. Moraes, R. O. Dror and D. E. Shaw, "Parallel
Random Numbers: As Easy as 1, 2, 3", SC'11: a 4 x 32-bit counter and a
2 x 32-bit key; each round multiplies counter words 0 and 2 by two fixed
constants, takes the high and low halves of the products, xors the high halves
with the other two counter words and the key, and permutes; the key is bumped
by two Weyl constants between rounds.

Readings this library takes (the same for the kernel; stated in the C header):
  * element i of row b uses output word i mod 4 of Philox4x32-10 at counter
    (i div 4, b, offset mod 2^32, offset div 2^32) with key (seed mod 2^32,
    seed div 2^32);
  * a 32-bit output x becomes u = ((x >> 9) + 1/2) * 2^-23, exactly an fp32
    in (0, 1);
  * E = -log2(u) (a positive multiple of -ln u, so the same argmax), and the
    key p / E, both rounded to fp32 -- the precision the decision is taken in;
  * ties go to the smallest index; a row of zeros yields index 0.
"""
import numpy as np

M32 = (0xD2511F53, 0xCD9E8D57)      # Philox4x32 round multipliers
W32 = (0x9E3779B9, 0xBB67AE85)      # Philox4x32 key increments (Weyl)
M64 = (0xD2E7470EE14C6C93, 0xCA5A826395121157)
W64 = (0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B)


def philox4x32(counter, key, rounds=10):
    """Philox4x32-R on arrays: counter [..., 4] and key [..., 2] of uint32
    (broadcast against each other). Returns [..., 4] uint32."""
    c = [np.asarray(counter, dtype=np.uint64)[..., j] for j in range(4)]
    k = [np.asarray(key, dtype=np.uint64)[..., j] for j in range(2)]
    lo32 = np.uint64(0xFFFFFFFF)
    for r in range(rounds):
        if r > 0:
            k = [(k[0] + np.uint64(W32[0])) & lo32, (k[1] + np.uint64(W32[1])) & lo32]
        p0 = np.uint64(M32[0]) * c[0]          # exact: both factors < 2^32
        p1 = np.uint64(M32[1]) * c[2]
        hi0, lo0 = p0 >> np.uint64(32), p0 & lo32
        hi1, lo1 = p1 >> np.uint64(32), p1 & lo32
        c = [hi1 ^ c[1] ^ k[0], lo1, hi0 ^ c[3] ^ k[1], lo0]
    return np.stack(c, axis=-1).astype(np.uint32)


def philox4x64(counter, key, rounds=10):
    """Philox4x64-R on Python ints (one block): the same round structure with
    64-bit words, multipliers and Weyl constants. Used to pin the structure
    against numpy's Philox bit generator."""
    c = [int(x) for x in counter]
    k = [int(x) for x in key]
    mask = (1 << 64) - 1
    for r in range(rounds):
        if r > 0:
            k = [(k[0] + W64[0]) & mask, (k[1] + W64[1]) & mask]
        p0 = M64[0] * c[0]
        p1 = M64[1] * c[2]
        c = [(p1 >> 64) ^ c[1] ^ k[0], p1 & mask, (p0 >> 64) ^ c[3] ^ k[1], p0 & mask]
    return c


def uniforms(x):
    """uint32 -> fp32 in (0, 1): ((x >> 9) + 0.5) * 2^-23 (exact)."""
    x = np.asarray(x, dtype=np.uint32)
    return ((x >> np.uint32(9)).astype(np.float32) + np.float32(0.5)) * np.float32(2.0 ** -23)


def row_bits(batch_rows, vocab, seed, offset):
    """Philox output word for every (row, element): [len(rows), vocab] uint32."""
    rows = np.asarray(batch_rows, dtype=np.uint64)
    n4 = (vocab + 3) // 4
    ctr = np.zeros((len(rows), n4, 4), dtype=np.uint64)
    ctr[..., 0] = np.arange(n4, dtype=np.uint64)[None, :]
    ctr[..., 1] = rows[:, None]
    ctr[..., 2] = np.uint64(offset & 0xFFFFFFFF)
    ctr[..., 3] = np.uint64(offset >> 32)
    key = np.array([seed & 0xFFFFFFFF, seed >> 32], dtype=np.uint64)
    out = philox4x32(ctr, key)
    return out.reshape(len(rows), n4 * 4)[:, :vocab]


def sample(probs, seed, offset, rows=None):
    """Token index per row (int32) and the fp64 keys of every element.

    probs: [B, V] float32 (non-negative). rows: the row indices of `probs`
    in the batch (for a sample of rows), default 0..B-1. The decision is
    argmax of the fp32 key p / (-log2 u); the fp64 keys (same u, exact log)
    let a caller judge near-ties."""
    p = np.asarray(probs, dtype=np.float32)
    B, V = p.shape
    rows = np.arange(B) if rows is None else np.asarray(rows)
    u = uniforms(row_bits(rows, V, seed, offset))
    # E = -log2(u) taken in fp64 and rounded once to fp32: exactly rounded
    # (numpy's own fp32 log2 carries no such guarantee).
    e32 = (-np.log2(u.astype(np.float64))).astype(np.float32)
    key32 = p / e32                            # float32, correctly rounded division
    tok = np.argmax(key32, axis=1).astype(np.int32)
    key64 = p.astype(np.float64) / -np.log2(u.astype(np.float64))
    return tok, key32, key64

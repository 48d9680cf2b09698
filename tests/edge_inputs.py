"""Host-side shaping of test inputs for sharp, high-dynamic-range attention.

The GPU edge-case tests start from the seeded workloads and then move keys and
queries so that scores climb along the context (the running maximum of an
online softmax must be raised again and again), or so that one late key
dominates. Everything here edits bf16 input tensors on the host (values are
rounded back to bf16, round to nearest even) and reports score statistics in
fp64 so a test can assert that its inputs really cross the kernels' rescale
thresholds. Nothing here computes attention outputs: those come from the
oracle only.
"""
import math

import numpy as np
import torch

LOG2E = 1.0 / math.log(2.0)


def _bf16(x):
    return x.to(torch.float32).to(torch.bfloat16)


def _slots(table_row, positions, block_size):
    pos = np.asarray(positions, dtype=np.int64)
    return table_row[pos // block_size].astype(np.int64) * block_size + pos % block_size


def _pool_rows(pool):
    """[num_blocks, bs, Hkv, D] -> [num_slots, Hkv, D] view."""
    return pool.view(-1, pool.shape[2], pool.shape[3])


def scale_queries(q, factor_per_row):
    """q[t] *= factor_per_row[t] (any 1-D sequence of floats), rounded to bf16."""
    f = torch.as_tensor(np.asarray(factor_per_row, dtype=np.float32)).view(-1, 1, 1)
    return _bf16(q.float() * f)


def decode_ramp(h, rise_log2, scale, rows=None):
    """Decode inputs whose scores for the first query head of every kv group
    rise linearly along the context by `rise_log2` (log2 units) from position 0
    to the new token: K at position j gets + c (j / (L-1)) q_hat, with q_hat the
    unit query of that head and c chosen so that scale * c * |q| * log2(e) =
    rise_log2. Edits h["k_cache"] (positions < L-1, through the block table)
    and h["k_new"] (position L-1) in place."""
    bs, hkv = h["block_size"], h["num_kv_heads"]
    G = h["num_q_heads"] // hkv
    kpool = _pool_rows(h["k_cache"])
    table = h["block_table"].numpy()
    lens = np.asarray(h["lens"])
    for b in range(len(lens)) if rows is None else rows:
        L = int(lens[b])
        if L < 2:
            continue
        slots = torch.from_numpy(_slots(table[b], np.arange(L - 1), bs))
        w = torch.arange(L, dtype=torch.float32) / (L - 1)
        for g in range(hkv):
            qv = h["q"][b, g * G].float()
            nq = float(qv.norm())
            if nq == 0.0:
                continue
            c = rise_log2 / (scale * nq * LOG2E)
            step = (c / nq) * qv  # c * q_hat
            kpool[slots, g] = _bf16(kpool[slots, g].float() + w[:L - 1, None] * step[None, :])
            h["k_new"][b, g] = _bf16(h["k_new"][b, g].float() + w[L - 1] * step)


def decode_dominant_key(h, pos_from_end, margin_log2, scale):
    """Key at position L-1-pos_from_end of every live row is set to
    c q_hat for the first query head of each kv group, with c such that its
    score is `margin_log2` above the largest other score of that head."""
    bs, hkv = h["block_size"], h["num_kv_heads"]
    G = h["num_q_heads"] // hkv
    kpool = _pool_rows(h["k_cache"])
    table = h["block_table"].numpy()
    lens = np.asarray(h["lens"])
    for b in range(len(lens)):
        L = int(lens[b])
        j = L - 1 - pos_from_end
        if j < 0:
            continue
        for g in range(hkv):
            qv = h["q"][b, g * G].double()
            s = decode_scores(h, b, g * G, scale)
            others = np.delete(s, j)
            top = float(others.max()) if others.size else 0.0
            target = top + margin_log2                       # log2 units
            c = target / (scale * LOG2E * float(qv.norm()))
            row = _bf16((c / float(qv.norm())) * qv.float())
            if j == L - 1:
                h["k_new"][b, g] = row
            else:
                kpool[int(_slots(table[b], [j], bs)[0]), g] = row


def decode_scores(h, b, head, scale):
    """fp64 scores (log2 units) of one decode row and query head over its
    context, the new token's key taken from k_new."""
    bs, hkv = h["block_size"], h["num_kv_heads"]
    g = head // (h["num_q_heads"] // hkv)
    L = int(np.asarray(h["lens"])[b])
    kpool = _pool_rows(h["k_cache"])
    slots = torch.from_numpy(_slots(h["block_table"][b].numpy(), np.arange(L - 1), bs))
    keys = torch.cat([kpool[slots, g].double(), h["k_new"][b, g].double()[None]], 0)
    return (keys @ h["q"][b, head].double()).numpy() * scale * LOG2E


def max_rise_over_first_chunk(s, chunk):
    """Largest (chunk maximum - first chunk maximum) over the later chunks."""
    n = len(s)
    first = s[:chunk].max()
    later = [s[c:c + chunk].max() for c in range(chunk, n, chunk)]
    return float(max(later) - first) if later else 0.0


def prefill_ramp(h, rise_log2, scale, q_push=8.0, seed=0):
    """Prefill inputs whose scores rise along the key positions: per
    (sequence, kv head) a random unit direction u; every query row of that kv
    group gets + q_push u, and the key at position j (of L) gets
    + c (j / (L-1)) u with scale * q_push * c * log2(e) = rise_log2. The new
    tokens' keys (k_new) and the cached prefix keys in the pool are both
    edited. Edits h in place; returns the directions [B, Hkv, D]."""
    rng = np.random.default_rng(seed)
    bs, hkv = h["block_size"], h["num_kv_heads"]
    G = h["num_q_heads"] // hkv
    kpool = _pool_rows(h["k_cache"])
    table = h["block_table"].numpy()
    cu = h["cu_seqlens_q"].numpy()
    L_all = h["context_lens"].numpy()
    B = len(L_all)
    dirs = np.zeros((B, hkv, h["head_dim"]))
    c = rise_log2 / (scale * q_push * LOG2E)
    for b in range(B):
        N = int(cu[b + 1] - cu[b])
        L = int(L_all[b])
        P = L - N
        if L < 2:
            continue
        for g in range(hkv):
            u = rng.standard_normal(h["head_dim"])
            u /= np.linalg.norm(u)
            dirs[b, g] = u
            ut = torch.from_numpy(u).float()
            w = torch.arange(L, dtype=torch.float32) / (L - 1)
            if P > 0:  # cached prefix keys sit only in the pool
                slots = torch.from_numpy(_slots(table[b], np.arange(P), bs))
                kpool[slots, g] = _bf16(kpool[slots, g].float() + c * w[:P, None] * ut[None])
            rows = slice(int(cu[b]), int(cu[b + 1]))
            h["k_new"][rows, g] = _bf16(h["k_new"][rows, g].float() +
                                        c * w[P:, None] * ut[None])
            qs = slice(g * G, (g + 1) * G)
            h["q"][rows, qs] = _bf16(h["q"][rows, qs].float() + q_push * ut[None, None])
    return dirs


def prefill_dominant_key(h, pos_from_end, margin_log2, scale, head_in_group=0):
    """For every sequence and kv head, the key at position L-1-pos_from_end
    (a new token, edited in k_new) is set to c q_hat, q_hat the unit query of
    the sequence's last row at head g*G + head_in_group, with c such that that
    row's score for it is `margin_log2` above the row's other scores."""
    hkv = h["num_kv_heads"]
    G = h["num_q_heads"] // hkv
    cu = h["cu_seqlens_q"].numpy()
    L_all = h["context_lens"].numpy()
    for b in range(len(L_all)):
        N = int(cu[b + 1] - cu[b])
        L = int(L_all[b])
        j = L - 1 - pos_from_end
        if N == 0 or j < L - N:
            continue
        t_last = int(cu[b + 1]) - 1
        for g in range(hkv):
            head = g * G + head_in_group
            qv = h["q"][t_last, head].double()
            s = prefill_scores(h, t_last, head, scale)
            others = np.delete(s, j)
            target = float(others.max()) + margin_log2
            cc = target / (scale * LOG2E * float(qv.norm()))
            h["k_new"][int(cu[b]) + (j - (L - N)), g] = _bf16((cc / float(qv.norm())) * qv.float())


def prefill_scores(h, t, head, scale):
    """fp64 scores (log2 units) of global query row t, query head `head`,
    over the keys it sees (positions 0 .. P + i): prefix keys from the pool,
    new keys from k_new."""
    bs, hkv = h["block_size"], h["num_kv_heads"]
    g = head // (h["num_q_heads"] // hkv)
    cu = h["cu_seqlens_q"].numpy()
    b = int(np.searchsorted(cu, t, side="right") - 1)
    N = int(cu[b + 1] - cu[b])
    L = int(h["context_lens"][b])
    P = L - N
    i = t - int(cu[b])
    kpool = _pool_rows(h["k_cache"])
    keys = []
    if P > 0:
        slots = torch.from_numpy(_slots(h["block_table"][b].numpy(), np.arange(P), bs))
        keys.append(kpool[slots, g].double())
    keys.append(h["k_new"][int(cu[b]):int(cu[b]) + i + 1, g].double())
    keys = torch.cat(keys, 0)
    return (keys @ h["q"][t, head].double()).numpy() * scale * LOG2E

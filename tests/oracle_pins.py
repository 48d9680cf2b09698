"""Pins of the CPU oracle to things other than itself.

Each `pin_*` function takes a loaded oracle library and raises AssertionError
when the oracle disagrees with what the pages or the mathematics fix:
  * hand-worked instances of the pages' examples (tests/golden/);
  * closed forms of softmax attention (one key, two keys, constant values,
    zero query, ramps under a causal mask, per-head constants for GQA);
  * brute force: dense attention over per-sequence arrays that never went
    through a block table;
  * invariants: physical block permutation, shared prefix blocks, cached
    prefix vs full recompute, prefill row vs decode, padding rows, -1 slots.
The mutation test compiles copies of the oracle with planted mistakes and
checks that every one of them trips at least one pin.
"""
import json
import math
import os

import numpy as np
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------- helpers --

def bf16(values):
    """Values rounded to bf16 (round to nearest even), as a torch CPU tensor."""
    return torch.as_tensor(np.asarray(values, dtype=np.float32)).to(torch.bfloat16)


def f64(t):
    return t.to(torch.float64).numpy()


def noise(shape, gen, scale=1.0):
    return (torch.randn(shape, generator=gen, dtype=torch.float32) * scale).to(torch.bfloat16)


def paged_from_logical(K_list, V_list, block_size, num_blocks, rng, gen, max_blocks=None):
    """Scatters per-sequence logical K/V ([L, Hkv, D] bf16) into noise-filled pools.

    Physical blocks are a random permutation; returns (k_pool, v_pool, table).
    """
    Hkv, D = K_list[0].shape[1], K_list[0].shape[2]
    k_pool = noise((num_blocks, block_size, Hkv, D), gen, 3.0)
    v_pool = noise((num_blocks, block_size, Hkv, D), gen, 3.0)
    perm = rng.permutation(num_blocks)
    nblk = [-(-len(K) // block_size) for K in K_list]
    if max_blocks is None:
        max_blocks = max(1, max(nblk))
    table = np.full((len(K_list), max_blocks), -1, dtype=np.int32)
    off = 0
    for b, (K, V) in enumerate(zip(K_list, V_list)):
        ids = perm[off:off + nblk[b]]
        off += nblk[b]
        table[b, :nblk[b]] = ids
        for j in range(len(K)):
            k_pool[ids[j // block_size], j % block_size] = K[j]
            v_pool[ids[j // block_size], j % block_size] = V[j]
    return k_pool, v_pool, table


def dense_attention(q, K, V, scale, causal_offset=None):
    """Dense softmax attention in fp64 with numpy matrix products.

    q [M, Hq, D]; K, V [L, Hkv, D] in logical order. With causal_offset=P, query
    row i sees keys 0 .. P + i; otherwise every row sees all keys.
    """
    q, K, V = f64(q), f64(K), f64(V)
    M, Hq, D = q.shape
    L, Hkv, _ = K.shape
    G = Hq // Hkv
    out = np.zeros((M, Hq, D))
    for h in range(Hq):
        S = scale * (q[:, h, :] @ K[:, h // G, :].T)      # [M, L]
        if causal_offset is not None:
            mask = np.arange(L)[None, :] > (causal_offset + np.arange(M))[:, None]
            S[mask] = -np.inf
        S = S - S.max(axis=1, keepdims=True)
        W = np.exp(S)
        out[:, h, :] = (W @ V[:, h // G, :]) / W.sum(axis=1, keepdims=True)
    return out


def _close(a, b, tol, what):
    err = float(np.max(np.abs(np.asarray(a) - np.asarray(b)))) if np.size(a) else 0.0
    assert err <= tol, f"{what}: max |err| {err:.3e} > {tol:.1e}"


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------- the store --

def pin_store_golden(lib):
    fx = _load("store_tiny.json")
    u16 = lambda a: np.asarray(a, dtype=np.uint16)
    kc, vc = oracle.store_kvcache(u16(fx["k_new"]), u16(fx["v_new"]), u16(fx["k_pool_before"]),
                                  u16(fx["v_pool_before"]), np.asarray(fx["slot_mapping"]),
                                  fx["block_size"], lib=lib)
    assert np.array_equal(kc, u16(fx["k_pool_after"])), "store golden: K pool"
    assert np.array_equal(vc, u16(fx["v_pool_after"])), "store golden: V pool"


def pin_store_skip_and_stride(lib):
    """-1 slots write nothing; k/v may be row slices of a wider fused buffer."""
    gen = torch.Generator().manual_seed(7)
    rng = np.random.default_rng(7)
    nb, bs, hkv, d, hq, T = 6, 16, 2, 8, 4, 40
    kc0 = noise((nb, bs, hkv, d), gen)
    vc0 = noise((nb, bs, hkv, d), gen)
    fused = noise((T, (hq + 2 * hkv) * d), gen)
    k = fused[:, hq * d:(hq + hkv) * d]
    v = fused[:, (hq + hkv) * d:]
    slots = rng.choice(nb * bs, size=T, replace=False).astype(np.int32)
    slots[rng.choice(T, size=9, replace=False)] = -1
    kc, vc = oracle.store_kvcache(k, v, kc0, vc0, slots, bs, lib=lib)
    kc_f = kc.reshape(nb * bs, hkv * d)
    vc_f = vc.reshape(nb * bs, hkv * d)
    k0 = kc0.view(torch.int16).numpy().view(np.uint16).reshape(nb * bs, -1)
    v0 = vc0.view(torch.int16).numpy().view(np.uint16).reshape(nb * bs, -1)
    kk = k.contiguous().view(torch.int16).numpy().view(np.uint16)
    vv = v.contiguous().view(torch.int16).numpy().view(np.uint16)
    written = set(int(s) for s in slots if s >= 0)
    for s in range(nb * bs):
        if s not in written:
            assert np.array_equal(kc_f[s], k0[s]) and np.array_equal(vc_f[s], v0[s]), \
                f"store touched slot {s} that no token names"
    for i, s in enumerate(slots):
        if s >= 0:
            assert np.array_equal(kc_f[s], kk[i]) and np.array_equal(vc_f[s], vv[i]), \
                f"store: token {i} not at slot {s}"


# ------------------------------------------------- the pages' worked example --

def _three_blocks_case():
    fx = _load("three_blocks.json")
    kc = bf16(fx["k_pool"]).reshape(fx["num_blocks"], fx["block_size"], 1, fx["head_dim"])
    vc = bf16(fx["v_pool"]).reshape(fx["num_blocks"], fx["block_size"], 1, fx["head_dim"])
    # The closed form written in the fixture, evaluated here.
    s = [0.0, 0.0, 1.0, 2.0, 0.0]
    v = [[1, 0], [0, 1], [2, -1], [-1, 0.5], [0.25, 4]]
    closed = []
    for i in range(5):
        w = [math.exp(x) for x in s[:i + 1]]
        closed.append([sum(w[j] * v[j][dd] for j in range(i + 1)) / sum(w) for dd in range(2)])
    _close(closed, fx["expected_prefill_rows"], 1e-15, "fixture numbers vs its closed form")
    return fx, kc, vc


def pin_three_blocks_decode(lib):
    fx, kc, vc = _three_blocks_case()
    q = bf16(fx["q"]).reshape(1, 1, 2)
    out = oracle.decode(q, kc, vc, np.asarray(fx["block_table"]), np.asarray([fx["context_len"]]),
                        fx["scale"], lib=lib)
    _close(out[0, 0], fx["expected_decode"], 1e-14, "three-block decode")


def pin_three_blocks_prefill(lib):
    fx, kc, vc = _three_blocks_case()
    q = bf16([fx["q"]] * 5).reshape(5, 1, 2)
    out = oracle.prefill(q, kc, vc, np.asarray([0, 5]), np.asarray([5]),
                         np.asarray(fx["block_table"]), fx["scale"], lib=lib)
    _close(out[:, 0, :], fx["expected_prefill_rows"], 1e-14, "three-block causal prefill")


# ------------------------------------------------------------ brute force --

def _random_logical(rng, gen, lens, hkv, d):
    K = [noise((L, hkv, d), gen) for L in lens]
    V = [noise((L, hkv, d), gen) for L in lens]
    return K, V


def pin_brute_force_decode(lib):
    rng = np.random.default_rng(11)
    gen = torch.Generator().manual_seed(11)
    for bs, hq, hkv, d, lens in [(256, 16, 8, 128, [100, 300, 257, 1]),
                                 (16, 8, 2, 64, [33, 16, 1, 90]),
                                 (4, 4, 4, 16, [7, 1, 12])]:
        K, V = _random_logical(rng, gen, lens, hkv, d)
        nb = sum(-(-L // bs) for L in lens) + 3
        kc, vc, table = paged_from_logical(K, V, bs, nb, rng, gen)
        q = noise((len(lens), hq, d), gen)
        scale = float(np.float32(1 / math.sqrt(d)))
        out = oracle.decode(q, kc, vc, table, np.asarray(lens), scale, lib=lib)
        for b, L in enumerate(lens):
            ref = dense_attention(q[b:b + 1], K[b], V[b], scale)[0]
            _close(out[b], ref, 1e-12, f"decode vs dense (bs={bs}, L={L})")


def pin_brute_force_prefill(lib):
    rng = np.random.default_rng(12)
    gen = torch.Generator().manual_seed(12)
    bs, hq, hkv, d = 16, 8, 2, 32
    prefix = [0, 32, 16, 48]
    new = [20, 5, 1, 17]
    lens = [p + n for p, n in zip(prefix, new)]
    K, V = _random_logical(rng, gen, lens, hkv, d)
    nb = sum(-(-L // bs) for L in lens) + 2
    kc, vc, table = paged_from_logical(K, V, bs, nb, rng, gen)
    q = noise((sum(new), hq, d), gen)
    cu = np.concatenate([[0], np.cumsum(new)])
    scale = 0.3
    out = oracle.prefill(q, kc, vc, cu, np.asarray(lens), table, scale, lib=lib)
    for b in range(len(lens)):
        ref = dense_attention(q[cu[b]:cu[b + 1]], K[b], V[b], scale, causal_offset=prefix[b])
        _close(out[cu[b]:cu[b + 1]], ref, 1e-12, f"prefill vs dense causal (seq {b})")


# ------------------------------------------------------------ closed forms --

def _one_seq(K, V, bs, gen, rng, nb_extra=2):
    nb = -(-len(K) // bs) + nb_extra
    return paged_from_logical([K], [V], bs, nb, rng, gen)


def pin_single_key(lib):
    """L = 1: the only weight is 1, so o equals v_0 exactly."""
    rng = np.random.default_rng(13)
    gen = torch.Generator().manual_seed(13)
    K, V = _random_logical(rng, gen, [1], 2, 16)
    kc, vc, table = _one_seq(K[0], V[0], 4, gen, rng)
    q = noise((1, 4, 16), gen)
    out = oracle.decode(q, kc, vc, table, np.asarray([1]), 0.25, lib=lib)
    for h in range(4):
        assert np.array_equal(out[0, h], f64(V[0][0, h // 2])), "L=1 must return v_0 exactly"


def pin_constant_values(lib):
    """Every value row equal to c gives o = c whatever the weights."""
    rng = np.random.default_rng(14)
    gen = torch.Generator().manual_seed(14)
    L, hkv, d = 37, 2, 16
    K = noise((L, hkv, d), gen)
    c = noise((1, hkv, d), gen)
    V = c.expand(L, hkv, d).clone()
    kc, vc, table = _one_seq(K, V, 8, gen, rng)
    q = noise((1, 4, d), gen, 4.0)
    out = oracle.decode(q, kc, vc, table, np.asarray([L]), 0.5, lib=lib)
    for h in range(4):
        _close(out[0, h], f64(c[0, h // 2]), 1e-14, "constant V")


def pin_zero_query_mean(lib):
    """q = 0 makes every score 0, so o is the plain mean of the value rows."""
    rng = np.random.default_rng(15)
    gen = torch.Generator().manual_seed(15)
    L, hkv, d = 45, 1, 8
    K, V = _random_logical(rng, gen, [L], hkv, d)
    kc, vc, table = _one_seq(K[0], V[0], 16, gen, rng)
    q = torch.zeros((1, 2, d), dtype=torch.bfloat16)
    out = oracle.decode(q, kc, vc, table, np.asarray([L]), 0.7, lib=lib)
    mean = f64(V[0][:, 0, :]).mean(axis=0)
    _close(out[0, 0], mean, 1e-14, "zero query mean")
    _close(out[0, 1], mean, 1e-14, "zero query mean")


def pin_two_keys_logistic(lib):
    """Two keys: o = sigma(x) v_0 + (1 - sigma(x)) v_1 with x = scale q.(k_0 - k_1)."""
    rng = np.random.default_rng(16)
    gen = torch.Generator().manual_seed(16)
    d = 4
    q = bf16([[[2.0, 0.0, -1.0, 0.0]]])
    K = bf16([[[1.5, 0.0, 0.5, 3.0]], [[0.0, 0.0, 0.0, -2.0]]])   # q.k0 = 2.5, q.k1 = 0
    V = bf16([[[1.0, -2.0, 0.5, 4.0]], [[-3.0, 1.0, 0.0, 2.0]]])
    kc, vc, table = _one_seq(K, V, 2, gen, rng)
    for scale in (0.125, 1.0, 0.0883883461356163):
        x = scale * 2.5
        sig = 1.0 / (1.0 + math.exp(-x))
        expect = [sig * a + (1 - sig) * b for a, b in zip([1.0, -2.0, 0.5, 4.0], [-3.0, 1.0, 0.0, 2.0])]
        out = oracle.decode(q, kc, vc, table, np.asarray([2]), scale, lib=lib)
        _close(out[0, 0], expect, 1e-14, f"two-key logistic (scale {scale})")


def pin_gqa_grouping(lib):
    """Query head h reads kv head h // (Hq/Hkv): give each kv head its own constant V."""
    rng = np.random.default_rng(17)
    gen = torch.Generator().manual_seed(17)
    for hq, hkv in [(8, 2), (16, 8), (32, 8), (4, 4), (8, 1)]:
        L, d = 20, 8
        K = noise((L, hkv, d), gen)
        V = torch.stack([bf16(np.full((L, d), g + 1.0)) for g in range(hkv)], dim=1)
        kc, vc, table = _one_seq(K, V, 8, gen, rng)
        q = noise((1, hq, d), gen)
        out = oracle.decode(q, kc, vc, table, np.asarray([L]), 0.3, lib=lib)
        for h in range(hq):
            expect = h // (hq // hkv) + 1.0
            _close(out[0, h], np.full(d, expect), 1e-13, f"GQA head {h} of {hq}/{hkv}")


def pin_dominant_key(lib):
    """A key aligned with q far more than the rest takes all the weight."""
    rng = np.random.default_rng(18)
    gen = torch.Generator().manual_seed(18)
    L, d = 30, 16
    q = bf16(np.ones((1, 1, d)))
    K = bf16(np.zeros((L, 1, d)))
    K[19] = bf16(np.full((1, d), 8.0))          # score 128 * scale against 0
    V = noise((L, 1, d), gen)
    kc, vc, table = _one_seq(K, V, 4, gen, rng)
    out = oracle.decode(q, kc, vc, table, np.asarray([L]), 1.0, lib=lib)
    _close(out[0, 0], f64(V[19, 0]), 1e-40 + 1e-12, "dominant key")
    # A key anti-aligned with q gets no weight at all: o = mean of the others.
    K[19] = bf16(np.full((1, d), -8.0))
    kc, vc, table = _one_seq(K, V, 4, gen, rng)
    out = oracle.decode(q, kc, vc, table, np.asarray([L]), 1.0, lib=lib)
    others = np.delete(f64(V[:, 0]), 19, axis=0).mean(axis=0)
    _close(out[0, 0], others, 1e-12, "anti-aligned key")


def pin_decode_ramp(lib):
    """q = 0 and V_j = j: o = (L - 1) / 2, so the new token at L - 1 is included."""
    rng = np.random.default_rng(19)
    gen = torch.Generator().manual_seed(19)
    for L, bs in [(1, 16), (17, 16), (100, 16), (256, 256), (200, 64)]:
        K = noise((L, 1, 4), gen)
        V = bf16(np.repeat(np.arange(L, dtype=np.float32)[:, None, None], 4, axis=2))
        kc, vc, table = _one_seq(K, V, bs, gen, rng)
        q = torch.zeros((1, 1, 4), dtype=torch.bfloat16)
        out = oracle.decode(q, kc, vc, table, np.asarray([L]), 1.0, lib=lib)
        _close(out[0, 0], np.full(4, (L - 1) / 2), 1e-12, f"decode ramp L={L}")


def pin_causal_ramp(lib):
    """Prefill with q = 0 and V_j = (j, j mod 2): row i of N new rows after a
    P-token prefix averages keys 0 .. P+i, giving ((P+i)/2, #odd/(P+i+1))."""
    rng = np.random.default_rng(20)
    gen = torch.Generator().manual_seed(20)
    bs = 16
    for P, N in [(0, 40), (32, 30), (48, 1), (16, 64)]:
        L = P + N
        K = noise((L, 1, 2), gen)
        j = np.arange(L, dtype=np.float32)
        V = bf16(np.stack([j, j % 2], axis=1)[:, None, :])
        kc, vc, table = _one_seq(K, V, bs, gen, rng)
        q = torch.zeros((N, 2, 2), dtype=torch.bfloat16)
        out = oracle.prefill(q, kc, vc, np.asarray([0, N]), np.asarray([L]), table, 1.0, lib=lib)
        for i in range(N):
            n_vis = P + i + 1
            expect = [(P + i) / 2, (n_vis // 2) / n_vis]
            for h in range(2):
                _close(out[i, h], expect, 1e-12, f"causal ramp P={P} row {i}")


# -------------------------------------------------------------- invariants --

def _random_paged_decode(seed, lens, bs, hq, hkv, d, extra_blocks=3):
    rng = np.random.default_rng(seed)
    gen = torch.Generator().manual_seed(seed)
    K, V = _random_logical(rng, gen, lens, hkv, d)
    nb = sum(-(-L // bs) for L in lens) + extra_blocks
    kc, vc, table = paged_from_logical(K, V, bs, nb, rng, gen)
    q = noise((len(lens), hq, d), gen)
    return q, kc, vc, table, rng


def pin_block_permutation(lib):
    """Relabelling physical blocks (pool and table together) changes no bit."""
    for bs in (16, 256):
        lens = [40, 300, 1, 129]
        q, kc, vc, table, rng = _random_paged_decode(21 + bs, lens, bs, 8, 2, 32)
        out = oracle.decode(q, kc, vc, table, np.asarray(lens), 0.2, lib=lib)
        nb = kc.shape[0]
        perm = rng.permutation(nb)            # old block id -> new block id
        kc2 = torch.empty_like(kc)
        vc2 = torch.empty_like(vc)
        kc2[torch.from_numpy(perm)] = kc
        vc2[torch.from_numpy(perm)] = vc
        table2 = np.where(table >= 0, perm[np.maximum(table, 0)], -1).astype(np.int32)
        out2 = oracle.decode(q, kc2, vc2, table2, np.asarray(lens), 0.2, lib=lib)
        assert np.array_equal(out, out2), f"block permutation changed the output (bs={bs})"


def pin_shared_prefix(lib):
    """Two sequences on the same first k physical blocks, with the same query rows
    there, get bit-identical outputs on those rows in a full causal recompute."""
    rng = np.random.default_rng(22)
    gen = torch.Generator().manual_seed(22)
    bs, hq, hkv, d, k = 16, 4, 2, 16, 2
    nb = 12
    kc = noise((nb, bs, hkv, d), gen)
    vc = noise((nb, bs, hkv, d), gen)
    table = np.array([[5, 9, 1, 3], [5, 9, 7, 0]], dtype=np.int32)
    lens = [60, 50]
    qs = noise((max(lens), hq, d), gen)
    q2 = noise((max(lens), hq, d), gen)
    q2[:k * bs] = qs[:k * bs]
    q = torch.cat([qs[:lens[0]], q2[:lens[1]]])
    cu = np.asarray([0, lens[0], lens[0] + lens[1]])
    out = oracle.prefill(q, kc, vc, cu, np.asarray(lens), table, 0.4, lib=lib)
    a = out[:k * bs]
    b = out[lens[0]:lens[0] + k * bs]
    assert np.array_equal(a, b), "shared prefix rows differ"
    assert not np.array_equal(out[k * bs:lens[0]][:5], out[lens[0] + k * bs:][:5])


def pin_cached_prefix_equals_recompute(lib):
    """New rows after a cached prefix equal the same rows of a full recompute."""
    rng = np.random.default_rng(23)
    gen = torch.Generator().manual_seed(23)
    bs, hq, hkv, d = 16, 8, 4, 32
    P, N = 48, 21
    L = P + N
    K, V = _random_logical(rng, gen, [L], hkv, d)
    kc, vc, table = _one_seq(K[0], V[0], bs, gen, rng)
    q_all = noise((L, hq, d), gen)
    full = oracle.prefill(q_all, kc, vc, np.asarray([0, L]), np.asarray([L]), table, 0.2, lib=lib)
    cached = oracle.prefill(q_all[P:], kc, vc, np.asarray([0, N]), np.asarray([L]), table, 0.2,
                            lib=lib)
    assert np.array_equal(full[P:], cached), "cached-prefix prefill != full recompute"


def pin_prefill_row_equals_decode(lib):
    """Prefill row i (prefix P) equals decode of the same query with L = P + i + 1."""
    rng = np.random.default_rng(24)
    gen = torch.Generator().manual_seed(24)
    bs, hq, hkv, d = 16, 8, 2, 32
    P, N = 32, 13
    L = P + N
    K, V = _random_logical(rng, gen, [L], hkv, d)
    kc, vc, table = _one_seq(K[0], V[0], bs, gen, rng)
    q = noise((N, hq, d), gen)
    pre = oracle.prefill(q, kc, vc, np.asarray([0, N]), np.asarray([L]), table, 0.25, lib=lib)
    for i in range(N):
        dec = oracle.decode(q[i:i + 1], kc, vc, table, np.asarray([P + i + 1]), 0.25, lib=lib)
        assert np.array_equal(pre[i], dec[0]), f"prefill row {i} != decode"


def pin_padding_rows_zero(lib):
    """A row with context length 0 (slot -1 padding) outputs zeros."""
    q, kc, vc, table, _ = _random_paged_decode(25, [20, 1, 33], 16, 4, 2, 16)
    table[1, :] = -1
    out = oracle.decode(q, kc, vc, table, np.asarray([20, 0, 33]), 0.3, lib=lib)
    assert np.all(out[1] == 0.0), "padding row must be zeros"
    assert np.all(np.abs(out[0]) > 0) or np.any(out[0] != 0)


def pin_row_subsets(lib):
    """Computing a subset of rows gives the same bits as computing them all."""
    lens = [40, 7, 120, 64, 3]
    q, kc, vc, table, _ = _random_paged_decode(26, lens, 16, 8, 2, 32)
    full = oracle.decode(q, kc, vc, table, np.asarray(lens), 0.2, lib=lib, nthreads=3)
    part = oracle.decode(q, kc, vc, table, np.asarray(lens), 0.2, rows=[4, 2], lib=lib)
    assert np.array_equal(full[[4, 2]], part[[4, 2]]) and np.all(part[[0, 1, 3]] == 0)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]

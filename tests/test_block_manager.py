"""Block manager: the oracle pinned to the pages' rules and to XXH64's
published definition, then libpa.so's C++ manager held to the oracle, op for
op. Host code only; nothing here touches the GPU."""
import json
import os
import random

import numpy as np
import pytest
import xxhash

from oracle.block_manager import (BadSequence, BlockManager as OracleBM, NoBlocks, block_hash,
                                  xxh64)
from paged_kv_cache_slot_amd import PAError
from paged_kv_cache_slot_amd import block_manager as native

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "block_manager_scenario.json")
PA_ERR_NO_BLOCKS, PA_ERR_SEQ, PA_ERR_SHAPE = -6, -7, -2


# --------------------------------------------------------------- XXH64 pins --

def test_xxh64_empty_input_published_value():
    # The xxHash specification's test value for XXH64 of no bytes, seed 0.
    assert xxh64(b"", 0) == 0xEF46DB3751D8E999


@pytest.mark.parametrize("impl", ["oracle", "native"])
def test_xxh64_matches_library_every_tail_shape(impl):
    """Lengths 0..130 cover every path: no stripe / stripes, and each mix of
    8-, 4- and 1-byte tail steps; seeds include 0, 1 and wrap-around values."""
    f = xxh64 if impl == "oracle" else native.xxh64
    rng = random.Random(7)
    for n in list(range(131)) + [1024, 1031, 4099]:
        data = bytes(rng.getrandbits(8) for _ in range(n))
        for seed in (0, 1, 2**64 - 1, rng.getrandbits(64)):
            assert f(data, seed) == xxhash.xxh64_intdigest(data, seed), (impl, n, seed)


@pytest.mark.parametrize("impl", ["oracle", "native"])
def test_block_hash_serialisation(impl):
    """The chained block hash is XXH64 over le64(parent) followed by the token
    ids as le32 (negative ids as two's complement); no parent, no prefix bytes."""
    f = block_hash if impl == "oracle" else native.block_hash
    toks = [0, 1, 151935, -1, 2**31 - 1, -2**31, 42, 7]
    raw = np.asarray(toks, dtype="<i4").tobytes()
    assert f(toks) == xxhash.xxh64_intdigest(raw, 0)
    parent = 0x0123456789ABCDEF
    assert f(toks, parent) == xxhash.xxh64_intdigest(parent.to_bytes(8, "little") + raw, 0)
    # position dependence: the same tokens after a prefix hash differently
    assert f([2, 2, 2, 2]) != f([2, 2, 2, 2], f([2, 2, 2, 2]))
    # the parent value 0 still differs from having no parent
    assert f(toks, 0) != f(toks)


# ----------------------------------------------------------- golden scenario --

def _run_golden(make, apply_checks):
    with open(GOLDEN) as f:
        g = json.load(f)
    bm = make(g["num_blocks"], g["block_size"])
    ids = {}
    for step, op in enumerate(g["ops"]):
        apply_checks(bm, op, ids, step)
    return bm, g


def _golden_oracle(bm, op, ids, step):
    kind = op["op"]
    sid = ids.setdefault(op.get("seq"), len(ids)) if "seq" in op else None
    ctx = f"step {step}: {op}"
    if kind == "allocate":
        if op.get("error") == "no_blocks":
            with pytest.raises(NoBlocks):
                bm.allocate(sid, op["tokens"])
        else:
            assert bm.allocate(sid, op["tokens"]) == op["cached"], ctx
            assert bm.seqs[sid]["table"] == op["table"], ctx
    elif kind == "deallocate":
        bm.deallocate(sid)
    elif kind == "append":
        if op.get("error") == "no_blocks":
            with pytest.raises(NoBlocks):
                bm.append(sid, op["token"])
        else:
            bm.append(sid, op["token"])
        if "table" in op:
            assert bm.seqs[sid]["table"] == op["table"], ctx
    elif kind == "can_allocate":
        assert bm.can_allocate(op["tokens"]) == op["ok"], ctx
    elif kind == "can_append":
        assert bm.can_append(sid) == op["ok"], ctx
    elif kind == "decode_metadata":
        seqs = [ids[s] for s in op["seqs"]]
        c, s, t = bm.decode_metadata(seqs, op["padded_batch"], op["stride"])
        assert (c, s, t) == (op["context_lens"], op["slot_mapping"], op["block_table"]), ctx
    elif kind == "prefill_metadata":
        seqs = [ids[s] for s in op["seqs"]]
        cu, c, s, t = bm.prefill_metadata(seqs, op["stride"])
        assert (cu, c, s, t) == (op["cu_seqlens_q"], op["context_lens"], op["slot_mapping"],
                                 op["block_table"]), ctx
    if "len" in op:
        assert len(bm.seqs[sid]["tokens"]) == op["len"], ctx
    if "refs" in op:
        assert bm.ref == op["refs"], ctx
    if "free" in op:
        assert bm.free == op["free"], ctx


def test_oracle_golden_scenario():
    bm, g = _run_golden(OracleBM, _golden_oracle)
    assert bm.stats == g["final_stats"]


def _golden_native(bm, op, ids, step):
    kind = op["op"]
    sid = ids.setdefault(op.get("seq"), 1000 + 17 * len(ids)) if "seq" in op else None
    ctx = f"step {step}: {op}"
    if kind == "allocate":
        if op.get("error") == "no_blocks":
            with pytest.raises(PAError) as e:
                bm.allocate(sid, op["tokens"])
            assert e.value.status == PA_ERR_NO_BLOCKS
        else:
            assert bm.allocate(sid, op["tokens"]) == op["cached"], ctx
            assert bm.block_table(sid).tolist() == op["table"], ctx
    elif kind == "deallocate":
        bm.deallocate(sid)
    elif kind == "append":
        if op.get("error") == "no_blocks":
            with pytest.raises(PAError) as e:
                bm.append(sid, op["token"])
            assert e.value.status == PA_ERR_NO_BLOCKS
        else:
            bm.append(sid, op["token"])
        if "table" in op:
            assert bm.block_table(sid).tolist() == op["table"], ctx
    elif kind == "can_allocate":
        assert bm.can_allocate(op["tokens"]) == op["ok"], ctx
    elif kind == "can_append":
        assert bm.can_append(sid) == op["ok"], ctx
    elif kind == "decode_metadata":
        seqs = [ids[s] for s in op["seqs"]]
        c, s, t, mx = bm.decode_metadata(seqs, op["padded_batch"], op["stride"])
        assert c.tolist() == op["context_lens"] and s.tolist() == op["slot_mapping"], ctx
        assert t.tolist() == op["block_table"] and mx == max(op["context_lens"]), ctx
    elif kind == "prefill_metadata":
        seqs = [ids[s] for s in op["seqs"]]
        cu, c, s, t, tq, mq = bm.prefill_metadata(seqs, op["stride"])
        assert cu.tolist() == op["cu_seqlens_q"] and c.tolist() == op["context_lens"], ctx
        assert s.tolist() == op["slot_mapping"] and t.tolist() == op["block_table"], ctx
        assert tq == op["cu_seqlens_q"][-1]
        assert mq == max(np.diff(op["cu_seqlens_q"]))
    if "len" in op:
        assert bm.seq_info(sid)[0] == op["len"], ctx
    if "refs" in op:
        assert [bm.block_info(b)[0] for b in range(bm.num_blocks)] == op["refs"], ctx
    if "free" in op:
        assert bm.num_free_blocks == len(op["free"]), ctx


def test_native_golden_scenario():
    bm, g = _run_golden(native.BlockManager, _golden_native)
    assert bm.stats() == g["final_stats"]


# ------------------------------------------- random ops: invariants and parity --

class PoolContent:
    """What each pool slot holds, modelled as the token prefix whose K/V sits
    there: the K/V of position p depends on tokens[0..p]. A sequence reads
    correct K/V exactly when every slot its table names holds its own prefix."""

    def __init__(self):
        self.slot = {}

    def write(self, slot, prefix):
        self.slot[slot] = prefix

    def check(self, bm, sid):
        toks = bm.seqs[sid]["tokens"]
        for p in range(len(toks)):
            assert self.slot.get(bm.slot(sid, p)) == tuple(toks[:p + 1]), (sid, p)


def _random_ops(seed, n_ops, num_blocks, bs):
    """Prompts built from a few shared stems so cache hits, take-backs and
    evictions all happen; ids are reused after deallocation."""
    rng = random.Random(seed)
    # Two stems over a large alphabet, two over {0, 1}: the latter repeat whole
    # blocks at different positions and after different prefixes.
    stems = [[rng.randrange(50) for _ in range(rng.randrange(bs, 4 * bs))] for _ in range(2)]
    stems += [[rng.randrange(2) for _ in range(rng.randrange(bs, 4 * bs))] for _ in range(2)]
    ops = []
    for _ in range(n_ops):
        r = rng.random()
        if r < 0.35:
            stem = rng.choice(stems)
            alphabet = 50 if rng.random() < 0.5 else 2
            cut = rng.randrange(len(stem) + 1)
            tail = [rng.randrange(alphabet)
                    for _ in range(rng.randrange(0 if cut else 1, 2 * bs))]
            ops.append(("allocate", rng.randrange(12), stem[:cut] + tail))
        elif r < 0.65:
            ops.append(("append", rng.randrange(12), rng.choice([rng.randrange(50), 1, 0])))
        elif r < 0.75:
            ids = [rng.randrange(12) for _ in range(rng.randrange(1, 6))]
            ops.append(("append_batch", ids, [rng.randrange(3) for _ in ids]))
        else:
            ops.append(("deallocate", rng.randrange(12), None))
    return ops


def _oracle_invariants(bm):
    bs = bm.block_size
    count = [0] * bm.num_blocks
    for sid, s in bm.seqs.items():
        assert len(s["table"]) == -(-len(s["tokens"]) // bs)
        assert len(set(s["table"])) == len(s["table"])
        assert s["cached"] % bs == 0 and s["cached"] < len(s["tokens"]) or s["cached"] == 0
        for b in s["table"]:
            count[b] += 1
    assert count == bm.ref
    assert sorted(bm.free) == [b for b in range(bm.num_blocks) if bm.ref[b] == 0]
    for h, b in bm.index.items():
        assert bm.hash[b] == h


@pytest.mark.parametrize("seed,num_blocks,bs", [(0, 24, 4), (1, 16, 4), (2, 40, 8), (3, 9, 2),
                                                (4, 64, 16)])
def test_oracle_invariants_under_random_ops(seed, num_blocks, bs):
    """Reference counts, the free queue and the index stay consistent, and every
    live sequence reads its own prefix's K/V through its table (this fails if
    the chain drops its parent, shares a block across positions, or hands out
    a block that is still cached under another prefix)."""
    bm = OracleBM(num_blocks, bs)
    pool = PoolContent()
    for kind, sid, arg in _random_ops(seed, 600, num_blocks, bs):
        if kind == "allocate":
            if sid in bm.seqs or not bm.can_allocate(arg):
                continue
            cached = bm.allocate(sid, arg)
            for p in range(cached, len(arg)):
                pool.write(bm.slot(sid, p), tuple(arg[:p + 1]))
        elif kind == "append":
            if sid not in bm.seqs or not bm.can_append(sid):
                continue
            bm.append(sid, arg)
            toks = bm.seqs[sid]["tokens"]
            pool.write(bm.slot(sid, len(toks) - 1), tuple(toks))
        elif kind == "append_batch":
            try:
                bm.append_batch(sid, arg)
            except (NoBlocks, BadSequence):
                continue
            for s in sid:
                toks = bm.seqs[s]["tokens"]
                pool.write(bm.slot(s, len(toks) - 1), tuple(toks))
        elif sid in bm.seqs:
            bm.deallocate(sid)
        _oracle_invariants(bm)
        for s in bm.seqs:
            pool.check(bm, s)
    st = bm.stats
    assert st["shared"] > 0 and st["fresh_alloc"] > 0 and st["fresh_append"] > 0
    assert st["taken_back"] > 0 and st["evicted"] > 0


@pytest.mark.parametrize("seed,num_blocks,bs", [(10, 24, 4), (11, 16, 4), (12, 40, 8),
                                                (13, 9, 2), (14, 64, 16), (15, 7, 1)])
def test_native_matches_oracle_op_for_op(seed, num_blocks, bs):
    """Both managers see the same calls, failures included; after each call
    their answers, tables, reference counts, hashes, free counts and totals
    are equal, and so are the metadata arrays of all live sequences."""
    ob, nb = OracleBM(num_blocks, bs), native.BlockManager(num_blocks, bs)
    for i, (kind, sid, arg) in enumerate(_random_ops(seed, 700, num_blocks, bs)):
        if kind == "allocate":
            assert nb.can_allocate(arg) == ob.can_allocate(arg)
            try:
                want = ob.allocate(sid, arg)
            except (NoBlocks, BadSequence) as e:
                with pytest.raises(PAError) as got:
                    nb.allocate(sid, arg)
                assert got.value.status == (PA_ERR_NO_BLOCKS if isinstance(e, NoBlocks)
                                            else PA_ERR_SEQ)
            else:
                assert nb.allocate(sid, arg) == want
        elif kind == "append":
            if sid in ob.seqs:
                assert nb.can_append(sid) == ob.can_append(sid)
            try:
                ob.append(sid, arg)
            except (NoBlocks, BadSequence) as e:
                with pytest.raises(PAError) as got:
                    nb.append(sid, arg)
                assert got.value.status == (PA_ERR_NO_BLOCKS if isinstance(e, NoBlocks)
                                            else PA_ERR_SEQ)
            else:
                nb.append(sid, arg)
        elif kind == "append_batch":
            try:
                ob.append_batch(sid, arg)
            except (NoBlocks, BadSequence) as e:
                with pytest.raises(PAError) as got:
                    nb.append_batch(sid, arg)
                assert got.value.status == (PA_ERR_NO_BLOCKS if isinstance(e, NoBlocks)
                                            else PA_ERR_SEQ)
            else:
                nb.append_batch(sid, arg)
        else:
            try:
                ob.deallocate(sid)
            except BadSequence:
                with pytest.raises(PAError) as got:
                    nb.deallocate(sid)
                assert got.value.status == PA_ERR_SEQ
            else:
                nb.deallocate(sid)
        assert nb.num_free_blocks == len(ob.free), i
        for b in range(num_blocks):
            ref, cached, h = nb.block_info(b)
            assert ref == ob.ref[b]
            assert h == (ob.hash[b] or 0)
            assert cached == (ob.hash[b] is not None and ob.index.get(ob.hash[b]) == b)
        for s, rec in ob.seqs.items():
            assert nb.block_table(s).tolist() == rec["table"]
            assert nb.seq_info(s) == (len(rec["tokens"]), rec["cached"], len(rec["table"]))
    assert nb.stats() == ob.stats
    live = sorted(ob.seqs)
    if live:
        stride = max(len(ob.seqs[s]["table"]) for s in live) + 1
        c, s, t, _ = nb.decode_metadata(live, len(live) + 3, stride)
        assert (c.tolist(), s.tolist(), t.tolist()) == ob.decode_metadata(live, len(live) + 3,
                                                                          stride)
        rows = [len(ob.seqs[x]["tokens"]) - ob.seqs[x]["cached"] for x in live]
        assert nb.batch_info(live) == (sum(rows), max(rows),
                                       max(len(ob.seqs[x]["tokens"]) for x in live),
                                       stride - 1)
        P = len(live) + 1
        out = (np.full(P, 7, np.int32), np.full(P, 7, np.int32), np.full((P, stride), 7, np.int32))
        c, s, t, _ = nb.decode_metadata(live, P, stride, out=out)
        assert c is out[0] and s is out[1] and t is out[2]
        assert (c.tolist(), s.tolist(), t.tolist()) == ob.decode_metadata(live, P, stride)
        cu, c, s, t, _, _ = nb.prefill_metadata(live, stride)
        assert (cu.tolist(), c.tolist(), s.tolist(), t.tolist()) == ob.prefill_metadata(live,
                                                                                        stride)


# ------------------------------------------------------------- error handling --

def test_native_errors_change_nothing():
    bm = native.BlockManager(4, 4)
    assert bm.allocate(1, list(range(10))) == 0
    before = ([bm.block_info(b) for b in range(4)], bm.num_free_blocks, bm.stats())
    with pytest.raises(PAError) as e:
        bm.allocate(1, [1, 2])                 # live id
    assert e.value.status == PA_ERR_SEQ
    with pytest.raises(PAError) as e:
        bm.allocate(2, list(range(100, 112)))   # 3 fresh blocks, 1 free
    assert e.value.status == PA_ERR_NO_BLOCKS
    with pytest.raises(PAError) as e:
        bm.allocate(3, [])
    assert e.value.status == PA_ERR_SHAPE
    for call in (lambda: bm.append(9, 1), lambda: bm.deallocate(9), lambda: bm.seq_info(9),
                 lambda: bm.decode_metadata([1, 9], 2, 4), lambda: bm.prefill_metadata([9], 4, 4)):
        with pytest.raises(PAError) as e:
            call()
        assert e.value.status == PA_ERR_SEQ
    with pytest.raises(PAError) as e:
        bm.decode_metadata([1], 1, 2)           # 3 blocks do not fit a stride of 2
    assert e.value.status == PA_ERR_SHAPE
    with pytest.raises(PAError) as e:
        bm.decode_metadata([1], 0, 4)           # padded batch below batch
    assert e.value.status == PA_ERR_SHAPE
    with pytest.raises(PAError) as e:
        bm.prefill_metadata([1], 4, slot_capacity=9)  # 10 rows, room for 9
    assert e.value.status == PA_ERR_SHAPE
    with pytest.raises(PAError) as e:
        bm.append_batch([1, 1], [5, 6])          # repeated id
    assert e.value.status == PA_ERR_SEQ
    with pytest.raises(PAError) as e:
        bm.append_batch([1, 9], [5, 6])          # unknown id after a valid one
    assert e.value.status == PA_ERR_SEQ
    assert ([bm.block_info(b) for b in range(4)], bm.num_free_blocks, bm.stats()) == before
    with pytest.raises(ValueError):
        native.BlockManager(0, 16)
    with pytest.raises(ValueError):
        native.BlockManager(16, 0)


def test_native_prefill_metadata_padding():
    bm = native.BlockManager(8, 4)
    bm.allocate(5, [1, 2, 3, 4, 5, 6])
    cu, c, s, t, tq, mq = bm.prefill_metadata([5], 3, slot_capacity=9)
    assert cu.tolist() == [0, 6] and c.tolist() == [6] and (tq, mq) == (6, 6)
    assert s.tolist() == [0, 1, 2, 3, 4, 5, -1, -1, -1]
    assert t.tolist() == [[0, 1, -1]]
    c, s, t, mx = bm.decode_metadata([], 2, 3)
    assert c.tolist() == [0, 0] and s.tolist() == [-1, -1] and mx == 0
    assert t.tolist() == [[-1, -1, -1], [-1, -1, -1]]

"""Block manager oracle: a plain, slow Python model of paged KV block
allocation with chained-hash prefix caching.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this module. It shares no code with the
product library's C++ block manager.

What it follows:
  [Report] "nano-vllm 深度分析报告" (nightvoyager), section "创新之处", the
  BlockManager item: paging and prefix caching in one structure; blocks are
  content-addressed by XXH64 chained over the prompt (each block's hash takes
  in the hash before it); allocate distinguishes a cached block still in use
  (shared), a cached block already freed (taken back) and a fresh block;
  may_append registers a block when it fills. Table "可复用的模式与技巧", row
  "xxhash64 链式哈希 KV Cache": chaining makes a block's identity depend on
  its position.
  [QbitAI] "DeepSeek研究员1200行代码复刻vLLM…", section "vLLM是什么？": a
  block table maps a sequence's logical blocks to physical blocks.

The pages leave these rules open; this model takes the plainest readings:
  * h_0 = XXH64(le32 tokens of block 0), h_i = XXH64(le64(h_{i-1}) || le32
    tokens of block i), seed 0; only full blocks are hashed.
  * A hit needs equal stored tokens and equal stored parent hash.
  * The cached prefix is contiguous (first miss ends it).
  * The block holding the sequence's last token is always fresh.
  * Free blocks are a FIFO queue: fresh blocks from the front, freed blocks to
    the back (a sequence frees last block first); a freed block keeps its cache
    entry until it is handed out fresh. A newer registration of a hash replaces
    the older entry.

Plain data structures on purpose: a Python list for the free queue (list.remove
for a taken-back block), dicts for the cache index and the sequences.
"""

MASK64 = (1 << 64) - 1

# The five 64-bit primes of the XXH64 specification.
P1 = 11400714785074694791
P2 = 14029467366897019727
P3 = 1609587929392839161
P4 = 9650029242287828579
P5 = 2870177450012600261


def _rotl(x, r):
    return ((x << r) | (x >> (64 - r))) & MASK64


def _round(acc, lane):
    acc = (acc + lane * P2) & MASK64
    acc = _rotl(acc, 31)
    return (acc * P1) & MASK64


def xxh64(data, seed=0):
    """XXH64 of a bytes object, step by step as the xxHash specification lays
    it out: (1) four accumulators over 32-byte stripes (only for inputs of 32
    bytes or more), converged and merged; otherwise seed + PRIME5; (2) add the
    input length; (3) consume the rest as 8-byte, then 4-byte, then 1-byte
    words; (4) avalanche."""
    n = len(data)
    i = 0
    if n >= 32:
        acc = [(seed + P1 + P2) & MASK64, (seed + P2) & MASK64, seed & MASK64,
               (seed - P1) & MASK64]
        while i + 32 <= n:
            for k in range(4):
                lane = int.from_bytes(data[i + 8 * k:i + 8 * k + 8], "little")
                acc[k] = _round(acc[k], lane)
            i += 32
        h = (_rotl(acc[0], 1) + _rotl(acc[1], 7) + _rotl(acc[2], 12) + _rotl(acc[3], 18)) & MASK64
        for k in range(4):
            h ^= _round(0, acc[k])
            h = (h * P1 + P4) & MASK64
    else:
        h = (seed + P5) & MASK64
    h = (h + n) & MASK64
    while i + 8 <= n:
        h ^= _round(0, int.from_bytes(data[i:i + 8], "little"))
        h = (_rotl(h, 27) * P1 + P4) & MASK64
        i += 8
    if i + 4 <= n:
        h ^= (int.from_bytes(data[i:i + 4], "little") * P1) & MASK64
        h = (_rotl(h, 23) * P2 + P3) & MASK64
        i += 4
    while i < n:
        h ^= (data[i] * P5) & MASK64
        h = (_rotl(h, 11) * P1) & MASK64
        i += 1
    h ^= h >> 33
    h = (h * P2) & MASK64
    h ^= h >> 29
    h = (h * P3) & MASK64
    h ^= h >> 32
    return h


def block_hash(tokens, parent=None):
    """Chained hash of one full block: parent (if any) as 8 little-endian
    bytes, then each token id as 4 little-endian bytes (two's complement)."""
    b = b"" if parent is None else int(parent).to_bytes(8, "little")
    for t in tokens:
        b += (int(t) & 0xFFFFFFFF).to_bytes(4, "little")
    return xxh64(b, 0)


class NoBlocks(Exception):
    """Not enough free blocks for the request."""


class BadSequence(Exception):
    """Sequence id unknown, or already live."""


class BlockManager:
    def __init__(self, num_blocks, block_size):
        assert num_blocks >= 1 and block_size >= 1
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.ref = [0] * num_blocks
        self.hash = [None] * num_blocks      # chained hash of a full block
        self.parent = [None] * num_blocks    # the hash before it (None = first block)
        self.tokens = [None] * num_blocks    # its token ids
        self.free = list(range(num_blocks))  # front = next fresh block
        self.index = {}                      # hash -> block id
        self.seqs = {}                       # id -> {"tokens", "table", "hashes", "cached"}
        self.stats = {"shared": 0, "taken_back": 0, "fresh_alloc": 0, "fresh_append": 0,
                      "evicted": 0}

    # -- helpers -----------------------------------------------------------
    def _fresh(self):
        b = self.free.pop(0)
        if self.hash[b] is not None and self.index.get(self.hash[b]) == b:
            del self.index[self.hash[b]]
            self.stats["evicted"] += 1
        self.hash[b] = self.parent[b] = self.tokens[b] = None
        self.ref[b] = 1
        return b

    def _register(self, b, h, parent, tokens):
        self.hash[b] = h
        self.parent[b] = parent
        self.tokens[b] = list(tokens)
        self.index[h] = b

    def _find(self, h, parent, tokens):
        b = self.index.get(h)
        if b is None or self.parent[b] != parent or self.tokens[b] != list(tokens):
            return None
        return b

    def _plan(self, tokens):
        """Per logical block: ("share"|"take_back", block) or ("fresh", None),
        plus the chained hashes of the full blocks. Changes nothing."""
        bs = self.block_size
        n = len(tokens)
        nblk = -(-n // bs)
        hashes = []
        plan = []
        missed = False
        for i in range(nblk):
            chunk = tokens[i * bs:(i + 1) * bs]
            parent = hashes[i - 1] if i > 0 else None
            full = len(chunk) == bs
            if full:
                hashes.append(block_hash(chunk, parent))
            if full and not missed and i != nblk - 1:
                b = self._find(hashes[i], parent, chunk)
                if b is not None:
                    plan.append(("share" if self.ref[b] > 0 else "take_back", b))
                    continue
            missed = True
            plan.append(("fresh", None))
        return plan, hashes

    # -- the calls ---------------------------------------------------------
    def can_allocate(self, tokens):
        plan, _ = self._plan(list(tokens))
        return sum(1 for kind, _ in plan if kind != "share") <= len(self.free)

    def allocate(self, seq_id, tokens):
        """Returns the number of cached leading tokens."""
        tokens = [int(t) for t in tokens]
        if seq_id in self.seqs:
            raise BadSequence(seq_id)
        if len(tokens) < 1:
            raise ValueError("empty sequence")
        plan, hashes = self._plan(tokens)
        if sum(1 for kind, _ in plan if kind != "share") > len(self.free):
            raise NoBlocks()
        bs = self.block_size
        table = []
        cached = 0
        for i, (kind, b) in enumerate(plan):
            if kind == "share":
                self.ref[b] += 1
                self.stats["shared"] += 1
                cached += bs
            elif kind == "take_back":
                self.free.remove(b)
                self.ref[b] = 1
                self.stats["taken_back"] += 1
                cached += bs
            else:
                b = self._fresh()
                self.stats["fresh_alloc"] += 1
                if i < len(hashes):
                    self._register(b, hashes[i], hashes[i - 1] if i > 0 else None,
                                   tokens[i * bs:(i + 1) * bs])
            table.append(b)
        self.seqs[seq_id] = {"tokens": tokens, "table": table, "hashes": list(hashes),
                             "cached": cached}
        return cached

    def can_append(self, seq_id):
        s = self.seqs[seq_id]
        return len(s["tokens"]) % self.block_size != 0 or len(self.free) > 0

    def append(self, seq_id, token):
        if seq_id not in self.seqs:
            raise BadSequence(seq_id)
        s = self.seqs[seq_id]
        bs = self.block_size
        if len(s["tokens"]) % bs == 0:
            if not self.free:
                raise NoBlocks()
            s["table"].append(self._fresh())
            self.stats["fresh_append"] += 1
        s["tokens"].append(int(token))
        n = len(s["tokens"])
        if n % bs == 0:
            i = n // bs - 1
            parent = s["hashes"][i - 1] if i > 0 else None
            chunk = s["tokens"][i * bs:n]
            h = block_hash(chunk, parent)
            s["hashes"].append(h)
            self._register(s["table"][i], h, parent, chunk)

    def append_batch(self, seq_ids, tokens):
        """Appends tokens[i] to seq_ids[i] for all i, or raises before any
        append if an id is unknown or repeated, or if the blocks the step needs
        are not all free."""
        seq_ids = list(seq_ids)
        if any(s not in self.seqs for s in seq_ids) or len(set(seq_ids)) != len(seq_ids):
            raise BadSequence(seq_ids)
        need = sum(1 for s in seq_ids if len(self.seqs[s]["tokens"]) % self.block_size == 0)
        if need > len(self.free):
            raise NoBlocks()
        for s, t in zip(seq_ids, tokens):
            self.append(s, t)

    def deallocate(self, seq_id):
        if seq_id not in self.seqs:
            raise BadSequence(seq_id)
        for b in reversed(self.seqs[seq_id]["table"]):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)
        del self.seqs[seq_id]

    # -- metadata for the attention calls ----------------------------------
    def slot(self, seq_id, pos):
        s = self.seqs[seq_id]
        return s["table"][pos // self.block_size] * self.block_size + pos % self.block_size

    def prefill_metadata(self, seq_ids, block_table_stride, slot_capacity=None):
        """(cu_seqlens_q, context_lens, slot_mapping, block_table) as lists."""
        cu = [0]
        ctx = []
        slots = []
        table = []
        for sid in seq_ids:
            s = self.seqs[sid]
            n = len(s["tokens"])
            for pos in range(s["cached"], n):
                slots.append(self.slot(sid, pos))
            cu.append(len(slots))
            ctx.append(n)
            row = list(s["table"])
            assert len(row) <= block_table_stride
            table.append(row + [-1] * (block_table_stride - len(row)))
        if slot_capacity is not None:
            assert slot_capacity >= len(slots)
            slots += [-1] * (slot_capacity - len(slots))
        return cu, ctx, slots, table

    def decode_metadata(self, seq_ids, padded_batch, block_table_stride):
        """(context_lens, slot_mapping, block_table), padded with length-0 rows,
        slot -1 and block-table rows of -1."""
        ctx, slots, table = [], [], []
        for sid in seq_ids:
            s = self.seqs[sid]
            n = len(s["tokens"])
            ctx.append(n)
            slots.append(self.slot(sid, n - 1))
            row = list(s["table"])
            table.append(row + [-1] * (block_table_stride - len(row)))
        for _ in range(padded_batch - len(seq_ids)):
            ctx.append(0)
            slots.append(-1)
            table.append([-1] * block_table_stride)
        return ctx, slots, table

// Host-side KV block allocator with chained-hash prefix caching (C ABI in
// include/pa_block_manager.h, where the rules it follows are listed with the
// passages they come from).
//
// Data structures, all sized once at creation except the per-sequence ones:
//   blocks_     one record per physical block: reference count, and for a
//               full block its chained hash, its parent's hash and its token ids
//               (kept to confirm a cache hit);
//   next_/prev_ an intrusive doubly linked free queue over block ids, so a
//               freed cached block can leave the middle of the queue in O(1);
//   index_      hash -> block id of the cache entries;
//   seqs_       sequence id -> tokens, block table and per-block hashes.
// Every public call checks everything it can before it changes any state, so
// a call that fails leaves the manager as it was.
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa_block_manager.h"

namespace {

// ------------------------------------------------------------------- XXH64 --
// XXH64 as the xxHash specification defines it: four 64-bit lanes over 32-byte
// stripes, a merge of the lanes, the tail in 8-, 4- and 1-byte steps, and a
// final avalanche. Input words are read little-endian.

constexpr uint64_t kPrime1 = 0x9E3779B185EBCA87ull;
constexpr uint64_t kPrime2 = 0xC2B2AE3D27D4EB4Full;
constexpr uint64_t kPrime3 = 0x165667B19E3779F9ull;
constexpr uint64_t kPrime4 = 0x85EBCA77C2B2AE63ull;
constexpr uint64_t kPrime5 = 0x27D4EB2F165667C5ull;

inline uint64_t rotl64(uint64_t x, int r) { return (x << r) | (x >> (64 - r)); }

// The hash is defined over little-endian words, which is the host's order.
static_assert(__BYTE_ORDER__ == __ORDER_LITTLE_ENDIAN__, "little-endian host assumed");

inline uint64_t read_le64(const uint8_t* p) {
  uint64_t v;
  std::memcpy(&v, p, sizeof(v));
  return v;
}

inline uint32_t read_le32(const uint8_t* p) {
  uint32_t v;
  std::memcpy(&v, p, sizeof(v));
  return v;
}

inline uint64_t lane_round(uint64_t acc, uint64_t input) {
  acc += input * kPrime2;
  acc = rotl64(acc, 31);
  return acc * kPrime1;
}

inline uint64_t merge_lane(uint64_t acc, uint64_t lane) {
  acc ^= lane_round(0, lane);
  return acc * kPrime1 + kPrime4;
}

uint64_t xxh64(const uint8_t* p, size_t len, uint64_t seed) {
  const uint8_t* const end = p + len;
  uint64_t h;
  if (len >= 32) {
    uint64_t v1 = seed + kPrime1 + kPrime2;
    uint64_t v2 = seed + kPrime2;
    uint64_t v3 = seed;
    uint64_t v4 = seed - kPrime1;
    const uint8_t* const last_stripe = end - 32;
    do {
      v1 = lane_round(v1, read_le64(p));
      v2 = lane_round(v2, read_le64(p + 8));
      v3 = lane_round(v3, read_le64(p + 16));
      v4 = lane_round(v4, read_le64(p + 24));
      p += 32;
    } while (p <= last_stripe);
    h = rotl64(v1, 1) + rotl64(v2, 7) + rotl64(v3, 12) + rotl64(v4, 18);
    h = merge_lane(h, v1);
    h = merge_lane(h, v2);
    h = merge_lane(h, v3);
    h = merge_lane(h, v4);
  } else {
    h = seed + kPrime5;
  }
  h += static_cast<uint64_t>(len);
  for (; p + 8 <= end; p += 8) {
    h ^= lane_round(0, read_le64(p));
    h = rotl64(h, 27) * kPrime1 + kPrime4;
  }
  if (p + 4 <= end) {
    h ^= static_cast<uint64_t>(read_le32(p)) * kPrime1;
    h = rotl64(h, 23) * kPrime2 + kPrime3;
    p += 4;
  }
  for (; p < end; ++p) {
    h ^= static_cast<uint64_t>(*p) * kPrime5;
    h = rotl64(h, 11) * kPrime1;
  }
  h ^= h >> 33;
  h *= kPrime2;
  h ^= h >> 29;
  h *= kPrime3;
  h ^= h >> 32;
  return h;
}

// Serialises (parent, tokens) as le64 || le32... into `buf` and hashes it
// (on the little-endian host both are their in-memory bytes).
uint64_t chained_hash(std::vector<uint8_t>& buf, bool has_parent, uint64_t parent,
                      const int32_t* tokens, int32_t n) {
  const size_t head = has_parent ? sizeof(parent) : 0;
  const size_t body = sizeof(int32_t) * static_cast<size_t>(n);
  buf.resize(head + body);
  if (has_parent) std::memcpy(buf.data(), &parent, head);
  if (body) std::memcpy(buf.data() + head, tokens, body);
  return xxh64(buf.data(), buf.size(), 0);
}

// --------------------------------------------------------------- the manager --

struct Block {
  int32_t ref = 0;
  bool hashed = false;       // a full block whose hash was computed
  bool has_parent = false;   // it is not the first block of its sequence
  uint64_t hash = 0;
  uint64_t parent = 0;
  std::vector<int32_t> tokens;  // the block's token ids while hashed
};

struct Seq {
  std::vector<int32_t> tokens;
  std::vector<int32_t> table;    // physical block of each logical block
  std::vector<uint64_t> hashes;  // chained hash of each full logical block
  int32_t cached = 0;            // leading tokens found in the cache at allocation
  uint64_t stamp = 0;            // last batched call that named it (repeat check)
};

// What allocate would do with one logical block.
enum class Plan : uint8_t { kShare, kTakeBack, kFresh };

}  // namespace

struct pa_block_manager {
  int32_t num_blocks;
  int32_t block_size;
  std::vector<Block> blocks;
  std::vector<int32_t> next, prev;  // free queue links, -1 = none
  std::vector<uint8_t> in_free;
  int32_t head = -1, tail = -1, num_free = 0;
  std::unordered_map<uint64_t, int32_t> index;
  std::unordered_map<int64_t, Seq> seqs;
  int64_t stats[5] = {0, 0, 0, 0, 0};
  uint64_t epoch = 0;                         // counts batched appends
  mutable std::vector<uint8_t> scratch;       // hash serialisation buffer
  std::vector<Seq*> rows;                     // a batch's sequences, reused
  mutable std::vector<const Seq*> crows;      // the same for read-only calls

  pa_block_manager(int32_t nb, int32_t bs)
      : num_blocks(nb), block_size(bs), blocks(nb), next(nb), prev(nb), in_free(nb, 0) {
    for (int32_t b = 0; b < nb; ++b) push_tail(b);
    index.reserve(static_cast<size_t>(nb) * 2);
  }

  void push_tail(int32_t b) {
    prev[b] = tail;
    next[b] = -1;
    if (tail >= 0) next[tail] = b; else head = b;
    tail = b;
    in_free[b] = 1;
    ++num_free;
  }

  void unlink(int32_t b) {
    if (prev[b] >= 0) next[prev[b]] = next[b]; else head = next[b];
    if (next[b] >= 0) prev[next[b]] = prev[b]; else tail = prev[b];
    prev[b] = next[b] = -1;
    in_free[b] = 0;
    --num_free;
  }

  // Hands out the head of the free queue as a fresh block: its old cache entry,
  // if the index still points at it, is dropped.
  int32_t take_fresh() {
    const int32_t b = head;
    unlink(b);
    Block& blk = blocks[b];
    if (blk.hashed) {
      auto it = index.find(blk.hash);
      if (it != index.end() && it->second == b) {
        index.erase(it);
        ++stats[4];
      }
    }
    blk.hashed = false;
    blk.has_parent = false;
    blk.hash = blk.parent = 0;
    blk.tokens.clear();
    blk.ref = 1;
    return b;
  }

  void register_block(int32_t b, uint64_t h, bool has_parent, uint64_t parent,
                      const int32_t* tokens) {
    Block& blk = blocks[b];
    blk.hashed = true;
    blk.has_parent = has_parent;
    blk.hash = h;
    blk.parent = parent;
    blk.tokens.assign(tokens, tokens + block_size);
    index[h] = b;
  }

  // The cached block holding exactly (parent, tokens) under hash h, or -1.
  int32_t lookup(uint64_t h, bool has_parent, uint64_t parent, const int32_t* tokens) const {
    auto it = index.find(h);
    if (it == index.end()) return -1;
    const Block& blk = blocks[it->second];
    if (blk.has_parent != has_parent || (has_parent && blk.parent != parent)) return -1;
    if (std::memcmp(blk.tokens.data(), tokens, sizeof(int32_t) * block_size) != 0) return -1;
    return it->second;
  }

  // Decides each logical block's case for a prompt without changing state.
  // Fills plan/hit_block/hashes; returns the number of free blocks it takes.
  int64_t plan_allocation(const int32_t* tokens, int32_t n, std::vector<Plan>& plan,
                          std::vector<int32_t>& hit_block, std::vector<uint64_t>& hashes) const {
    const int32_t nblk = (n + block_size - 1) / block_size;
    const int32_t nfull = n / block_size;
    plan.assign(nblk, Plan::kFresh);
    hit_block.assign(nblk, -1);
    hashes.assign(nfull, 0);
    int64_t need = 0;
    bool missed = false;
    for (int32_t i = 0; i < nblk; ++i) {
      const int32_t* blk_tokens = tokens + static_cast<int64_t>(i) * block_size;
      if (i < nfull) {
        hashes[i] = chained_hash(scratch, i > 0, i > 0 ? hashes[i - 1] : 0, blk_tokens,
                                 block_size);
      }
      // The block with the last token is always fresh.
      const bool last = (i == nblk - 1);
      if (!missed && !last && i < nfull) {
        const int32_t b = lookup(hashes[i], i > 0, i > 0 ? hashes[i - 1] : 0, blk_tokens);
        if (b >= 0) {
          hit_block[i] = b;
          plan[i] = blocks[b].ref > 0 ? Plan::kShare : Plan::kTakeBack;
          if (plan[i] == Plan::kTakeBack) ++need;
          continue;
        }
      }
      missed = true;
      ++need;
    }
    return need;
  }
};

namespace {

inline int32_t slot_of(const pa_block_manager* bm, const Seq& s, int32_t pos) {
  return s.table[pos / bm->block_size] * bm->block_size + pos % bm->block_size;
}

}  // namespace

extern "C" {

uint64_t pa_xxh64(const void* data, size_t len, uint64_t seed) {
  static const uint8_t kEmpty = 0;
  return xxh64(len ? static_cast<const uint8_t*>(data) : &kEmpty, len, seed);
}

uint64_t pa_block_hash(uint64_t parent, int32_t has_parent, const int32_t* tokens,
                       int32_t num_tokens) {
  std::vector<uint8_t> buf;
  return chained_hash(buf, has_parent != 0, parent, tokens, num_tokens < 0 ? 0 : num_tokens);
}

pa_block_manager* pa_bm_create(int32_t num_blocks, int32_t block_size) {
  if (num_blocks < 1 || block_size < 1) return nullptr;
  return new (std::nothrow) pa_block_manager(num_blocks, block_size);
}

void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

int32_t pa_bm_num_free_blocks(const pa_block_manager* bm) { return bm ? bm->num_free : 0; }

int pa_bm_can_allocate(const pa_block_manager* bm, const int32_t* tokens, int32_t num_tokens,
                       int32_t* ok) {
  if (!bm || !ok) return PA_ERR_NULL;
  if (num_tokens < 1) return PA_ERR_SHAPE;
  if (!tokens) return PA_ERR_NULL;
  std::vector<Plan> plan;
  std::vector<int32_t> hit;
  std::vector<uint64_t> hashes;
  *ok = bm->plan_allocation(tokens, num_tokens, plan, hit, hashes) <= bm->num_free ? 1 : 0;
  return PA_OK;
}

int pa_bm_allocate(pa_block_manager* bm, int64_t seq_id, const int32_t* tokens,
                   int32_t num_tokens, int32_t* num_cached_tokens) {
  if (!bm) return PA_ERR_NULL;
  if (num_tokens < 1) return PA_ERR_SHAPE;
  if (!tokens) return PA_ERR_NULL;
  if (bm->seqs.count(seq_id)) return PA_ERR_SEQ;
  std::vector<Plan> plan;
  std::vector<int32_t> hit;
  std::vector<uint64_t> hashes;
  if (bm->plan_allocation(tokens, num_tokens, plan, hit, hashes) > bm->num_free)
    return PA_ERR_NO_BLOCKS;

  Seq s;
  s.tokens.assign(tokens, tokens + num_tokens);
  s.hashes = hashes;
  const int32_t nblk = static_cast<int32_t>(plan.size());
  s.table.reserve(nblk);
  const int32_t bs = bm->block_size;
  for (int32_t i = 0; i < nblk; ++i) {
    int32_t b;
    switch (plan[i]) {
      case Plan::kShare:
        b = hit[i];
        ++bm->blocks[b].ref;
        ++bm->stats[0];
        s.cached += bs;
        break;
      case Plan::kTakeBack:
        b = hit[i];
        bm->unlink(b);
        bm->blocks[b].ref = 1;
        ++bm->stats[1];
        s.cached += bs;
        break;
      default:
        b = bm->take_fresh();
        ++bm->stats[2];
        if (i < static_cast<int32_t>(hashes.size()))
          bm->register_block(b, hashes[i], i > 0, i > 0 ? hashes[i - 1] : 0,
                             tokens + static_cast<int64_t>(i) * bs);
        break;
    }
    s.table.push_back(b);
  }
  if (num_cached_tokens) *num_cached_tokens = s.cached;
  bm->seqs.emplace(seq_id, std::move(s));
  return PA_OK;
}

int pa_bm_can_append(const pa_block_manager* bm, int64_t seq_id, int32_t* ok) {
  if (!bm || !ok) return PA_ERR_NULL;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PA_ERR_SEQ;
  const bool needs_block = it->second.tokens.size() % bm->block_size == 0;
  *ok = (!needs_block || bm->num_free > 0) ? 1 : 0;
  return PA_OK;
}

}  // extern "C"

namespace {

// Appends one token; the caller has checked that a block is free if needed.
void append_token(pa_block_manager* bm, Seq& s, int32_t token) {
  const int32_t bs = bm->block_size;
  const int64_t len_before = static_cast<int64_t>(s.tokens.size());
  if (len_before % bs == 0) {
    s.table.push_back(bm->take_fresh());
    ++bm->stats[3];
  }
  s.tokens.push_back(token);
  const int64_t len = len_before + 1;
  if (len % bs == 0) {
    const int64_t i = len / bs - 1;
    const bool has_parent = i > 0;
    const uint64_t parent = has_parent ? s.hashes[i - 1] : 0;
    const int32_t* blk_tokens = s.tokens.data() + i * bs;
    const uint64_t h = chained_hash(bm->scratch, has_parent, parent, blk_tokens, bs);
    s.hashes.push_back(h);
    bm->register_block(s.table[i], h, has_parent, parent, blk_tokens);
  }
}

}  // namespace

extern "C" {

int pa_bm_append(pa_block_manager* bm, int64_t seq_id, int32_t token) {
  if (!bm) return PA_ERR_NULL;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PA_ERR_SEQ;
  if (it->second.tokens.size() % bm->block_size == 0 && bm->num_free == 0)
    return PA_ERR_NO_BLOCKS;
  append_token(bm, it->second, token);
  return PA_OK;
}

int pa_bm_append_batch(pa_block_manager* bm, const int64_t* seq_ids, const int32_t* tokens,
                       int32_t batch) {
  if (!bm) return PA_ERR_NULL;
  if (batch < 0) return PA_ERR_SHAPE;
  if (batch == 0) return PA_OK;
  if (!seq_ids || !tokens) return PA_ERR_NULL;
  std::vector<Seq*>& rows = bm->rows;
  rows.resize(batch);
  const uint64_t epoch = ++bm->epoch;
  int64_t need = 0;
  for (int32_t b = 0; b < batch; ++b) {
    auto it = bm->seqs.find(seq_ids[b]);
    if (it == bm->seqs.end() || it->second.stamp == epoch) return PA_ERR_SEQ;
    rows[b] = &it->second;
    rows[b]->stamp = epoch;
    if (rows[b]->tokens.size() % bm->block_size == 0) ++need;
  }
  if (need > bm->num_free) return PA_ERR_NO_BLOCKS;
  for (int32_t b = 0; b < batch; ++b) append_token(bm, *rows[b], tokens[b]);
  return PA_OK;
}

int pa_bm_deallocate(pa_block_manager* bm, int64_t seq_id) {
  if (!bm) return PA_ERR_NULL;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PA_ERR_SEQ;
  const std::vector<int32_t>& table = it->second.table;
  for (auto b = table.rbegin(); b != table.rend(); ++b) {
    if (--bm->blocks[*b].ref == 0) bm->push_tail(*b);
  }
  bm->seqs.erase(it);
  return PA_OK;
}

int pa_bm_seq_info(const pa_block_manager* bm, int64_t seq_id, int32_t* num_tokens,
                   int32_t* num_cached_tokens, int32_t* num_blocks) {
  if (!bm) return PA_ERR_NULL;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PA_ERR_SEQ;
  if (num_tokens) *num_tokens = static_cast<int32_t>(it->second.tokens.size());
  if (num_cached_tokens) *num_cached_tokens = it->second.cached;
  if (num_blocks) *num_blocks = static_cast<int32_t>(it->second.table.size());
  return PA_OK;
}

int pa_bm_block_table(const pa_block_manager* bm, int64_t seq_id, int32_t* out,
                      int32_t capacity) {
  if (!bm || !out) return PA_ERR_NULL;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PA_ERR_SEQ;
  const std::vector<int32_t>& table = it->second.table;
  if (capacity < static_cast<int64_t>(table.size())) return PA_ERR_SHAPE;
  std::memcpy(out, table.data(), sizeof(int32_t) * table.size());
  return PA_OK;
}

int pa_bm_block_info(const pa_block_manager* bm, int32_t block, int32_t* ref_count,
                     int32_t* cached, uint64_t* hash) {
  if (!bm) return PA_ERR_NULL;
  if (block < 0 || block >= bm->num_blocks) return PA_ERR_SHAPE;
  const Block& blk = bm->blocks[block];
  bool indexed = false;
  if (blk.hashed) {
    auto it = bm->index.find(blk.hash);
    indexed = it != bm->index.end() && it->second == block;
  }
  if (ref_count) *ref_count = blk.ref;
  if (cached) *cached = indexed ? 1 : 0;
  if (hash) *hash = blk.hashed ? blk.hash : 0;
  return PA_OK;
}

int pa_bm_stats(const pa_block_manager* bm, int64_t* out) {
  if (!bm || !out) return PA_ERR_NULL;
  for (int i = 0; i < 5; ++i) out[i] = bm->stats[i];
  return PA_OK;
}

int pa_bm_batch_info(const pa_block_manager* bm, const int64_t* seq_ids, int32_t batch,
                     int64_t* new_tokens, int32_t* max_new_tokens, int32_t* max_len,
                     int32_t* max_blocks) {
  if (!bm) return PA_ERR_NULL;
  if (batch < 0) return PA_ERR_SHAPE;
  if (batch > 0 && !seq_ids) return PA_ERR_NULL;
  int64_t total = 0;
  int32_t mq = 0, ml = 0, mb = 0;
  for (int32_t b = 0; b < batch; ++b) {
    auto it = bm->seqs.find(seq_ids[b]);
    if (it == bm->seqs.end()) return PA_ERR_SEQ;
    const Seq& s = it->second;
    const int32_t len = static_cast<int32_t>(s.tokens.size());
    total += len - s.cached;
    mq = std::max(mq, len - s.cached);
    ml = std::max(ml, len);
    mb = std::max(mb, static_cast<int32_t>(s.table.size()));
  }
  if (new_tokens) *new_tokens = total;
  if (max_new_tokens) *max_new_tokens = mq;
  if (max_len) *max_len = ml;
  if (max_blocks) *max_blocks = mb;
  return PA_OK;
}

int pa_bm_prefill_metadata(const pa_block_manager* bm, const int64_t* seq_ids, int32_t batch,
                           int32_t* cu_seqlens_q, int32_t* context_lens,
                           int32_t* slot_mapping, int32_t slot_capacity, int32_t* block_table,
                           int32_t block_table_stride, int32_t* total_q,
                           int32_t* max_seqlen_q) {
  if (!bm || !cu_seqlens_q || !context_lens || !block_table) return PA_ERR_NULL;
  if (batch < 0 || slot_capacity < 0 || block_table_stride < 0) return PA_ERR_SHAPE;
  if (batch > 0 && !seq_ids) return PA_ERR_NULL;
  if (slot_capacity > 0 && !slot_mapping) return PA_ERR_NULL;
  // Check every sequence before writing anything.
  std::vector<const Seq*>& rows = bm->crows;
  rows.resize(batch);
  int64_t total = 0;
  int32_t max_q = 0;
  for (int32_t b = 0; b < batch; ++b) {
    auto it = bm->seqs.find(seq_ids[b]);
    if (it == bm->seqs.end()) return PA_ERR_SEQ;
    rows[b] = &it->second;
    if (static_cast<int64_t>(rows[b]->table.size()) > block_table_stride) return PA_ERR_SHAPE;
    const int32_t nq = static_cast<int32_t>(rows[b]->tokens.size()) - rows[b]->cached;
    total += nq;
    if (nq > max_q) max_q = nq;
  }
  if (total > slot_capacity) return PA_ERR_SHAPE;
  cu_seqlens_q[0] = 0;
  int32_t t = 0;
  for (int32_t b = 0; b < batch; ++b) {
    const Seq& s = *rows[b];
    const int32_t len = static_cast<int32_t>(s.tokens.size());
    const int32_t bs = bm->block_size;
    for (int32_t pos = s.cached; pos < len;) {  // one block at a time
      const int32_t base = s.table[pos / bs] * bs;
      const int32_t end = std::min(len, (pos / bs + 1) * bs);
      for (int32_t off = pos % bs; pos < end; ++pos, ++off) slot_mapping[t++] = base + off;
    }
    cu_seqlens_q[b + 1] = t;
    context_lens[b] = len;
    int32_t* row = block_table + static_cast<int64_t>(b) * block_table_stride;
    const int32_t nblk = static_cast<int32_t>(s.table.size());
    std::memcpy(row, s.table.data(), sizeof(int32_t) * nblk);
    for (int32_t j = nblk; j < block_table_stride; ++j) row[j] = -1;
  }
  for (int32_t j = t; j < slot_capacity; ++j) slot_mapping[j] = -1;
  if (total_q) *total_q = t;
  if (max_seqlen_q) *max_seqlen_q = max_q;
  return PA_OK;
}

int pa_bm_decode_metadata(const pa_block_manager* bm, const int64_t* seq_ids, int32_t batch,
                          int32_t padded_batch, int32_t* context_lens, int32_t* slot_mapping,
                          int32_t* block_table, int32_t block_table_stride,
                          int32_t* max_context_len) {
  if (!bm || !context_lens || !slot_mapping || !block_table) return PA_ERR_NULL;
  if (batch < 0 || padded_batch < batch || block_table_stride < 0) return PA_ERR_SHAPE;
  if (batch > 0 && !seq_ids) return PA_ERR_NULL;
  std::vector<const Seq*>& rows = bm->crows;
  rows.resize(batch);
  for (int32_t b = 0; b < batch; ++b) {
    auto it = bm->seqs.find(seq_ids[b]);
    if (it == bm->seqs.end()) return PA_ERR_SEQ;
    rows[b] = &it->second;
    if (static_cast<int64_t>(rows[b]->table.size()) > block_table_stride) return PA_ERR_SHAPE;
  }
  int32_t max_len = 0;
  for (int32_t b = 0; b < padded_batch; ++b) {
    int32_t* row = block_table + static_cast<int64_t>(b) * block_table_stride;
    int32_t nblk = 0;
    if (b < batch) {
      const Seq& s = *rows[b];
      const int32_t len = static_cast<int32_t>(s.tokens.size());
      context_lens[b] = len;
      slot_mapping[b] = slot_of(bm, s, len - 1);
      nblk = static_cast<int32_t>(s.table.size());
      std::memcpy(row, s.table.data(), sizeof(int32_t) * nblk);
      if (len > max_len) max_len = len;
    } else {
      context_lens[b] = 0;
      slot_mapping[b] = -1;
    }
    for (int32_t j = nblk; j < block_table_stride; ++j) row[j] = -1;
  }
  if (max_context_len) *max_context_len = max_len;
  return PA_OK;
}

int64_t pa_kv_cache_num_blocks(uint64_t total_bytes, uint64_t used_bytes, uint64_t peak_bytes,
                               uint64_t current_bytes, double utilization, int32_t num_layers,
                               int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                               int32_t dtype_bytes) {
  if (!(utilization > 0.0 && utilization <= 1.0) || num_layers < 1 || block_size < 1 ||
      num_kv_heads < 1 || head_dim < 1 || dtype_bytes < 1)
    return -1;
  // Exact in long double for any realistic device (64-bit mantissa).
  const long double available = static_cast<long double>(total_bytes) * utilization -
                                static_cast<long double>(used_bytes) -
                                static_cast<long double>(peak_bytes) +
                                static_cast<long double>(current_bytes);
  const long double block_bytes = 2.0L * num_layers * block_size * num_kv_heads * head_dim *
                                  dtype_bytes;
  if (available <= 0.0L) return 0;
  return static_cast<int64_t>(available / block_bytes);
}

}  // extern "C"

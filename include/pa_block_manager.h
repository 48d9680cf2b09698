/*
 * pa_block_manager.h -- host-side allocator of KV-cache blocks with prefix
 * caching, part of libpa.so. It produces the block_table, slot_mapping,
 * context_lens and cu_seqlens_q arrays that pa_store_kvcache, pa_decode and
 * pa_prefill_varlen (pa.h) consume.
 *
 * Behaviour follows:
 *   [Report] "nano-vllm 深度分析报告" (nightvoyager), section "创新之处",
 *            item on the BlockManager: one structure serves both paging and
 *            prefix caching; blocks are content-addressed by a 64-bit xxHash
 *            (XXH64) chained over the prompt, so each block's hash covers the
 *            hash of everything before it; allocate meets three cases (a
 *            cached block still in use is shared, a cached block already freed
 *            is taken back, otherwise a fresh block is handed out); may_append
 *            registers a block in the cache at the moment it fills.
 *            Table "可复用的模式与技巧", row "xxhash64 链式哈希 KV Cache"
 *            (the chained hash makes a block's identity depend on its
 *            position in the prompt).
 *   [QbitAI] "DeepSeek研究员1200行代码复刻vLLM…", section "vLLM是什么？"
 *            (a sequence's logical blocks map to physical blocks through its
 *            block table).
 *
 * Where the pages leave a rule open, this library takes these readings:
 *   - Hash of logical block i of a sequence, over its block_size token ids:
 *       h_0 = XXH64(tokens_0, seed 0)
 *       h_i = XXH64(le64(h_{i-1}) || tokens_i, seed 0)          (i > 0)
 *     with every token id written as a little-endian int32. Only full blocks
 *     get a hash; a partial block is never looked up or registered.
 *   - A cached block matches only if its stored token ids and stored parent
 *     hash equal the candidate's, so a 64-bit collision of h_i alone cannot
 *     alias two different blocks.
 *   - The cached prefix is contiguous: after the first block that misses, the
 *     rest of the sequence misses too.
 *   - The block that holds a sequence's last token is always a fresh block,
 *     so at least one token is recomputed and no prefill writes into a block
 *     another sequence shares.
 *   - Free blocks form a queue. Fresh blocks come from its head; a freed
 *     block goes to its tail (a sequence frees its blocks last to first, so a
 *     prefix outlives its tail); a freed block keeps its hash until it is
 *     handed out fresh, when its cache entry is dropped. Registering a hash
 *     that is already cached points the entry at the newer block.
 *
 * Ownership: the caller owns every array it passes; the manager copies what
 * it keeps. All arrays are HOST memory. A manager is not thread-safe: calls on
 * one handle must not overlap. Sequence ids are any int64 the caller chooses,
 * unique among live sequences. A call that returns an error changes nothing.
 */
#ifndef PA_BLOCK_MANAGER_H
#define PA_BLOCK_MANAGER_H

#include <stddef.h>
#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_block_manager pa_block_manager;

/*
 * XXH64 of `len` bytes at `data` with `seed`, from the published xxHash
 * specification (algorithm XXH64). data may be NULL when len == 0.
 */
uint64_t pa_xxh64(const void* data, size_t len, uint64_t seed);

/*
 * The chained hash of one full block: XXH64(le64(parent) || le32 tokens) when
 * has_parent != 0, else XXH64(le32 tokens); both with seed 0.
 */
uint64_t pa_block_hash(uint64_t parent, int32_t has_parent, const int32_t* tokens,
                       int32_t num_tokens);

/*
 * Creates a manager of num_blocks physical blocks of block_size tokens each
 * (num_blocks >= 1, block_size >= 1). Block ids are 0 .. num_blocks-1 and the
 * free queue starts in that order. Returns NULL on bad sizes or out of memory.
 */
pa_block_manager* pa_bm_create(int32_t num_blocks, int32_t block_size);

/* Frees the manager (NULL is ignored). */
void pa_bm_destroy(pa_block_manager* bm);

/* Number of blocks in the free queue (cached ones included). */
int32_t pa_bm_num_free_blocks(const pa_block_manager* bm);

/*
 * Would pa_bm_allocate succeed for these tokens? Writes 1 or 0 to *ok.
 * It counts exactly the blocks the allocation would take from the free queue
 * (fresh blocks and freed cached blocks taken back; shared blocks cost none).
 */
int pa_bm_can_allocate(const pa_block_manager* bm, const int32_t* tokens, int32_t num_tokens,
                       int32_t* ok);

/*
 * Gives sequence seq_id (not live yet) the blocks for its num_tokens >= 1
 * tokens, reusing cached prefix blocks. *num_cached_tokens (if non-NULL)
 * receives the number of leading tokens whose K/V is already in the pool (a
 * multiple of block_size); prefill then computes only the rest.
 * PA_ERR_NO_BLOCKS if the free queue is too short, PA_ERR_SEQ if seq_id is
 * live, PA_ERR_SHAPE if num_tokens < 1.
 */
int pa_bm_allocate(pa_block_manager* bm, int64_t seq_id, const int32_t* tokens,
                   int32_t num_tokens, int32_t* num_cached_tokens);

/*
 * Would appending one token to seq_id succeed? (It needs a free block exactly
 * when the sequence's length is a multiple of block_size.) Writes 1 or 0.
 */
int pa_bm_can_append(const pa_block_manager* bm, int64_t seq_id, int32_t* ok);

/*
 * Appends one generated token to seq_id (the "may_append" step): takes a fresh
 * block when the token starts a new block, and registers the block's chained
 * hash when the token fills it. Call it before the decode step that stores the
 * token's K/V. PA_ERR_NO_BLOCKS if a block is needed and none is free.
 */
int pa_bm_append(pa_block_manager* bm, int64_t seq_id, int32_t token);

/*
 * One decode step's appends: tokens[i] is appended to seq_ids[i] for every i
 * in [0, batch), as pa_bm_append does, in order. The ids must be live and
 * distinct (else PA_ERR_SEQ), and the blocks the step needs must all be free
 * (else PA_ERR_NO_BLOCKS); either failure is detected before any append, so
 * the call appends to all sequences or to none.
 */
int pa_bm_append_batch(pa_block_manager* bm, const int64_t* seq_ids, const int32_t* tokens,
                       int32_t batch);

/*
 * Ends seq_id: drops one reference from each of its blocks, last block first;
 * blocks whose count reaches zero join the tail of the free queue with their
 * cache entries kept. PA_ERR_SEQ if seq_id is not live.
 */
int pa_bm_deallocate(pa_block_manager* bm, int64_t seq_id);

/*
 * Length, cached-prefix length and block count of a live sequence (any
 * output pointer may be NULL). PA_ERR_SEQ if it is not live.
 */
int pa_bm_seq_info(const pa_block_manager* bm, int64_t seq_id, int32_t* num_tokens,
                   int32_t* num_cached_tokens, int32_t* num_blocks);

/*
 * Copies seq_id's block table (ceil(len/block_size) physical block ids) to
 * out[0 .. capacity). PA_ERR_SHAPE if capacity is smaller.
 */
int pa_bm_block_table(const pa_block_manager* bm, int64_t seq_id, int32_t* out,
                      int32_t capacity);

/*
 * Reference count, whether the block carries a cache entry of its own (1) or
 * not (0), and its hash (0 when it has none) of physical block `block`.
 */
int pa_bm_block_info(const pa_block_manager* bm, int32_t block, int32_t* ref_count,
                     int32_t* cached, uint64_t* hash);

/*
 * Running totals since creation, written to out[0..5):
 *   [0] blocks shared (cached and in use: reference count raised),
 *   [1] blocks taken back (cached and free: removed from the free queue),
 *   [2] fresh blocks handed out by pa_bm_allocate,
 *   [3] fresh blocks handed out by pa_bm_append,
 *   [4] cache entries dropped because their block was handed out fresh.
 */
int pa_bm_stats(const pa_block_manager* bm, int64_t* out);

/*
 * Sizes of a batch of live sequences, for sizing metadata buffers (any output
 * pointer may be NULL): the total and largest count of tokens past the cached
 * prefix (prefill query rows), the largest length and the largest block count.
 * PA_ERR_SEQ for an id that is not live.
 */
int pa_bm_batch_info(const pa_block_manager* bm, const int64_t* seq_ids, int32_t batch,
                     int64_t* new_tokens, int32_t* max_new_tokens, int32_t* max_len,
                     int32_t* max_blocks);

/*
 * Builds the metadata of a prefill batch over live sequences seq_ids[0..batch)
 * (normally just allocated): sequence b contributes its tokens past the cached
 * prefix, N_b = len - num_cached_tokens, as query rows.
 *   cu_seqlens_q    [batch+1]: running sum of N_b, starting at 0.
 *   context_lens    [batch]: len of each sequence.
 *   slot_mapping    [slot_capacity]: the pool slot of each query row's token,
 *                   in row order; entries past total_q are set to -1.
 *   block_table     [batch][block_table_stride]: each sequence's physical
 *                   blocks, the rest of the row set to -1.
 *   *total_q, *max_seqlen_q (may be NULL): sum and maximum of N_b.
 * PA_ERR_SHAPE if slot_capacity < total_q or a table does not fit the stride;
 * PA_ERR_SEQ for an id that is not live.
 */
int pa_bm_prefill_metadata(const pa_block_manager* bm, const int64_t* seq_ids, int32_t batch,
                           int32_t* cu_seqlens_q, int32_t* context_lens,
                           int32_t* slot_mapping, int32_t slot_capacity, int32_t* block_table,
                           int32_t block_table_stride, int32_t* total_q,
                           int32_t* max_seqlen_q);

/*
 * Builds the metadata of a decode step over live sequences seq_ids[0..batch),
 * padded to padded_batch >= batch rows (a captured batch size): row b < batch
 * gets context_lens[b] = len and slot_mapping[b] = the slot of the sequence's
 * last token (the one this step stores); padding rows get context length 0,
 * slot -1 and a block-table row of -1 ([Report], table
 * "可复用的模式与技巧", row "slot_mapping -1 padding").
 *   context_lens, slot_mapping  [padded_batch];
 *   block_table                 [padded_batch][block_table_stride];
 *   *max_context_len (may be NULL): the largest len.
 */
int pa_bm_decode_metadata(const pa_block_manager* bm, const int64_t* seq_ids, int32_t batch,
                          int32_t padded_batch, int32_t* context_lens, int32_t* slot_mapping,
                          int32_t* block_table, int32_t block_table_stride,
                          int32_t* max_context_len);

/*
 * How many KV blocks fit in device memory after a warm-up run.
 * [Report] "nano-vllm 深度分析报告", section "创新之处" (the dynamic KV-cache
 * sizing item) and table "可复用的模式与技巧", row "warmup → peak → 分配": run
 * one warm-up step, record the allocator's peak, and budget
 *     available = total * utilization - used - peak + current
 * bytes, where -peak + current removes what the warm-up's temporaries took.
 *   total_bytes    device memory size;
 *   used_bytes     device memory in use now (total - free);
 *   peak_bytes     the allocator's peak during the warm-up;
 *   current_bytes  the allocator's current allocation after the warm-up;
 *   utilization    fraction of the device to plan for (the pages use 0.9).
 * One block holds K and V of block_size tokens for every layer:
 *     block_bytes = 2 * num_layers * block_size * num_kv_heads * head_dim * dtype_bytes.
 * Returns floor(available / block_bytes), 0 if available <= 0, or -1 on bad
 * arguments (a size < 1, or utilization outside (0, 1]).
 */
int64_t pa_kv_cache_num_blocks(uint64_t total_bytes, uint64_t used_bytes, uint64_t peak_bytes,
                               uint64_t current_bytes, double utilization, int32_t num_layers,
                               int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                               int32_t dtype_bytes);

#ifdef __cplusplus
}
#endif

#endif /* PA_BLOCK_MANAGER_H */

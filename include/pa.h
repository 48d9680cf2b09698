/*
 * pa.h -- C ABI of libpa.so, paged KV-cache attention for AMD Instinct MI355X
 * (gfx950).
 *
 * The operations follow two pages:
 *   [QbitAI] "DeepSeek研究员1200行代码复刻vLLM，H800硬件实测性能反超原版"
 *            (163.com), section "vLLM是什么？": PagedAttention splits the KV
 *            cache into fixed-size blocks, maps each sequence's logical blocks
 *            to physical blocks through a block table, and the attention kernel
 *            fetches each KV block separately.
 *   [Report] "nano-vllm 深度分析报告" (nightvoyager): table "可复用的模式与技巧",
 *            row "slot_mapping -1 padding" (padding positions carry -1 in
 *            slot_mapping and the KV-store kernel skips them); table
 *            "关键设计决策", row "block_size=256" (nano-vLLM uses 256-token
 *            blocks where vLLM uses 16); section "创新之处" (prefix caching
 *            shares cached blocks between sequences).
 *
 * Conventions shared by every call:
 *   - Pointers named k, v, q, out, *_cache and workspace are DEVICE pointers
 *     (hipMalloc'd or torch CUDA tensors). bf16 buffers are passed as void*:
 *     each element is the 16-bit bfloat16 bit pattern. Metadata arrays
 *     (slot_mapping, block_table, context_lens, cu_seqlens_q) are int32 device
 *     arrays, except in pa_validate_metadata, which reads host arrays.
 *   - KV pool layout (one pool for K, one for V):
 *         [num_blocks][block_size][num_kv_heads][head_dim]   bf16, row-major.
 *     Token slot s = physical_block * block_size + offset_in_block; the
 *     (slot, kv_head) row of head_dim elements starts at element
 *     (s * num_kv_heads + kv_head) * head_dim.
 *   - GQA: query head h reads kv head h / (num_q_heads / num_kv_heads).
 *   - The caller owns every buffer. No call allocates, frees or synchronises;
 *     each one only enqueues kernels on `stream` (a hipStream_t; NULL = the
 *     default stream) and returns. Kernel faults surface at the caller's next
 *     synchronisation.
 *   - Scalar arguments are checked on the host; a call that fails a check
 *     enqueues nothing. Device metadata (block ids, slots, lengths) is NOT
 *     read on the host: keeping it in range is the caller's contract, and
 *     pa_validate_metadata checks a host copy of it.
 *   - Supported shapes: head_dim == 128; block_size a power of two in
 *     [16, 256]; num_q_heads / num_kv_heads in {1, 2, 4, 8}. bf16 device
 *     buffers must be 16-byte aligned. The softmax scale of pa_decode and
 *     pa_prefill_varlen must be positive and finite (else PA_ERR_SHAPE).
 *   - All calls are safe to enqueue from several host threads on different
 *     streams; there is no global state beyond the cached device properties.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every int-returning call. */
#define PA_OK 0
#define PA_ERR_NULL (-1)        /* a required pointer is NULL                   */
#define PA_ERR_SHAPE (-2)       /* inconsistent or negative sizes, bad metadata */
#define PA_ERR_UNSUPPORTED (-3) /* valid but unsupported shape or alignment     */
#define PA_ERR_WORKSPACE (-4)   /* workspace missing or smaller than required   */
#define PA_ERR_HIP (-5)         /* the HIP runtime reported an error on launch  */
#define PA_ERR_NO_BLOCKS (-6)   /* block manager: not enough free blocks        */
#define PA_ERR_SEQ (-7)         /* block manager: sequence id unknown or in use */
#define PA_ERR_SCRATCH (-8)     /* pa_decode_store_noalloc: beyond its scratch   */

/* Static text for a status code (never NULL). [not on the pages: library
 * plumbing, no operation of the method] */
const char* pa_status_string(int status);

/*
 * pa_store_kvcache -- write new tokens' K and V into the paged pools.
 * [Report], table "可复用的模式与技巧", row "slot_mapping -1 padding".
 *
 *   For each token i in [0, num_tokens) with s = slot_mapping[i]:
 *     s == -1 : nothing is written (a padding position);
 *     s >= 0  : the num_kv_heads*head_dim bf16 words of k[i] and v[i] are
 *               copied bit for bit to slot s of k_cache and v_cache.
 *
 *   k, v            [num_tokens][kv_token_stride] bf16; the first
 *                   num_kv_heads*head_dim elements of each row are the token's
 *                   K (resp. V) laid out [num_kv_heads][head_dim]. A stride
 *                   larger than num_kv_heads*head_dim lets the caller pass
 *                   slices of a fused QKV projection output. kv_token_stride
 *                   must be a multiple of 8.
 *   k_cache,v_cache pools, [num_blocks][block_size][num_kv_heads][head_dim].
 *   slot_mapping    [num_tokens] int32, each -1 or in [0, num_blocks*block_size).
 *   Two tokens naming the same slot is undefined (one of them wins).
 *   num_tokens == 0 is valid and enqueues nothing.
 */
int pa_store_kvcache(const void* k, const void* v, int64_t kv_token_stride,
                     void* k_cache, void* v_cache, const int32_t* slot_mapping,
                     int32_t num_tokens, int32_t num_blocks, int32_t block_size,
                     int32_t num_kv_heads, int32_t head_dim, void* stream);

/*
 * [not on the pages: the pages give no split of a long context across the
 * GPU; this sizes the split-K partials of pa_decode's own design.]
 * Bytes of device workspace pa_decode needs for these sizes: a small header,
 * then per working wavefront the merge job of the boundary where its range of
 * the work starts, and two partial (acc, max, sum) records per query head,
 * for the (sequence, kv head) pairs its range cuts. The bound
 * depends on min(batch, 1024) (longer batches run in consecutive launches
 * that reuse the workspace), num_q_heads and max_context_len only; block_size
 * and head_dim are accepted for symmetry. 0 only for batch <= 0.
 */
size_t pa_decode_workspace_bytes(int32_t batch, int32_t num_q_heads,
                                 int32_t head_dim, int32_t max_context_len,
                                 int32_t block_size);

/*
 * pa_decode -- one query token per sequence attends over its paged context.
 * [QbitAI], section "vLLM是什么？" (block-table addressed KV blocks).
 *
 *   For row b with L = context_lens[b] and query head h (kv head g = h/G):
 *     key/value j in [0, L) live at slot
 *        block_table[b*block_table_stride + j/block_size]*block_size + j%block_size;
 *     s_j = scale * <q[b,h,:], K_j[g,:]>,
 *     out[b,h,:] = sum_j softmax(s)_j V_j[g,:]      (fp32 math, bf16 RNE out).
 *   L counts the new token, which must already be in the pool (store it with
 *   pa_store_kvcache first, on the same stream). L == 0 marks a padding row:
 *   its output is written as zeros and its block_table row is not read.
 *
 *   out, q          [batch][num_q_heads][head_dim] bf16.
 *   block_table     [batch][block_table_stride] int32; only the first
 *                   ceil(L/block_size) entries of a row are read.
 *   context_lens    [batch] int32, each in [0, max_context_len].
 *   max_context_len host-side upper bound of context_lens (sizes the grid);
 *                   ceil(max_context_len/block_size) <= block_table_stride.
 *   workspace       device scratch of at least pa_decode_workspace_bytes(...)
 *                   bytes, 256-byte aligned; its contents need no
 *                   initialisation and are garbage afterwards. Two calls in
 *                   flight at once must not share a workspace.
 *   The result is bitwise independent of which physical blocks hold the
 *   context (the summation order follows logical positions only).
 */
int pa_decode(void* out, const void* q, const void* k_cache,
              const void* v_cache, const int32_t* block_table,
              int32_t block_table_stride, const int32_t* context_lens,
              int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
              int32_t head_dim, int32_t block_size, int32_t max_context_len,
              float scale, void* workspace, size_t workspace_bytes,
              void* stream);

/*
 * pa_decode_store -- the decode step in one call: pa_store_kvcache of the
 * step's new tokens fused into pa_decode (one decode launch and its merge
 * instead of a separate store launch before them).
 * [Report] "nano-vllm 深度分析报告", table "可复用的模式与技巧" (the store
 * of each step's K/V through slot_mapping, -1 skipped); [QbitAI], section
 * "vLLM是什么？" (block-table addressed KV blocks).
 *
 *   Same result, bit for bit (output and pools), as
 *     pa_store_kvcache(k_new, v_new, kv_token_stride, k_cache, v_cache,
 *                      slot_mapping, batch, num_blocks, block_size, ...);
 *     pa_decode(out, q, k_cache, v_cache, block_table, ..., context_lens, ...);
 *   under the decode-step layout of slot_mapping: for a live row
 *   (context_lens[b] > 0) slot_mapping[b] is the slot of its position
 *   context_lens[b] - 1 (the new token), or -1 when that token is already in
 *   the pool; for a padding row (context_lens[b] == 0) it is -1. Other
 *   layouts are undefined (the separate calls handle any slot_mapping).
 *   The decode launch reads each new token from k_new/v_new; the merge
 *   launch after it writes the rows into their slots; nothing else in the
 *   call reads those slots.
 *
 *   k_new, v_new  [batch][kv_token_stride] bf16, first num_kv_heads*head_dim
 *                 used; kv_token_stride a multiple of 8.
 *   k_cache, v_cache are read and written; the other arguments, the workspace
 *   and the errors are as for pa_store_kvcache and pa_decode.
 */
int pa_decode_store(void* out, const void* q, const void* k_new, const void* v_new,
                    int64_t kv_token_stride, void* k_cache, void* v_cache,
                    const int32_t* slot_mapping, const int32_t* block_table,
                    int32_t block_table_stride, const int32_t* context_lens, int32_t batch,
                    int32_t num_blocks, int32_t num_q_heads, int32_t num_kv_heads,
                    int32_t head_dim, int32_t block_size, int32_t max_context_len, float scale,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_store_noalloc -- pa_decode_store without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).
 *
 *   Same arguments, result (output and pools, bit for bit) and errors as
 *   pa_decode_store, minus workspace/workspace_bytes. The split-K records live
 *   in a file-scope device array of 16 MiB inside libpa.so, one copy per GPU,
 *   held until the process ends; the call allocates nothing (no hipMalloc,
 *   hipFree or allocating library routine), and its first call on a device
 *   looks up that device's copy (hipGetSymbolAddress) and keeps the address.
 *   A call needing more scratch than 16 MiB returns PA_ERR_SCRATCH and
 *   enqueues nothing; on a 256-CU MI355X every batch, head count and context
 *   length fits (at most ~8.7 MB is used: the records are bounded by the
 *   launch grid, one work-group per compute unit). Every call on one GPU
 *   shares that GPU's array, so calls that overlap on one GPU (concurrent
 *   streams, or host threads without ordering) race; calls ordered on one
 *   stream do not. Nothing in the array needs clearing between calls.
 */
int pa_decode_store_noalloc(void* out, const void* q, const void* k_new, const void* v_new,
                            int64_t kv_token_stride, void* k_cache, void* v_cache,
                            const int32_t* slot_mapping, const int32_t* block_table,
                            int32_t block_table_stride, const int32_t* context_lens,
                            int32_t batch, int32_t num_blocks, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                            int32_t max_context_len, float scale, void* stream);

/*
 * pa_prefill_varlen -- causal attention for a batch of variable-length
 * prompts whose leading blocks may come from the prefix cache.
 * [QbitAI] "vLLM是什么？" (paging) and [Report] "创新之处" (prefix caching).
 *
 *   Sequence b owns query rows t in [cu_seqlens_q[b], cu_seqlens_q[b+1]):
 *   its N_b new tokens. Its context holds L_b = context_lens[b] tokens: a
 *   cached prefix of P_b = L_b - N_b tokens followed by the new ones, all
 *   already in the pool (store the new ones with pa_store_kvcache first).
 *   New row i (0-based) sits at position P_b + i and sees keys 0 .. P_b + i
 *   (causal mask aligned to the end of the context):
 *     out[t,h,:] = sum_{j <= P_b+i} softmax(scale*<q[t,h,:],K_j[g,:]>) V_j[g,:].
 *
 *   out, q          [total_q][num_q_heads][head_dim] bf16,
 *                   total_q == cu_seqlens_q[batch].
 *   cu_seqlens_q    [batch+1] int32, non-decreasing, cu_seqlens_q[0] == 0.
 *   context_lens    [batch] int32, context_lens[b] >= N_b.
 *   block_table     [batch][block_table_stride] int32.
 *   max_seqlen_q    host-side upper bound of every N_b (sizes the grid).
 *   A sequence with N_b == 0 produces no rows.
 */
int pa_prefill_varlen(void* out, const void* q, const void* k_cache,
                      const void* v_cache, const int32_t* cu_seqlens_q,
                      const int32_t* context_lens, const int32_t* block_table,
                      int32_t block_table_stride, int32_t batch,
                      int32_t total_q, int32_t max_seqlen_q,
                      int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t head_dim, int32_t block_size, float scale,
                      void* stream);

/*
 * pa_validate_metadata -- host-side check of the metadata contract.
 * [not on the pages: a test aid; the pages state the metadata (block table,
 * slot_mapping with -1) but no checks of it.]
 * All pointers are HOST arrays; nothing touches the GPU. Checks that every
 * context length is in [0, max_context_len] (max_context_len < 0 skips that
 * bound), that every block-table entry a row reads is in [0, num_blocks), that
 * no physical block is read by a row twice, that slot_mapping entries are -1
 * or in [0, num_blocks*block_size) with no valid slot repeated, and, when
 * cu_seqlens_q is given, that it is non-decreasing from 0 with
 * N_b <= context_lens[b]. cu_seqlens_q and slot_mapping may be NULL.
 * Returns PA_OK or PA_ERR_SHAPE; on failure writes a message into `detail`
 * (if non-NULL, up to detail_len bytes including the terminator).
 */
int pa_validate_metadata(const int32_t* block_table, int32_t block_table_stride,
                         const int32_t* context_lens, int32_t batch,
                         const int32_t* cu_seqlens_q,
                         const int32_t* slot_mapping, int32_t num_slots,
                         int32_t num_blocks, int32_t block_size,
                         int32_t max_context_len, char* detail,
                         size_t detail_len);

/*
 * pa_sample_gumbel -- draw one token per row from per-row probabilities by
 * Gumbel-max sampling: the index of the largest p / E with E ~ Exp(1).
 * [Report] "nano-vllm 深度分析报告", section "创新之处" (the Gumbel-Max item:
 * divide the probabilities by Exp(1) draws and take the argmax instead of a
 * multinomial draw) and table "可复用的模式与技巧", row "Gumbel-Max 采样".
 *
 *   For row b and element i < vocab, with x the 32-bit word i mod 4 of
 *   Philox4x32-10 (Salmon et al., SC'11) at counter
 *   (i / 4, b, offset mod 2^32, offset / 2^32) and key (seed mod 2^32, seed / 2^32):
 *     u   = ((x >> 9) + 1/2) * 2^-23            (exact fp32, in (0, 1))
 *     E   = -log2(u)                            (a positive multiple of an Exp(1)
 *                                                variable: same argmax)
 *     key = p[b,i] / E                          (fp32; the kernel uses hardware
 *                                                log2 and reciprocal, within ~2
 *                                                ulp of exactly rounded steps)
 *     tokens[b] = the index of the largest key, the smallest index among equal
 *                 keys (a row of zeros gives 0).
 *   The same (seed, offset) gives the same draws; use a new offset per step.
 *
 *   probs      [batch][row_stride] fp32 device array, 4-byte aligned,
 *              row_stride >= vocab (rows that start 16-byte aligned, i.e. a
 *              16-byte aligned base and row_stride a multiple of 4, are read
 *              with 16-byte loads); entries must be non-negative and finite
 *              (they need not sum to 1: the draw is proportional to p).
 *   tokens     [batch] int32 device array.
 *   workspace  device scratch of pa_sample_workspace_bytes(batch, vocab)
 *              bytes, 8-byte aligned; no initialisation needed.
 *   batch in [0, 65535]; vocab >= 1. batch == 0 enqueues nothing.
 */
size_t pa_sample_workspace_bytes(int32_t batch, int32_t vocab);

int pa_sample_gumbel(int32_t* tokens, const float* probs, int64_t row_stride, int32_t batch,
                     int32_t vocab, uint64_t seed, uint64_t offset, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * Decode-step graphs: one HIP graph per batch-size bucket, each holding a
 * whole decode step (the launches of pa_decode_store: the decode kernel,
 * which reads the step's new tokens from their input rows, then the merge,
 * which also writes them into the pools) captured once and replayed with a
 * single launch.
 * [Report] "nano-vllm 深度分析报告", section "创新之处" (graph capture at a
 * few batch sizes only, a batch rounded up to the next captured size, captured
 * from the largest size down with one memory pool shared by all graphs) and
 * table "可复用的模式与技巧", rows on the discrete batch sizes and on
 * slot_mapping -1 padding.
 *
 * Every graph reads and writes the same caller-owned device buffers, sized for
 * the largest bucket; that single set of buffers is what the shared pool is in
 * the pages, and the graphs allocate no device memory of their own. Before a
 * replay for `batch` rows the caller writes rows [0, bucket) of the inputs,
 * with rows past `batch` as padding: context length 0 and slot -1 (what
 * pa_bm_decode_metadata writes for padded_batch = bucket); their q, k_new and
 * v_new rows may hold anything finite and their output rows come back zero.
 * A live row's slot is the slot of its new token (position context_lens[b]
 * - 1) or -1, the layout pa_decode_store requires (pa_bm_decode_metadata
 * writes it).
 * Rows [0, bucket) of `out` are written. Every context length of a replay
 * must be <= max_context_len given at creation.
 */
typedef struct pa_decode_step_buffers {
  void* out;                   /* [B][num_q_heads][head_dim] bf16                */
  const void* q;               /* [B][num_q_heads][head_dim] bf16                */
  const void* k_new;           /* [B][kv_token_stride] bf16 (first Hkv*D used)   */
  const void* v_new;           /* [B][kv_token_stride] bf16                      */
  int64_t kv_token_stride;     /* multiple of 8, >= num_kv_heads*head_dim       */
  void* k_cache;               /* [num_blocks][block_size][Hkv][head_dim] bf16   */
  void* v_cache;
  const int32_t* slot_mapping; /* [B]                                            */
  const int32_t* context_lens; /* [B]                                            */
  const int32_t* block_table;  /* [B][block_table_stride]                        */
  int32_t block_table_stride;
  void* workspace;             /* >= pa_decode_workspace_bytes(B, Hq, D, max_context_len, bs) */
  size_t workspace_bytes;
  int32_t num_blocks, block_size, num_q_heads, num_kv_heads, head_dim;
  int32_t max_context_len;     /* bound of every replay's context lengths       */
  float scale;                 /* softmax scale, positive and finite            */
} pa_decode_step_buffers;
/* B = the largest bucket. */

typedef struct pa_decode_graphs pa_decode_graphs;

/*
 * Captures one graph per bucket, largest first. buckets[0..num_buckets) must
 * be strictly increasing and >= 1; buckets == NULL means 1, 2, 4, ..., 512.
 * The buffers are checked as pa_store_kvcache and pa_decode check theirs, for
 * the largest bucket. Nothing runs on the GPU during creation (capture only
 * records). Creation allocates host-side graph objects, not device memory; it
 * must not itself be called inside a stream capture. *graphs receives the
 * handle (NULL on failure).
 */
int pa_decode_graphs_create(const pa_decode_step_buffers* buffers, const int32_t* buckets,
                            int32_t num_buckets, pa_decode_graphs** graphs);

/* The smallest bucket >= batch (1 <= batch <= the largest), else PA_ERR_SHAPE. */
int pa_decode_graphs_bucket(const pa_decode_graphs* graphs, int32_t batch, int32_t* bucket);

/*
 * Enqueues the decode step of `batch` rows on `stream` (NULL = the default
 * stream) as one launch of the graph of its bucket; batch == 0 enqueues
 * nothing, batch above the largest bucket is PA_ERR_SHAPE. Replays of graphs
 * of one handle share the buffers: replays in flight at once on different
 * streams race.
 */
int pa_decode_graphs_launch(pa_decode_graphs* graphs, int32_t batch, void* stream);

/* Frees the graphs (NULL is ignored). Call it when no replay is in flight. */
void pa_decode_graphs_destroy(pa_decode_graphs* graphs);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */

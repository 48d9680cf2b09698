// Paged-attention ORACLE — test infrastructure only.
//
// This file is a plain, slow CPU implementation of what the paged-attention
// path computes. It exists so that the GPU library can be checked against
// something obviously correct. Only the test-suite, the smoke check and the
// CPU-baseline leg of the benchmark load it. The product library never links,
// loads or calls it, and it shares no code, header or helper with that library.
//
// Sources (the pages this follows):
//   [QbitAI] "DeepSeek研究员1200行代码复刻vLLM，H800硬件实测性能反超原版"
//            (163.com), section "vLLM是什么？": the KV cache is cut into
//            fixed-size blocks; a block table maps each sequence's logical
//            blocks to physical blocks; the attention kernel fetches the
//            blocks one by one. Paging moves where keys and values live, not
//            what attention computes, so the oracle gathers the blocks back
//            into logical order and runs textbook softmax attention in fp64.
//   [Report] "nano-vllm 深度分析报告" (nightvoyager), table
//            "可复用的模式与技巧", row "slot_mapping -1 padding": positions
//            marked -1 in slot_mapping are skipped by the KV-store kernel.
//            Same page, table "关键设计决策": block_size 256 (vLLM uses 16).
//
// Readings where the pages are silent (each one is listed in the design
// notes of the repository):
//   * pool layout: K and V are each [num_blocks, block_size, Hkv, D] bf16,
//     and slot = physical_block * block_size + offset_in_block;
//   * GQA grouping: query head h reads kv head h / (Hq / Hkv);
//   * causal prefill with a cached prefix of P = L - N tokens: new query row
//     i (0-based among the N new rows) sees keys 0 .. P + i;
//   * a decode row with context_len 0 is a padding row; its output is zero.
//
// All arithmetic on values is fp64. bf16 -> fp64 is exact. Sums run in
// ascending index order. No blocking, fusion or reordering.
//
// Build: g++ -O2 -std=c++17 -shared -fPIC -pthread oracle.cpp -o liboracle.so

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

namespace {

// Status codes of the oracle (its own, unrelated to any other library's).
constexpr int kOk = 0;
constexpr int kBadArg = 1;      // null pointer or impossible size
constexpr int kBadMeta = 2;     // metadata out of range (block id, slot, length)

// bf16 is the top half of an IEEE binary32; widening it is exact.
double bf16_to_double(uint16_t bits) {
  uint32_t w = static_cast<uint32_t>(bits) << 16;
  float f;
  std::memcpy(&f, &w, sizeof f);
  return static_cast<double>(f);
}

// Runs fn(item) for item in [0, n) on `nthreads` threads (1 = serial).
template <class Fn>
void parallel_for(int64_t n, int nthreads, Fn fn) {
  if (nthreads <= 1 || n <= 1) {
    for (int64_t i = 0; i < n; ++i) fn(i);
    return;
  }
  std::atomic<int64_t> next{0};
  std::vector<std::thread> pool;
  for (int t = 0; t < nthreads; ++t) {
    pool.emplace_back([&] {
      for (;;) {
        int64_t i = next.fetch_add(1);
        if (i >= n) break;
        fn(i);
      }
    });
  }
  for (auto& th : pool) th.join();
}

// Logical token j of a sequence -> pool slot, through that sequence's row of
// the block table ([QbitAI], "vLLM是什么？": logical block -> physical block).
// Returns -1 when the table entry or the slot is out of range.
int64_t slot_of(const int32_t* table_row, int32_t j, int32_t block_size,
                int32_t num_blocks) {
  int32_t logical_block = j / block_size;
  int32_t offset = j % block_size;
  int32_t physical = table_row[logical_block];
  if (physical < 0 || physical >= num_blocks) return -1;
  return static_cast<int64_t>(physical) * block_size + offset;
}

// Softmax attention of one query over L gathered keys/values, fp64.
//   s_j = scale * sum_d q[d] * K[j][d]
//   w_j = exp(s_j - max_j s_j),  o[d] = sum_j w_j V[j][d] / sum_j w_j
// K and V are [L][D] in logical order.
void attend(const std::vector<double>& q, const std::vector<double>& K,
            const std::vector<double>& V, int32_t L, int32_t D, double scale,
            double* out) {
  if (L == 0) {
    for (int32_t d = 0; d < D; ++d) out[d] = 0.0;
    return;
  }
  std::vector<double> s(L);
  for (int32_t j = 0; j < L; ++j) {
    double acc = 0.0;
    for (int32_t d = 0; d < D; ++d) acc += q[d] * K[static_cast<size_t>(j) * D + d];
    s[j] = scale * acc;
  }
  double m = s[0];
  for (int32_t j = 1; j < L; ++j) m = s[j] > m ? s[j] : m;
  double Z = 0.0;
  for (int32_t j = 0; j < L; ++j) {
    s[j] = std::exp(s[j] - m);
    Z += s[j];
  }
  for (int32_t d = 0; d < D; ++d) {
    double acc = 0.0;
    for (int32_t j = 0; j < L; ++j) acc += s[j] * V[static_cast<size_t>(j) * D + d];
    out[d] = acc / Z;
  }
}

// Gathers the first L tokens of kv head g of one sequence into logical order.
int gather(const uint16_t* cache, const int32_t* table_row, int32_t L,
           int32_t g, int32_t Hkv, int32_t D, int32_t block_size,
           int32_t num_blocks, std::vector<double>& dst) {
  dst.assign(static_cast<size_t>(L) * D, 0.0);
  for (int32_t j = 0; j < L; ++j) {
    int64_t slot = slot_of(table_row, j, block_size, num_blocks);
    if (slot < 0) return kBadMeta;
    const uint16_t* src = cache + (slot * Hkv + g) * D;
    for (int32_t d = 0; d < D; ++d)
      dst[static_cast<size_t>(j) * D + d] = bf16_to_double(src[d]);
  }
  return kOk;
}

}  // namespace

extern "C" {

// KV store ([Report], "slot_mapping -1 padding"): for each new token i with
// s = slot_mapping[i] >= 0, the bf16 words of k[i] and v[i] (Hkv*D each) are
// copied bit for bit into slot s of the pools; tokens with s = -1 are skipped.
// k and v rows are kv_token_stride elements apart. The copy runs in token
// order, so with duplicate slots the last token wins (the GPU leaves that
// case undefined; the generated inputs never contain it).
int oracle_store_kvcache(const uint16_t* k, const uint16_t* v,
                         int64_t kv_token_stride, uint16_t* k_cache,
                         uint16_t* v_cache, const int32_t* slot_mapping,
                         int32_t num_tokens, int32_t num_blocks,
                         int32_t block_size, int32_t num_kv_heads,
                         int32_t head_dim) {
  if (num_tokens < 0 || num_blocks < 0 || block_size <= 0 ||
      num_kv_heads <= 0 || head_dim <= 0)
    return kBadArg;
  if (num_tokens == 0) return kOk;
  if (!k || !v || !k_cache || !v_cache || !slot_mapping) return kBadArg;
  const int64_t row = static_cast<int64_t>(num_kv_heads) * head_dim;
  const int64_t num_slots = static_cast<int64_t>(num_blocks) * block_size;
  for (int32_t i = 0; i < num_tokens; ++i) {
    int64_t s = slot_mapping[i];
    if (s == -1) continue;
    if (s < 0 || s >= num_slots) return kBadMeta;
    for (int64_t e = 0; e < row; ++e) {
      k_cache[s * row + e] = k[i * kv_token_stride + e];
      v_cache[s * row + e] = v[i * kv_token_stride + e];
    }
  }
  return kOk;
}

// Paged decode ([QbitAI], "vLLM是什么？"): one query token per sequence b,
// attending over its context_lens[b] cached tokens (the new token included,
// already stored). q and out are [batch, Hq, D]; out is fp64.
// rows/num_rows: optional subset of b to compute (null = all rows); rows not
// listed are left untouched in out. nthreads: worker threads over (b, h).
int oracle_decode(double* out, const uint16_t* q, const uint16_t* k_cache,
                  const uint16_t* v_cache, const int32_t* block_table,
                  int32_t block_table_stride, const int32_t* context_lens,
                  int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                  int32_t head_dim, int32_t block_size, int32_t num_blocks,
                  double scale, const int32_t* rows, int32_t num_rows,
                  int32_t nthreads) {
  if (batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      block_size <= 0 || num_blocks < 0 || num_q_heads % num_kv_heads != 0)
    return kBadArg;
  if (!rows) num_rows = batch;
  if (num_rows == 0) return kOk;
  if (!out || !q || !k_cache || !v_cache || !block_table || !context_lens)
    return kBadArg;
  const int32_t group = num_q_heads / num_kv_heads;
  const int32_t D = head_dim;
  for (int32_t r = 0; r < num_rows; ++r) {
    int32_t b = rows ? rows[r] : r;
    if (b < 0 || b >= batch) return kBadArg;
    int32_t L = context_lens[b];
    if (L < 0 || (L > 0 && (L - 1) / block_size >= block_table_stride))
      return kBadMeta;
    const int32_t* table_row = block_table + static_cast<int64_t>(b) * block_table_stride;
    for (int32_t j = 0; j < L; j += block_size) {
      int32_t p = table_row[j / block_size];
      if (p < 0 || p >= num_blocks) return kBadMeta;
    }
  }
  std::atomic<int> status{kOk};
  parallel_for(static_cast<int64_t>(num_rows) * num_q_heads, nthreads, [&](int64_t item) {
    int32_t r = static_cast<int32_t>(item / num_q_heads);
    int32_t h = static_cast<int32_t>(item % num_q_heads);
    int32_t b = rows ? rows[r] : r;
    int32_t g = h / group;
    int32_t L = context_lens[b];
    const int32_t* table_row = block_table + static_cast<int64_t>(b) * block_table_stride;
    std::vector<double> K, V, qv(D);
    if (gather(k_cache, table_row, L, g, num_kv_heads, D, block_size, num_blocks, K) != kOk ||
        gather(v_cache, table_row, L, g, num_kv_heads, D, block_size, num_blocks, V) != kOk) {
      status = kBadMeta;
      return;
    }
    const uint16_t* qrow = q + (static_cast<int64_t>(b) * num_q_heads + h) * D;
    for (int32_t d = 0; d < D; ++d) qv[d] = bf16_to_double(qrow[d]);
    attend(qv, K, V, L, D, scale, out + (static_cast<int64_t>(b) * num_q_heads + h) * D);
  });
  return status.load();
}

// Varlen causal prefill with a cached prefix ([QbitAI], "vLLM是什么？" for the
// paging; [QbitAI] feature list and [Report] "创新之处" for prefix caching):
// sequence b owns query rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 (its N new
// tokens) and context_lens[b] = P + N cached-plus-new tokens in the pool, the
// new ones already stored. New row i sees keys 0 .. P + i. q and out are
// [total_q, Hq, D]; out is fp64.
// tokens/num_tokens: optional subset of global query rows to compute (null =
// all rows); rows not listed are left untouched in out.
int oracle_prefill(double* out, const uint16_t* q, const uint16_t* k_cache,
                   const uint16_t* v_cache, const int32_t* cu_seqlens_q,
                   const int32_t* context_lens, const int32_t* block_table,
                   int32_t block_table_stride, int32_t batch, int32_t total_q,
                   int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                   int32_t block_size, int32_t num_blocks, double scale,
                   const int32_t* tokens, int32_t num_tokens, int32_t nthreads) {
  if (batch < 0 || total_q < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      head_dim <= 0 || block_size <= 0 || num_blocks < 0 ||
      num_q_heads % num_kv_heads != 0)
    return kBadArg;
  if (!tokens) num_tokens = total_q;
  if (num_tokens == 0) return kOk;
  if (!out || !q || !k_cache || !v_cache || !cu_seqlens_q || !context_lens ||
      !block_table)
    return kBadArg;
  if (cu_seqlens_q[0] != 0 || cu_seqlens_q[batch] != total_q) return kBadMeta;
  for (int32_t b = 0; b < batch; ++b) {
    int32_t N = cu_seqlens_q[b + 1] - cu_seqlens_q[b];
    int32_t L = context_lens[b];
    if (N < 0 || L < N) return kBadMeta;
    if (L > 0 && (L - 1) / block_size >= block_table_stride) return kBadMeta;
  }
  // Which sequence owns each global query row: a linear scan of cu_seqlens_q.
  std::vector<int32_t> owner(total_q);
  for (int32_t b = 0; b < batch; ++b)
    for (int32_t t = cu_seqlens_q[b]; t < cu_seqlens_q[b + 1]; ++t) owner[t] = b;
  for (int32_t r = 0; r < num_tokens; ++r) {
    int32_t t = tokens ? tokens[r] : r;
    if (t < 0 || t >= total_q) return kBadArg;
  }
  const int32_t group = num_q_heads / num_kv_heads;
  const int32_t D = head_dim;
  std::atomic<int> status{kOk};
  parallel_for(static_cast<int64_t>(num_tokens) * num_q_heads, nthreads, [&](int64_t item) {
    int32_t r = static_cast<int32_t>(item / num_q_heads);
    int32_t h = static_cast<int32_t>(item % num_q_heads);
    int32_t t = tokens ? tokens[r] : r;
    int32_t b = owner[t];
    int32_t N = cu_seqlens_q[b + 1] - cu_seqlens_q[b];
    int32_t P = context_lens[b] - N;
    int32_t i = t - cu_seqlens_q[b];
    int32_t visible = P + i + 1;  // keys 0 .. P + i
    int32_t g = h / group;
    const int32_t* table_row = block_table + static_cast<int64_t>(b) * block_table_stride;
    std::vector<double> K, V, qv(D);
    if (gather(k_cache, table_row, visible, g, num_kv_heads, D, block_size, num_blocks, K) != kOk ||
        gather(v_cache, table_row, visible, g, num_kv_heads, D, block_size, num_blocks, V) != kOk) {
      status = kBadMeta;
      return;
    }
    const uint16_t* qrow = q + (static_cast<int64_t>(t) * num_q_heads + h) * D;
    for (int32_t d = 0; d < D; ++d) qv[d] = bf16_to_double(qrow[d]);
    attend(qv, K, V, visible, D, scale, out + (static_cast<int64_t>(t) * num_q_heads + h) * D);
  });
  return status.load();
}

// Number of hardware threads the host reports (for the CPU-baseline line).
int32_t oracle_hardware_threads(void) {
  unsigned n = std::thread::hardware_concurrency();
  return n == 0 ? 1 : static_cast<int32_t>(n);
}

}  // extern "C"

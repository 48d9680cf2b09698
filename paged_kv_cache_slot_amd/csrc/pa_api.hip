// C ABI of libpa.so: host-side argument checks, then kernel launches on the
// caller's stream. Nothing here allocates device memory or synchronises; only
// the decode-step graphs create host-side graph objects (at creation). The
// operations and their sources are documented in include/pa.h.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <new>
#include <vector>

#include "pa.h"
#include "pa_internal.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool supported_block_size(int32_t bs) { return bs >= 16 && bs <= 256 && (bs & (bs - 1)) == 0; }

bool supported_group(int32_t hq, int32_t hkv) {
  const int32_t g = hq / hkv;
  return g == 1 || g == 2 || g == 4 || g == 8;
}

int from_hip(hipError_t e) { return e == hipSuccess ? PA_OK : PA_ERR_HIP; }

// The kernels track each row's maximum raw score, which is the maximum scaled
// score only for a positive scale.
bool valid_scale(float scale) { return scale > 0.f && std::isfinite(scale); }

// Checks shared by decode and prefill. Returns PA_OK or the first failure.
int check_heads(int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                int32_t block_size) {
  if (num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0)
    return PA_ERR_SHAPE;
  if (num_q_heads % num_kv_heads != 0) return PA_ERR_SHAPE;
  if (head_dim != pa::kHeadDim || !supported_block_size(block_size) ||
      !supported_group(num_q_heads, num_kv_heads))
    return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

void write_detail(char* detail, size_t len, const char* msg) {
  if (detail && len > 0) {
    std::strncpy(detail, msg, len - 1);
    detail[len - 1] = '\0';
  }
}

}  // namespace

extern "C" {

const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "a required pointer is NULL";
    case PA_ERR_SHAPE: return "inconsistent or negative sizes";
    case PA_ERR_UNSUPPORTED: return "unsupported shape or alignment";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_HIP: return "HIP launch error";
    case PA_ERR_NO_BLOCKS: return "not enough free KV blocks";
    case PA_ERR_SEQ: return "sequence id unknown or already live";
    case PA_ERR_SCRATCH:
      return "the call needs more than the fixed 16 MiB device scratch of "
             "pa_decode_store_noalloc";
    default: return "unknown status";
  }
}

int pa_store_kvcache(const void* k, const void* v, int64_t kv_token_stride, void* k_cache,
                     void* v_cache, const int32_t* slot_mapping, int32_t num_tokens,
                     int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                     int32_t head_dim, void* stream) {
  if (num_tokens < 0 || num_blocks < 0 || block_size <= 0 || num_kv_heads <= 0 || head_dim <= 0)
    return PA_ERR_SHAPE;
  if (kv_token_stride < static_cast<int64_t>(num_kv_heads) * head_dim) return PA_ERR_SHAPE;
  if (head_dim != pa::kHeadDim || !supported_block_size(block_size)) return PA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  if (!k || !v || !k_cache || !v_cache || !slot_mapping) return PA_ERR_NULL;
  if (kv_token_stride % 8 != 0 || !aligned16(k) || !aligned16(v) || !aligned16(k_cache) ||
      !aligned16(v_cache))
    return PA_ERR_UNSUPPORTED;
  return from_hip(pa::launch_store_kvcache(
      static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), kv_token_stride,
      static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache), slot_mapping, num_tokens,
      num_kv_heads, static_cast<hipStream_t>(stream)));
}

size_t pa_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t head_dim,
                                 int32_t max_context_len, int32_t block_size) {
  (void)head_dim;
  (void)block_size;
  if (batch <= 0 || num_q_heads <= 0 || max_context_len < 0) return 0;
  return pa::decode_workspace_bytes(batch, num_q_heads, max_context_len);
}

int pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_table, int32_t block_table_stride,
              const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
              int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
              int32_t max_context_len, float scale, void* workspace, size_t workspace_bytes,
              void* stream) {
  if (batch < 0 || max_context_len < 0 || block_table_stride < 0 || !valid_scale(scale))
    return PA_ERR_SHAPE;
  int st = check_heads(num_q_heads, num_kv_heads, head_dim, block_size);
  if (st != PA_OK) return st;
  if (static_cast<int64_t>(block_table_stride) * block_size < max_context_len)
    return PA_ERR_SHAPE;
  if (batch == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_table || !context_lens) return PA_ERR_NULL;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return PA_ERR_UNSUPPORTED;
  const size_t need = pa::decode_workspace_bytes(batch, num_q_heads, max_context_len);
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return PA_ERR_WORKSPACE;
  return from_hip(pa::launch_decode(
      static_cast<uint16_t*>(out), static_cast<const uint16_t*>(q),
      static_cast<const uint16_t*>(k_cache), static_cast<const uint16_t*>(v_cache), block_table,
      block_table_stride, context_lens, batch, num_q_heads, num_kv_heads, block_size,
      max_context_len, scale, workspace, pa::FusedStore{}, static_cast<hipStream_t>(stream)));
}

int pa_decode_store(void* out, const void* q, const void* k_new, const void* v_new,
                    int64_t kv_token_stride, void* k_cache, void* v_cache,
                    const int32_t* slot_mapping, const int32_t* block_table,
                    int32_t block_table_stride, const int32_t* context_lens, int32_t batch,
                    int32_t num_blocks, int32_t num_q_heads, int32_t num_kv_heads,
                    int32_t head_dim, int32_t block_size, int32_t max_context_len, float scale,
                    void* workspace, size_t workspace_bytes, void* stream) {
  if (batch < 0 || num_blocks < 0 || max_context_len < 0 || block_table_stride < 0 ||
      !valid_scale(scale))
    return PA_ERR_SHAPE;
  int st = check_heads(num_q_heads, num_kv_heads, head_dim, block_size);
  if (st != PA_OK) return st;
  if (static_cast<int64_t>(block_table_stride) * block_size < max_context_len)
    return PA_ERR_SHAPE;
  if (kv_token_stride < static_cast<int64_t>(num_kv_heads) * head_dim) return PA_ERR_SHAPE;
  if (batch == 0) return PA_OK;
  if (!out || !q || !k_new || !v_new || !k_cache || !v_cache || !slot_mapping || !block_table ||
      !context_lens)
    return PA_ERR_NULL;
  if (kv_token_stride % 8 != 0 || !aligned16(out) || !aligned16(q) || !aligned16(k_new) ||
      !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache))
    return PA_ERR_UNSUPPORTED;
  const size_t need = pa::decode_workspace_bytes(batch, num_q_heads, max_context_len);
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return PA_ERR_WORKSPACE;
  pa::FusedStore fs;
  fs.k_new = static_cast<const uint16_t*>(k_new);
  fs.v_new = static_cast<const uint16_t*>(v_new);
  fs.kv_stride = kv_token_stride;
  fs.slot_mapping = slot_mapping;
  fs.k_store = static_cast<uint16_t*>(k_cache);
  fs.v_store = static_cast<uint16_t*>(v_cache);
  return from_hip(pa::launch_decode(
      static_cast<uint16_t*>(out), static_cast<const uint16_t*>(q),
      static_cast<const uint16_t*>(k_cache), static_cast<const uint16_t*>(v_cache), block_table,
      block_table_stride, context_lens, batch, num_q_heads, num_kv_heads, block_size,
      max_context_len, scale, workspace, fs, static_cast<hipStream_t>(stream)));
}

int pa_decode_store_noalloc(void* out, const void* q, const void* k_new, const void* v_new,
                            int64_t kv_token_stride, void* k_cache, void* v_cache,
                            const int32_t* slot_mapping, const int32_t* block_table,
                            int32_t block_table_stride, const int32_t* context_lens,
                            int32_t batch, int32_t num_blocks, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                            int32_t max_context_len, float scale, void* stream) {
  if (batch < 0 || num_blocks < 0 || max_context_len < 0 || block_table_stride < 0 ||
      !valid_scale(scale))
    return PA_ERR_SHAPE;
  int st = check_heads(num_q_heads, num_kv_heads, head_dim, block_size);
  if (st != PA_OK) return st;
  if (static_cast<int64_t>(block_table_stride) * block_size < max_context_len)
    return PA_ERR_SHAPE;
  if (kv_token_stride < static_cast<int64_t>(num_kv_heads) * head_dim) return PA_ERR_SHAPE;
  if (batch == 0) return PA_OK;
  if (!out || !q || !k_new || !v_new || !k_cache || !v_cache || !slot_mapping || !block_table ||
      !context_lens)
    return PA_ERR_NULL;
  if (kv_token_stride % 8 != 0 || !aligned16(out) || !aligned16(q) || !aligned16(k_new) ||
      !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache))
    return PA_ERR_UNSUPPORTED;
  if (pa::decode_scratch_need(batch, num_q_heads, num_kv_heads, max_context_len) >
      pa::kDecodeScratchBytes)
    return PA_ERR_SCRATCH;
  void* scratch = nullptr;
  if (pa::decode_scratch(&scratch) != hipSuccess) return PA_ERR_HIP;
  pa::FusedStore fs;
  fs.k_new = static_cast<const uint16_t*>(k_new);
  fs.v_new = static_cast<const uint16_t*>(v_new);
  fs.kv_stride = kv_token_stride;
  fs.slot_mapping = slot_mapping;
  fs.k_store = static_cast<uint16_t*>(k_cache);
  fs.v_store = static_cast<uint16_t*>(v_cache);
  return from_hip(pa::launch_decode(
      static_cast<uint16_t*>(out), static_cast<const uint16_t*>(q),
      static_cast<const uint16_t*>(k_cache), static_cast<const uint16_t*>(v_cache), block_table,
      block_table_stride, context_lens, batch, num_q_heads, num_kv_heads, block_size,
      max_context_len, scale, scratch, fs, static_cast<hipStream_t>(stream)));
}

int pa_prefill_varlen(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* cu_seqlens_q, const int32_t* context_lens,
                      const int32_t* block_table, int32_t block_table_stride, int32_t batch,
                      int32_t total_q, int32_t max_seqlen_q, int32_t num_q_heads,
                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size, float scale,
                      void* stream) {
  if (batch < 0 || total_q < 0 || max_seqlen_q < 0 || block_table_stride <= 0 ||
      !valid_scale(scale))
    return PA_ERR_SHAPE;
  int st = check_heads(num_q_heads, num_kv_heads, head_dim, block_size);
  if (st != PA_OK) return st;
  if (batch == 0 || total_q == 0 || max_seqlen_q == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !cu_seqlens_q || !context_lens || !block_table)
    return PA_ERR_NULL;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return PA_ERR_UNSUPPORTED;
  return from_hip(pa::launch_prefill(
      static_cast<uint16_t*>(out), static_cast<const uint16_t*>(q),
      static_cast<const uint16_t*>(k_cache), static_cast<const uint16_t*>(v_cache), cu_seqlens_q,
      context_lens, block_table, block_table_stride, batch, max_seqlen_q, num_q_heads,
      num_kv_heads, block_size, scale, static_cast<hipStream_t>(stream)));
}

int pa_validate_metadata(const int32_t* block_table, int32_t block_table_stride,
                         const int32_t* context_lens, int32_t batch, const int32_t* cu_seqlens_q,
                         const int32_t* slot_mapping, int32_t num_slots, int32_t num_blocks,
                         int32_t block_size, int32_t max_context_len, char* detail,
                         size_t detail_len) {
  char msg[256];
  auto fail = [&](const char* text) {
    write_detail(detail, detail_len, text);
    return PA_ERR_SHAPE;
  };
  if (batch < 0 || num_slots < 0 || num_blocks < 0 || block_size <= 0 || block_table_stride < 0)
    return fail("negative size");
  if (batch > 0 && (!block_table || !context_lens)) return fail("block_table or context_lens is NULL");
  if (num_slots > 0 && !slot_mapping) return fail("slot_mapping is NULL");
  std::vector<int32_t> seen(static_cast<size_t>(num_blocks), -1);
  for (int32_t b = 0; b < batch; ++b) {
    const int32_t L = context_lens[b];
    if (L < 0 || (max_context_len >= 0 && L > max_context_len)) {
      std::snprintf(msg, sizeof msg, "context_lens[%d] = %d out of range", b, L);
      return fail(msg);
    }
    const int64_t nblk = (static_cast<int64_t>(L) + block_size - 1) / block_size;
    if (nblk > block_table_stride) {
      std::snprintf(msg, sizeof msg, "row %d needs %lld blocks > block_table_stride %d", b,
                    static_cast<long long>(nblk), block_table_stride);
      return fail(msg);
    }
    for (int64_t j = 0; j < nblk; ++j) {
      const int32_t p = block_table[static_cast<int64_t>(b) * block_table_stride + j];
      if (p < 0 || p >= num_blocks) {
        std::snprintf(msg, sizeof msg, "block_table[%d][%lld] = %d out of [0, %d)", b,
                      static_cast<long long>(j), p, num_blocks);
        return fail(msg);
      }
      if (seen[p] == b) {
        std::snprintf(msg, sizeof msg, "row %d reads physical block %d twice", b, p);
        return fail(msg);
      }
      seen[p] = b;
    }
    if (cu_seqlens_q) {
      if (b == 0 && cu_seqlens_q[0] != 0) return fail("cu_seqlens_q[0] != 0");
      const int32_t n = cu_seqlens_q[b + 1] - cu_seqlens_q[b];
      if (n < 0 || n > L) {
        std::snprintf(msg, sizeof msg, "sequence %d has %d new tokens and context %d", b, n, L);
        return fail(msg);
      }
    }
  }
  if (num_slots > 0) {
    const int64_t total = static_cast<int64_t>(num_blocks) * block_size;
    std::vector<uint8_t> used(static_cast<size_t>(total), 0);
    for (int32_t i = 0; i < num_slots; ++i) {
      const int32_t s = slot_mapping[i];
      if (s == -1) continue;
      if (s < 0 || s >= total) {
        std::snprintf(msg, sizeof msg, "slot_mapping[%d] = %d out of range", i, s);
        return fail(msg);
      }
      if (used[s]) {
        std::snprintf(msg, sizeof msg, "slot %d named twice in slot_mapping", s);
        return fail(msg);
      }
      used[s] = 1;
    }
  }
  write_detail(detail, detail_len, "ok");
  return PA_OK;
}

size_t pa_sample_workspace_bytes(int32_t batch, int32_t vocab) {
  return pa::sample_workspace_bytes(batch, vocab);
}

int pa_sample_gumbel(int32_t* tokens, const float* probs, int64_t row_stride, int32_t batch,
                     int32_t vocab, uint64_t seed, uint64_t offset, void* workspace,
                     size_t workspace_bytes, void* stream) {
  if (batch < 0 || vocab < 1 || row_stride < vocab) return PA_ERR_SHAPE;
  if (batch > 65535) return PA_ERR_UNSUPPORTED;
  if (batch == 0) return PA_OK;
  if (!tokens || !probs) return PA_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(probs) & 3u) return PA_ERR_UNSUPPORTED;
  const size_t need = pa::sample_workspace_bytes(batch, vocab);
  if (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 7u))
    return PA_ERR_WORKSPACE;
  return from_hip(pa::launch_sample(tokens, probs, row_stride, batch, vocab, seed, offset,
                                    workspace, static_cast<hipStream_t>(stream)));
}

// ------------------------------------------------------ decode-step graphs --

}  // extern "C"

struct pa_decode_graphs {
  pa_decode_step_buffers buf;
  std::vector<int32_t> buckets;          // increasing
  std::vector<hipGraph_t> graphs;        // one per bucket
  std::vector<hipGraphExec_t> execs;

  ~pa_decode_graphs() {
    for (hipGraphExec_t e : execs)
      if (e) (void)hipGraphExecDestroy(e);
    for (hipGraph_t g : graphs)
      if (g) (void)hipGraphDestroy(g);
  }
};

namespace {

// The checks pa_store_kvcache and pa_decode make, for `batch` rows of `b`.
int check_step_buffers(const pa_decode_step_buffers& b, int32_t batch) {
  if (b.block_table_stride <= 0 || b.max_context_len < 0 || b.num_blocks <= 0 ||
      !valid_scale(b.scale))
    return PA_ERR_SHAPE;
  int st = check_heads(b.num_q_heads, b.num_kv_heads, b.head_dim, b.block_size);
  if (st != PA_OK) return st;
  if (static_cast<int64_t>(b.block_table_stride) * b.block_size < b.max_context_len)
    return PA_ERR_SHAPE;
  if (b.kv_token_stride < static_cast<int64_t>(b.num_kv_heads) * b.head_dim)
    return PA_ERR_SHAPE;
  if (!b.out || !b.q || !b.k_new || !b.v_new || !b.k_cache || !b.v_cache || !b.slot_mapping ||
      !b.context_lens || !b.block_table)
    return PA_ERR_NULL;
  if (b.kv_token_stride % 8 != 0 || !aligned16(b.out) || !aligned16(b.q) ||
      !aligned16(b.k_new) || !aligned16(b.v_new) || !aligned16(b.k_cache) ||
      !aligned16(b.v_cache))
    return PA_ERR_UNSUPPORTED;
  const size_t need = pa::decode_workspace_bytes(batch, b.num_q_heads, b.max_context_len);
  if (!b.workspace || b.workspace_bytes < need || !aligned16(b.workspace))
    return PA_ERR_WORKSPACE;
  return PA_OK;
}

// Records the decode step for `batch` rows on `stream` (which is capturing):
// the decode and merge launches with the store fused, as pa_decode_store runs
// them.
hipError_t record_step(const pa_decode_step_buffers& b, int32_t batch, hipStream_t stream) {
  pa::FusedStore fs;
  fs.k_new = static_cast<const uint16_t*>(b.k_new);
  fs.v_new = static_cast<const uint16_t*>(b.v_new);
  fs.kv_stride = b.kv_token_stride;
  fs.slot_mapping = b.slot_mapping;
  fs.k_store = static_cast<uint16_t*>(b.k_cache);
  fs.v_store = static_cast<uint16_t*>(b.v_cache);
  return pa::launch_decode(
      static_cast<uint16_t*>(b.out), static_cast<const uint16_t*>(b.q),
      static_cast<const uint16_t*>(b.k_cache), static_cast<const uint16_t*>(b.v_cache),
      b.block_table, b.block_table_stride, b.context_lens, batch, b.num_q_heads,
      b.num_kv_heads, b.block_size, b.max_context_len, b.scale, b.workspace, fs, stream);
}

}  // namespace

extern "C" {

int pa_decode_graphs_create(const pa_decode_step_buffers* buffers, const int32_t* buckets,
                            int32_t num_buckets, pa_decode_graphs** graphs) {
  if (!graphs) return PA_ERR_NULL;
  *graphs = nullptr;
  if (!buffers) return PA_ERR_NULL;
  std::vector<int32_t> bk;
  if (!buckets) {
    for (int32_t x = 1; x <= 512; x *= 2) bk.push_back(x);
  } else {
    if (num_buckets < 1) return PA_ERR_SHAPE;
    bk.assign(buckets, buckets + num_buckets);
    for (size_t i = 0; i < bk.size(); ++i)
      if (bk[i] < 1 || (i > 0 && bk[i] <= bk[i - 1])) return PA_ERR_SHAPE;
  }
  const int st = check_step_buffers(*buffers, bk.back());
  if (st != PA_OK) return st;

  auto* g = new (std::nothrow) pa_decode_graphs();
  if (!g) return PA_ERR_HIP;
  g->buf = *buffers;
  g->buckets = bk;
  g->graphs.assign(bk.size(), nullptr);
  g->execs.assign(bk.size(), nullptr);
  pa::prepare_decode(buffers->num_q_heads, buffers->num_kv_heads);
  hipStream_t stream = nullptr;
  if (hipStreamCreateWithFlags(&stream, hipStreamNonBlocking) != hipSuccess) {
    delete g;
    return PA_ERR_HIP;
  }
  int rc = PA_OK;
  // Largest bucket first.
  for (size_t i = bk.size(); i-- > 0 && rc == PA_OK;) {
    if (hipStreamBeginCapture(stream, hipStreamCaptureModeThreadLocal) != hipSuccess) {
      rc = PA_ERR_HIP;
      break;
    }
    const hipError_t rec = record_step(g->buf, bk[i], stream);
    const hipError_t end = hipStreamEndCapture(stream, &g->graphs[i]);
    if (rec != hipSuccess || end != hipSuccess ||
        hipGraphInstantiate(&g->execs[i], g->graphs[i], nullptr, nullptr, 0) != hipSuccess)
      rc = PA_ERR_HIP;
  }
  (void)hipStreamDestroy(stream);
  if (rc != PA_OK) {
    delete g;
    return rc;
  }
  *graphs = g;
  return PA_OK;
}

int pa_decode_graphs_bucket(const pa_decode_graphs* graphs, int32_t batch, int32_t* bucket) {
  if (!graphs || !bucket) return PA_ERR_NULL;
  for (int32_t b : graphs->buckets)
    if (b >= batch && batch >= 1) {
      *bucket = b;
      return PA_OK;
    }
  return PA_ERR_SHAPE;
}

int pa_decode_graphs_launch(pa_decode_graphs* graphs, int32_t batch, void* stream) {
  if (!graphs) return PA_ERR_NULL;
  if (batch == 0) return PA_OK;
  for (size_t i = 0; i < graphs->buckets.size(); ++i)
    if (graphs->buckets[i] >= batch && batch >= 1)
      return from_hip(hipGraphLaunch(graphs->execs[i], static_cast<hipStream_t>(stream)));
  return PA_ERR_SHAPE;
}

void pa_decode_graphs_destroy(pa_decode_graphs* graphs) { delete graphs; }

}  // extern "C"

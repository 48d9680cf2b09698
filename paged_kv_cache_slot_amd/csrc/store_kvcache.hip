// KV store: copies each new token's K and V rows into the pool slot named by
// slot_mapping, skipping -1 entries ("nano-vllm 深度分析报告", table
// 可复用的模式与技巧, row "slot_mapping -1 padding").
//
// HBM-bound copy. A token's K (or V) row is num_kv_heads * 128 bf16 =
// num_kv_heads * 16 sixteen-byte vectors; each thread moves one vector of K and
// the matching vector of V, so a wavefront reads and writes whole 1 KiB runs.
#include "pa_internal.h"

namespace pa {
namespace {

__global__ __launch_bounds__(256) void store_kvcache_kernel(
    const uint4* __restrict__ k, const uint4* __restrict__ v, int64_t row_stride_vec,
    uint4* __restrict__ k_cache, uint4* __restrict__ v_cache,
    const int32_t* __restrict__ slot_mapping, int32_t num_tokens, int32_t vec_per_token) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t token = idx / vec_per_token;
  const int32_t e = static_cast<int32_t>(idx - token * vec_per_token);
  if (token >= num_tokens) return;
  const int32_t slot = slot_mapping[token];
  if (slot < 0) return;  // -1: a padding position, nothing is written
  const int64_t dst = static_cast<int64_t>(slot) * vec_per_token + e;
  const int64_t src = token * row_stride_vec + e;
  const uint4 kv = k[src];
  const uint4 vv = v[src];
  k_cache[dst] = kv;
  v_cache[dst] = vv;
}

}  // namespace

hipError_t launch_store_kvcache(const uint16_t* k, const uint16_t* v, int64_t kv_token_stride,
                                uint16_t* k_cache, uint16_t* v_cache,
                                const int32_t* slot_mapping, int32_t num_tokens,
                                int32_t num_kv_heads, hipStream_t stream) {
  const int32_t vec_per_token = num_kv_heads * (kHeadDim / 8);
  const int64_t threads = static_cast<int64_t>(num_tokens) * vec_per_token;
  const int64_t blocks = (threads + 255) / 256;
  hipLaunchKernelGGL(store_kvcache_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0,
                     stream, reinterpret_cast<const uint4*>(k), reinterpret_cast<const uint4*>(v),
                     kv_token_stride / 8, reinterpret_cast<uint4*>(k_cache),
                     reinterpret_cast<uint4*>(v_cache), slot_mapping, num_tokens, vec_per_token);
  return hipGetLastError();
}

}  // namespace pa

// Internal declarations and device helpers of libpa.so (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace pa {

// Every kernel is written for head_dim 128: one 256-byte (kv head) row per
// token, i.e. sixteen 16-byte vectors.
constexpr int kHeadDim = 128;


// Devices whose per-device launch data (occupancy, symbol addresses) is cached.
constexpr int kMaxDevices = 64;

// ------------------------------------------------------------------ launch --

hipError_t launch_store_kvcache(const uint16_t* k, const uint16_t* v, int64_t kv_token_stride,
                                uint16_t* k_cache, uint16_t* v_cache,
                                const int32_t* slot_mapping, int32_t num_tokens,
                                int32_t num_kv_heads, hipStream_t stream);

// A store fused into a decode (its decode and merge launches): row b's new
// token (position context_lens[b] - 1) has its K/V in row b of k_new/v_new
// (token stride kv_stride elements), which the decode launch reads, and goes
// into pool slot slot_mapping[b] (-1: already in the pool), which the merge
// launch writes. k_store/v_store are the pools decode reads. No fused store
// when slot_mapping is null.
struct FusedStore {
  const uint16_t* k_new = nullptr;
  const uint16_t* v_new = nullptr;
  int64_t kv_stride = 0;
  const int32_t* slot_mapping = nullptr;
  uint16_t* k_store = nullptr;
  uint16_t* v_store = nullptr;
};

hipError_t launch_decode(uint16_t* out, const uint16_t* q, const uint16_t* k_cache,
                         const uint16_t* v_cache, const int32_t* block_table,
                         int32_t block_table_stride, const int32_t* context_lens, int32_t batch,
                         int32_t num_q_heads, int32_t num_kv_heads, int32_t block_size,
                         int32_t max_context_len, float scale, void* workspace,
                         const FusedStore& fused, hipStream_t stream);

size_t decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t max_context_len);

// Fixed device scratch of the decode entry point that allocates nothing: a
// file-scope device array of this many bytes, one copy per device.
constexpr size_t kDecodeScratchBytes = size_t(16) << 20;

// Bytes of that scratch a decode of these sizes uses on the current device:
// the smaller of decode_workspace_bytes and the bound set by the launch grid,
// which never exceeds one work-group per resident slot of the device.
size_t decode_scratch_need(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                           int32_t max_context_len);

// Device address of the scratch array on the current device, looked up once
// per device with hipGetSymbolAddress (the array's name is only a host-side
// stand-in) and kept.
hipError_t decode_scratch(void** ptr);

size_t sample_workspace_bytes(int32_t batch, int32_t vocab);

hipError_t launch_sample(int32_t* tokens, const float* probs, int64_t row_stride, int32_t batch,
                         int32_t vocab, uint64_t seed, uint64_t offset, void* workspace,
                         hipStream_t stream);

// Runs the host-side queries launch_decode makes on first use for this head
// grouping (occupancy of its kernel on the current device), so that a later
// launch_decode inside a stream capture only records kernel launches.
void prepare_decode(int32_t num_q_heads, int32_t num_kv_heads);

hipError_t launch_prefill(uint16_t* out, const uint16_t* q, const uint16_t* k_cache,
                          const uint16_t* v_cache, const int32_t* cu_seqlens_q,
                          const int32_t* context_lens, const int32_t* block_table,
                          int32_t block_table_stride, int32_t batch, int32_t max_seqlen_q,
                          int32_t num_q_heads, int32_t num_kv_heads, int32_t block_size,
                          float scale, hipStream_t stream);

// ------------------------------------------------------------ device helpers --

constexpr float kLog2e = 1.4426950408889634f;

// bf16 bits -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t packed) {
  return __builtin_bit_cast(float, packed << 16);
}
__device__ __forceinline__ float bf16_hi(uint32_t packed) {
  return __builtin_bit_cast(float, packed & 0xffff0000u);
}

// fp32 -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v;
  v.x = static_cast<__bf16>(lo);
  v.y = static_cast<__bf16>(hi);
  return __builtin_bit_cast(uint32_t, v);
}

// DPP lane exchanges inside one row of 16 lanes.
template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), kCtrl, 0xf, 0xf,
                                                     false));
}
constexpr int kDppQuadSwap1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadSwap2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141; // lane i <- lane 7-i within 8
constexpr int kDppRowMirror = 0x140;     // lane i <- lane 15-i within 16

// Sum over the 16 lanes of a DPP row; every lane of the row gets the total.
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp<kDppQuadSwap1>(x);
  x += dpp<kDppQuadSwap2>(x);
  x += dpp<kDppRowHalfMirror>(x);
  x += dpp<kDppRowMirror>(x);
  return x;
}

// Dot product of two packed bf16 pairs, accumulated in fp32 (v_dot2c_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Streaming (non-temporal) 16-byte load: data read once does not displace
// reusable lines in the caches.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(static_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

}  // namespace pa

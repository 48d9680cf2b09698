// Varlen causal prefill over a paged KV cache with a cached prefix
// ("DeepSeek研究员1200行代码复刻vLLM…", section "vLLM是什么？" for the paging;
// "nano-vllm 深度分析报告", section 创新之处, for prefix caching).
//
// Sequence b has P cached tokens and N new ones (all stored in the pool); new
// row i sits at position P + i and attends to keys 0 .. P + i.
//
// Work split. One work-group (4 wavefronts) owns one (sequence, kv head,
// tile of 128/G new tokens) and all G query heads of that kv head: 128 query
// rows, 32 per wavefront. It walks the context in tiles of 64 keys, gathering
// each tile's K and V rows through the block table into LDS (V transposed),
// and runs flash-attention style:
//   S^T = K Q^T      bf16 MFMA 32x32x16, fp32 accumulate (per wavefront:
//                    64 keys x 32 rows), so each lane holds the scores of ONE
//                    query row and the row max/sum stay in-lane except for
//                    one exchange with the lane 32 apart;
//   p = exp2(s*scale*log2e - m), online rescaling of the output;
//   O^T += V^T P^T   bf16 MFMA 32x32x16 with P taken straight from the S^T
//                    accumulators (converted to bf16), and V^T read from LDS
//                    with keys ordered to match the accumulator layout.
// Tiles wholly above the causal diagonal are never visited; tiles wholly
// below it skip the mask.
//
// Roofline: MFMA (bf16). Algorithmic flops = 4 * Hq * 128 * sum over
// sequences of (N*P + N*(N+1)/2) (only the causal pairs).
#include <cmath>

#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kRows = 128;         // query rows (token, head) per work-group
constexpr int kKeys = 64;          // keys per tile
constexpr int kKStride = kHeadDim + 8;  // LDS row of K: 128 bf16 + 16 B pad
constexpr int kVStride = kKeys + 8;     // LDS row of V^T: 64 bf16 + 16 B pad

// Position of key k (0..63) in a V^T row. Within each group of 16 keys, bits 2
// and 3 are exchanged, so the eight keys a lane's accumulator rows hold for one
// 16-key MFMA step (keys 4h..4h+3 and 8+4h..8+4h+3, h = lane/32) sit together.
__device__ __forceinline__ int vt_col(int k) {
  return (k & ~0xc) | ((k & 0x4) << 1) | ((k & 0x8) >> 1);
}

__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int G>
__global__ __launch_bounds__(256, 2) void prefill_kernel(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ k_cache, const uint16_t* __restrict__ v_cache,
    const int32_t* __restrict__ cu_seqlens_q, const int32_t* __restrict__ context_lens,
    const int32_t* __restrict__ block_table, int32_t bt_stride, int32_t batch,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t log2_bs, int32_t q_tiles,
    float scale_log2) {
  constexpr int TQ = kRows / G;  // new tokens per work-group
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[kKeys * kKStride];
  __shared__ __attribute__((aligned(16))) uint16_t vt_lds[kHeadDim * kVStride];

  // Heaviest tiles (the last query tiles) are dispatched first.
  const int idx = blockIdx.x;
  const int b = idx % batch;
  const int rest = idx / batch;
  const int g = rest % num_kv_heads;
  const int qtile = q_tiles - 1 - rest / num_kv_heads;

  const int q0 = cu_seqlens_q[b];
  const int N = cu_seqlens_q[b + 1] - q0;
  const int tok0 = qtile * TQ;
  if (tok0 >= N) return;
  const int L = context_lens[b];
  const int P = L - N;
  if (P < 0) return;  // breaks the contract context_lens[b] >= N; nothing is read
  const int tok_end = min(N, tok0 + TQ);     // exclusive
  const int key_end = P + tok_end;           // keys [0, key_end) are visible to some row
  const int num_tiles = (key_end + kKeys - 1) / kKeys;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;   // this lane's query row within the wavefront
  const int half = lane >> 5;  // which half of the MFMA k-slices this lane holds

  // This lane's query row.
  const int row = wave * 32 + col;
  const int hh = row / TQ;
  const int tok = row % TQ;
  const int qpos = P + tok0 + tok;                      // absolute position
  const int qt = q0 + min(tok0 + tok, N - 1);           // clamped for loads
  const int head = g * G + hh;

  bf16x8_t qreg[kHeadDim / 16];
  {
    const uint16_t* qp = q + (static_cast<int64_t>(qt) * num_q_heads + head) * kHeadDim + half * 8;
#pragma unroll
    for (int ks = 0; ks < kHeadDim / 16; ++ks)
      qreg[ks] = *reinterpret_cast<const bf16x8_t*>(qp + ks * 16);
  }

  f32x16_t o[kHeadDim / 32];
#pragma unroll
  for (int db = 0; db < kHeadDim / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  float m = -INFINITY;  // running max (base 2) of this lane's row
  float lsum = 0.f;     // running sum over this lane's keys

  const int bs_mask = (1 << log2_bs) - 1;
  const int32_t* bt = block_table + static_cast<int64_t>(b) * bt_stride;
  const int64_t slot_stride = static_cast<int64_t>(num_kv_heads) * kHeadDim;
  const uint16_t* kbase = k_cache + g * kHeadDim;
  const uint16_t* vbase = v_cache + g * kHeadDim;

  // Global -> register staging of one tile.
  // K: thread -> part (16 B of head_dim) = tid % 16, keys tid/16 + 16 r.
  // V: thread -> keys 4a .. 4a+3 with a = lane % 16, part = wave*4 + lane/16.
  const int k_part = tid & 15;
  const int k_key0 = tid >> 4;
  const int v_a = lane & 15;
  const int v_part = wave * 4 + (lane >> 4);
  uint4 kst[4], vst[4];

  auto slot_of = [&](int kp) -> int64_t {
    const int kc = min(kp, L - 1);
    const int blk = bt[kc >> log2_bs];
    return ((static_cast<int64_t>(blk) << log2_bs) | (kc & bs_mask)) * slot_stride;
  };
  auto load_tile = [&](int kt) {
    const int base = kt * kKeys;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      kst[r] = *reinterpret_cast<const uint4*>(kbase + slot_of(base + k_key0 + 16 * r) + k_part * 8);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      vst[r] = *reinterpret_cast<const uint4*>(vbase + slot_of(base + 4 * v_a + r) + v_part * 8);
  };

  load_tile(0);
  for (int kt = 0; kt < num_tiles; ++kt) {
    __syncthreads();  // everyone is done reading the previous tile
#pragma unroll
    for (int r = 0; r < 4; ++r)
      *reinterpret_cast<uint4*>(&k_lds[(k_key0 + 16 * r) * kKStride + k_part * 8]) = kst[r];
    {
      // Transpose 4 keys x 8 elements into 8 rows of V^T, 4 keys (8 B) each.
      const uint32_t* w = reinterpret_cast<const uint32_t*>(vst);
      const int c0 = vt_col(4 * v_a);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int wi = e >> 1;
        const bool hi = e & 1;
        uint32_t x[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint32_t word = w[r * 4 + wi];
          x[r] = hi ? (word >> 16) : (word & 0xffffu);
        }
        uint2 packed;
        packed.x = x[0] | (x[1] << 16);
        packed.y = x[2] | (x[3] << 16);
        *reinterpret_cast<uint2*>(&vt_lds[(v_part * 8 + e) * kVStride + c0]) = packed;
      }
    }
    __syncthreads();
    if (kt + 1 < num_tiles) load_tile(kt + 1);

    // S^T for the two 32-key halves of the tile.
    f32x16_t s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < kHeadDim / 16; ++ks) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(
            &k_lds[(kb * 32 + col) * kKStride + ks * 16 + half * 8]);
        s[kb] = mfma32(a, qreg[ks], s[kb]);
      }
    }
    // Scale, mask, row max. Lane holds keys kb*32 + (r/4)*8 + half*4 + r%4.
    const int kbase_pos = kt * kKeys;
    const bool full = kbase_pos + kKeys - 1 <= P + tok0;  // every row sees every key
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = s[kb][r] * scale_log2;
        if (!full) {
          const int kp = kbase_pos + kb * 32 + (r >> 2) * 8 + half * 4 + (r & 3);
          x = kp <= qpos ? x : -INFINITY;
        }
        s[kb][r] = x;
        tmax = fmaxf(tmax, x);
      }
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float mn = fmaxf(m, tmax);  // finite: key 0 is visible to every row
    const float alpha = fast_exp2(m - mn);
    m = mn;
    lsum *= alpha;
#pragma unroll
    for (int db = 0; db < kHeadDim / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] *= alpha;

    // P (bf16) as the B operand, 16 keys per MFMA step.
    bf16x8_t pb[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int hstep = 0; hstep < 2; ++hstep) {
        float p[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          p[i] = fast_exp2(s[kb][hstep * 8 + i] - mn);
          lsum += p[i];
        }
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(p[2 * i], p[2 * i + 1]);
        pb[kb * 2 + hstep] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<uint4*>(w));
      }
    }
    // O^T += V^T P^T.
#pragma unroll
    for (int db = 0; db < kHeadDim / 32; ++db) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(
            &vt_lds[(db * 32 + col) * kVStride + ks * 16 + half * 8]);
        o[db] = mfma32(a, pb[ks], o[db]);
      }
    }
  }

  // Normalise and write. Lane holds d = db*32 + (r/4)*8 + half*4 + r%4.
  lsum += __shfl_xor(lsum, 32);
  const float inv = 1.f / lsum;
  if (tok0 + tok < N) {
    uint16_t* op = out + (static_cast<int64_t>(q0 + tok0 + tok) * num_q_heads + head) * kHeadDim;
#pragma unroll
    for (int db = 0; db < kHeadDim / 32; ++db) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint2 w;
        w.x = pack_bf16x2(o[db][j * 4 + 0] * inv, o[db][j * 4 + 1] * inv);
        w.y = pack_bf16x2(o[db][j * 4 + 2] * inv, o[db][j * 4 + 3] * inv);
        *reinterpret_cast<uint2*>(op + db * 32 + j * 8 + half * 4) = w;
      }
    }
  }
}

}  // namespace

hipError_t launch_prefill(uint16_t* out, const uint16_t* q, const uint16_t* k_cache,
                          const uint16_t* v_cache, const int32_t* cu_seqlens_q,
                          const int32_t* context_lens, const int32_t* block_table,
                          int32_t block_table_stride, int32_t batch, int32_t max_seqlen_q,
                          int32_t num_q_heads, int32_t num_kv_heads, int32_t block_size,
                          float scale, hipStream_t stream) {
  const int G = num_q_heads / num_kv_heads;
  const int TQ = kRows / G;
  const int q_tiles = (max_seqlen_q + TQ - 1) / TQ;
  const int64_t blocks = static_cast<int64_t>(q_tiles) * num_kv_heads * batch;
  if (blocks == 0) return hipSuccess;
  const int log2_bs = __builtin_ctz(static_cast<unsigned>(block_size));
  const float scale_log2 = scale * kLog2e;
#define PA_PREFILL_CASE(GG)                                                                    \
  case GG:                                                                                     \
    hipLaunchKernelGGL((prefill_kernel<GG>), dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, \
                       stream, out, q, k_cache, v_cache, cu_seqlens_q, context_lens,           \
                       block_table, block_table_stride, batch, num_q_heads, num_kv_heads,      \
                       log2_bs, q_tiles, scale_log2);                                          \
    break;
  switch (G) {
    PA_PREFILL_CASE(1)
    PA_PREFILL_CASE(2)
    PA_PREFILL_CASE(4)
    PA_PREFILL_CASE(8)
    default:
      return hipErrorInvalidValue;
  }
#undef PA_PREFILL_CASE
  return hipGetLastError();
}

}  // namespace pa

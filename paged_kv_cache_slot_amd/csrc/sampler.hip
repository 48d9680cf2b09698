// Gumbel-max token sampler: token[b] = argmax_i p[b,i] / E[b,i] with
// E ~ Exp(1) drawn from Philox4x32-10 (the exact definition of every step is
// in include/pa.h, pa_sample_gumbel).
//
// [Report] "nano-vllm 深度分析报告", section "创新之处" (the Gumbel-Max item)
// and table "可复用的模式与技巧" (row "Gumbel-Max 采样"): the draw is the
// largest probability divided by an independent Exp(1) variable.
//
// One pass over the [B, V] probabilities. Work-group (c, b) owns a contiguous
// chunk of row b; each thread takes 4 consecutive elements per step (one
// 16-byte load, one Philox call whose four 32-bit words serve the four
// elements), keeps its best (key, index), and the work-group's best goes to a
// workspace slot. A second kernel merges the chunks of each row (one wavefront
// per row). The kernel is bound by the vector ALU (the Philox multiplies and
// the per-element log and reciprocal) rather than by HBM; full tiles run
// without element checks, two quads per iteration so that two coalesced
// 16-byte loads and two Philox calls are in flight per thread.
#include <cstdint>

#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kSampleThreads = 256;
constexpr int kSampleTile = kSampleThreads * 4;   // elements per work-group step
constexpr int kTargetGroups = 2048;                // work-groups to aim for

typedef float f32x4 __attribute__((ext_vector_type(4)));

// a ^ b ^ c in one v_bitop3_b32 (truth table 0x96 over the operand bits).
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}

// Philox4x32 with 10 rounds (Salmon et al., SC'11): two 32x32 -> 64-bit
// products per round, high halves mixed into the other two words with the
// key, key bumped by the Weyl constants between rounds.
__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t a = static_cast<uint64_t>(0xD2511F53u) * c.x;
    const uint64_t b = static_cast<uint64_t>(0xCD9E8D57u) * c.z;
    c = make_uint4(xor3(static_cast<uint32_t>(b >> 32), c.y, k0), static_cast<uint32_t>(b),
                   xor3(static_cast<uint32_t>(a >> 32), c.w, k1), static_cast<uint32_t>(a));
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

// Key of one element: p / E with u = ((x >> 9) + 1/2) 2^-23 (exact) and
// E = -log2(u) > 0, in fp32 (hardware log2 and reciprocal).
__device__ __forceinline__ float gumbel_key(float p, uint32_t x) {
  const float u = __builtin_fmaf(static_cast<float>(x >> 9), 0x1p-23f, 0x1p-24f);
  const float e = -__builtin_amdgcn_logf(u);
  return p * __builtin_amdgcn_rcpf(e);
}

// (key, index) order: larger key first, then smaller index.
__device__ __forceinline__ bool better(float k, int i, float bk, int bi) {
  return k > bk || (k == bk && i < bi);
}

__device__ __forceinline__ void wave_best(float& k, int& i) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float ok = __shfl_xor(k, m, 64);
    const int oi = __shfl_xor(i, m, 64);
    if (better(ok, oi, k, i)) {
      k = ok;
      i = oi;
    }
  }
}

// Folds the four keys of quad index q (elements 4q .. 4q+3, all < vocab) into
// the thread's best.
__device__ __forceinline__ void fold_quad(const f32x4& v, int q, int row, uint32_t off0,
                                          uint32_t off1, uint32_t key0, uint32_t key1,
                                          float& best, int& bidx) {
  const uint4 r = philox4x32_10(
      make_uint4(static_cast<uint32_t>(q), static_cast<uint32_t>(row), off0, off1), key0, key1);
  const float k[4] = {gumbel_key(v.x, r.x), gumbel_key(v.y, r.y), gumbel_key(v.z, r.z),
                      gumbel_key(v.w, r.w)};
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (k[j] > best) {
      best = k[j];
      bidx = 4 * q + j;
    }
}

// kVec: rows start 16-byte aligned (stride a multiple of 4), so a quad is one
// 16-byte load; otherwise four 4-byte loads.
template <bool kVec>
__device__ __forceinline__ f32x4 load_quad(const float* p) {
  if constexpr (kVec) {
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  } else {
    f32x4 v;
    v.x = __builtin_nontemporal_load(p);
    v.y = __builtin_nontemporal_load(p + 1);
    v.z = __builtin_nontemporal_load(p + 2);
    v.w = __builtin_nontemporal_load(p + 3);
    return v;
  }
}

template <bool kVec>
__global__ __launch_bounds__(kSampleThreads) void sample_partial_kernel(
    const float* __restrict__ probs, int64_t row_stride, int32_t vocab, int32_t tiles_per_chunk,
    uint32_t key0, uint32_t key1, uint32_t off0, uint32_t off1, int2* __restrict__ partial) {
  const int row = blockIdx.y;
  const int chunk = blockIdx.x;
  const float* p = probs + static_cast<int64_t>(row) * row_stride;
  const int full_tiles = vocab / kSampleTile;           // tiles with every element < vocab
  const int ntiles = (vocab + kSampleTile - 1) / kSampleTile;
  const int t0 = chunk * tiles_per_chunk;
  const int t1 = min(t0 + tiles_per_chunk, ntiles);
  const int f1 = min(t1, full_tiles);
  const int tid = static_cast<int>(threadIdx.x);
  float best = -1.f;
  int bidx = 0x7fffffff;

  // Full tiles, two per iteration: two loads and two Philox calls in flight.
  int t = t0;
  for (; t + 1 < f1; t += 2) {
    const int qa = t * kSampleThreads + tid;
    const int qb = qa + kSampleThreads;
    const f32x4 va = load_quad<kVec>(p + 4 * qa);
    const f32x4 vb = load_quad<kVec>(p + 4 * qb);
    fold_quad(va, qa, row, off0, off1, key0, key1, best, bidx);
    fold_quad(vb, qb, row, off0, off1, key0, key1, best, bidx);
  }
  if (t < f1) {
    const int q = t * kSampleThreads + tid;
    fold_quad(load_quad<kVec>(p + 4 * q), q, row, off0, off1, key0, key1, best, bidx);
    ++t;
  }
  // The last tile of the row, if it is partial and ours: element checks.
  if (t < t1) {
    const int q = t * kSampleThreads + tid;
    const int i = 4 * q;
    if (i < vocab) {
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      v.x = p[i];
      if (i + 1 < vocab) v.y = p[i + 1];
      if (i + 2 < vocab) v.z = p[i + 2];
      if (i + 3 < vocab) v.w = p[i + 3];
      const uint4 r = philox4x32_10(
          make_uint4(static_cast<uint32_t>(q), static_cast<uint32_t>(row), off0, off1), key0,
          key1);
      const float k[4] = {gumbel_key(v.x, r.x), gumbel_key(v.y, r.y), gumbel_key(v.z, r.z),
                          gumbel_key(v.w, r.w)};
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (i + j < vocab && k[j] > best) {
          best = k[j];
          bidx = i + j;
        }
    }
  }
  // A thread's candidates rise in index, so `>` above keeps the first of equal
  // keys; across threads the order rule does.
  wave_best(best, bidx);
  __shared__ float s_key[kSampleThreads / 64];
  __shared__ int s_idx[kSampleThreads / 64];
  const int wave = tid / 64;
  if ((tid & 63) == 0) {
    s_key[wave] = best;
    s_idx[wave] = bidx;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < kSampleThreads / 64; ++w)
      if (better(s_key[w], s_idx[w], best, bidx)) {
        best = s_key[w];
        bidx = s_idx[w];
      }
    partial[static_cast<int64_t>(row) * gridDim.x + chunk] =
        make_int2(__float_as_int(best), bidx);
  }
}

// One wavefront per row: the best of the row's chunk results.
__global__ __launch_bounds__(256) void sample_merge_kernel(const int2* __restrict__ partial,
                                                           int32_t chunks, int32_t batch,
                                                           int32_t* __restrict__ tokens) {
  const int row = blockIdx.x * 4 + threadIdx.x / 64;
  const int lane = threadIdx.x & 63;
  if (row >= batch) return;
  float best = -1.f;
  int bidx = 0x7fffffff;
  for (int c = lane; c < chunks; c += 64) {
    const int2 v = partial[static_cast<int64_t>(row) * chunks + c];
    const float k = __int_as_float(v.x);
    if (better(k, v.y, best, bidx)) {
      best = k;
      bidx = v.y;
    }
  }
  wave_best(best, bidx);
  if (lane == 0) tokens[row] = bidx == 0x7fffffff ? 0 : bidx;
}

struct SampleGrid {
  int chunks;
  int tiles_per_chunk;
};

SampleGrid sample_grid(int32_t batch, int32_t vocab) {
  const int ntiles = (vocab + kSampleTile - 1) / kSampleTile;
  int chunks = batch > 0 ? (kTargetGroups + batch - 1) / batch : 1;
  chunks = chunks < 1 ? 1 : (chunks > ntiles ? ntiles : chunks);
  const int per = (ntiles + chunks - 1) / chunks;
  return {(ntiles + per - 1) / per, per};
}

}  // namespace

size_t sample_workspace_bytes(int32_t batch, int32_t vocab) {
  if (batch <= 0 || vocab <= 0) return 0;
  return static_cast<size_t>(batch) * sample_grid(batch, vocab).chunks * sizeof(int2);
}

hipError_t launch_sample(int32_t* tokens, const float* probs, int64_t row_stride, int32_t batch,
                         int32_t vocab, uint64_t seed, uint64_t offset, void* workspace,
                         hipStream_t stream) {
  const SampleGrid g = sample_grid(batch, vocab);
  int2* partial = static_cast<int2*>(workspace);
  const bool vec = row_stride % 4 == 0 && (reinterpret_cast<uintptr_t>(probs) & 15u) == 0;
  auto kernel = vec ? sample_partial_kernel<true> : sample_partial_kernel<false>;
  hipLaunchKernelGGL(kernel, dim3(g.chunks, batch), dim3(kSampleThreads), 0, stream, probs,
                     row_stride, vocab, g.tiles_per_chunk, static_cast<uint32_t>(seed),
                     static_cast<uint32_t>(seed >> 32), static_cast<uint32_t>(offset),
                     static_cast<uint32_t>(offset >> 32), partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(sample_merge_kernel, dim3((batch + 3) / 4), dim3(256), 0, stream, partial,
                     g.chunks, batch, tokens);
  return hipGetLastError();
}

}  // namespace pa

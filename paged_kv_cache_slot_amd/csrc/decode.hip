// Paged decode: one query token per sequence attends over its context, whose
// keys and values sit in fixed-size blocks reached through the sequence's
// block table ("DeepSeek研究员1200行代码复刻vLLM…", section "vLLM是什么？").
//
// Work split. The context of each sequence is cut into pieces of
// kDecodeSplit (256) tokens; one work-group of 4 wavefronts owns one
// (sequence, kv head, piece) and all G = Hq/Hkv query heads that read that kv
// head, so every K/V byte is fetched from HBM once. Each wavefront takes 64
// consecutive tokens; within it, each row of 16 lanes takes every fourth token
// and each lane one 16-byte slice (8 elements of head_dim) of that token's
// 256-byte kv-head row. One load instruction thus reads four whole rows.
//
// Per token: q.k from four v_dot2c_f32_bf16 per lane, summed over the 16-lane
// row with DPP; online softmax in base 2 (scale*log2e folded in) per row of
// lanes, updated once per chunk of tokens; p*V accumulated in fp32. Rows of
// lanes, then wavefronts (through LDS), are merged with the usual
// (max, sum, acc) rescaling. A sequence with one piece writes its bf16 output
// directly; longer ones leave (acc, max, sum) per piece in the workspace and
// the reduce kernel merges them.
//
// Roofline: HBM. Algorithmic bytes = 2 (K and V) * L * 256 B per (sequence,
// kv head), plus q and out, which are small.
#include <cmath>

#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kWaves = 4;
constexpr int kTokensPerWave = kDecodeSplit / kWaves;  // 64
constexpr int kTokensPerRow = kTokensPerWave / 4;      // 16, one 16-lane row

// Merges (m2, l2, acc2) into (m, l, acc): base-2 online-softmax states.
template <int N>
__device__ __forceinline__ void merge_state(float& m, float& l, float (&acc)[N], float m2,
                                            float l2, const float (&acc2)[N]) {
  const float mn = fmaxf(m, m2);
  const float mu = mn == -INFINITY ? 0.f : mn;
  const float a = fast_exp2(m - mu);
  const float c = fast_exp2(m2 - mu);
  l = l * a + l2 * c;
#pragma unroll
  for (int e = 0; e < N; ++e) acc[e] = acc[e] * a + acc2[e] * c;
  m = mn;
}

template <int G, int CH>
__global__ __launch_bounds__(256) void decode_split_kernel(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ k_cache, const uint16_t* __restrict__ v_cache,
    const int32_t* __restrict__ block_table, int32_t bt_stride,
    const int32_t* __restrict__ context_lens, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t log2_bs, int32_t max_context_len, float scale_log2, int32_t max_splits,
    float* __restrict__ ws_o, float* __restrict__ ws_ml) {
  __shared__ float s_part[kWaves][G][kHeadDim + 2];

  const int idx = blockIdx.x;
  const int split = idx % max_splits;
  const int rest = idx / max_splits;
  const int g = rest % num_kv_heads;
  const int b = rest / num_kv_heads;
  const int h0 = g * G;
  const int tid = threadIdx.x;
  const int L = min(context_lens[b], max_context_len);

  if (L <= 0) {  // padding row: zeros, written once
    if (split == 0) {
      for (int e = tid; e < G * kHeadDim; e += 256)
        out[(static_cast<int64_t>(b) * num_q_heads + h0) * kHeadDim + e] = 0;
    }
    return;
  }
  const int t0 = split * kDecodeSplit;
  if (t0 >= L) return;
  const int nsplit = min((L + kDecodeSplit - 1) / kDecodeSplit, max_splits);

  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = lane >> 4;  // which token of four
  const int sub = lane & 15;  // which 8-element slice of head_dim

  uint32_t qv[G][4];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const uint4 t = *reinterpret_cast<const uint4*>(
        q + (static_cast<int64_t>(b) * num_q_heads + h0 + hh) * kHeadDim + sub * 8);
    qv[hh][0] = t.x; qv[hh][1] = t.y; qv[hh][2] = t.z; qv[hh][3] = t.w;
  }

  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[hh][e] = 0.f;
  }

  const int bs_mask = (1 << log2_bs) - 1;
  const int32_t* bt = block_table + static_cast<int64_t>(b) * bt_stride;
  const int64_t slot_stride = static_cast<int64_t>(num_kv_heads) * kHeadDim;
  const uint16_t* kbase = k_cache + g * kHeadDim + sub * 8;
  const uint16_t* vbase = v_cache + g * kHeadDim + sub * 8;
  const int wbase = t0 + wave * kTokensPerWave;

#pragma unroll
  for (int c = 0; c < kTokensPerRow / CH; ++c) {
    const int cbase = wbase + c * CH * 4;
    if (cbase >= L) break;  // uniform over the wavefront
    int64_t off[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int tw = cbase + 4 * i;  // first token of this load, uniform
      const int blk = bt[min(tw, L - 1) >> log2_bs];
      const int tc = min(tw + grp, L - 1);  // past the end: re-read the last token
      off[i] = ((static_cast<int64_t>(blk) << log2_bs) | (tc & bs_mask)) * slot_stride;
    }
    uint4 kr[CH], vr[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) kr[i] = *reinterpret_cast<const uint4*>(kbase + off[i]);
#pragma unroll
    for (int i = 0; i < CH; ++i) vr[i] = *reinterpret_cast<const uint4*>(vbase + off[i]);

    float s[CH][G];
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const bool valid = cbase + 4 * i + grp < L;
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        float d = dot2_bf16(qv[hh][0], kr[i].x, 0.f);
        d = dot2_bf16(qv[hh][1], kr[i].y, d);
        d = dot2_bf16(qv[hh][2], kr[i].z, d);
        d = dot2_bf16(qv[hh][3], kr[i].w, d);
        d = row16_sum(d) * scale_log2;
        s[i][hh] = valid ? d : -INFINITY;
      }
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float cm = s[0][hh];
#pragma unroll
      for (int i = 1; i < CH; ++i) cm = fmaxf(cm, s[i][hh]);
      const float mn = fmaxf(m[hh], cm);
      const float mu = mn == -INFINITY ? 0.f : mn;
      const float alpha = fast_exp2(m[hh] - mu);
      m[hh] = mn;
      l[hh] *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[hh][e] *= alpha;
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        const float p = fast_exp2(s[i][hh] - mu);
        s[i][hh] = p;
        l[hh] += p;
      }
    }
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const float v[8] = {bf16_lo(vr[i].x), bf16_hi(vr[i].x), bf16_lo(vr[i].y), bf16_hi(vr[i].y),
                          bf16_lo(vr[i].z), bf16_hi(vr[i].z), bf16_lo(vr[i].w), bf16_hi(vr[i].w)};
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[hh][e] += s[i][hh] * v[e];
      }
    }
  }

  // Merge the four rows of lanes of this wavefront (lanes 16 and 32 apart).
#pragma unroll
  for (int mask = 16; mask <= 32; mask <<= 1) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float acc2[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc2[e] = __shfl_xor(acc[hh][e], mask);
      const float m2 = __shfl_xor(m[hh], mask);
      const float l2 = __shfl_xor(l[hh], mask);
      merge_state(m[hh], l[hh], acc[hh], m2, l2, acc2);
    }
  }
  if (grp == 0) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
#pragma unroll
      for (int e = 0; e < 8; ++e) s_part[wave][hh][sub * 8 + e] = acc[hh][e];
      if (sub == 0) {
        s_part[wave][hh][kHeadDim] = m[hh];
        s_part[wave][hh][kHeadDim + 1] = l[hh];
      }
    }
  }
  __syncthreads();

  // Merge the wavefronts and write this piece's result.
  for (int e = tid; e < G * kHeadDim; e += 256) {
    const int hh = e / kHeadDim;
    const int d = e % kHeadDim;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_part[w][hh][kHeadDim]);
    float o = 0.f, lt = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float a = fast_exp2(s_part[w][hh][kHeadDim] - M);
      o += a * s_part[w][hh][d];
      lt += a * s_part[w][hh][kHeadDim + 1];
    }
    const int64_t bh = static_cast<int64_t>(b) * num_q_heads + h0 + hh;
    if (nsplit == 1) {
      const float r = o / lt;
      out[bh * kHeadDim + d] = static_cast<uint16_t>(pack_bf16x2(r, 0.f) & 0xffffu);
    } else {
      const int64_t piece = bh * max_splits + split;
      ws_o[piece * kHeadDim + d] = o;
      if (d == 0) {
        ws_ml[piece * 2] = M;
        ws_ml[piece * 2 + 1] = lt;
      }
    }
  }
}

// Merges the pieces of sequences with more than one piece: one work-group per
// (sequence, query head), one thread per element of head_dim.
__global__ __launch_bounds__(kHeadDim) void decode_reduce_kernel(
    uint16_t* __restrict__ out, const int32_t* __restrict__ context_lens, int32_t num_q_heads,
    int32_t max_context_len, int32_t max_splits, const float* __restrict__ ws_o,
    const float* __restrict__ ws_ml) {
  const int64_t bh = blockIdx.x;
  const int b = static_cast<int>(bh / num_q_heads);
  const int L = min(context_lens[b], max_context_len);
  const int nsplit = min((L + kDecodeSplit - 1) / kDecodeSplit, max_splits);
  if (nsplit <= 1) return;  // written by the split kernel (or a padding row)
  const int d = threadIdx.x;
  const float* ml = ws_ml + bh * max_splits * 2;
  float M = -INFINITY;
  for (int i = 0; i < nsplit; ++i) M = fmaxf(M, ml[2 * i]);
  float o = 0.f, lt = 0.f;
  for (int i = 0; i < nsplit; ++i) {
    const float a = fast_exp2(ml[2 * i] - M);
    lt += a * ml[2 * i + 1];
    o += a * ws_o[(bh * max_splits + i) * kHeadDim + d];
  }
  out[bh * kHeadDim + d] = static_cast<uint16_t>(pack_bf16x2(o / lt, 0.f) & 0xffffu);
}

int max_splits_for(int32_t max_context_len) {
  return max(1, (max_context_len + kDecodeSplit - 1) / kDecodeSplit);
}

template <int G, int CH>
void launch_split(uint16_t* out, const uint16_t* q, const uint16_t* k_cache,
                  const uint16_t* v_cache, const int32_t* block_table, int32_t bt_stride,
                  const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
                  int32_t num_kv_heads, int32_t log2_bs, int32_t max_context_len,
                  float scale_log2, int32_t max_splits, float* ws_o, float* ws_ml,
                  hipStream_t stream) {
  const int64_t blocks = static_cast<int64_t>(batch) * num_kv_heads * max_splits;
  hipLaunchKernelGGL((decode_split_kernel<G, CH>), dim3(static_cast<uint32_t>(blocks)), dim3(256),
                     0, stream, out, q, k_cache, v_cache, block_table, bt_stride, context_lens,
                     num_q_heads, num_kv_heads, log2_bs, max_context_len, scale_log2, max_splits,
                     ws_o, ws_ml);
}

}  // namespace

size_t decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t max_context_len) {
  const size_t pieces = static_cast<size_t>(batch) * num_q_heads * max_splits_for(max_context_len);
  return pieces * (kHeadDim + 2) * sizeof(float);
}

hipError_t launch_decode(uint16_t* out, const uint16_t* q, const uint16_t* k_cache,
                         const uint16_t* v_cache, const int32_t* block_table,
                         int32_t block_table_stride, const int32_t* context_lens, int32_t batch,
                         int32_t num_q_heads, int32_t num_kv_heads, int32_t block_size,
                         int32_t max_context_len, float scale, void* workspace,
                         hipStream_t stream) {
  const int max_splits = max_splits_for(max_context_len);
  const size_t pieces = static_cast<size_t>(batch) * num_q_heads * max_splits;
  float* ws_o = static_cast<float*>(workspace);
  float* ws_ml = ws_o + pieces * kHeadDim;
  const int log2_bs = __builtin_ctz(static_cast<unsigned>(block_size));
  const float scale_log2 = scale * kLog2e;
  const int G = num_q_heads / num_kv_heads;
#define PA_DECODE_CASE(GG, CC)                                                              \
  case GG:                                                                                 \
    launch_split<GG, CC>(out, q, k_cache, v_cache, block_table, block_table_stride,        \
                         context_lens, batch, num_q_heads, num_kv_heads, log2_bs,          \
                         max_context_len, scale_log2, max_splits, ws_o, ws_ml, stream);    \
    break;
  switch (G) {
    PA_DECODE_CASE(1, 8)
    PA_DECODE_CASE(2, 8)
    PA_DECODE_CASE(4, 8)
    PA_DECODE_CASE(8, 4)
    default:
      return hipErrorInvalidValue;
  }
#undef PA_DECODE_CASE
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (max_splits > 1) {
    hipLaunchKernelGGL(decode_reduce_kernel,
                       dim3(static_cast<uint32_t>(static_cast<int64_t>(batch) * num_q_heads)),
                       dim3(kHeadDim), 0, stream, out, context_lens, num_q_heads, max_context_len,
                       max_splits, ws_o, ws_ml);
    err = hipGetLastError();
  }
  return err;
}

}  // namespace pa

// Varlen causal prefill over a paged KV cache with a cached prefix
// ("DeepSeek研究员1200行代码复刻vLLM…", section "vLLM是什么？" for the paging;
// "nano-vllm 深度分析报告", section 创新之处, for prefix caching).
//
// Sequence b has P cached tokens and N new ones (all stored in the pool); new
// row i sits at position P + i and attends to keys 0 .. P + i.
//
// Work split. One work-group (4 wavefronts) owns one (sequence, kv head,
// tile of 128/G new tokens) and all G query heads of that kv head: 128 query
// rows, 32 per wavefront. It walks the context in tiles of 64 keys.
//
// Tile pipeline (two LDS stages). Each tile's K and V rows are copied from the
// pool straight into LDS by global_load_lds (16 bytes per lane, no registers),
// addressed through the block table (block ids fetched one tile ahead). While
// tile t is computed, tile t+1 is in flight. Inside a 256-byte row the sixteen
// 16-byte units are stored XOR-swizzled by the key index, so the MFMA operand
// reads below hit distinct LDS banks.
//
// Per wavefront and tile, flash-attention style:
//   S^T = K Q^T      bf16 MFMA 32x32x16, fp32 accumulate: each lane holds the
//                    scores of ONE query row, so the row max and sum stay
//                    in-lane except for one exchange with the lane 32 apart;
//   p = exp2(s*scale*log2e - m*scale*log2e) with a lazy rescale of the output
//                    (skipped while no row max of the wavefront moves);
//   O^T += V^T P^T   bf16 MFMA 32x32x16 with P taken straight from the S^T
//                    accumulators (converted to bf16) and V^T built by
//                    ds_read_b64_tr_b16 transposed reads from the row-major V
//                    tile, with keys ordered to match the accumulator layout.
// Tiles wholly above the causal diagonal are skipped per wavefront; tiles
// wholly below it skip the mask.
//
// Roofline: MFMA (bf16). Algorithmic flops = 4 * Hq * 128 * sum over
// sequences of (N*P + N*(N+1)/2) (only the causal pairs).
#include <cmath>

#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kWaves = 4;
constexpr int kRows = kWaves * 32;  // query rows (token, head) per work-group
constexpr int kKeys = 64;           // keys per tile
constexpr int kTileElems = kKeys * kHeadDim;
constexpr int kXcds = 8;            // MI355X: 8 accelerator dies, each with its own L2

__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// LDS swizzle of the sixteen 16-byte units of a key's 256-byte row: logical
// unit u of key k is stored at unit u ^ swz(k). swz is a bijection on k % 16
// such that 16 consecutive keys (the K operand read) and, for any 4 consecutive
// keys starting at a multiple of 4, the units u and u+1 with u even (one
// transposed V read) all land on distinct units, i.e. distinct LDS banks.
__device__ __forceinline__ int swz(int key) { return ((key << 1) & 14) | ((key >> 3) & 1); }

typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(3))) i16x4_t* lds_i16x4_ptr;

// 16 bytes per lane from global memory into LDS at dst + 16 * lane.
__device__ __forceinline__ void dma16(const void* src, uint16_t* dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void_ptr)(dst), 16, 0, 0);
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
  // One array per stage (not one indexed array): with the stage known at
  // compile time the compiler can prove that the copies into one stage do not
  // alias the reads of the other, so it does not wait for them.
  __shared__ __attribute__((aligned(1024))) uint16_t lds_k0[kTileElems];
  __shared__ __attribute__((aligned(1024))) uint16_t lds_v0[kTileElems];
  __shared__ __attribute__((aligned(1024))) uint16_t lds_k1[kTileElems];
  __shared__ __attribute__((aligned(1024))) uint16_t lds_v1[kTileElems];

  // Work-group i runs on XCD i % 8. Each (sequence, kv head) pair is given to
  // one XCD and all its query tiles are dispatched there back to back
  // (heaviest, i.e. last, first), so the pair's K/V tiles, which every query
  // tile reads, stay in that XCD's L2 while they are in use.
  const int idx = blockIdx.x;
  const int xcd = idx & (kXcds - 1);
  const int j = idx / kXcds;
  const int pair = (j / q_tiles) * kXcds + xcd;
  const int qtile = q_tiles - 1 - j % q_tiles;
  if (pair >= batch * num_kv_heads) return;
  const int b = pair / num_kv_heads;
  const int g = pair % num_kv_heads;

  const int q0 = cu_seqlens_q[b];
  const int N = cu_seqlens_q[b + 1] - q0;
  const int tok0 = qtile * TQ;
  if (tok0 >= N) return;
  const int L = context_lens[b];
  const int P = L - N;
  if (P < 0) return;  // breaks the contract context_lens[b] >= N; nothing is read
  const int tok_end = min(N, tok0 + TQ);   // exclusive
  const int key_end = P + tok_end;         // keys [0, key_end) are visible to some row
  const int num_tiles = (key_end + kKeys - 1) / kKeys;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;   // this lane's query row within the wavefront
  const int half = lane >> 5;  // which half of the MFMA k-slices this lane holds

  // This lane's query row; a wavefront's 32 rows are 32 consecutive tokens of
  // one head (TQ >= 32).
  const int row = wave * 32 + col;
  const int hh = row / TQ;
  const int tok = row % TQ;
  const int qpos = P + tok0 + tok;                      // absolute position
  const int qt = q0 + min(tok0 + tok, N - 1);           // clamped for loads
  const int head = g * G + hh;
  const int wave_pos0 = P + tok0 + (wave * 32) % TQ;    // position of the wavefront's first row

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
  float m = -INFINITY;  // running max of this lane's row (raw scores)
  float lsum = 0.f;     // running sum over this lane's keys

  const int bs_mask = (1 << log2_bs) - 1;
  const int32_t* bt = block_table + static_cast<int64_t>(b) * bt_stride;
  const int64_t slot_stride = static_cast<int64_t>(num_kv_heads) * kHeadDim;
  const uint16_t* kbase = k_cache + g * kHeadDim;
  const uint16_t* vbase = v_cache + g * kHeadDim;

  // ---- tile loads -----------------------------------------------------------
  // A tile is 64 keys x 256 B per tensor = 16 global_load_lds instructions of
  // 1 KiB (4 keys each); wavefront w issues instructions 4w .. 4w+3 for K and
  // the same for V. Lane l of an instruction carries key (4*instr + l/16) and
  // the 16-byte unit (l%16) of its LDS row, which holds logical unit
  // (l%16) ^ swz(key) of the key's 256-byte row. The 4 keys of an instruction
  // share a block (block_size >= 16), so its block id is one scalar load.
  const int dma_row = lane >> 4;
  const int dma_unit = lane & 15;
  auto issue_tile = [&](int t, uint16_t* lk, uint16_t* lv) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key0 = (4 * wave + j) * 4;                  // uniform
      const int kf = min(t * kKeys + key0, L - 1);          // uniform
      const int blk = bt[kf >> log2_bs];                    // scalar load
      const int key = key0 + dma_row;
      const int kc = min(t * kKeys + key, L - 1);  // past the context: re-read token L-1
      const int64_t off = ((static_cast<int64_t>(blk) << log2_bs) | (kc & bs_mask)) * slot_stride +
                          ((dma_unit ^ swz(key)) * 8);
      const int dst = key0 * kHeadDim;  // uniform: 4 rows of 128 elements
      dma16(kbase + off, lk + dst);
      dma16(vbase + off, lv + dst);
    }
  };

  // ---- operand addressing (element offsets inside one LDS tile) -------------
  // K (A operand of S^T = K Q^T): key kb*32 + col, logical unit ks*2 + half.
  // V^T (A operand of O^T): transposed reads; this lane supplies, for read r
  // of a 16-key step, the 8-byte address of key (16ks + 8r + 4h + a/4) and
  // elements d .. d+3 with d = 32db + 16(group & 1) + 4(a & 3), where a is the
  // lane within its 16-lane group and h = lane / 32; the transposed read then
  // hands lane i of the group the 4 keys of the group's addresses at d + i.
  const int a16 = lane & 15;
  const int grp16 = lane >> 4;
  int v_off[kHeadDim / 32][2];  // for ks = 0; step ks adds 16 keys
#pragma unroll
  for (int db = 0; db < kHeadDim / 32; ++db) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int key = r * 8 + 4 * half + (a16 >> 2);  // key within the 16-key step
      const int d = db * 32 + (grp16 & 1) * 16 + 4 * (a16 & 3);
      v_off[db][r] = key * kHeadDim + (((d >> 3) ^ swz(key)) * 8) + (d & 7);
    }
  }

  // ---- pipeline ------------------------------------------------------------
  // Computes tile t from the LDS stage (kt, vt).
  auto compute_tile = [&](int t, const uint16_t* kt, uint16_t* vt) {
      const int kstart = t * kKeys;
      if (kstart > wave_pos0 + 31) return;       // above the diagonal for every row here
      const bool full = kstart + kKeys - 1 <= wave_pos0;  // every row sees every key

      // S^T for the two 32-key halves of the tile.
      f32x16_t s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
        const int key = kb * 32 + col;
#pragma unroll
        for (int ks = 0; ks < kHeadDim / 16; ++ks) {
          const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(
              kt + key * kHeadDim + (((ks * 2 + half) ^ swz(key)) * 8));
          s[kb] = mfma32(a, qreg[ks], s[kb]);
        }
      }
      // Mask, row max. Lane holds keys kb*32 + (r/4)*8 + half*4 + r%4.
      float tmax = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if (!full) {
            const int kp = kstart + kb * 32 + (r >> 2) * 8 + half * 4 + (r & 3);
            s[kb][r] = kp <= qpos ? s[kb][r] : -INFINITY;
          }
          tmax = fmaxf(tmax, s[kb][r]);
        }
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      const float mn = fmaxf(m, tmax);  // finite: key 0 is visible to every row
      const float alpha = fast_exp2((m - mn) * scale_log2);
      m = mn;
      if (__any(alpha != 1.f)) {  // rescale only when some row max moved
        lsum *= alpha;
#pragma unroll
        for (int db = 0; db < kHeadDim / 32; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      }
      const float mc = mn * scale_log2;

      // P (bf16) as the B operand, 16 keys per MFMA step.
      bf16x8_t pb[4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
          uint32_t w[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p0 = fast_exp2(fmaf(s[kb][hs * 8 + 2 * i], scale_log2, -mc));
            const float p1 = fast_exp2(fmaf(s[kb][hs * 8 + 2 * i + 1], scale_log2, -mc));
            lsum += p0 + p1;
            w[i] = pack_bf16x2(p0, p1);
          }
          pb[kb * 2 + hs] = __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
        }
      }
      // O^T += V^T P^T.
#pragma unroll
      for (int db = 0; db < kHeadDim / 32; ++db) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4_ptr)(vt + ks * 16 * kHeadDim + v_off[db][0]));
          const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4_ptr)(vt + ks * 16 * kHeadDim + v_off[db][1]));
          const i16x8_t a8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          o[db] = mfma32(__builtin_bit_cast(bf16x8_t, a8), pb[ks], o[db]);
        }
      }
  };
  // One pipeline step: tile t is in (kc, vc); tile t+1 goes into (kn, vn).
  auto step = [&](int t, uint16_t* kc, uint16_t* vc, uint16_t* kn, uint16_t* vn) {
    // Tile t has landed (this wavefront's copies), then everyone's have, and
    // everyone is done with the stage that tile t+1 will overwrite.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (t + 1 < num_tiles) issue_tile(t + 1, kn, vn);
    compute_tile(t, kc, vc);
  };
  issue_tile(0, lds_k0, lds_v0);
  for (int t = 0; t < num_tiles; t += 2) {
    step(t, lds_k0, lds_v0, lds_k1, lds_v1);
    if (t + 1 < num_tiles) step(t + 1, lds_k1, lds_v1, lds_k0, lds_v0);
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
  const int64_t pairs = static_cast<int64_t>(num_kv_heads) * batch;
  const int64_t blocks = (pairs + kXcds - 1) / kXcds * kXcds * q_tiles;
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

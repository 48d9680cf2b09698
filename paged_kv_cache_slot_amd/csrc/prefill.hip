// Varlen causal prefill over a paged KV cache with a cached prefix
// ("DeepSeek研究员1200行代码复刻vLLM…", section "vLLM是什么？" for the paging;
// "nano-vllm 深度分析报告", section 创新之处, for prefix caching).
//
// Sequence b has P cached tokens and N new ones (all stored in the pool); new
// row i sits at position P + i and attends to keys 0 .. P + i.
//
// Work split. One work-group (4 wavefronts) owns one (sequence, kv head,
// tile of 128/G new tokens) and all G query heads of that kv head: 128 query
// rows, 32 per wavefront. It walks the context in tiles of 64 keys. The
// work-groups of one (sequence, kv head) pair are all placed on one XCD, back
// to back, so the pair's K/V stays in that XCD's L2 while they run.
//
// Tile pipeline (two LDS stages). Each tile's K and V rows are copied from the
// pool straight into LDS (buffer/global loads with the LDS-DMA bit, 16 bytes
// per lane, no registers). A wavefront copies 16 keys, which lie in one cache
// block, from one scalar base address; keys past the context (a sequence's
// last tile) re-read token L-1 through per-lane addresses instead. While tile
// t is computed, tile t+1 is in flight. The work-group's Q rows are copied
// into the second stage together with the first tile and moved into
// registers in the first step; at the end each wavefront stages its output
// rows in the first stage, so that every global access moves whole rows.
// Inside a 256-byte row the sixteen 16-byte units are stored XOR-swizzled by
// the key index, so the MFMA operand reads below hit distinct LDS banks.
//
// Per wavefront and tile, flash-attention style, in log2 units:
//   S^T = K Q^T      bf16 MFMA 32x32x16, fp32 accumulate: each lane holds the
//                    scores of ONE query row, so row reductions stay in-lane
//                    except for one exchange with the lane 32 apart;
//   s = S * scale * log2(e) in fp32 (one fma per score, which also subtracts
//                    the reference below): the scale is never rounded into a
//                    bf16 operand, whose error would grow with |S|;
//   p = 2^(s - mc)   against a per-row reference mc, set from the first
//                    tile's row maximum and raised (rescaling the output) only
//                    when a tile's per-lane row sum of p exceeds 256, so no
//                    per-tile row maximum is needed and p stays <= 256;
//   O^T += V^T P^T   bf16 MFMA 32x32x16 with P taken straight from the S^T
//                    accumulators (converted to bf16) and V^T built by
//                    ds_read_b64_tr_b16 transposed reads from the row-major V
//                    tile, with keys ordered to match the accumulator layout;
//                    the row sum adds the fp32 exponentials.
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

// Largest per-lane share of a tile's row sum of exponentials before the row's
// reference is raised; every exponential stays below it.
constexpr float kRescaleSum = 256.f;

// v_permlane32_swap of x with itself: the first result holds the low half's
// values in both halves, the second the high half's, so a symmetric
// combination of the two gives every lane the combination of itself and the
// lane 32 apart. (The elements are copied out before the bit casts: a bit cast
// of a vector element in place reads element 0.)
__device__ __forceinline__ void halves(float x, float& lo, float& hi) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const uint32_t r0 = r[0];
  const uint32_t r1 = r[1];
  lo = __builtin_bit_cast(float, r0);
  hi = __builtin_bit_cast(float, r1);
}
__device__ __forceinline__ float max_halves(float x) {
  float lo, hi;
  halves(x, lo, hi);
  return fmaxf(lo, hi);
}
__device__ __forceinline__ float sum_halves(float x) {
  float lo, hi;
  halves(x, lo, hi);
  return lo + hi;
}

// Instruction classes of the scheduling-group hint (LLVM AMDGPU).
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;
// Asks the scheduler for `count` instructions of class `mask` next in the
// current scheduling region (groups are filled in the order they appear).
#define sched_group(mask, count) __builtin_amdgcn_sched_group_barrier((mask), (count), 0)

typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(3))) i16x4_t* lds_i16x4_ptr;

// Raw buffer resource over [base, base + 2^31): scalar base, no stride, no
// swizzle (dword 3 as for gfx9 raw buffers).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff, 0x00020000);
}

// 16 bytes per lane from a buffer into LDS at dst + 16 * lane: lane reads
// rsrc.base + soff + voff.
__device__ __forceinline__ void dma16_buf(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, int soff,
                                          uint16_t* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_ptr)(dst), 16, voff, soff, 0, 0);
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

  // This lane's query row. A wavefront's 32 rows are min(32, TQ) consecutive
  // tokens of 32 / min(32, TQ) heads.
  const int row = wave * 32 + col;
  const int hh = row / TQ;
  const int tok = row % TQ;
  const int qpos = P + tok0 + tok;                      // absolute position
  const int head = g * G + hh;
  const int wave_pos0 = P + tok0 + (wave * 32) % TQ;    // lowest position of the wavefront's rows
  const int wave_pos1 = wave_pos0 + min(32, TQ) - 1;    // highest

  // Q of this lane's row, the B operand of the score MFMAs as it is; read
  // from LDS in the first step (the rows are copied there with the first tile).
  bf16x8_t qreg[kHeadDim / 16];
  auto read_q = [&]() {
    const int lr = tok * G + hh;
    const uint16_t* qs = (lr < 64 ? lds_k1 : lds_v1) + (lr & 63) * kHeadDim;
#pragma unroll
    for (int ks = 0; ks < kHeadDim / 16; ++ks)
      qreg[ks] = *reinterpret_cast<const bf16x8_t*>(qs + (((ks * 2 + half) ^ (tok & 15)) * 8));
  };

  f32x16_t o[kHeadDim / 32];
#pragma unroll
  for (int db = 0; db < kHeadDim / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  // Softmax state of this lane's row, in log2 units: mc is the reference the
  // exponentials are taken against, p = 2^(s - mc). mc is set from the first
  // tile's row maximum and afterwards raised only when a tile's row sum of p
  // exceeds kRescaleSum, which keeps every p below that bound; the final
  // o / lsum is the same for any reference.
  float mc = 0.f;
  f32x16_t zero16;
#pragma unroll
  for (int r = 0; r < 16; ++r) zero16[r] = 0.f;
  float lsum = 0.f;

  const int bs_mask = (1 << log2_bs) - 1;
  const int32_t* bt = block_table + static_cast<int64_t>(b) * bt_stride;
  const int slot_bytes = num_kv_heads * kHeadDim * 2;  // bytes from one slot to the next

  // ---- tile loads -----------------------------------------------------------
  // A tile is 64 keys x 256 B per tensor = 16 DMA instructions of 1 KiB (4 keys
  // each); wavefront w issues instructions 4w .. 4w+3 for K and the same for V,
  // i.e. keys 16w .. 16w+15 of the tile, which lie in one cache block
  // (block_size >= 16). Lane l of an instruction carries key (4j + l/16) of
  // those and the 16-byte unit (l%16) of its LDS row, which holds logical unit
  // (l%16) ^ swz(key) of the key's 256-byte row.
  //
  // All copies are buffer loads with a scalar base: the block holding key
  // min(k0, L-1), k0 the first of the wavefront's 16 keys. Fast path (all 16
  // keys inside the context): each lane adds a fixed 32-bit offset. Keys past
  // the context (only in a sequence's last tile) re-read token L-1 instead, so
  // V never holds stale values there; the group's keys that remain, and token
  // L-1, then lie in that same block, so a per-lane offset from the same base
  // still reaches them. (With the flat-encoded global form of these copies in
  // flight the compiler no longer counts the LDS reads' waits exactly and
  // waits for all of them; with buffer loads it does count them.)
  const int dma_row = lane >> 4;
  const int dma_unit = lane & 15;
  uint32_t lane_off[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    lane_off[j] = dma_row * slot_bytes + ((dma_unit ^ swz(4 * j + dma_row)) * 16);
  const char* kbase = reinterpret_cast<const char*>(k_cache) + g * (kHeadDim * 2);
  const char* vbase = reinterpret_cast<const char*>(v_cache) + g * (kHeadDim * 2);
  // Block id of key min(first of this wavefront's keys in tile t, L-1).
  auto block_of = [&](int t) { return bt[min(t * kKeys + 16 * wave, L - 1) >> log2_bs]; };
  auto issue_tile = [&](int t, int blk, uint16_t* lk, uint16_t* lv) {
    const int k0 = t * kKeys + 16 * wave;  // first key of this wavefront's 16
    const int kfirst = min(k0, L - 1);
    uint16_t* dk = lk + 16 * wave * kHeadDim;
    uint16_t* dv = lv + 16 * wave * kHeadDim;
    const int64_t first =
        ((static_cast<int64_t>(blk) << log2_bs) | (kfirst & bs_mask)) * slot_bytes;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kbase + first);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase + first);
    if (k0 + 15 < L) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        dma16_buf(rk, lane_off[j], j * 4 * slot_bytes, dk + j * 4 * kHeadDim);
        dma16_buf(rv, lane_off[j], j * 4 * slot_bytes, dv + j * 4 * kHeadDim);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kc = min(k0 + 4 * j + dma_row, L - 1);
        const uint32_t off = (kc - kfirst) * slot_bytes + ((dma_unit ^ swz(4 * j + dma_row)) * 16);
        dma16_buf(rk, off, 0, dk + j * 4 * kHeadDim);
        dma16_buf(rv, off, 0, dv + j * 4 * kHeadDim);
      }
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

  // ---- one tile --------------------------------------------------------------
  // Computes tile t from the LDS stage (kt, vt); masked selects the causal
  // mask (diagonal tiles only).
  auto compute_tile = [&](int t, const uint16_t* kt, uint16_t* vt, bool masked) {
    // S^T for the two 32-key halves of the tile. The K operands of step ks+2
    // are read while step ks multiplies.
    auto read_k = [&](int kb, int ks) {
      const int key = kb * 32 + col;
      return *reinterpret_cast<const bf16x8_t*>(kt + key * kHeadDim +
                                                (((ks * 2 + half) ^ swz(key)) * 8));
    };
    // Issue priority: raised while this wavefront feeds the matrix core, so
    // that the other wavefront on the SIMD runs its softmax in the gaps.
    __builtin_amdgcn_s_setprio(1);
    f32x16_t s[2] = {zero16, zero16};
    bf16x8_t ka[3][2];
    ka[0][0] = read_k(0, 0);
    ka[0][1] = read_k(1, 0);
    ka[1][0] = read_k(0, 1);
    ka[1][1] = read_k(1, 1);
#pragma unroll
    for (int ks = 0; ks < kHeadDim / 16; ++ks) {
      if (ks + 2 < kHeadDim / 16) {
        ka[(ks + 2) % 3][0] = read_k(0, ks + 2);
        ka[(ks + 2) % 3][1] = read_k(1, ks + 2);
      }
      s[0] = mfma32(ka[ks % 3][0], qreg[ks], s[0]);
      s[1] = mfma32(ka[ks % 3][1], qreg[ks], s[1]);
    }
    // Keep that order: two LDS reads in flight ahead of each MFMA pair.
    sched_group(kSchedDsRead, 4);
#pragma unroll
    for (int ks = 0; ks + 2 < kHeadDim / 16; ++ks) {
      sched_group(kSchedMfma, 2);
      sched_group(kSchedDsRead, 2);
    }
    sched_group(kSchedMfma, 4);
    __builtin_amdgcn_s_setprio(0);

    // Scaled scores in log2 units, relative to the reference.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = fmaf(s[kb][r], scale_log2, -mc);

    // Mask (lane holds keys kb*32 + (r/4)*8 + half*4 + r%4 of the tile).
    if (masked) {  // one uniform branch around the whole mask
      const int rel = qpos - t * kKeys - half * 4;  // key offsets <= rel are visible
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          s[kb][r] = kb * 32 + (r >> 2) * 8 + (r & 3) <= rel ? s[kb][r] : -INFINITY;
    }
    __builtin_amdgcn_s_setprio(1);

    // P = 2^(s - mc) in bf16 as the B operand, 16 keys per MFMA step; tsum is
    // this lane's share of the tile's row sum, added in fp32 from the
    // exponentials before they are rounded to bf16. (Plain adds, not v_dot2:
    // the dot instructions do not issue while the matrix core is busy, fp32
    // adds do, beside the other wavefront's MFMAs.)
    bf16x8_t pb[4];
    float tsum;
    auto make_p = [&]() {
      float t[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
          float e[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            e[i] = fast_exp2(s[kb][hs * 8 + i]);
            t[i & 3] += e[i];
          }
          pb[kb * 2 + hs] = __builtin_bit_cast(
              bf16x8_t, make_uint4(pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3]),
                                   pack_bf16x2(e[4], e[5]), pack_bf16x2(e[6], e[7])));
        }
      }
      tsum = (t[0] + t[1]) + (t[2] + t[3]);
    };
    // The row's maximum of s - mc over this tile's visible keys.
    auto row_max = [&]() {
      float tmax = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, s[kb][r]);
      return max_halves(tmax);
    };
    // Moves the reference up to the row maximum where that is higher,
    // rescales the state and recomputes P.
    auto raise_reference = [&]() {
      const float d = fmaxf(row_max(), 0.f);
      const float alpha = fast_exp2(-d);
      mc += d;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < kHeadDim / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] -= d;
      make_p();
    };
    // The first tile sets the reference to its row maximum (every row sees
    // key 0, so it is finite) before any exponential is taken.
    if (t == 0) {
      const float m0 = row_max();
      mc = m0;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] -= m0;
    }
    make_p();
    // The sum test also catches an overflow to infinity. Per lane: each half
    // of a row stays below the bound, the row below twice it.
    if (t != 0 && __any(!(tsum <= kRescaleSum))) raise_reference();
    lsum += tsum;

    // V^T operands: two transposed reads per (32-row block db, 16-key step ks).
    auto read_v = [&](int db, int ks, int r) {
      return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4_ptr)(vt + ks * 16 * kHeadDim + v_off[db][r]));
    };
    i16x4_t tr[2][4][2];  // two db blocks in flight
#pragma unroll
    for (int d = 0; d < 2; ++d)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int r = 0; r < 2; ++r) tr[d][ks][r] = read_v(d, ks, r);

    // O^T += V^T P^T, block db from tr[db % 2]; blocks 2 and 3 are read once
    // blocks 0 and 1 have been consumed.
    auto pv = [&](int db, int ks, const i16x4_t (&v)[4][2]) {
      const i16x8_t a8 = {v[ks][0][0], v[ks][0][1], v[ks][0][2], v[ks][0][3],
                          v[ks][1][0], v[ks][1][1], v[ks][1][2], v[ks][1][3]};
      o[db] = mfma32(__builtin_bit_cast(bf16x8_t, a8), pb[ks], o[db]);
    };
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) pv(db, ks, tr[db]);
#pragma unroll
    for (int d = 0; d < 2; ++d)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int r = 0; r < 2; ++r) tr[d][ks][r] = read_v(2 + d, ks, r);
#pragma unroll
    for (int db = 2; db < 4; ++db)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) pv(db, ks, tr[db - 2]);
    // Reads of blocks 2, 3 go between the products of blocks 0, 1.
    sched_group(kSchedDsRead, 16);
    sched_group(kSchedMfma, 6);
    sched_group(kSchedDsRead, 16);
    sched_group(kSchedMfma, 10);
    __builtin_amdgcn_s_setprio(0);
  };
  auto tile = [&](int t, const uint16_t* kt, uint16_t* vt) {
    const int kstart = t * kKeys;
    if (kstart > wave_pos1) return;  // above the diagonal for every row here
    compute_tile(t, kt, vt, kstart + kKeys - 1 > wave_pos0);
  };

  // ---- pipeline ------------------------------------------------------------
  // One step: tile t is in (kc, vc); tile t+1 goes into (kn, vn). Block ids
  // are fetched one step ahead of their DMA.
  int blk_next = 0;  // block ids of the next tile's copy, fetched one step ahead
  auto step = [&](int t, uint16_t* kc, uint16_t* vc, uint16_t* kn, uint16_t* vn) {
    // Tile t has landed (this wavefront's copies), then everyone's have, and
    // everyone is done with the stage that tile t+1 will overwrite.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (t == 0) {  // Q, then everyone is past it before tile 1 overwrites stage 1
      read_q();
      __syncthreads();
    }
    if (t + 1 < num_tiles) issue_tile(t + 1, blk_next, kn, vn);
    tile(t, kc, vc);
    // Fetched after the tile so that no scalar load is in flight while the
    // tile's LDS reads are counted (scalar loads return out of order).
    blk_next = block_of(t + 2);
  };
  issue_tile(0, block_of(0), lds_k0, lds_v0);
  // The work-group's Q rows into stage 1 with the first tile, 1 KB per copy
  // (the G rows of one token are contiguous in q; rows past the sequence read
  // its last token): LDS row lr = tok * G + hh (rows 0..63 in lds_k1, 64..127
  // in lds_v1), its 16-byte unit u at u ^ (tok % 16), so that the 32 rows one
  // operand read covers spread over the banks. Loaded lane by lane, each
  // instruction would take 32 bytes of each of 32 rows.
  {
    const __amdgpu_buffer_rsrc_t rq =
        make_rsrc(q + static_cast<int64_t>(q0 + tok0) * num_q_heads * kHeadDim);
    uint16_t* const qdst = (wave < 2 ? lds_k1 : lds_v1) + (wave & 1) * 32 * kHeadDim;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int lr = wave * 32 + 4 * j + dma_row;
      const int qtok = lr / G;
      const int qrow = min(tok0 + qtok, N - 1) - tok0;
      const uint32_t voff = (static_cast<uint32_t>(qrow * num_q_heads + g * G + lr % G) * kHeadDim +
                             ((dma_unit ^ (qtok & 15)) * 8)) * 2;
      dma16_buf(rq, voff, 0, qdst + 4 * j * kHeadDim);
    }
  }
  blk_next = block_of(1);

  for (int t = 0; t < num_tiles; t += 2) {
    step(t, lds_k0, lds_v0, lds_k1, lds_v1);
    if (t + 1 < num_tiles) step(t + 1, lds_k1, lds_v1, lds_k0, lds_v0);
  }

  // Normalise and write. Lane holds d = db*32 + (r/4)*8 + half*4 + r%4 of its
  // row: written straight out, each store would put 8 bytes in each of 32
  // rows. Instead each wavefront stages its 32 rows (bf16, 8 KB) in LDS, the
  // stages being free once every wavefront is past the last tile, and reads
  // them back a row per 16 lanes, so that each store writes four whole
  // 256-byte rows. In LDS the 16-byte unit u of row r sits at u ^ (r % 16),
  // which keeps the 8-byte writes of 32 rows to two per bank.
  const float inv = 1.f / sum_halves(lsum);
  __syncthreads();
  uint16_t* const ostage = (wave < 2 ? lds_k0 : lds_v0) + (wave & 1) * 32 * kHeadDim;
#pragma unroll
  for (int db = 0; db < kHeadDim / 32; ++db) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint2 w;
      w.x = pack_bf16x2(o[db][j * 4 + 0] * inv, o[db][j * 4 + 1] * inv);
      w.y = pack_bf16x2(o[db][j * 4 + 2] * inv, o[db][j * 4 + 3] * inv);
      const int u = db * 4 + j;  // 16-byte unit of d = db*32 + j*8 .. + 7
      *reinterpret_cast<uint2*>(ostage + col * kHeadDim + ((u ^ (col & 15)) * 8) + half * 4) = w;
    }
  }
  // Read back (LDS operations of one wavefront complete in order).
  const int unit = lane & 15;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = i * 4 + (lane >> 4);  // row within the wavefront
    const uint4 v =
        *reinterpret_cast<const uint4*>(ostage + r * kHeadDim + ((unit ^ (r & 15)) * 8));
    const int rrow = wave * 32 + r;
    const int rtok = rrow % TQ;
    if (tok0 + rtok < N) {
      uint16_t* op = out + (static_cast<int64_t>(q0 + tok0 + rtok) * num_q_heads + g * G +
                            rrow / TQ) * kHeadDim;
      *reinterpret_cast<uint4*>(op + unit * 8) = v;
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

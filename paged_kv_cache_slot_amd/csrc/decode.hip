// Paged decode: one query token per sequence attends over its context, whose
// keys and values sit in fixed-size blocks reached through the sequence's
// block table ("DeepSeek研究员1200行代码复刻vLLM…", section "vLLM是什么？").
//
// Work split. Each context is cut into pieces of 512 or 1024 tokens (64 blocks at most,
// see launch_split); an item is one (piece, kv head) with all G = Hq/Hkv query
// heads that read that kv head, so every K/V byte is fetched from HBM once.
// The grid is one work-group per CU (as many wavefronts as fit), resident
// together. Every work-group derives the same global order of the items from
// context_lens -- all full pieces, then each sequence's partial last piece --
// with a cost per item (its 32-token chunks plus one), and takes the items
// whose first cost unit falls in its 1/grid share: all work-groups get the
// same cost to within one item, with no atomics in global memory. It keeps
// them in an LDS table, largest first, and its wavefronts take them from an
// LDS counter: wavefronts that run faster take more, and the small items come
// last, so they all finish together. (A counter in global memory is no good:
// under full HBM load its returned value arrives so late that the in-order
// vmcnt accounting stalls every load issued after it.)
//
// Within an item, each row of 16 lanes takes every fourth token and each lane
// a 16-byte slice (8 elements of head_dim) of that token's 256-byte kv-head
// row: one load instruction reads four whole rows. The item streams through
// chunks of CH groups of 4 tokens held in two alternating register buffers:
// the loads of the next chunk -- or of the next item's first chunk, whose
// block ids and q were fetched one item ahead -- are in flight while the
// current chunk is computed, so HBM requests never stop. After building the
// item table there is no barrier: wavefronts never wait for each other.
//
// Per token: q.k from four v_dot2c_f32_bf16 per lane, summed over the 16-lane
// row with DPP; online softmax in base 2 (scale*log2e folded in), updated once
// per chunk; p*V accumulated in fp32. At the end of an item the four rows of
// lanes are merged with the usual (max, sum, acc) rescaling; a sequence with
// one piece writes its bf16 output directly, longer ones leave (acc, max, sum)
// per piece in the workspace for the reduce kernel.
//
// Roofline: HBM. Algorithmic bytes = 2 (K and V) * L * 256 B per (sequence,
// kv head), plus q and out, which are small.
#include <algorithm>
#include <atomic>
#include <cmath>

#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kScanRows = 1024;        // rows of context_lens held in LDS at a time
constexpr int kMaxGroupItems = 4096;   // items one work-group can own (LDS table)
constexpr int kSizeClasses = 16;       // item-size classes of the largest-first order
constexpr float kLazyLog2 = 8.f;       // headroom of the softmax reference (log2 units)

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

// Scans rows [start, start + n), n = min(kScanRows, batch - start), of
// context_lens into LDS (one wavefront): s_len[i] = clamped length,
// s_pref[i] = `base` + the number of pieces of rows start .. start+i-1,
// s_pref[n] = base + all of them. A padding row (length 0) counts as one piece,
// which writes its zeros.
// One work item: piece `split` (tokens [split*256, min(L, split*256+256))) of
// sequence b, kv head g. L is the clamped context length (0: padding row) and
// nsplit the sequence's number of pieces. All fields are uniform.
struct Item {
  int valid, b, g, split, L, nsplit;
};

// Wavefronts per work-group: all that fit on a CU at once: three per SIMD for
// G <= 2 (chunks of 4 token groups), two for G = 4, one for G = 8.
template <int G>
constexpr int decode_waves() { return G >= 8 ? 4 : (G <= 2 ? 12 : 8); }

template <int G, int CH>
__global__ __launch_bounds__(64 * decode_waves<G>(), 1) void decode_kernel(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ k_cache, const uint16_t* __restrict__ v_cache,
    const int32_t* __restrict__ block_table, int32_t bt_stride,
    const int32_t* __restrict__ context_lens, int32_t batch, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t log2_bs, int32_t max_context_len, float scale_log2,
    int32_t max_splits, int32_t log2_split, float* __restrict__ ws_o, float* __restrict__ ws_ml,
    int32_t zero) {
  // `zero` is always 0. Adding it to the address of a stand-in load keeps the
  // compiler from merging that load with an identical one (and from turning
  // the stand-in back into a branch).
  constexpr int W = decode_waves<G>();
  constexpr int kThreads = 64 * W;
  const int split = 1 << log2_split;  // tokens per piece
  __shared__ int s_pref[kScanRows + 1];         // full pieces before each sequence
  __shared__ int s_len[kScanRows];              // clamped lengths
  __shared__ int4 s_items[kMaxGroupItems];      // this work-group's items: (b, piece, L, g)
  __shared__ int s_order[kMaxGroupItems];       // item indices, largest first
  __shared__ int s_class[kSizeClasses];         // per size class: count, then next slot
  __shared__ int s_misc[4];                     // [1] items handed out, [2] items owned

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = lane >> 4;  // which token of four
  const int sub = lane & 15;  // which 8-element slice of head_dim
  const int bs_mask = (1 << log2_bs) - 1;
  const int64_t slot_stride = static_cast<int64_t>(num_kv_heads) * kHeadDim;

  // ---- the item list -------------------------------------------------------
  // A launch covers at most kScanRows sequences (larger batches go in slices).
  // Sequence b has nfull_b = L_b / split full pieces and, when L_b is not a
  // multiple of split, one partial piece of r_b tokens (a padding row, L = 0,
  // has one item that writes its zeros). An item is (piece, kv head); its cost
  // is its number of 32-token chunks plus one. In the global order all full
  // items come first, in (sequence, piece, kv head) order, then the partial
  // ones in (sequence, kv head) order. Work-group i takes the items whose first
  // cost unit falls in its share [i C / grid, (i+1) C / grid) of the total C,
  // so all work-groups get the same cost to within one item; it keeps them in
  // LDS, largest first (full pieces, then partial pieces by size), so the small
  // ones come last and the wavefronts finish together.
  const int grid = static_cast<int>(gridDim.x);
  const int hkv = num_kv_heads;
  const int full_cost = (split >> 5) + 1;
  auto part_cost = [](int r) { return ((r + 31) >> 5) + 1; };  // r tokens, r < split
  constexpr int kPer = (kScanRows + kThreads - 1) / kThreads;  // sequences per thread
  int nfull[kPer], pcost[kPer];
  int fsum = 0, psum = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int b = tid * kPer + j;
    int nf = 0, pc = 0;
    if (b < batch) {
      const int L = max(0, min(context_lens[b], max_context_len));
      s_len[b] = L;
      nf = L >> log2_split;
      const int r = L - (nf << log2_split);
      pc = (r > 0 || L == 0) ? part_cost(r) : 0;
    }
    nfull[j] = nf;
    pcost[j] = pc;
    fsum += nf;
    psum += pc;
  }
  // Exclusive scans of full pieces and partial costs over the sequences.
  int fincl = fsum, pincl = psum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int fv = __shfl_up(fincl, off), pv = __shfl_up(pincl, off);
    if (lane >= off) {
      fincl += fv;
      pincl += pv;
    }
  }
  if (lane == 63) {
    s_pref[wave] = fincl;       // per-wavefront totals (s_pref reused as scratch)
    s_pref[W + wave] = pincl;
  }
  if (tid < kSizeClasses) s_class[tid] = 0;
  if (tid == 0) s_misc[2] = 0;
  __syncthreads();
  int fbase = fincl - fsum, pbase = pincl - psum, ftot = 0, ptot = 0;
  for (int w2 = 0; w2 < W; ++w2) {
    const int fw = s_pref[w2], pw = s_pref[W + w2];
    if (w2 < wave) {
      fbase += fw;
      pbase += pw;
    }
    ftot += fw;
    ptot += pw;
  }
  __syncthreads();  // s_pref is rewritten below
  int* s_fpre = s_pref;  // full pieces before sequence b (s_fpre[batch] = all)
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int b = tid * kPer + j;
    if (b < batch) s_fpre[b] = fbase;
    fbase += nfull[j];
  }
  if (tid == 0) s_fpre[batch] = ftot;
  __syncthreads();
  const int64_t full_items = static_cast<int64_t>(ftot) * hkv;
  const int64_t total = full_items * full_cost + static_cast<int64_t>(ptot) * hkv;
  const int64_t lo = total * blockIdx.x / grid, hi = total * (blockIdx.x + 1) / grid;
  auto add_item = [&](int b, int piece, int g) {
    const int slot = atomicAdd(&s_misc[2], 1);
    if (slot < kMaxGroupItems) s_items[slot] = make_int4(b, piece, s_len[b], g);
  };
  // Full items f whose first unit f * full_cost is in [lo, hi).
  const int64_t f0 = std::min<int64_t>(full_items, (lo + full_cost - 1) / full_cost);
  const int64_t f1 = std::min<int64_t>(full_items, (hi + full_cost - 1) / full_cost);
  for (int64_t f = f0 + tid; f < f1; f += kThreads) {
    const int pg = static_cast<int>(f / hkv);  // global full piece
    int blo = 0, bhi = batch - 1;             // sequence b with s_fpre[b] <= pg < s_fpre[b+1]
    while (blo < bhi) {
      const int mid = (blo + bhi + 1) >> 1;
      if (s_fpre[mid] <= pg) blo = mid; else bhi = mid - 1;
    }
    add_item(blo, pg - s_fpre[blo], static_cast<int>(f - static_cast<int64_t>(pg) * hkv));
  }
  // Partial items: (b, g) starts at full_items * full_cost + hkv * pbase_b + g * pcost_b.
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int b = tid * kPer + j;
    const int pb0 = pbase;
    pbase += pcost[j];
    if (b >= batch || pcost[j] == 0) continue;
    for (int g = 0; g < hkv; ++g) {
      const int64_t st = full_items * full_cost + static_cast<int64_t>(hkv) * pb0 +
                         static_cast<int64_t>(g) * pcost[j];
      if (st >= lo && st < hi) add_item(b, nfull[j], g);
    }
  }
  __syncthreads();
  const int nitems = min(kMaxGroupItems, s_misc[2]);
  // Largest first: a counting sort over size classes (class kSizeClasses-1
  // holds the full pieces and the padding rows).
  auto size_class = [&](int4 it) {
    const int tokens = it.z > 0 ? min(split, it.z - it.y * split) : split;
    return min(kSizeClasses - 1, (tokens * kSizeClasses - 1) >> log2_split);
  };
  for (int k = tid; k < nitems; k += kThreads) atomicAdd(&s_class[size_class(s_items[k])], 1);
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    for (int c = kSizeClasses - 1; c >= 0; --c) {
      const int cnt = s_class[c];
      s_class[c] = acc;
      acc += cnt;
    }
    s_misc[1] = 0;
  }
  __syncthreads();
  for (int k = tid; k < nitems; k += kThreads)
    s_order[atomicAdd(&s_class[size_class(s_items[k])], 1)] = k;
  __syncthreads();  // the last work-group barrier: from here on wavefronts run independently

  // The rank-th item (largest first). Past the last item it returns
  // `fallback` marked invalid, so that the loads issued for it still read
  // valid memory.
  auto lookup = [&](int rank, Item fallback) -> Item {
    fallback.valid = 0;
    if (rank >= nitems) return fallback;
    const int4 e = s_items[__builtin_amdgcn_readfirstlane(s_order[rank])];
    Item it;
    it.valid = 1;
    it.b = __builtin_amdgcn_readfirstlane(e.x);
    it.split = __builtin_amdgcn_readfirstlane(e.y);
    it.L = __builtin_amdgcn_readfirstlane(e.z);
    it.g = __builtin_amdgcn_readfirstlane(e.w);
    it.nsplit = max(1, (it.L + split - 1) >> log2_split);
    return it;
  };
  // Every path issues the same vector loads in the same order (a load that is
  // not needed reads the item's own q row instead of being skipped): the
  // compiler's wait counts are then exact on every path, and a prefetch is never
  // waited for early.
  auto q_row = [&](const Item& it) -> const uint16_t* {
    return q + (static_cast<int64_t>(it.b) * num_q_heads + it.g * G) * kHeadDim + sub * 8;
  };
  // The item's block ids: lane l holds the block-table entry (first block of
  // the piece) + l, clamped into the row (entries past the context are never
  // used). A piece spans at most 64 blocks (the host keeps the piece size at
  // or below 64 blocks), and each group of 4 tokens lies in one block.
  auto load_blocks = [&](const Item& it) -> int {
    const int bidx0 = (it.split << log2_split) >> log2_bs;
    const int32_t* src = it.L > 0 ? block_table + static_cast<int64_t>(it.b) * bt_stride +
                                        min(bidx0 + lane, bt_stride - 1)
                                  : reinterpret_cast<const int32_t*>(q_row(it) + zero);
    return *src;
  };
  auto load_q = [&](const Item& it, uint32_t (&qv)[G][4]) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const uint4 t = *reinterpret_cast<const uint4*>(q_row(it) + hh * kHeadDim);
      qv[hh][0] = t.x; qv[hh][1] = t.y; qv[hh][2] = t.z; qv[hh][3] = t.w;
    }
  };

  // ---- one chunk: loads, then arithmetic ------------------------------------
  // Chunk c of an item covers tokens t0 + 4*CH*c .. t0 + 4*CH*c + 4*CH - 1; row
  // grp of lanes takes token (first + 4j + grp) for j < CH. Groups past the
  // context re-read the chunk's first token (cached), tokens past the context
  // inside the last group re-read token L-1 of the same block, and a chunk with
  // no tokens at all reads the item's q row.
  auto issue = [&](const Item& it, int my_blk, int c, uint4 (&kb)[CH], uint4 (&vb)[CH]) {
    const int t0 = it.split << log2_split;
    const int cbase = t0 + c * CH * 4;
    const bool active = cbase < it.L;  // uniform
    const int bidx0 = t0 >> log2_bs;
    const int ngroups = min(CH, (it.L - cbase + 3) >> 2);
    const int64_t head_off = it.g * kHeadDim + sub * 8;
    const int blk0 = __builtin_amdgcn_readlane(my_blk, (cbase >> log2_bs) - bidx0);
    const int64_t off0 =
        ((static_cast<int64_t>(blk0) << log2_bs) | (min(cbase + grp, it.L - 1) & bs_mask)) *
            slot_stride + head_off;
    const uint16_t* dummy = q_row(it) + zero;
    const uint16_t* kp[CH];
    const uint16_t* vp[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int tw = cbase + 4 * j;
      const int blk = __builtin_amdgcn_readlane(my_blk, (tw >> log2_bs) - bidx0);
      const int tc = min(tw + grp, it.L - 1);
      const int64_t o =
          ((static_cast<int64_t>(blk) << log2_bs) | (tc & bs_mask)) * slot_stride + head_off;
      const int64_t off = j < ngroups ? o : off0;
      kp[j] = active ? k_cache + off : dummy;
      vp[j] = active ? v_cache + off : dummy;
    }
#pragma unroll
    for (int j = 0; j < CH; ++j) kb[j] = load_stream(kp[j]);
#pragma unroll
    for (int j = 0; j < CH; ++j) vb[j] = load_stream(vp[j]);
    // The chunk's loads leave before any arithmetic of the previous chunk.
    __builtin_amdgcn_sched_barrier(0);
  };

  float m[G], l[G], acc[G][8];
  auto reset = [&]() {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      m[hh] = -INFINITY;
      l[hh] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[hh][e] = 0.f;
    }
  };
  auto compute = [&](const Item& it, int c, const uint32_t (&qv)[G][4], const uint4 (&kb)[CH],
                     const uint4 (&vb)[CH]) {
    const int cbase = (it.split << log2_split) + c * CH * 4;
    if (cbase >= it.L) return;  // uniform
    float s[CH][G];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const bool valid = cbase + 4 * j + grp < it.L;
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        float d = dot2_bf16(qv[hh][0], kb[j].x, 0.f);
        d = dot2_bf16(qv[hh][1], kb[j].y, d);
        d = dot2_bf16(qv[hh][2], kb[j].z, d);
        d = dot2_bf16(qv[hh][3], kb[j].w, d);
        d = row16_sum(d) * scale_log2;
        s[j][hh] = valid ? d : -INFINITY;
      }
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float cm = s[0][hh];
#pragma unroll
      for (int j = 1; j < CH; ++j) cm = fmaxf(cm, s[j][hh]);
      // m is the reference of this lane's (acc, l), -inf until it sees a token.
      // It is raised only when a chunk's maximum exceeds it by more than
      // kLazyLog2, so p <= 2^kLazyLog2 and the rescale is rare.
      const bool raise = cm > m[hh] + kLazyLog2;
      if (__any(raise)) {
        const float alpha = raise ? fast_exp2(m[hh] - cm) : 1.f;  // 0 from -inf
        m[hh] = raise ? cm : m[hh];
        l[hh] *= alpha;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[hh][e] *= alpha;
      }
      const float mu = m[hh] == -INFINITY ? 0.f : m[hh];  // no token yet: every s is -inf
#pragma unroll
      for (int j = 0; j < CH; ++j) {
        const float p = fast_exp2(s[j][hh] - mu);
        s[j][hh] = p;
        l[hh] += p;
      }
    }
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const uint4 vj = vb[j];  // p = 0 for tokens past the context
      const float v[8] = {bf16_lo(vj.x), bf16_hi(vj.x), bf16_lo(vj.y), bf16_hi(vj.y),
                          bf16_lo(vj.z), bf16_hi(vj.z), bf16_lo(vj.w), bf16_hi(vj.w)};
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[hh][e] += s[j][hh] * v[e];
      }
    }
  };

  // ---- end of an item: merge the rows of lanes, write ----------------------
  auto finalize = [&](const Item& it) {
    const int64_t bh0 = static_cast<int64_t>(it.b) * num_q_heads + it.g * G;
    if (it.L <= 0) {  // padding row: zeros
      for (int e = lane; e < G * kHeadDim; e += 64) out[bh0 * kHeadDim + e] = 0;
      return;
    }
#pragma unroll
    for (int mask = 16; mask <= 32; mask <<= 1) {  // rows of lanes 16 and 32 apart
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
    if (grp != 0) return;  // every row now holds the merged state; row 0 writes it
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const int64_t bh = bh0 + hh;
      if (it.nsplit == 1) {
        const float inv = 1.f / l[hh];
        uint4 w;
        w.x = pack_bf16x2(acc[hh][0] * inv, acc[hh][1] * inv);
        w.y = pack_bf16x2(acc[hh][2] * inv, acc[hh][3] * inv);
        w.z = pack_bf16x2(acc[hh][4] * inv, acc[hh][5] * inv);
        w.w = pack_bf16x2(acc[hh][6] * inv, acc[hh][7] * inv);
        store_stream(out + bh * kHeadDim + sub * 8, w);
      } else {
        const int64_t piece = bh * max_splits + it.split;
        float* dst = ws_o + piece * kHeadDim + sub * 8;
        store_stream(dst, make_float4(acc[hh][0], acc[hh][1], acc[hh][2], acc[hh][3]));
        store_stream(dst + 4, make_float4(acc[hh][4], acc[hh][5], acc[hh][6], acc[hh][7]));
        if (sub == 0) {
          ws_ml[piece * 2] = m[hh];
          ws_ml[piece * 2 + 1] = l[hh];
        }
      }
    }
  };

  // ---- the pipeline ---------------------------------------------------------
  // Two item slots, A and B, alternate: while one item is processed, the other
  // holds the next item (block ids, q and first chunk already requested). The
  // slot of the finished item is then refilled with the item after that. The
  // loop body is unrolled over the two slots so that no register holding an
  // in-flight load is ever copied (a copy would wait for the load).
  //
  // Wavefront j takes the work-group's items of rank j and W + j first; every
  // later rank comes from the work-group's LDS counter, fetched when the item
  // two places before it starts, so wavefronts that run faster take more.
  Item ia = lookup(wave, Item{0, 0, 0, 0, 0, 0});
  if (ia.valid) {
  int blk_a = load_blocks(ia);
  uint32_t q_a[G][4], q_b[G][4];
  load_q(ia, q_a);
  uint4 kr0[CH], vr0[CH], kr1[CH], vr1[CH];
  issue(ia, blk_a, 0, kr0, vr0);
  Item ib = lookup(W + wave, ia);
  int blk_b = load_blocks(ib);
  load_q(ib, q_b);

  // Processes `cur` (its first chunk in flight in buffer 0), requests `nxt`'s
  // first chunk, then refills cur's slot with the item after `nxt`. Returns
  // false when `nxt` does not exist.
  auto run = [&](Item& cur, int& cur_blk, uint32_t (&qc)[G][4], const Item& nxt, int nxt_blk)
      -> bool {
    int grabbed = 0;  // lane 0: rank - 2W of the item that will refill this slot
    if (lane == 0) grabbed = atomicAdd(&s_misc[1], 1);
    reset();
    const int t0 = cur.split << log2_split;
    const int ntok = min(cur.L, t0 + split) - t0;  // <= 0 on a padding row
    const int nch = max(0, (ntok + 4 * CH - 1) / (4 * CH));
    for (int c = 0;; c += 2) {
      issue(cur, cur_blk, c + 1, kr1, vr1);
      compute(cur, c, qc, kr0, vr0);
      // Next: chunk c+2 of this item, or the next item's first chunk.
      const bool last = c + 2 >= nch;
      issue(last ? nxt : cur, last ? nxt_blk : cur_blk, last ? 0 : c + 2, kr0, vr0);
      compute(cur, c + 1, qc, kr1, vr1);
      if (last) break;
    }
    finalize(cur);
    if (!nxt.valid) return false;
    cur = lookup(2 * W + __builtin_amdgcn_readfirstlane(grabbed), nxt);
    cur_blk = load_blocks(cur);
    load_q(cur, qc);
    return true;
  };
  for (;;) {
    if (!run(ia, blk_a, q_a, ib, blk_b)) break;
    if (!run(ib, blk_b, q_b, ia, blk_a)) break;
  }
  }
}

// Merges the pieces of sequences with more than one piece: one wavefront per
// (sequence, query head), two elements of head_dim per lane, four wavefronts
// per work-group.
constexpr int kReduceRows = 4;
__global__ __launch_bounds__(64 * kReduceRows) void decode_reduce_kernel(
    uint16_t* __restrict__ out, const int32_t* __restrict__ context_lens, int32_t rows,
    int32_t num_q_heads, int32_t max_context_len, int32_t max_splits, int32_t log2_split,
    const float* __restrict__ ws_o, const float* __restrict__ ws_ml) {
  const int64_t bh = static_cast<int64_t>(blockIdx.x) * kReduceRows + (threadIdx.x >> 6);
  if (bh >= rows) return;
  const int b = static_cast<int>(bh / num_q_heads);
  const int L = min(context_lens[b], max_context_len);
  const int nsplit = min((L + (1 << log2_split) - 1) >> log2_split, max_splits);
  if (nsplit <= 1) return;  // written by the split kernel (or a padding row)
  const int d = (threadIdx.x & 63) * 2;
  const float* ml = ws_ml + bh * max_splits * 2;
  float M = -INFINITY;
  for (int i = 0; i < nsplit; ++i) M = fmaxf(M, ml[2 * i]);
  float o0 = 0.f, o1 = 0.f, lt = 0.f;
  for (int i = 0; i < nsplit; ++i) {
    const float a = fast_exp2(ml[2 * i] - M);
    const float2 v = *reinterpret_cast<const float2*>(ws_o + (bh * max_splits + i) * kHeadDim + d);
    lt += a * ml[2 * i + 1];
    o0 += a * v.x;
    o1 += a * v.y;
  }
  const float inv = 1.f / lt;
  *reinterpret_cast<uint32_t*>(out + bh * kHeadDim + d) = pack_bf16x2(o0 * inv, o1 * inv);
}

// Pieces per context of max_context_len tokens, for pieces of 2^log2_split.
int max_splits_for(int32_t max_context_len, int log2_split) {
  return max(1, (max_context_len + (1 << log2_split) - 1) >> log2_split);
}

// Work-groups of decode_kernel<G, CH> resident at once on the current device
// (occupancy x compute units), computed once per device and G.
template <int G, int CH>
int resident_groups() {
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_kernel<G, CH>,
                                                   64 * decode_waves<G>(), 0) !=
          hipSuccess || per_cu <= 0)
    per_cu = 1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  v = per_cu * cus;
  cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

// One launch of the split kernel (and the reduce, if needed) over the first
// sequences of `batch`: at most kScanRows of them, and few enough that no
// work-group can own more than kMaxGroupItems items (a work-group's share of
// the cost, over the cheapest item's cost). Returns the number of sequences
// handled (the caller goes on with the rest).
template <int G, int CH>
int launch_split(uint16_t* out, const uint16_t* q, const uint16_t* k_cache,
                 const uint16_t* v_cache, const int32_t* block_table, int32_t bt_stride,
                 const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
                 int32_t num_kv_heads, int32_t log2_bs, int32_t max_context_len, float scale_log2,
                 float* workspace, hipStream_t stream, hipError_t* err) {
  constexpr int W = decode_waves<G>();
  const int groups = resident_groups<G, CH>();
  // 512-token pieces; 1024 for batches of more than 4096 (sequence, kv head)
  // pairs, whose work-groups own enough items that the per-item cost matters
  // more than the finer balance (measured: configs 2 and 3 prefer 512, the
  // 1024-sequence block-16 batch 1024). Never more than 64 blocks.
  const int log2_split =
      std::min(static_cast<int64_t>(batch) * num_kv_heads > 4096 ? 10 : 9, log2_bs + 6);
  const int64_t per_seq = static_cast<int64_t>(num_kv_heads) *
                          max_splits_for(max_context_len, log2_split) *
                          ((1 << (log2_split - 5)) + 1);  // items x highest item cost
  const int64_t nb_max = static_cast<int64_t>(kMaxGroupItems - 4) * groups / per_seq;
  const int nb = static_cast<int>(std::min<int64_t>({batch, kScanRows, nb_max}));
  if (nb <= 0) {
    *err = hipErrorInvalidValue;
    return 0;
  }
  auto items_for = [&](int lg, int64_t n) {
    return n * num_kv_heads * max_splits_for(max_context_len, lg);
  };
  const int max_splits = max_splits_for(max_context_len, log2_split);
  float* ws_o = workspace;
  float* ws_ml = ws_o + static_cast<size_t>(nb) * num_q_heads * max_splits * kHeadDim;
  // Never more wavefronts than items.
  const int64_t blocks = std::min<int64_t>((items_for(log2_split, nb) + W - 1) / W, groups);
  hipLaunchKernelGGL((decode_kernel<G, CH>), dim3(static_cast<uint32_t>(blocks)), dim3(64 * W),
                     0, stream, out, q, k_cache, v_cache, block_table, bt_stride, context_lens,
                     nb, num_q_heads, num_kv_heads, log2_bs, max_context_len, scale_log2,
                     max_splits, log2_split, ws_o, ws_ml, 0);
  *err = hipGetLastError();
  if (*err == hipSuccess && max_splits > 1) {
    const int64_t rows = static_cast<int64_t>(nb) * num_q_heads;
    hipLaunchKernelGGL(decode_reduce_kernel,
                       dim3(static_cast<uint32_t>((rows + kReduceRows - 1) / kReduceRows)),
                       dim3(64 * kReduceRows), 0, stream, out, context_lens,
                       static_cast<int32_t>(rows), num_q_heads, max_context_len, max_splits,
                       log2_split, ws_o, ws_ml);
    *err = hipGetLastError();
  }
  return nb;
}

}  // namespace

void prepare_decode(int32_t num_q_heads, int32_t num_kv_heads) {
  switch (num_q_heads / num_kv_heads) {
    case 1: resident_groups<1, 4>(); break;
    case 2: resident_groups<2, 4>(); break;
    case 4: resident_groups<4, 4>(); break;
    case 8: resident_groups<8, 2>(); break;
    default: break;
  }
}

size_t decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t max_context_len) {
  // Sized for the smallest piece (the most pieces); larger pieces need less.
  const size_t pieces = static_cast<size_t>(batch) * num_q_heads *
                        max_splits_for(max_context_len, __builtin_ctz(kDecodeSplit));
  return pieces * (kHeadDim + 2) * sizeof(float);
}

hipError_t launch_decode(uint16_t* out, const uint16_t* q, const uint16_t* k_cache,
                         const uint16_t* v_cache, const int32_t* block_table,
                         int32_t block_table_stride, const int32_t* context_lens, int32_t batch,
                         int32_t num_q_heads, int32_t num_kv_heads, int32_t block_size,
                         int32_t max_context_len, float scale, void* workspace,
                         hipStream_t stream) {
  const int log2_bs = __builtin_ctz(static_cast<unsigned>(block_size));
  const float scale_log2 = scale * kLog2e;
  const int G = num_q_heads / num_kv_heads;
  hipError_t err = hipSuccess;
  // Consecutive launches over slices of the sequences, in stream order, each
  // using the workspace from its start (the previous slice is merged by then).
  for (int b0 = 0; b0 < batch && err == hipSuccess;) {
    const int64_t row = static_cast<int64_t>(b0) * num_q_heads * kHeadDim;
    int done = 0;
#define PA_DECODE_CASE(GG, CC)                                                              \
  case GG:                                                                                 \
    done = launch_split<GG, CC>(out + row, q + row, k_cache, v_cache,                      \
                                block_table + static_cast<int64_t>(b0) * block_table_stride, \
                                block_table_stride, context_lens + b0, batch - b0,         \
                                num_q_heads, num_kv_heads, log2_bs, max_context_len,       \
                                scale_log2, static_cast<float*>(workspace), stream, &err); \
    break;
  switch (G) {
    PA_DECODE_CASE(1, 4)
    PA_DECODE_CASE(2, 4)
    PA_DECODE_CASE(4, 4)
    PA_DECODE_CASE(8, 2)
    default:
      return hipErrorInvalidValue;
  }
#undef PA_DECODE_CASE
    if (done <= 0) return hipErrorInvalidValue;
    b0 += done;
  }
  return err;
}

}  // namespace pa

// Paged decode: one query token per sequence attends over its context, whose
// keys and values sit in fixed-size blocks reached through the sequence's
// block table ("DeepSeek研究员1200行代码复刻vLLM…", section "vLLM是什么？").
//
// Work split (stream-K). The work is one long line of cost units: the
// (sequence, kv head) pairs in order, each costing its chunks of 4*CH tokens
// plus kPairCost units of per-pair overhead (a padding row, length 0, costs
// only those). Every wavefront of the grid -- one work-group per CU, all
// resident -- takes a contiguous range of that line (of equal cost, but for
// a smaller share on the slower odd XCDs) and walks it,
// cutting pairs at chunk boundaries where its range starts or ends. A pair
// that a wavefront covers entirely gets its bf16 output written directly; the
// pieces of a pair cut by range boundaries leave (acc, max, sum) partials in
// the workspace (at most two per wavefront: its first and its last pair), and
// decode_merge_kernel combines them. Every wavefront gets its weighted share
// to within one unit, without atomics or work queues; every work-group derives
// the whole partition from context_lens, which it scans into LDS. Wavefronts
// that share a SIMD do not progress at the same rate, so each posts its
// progress in LDS and one behind its work-group's mean raises its issue
// priority.
//
// An item (one pass of the pipeline) is a segment of a pair: up to 64 cache
// blocks of its chunks. Within a segment each row of 16 lanes takes every
// fourth token and each lane a 16-byte slice (8 elements of head_dim) of that
// token's 256-byte kv-head row: one load instruction reads four whole rows.
// The segment streams through chunks of CH groups of 4 tokens held in two
// alternating register buffers: the loads of the next chunk -- or of the next
// segment's first chunk, whose block ids and q were fetched one segment ahead
// -- are in flight while the current chunk is computed, so HBM requests never
// stop. After the LDS scan there is no barrier: wavefronts never wait for
// each other.
//
// Per token: q.k from four v_dot2c_f32_bf16 per lane, summed over the 16-lane
// row with DPP; online softmax in base 2 (scale*log2e folded in), updated once
// per chunk; p*V accumulated in fp32. At the end of a pair the four rows of
// lanes are merged with the usual (max, sum, acc) rescaling.
//
// Each wavefront also records, at its start, the merge job of the range
// boundary at its first unit (which pair it cuts, which wavefronts hold the
// pieces), so that the merge reads its job in one round of loads.
//
// With a fused store (the decode step's pa_store_kvcache folded in), the
// wavefront holding a pair's last chunk reads the new token (position L - 1)
// from the step's input rows, and the merge kernel, which runs next, writes
// those rows into the pool slots they belong in. (A store issued inside the
// chunk loop would hold up the loads behind it: vmcnt counts stores too, in
// order, so the next chunk's wait would also wait for the store's
// acknowledgement.)
//
// Roofline: HBM. Algorithmic bytes = 2 (K and V) * L * 256 B per (sequence,
// kv head), plus q and out, which are small (plus the new tokens' rows written
// into the pools when the store is fused).
#include <algorithm>
#include <atomic>
#include <cmath>

#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kScanRows = 1024;        // sequences per launch (their lengths sit in LDS)
constexpr int kPairCost = 2;           // per-(sequence, kv head) overhead, in chunk units
constexpr int kFullUnits = 16;         // cost units per wavefront once kFillWaves are busy
constexpr int kFewUnits = 4;           // fewest cost units a wavefront is given
constexpr int64_t kFillWaves = 2048;   // working wavefronts that keep HBM streaming
constexpr float kLazyLog2 = 8.f;       // headroom of the softmax reference (log2 units)
constexpr int kRecord = 132;           // floats per partial record: acc[128], max, sum, pad
constexpr int kInfoOffset = 64;        // workspace bytes before the per-wavefront records
constexpr int kMergeWaves = 4;         // wavefronts per work-group of the merge (small groups
                                       // spread its latency-bound jobs over every CU)

// Working wavefronts for a cost line of C units, before the grid's cap. A
// wavefront is given kFullUnits units; when that leaves fewer than kFillWaves
// wavefronts, it is given fewer (down to kFewUnits): a small batch is bound by
// the latency of each wavefront's chain of chunks, not by HBM, and the extra
// pieces cost only their merge. Non-decreasing in C.
__host__ __device__ inline int64_t wave_target(int64_t C) {
  const int64_t few = C / kFewUnits;
  const int64_t fill = few < kFillWaves ? few : kFillWaves;
  const int64_t full = C / kFullUnits;
  return full > fill ? full : fill;
}

// Workspace layout. Header (int64): the total cost C and the number of working
// wavefronts nw. Then per wavefront w < nw, the merge job of the range
// boundary at w's first unit, four int64: sequence, kv head, the first
// wavefront w_a holding a piece of that pair, and (pieces | slot of w_a's
// piece << 32), with 0 pieces where w is not the last boundary cutting the
// pair. Then per wavefront two partial slots (0: its first pair, 1: its last
// pair), each G records of kRecord floats, one per query head of the pair.
__host__ __device__ constexpr size_t partial_offset(int64_t nw) {
  return kInfoOffset + static_cast<size_t>(nw) * 4 * sizeof(int64_t);
}

// 16-byte store of a result: streaming (non-temporal) or plain (written back
// through L2). Either way vmcnt counts it, in order, so the first wait after
// it also waits for its acknowledgement, which L2 gives sooner than memory;
// but plain stores take L2 lines from the read stream. Measured on the decode
// call: plain is 1.2% faster at G = 2, streaming 2.5-3.6% faster at G = 4.
template <bool kStream>
__device__ __forceinline__ void store16(void* p, uint4 x) {
  if constexpr (kStream) {
    const u32x4_t v = {x.x, x.y, x.z, x.w};
    __builtin_nontemporal_store(v, static_cast<u32x4_t*>(p));
  } else {
    *static_cast<uint4*>(p) = x;
  }
}
__device__ __forceinline__ uint4 bits4(float a, float b, float c, float d) {
  return make_uint4(__float_as_uint(a), __float_as_uint(b), __float_as_uint(c), __float_as_uint(d));
}

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

// One segment: tokens [t0, tend) of pair (b, g), tend <= L (the clamped
// context length; 0 on a padding row). first: the wavefront starts its work on
// the pair here (reset the state); last: it ends it here (write out); whole:
// the wavefront covers every chunk of the pair (bf16 output, else a partial in
// slot `slot`). An invalid segment keeps the fields of a real row so that the
// loads issued for it read valid memory.
struct Seg {
  int valid, b, g, L, t0, tend, first, last, whole, slot;
};

// Wavefronts per work-group (one work-group per CU): two per SIMD for G <= 4,
// one for G = 8 (whose registers take a whole SIMD). Three per SIMD fit at
// G <= 2, but measured 2.2-2.3% slower: the first wavefront of each SIMD
// finished well ahead of the other two.
template <int G>
constexpr int decode_waves() { return G >= 8 ? 4 : 8; }

template <int G, int CH>
__global__ __launch_bounds__(64 * decode_waves<G>(), 1) void decode_kernel(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ k_cache, const uint16_t* __restrict__ v_cache,
    const int32_t* __restrict__ block_table, int32_t bt_stride,
    const int32_t* __restrict__ context_lens, int32_t batch, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t log2_bs, int32_t max_context_len, float scale_log2,
    char* __restrict__ ws, int32_t zero, const uint16_t* __restrict__ k_new,
    const uint16_t* __restrict__ v_new, int64_t kv_stride,
    const int32_t* __restrict__ slot_mapping) {
  // `zero` is always 0. Adding it to the address of a stand-in load keeps the
  // compiler from merging that load with an identical one (and from turning
  // the stand-in back into a branch).
  //
  // Fused store (slot_mapping != nullptr): row b's new token, at position
  // L - 1, has its K/V in k_new/v_new row b and belongs in pool slot
  // slot_mapping[b] (-1: already stored). The wavefront holding a pair's last
  // chunk reads that token from k_new/v_new instead of the pool; the merge
  // kernel writes it into the pool afterwards, and nothing in this kernel
  // reads that slot.
  constexpr int W = decode_waves<G>();
  constexpr int kThreads = 64 * W;
  constexpr int T = 4 * CH;  // tokens per chunk
  __shared__ int64_t s_pref[kScanRows + 1];  // cost units before sequence b (s_pref[batch] = C)
  __shared__ int s_len[kScanRows];           // clamped lengths
  __shared__ int64_t s_tot[W];               // per-wavefront sums of the scan
  __shared__ int s_prog[W];                  // chunks done so far, per wavefront

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = lane >> 4;  // which token of four
  const int sub = lane & 15;  // which 8-element slice of head_dim
  const int bs_mask = (1 << log2_bs) - 1;
  const int64_t slot_stride = static_cast<int64_t>(num_kv_heads) * kHeadDim;
  const int hkv = num_kv_heads;

  // ---- the cost line ---------------------------------------------------------
  // Sequence b (clamped length L_b) contributes hkv pairs of n_b + kPairCost
  // units each, n_b = ceil(L_b / T); pair (b, g) holds units
  // [s_pref[b] + g (n_b + kPairCost), ... + n_b + kPairCost), its overhead
  // units first, then chunk c at unit + kPairCost + c.
  constexpr int kPer = (kScanRows + kThreads - 1) / kThreads;  // sequences per thread
  int64_t cst[kPer];
  int64_t csum = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int b = tid * kPer + j;
    int64_t c = 0;
    if (b < batch) {
      const int L = max(0, min(context_lens[b], max_context_len));
      s_len[b] = L;
      c = static_cast<int64_t>(hkv) * ((L + T - 1) / T + kPairCost);
    }
    cst[j] = c;
    csum += c;
  }
  int64_t incl = csum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t v = __shfl_up(incl, off);
    if (lane >= off) incl += v;
  }
  if (lane == 63) s_tot[wave] = incl;
  __syncthreads();
  int64_t base = incl - csum, C = 0;
  for (int w2 = 0; w2 < W; ++w2) {
    const int64_t t = s_tot[w2];
    if (w2 < wave) base += t;
    C += t;
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int b = tid * kPer + j;
    if (b < batch) s_pref[b] = base;
    base += cst[j];
  }
  if (tid == 0) s_pref[batch] = C;
  if (tid < W) s_prog[tid] = 0;
  __syncthreads();  // the only work-group barriers: from here on wavefronts run independently

  const int64_t nw = std::max<int64_t>(
      1, std::min<int64_t>(static_cast<int64_t>(gridDim.x) * W, wave_target(C)));
  int64_t* hdr = reinterpret_cast<int64_t*>(ws);
  int64_t* info = reinterpret_cast<int64_t*>(ws + kInfoOffset);
  float* part = reinterpret_cast<float*>(ws + partial_offset(nw));
  if (blockIdx.x == 0 && tid == 0) {
    hdr[0] = C;
    hdr[1] = nw;
  }
  const int gw = static_cast<int>(blockIdx.x) * W + wave;
  if (gw >= nw) return;
  // Range weights: a wavefront of a work-group on an odd XCD (odd work-group
  // index; work-group i runs on XCD i % 8) gets kWOdd / kWEven of the
  // others' share. On MI355X the odd XCDs stream about 7% slower than the
  // even ones (median finish times of the decode's wavefronts, every box
  // measured), so equal shares leave them finishing last. cumw(w) is the
  // total weight of wavefronts 0 .. w-1; wavefront w takes units
  // [lo_of(w), lo_of(w + 1)) of the line.
  constexpr int64_t kWEven = 16, kWOdd = 15;
  auto cumw = [&](int64_t w) -> int64_t {
    const int64_t i = w / W, j = w % W;
    return W * (((i + 1) >> 1) * kWEven + (i >> 1) * kWOdd) + j * ((i & 1) ? kWOdd : kWEven);
  };
  const int64_t wtot = cumw(nw);
  auto lo_of = [&](int64_t w) -> int64_t { return C * cumw(w) / wtot; };
  // The wavefront whose range holds unit u: the largest w with
  // lo_of(w) <= u, i.e. with cumw(w) <= t below, found by inverting cumw
  // (pairs of work-groups weigh W * (kWEven + kWOdd) together).
  auto wave_of = [&](int64_t u) -> int64_t {
    const int64_t t = ((u + 1) * wtot + C - 1) / C - 1;
    const int64_t pw = W * (kWEven + kWOdd);
    const int64_t p = t / pw;
    int64_t r = t - p * pw;
    int64_t w;
    if (r >= W * kWEven) {
      r -= W * kWEven;
      w = (2 * p + 1) * W + std::min<int64_t>(W - 1, r / kWOdd);
    } else {
      w = 2 * p * W + r / kWEven;
    }
    return std::min<int64_t>(w, nw - 1);
  };
  const int64_t lo = lo_of(gw), hi = lo_of(gw + 1);

  // ---- the walk over this wavefront's range -------------------------------
  int wb, wg, wL, wn, cn, started, pair_c0;
  int64_t P0;
  {
    int blo = 0, bhi = batch - 1;  // the sequence whose units hold `lo`
    while (blo < bhi) {
      const int mid = (blo + bhi + 1) >> 1;
      if (s_pref[mid] <= lo) blo = mid; else bhi = mid - 1;
    }
    wb = blo;
    wL = s_len[wb];
    wn = (wL + T - 1) / T;
    wg = static_cast<int>((lo - s_pref[wb]) / (wn + kPairCost));
    P0 = s_pref[wb] + static_cast<int64_t>(wg) * (wn + kPairCost);
    cn = static_cast<int>(std::max<int64_t>(0, lo - (P0 + kPairCost)));
    started = 0;
    pair_c0 = 0;
    if (lane == 0) {
      // The boundary at lo merges its pair when it cuts the pair's chunks and
      // no later boundary does. Pieces of wavefronts after w_a start with the
      // pair (slot 0); w_a's piece is its last pair unless the pair began
      // where its range begins.
      const int64_t P1 = P0 + wn + kPairCost;
      int64_t wa = 0, job = 0;
      if (P0 + kPairCost < lo && lo < P1 && hi >= P1) {
        wa = wave_of(P0 + kPairCost);
        const int64_t slot_wa = lo_of(wa) >= P0 ? 0 : 1;
        job = (gw - wa + 1) | (slot_wa << 32);
      }
      info[4 * gw + 0] = wb;
      info[4 * gw + 1] = wg;
      info[4 * gw + 2] = wa;
      info[4 * gw + 3] = job;
    }
  }
  auto advance = [&]() {
    if (++wg == hkv) {
      wg = 0;
      ++wb;
      if (wb < batch) {
        wL = s_len[wb];
        wn = (wL + T - 1) / T;
        P0 = s_pref[wb];
      } else {
        P0 = C;
      }
    } else {
      P0 += wn + kPairCost;
    }
    cn = 0;
    started = 0;
  };
  // The next segment of the range (invalid past its end, with the fields of
  // `fallback`).
  auto next_seg = [&](Seg fallback) -> Seg {
    fallback.valid = 0;
    for (;;) {
      if (wb >= batch || P0 >= hi) return fallback;
      if (wn == 0) {  // padding row: written by the wavefront holding its first unit
        const bool mine = P0 >= lo;
        const Seg s{1, wb, wg, 0, 0, 0, 1, 1, 1, 0};
        advance();
        if (mine) return s;
        continue;
      }
      const int64_t lim64 = std::min<int64_t>(wn, hi - (P0 + kPairCost));
      if (lim64 <= cn) {  // no (further) chunk of this pair in the range
        advance();
        continue;
      }
      const int lim = static_cast<int>(lim64);
      const int t0 = cn * T;
      const int cap = (((t0 >> log2_bs) + 64) << log2_bs) / T;  // 64 blocks at most
      const int c1 = std::min(lim, cap);
      if (!started) pair_c0 = cn;
      Seg s;
      s.valid = 1;
      s.b = wb;
      s.g = wg;
      s.L = wL;
      s.t0 = t0;
      s.tend = std::min(wL, c1 * T);
      s.first = !started;
      s.last = c1 == lim;
      s.whole = pair_c0 == 0 && lim == wn;
      s.slot = lo >= P0 ? 0 : 1;
      started = 1;
      cn = c1;
      if (s.last) advance();
      return s;
    }
  };

  // Every path issues the same vector loads in the same order (a load that is
  // not needed reads the segment's own q row instead of being skipped): the
  // compiler's wait counts are then exact on every path, and a prefetch is never
  // waited for early.
  auto q_row = [&](const Seg& it) -> const uint16_t* {
    return q + (static_cast<int64_t>(it.b) * num_q_heads + it.g * G) * kHeadDim + sub * 8;
  };
  // The segment's block ids: lane l holds the block-table entry (block of the
  // segment's first token) + l, clamped into the row (entries past the context
  // are never used). A segment spans at most 64 blocks, and each group of 4
  // tokens lies in one block.
  auto load_blocks = [&](const Seg& it) -> int {
    const int bidx0 = it.t0 >> log2_bs;
    const int32_t* src = it.L > 0 ? block_table + static_cast<int64_t>(it.b) * bt_stride +
                                        min(bidx0 + lane, bt_stride - 1)
                                  : reinterpret_cast<const int32_t*>(q_row(it) + zero);
    return *src;
  };
  auto load_q = [&](const Seg& it, uint32_t (&qv)[G][4]) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const uint4 t = *reinterpret_cast<const uint4*>(q_row(it) + hh * kHeadDim);
      qv[hh][0] = t.x; qv[hh][1] = t.y; qv[hh][2] = t.z; qv[hh][3] = t.w;
    }
  };
  // The pool slot the segment's new token goes to: only a segment that ends
  // its pair's context, with a fused store; else -1.
  auto load_ns = [&](const Seg& it) -> int {
    if (slot_mapping == nullptr || !it.valid || it.L <= 0 || it.tend != it.L) return -1;
    return slot_mapping[it.b];
  };

  // ---- one chunk: loads, then arithmetic ------------------------------------
  // Chunk c of a segment covers tokens t0 + T*c .. t0 + T*c + T - 1; row grp of
  // lanes takes token (first + 4j + grp) for j < CH. Groups past the segment,
  // a chunk with no tokens at all, and every chunk of an invalid segment read
  // the segment's q row instead (a few hundred bytes the wavefront has just
  // loaded); tokens past it inside the last group re-read token tend-1 in the
  // same instruction as the lane that needs it.
  auto issue = [&](const Seg& it, int my_blk, int ns, int c, uint4 (&kb)[CH],
                   uint4 (&vb)[CH]) {
    const int cbase = it.t0 + c * T;
    // Uniform. An invalid segment (the prefetch past the end of the range)
    // carries the fields of a real one, so that its stand-in loads have
    // valid addresses; it loads nothing of the pool.
    const bool active = it.valid && cbase < it.tend;
    // The new token's row comes from k_new/v_new when this chunk holds it.
    const int new_tok = ns >= 0 && cbase + T > it.L - 1 ? it.L - 1 : -1;
    const int64_t new_off = static_cast<int64_t>(it.b) * kv_stride + it.g * kHeadDim + sub * 8;
    const int bidx0 = it.t0 >> log2_bs;
    const int ngroups = min(CH, (it.tend - cbase + 3) >> 2);
    const int64_t head_off = it.g * kHeadDim + sub * 8;
    const uint16_t* dummy = q_row(it) + zero;
    const uint16_t* kp[CH];
    const uint16_t* vp[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int tw = cbase + 4 * j;
      const int blk = __builtin_amdgcn_readlane(my_blk, (tw >> log2_bs) - bidx0);
      const int tc = min(tw + grp, it.tend - 1);
      const int64_t o =
          ((static_cast<int64_t>(blk) << log2_bs) | (tc & bs_mask)) * slot_stride + head_off;
      const bool fresh = active && tc == new_tok;
      const bool real = active && j < ngroups;
      kp[j] = fresh ? k_new + new_off : (real ? k_cache + o : dummy);
      vp[j] = fresh ? v_new + new_off : (real ? v_cache + o : dummy);
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
  auto compute = [&](const Seg& it, int ns, int c, const uint32_t (&qv)[G][4],
                     const uint4 (&kb)[CH], const uint4 (&vb)[CH]) {
    const int cbase = it.t0 + c * T;
    if (cbase >= it.tend) return;  // uniform
    float s[CH][G];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const bool valid = cbase + 4 * j + grp < it.tend;
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
      const uint4 vj = vb[j];  // p = 0 for tokens past the segment
      const float v[8] = {bf16_lo(vj.x), bf16_hi(vj.x), bf16_lo(vj.y), bf16_hi(vj.y),
                          bf16_lo(vj.z), bf16_hi(vj.z), bf16_lo(vj.w), bf16_hi(vj.w)};
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[hh][e] += s[j][hh] * v[e];
      }
    }
  };

  // ---- end of the wavefront's part of a pair: merge the rows of lanes, write --
  auto finalize = [&](const Seg& it) {
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
    constexpr bool kStream = G >= 4;  // see store16
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      if (it.whole) {
        const float inv = 1.f / l[hh];
        uint4 w;
        w.x = pack_bf16x2(acc[hh][0] * inv, acc[hh][1] * inv);
        w.y = pack_bf16x2(acc[hh][2] * inv, acc[hh][3] * inv);
        w.z = pack_bf16x2(acc[hh][4] * inv, acc[hh][5] * inv);
        w.w = pack_bf16x2(acc[hh][6] * inv, acc[hh][7] * inv);
        store16<kStream>(out + (bh0 + hh) * kHeadDim + sub * 8, w);
      } else {
        float* dst = part + ((static_cast<int64_t>(gw) * 2 + it.slot) * G + hh) * kRecord;
        store16<kStream>(dst + sub * 8, bits4(acc[hh][0], acc[hh][1], acc[hh][2], acc[hh][3]));
        store16<kStream>(dst + sub * 8 + 4, bits4(acc[hh][4], acc[hh][5], acc[hh][6], acc[hh][7]));
        if (sub == 0) {
          dst[kHeadDim] = m[hh];
          dst[kHeadDim + 1] = l[hh];
        }
      }
    }
  };

  // ---- the pipeline ---------------------------------------------------------
  // Two segment slots, A and B, alternate: while one segment is processed, the
  // other holds the next one (block ids, q and first chunk already requested).
  // The slot of the finished segment is then refilled with the segment after
  // that. The loop body is unrolled over the two slots so that no register
  // holding an in-flight load is ever copied (a copy would wait for the load).
  int done = 0;  // chunks processed (two per step of the loop below)
  Seg ia = next_seg(Seg{0, wb, wg, 0, 0, 0, 0, 0, 0, 0});
  if (ia.valid) {
  int blk_a = load_blocks(ia);
  int ns_a = load_ns(ia);
  uint32_t q_a[G][4], q_b[G][4];
  load_q(ia, q_a);
  uint4 kr0[CH], vr0[CH], kr1[CH], vr1[CH];
  issue(ia, blk_a, ns_a, 0, kr0, vr0);
  Seg ib = next_seg(ia);
  int blk_b = load_blocks(ib);
  int ns_b = load_ns(ib);
  load_q(ib, q_b);

  // Processes `cur` (its first chunk in flight in buffer 0), requests `nxt`'s
  // first chunk, then refills cur's slot with the segment after `nxt`. Returns
  // false when `nxt` does not exist.
  auto run = [&](Seg& cur, int& cur_blk, int& cur_ns, uint32_t (&qc)[G][4], const Seg& nxt,
                 int nxt_blk, int nxt_ns) -> bool {
    if (cur.first) reset();
    const int nch = max(0, (cur.tend - cur.t0 + T - 1) / T);
    for (int c = 0;; c += 2) {
      issue(cur, cur_blk, cur_ns, c + 1, kr1, vr1);
      compute(cur, cur_ns, c, qc, kr0, vr0);
      // Next: chunk c+2 of this segment, or the next segment's first chunk.
      const bool last = c + 2 >= nch;
      issue(last ? nxt : cur, last ? nxt_blk : cur_blk, last ? nxt_ns : cur_ns,
            last ? 0 : c + 2, kr0, vr0);
      compute(cur, cur_ns, c + 1, qc, kr1, vr1);
      // Wavefronts sharing a SIMD do not progress at the same rate, and every
      // range holds the same work: one behind its work-group's mean progress
      // issues at a higher priority.
      done += 2;
      if (lane == 0) __atomic_store_n(&s_prog[wave], done, __ATOMIC_RELAXED);
      int total = 0;
#pragma unroll
      for (int w2 = 0; w2 < W; ++w2) total += __atomic_load_n(&s_prog[w2], __ATOMIC_RELAXED);
      if (done * W < total) __builtin_amdgcn_s_setprio(2);
      else __builtin_amdgcn_s_setprio(0);
      if (last) break;
    }
    if (cur.last) finalize(cur);
    if (!nxt.valid) return false;
    cur = next_seg(nxt);
    cur_blk = load_blocks(cur);
    cur_ns = load_ns(cur);
    load_q(cur, qc);
    return true;
  };
  for (;;) {
    if (!run(ia, blk_a, ns_a, q_a, ib, blk_b, ns_b)) break;
    if (!run(ib, blk_b, ns_b, q_b, ia, blk_a, ns_a)) break;
  }
  }
}

// Merges the pieces of pairs cut by range boundaries: one wavefront per
// boundary w, kMergeWaves per work-group, working on the job wavefront w
// recorded.
// The job and the header are read together (an entry past nw is stale but
// inside the workspace, and is ignored); the pieces are then read four at a
// time, all loads in flight together, and folded in order with the online
// (max, sum, acc) rescaling. Each lane handles two elements of head_dim for
// every query head.
template <int G>
__global__ __launch_bounds__(64 * kMergeWaves) void decode_merge_kernel(uint16_t* __restrict__ out,
                                                           int32_t num_q_heads,
                                                           const char* __restrict__ ws,
                                                           int32_t batch, int32_t num_kv_heads,
                                                           const int32_t* __restrict__ context_lens,
                                                           int32_t max_context_len,
                                                           const uint16_t* __restrict__ k_new,
                                                           const uint16_t* __restrict__ v_new,
                                                           int64_t kv_stride,
                                                           const int32_t* __restrict__ slot_mapping,
                                                           uint16_t* k_store, uint16_t* v_store) {
  // Fused store: the new tokens' K/V rows go from k_new/v_new into their pool
  // slots here, one 16-byte unit per thread, for the rows whose clamped
  // length is positive and whose slot is not -1 (the decode kernel read
  // these tokens from k_new/v_new, and nothing in it reads those slots).
  if (slot_mapping != nullptr) {
    const int64_t units = static_cast<int64_t>(batch) * num_kv_heads * (kHeadDim / 8);
    const int64_t nthreads = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t u = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; u < units;
         u += nthreads) {
      const int64_t row = u / (kHeadDim / 8);  // (sequence, kv head)
      const int b = static_cast<int>(row / num_kv_heads);
      const int gh = static_cast<int>(row % num_kv_heads);
      const int slot = slot_mapping[b];
      if (slot < 0 || min(context_lens[b], max_context_len) <= 0) continue;
      const int e = static_cast<int>(u % (kHeadDim / 8)) * 8;
      const int64_t src = static_cast<int64_t>(b) * kv_stride + gh * kHeadDim + e;
      const int64_t dst = (static_cast<int64_t>(slot) * num_kv_heads + gh) * kHeadDim + e;
      *reinterpret_cast<uint4*>(k_store + dst) = *reinterpret_cast<const uint4*>(k_new + src);
      *reinterpret_cast<uint4*>(v_store + dst) = *reinterpret_cast<const uint4*>(v_new + src);
    }
  }
  const int64_t w = static_cast<int64_t>(blockIdx.x) * kMergeWaves + (threadIdx.x >> 6);
  const int64_t nw = reinterpret_cast<const int64_t*>(ws)[1];
  const int64_t* job = reinterpret_cast<const int64_t*>(ws + kInfoOffset) + 4 * w;
  const int64_t b = job[0], g = job[1], wa = job[2], pj = job[3];
  if (w >= nw) return;
  const int np = static_cast<int>(pj & 0xffffffff);
  if (np == 0) return;
  const int slot_wa = static_cast<int>(pj >> 32);
  const float* part = reinterpret_cast<const float*>(ws + partial_offset(nw));
  const int d = (threadIdx.x & 63) * 2;
  float M[G], o0[G], o1[G], lt[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    M[hh] = -INFINITY;
    o0[hh] = o1[hh] = lt[hh] = 0.f;
  }
  // Pieces read per round: their loads are all in flight together. Four at
  // G = 8 would need more than the 128 registers a 1024-thread work-group
  // allows (they spilled), so two there.
  constexpr int kU = G >= 8 ? 2 : 4;
  for (int x0 = 0; x0 < np; x0 += kU) {
    float mx[kU][G], lx[kU][G];
    float2 vx[kU][G];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int x = x0 + u;
      const int slot = x == 0 ? slot_wa : 0;
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        if (x < np) {
          const float* rec = part + (((wa + x) * 2 + slot) * G + hh) * kRecord;
          mx[u][hh] = rec[kHeadDim];
          lx[u][hh] = rec[kHeadDim + 1];
          vx[u][hh] = *reinterpret_cast<const float2*>(rec + d);
        } else {
          mx[u][hh] = -INFINITY;
          lx[u][hh] = 0.f;
          vx[u][hh] = make_float2(0.f, 0.f);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float mn = fmaxf(M[hh], mx[u][hh]);
        const float mu = mn == -INFINITY ? 0.f : mn;
        const float a = fast_exp2(M[hh] - mu);  // 0 while M is -inf
        const float c = fast_exp2(mx[u][hh] - mu);
        o0[hh] = o0[hh] * a + c * vx[u][hh].x;
        o1[hh] = o1[hh] * a + c * vx[u][hh].y;
        lt[hh] = lt[hh] * a + c * lx[u][hh];
        M[hh] = mn;
      }
    }
  }
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const float inv = 1.f / lt[hh];
    *reinterpret_cast<uint32_t*>(out + (b * num_q_heads + g * G + hh) * kHeadDim + d) =
        pack_bf16x2(o0[hh] * inv, o1[hh] * inv);
  }
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

// One launch of the decode kernel and its merge over the first
// min(batch, kScanRows) sequences. Returns the number handled (the caller
// goes on with the rest).
template <int G, int CH>
int launch_split(uint16_t* out, const uint16_t* q, const uint16_t* k_cache,
                 const uint16_t* v_cache, const int32_t* block_table, int32_t bt_stride,
                 const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
                 int32_t num_kv_heads, int32_t log2_bs, int32_t max_context_len, float scale_log2,
                 char* workspace, const FusedStore& fs, hipStream_t stream, hipError_t* err) {
  constexpr int W = decode_waves<G>();
  const int nb = std::min(batch, kScanRows);
  // No more work-groups than the most work these rows can hold needs (the
  // kernel's wave_target is non-decreasing in the cost): small batches then do
  // not start a work-group per CU only to scan context_lens and leave.
  const int64_t max_units =
      static_cast<int64_t>(nb) * num_kv_heads *
      ((std::max(0, max_context_len) + 4 * CH - 1) / (4 * CH) + kPairCost);
  const int groups = static_cast<int>(std::max<int64_t>(
      1, std::min<int64_t>(resident_groups<G, CH>(), (wave_target(max_units) + W - 1) / W)));
  hipLaunchKernelGGL((decode_kernel<G, CH>), dim3(static_cast<uint32_t>(groups)), dim3(64 * W),
                     0, stream, out, q, k_cache, v_cache, block_table, bt_stride, context_lens,
                     nb, num_q_heads, num_kv_heads, log2_bs, max_context_len, scale_log2,
                     workspace, 0, fs.k_new, fs.v_new, fs.kv_stride, fs.slot_mapping);
  *err = hipGetLastError();
  if (*err == hipSuccess) {
    const int merge_groups = (groups * W + kMergeWaves - 1) / kMergeWaves;
    hipLaunchKernelGGL((decode_merge_kernel<G>), dim3(static_cast<uint32_t>(merge_groups)),
                       dim3(64 * kMergeWaves), 0, stream, out, num_q_heads,
                       static_cast<const char*>(workspace), nb, num_kv_heads, context_lens,
                       max_context_len, fs.k_new, fs.v_new,
                       fs.kv_stride, fs.slot_mapping, fs.k_store, fs.v_store);
    *err = hipGetLastError();
  }
  return nb;
}

// The scratch of the no-allocation decode entry point (pa_decode_store_noalloc):
// a file-scope device array, one copy per device, held until the process
// ends. Host code never passes its name to a kernel: on the host the name is
// a stand-in, not a device address; decode_scratch() returns the address
// hipGetSymbolAddress gives for the current device.
static __device__ __align__(256) char scratch[kDecodeScratchBytes];

// Bound on the workspace bytes one launch of decode_kernel<G, CH> + its merge
// touches on the current device: nw <= grid * W working wavefronts, grid <=
// the resident work-groups; the merge reads job records of up to
// grid * W + kMergeWaves - 1 boundaries (those past nw are ignored).
template <int G, int CH>
size_t grid_workspace_bound() {
  const int64_t waves = static_cast<int64_t>(resident_groups<G, CH>()) * decode_waves<G>();
  return std::max(partial_offset(waves + kMergeWaves),
                  partial_offset(waves) +
                      static_cast<size_t>(2 * waves * G) * kRecord * sizeof(float));
}

}  // namespace

size_t decode_scratch_need(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                           int32_t max_context_len) {
  size_t grid = 0;
  switch (num_q_heads / num_kv_heads) {
    case 1: grid = grid_workspace_bound<1, 4>(); break;
    case 2: grid = grid_workspace_bound<2, 4>(); break;
    case 4: grid = grid_workspace_bound<4, 4>(); break;
    case 8: grid = grid_workspace_bound<8, 2>(); break;
    default: return 0;
  }
  return std::min(grid, decode_workspace_bytes(batch, num_q_heads, max_context_len));
}

hipError_t decode_scratch(void** ptr) {
  static std::atomic<void*> addr[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return hipSuccess;
}

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
  // Per launch (at most kScanRows sequences): nw <= max(1, wave_target(C))
  // working wavefronts, with C <= rows * Hkv * (ceil(max_context_len / 8) +
  // kPairCost) (a chunk holds at least 8 tokens). With U = rows * Hq * (...),
  // G * Hkv = Hq and G <= Hq: nw <= max(U / kFullUnits, min(U / kFewUnits,
  // kFillWaves)) + 1 and nw * G <= max(U / kFullUnits, min(U / kFewUnits,
  // Hq * kFillWaves)) + Hq.
  if (batch <= 0) return 0;
  const int64_t rows = std::min(batch, kScanRows);
  const int64_t units = (std::max(0, max_context_len) + 7) / 8 + kPairCost;
  const int64_t u = rows * num_q_heads * units;
  const int64_t nw = std::max(u / kFullUnits, std::min(u / kFewUnits, kFillWaves)) + 1;
  const int64_t records =                          // bound on 2 * nw * G
      2 * (std::max(u / kFullUnits, std::min(u / kFewUnits, num_q_heads * kFillWaves)) +
           num_q_heads);
  return partial_offset(nw) + static_cast<size_t>(records) * kRecord * sizeof(float);
}

hipError_t launch_decode(uint16_t* out, const uint16_t* q, const uint16_t* k_cache,
                         const uint16_t* v_cache, const int32_t* block_table,
                         int32_t block_table_stride, const int32_t* context_lens, int32_t batch,
                         int32_t num_q_heads, int32_t num_kv_heads, int32_t block_size,
                         int32_t max_context_len, float scale, void* workspace,
                         const FusedStore& fused, hipStream_t stream) {
  const int log2_bs = __builtin_ctz(static_cast<unsigned>(block_size));
  const float scale_log2 = scale * kLog2e;
  const int G = num_q_heads / num_kv_heads;
  hipError_t err = hipSuccess;
  // Consecutive launches over slices of the sequences, in stream order, each
  // using the workspace from its start (the previous slice is merged by then).
  for (int b0 = 0; b0 < batch && err == hipSuccess;) {
    const int64_t row = static_cast<int64_t>(b0) * num_q_heads * kHeadDim;
    FusedStore fs = fused;
    if (fs.slot_mapping) {
      fs.k_new += b0 * fs.kv_stride;
      fs.v_new += b0 * fs.kv_stride;
      fs.slot_mapping += b0;
    }
    int done = 0;
#define PA_DECODE_CASE(GG, CC)                                                              \
  case GG:                                                                                 \
    done = launch_split<GG, CC>(out + row, q + row, k_cache, v_cache,                      \
                                block_table + static_cast<int64_t>(b0) * block_table_stride, \
                                block_table_stride, context_lens + b0, batch - b0,         \
                                num_q_heads, num_kv_heads, log2_bs, max_context_len,       \
                                scale_log2, static_cast<char*>(workspace), fs, stream,     \
                                &err);                                                     \
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

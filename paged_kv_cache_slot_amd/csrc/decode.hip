// Paged decode: one query token per sequence attends over its context, whose
// keys and values sit in fixed-size blocks reached through the sequence's
// block table ("DeepSeek研究员1200行代码复刻vLLM…", section "vLLM是什么？").
//
// Work split. Each context is cut into pieces of kDecodeSplit (256) tokens; an
// item is one (piece, kv head) with all G = Hq/Hkv query heads that read that
// kv head, so every K/V byte is fetched from HBM once. A work-group is a single
// wavefront and a persistent worker: the grid holds as many as fit on the GPU
// at once, and they take items round-robin. Item w is piece p = w / Hkv of the
// concatenated pieces of all sequences and kv head w % Hkv (the kv heads of a
// piece are neighbours, so the same token rows are read together). The list
// is never materialised: each wavefront scans context_lens into LDS prefix sums
// and binary-searches the sequence of p, so nothing is spent on the empty
// tail of a short sequence.
//
// Within an item, each row of 16 lanes takes every fourth token and each lane
// a 16-byte slice (8 elements of head_dim) of that token's 256-byte kv-head
// row: one load instruction reads four whole rows. The item streams through
// chunks of CH groups of 4 tokens held in two alternating register buffers:
// the loads of the next chunk -- or of the next item's first chunk, whose
// block ids and q were fetched one item ahead -- are in flight while the
// current chunk is computed, so HBM requests never stop. There is no barrier:
// wavefronts never wait for each other.
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

constexpr int kTokensPerRow = kDecodeSplit / 4;  // 64: each 16-lane row takes every 4th token
constexpr int kScanRows = 1024;                  // rows of context_lens held in LDS at a time

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
// Orders the LDS accesses of one wavefront (the wavefronts of a work-group
// run independently, so a work-group barrier must not be used).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ int scan_rows(const int32_t* __restrict__ context_lens, int start, int batch,
                         int max_context_len, int base, int* s_pref, int* s_len) {
  constexpr int kPer = kScanRows / 64;
  const int n = min(kScanRows, batch - start);
  const int lane = threadIdx.x & 63;
  int raw[kPer];  // all loads first (index clamped), so they share one round trip
#pragma unroll
  for (int r = 0; r < kPer; ++r) raw[r] = context_lens[start + min(lane * kPer + r, n - 1)];
  int cnt[kPer];
  int local = 0;
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int i = lane * kPer + r;
    int c = 0;
    if (i < n) {
      const int L = max(0, min(raw[r], max_context_len));
      s_len[i] = L;
      c = max(1, (L + kDecodeSplit - 1) / kDecodeSplit);
    }
    cnt[r] = c;
    local += c;
  }
  int incl = local;  // inclusive scan over the 64 lanes
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off);
    if (lane >= off) incl += v;
  }
  int excl = base + incl - local;
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int i = lane * kPer + r;
    if (i < n) s_pref[i] = excl;
    excl += cnt[r];
  }
  if (lane == 63) s_pref[n] = excl;
  wave_sync();
  return n;
}

// One work item: piece `split` (tokens [split*256, min(L, split*256+256))) of
// sequence b, kv head g. L is the clamped context length (0: padding row) and
// nsplit the sequence's number of pieces. All fields are uniform.
struct Item {
  int valid, b, g, split, L, nsplit;
};

// Wavefronts per work-group: all that fit on a CU at once (two per SIMD, one
// for G = 8, whose register use allows only one).
template <int G>
constexpr int decode_waves() { return G >= 8 ? 4 : 8; }

template <int G, int CH>
__global__ __launch_bounds__(64 * decode_waves<G>(), 1) void decode_kernel(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ k_cache, const uint16_t* __restrict__ v_cache,
    const int32_t* __restrict__ block_table, int32_t bt_stride,
    const int32_t* __restrict__ context_lens, int32_t batch, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t log2_bs, int32_t max_context_len, float scale_log2,
    int32_t max_splits, float* __restrict__ ws_o, float* __restrict__ ws_ml, int32_t zero) {
  // `zero` is always 0. Adding it to the address of a stand-in load keeps the
  // compiler from merging that load with an identical one (and from turning
  // the stand-in back into a branch).
  constexpr int NCH = kTokensPerRow / CH;  // chunks per piece
  static_assert(NCH % 2 == 0, "chunk buffers alternate, so a piece has an even chunk count");
  constexpr int W = decode_waves<G>();
  __shared__ int s_pref_all[W][kScanRows + 1];  // each wavefront's window of context_lens
  __shared__ int s_len_all[W][kScanRows];
  __shared__ int s_taken;                       // items of this work-group handed out so far
  if (threadIdx.x == 0) s_taken = 0;
  __syncthreads();  // the only work-group barrier: every wavefront is here once, at the start

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int* s_pref = s_pref_all[wave];
  int* s_len = s_len_all[wave];
  const int grp = lane >> 4;  // which token of four
  const int sub = lane & 15;  // which 8-element slice of head_dim
  const int bs_mask = (1 << log2_bs) - 1;
  const int64_t slot_stride = static_cast<int64_t>(num_kv_heads) * kHeadDim;

  // ---- the item list -------------------------------------------------------
  int chunk_start = 0;
  int nrows = scan_rows(context_lens, 0, batch, max_context_len, 0, s_pref, s_len);
  // Item w (may rescan the LDS window). Past the last item it returns
  // `fallback` marked invalid, so that the loads issued for it still read
  // valid memory.
  auto lookup = [&](int w, Item fallback) -> Item {
    fallback.valid = 0;
    Item it = fallback;
    const int p = w / num_kv_heads;
    while (p >= __builtin_amdgcn_readfirstlane(s_pref[nrows])) {
      if (chunk_start + nrows >= batch) return fallback;  // past the last item
      const int base = __builtin_amdgcn_readfirstlane(s_pref[nrows]);
      wave_sync();
      chunk_start += nrows;
      nrows = scan_rows(context_lens, chunk_start, batch, max_context_len, base, s_pref, s_len);
    }
    int lo = 0, hi = nrows - 1;  // row r with s_pref[r] <= p < s_pref[r + 1]
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (__builtin_amdgcn_readfirstlane(s_pref[mid]) <= p) lo = mid; else hi = mid - 1;
    }
    const int first = __builtin_amdgcn_readfirstlane(s_pref[lo]);
    it.valid = 1;
    it.b = chunk_start + lo;
    it.g = w - p * num_kv_heads;
    it.split = p - first;
    it.nsplit = __builtin_amdgcn_readfirstlane(s_pref[lo + 1]) - first;
    it.L = __builtin_amdgcn_readfirstlane(s_len[lo]);
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
  // the piece) + l % 16, clamped into the row (entries past the context are
  // never used). A piece of 256 tokens spans at most 16 blocks because
  // block_size >= 16, and each group of 4 tokens lies in one block.
  auto load_blocks = [&](const Item& it) -> int {
    const int bidx0 = (it.split * kDecodeSplit) >> log2_bs;
    const int32_t* src = it.L > 0 ? block_table + static_cast<int64_t>(it.b) * bt_stride +
                                        min(bidx0 + (lane & 15), bt_stride - 1)
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
    const int t0 = it.split * kDecodeSplit;
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
    const int cbase = it.split * kDecodeSplit + c * CH * 4;
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
      const float mn = fmaxf(m[hh], cm);
      const float mu = mn == -INFINITY ? 0.f : mn;
      const float alpha = fast_exp2(m[hh] - mu);
      m[hh] = mn;
      l[hh] *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[hh][e] *= alpha;
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
  // Work-group i owns items i, i + grid, i + 2 grid, ...: its k-th item is
  // k * grid + i. Wavefront j takes its k = j and k = W + j first; every later
  // k comes from the work-group's LDS counter, fetched when the item two
  // places before it starts, so wavefronts that run faster take more items.
  auto item_index = [&](int k) { return k * static_cast<int>(gridDim.x) + blockIdx.x; };
  Item ia = lookup(item_index(wave), Item{0, 0, 0, 0, 0, 0});
  if (ia.valid) {
  int blk_a = load_blocks(ia);
  uint32_t q_a[G][4], q_b[G][4];
  load_q(ia, q_a);
  uint4 kr0[CH], vr0[CH], kr1[CH], vr1[CH];
  issue(ia, blk_a, 0, kr0, vr0);
  Item ib = lookup(item_index(W + wave), ia);
  int blk_b = load_blocks(ib);
  load_q(ib, q_b);

  // Processes `cur` (its first chunk in flight in buffer 0), requests `nxt`'s
  // first chunk, then refills cur's slot with the item after `nxt`. Returns
  // false when `nxt` does not exist.
  auto run = [&](Item& cur, int& cur_blk, uint32_t (&qc)[G][4], const Item& nxt, int nxt_blk)
      -> bool {
    int grabbed = 0;  // lane 0: k - 2W of the item that will refill this slot
    if (lane == 0) grabbed = atomicAdd(&s_taken, 1);
    reset();
    const int t0 = cur.split * kDecodeSplit;
    const int ntok = min(cur.L, t0 + kDecodeSplit) - t0;  // <= 0 on a padding row
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
    cur = lookup(item_index(2 * W + __builtin_amdgcn_readfirstlane(grabbed)), nxt);
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

template <int G, int CH>
hipError_t launch_split(uint16_t* out, const uint16_t* q, const uint16_t* k_cache,
                  const uint16_t* v_cache, const int32_t* block_table, int32_t bt_stride,
                  const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
                  int32_t num_kv_heads, int32_t log2_bs, int32_t max_context_len,
                  float scale_log2, int32_t max_splits, float* ws_o, float* ws_ml,
                  hipStream_t stream) {
  // Never more wavefronts than items (pieces x kv heads).
  const int64_t items = static_cast<int64_t>(batch) * num_kv_heads * max_splits;
  constexpr int W = decode_waves<G>();
  const int64_t blocks = std::min<int64_t>((items + W - 1) / W, resident_groups<G, CH>());
  hipLaunchKernelGGL((decode_kernel<G, CH>), dim3(static_cast<uint32_t>(blocks)),
                     dim3(64 * decode_waves<G>()), 0, stream, out, q, k_cache, v_cache,
                     block_table, bt_stride, context_lens, batch, num_q_heads, num_kv_heads,
                     log2_bs, max_context_len, scale_log2, max_splits, ws_o, ws_ml, 0);
  return hipGetLastError();
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
  hipError_t err = hipSuccess;
#define PA_DECODE_CASE(GG, CC)                                                              \
  case GG:                                                                                 \
    err = launch_split<GG, CC>(out, q, k_cache, v_cache, block_table, block_table_stride,  \
                               context_lens, batch, num_q_heads, num_kv_heads, log2_bs,    \
                               max_context_len, scale_log2, max_splits, ws_o, ws_ml,       \
                               stream);                                                    \
    break;
  switch (G) {
    PA_DECODE_CASE(1, 8)
    PA_DECODE_CASE(2, 8)
    PA_DECODE_CASE(4, 4)
    PA_DECODE_CASE(8, 2)
    default:
      return hipErrorInvalidValue;
  }
#undef PA_DECODE_CASE
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

// Random calls against the C++ block manager for a host sanitizer build
// (AddressSanitizer + UndefinedBehaviorSanitizer). It exercises every entry
// point of pa_block_manager.h, failures included, and checks the answers
// that need no model: reference counts against the live tables, the free
// count, metadata shapes and -1 padding.
#include <cstdio>
#include <cstdlib>
#include <map>
#include <vector>

#include "pa_block_manager.h"

namespace {

uint64_t rng_state = 0x9e3779b97f4a7c15ull;
uint32_t next_rand() {  // splitmix64, upper half
  uint64_t z = (rng_state += 0x9e3779b97f4a7c15ull);
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return static_cast<uint32_t>((z ^ (z >> 31)) >> 32);
}
uint32_t below(uint32_t n) { return next_rand() % n; }

int failures = 0;
void expect(bool ok, const char* what, int step) {
  if (!ok) {
    std::fprintf(stderr, "step %d: %s\n", step, what);
    ++failures;
  }
}

}  // namespace

int main(int argc, char** argv) {
  const int steps = argc > 1 ? std::atoi(argv[1]) : 20000;
  const int32_t nb = 40, bs = 4, stride = 64;
  pa_block_manager* bm = pa_bm_create(nb, bs);
  if (!bm || pa_bm_create(0, 4) != nullptr || pa_bm_create(4, 0) != nullptr) return 2;
  std::vector<std::vector<int32_t>> stems(3);
  for (auto& s : stems)
    for (int i = 0; i < 14; ++i) s.push_back(static_cast<int32_t>(below(3)));
  std::map<int64_t, int32_t> live;  // id -> length
  for (int step = 0; step < steps; ++step) {
    const uint32_t r = below(100);
    const int64_t id = below(10);
    if (r < 30) {
      const std::vector<int32_t>& stem = stems[below(3)];
      std::vector<int32_t> t(stem.begin(), stem.begin() + below(15));
      for (uint32_t i = 0, n = below(10); i < n; ++i) t.push_back(static_cast<int32_t>(below(4)));
      int32_t ok = -1, cached = -1;
      const int rc_can = t.empty() ? PA_ERR_SHAPE
                                   : pa_bm_can_allocate(bm, t.data(), static_cast<int32_t>(t.size()), &ok);
      const int rc = pa_bm_allocate(bm, id, t.data(), static_cast<int32_t>(t.size()), &cached);
      if (t.empty()) {
        expect(rc == PA_ERR_SHAPE && rc_can == PA_ERR_SHAPE, "empty prompt accepted", step);
      } else if (live.count(id)) {
        expect(rc == PA_ERR_SEQ, "live id accepted", step);
      } else {
        expect((rc == PA_OK) == (ok == 1), "can_allocate disagrees with allocate", step);
        if (rc == PA_OK) {
          live[id] = static_cast<int32_t>(t.size());
          expect(cached % bs == 0 && cached < static_cast<int32_t>(t.size()), "cached count", step);
        }
      }
    } else if (r < 60) {
      int32_t ok = -1;
      const int rc_can = pa_bm_can_append(bm, id, &ok);
      const int rc = pa_bm_append(bm, id, static_cast<int32_t>(below(3)));
      if (!live.count(id)) {
        expect(rc == PA_ERR_SEQ && rc_can == PA_ERR_SEQ, "append to dead id", step);
      } else {
        expect((rc == PA_OK) == (ok == 1), "can_append disagrees with append", step);
        if (rc == PA_OK) ++live[id];
      }
    } else if (r < 70) {
      std::vector<int64_t> ids;
      std::vector<int32_t> toks;
      for (uint32_t i = 0, n = below(5); i < n; ++i) {
        ids.push_back(below(10));
        toks.push_back(static_cast<int32_t>(below(3)));
      }
      const int rc = pa_bm_append_batch(bm, ids.data(), toks.data(), static_cast<int32_t>(ids.size()));
      if (rc == PA_OK)
        for (int64_t s : ids) ++live[s];
    } else if (r < 85) {
      const int rc = pa_bm_deallocate(bm, id);
      expect((rc == PA_OK) == (live.count(id) == 1), "deallocate result", step);
      live.erase(id);
    } else {
      std::vector<int64_t> ids;
      for (auto& kv : live) ids.push_back(kv.first);
      const int32_t B = static_cast<int32_t>(ids.size()), P = B + static_cast<int32_t>(below(3));
      std::vector<int32_t> ctx(P + 1), slots(P + 1), bt(static_cast<size_t>(P + 1) * stride);
      std::vector<int32_t> cu(B + 1);
      int32_t mx = -1, tq = -1, mq = -1;
      int rc = pa_bm_decode_metadata(bm, ids.data(), B, P, ctx.data(), slots.data(), bt.data(),
                                     stride, &mx);
      expect(rc == PA_OK, "decode metadata", step);
      for (int32_t b = 0; b < P; ++b) {
        const int32_t want = b < B ? live[ids[b]] : 0;
        expect(ctx[b] == want, "decode context length", step);
        expect((slots[b] < 0) == (b >= B), "decode slot padding", step);
        expect(b >= B || (slots[b] >= 0 && slots[b] < nb * bs), "decode slot range", step);
      }
      std::vector<int32_t> sm(nb * bs);
      rc = pa_bm_prefill_metadata(bm, ids.data(), B, cu.data(), ctx.data(), sm.data(),
                                  static_cast<int32_t>(sm.size()), bt.data(), stride, &tq, &mq);
      expect(rc == PA_OK && cu[B] == tq, "prefill metadata", step);
    }
    // Reference counts equal the number of live tables holding each block.
    std::vector<int32_t> count(nb, 0);
    int32_t used = 0;
    for (auto& kv : live) {
      int32_t n = 0, c = 0, k = 0;
      expect(pa_bm_seq_info(bm, kv.first, &n, &c, &k) == PA_OK && n == kv.second, "seq_info", step);
      std::vector<int32_t> table(k + 1);
      expect(pa_bm_block_table(bm, kv.first, table.data(), k) == PA_OK, "block_table", step);
      for (int32_t j = 0; j < k; ++j) ++count[table[j]];
    }
    for (int32_t b = 0; b < nb; ++b) {
      int32_t ref = -1, cached = -1;
      uint64_t h = 0;
      expect(pa_bm_block_info(bm, b, &ref, &cached, &h) == PA_OK && ref == count[b], "ref count",
             step);
      used += ref > 0;
    }
    expect(pa_bm_num_free_blocks(bm) == nb - used, "free count", step);
  }
  int64_t st[5];
  pa_bm_stats(bm, st);
  std::printf("stats shared %lld taken_back %lld fresh_alloc %lld fresh_append %lld evicted %lld\n",
              (long long)st[0], (long long)st[1], (long long)st[2], (long long)st[3],
              (long long)st[4]);
  pa_bm_destroy(bm);
  std::printf("%s after %d steps\n", failures ? "FAILED" : "ok", steps);
  return failures ? 1 : 0;
}

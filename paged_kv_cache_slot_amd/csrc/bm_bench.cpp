// Host benchmark of the block manager, run by bench.py: times the C++ calls
// directly (no Python in the loop) and prints one JSON object.
//
//   bm_bench [sequences] [block_size] [decode_steps] [seed]
//
// Workload: `sequences` prompts of U[100,1024] tokens (token ids < 151936);
// the first 0..3 blocks of a prompt (as many as fit) come from one of 8 shared
// prefix chains of 3 blocks, the rest is fresh. The pool holds every block the
// batch can reach plus 64. Timed: allocation of the batch; `decode_steps`
// decode steps, each one pa_bm_append_batch (one token per sequence) and one
// pa_bm_decode_metadata; one pa_bm_prefill_metadata over the batch; XXH64 over
// a 1 MiB buffer.
#include <algorithm>
#include <chrono>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "pa_block_manager.h"

namespace {

using Clock = std::chrono::steady_clock;

double micros(Clock::time_point a, Clock::time_point b) {
  return std::chrono::duration<double, std::micro>(b - a).count();
}

}  // namespace

int main(int argc, char** argv) {
  const int B = argc > 1 ? std::atoi(argv[1]) : 256;
  const int bs = argc > 2 ? std::atoi(argv[2]) : 256;
  const int steps = argc > 3 ? std::atoi(argv[3]) : 256;
  const unsigned seed = argc > 4 ? static_cast<unsigned>(std::atoi(argv[4])) : 4242u;
  if (B < 1 || bs < 1 || steps < 1) return 2;
  std::mt19937 rng(seed);
  auto uniform = [&rng](int lo, int hi) {  // inclusive
    return std::uniform_int_distribution<int>(lo, hi)(rng);
  };
  const int vocab = 151936;
  std::vector<std::vector<int32_t>> chains(8, std::vector<int32_t>(3 * bs));
  for (auto& c : chains)
    for (auto& x : c) x = uniform(0, vocab - 1);
  std::vector<std::vector<int32_t>> prompts(B);
  int64_t tokens = 0, blocks = 0;
  int max_len = 0;
  for (auto& p : prompts) {
    const int n = uniform(100, 1024);
    const int k = std::min(uniform(0, 3), n / bs);
    const auto& chain = chains[uniform(0, 7)];
    p.assign(chain.begin(), chain.begin() + k * bs);
    while (static_cast<int>(p.size()) < n) p.push_back(uniform(0, vocab - 1));
    tokens += n;
    blocks += (n + steps + bs - 1) / bs;
    max_len = std::max(max_len, n + steps);
  }
  const int stride = (max_len + bs - 1) / bs;
  pa_block_manager* bm = pa_bm_create(static_cast<int32_t>(blocks + 64), bs);
  if (!bm) return 3;

  int64_t cached = 0;
  const auto t0 = Clock::now();
  for (int i = 0; i < B; ++i) {
    int32_t c = 0;
    if (pa_bm_allocate(bm, i, prompts[i].data(), static_cast<int32_t>(prompts[i].size()), &c))
      return 4;
    cached += c;
  }
  const auto t1 = Clock::now();

  std::vector<int64_t> ids(B);
  for (int i = 0; i < B; ++i) ids[i] = i;
  std::vector<int32_t> tok(B), ctx(B), slots(B), table(static_cast<size_t>(B) * stride);
  double t_append = 0, t_meta = 0;
  for (int s = 0; s < steps; ++s) {
    for (auto& x : tok) x = uniform(0, vocab - 1);
    const auto a = Clock::now();
    if (pa_bm_append_batch(bm, ids.data(), tok.data(), B)) return 5;
    const auto b = Clock::now();
    if (pa_bm_decode_metadata(bm, ids.data(), B, B, ctx.data(), slots.data(), table.data(),
                              stride, nullptr))
      return 6;
    const auto c = Clock::now();
    t_append += micros(a, b);
    t_meta += micros(b, c);
  }

  int64_t rows = 0;
  if (pa_bm_batch_info(bm, ids.data(), B, &rows, nullptr, nullptr, nullptr)) return 7;
  std::vector<int32_t> cu(B + 1), sm(static_cast<size_t>(rows));
  int32_t total_q = 0;
  const auto p0 = Clock::now();
  if (pa_bm_prefill_metadata(bm, ids.data(), B, cu.data(), ctx.data(), sm.data(),
                             static_cast<int32_t>(rows), table.data(), stride, &total_q, nullptr))
    return 8;
  const auto p1 = Clock::now();

  std::vector<uint8_t> buf(1 << 20);
  for (auto& x : buf) x = static_cast<uint8_t>(uniform(0, 255));
  uint64_t sink = 0;
  const int reps = 64;
  const auto h0 = Clock::now();
  for (int r = 0; r < reps; ++r) sink += pa_xxh64(buf.data(), buf.size(), r);
  const auto h1 = Clock::now();

  int64_t st[5];
  pa_bm_stats(bm, st);
  pa_bm_destroy(bm);
  std::printf(
      "{\"sequences\": %d, \"block_size\": %d, \"prompt_tokens\": %lld, \"cached_tokens\": %lld, "
      "\"decode_steps\": %d, \"allocate_us_per_seq\": %.3f, \"append_batch_us\": %.3f, "
      "\"decode_metadata_us\": %.3f, \"decode_step_us\": %.3f, \"prefill_metadata_us\": %.2f, "
      "\"prefill_rows\": %d, \"xxh64_GBps\": %.2f, \"stats\": {\"shared\": %lld, "
      "\"taken_back\": %lld, \"fresh_alloc\": %lld, \"fresh_append\": %lld, \"evicted\": %lld}, "
      "\"check\": %llu}\n",
      B, bs, static_cast<long long>(tokens), static_cast<long long>(cached), steps,
      micros(t0, t1) / B, t_append / steps, t_meta / steps, (t_append + t_meta) / steps,
      micros(p0, p1), total_q, reps * static_cast<double>(buf.size()) / micros(h0, h1) / 1e3,
      static_cast<long long>(st[0]), static_cast<long long>(st[1]), static_cast<long long>(st[2]),
      static_cast<long long>(st[3]), static_cast<long long>(st[4]),
      static_cast<unsigned long long>(sink & 0xffff));
  return 0;
}

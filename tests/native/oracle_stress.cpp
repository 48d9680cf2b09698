// Stress program for the CPU oracle (oracle/oracle.cpp), built with host
// sanitizers by tests/test_oracle_sanitized.py. Random small cases drive
// oracle_store_kvcache, oracle_decode and oracle_prefill: padding rows
// (length 0), -1 slots, ragged lengths, row subsets, several block sizes,
// head groupings and thread counts. Each case checks what holds whatever the
// values:
//   * the output does not depend on the thread count (bitwise);
//   * rows outside a requested subset are left untouched;
//   * every output is a convex combination of the visible V rows, so each
//     component lies between their minimum and maximum (0 for length 0);
//   * the store copies exactly the named slots and skips -1;
//   * out-of-range block ids or slots and null pointers are rejected.
// Usage: oracle_stress <cases> [seed]; prints "ok after N cases".
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

extern "C" {
int oracle_store_kvcache(const uint16_t* k, const uint16_t* v, int64_t kv_token_stride,
                         uint16_t* k_cache, uint16_t* v_cache, const int32_t* slot_mapping,
                         int32_t num_tokens, int32_t num_blocks, int32_t block_size,
                         int32_t num_kv_heads, int32_t head_dim);
int oracle_decode(double* out, const uint16_t* q, const uint16_t* k_cache,
                  const uint16_t* v_cache, const int32_t* block_table,
                  int32_t block_table_stride, const int32_t* context_lens, int32_t batch,
                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                  int32_t block_size, int32_t num_blocks, double scale, const int32_t* rows,
                  int32_t num_rows, int32_t nthreads);
int oracle_prefill(double* out, const uint16_t* q, const uint16_t* k_cache,
                   const uint16_t* v_cache, const int32_t* cu_seqlens_q,
                   const int32_t* context_lens, const int32_t* block_table,
                   int32_t block_table_stride, int32_t batch, int32_t total_q,
                   int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                   int32_t block_size, int32_t num_blocks, double scale,
                   const int32_t* tokens, int32_t num_tokens, int32_t nthreads);
}

namespace {

std::mt19937_64 rng;

int uni(int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); }

// A finite bf16 of moderate magnitude (sign, exponent 2^-8 .. 2^3, mantissa).
uint16_t rand_bf16() {
  const uint32_t sign = static_cast<uint32_t>(uni(0, 1)) << 15;
  const uint32_t exp = static_cast<uint32_t>(uni(127 - 8, 127 + 3)) << 7;
  const uint32_t man = static_cast<uint32_t>(uni(0, 127));
  return static_cast<uint16_t>(sign | exp | man);
}

double bf16(uint16_t b) {
  uint32_t w = static_cast<uint32_t>(b) << 16;
  float f;
  std::memcpy(&f, &w, sizeof f);
  return f;
}

void fail(const char* what, int c) {
  std::printf("FAIL case %d: %s\n", c, what);
  std::exit(1);
}

struct Paged {
  int hkv, g, d, bs, batch, num_blocks, stride;
  std::vector<int32_t> lens, table;
  std::vector<uint16_t> kc, vc;
};

// A paged context per row: lens[b] tokens in randomly chosen distinct blocks;
// table entries past a row's blocks hold junk the oracle must not read.
Paged make_paged(int batch, int max_len) {
  Paged p;
  p.hkv = 1 << uni(0, 2);
  p.g = 1 << uni(0, 2);
  p.d = 8 << uni(0, 2);
  p.bs = std::vector<int>{1, 2, 4, 16}[uni(0, 3)];
  p.batch = batch;
  p.lens.resize(batch);
  int need = 0, maxb = 0;
  for (int b = 0; b < batch; ++b) {
    p.lens[b] = uni(0, 4) == 0 ? 0 : uni(1, max_len);
    const int nb = (p.lens[b] + p.bs - 1) / p.bs;
    need += nb;
    maxb = nb > maxb ? nb : maxb;
  }
  p.num_blocks = need + uni(1, 3);  // never an empty (null) pool
  p.stride = maxb + uni(0, 2);
  if (p.stride == 0) p.stride = 1;
  std::vector<int32_t> perm(p.num_blocks);
  for (int i = 0; i < p.num_blocks; ++i) perm[i] = i;
  std::shuffle(perm.begin(), perm.end(), rng);
  p.table.assign(static_cast<size_t>(batch) * p.stride, 0);
  int next = 0;
  for (int b = 0; b < batch; ++b) {
    const int nb = (p.lens[b] + p.bs - 1) / p.bs;
    for (int j = 0; j < p.stride; ++j)
      p.table[static_cast<size_t>(b) * p.stride + j] = j < nb ? perm[next++] : uni(-5, 1 << 20);
  }
  const size_t pool = static_cast<size_t>(p.num_blocks) * p.bs * p.hkv * p.d;
  p.kc.resize(pool);
  p.vc.resize(pool);
  for (auto& x : p.kc) x = rand_bf16();
  for (auto& x : p.vc) x = rand_bf16();
  return p;
}

// Bounds of component d of the V rows of tokens 0..n-1 of row b, kv head g.
void v_bounds(const Paged& p, int b, int n, int g, int d, double& lo, double& hi) {
  lo = INFINITY;
  hi = -INFINITY;
  for (int j = 0; j < n; ++j) {
    const int64_t blk = p.table[static_cast<size_t>(b) * p.stride + j / p.bs];
    const int64_t slot = blk * p.bs + j % p.bs;
    const double x = bf16(p.vc[(static_cast<size_t>(slot) * p.hkv + g) * p.d + d]);
    lo = x < lo ? x : lo;
    hi = x > hi ? x : hi;
  }
}

bool within(double x, double lo, double hi) {
  const double tol = 1e-12 * (std::fabs(lo) + std::fabs(hi) + 1.0);
  return std::isfinite(x) && x >= lo - tol && x <= hi + tol;
}

void check_store(int c) {
  Paged p = make_paged(uni(1, 4), 40);
  const int row = p.hkv * p.d;
  const int T = uni(0, 8);
  const int64_t stride = row + 8 * uni(0, 2);
  std::vector<uint16_t> k(static_cast<size_t>(T) * stride), v(k.size());
  for (auto& x : k) x = rand_bf16();
  for (auto& x : v) x = rand_bf16();
  const int slots = p.num_blocks * p.bs;
  std::vector<int32_t> sm(T);
  std::vector<int32_t> perm(slots);
  for (int i = 0; i < slots; ++i) perm[i] = i;
  std::shuffle(perm.begin(), perm.end(), rng);
  for (int i = 0; i < T; ++i) sm[i] = (uni(0, 3) == 0 || i >= slots) ? -1 : perm[i];
  std::vector<uint16_t> kc = p.kc, vc = p.vc;
  if (oracle_store_kvcache(k.data(), v.data(), stride, kc.data(), vc.data(), sm.data(), T,
                           p.num_blocks, p.bs, p.hkv, p.d) != 0)
    fail("store rejected valid input", c);
  std::vector<char> written(slots, 0);
  for (int i = 0; i < T; ++i) {
    if (sm[i] < 0) continue;
    written[sm[i]] = 1;
    for (int e = 0; e < row; ++e)
      if (kc[static_cast<size_t>(sm[i]) * row + e] != k[static_cast<size_t>(i) * stride + e] ||
          vc[static_cast<size_t>(sm[i]) * row + e] != v[static_cast<size_t>(i) * stride + e])
        fail("store: a named slot differs from its token", c);
  }
  for (int s = 0; s < slots; ++s)
    if (!written[s])
      for (int e = 0; e < row; ++e)
        if (kc[static_cast<size_t>(s) * row + e] != p.kc[static_cast<size_t>(s) * row + e])
          fail("store: an unnamed slot changed", c);
  if (T > 0) {
    std::vector<int32_t> bad = sm;
    bad[uni(0, T - 1)] = slots + uni(0, 3);
    if (oracle_store_kvcache(k.data(), v.data(), stride, kc.data(), vc.data(), bad.data(), T,
                             p.num_blocks, p.bs, p.hkv, p.d) != 2)
      fail("store: slot out of range not rejected", c);
    if (oracle_store_kvcache(nullptr, v.data(), stride, kc.data(), vc.data(), sm.data(), T,
                             p.num_blocks, p.bs, p.hkv, p.d) != 1)
      fail("store: null pointer not rejected", c);
  }
}

void check_decode(int c) {
  Paged p = make_paged(uni(0, 6), 60);
  const int hq = p.hkv * p.g;
  const size_t n_out = static_cast<size_t>(p.batch) * hq * p.d;
  std::vector<uint16_t> q(n_out);
  for (auto& x : q) x = rand_bf16();
  const double scale = std::ldexp(1.0, -uni(0, 4));
  std::vector<double> o1(n_out, 7.5), o3(n_out, 7.5);
  if (oracle_decode(o1.data(), q.data(), p.kc.data(), p.vc.data(), p.table.data(), p.stride,
                    p.lens.data(), p.batch, hq, p.hkv, p.d, p.bs, p.num_blocks, scale, nullptr,
                    0, 1) != 0)
    fail("decode rejected valid input", c);
  if (oracle_decode(o3.data(), q.data(), p.kc.data(), p.vc.data(), p.table.data(), p.stride,
                    p.lens.data(), p.batch, hq, p.hkv, p.d, p.bs, p.num_blocks, scale, nullptr,
                    0, 3) != 0)
    fail("decode rejected valid input (3 threads)", c);
  if (n_out > 0 && std::memcmp(o1.data(), o3.data(), n_out * sizeof(double)) != 0)
    fail("decode depends on the thread count", c);
  for (int b = 0; b < p.batch; ++b)
    for (int h = 0; h < hq; ++h)
      for (int d = 0; d < p.d; ++d) {
        const double x = o1[(static_cast<size_t>(b) * hq + h) * p.d + d];
        if (p.lens[b] == 0) {
          if (x != 0.0) fail("decode: padding row not zero", c);
          continue;
        }
        double lo, hi;
        v_bounds(p, b, p.lens[b], h / p.g, d, lo, hi);
        if (!within(x, lo, hi)) fail("decode: output outside the V rows' range", c);
      }
  if (p.batch > 0) {
    std::vector<int32_t> rows;
    for (int b = 0; b < p.batch; ++b)
      if (uni(0, 1)) rows.push_back(b);
    if (rows.empty()) rows.push_back(uni(0, p.batch - 1));  // a null subset means every row
    std::vector<double> os(n_out, 7.5);
    if (oracle_decode(os.data(), q.data(), p.kc.data(), p.vc.data(), p.table.data(), p.stride,
                      p.lens.data(), p.batch, hq, p.hkv, p.d, p.bs, p.num_blocks, scale,
                      rows.data(), static_cast<int32_t>(rows.size()), 2) != 0)
      fail("decode rejected a row subset", c);
    std::vector<char> listed(p.batch, 0);
    for (int b : rows) listed[b] = 1;
    for (int b = 0; b < p.batch; ++b)
      for (size_t e = 0; e < static_cast<size_t>(hq) * p.d; ++e) {
        const size_t i = static_cast<size_t>(b) * hq * p.d + e;
        if (listed[b] ? os[i] != o1[i] : os[i] != 7.5) fail("decode: row subset", c);
      }
    for (int b = 0; b < p.batch; ++b)
      if (p.lens[b] > 0) {
        std::vector<int32_t> bad = p.table;
        bad[static_cast<size_t>(b) * p.stride + uni(0, (p.lens[b] - 1) / p.bs)] =
            uni(0, 1) ? -1 : p.num_blocks + uni(0, 5);
        if (oracle_decode(os.data(), q.data(), p.kc.data(), p.vc.data(), bad.data(), p.stride,
                          p.lens.data(), p.batch, hq, p.hkv, p.d, p.bs, p.num_blocks, scale,
                          nullptr, 0, 2) != 2)
          fail("decode: bad block id not rejected", c);
        break;
      }
  }
}

void check_prefill(int c) {
  Paged p = make_paged(uni(0, 5), 50);
  const int hq = p.hkv * p.g;
  std::vector<int32_t> cu(p.batch + 1, 0);
  for (int b = 0; b < p.batch; ++b) cu[b + 1] = cu[b] + uni(0, p.lens[b]);  // N <= L
  const int total = cu[p.batch];
  const size_t n_out = static_cast<size_t>(total) * hq * p.d;
  std::vector<uint16_t> q(n_out);
  for (auto& x : q) x = rand_bf16();
  const double scale = std::ldexp(1.0, -uni(0, 4));
  std::vector<double> o1(n_out, 7.5), o3(n_out, 7.5);
  if (oracle_prefill(o1.data(), q.data(), p.kc.data(), p.vc.data(), cu.data(), p.lens.data(),
                     p.table.data(), p.stride, p.batch, total, hq, p.hkv, p.d, p.bs,
                     p.num_blocks, scale, nullptr, 0, 1) != 0)
    fail("prefill rejected valid input", c);
  if (oracle_prefill(o3.data(), q.data(), p.kc.data(), p.vc.data(), cu.data(), p.lens.data(),
                     p.table.data(), p.stride, p.batch, total, hq, p.hkv, p.d, p.bs,
                     p.num_blocks, scale, nullptr, 0, 3) != 0)
    fail("prefill rejected valid input (3 threads)", c);
  if (n_out > 0 && std::memcmp(o1.data(), o3.data(), n_out * sizeof(double)) != 0)
    fail("prefill depends on the thread count", c);
  for (int b = 0; b < p.batch; ++b) {
    const int N = cu[b + 1] - cu[b], P = p.lens[b] - N;
    for (int i = 0; i < N; ++i)
      for (int h = 0; h < hq; ++h)
        for (int d = 0; d < p.d; ++d) {
          double lo, hi;
          v_bounds(p, b, P + i + 1, h / p.g, d, lo, hi);
          const double x = o1[(static_cast<size_t>(cu[b] + i) * hq + h) * p.d + d];
          if (!within(x, lo, hi)) fail("prefill: output outside the visible V rows' range", c);
        }
  }
  if (total > 0) {
    std::vector<int32_t> toks;
    for (int t = 0; t < total; ++t)
      if (uni(0, 1)) toks.push_back(t);
    if (toks.empty()) toks.push_back(uni(0, total - 1));  // a null subset means every row
    std::vector<double> os(n_out, 7.5);
    if (oracle_prefill(os.data(), q.data(), p.kc.data(), p.vc.data(), cu.data(), p.lens.data(),
                       p.table.data(), p.stride, p.batch, total, hq, p.hkv, p.d, p.bs,
                       p.num_blocks, scale, toks.data(), static_cast<int32_t>(toks.size()),
                       2) != 0)
      fail("prefill rejected a row subset", c);
    std::vector<char> listed(total, 0);
    for (int t : toks) listed[t] = 1;
    for (int t = 0; t < total; ++t)
      for (size_t e = 0; e < static_cast<size_t>(hq) * p.d; ++e) {
        const size_t i = static_cast<size_t>(t) * hq * p.d + e;
        if (listed[t] ? os[i] != o1[i] : os[i] != 7.5) fail("prefill: row subset", c);
      }
    std::vector<int32_t> bad_cu = cu;
    bad_cu[p.batch] = total + 1;
    if (oracle_prefill(os.data(), q.data(), p.kc.data(), p.vc.data(), bad_cu.data(),
                       p.lens.data(), p.table.data(), p.stride, p.batch, total, hq, p.hkv, p.d,
                       p.bs, p.num_blocks, scale, nullptr, 0, 1) != 2)
      fail("prefill: inconsistent cu_seqlens_q not rejected", c);
  }
}

}  // namespace

int main(int argc, char** argv) {
  const int cases = argc > 1 ? std::atoi(argv[1]) : 200;
  rng.seed(argc > 2 ? std::strtoull(argv[2], nullptr, 10) : 12345u);
  for (int c = 0; c < cases; ++c) {
    check_store(c);
    check_decode(c);
    check_prefill(c);
  }
  std::printf("ok after %d cases\n", cases);
  return 0;
}

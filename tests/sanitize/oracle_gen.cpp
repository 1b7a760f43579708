// Address and undefined-behaviour sanitizer run of the oracle and the input
// generator on the CPU: every oracle function on small seeded inputs (ragged
// vocabularies, every dtype, both modes, empty batches, error rows), with a few
// sanity checks on the results. Built and run by tests/test_sanitizers.py; exits
// non-zero on a failed check, and the sanitizers abort on the first error.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "oracle.h"

extern "C" {
uint64_t svg_key(uint64_t cfg, uint64_t seed, uint64_t purpose);
void svg_normal_pair(uint64_t key_a, double sig_a, uint64_t key_b, double sig_b, uint64_t first, uint64_t n,
                     int dtype, void* out_a, void* out_b, int nthreads);
void svg_uniform24(uint64_t key, uint64_t first, uint64_t n, float* out);
void svg_gumbel_rows(uint64_t key, int dtype, int64_t rows, int64_t V, const void* logits, double T,
                     int32_t* out, int nthreads);
void svg_argmax_rows(int dtype, int64_t rows, int64_t V, const void* logits, int32_t* out, int nthreads);
void svg_round(int dtype, int64_t n, const double* in, void* out);
void svg_decode(int dtype, int64_t n, const void* in, double* out);
}

static int g_fail = 0;
#define CHECK(c)                                                      \
  do {                                                                \
    if (!(c)) {                                                       \
      std::fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
      ++g_fail;                                                       \
    }                                                                 \
  } while (0)

static size_t esize(int dt) { return dt == 0 ? 4 : 2; }

struct Logits {
  std::vector<unsigned char> a, b;
};

static Logits make(uint64_t cfg, int dt, size_t n, double sa, double sb) {
  Logits L;
  L.a.resize(n * esize(dt) + 1);
  L.b.resize(n * esize(dt) + 1);
  svg_normal_pair(svg_key(cfg, 1, 1), sa, svg_key(cfg, 1, 2), sb, 0, n, dt, L.a.data(), L.b.data(), 3);
  return L;
}

static void linear(int dt, int mode, int64_t B, int64_t k, int64_t V) {
  Logits t = make(100 + V, dt, (size_t)(B * (k + 1) * V), 2.0, 0.5);
  Logits d = make(200 + V, dt, (size_t)(B * k * V), 2.0, 0.5);
  std::vector<int32_t> x((size_t)(B * k + 1));
  if (B * k > 0) svg_gumbel_rows(svg_key(3, 1, 3), dt, B * k, V, d.a.data(), 0.8, x.data(), 2);
  std::vector<float> u((size_t)(B * (k + 1) + 1));
  svg_uniform24(svg_key(4, 1, 4), 0, (uint64_t)(B * (k + 1)), u.data());
  std::vector<int32_t> acc((size_t)B + 1), out((size_t)(B * (k + 1)) + 1), ef((size_t)B + 1), nt((size_t)B + 1),
      ne((size_t)B + 1);
  std::vector<double> pt((size_t)(B * k) + 1), pd((size_t)(B * k) + 1);
  const int r = orc_verify_linear(mode, 0.8, B, k, V, dt, t.a.data(), d.a.data(), x.data(), u.data(), 1e-6,
                                  acc.data(), out.data(), pt.data(), pd.data(), ef.data(), nt.data(), ne.data());
  CHECK(r == 0);
  for (int64_t b = 0; b < B; ++b) {
    CHECK(acc[b] >= 0 && acc[b] <= k);
    CHECK(ef[b] == 0);
    CHECK(out[b * (k + 1) + acc[b]] >= 0 && out[b * (k + 1) + acc[b]] < V);
  }
}

static void tree(int dt, int mode, int64_t B, int64_t V) {
  // a small Cartesian-style tree: root, 3 children, 2 grandchildren each
  std::vector<int32_t> par = {-1, 0, 0, 0, 1, 1, 2, 2, 3, 3};
  const int64_t n = (int64_t)par.size();
  Logits lg = make(300 + V, dt, (size_t)(B * n * V), 3.0, 0.0);
  std::vector<int32_t> am((size_t)(B * n));
  svg_argmax_rows(dt, B * n, V, lg.a.data(), am.data(), 2);
  std::vector<int32_t> cand((size_t)(B * n));
  for (int64_t b = 0; b < B; ++b)
    for (int64_t i = 0; i < n; ++i)
      cand[b * n + i] = i == 0 ? -1 : ((i + b) % 3 ? am[b * n + par[i]] : (int32_t)((i * 7919) % V));
  std::vector<float> u((size_t)(B * n));
  svg_uniform24(svg_key(5, 1, 5), 0, (uint64_t)(B * n), u.data());
  std::vector<int32_t> acc(B), path(B * 3), out(B * 3), ef(B), nt(B), ne(B), ntok(B * n);
  int r = orc_verify_tree(mode, 1.0, B, n, V, dt, par.data(), 0, cand.data(), lg.a.data(), u.data(), 2, 1e-6,
                          acc.data(), path.data(), out.data(), ef.data(), nt.data(), ne.data(), ntok.data());
  CHECK(r == 0);
  for (int64_t b = 0; b < B; ++b) CHECK(acc[b] >= 0 && acc[b] <= 2);
  r = orc_verify_tree_typical(1.0, 0.09, 0.3, B, n, V, dt, par.data(), 0, cand.data(), lg.a.data(), u.data(), 2,
                              1e-6, acc.data(), path.data(), out.data(), ef.data(), nt.data(), ne.data());
  CHECK(r == 0);
  std::vector<uint8_t> dense((size_t)(n * n));
  CHECK(orc_tree_mask(n, par.data(), dense.data()) == 0);
  for (int64_t i = 0; i < n; ++i) CHECK(dense[i * n + i] == 1 && dense[i * n + 0] == 1);
  // ranks 1..S among siblings (the function's documented range)
  std::vector<int32_t> rank = {0, 1, 2, 3, 1, 2, 1, 2, 1, 2};
  std::vector<double> a = {0.6, 0.3, 0.1, 0.5, 0.2, 0.1};
  const double E = orc_expected_accept_len(n, par.data(), rank.data(), 3, a.data());
  CHECK(std::isfinite(E) && E >= 0.0);
}

static void rows(int dt, int64_t R, int64_t V) {
  Logits x = make(400 + V, dt, (size_t)(R * V), 2.0, 0.0);
  std::vector<double> m(R + 1), lse(R + 1);
  std::vector<int32_t> am(R + 1), fl(R + 1), tok(R + 1), ef(R + 1), nt(R + 1);
  CHECK(orc_row_stats(dt, 0.7, R, V, x.a.data(), m.data(), lse.data(), am.data(), fl.data()) == 0);
  std::vector<float> u(R + 1);
  svg_uniform24(svg_key(6, 1, 6), 0, (uint64_t)R, u.data());
  CHECK(orc_sample(1, 0.7, R, V, dt, x.a.data(), u.data(), 1e-6, tok.data(), ef.data(), nt.data()) == 0);
  CHECK(orc_sample(0, 1.0, R, V, dt, x.a.data(), nullptr, 1e-6, tok.data(), ef.data(), nt.data()) == 0);
  for (int64_t r = 0; r < R; ++r) CHECK(tok[r] == am[r]);
  std::vector<double> dec((size_t)(R * V));
  svg_decode(dt, R * V, x.a.data(), dec.data());
  std::vector<unsigned char> back(dec.size() * esize(dt));
  svg_round(dt, R * V, dec.data(), back.data());
  for (size_t i = 0; i < back.size(); ++i) CHECK(back[i] == x.a[i]);
}

int main() {
  for (int dt = 0; dt < 3; ++dt) {
    for (int mode = 0; mode < 2; ++mode) {
      linear(dt, mode, 3, 4, 1000);
      linear(dt, mode, 2, 1, 7);
      linear(dt, mode, 1, 0, 33);
      linear(dt, mode, 0, 4, 100);
      tree(dt, mode, 2, 517);
    }
    rows(dt, 5, 1031);
  }
  // weights for the inverse CDF, including zeros and u at the ends
  std::vector<double> w = {0.0, 1.0, 0.0, 2.5, 1e-300, 0.5};
  double lo = 0, hi = 0;
  CHECK(orc_invcdf(w.data(), (int64_t)w.size(), 0.0, &lo, &hi) == 1);
  CHECK(orc_invcdf(w.data(), (int64_t)w.size(), 0.99999994, &lo, &hi) == 5);
  // commit: one sequence of each accepted length
  const int64_t B = 3, k = 2, cap = 16;
  std::vector<int32_t> acc = {0, 1, 2}, out = {5, -1, -1, 6, 7, -1, 8, 9, 10}, drafts = {1, 2, 3, 4, 5, 6};
  std::vector<int32_t> len = {0, 3, 14}, hist(B * cap, 0), sh(B * (k + 1)), nx(B), ef(B);
  CHECK(orc_commit_linear(B, k, acc.data(), out.data(), drafts.data(), len.data(), hist.data(), cap, sh.data(),
                          nx.data(), ef.data()) == 0);
  // greedy sparse tree
  std::vector<double> a = {0.8, 0.15, 0.05, 0.6, 0.25, 0.1, 0.45, 0.3, 0.15};
  std::vector<int32_t> par(65), dep(65), rk(65);
  double E = 0.0;
  const int64_t n = orc_tree_build_greedy(3, 3, a.data(), 64, par.data(), dep.data(), rk.data(), &E);
  CHECK(n == 40);   // the full tree of depth 3 and width 3 has 39 nodes besides the root
  for (int64_t i = 1; i < n; ++i) CHECK(par[i] >= 0 && par[i] < i && dep[i] == dep[par[i]] + 1);
  if (g_fail) {
    std::fprintf(stderr, "%d checks failed\n", g_fail);
    return 1;
  }
  std::printf("oracle and generator: all checks passed\n");
  return 0;
}

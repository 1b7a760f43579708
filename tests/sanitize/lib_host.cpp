// Address and undefined-behaviour sanitizer run of the library's host code on the
// CPU: the workspace-size queries (layouts) of every entry point over many
// shapes, every argument check that rejects a call before anything reaches the
// GPU, and the greedy sparse-tree builder (host code). No call here passes its
// checks, so nothing is launched and no device is needed; the pointers given are
// stand-ins that are never dereferenced. Built and run by tests/test_sanitizers.py.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <vector>

#include "specverify.h"

static int g_fail = 0;
#define CHECK(c)                                                          \
  do {                                                                    \
    if (!(c)) {                                                           \
      std::fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
      ++g_fail;                                                           \
    }                                                                     \
  } while (0)

// stand-ins: 256-byte aligned, never dereferenced (every call below is rejected
// before its pointers are used)
static void* const FAKE = reinterpret_cast<void*>((uintptr_t)1 << 40);
static void* const MISALIGNED = reinterpret_cast<void*>(((uintptr_t)1 << 40) + 16);
template <class T>
static T* fk() { return static_cast<T*>(FAKE); }

static void linear_checks() {
  const int64_t Bs[] = {1, 2, 31, 32, 256, 4096};
  const int64_t ks[] = {0, 1, 4, SV_MAX_K};
  const int64_t Vs[] = {1, 7, 1000, 4097, 128256, 129280};
  for (int dt = 0; dt < 3; ++dt)
    for (int mode = 0; mode < 2; ++mode)
      for (int64_t k : ks)
        for (int64_t V : Vs) {
          size_t prev = 0;
          for (int64_t B : Bs) {
            const size_t need = spec_verify_linear_workspace(B, k, V, (sv_dtype)dt, (sv_mode)mode);
            CHECK(need > 0 && need % 256 == 0 && need >= prev);
            CHECK(need == spec_verify_linear_workspace(B, k, V, (sv_dtype)dt, (sv_mode)mode));
            prev = need;
            // one byte short, misaligned, missing: rejected after the layout is formed
            const sv_mode m = (sv_mode)mode;
            const sv_status a = spec_verify_linear(m, 0.7f, B, k, V, (sv_dtype)dt, FAKE, FAKE, fk<int32_t>(),
                                                   fk<float>(), fk<int32_t>(), fk<int32_t>(), nullptr, nullptr,
                                                   nullptr, FAKE, need - 1, nullptr);
            CHECK(a == SV_EWORKSPACE);
            CHECK(spec_verify_linear(m, 0.7f, B, k, V, (sv_dtype)dt, FAKE, FAKE, fk<int32_t>(), fk<float>(),
                                     fk<int32_t>(), fk<int32_t>(), nullptr, nullptr, nullptr, MISALIGNED,
                                     need, nullptr) == SV_EWORKSPACE);
            CHECK(spec_verify_linear_commit(m, 0.7f, B, k, V, (sv_dtype)dt, FAKE, FAKE, fk<int32_t>(),
                                            fk<float>(), fk<int32_t>(), fk<int32_t>(), nullptr, nullptr, nullptr,
                                            fk<int32_t>(), fk<int32_t>(), 64, nullptr, nullptr, nullptr, need,
                                            nullptr) == SV_EWORKSPACE);
          }
        }
  const float T = 0.7f;
  // dtype, mode, sizes, limits
  CHECK(spec_verify_linear_workspace(4, 2, 100, (sv_dtype)7, SV_GREEDY) == 0);
  CHECK(spec_verify_linear_workspace(-1, 2, 100, SV_BF16, SV_GREEDY) == 0);
  CHECK(spec_verify_linear(SV_GREEDY, T, 4, 2, 100, (sv_dtype)7, FAKE, nullptr, fk<int32_t>(), nullptr,
                           fk<int32_t>(), fk<int32_t>(), nullptr, nullptr, nullptr, FAKE, 1 << 20,
                           nullptr) == SV_EDTYPE);
  CHECK(spec_verify_linear((sv_mode)5, T, 4, 2, 100, SV_BF16, FAKE, nullptr, fk<int32_t>(), nullptr,
                           fk<int32_t>(), fk<int32_t>(), nullptr, nullptr, nullptr, FAKE, 1 << 20,
                           nullptr) == SV_EINVAL);
  CHECK(spec_verify_linear(SV_GREEDY, T, -1, 2, 100, SV_BF16, FAKE, nullptr, fk<int32_t>(), nullptr,
                           fk<int32_t>(), fk<int32_t>(), nullptr, nullptr, nullptr, FAKE, 1 << 20,
                           nullptr) == SV_EINVAL);
  CHECK(spec_verify_linear(SV_GREEDY, T, 4, SV_MAX_K + 1, 100, SV_BF16, FAKE, nullptr, fk<int32_t>(), nullptr,
                           fk<int32_t>(), fk<int32_t>(), nullptr, nullptr, nullptr, FAKE, 1 << 20,
                           nullptr) == SV_ELIMIT);
  CHECK(spec_verify_linear(SV_GREEDY, T, 4, 2, (int64_t)SV_MAX_ROW_BYTES, SV_BF16, FAKE, nullptr, fk<int32_t>(),
                           nullptr, fk<int32_t>(), fk<int32_t>(), nullptr, nullptr, nullptr, FAKE, 1 << 20,
                           nullptr) == SV_ELIMIT);
  CHECK(spec_verify_linear(SV_GREEDY, T, 0, 2, 100, SV_BF16, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                           nullptr, nullptr, nullptr, nullptr, 0, nullptr) == SV_OK);
  // missing pointers, temperatures
  CHECK(spec_verify_linear(SV_GREEDY, T, 4, 2, 100, SV_BF16, nullptr, nullptr, fk<int32_t>(), nullptr,
                           fk<int32_t>(), fk<int32_t>(), nullptr, nullptr, nullptr, FAKE, 1 << 20,
                           nullptr) == SV_EINVAL);
  CHECK(spec_verify_linear(SV_GREEDY, T, 4, 2, 100, SV_BF16, FAKE, nullptr, nullptr, nullptr, fk<int32_t>(),
                           fk<int32_t>(), nullptr, nullptr, nullptr, FAKE, 1 << 20, nullptr) == SV_EINVAL);
  const float bad_T[] = {0.0f, -1.0f, NAN, INFINITY};
  for (float bt : bad_T)
    CHECK(spec_verify_linear(SV_STOCHASTIC, bt, 4, 2, 100, SV_BF16, FAKE, FAKE, fk<int32_t>(), fk<float>(),
                             fk<int32_t>(), fk<int32_t>(), nullptr, nullptr, nullptr, FAKE, 1 << 20,
                             nullptr) == SV_EINVAL);
  CHECK(spec_verify_linear(SV_STOCHASTIC, T, 4, 2, 100, SV_BF16, FAKE, nullptr, fk<int32_t>(), fk<float>(),
                           fk<int32_t>(), fk<int32_t>(), nullptr, nullptr, nullptr, FAKE, 1 << 20,
                           nullptr) == SV_EINVAL);
  CHECK(spec_verify_linear(SV_STOCHASTIC, T, 4, 2, 100, SV_BF16, FAKE, FAKE, fk<int32_t>(), nullptr,
                           fk<int32_t>(), fk<int32_t>(), nullptr, nullptr, nullptr, FAKE, 1 << 20,
                           nullptr) == SV_EINVAL);
  CHECK(spec_verify_linear_commit(SV_GREEDY, T, 4, 2, 100, SV_BF16, FAKE, nullptr, fk<int32_t>(), nullptr,
                                  fk<int32_t>(), fk<int32_t>(), nullptr, nullptr, nullptr, fk<int32_t>(),
                                  fk<int32_t>(), -1, nullptr, nullptr, FAKE, 1 << 20, nullptr) == SV_EINVAL);
  // without allocation: shapes beyond the scratch array, and plain argument errors
  CHECK(spec_verify_linear_static(SV_STOCHASTIC, T, 100000, 4, 128256, SV_BF16, FAKE, FAKE, fk<int32_t>(),
                                  fk<float>(), fk<int32_t>(), fk<int32_t>(), nullptr, nullptr, nullptr,
                                  nullptr) == SV_ELIMIT);
  CHECK(spec_verify_linear_static(SV_STOCHASTIC, T, 4, SV_MAX_K + 1, 100, SV_BF16, FAKE, FAKE, fk<int32_t>(),
                                  fk<float>(), fk<int32_t>(), fk<int32_t>(), nullptr, nullptr, nullptr,
                                  nullptr) == SV_ELIMIT);
  CHECK(spec_verify_linear_static(SV_STOCHASTIC, T, 4, 2, 100, (sv_dtype)3, FAKE, FAKE, fk<int32_t>(),
                                  fk<float>(), fk<int32_t>(), fk<int32_t>(), nullptr, nullptr, nullptr,
                                  nullptr) == SV_EDTYPE);
  CHECK(spec_verify_linear_static(SV_GREEDY, T, 0, 2, 100, SV_BF16, nullptr, nullptr, nullptr, nullptr, nullptr,
                                  nullptr, nullptr, nullptr, nullptr, nullptr) == SV_OK);
}

static void tree_checks() {
  const int64_t Ns[] = {1, 2, 65, 257, 4681, SV_MAX_TREE_NODES};
  const int64_t Vs[] = {1, 7, 32000, 129280};
  for (int dt = 0; dt < 3; ++dt)
    for (int64_t N : Ns)
      for (int64_t V : Vs) {
        size_t prev = 0;
        for (int64_t B : {1, 4, 16}) {
          const size_t need = spec_verify_tree_workspace(B, N, V, (sv_dtype)dt, SV_STOCHASTIC);
          CHECK(need > 0 && need % 256 == 0 && need >= prev);
          prev = need;
          for (int mode = 0; mode < 2; ++mode)
            CHECK(spec_verify_tree((sv_mode)mode, 1.0f, B, N, V, (sv_dtype)dt, fk<int32_t>(), 0, fk<int32_t>(),
                                   FAKE, fk<float>(), 4, fk<int32_t>(), fk<int32_t>(), fk<int32_t>(), nullptr,
                                   FAKE, need - 1, nullptr) == SV_EWORKSPACE);
          CHECK(spec_verify_tree_typical(1.0f, 0.09, 0.3, B, N, V, (sv_dtype)dt, fk<int32_t>(), 0, fk<int32_t>(),
                                         FAKE, fk<float>(), 4, fk<int32_t>(), fk<int32_t>(), fk<int32_t>(), nullptr,
                                         MISALIGNED, need, nullptr) == SV_EWORKSPACE);
        }
      }
  CHECK(spec_verify_tree(SV_GREEDY, 1.0f, 2, SV_MAX_TREE_NODES + 1, 100, SV_F16, fk<int32_t>(), 0, fk<int32_t>(),
                         FAKE, nullptr, 4, fk<int32_t>(), fk<int32_t>(), fk<int32_t>(), nullptr, FAKE, 1 << 20,
                         nullptr) == SV_ELIMIT);
  CHECK(spec_verify_tree(SV_GREEDY, 1.0f, 2, 10, 100, SV_F16, nullptr, 0, fk<int32_t>(), FAKE, nullptr, 4,
                         fk<int32_t>(), fk<int32_t>(), fk<int32_t>(), nullptr, FAKE, 1 << 20, nullptr) == SV_EINVAL);
  CHECK(spec_verify_tree(SV_GREEDY, 1.0f, 2, 10, 100, SV_F16, fk<int32_t>(), -3, fk<int32_t>(), FAKE, nullptr, 4,
                         fk<int32_t>(), fk<int32_t>(), fk<int32_t>(), nullptr, FAKE, 1 << 20, nullptr) == SV_EINVAL);
  CHECK(spec_verify_tree(SV_GREEDY, 1.0f, 2, 10, 100, SV_F16, fk<int32_t>(), 0, fk<int32_t>(), FAKE, nullptr, -1,
                         fk<int32_t>(), fk<int32_t>(), fk<int32_t>(), nullptr, FAKE, 1 << 20, nullptr) == SV_EINVAL);
  CHECK(spec_verify_tree(SV_STOCHASTIC, 1.0f, 2, 10, 100, SV_F16, fk<int32_t>(), 0, fk<int32_t>(), FAKE, nullptr,
                         4, fk<int32_t>(), fk<int32_t>(), fk<int32_t>(), nullptr, FAKE, 1 << 20,
                         nullptr) == SV_EINVAL);
  CHECK(spec_verify_tree((sv_mode)2, 1.0f, 2, 10, 100, SV_F16, fk<int32_t>(), 0, fk<int32_t>(), FAKE, nullptr, 4,
                         fk<int32_t>(), fk<int32_t>(), fk<int32_t>(), nullptr, FAKE, 1 << 20, nullptr) == SV_EINVAL);
  const double bad[] = {-0.1, NAN, INFINITY};
  for (double e : bad) {
    CHECK(spec_verify_tree_typical(1.0f, e, 0.3, 2, 10, 100, SV_F16, fk<int32_t>(), 0, fk<int32_t>(), FAKE,
                                   fk<float>(), 4, fk<int32_t>(), fk<int32_t>(), fk<int32_t>(), nullptr, FAKE,
                                   1 << 20, nullptr) == SV_EINVAL);
    CHECK(spec_verify_tree_typical(1.0f, 0.1, e, 2, 10, 100, SV_F16, fk<int32_t>(), 0, fk<int32_t>(), FAKE,
                                   fk<float>(), 4, fk<int32_t>(), fk<int32_t>(), fk<int32_t>(), nullptr, FAKE,
                                   1 << 20, nullptr) == SV_EINVAL);
  }
  CHECK(spec_verify_tree(SV_GREEDY, 1.0f, 0, 10, 100, SV_F16, nullptr, 0, nullptr, nullptr, nullptr, 4, nullptr,
                         nullptr, nullptr, nullptr, nullptr, 0, nullptr) == SV_OK);
  // masks
  CHECK(spec_tree_mask(2, SV_MAX_TREE_NODES + 1, fk<int32_t>(), 0, fk<uint32_t>(), nullptr, nullptr) == SV_ELIMIT);
  CHECK(spec_tree_mask(2, 10, nullptr, 0, fk<uint32_t>(), nullptr, nullptr) == SV_EINVAL);
  CHECK(spec_tree_mask(-1, 10, fk<int32_t>(), 0, fk<uint32_t>(), nullptr, nullptr) == SV_EINVAL);
  CHECK(spec_tree_mask(0, 10, nullptr, 0, nullptr, nullptr, nullptr) == SV_OK);
}

static void row_checks() {
  for (int dt = 0; dt < 3; ++dt)
    for (int64_t V : {1, 5, 32000, 128256, 129280})
      for (int64_t R : {1, 33, 1024}) {
        const size_t ns = spec_sample_workspace(R, V, (sv_dtype)dt);
        const size_t nr = spec_row_stats_workspace(R, V, (sv_dtype)dt);
        CHECK(ns > 0 && nr > 0);
        CHECK(spec_sample(SV_STOCHASTIC, 0.7f, R, V, (sv_dtype)dt, FAKE, fk<float>(), fk<int32_t>(), nullptr, FAKE,
                          ns - 1, nullptr) == SV_EWORKSPACE);
        CHECK(spec_row_stats((sv_dtype)dt, 0.7f, R, V, FAKE, fk<float>(), fk<float>(), fk<int32_t>(), nullptr,
                             MISALIGNED, nr, nullptr) == SV_EWORKSPACE);
      }
  CHECK(spec_sample((sv_mode)9, 0.7f, 4, 100, SV_BF16, FAKE, fk<float>(), fk<int32_t>(), nullptr, FAKE, 1 << 20,
                    nullptr) == SV_EINVAL);
  CHECK(spec_sample(SV_STOCHASTIC, 0.7f, 4, 100, SV_BF16, FAKE, nullptr, fk<int32_t>(), nullptr, FAKE, 1 << 20,
                    nullptr) == SV_EINVAL);
  CHECK(spec_sample(SV_GREEDY, 0.7f, 4, 100, SV_BF16, FAKE, nullptr, nullptr, nullptr, FAKE, 1 << 20,
                    nullptr) == SV_EINVAL);
  CHECK(spec_row_stats(SV_BF16, 0.0f, 4, 100, FAKE, nullptr, nullptr, nullptr, nullptr, FAKE, 1 << 20,
                       nullptr) == SV_EINVAL);
  CHECK(spec_row_stats(SV_BF16, 1.0f, 4, (int64_t)SV_MAX_ROW_BYTES, FAKE, nullptr, nullptr, nullptr, nullptr, FAKE,
                       1 << 20, nullptr) == SV_ELIMIT);
  CHECK(spec_row_stats(SV_BF16, 1.0f, 4, 100, nullptr, nullptr, nullptr, nullptr, nullptr, FAKE, 1 << 20,
                       nullptr) == SV_EINVAL);
  CHECK(spec_row_stats(SV_BF16, 1.0f, 0, 100, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0,
                       nullptr) == SV_OK);
  // commit
  CHECK(spec_commit_linear(-1, 2, fk<int32_t>(), fk<int32_t>(), fk<int32_t>(), fk<int32_t>(), fk<int32_t>(), 8,
                           nullptr, nullptr, nullptr, nullptr) == SV_EINVAL);
  CHECK(spec_commit_linear(4, SV_MAX_K + 1, fk<int32_t>(), fk<int32_t>(), fk<int32_t>(), fk<int32_t>(),
                           fk<int32_t>(), 8, nullptr, nullptr, nullptr, nullptr) == SV_ELIMIT);
  CHECK(spec_commit_linear(4, 2, fk<int32_t>(), fk<int32_t>(), fk<int32_t>(), nullptr, fk<int32_t>(), 8, nullptr,
                           nullptr, nullptr, nullptr) == SV_EINVAL);
  CHECK(spec_commit_linear(4, 2, fk<int32_t>(), fk<int32_t>(), nullptr, fk<int32_t>(), fk<int32_t>(), 8,
                           fk<int32_t>(), nullptr, nullptr, nullptr) == SV_EINVAL);
  CHECK(spec_commit_linear(4, 2, fk<int32_t>(), fk<int32_t>(), fk<int32_t>(), fk<int32_t>(), nullptr, 8, nullptr,
                           nullptr, nullptr, nullptr) == SV_EINVAL);
  CHECK(spec_commit_linear(0, 2, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr, nullptr, nullptr,
                           nullptr) == SV_OK);
  CHECK(spec_workspace_clear(nullptr, 256, nullptr) == SV_EINVAL);
  CHECK(spec_set_wait_limit(-1.0) == SV_EINVAL);
  CHECK(spec_set_wait_limit(61.0) == SV_EINVAL);
  CHECK(spec_set_wait_limit(NAN) == SV_EINVAL);
  CHECK(spec_workspace_clear(reinterpret_cast<void*>(((uintptr_t)1 << 40) + 8), 256, nullptr) == SV_EINVAL);
}

static void builder_checks() {
  // accuracies with ties, zeros and ones; budgets around the full tree's size
  const std::vector<std::vector<double>> accs = {
      {0.8, 0.15, 0.05, 0.6, 0.25, 0.1, 0.45, 0.3, 0.15},
      {0.5, 0.5, 0.5, 0.5, 0.5, 0.5, 0.5, 0.5, 0.5},
      {1.0, 0.0, 0.0, 1.0, 0.0, 0.0, 0.0, 1.0, 0.0},
  };
  for (const auto& a : accs)
    for (int64_t budget : {0, 1, 2, 12, 38, 39, 40, 200}) {
      std::vector<int32_t> par(budget + 1), dep(budget + 1), rk(budget + 1);
      double E = -1.0;
      const int64_t n = spec_tree_build_greedy(3, 3, a.data(), budget, par.data(), dep.data(), rk.data(), &E);
      CHECK(n >= 1 && n <= budget + 1 && n <= 40);
      CHECK(par[0] == -1 && dep[0] == 0);
      for (int64_t i = 1; i < n; ++i) {
        CHECK(par[i] >= 0 && par[i] < i && dep[i] == dep[par[i]] + 1 && rk[i] >= 1 && rk[i] <= 3);
        if (i > 1) CHECK(dep[i] >= dep[i - 1]);
      }
      CHECK(std::isfinite(E) && E >= 0.0 && E <= (double)(n - 1) + 1e-12);
      // optional outputs left out
      CHECK(spec_tree_build_greedy(3, 3, a.data(), budget, par.data(), nullptr, nullptr, nullptr) == n);
    }
  std::vector<double> big(16 * 16, 0.9);
  std::vector<int32_t> par(5001);
  CHECK(spec_tree_build_greedy(16, 16, big.data(), 5000, par.data(), nullptr, nullptr, nullptr) == 5001);
  const double badv[] = {-0.5, 1.5, NAN};
  for (double v : badv) {
    std::vector<double> a(9, 0.5);
    a[4] = v;
    CHECK(spec_tree_build_greedy(3, 3, a.data(), 10, par.data(), nullptr, nullptr, nullptr) < 0);
  }
  std::vector<double> a(9, 0.5);
  CHECK(spec_tree_build_greedy(0, 3, a.data(), 10, par.data(), nullptr, nullptr, nullptr) < 0);
  CHECK(spec_tree_build_greedy(3, 0, a.data(), 10, par.data(), nullptr, nullptr, nullptr) < 0);
  CHECK(spec_tree_build_greedy(3, 3, a.data(), -1, par.data(), nullptr, nullptr, nullptr) < 0);
  CHECK(spec_tree_build_greedy(3, 3, nullptr, 10, par.data(), nullptr, nullptr, nullptr) < 0);
  CHECK(spec_tree_build_greedy(3, 3, a.data(), 10, nullptr, nullptr, nullptr, nullptr) < 0);
  CHECK(spec_tree_build_greedy(3, 3, a.data(), SV_MAX_TREE_NODES, par.data(), nullptr, nullptr, nullptr) < 0);
}

int main() {
  linear_checks();
  tree_checks();
  row_checks();
  builder_checks();
  if (g_fail) {
    std::fprintf(stderr, "%d checks failed\n", g_fail);
    return 1;
  }
  std::printf("library host code: all checks passed\n");
  return 0;
}

// Reference oracle for speculative-decoding verification -- TEST INFRASTRUCTURE.
// Only tests, the smoke check and the benchmark's CPU-baseline leg use it.
//
// Plain single-threaded C++17; every quantity in double, every sum in ascending
// index order, inputs decoded exactly (bf16 = bits << 16, fp16 with subnormals,
// fp32 as stored). Citations and the rule set are in oracle.h.
#include "oracle.h"

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <vector>

namespace {

int g_mutation = 0;
enum {
  MUT_NONE = 0,
  MUT_RESIDUAL_AS_TARGET = 1,  // correction drawn from p_t,L instead of the residual
  MUT_SWAPPED_RATIO = 2,       // acceptance ratio p_d / p_t
  MUT_NO_BONUS = 3,            // no extra target token after a fully accepted draft
  MUT_INVCDF_GE = 4,           // inverse CDF with C_v >= u*S
  MUT_TREE_NO_ANCESTOR = 5,    // tree node accepted on its own match, ancestry ignored
  MUT_TEMPERATURE_IGNORED = 6, // softmax at T = 1 whatever T is
  MUT_LSE_WITHOUT_MAX = 7,     // lse missing the m/T term
  MUT_COMMIT_REJECTED_DRAFT = 8,  // commit keeps the rejected draft x_L in place of the target's token
  MUT_NEAR_LO_ONLY = 9,        // a draw's near tie checked against the lower bin edge only
  MUT_NEVAL_ALL = 10,          // every draw counted as evaluated, also those the result ignores
  MUT_ACCEPT_TIE_OFF = 11,     // accept-test near ties not flagged
};

// near_tie bits: a draw within tie_eps of its threshold that can change the
// accepted length (and so every output), and one that can change only the final
// token.
constexpr int32_t NT_DECISION = 1;
constexpr int32_t NT_FINAL = 2;

const double kNaN = std::numeric_limits<double>::quiet_NaN();
const double kInf = std::numeric_limits<double>::infinity();

double decode(int dtype, const void* base, int64_t i) {
  if (dtype == 0) {
    return (double) static_cast<const float*>(base)[i];
  }
  const uint16_t h = static_cast<const uint16_t*>(base)[i];
  if (dtype == 1) {  // bf16: the upper half of an fp32
    const uint32_t bits = (uint32_t)h << 16;
    float f;
    std::memcpy(&f, &bits, 4);
    return (double)f;
  }
  // IEEE binary16
  const int sign = (h >> 15) & 1, ex = (h >> 10) & 31, man = h & 1023;
  double mag;
  if (ex == 0) mag = std::ldexp((double)man, -24);
  else if (ex == 31) mag = man ? kNaN : kInf;
  else mag = std::ldexp((double)(1024 + man), ex - 25);
  return sign ? -mag : mag;
}

double effective_T(double T) { return g_mutation == MUT_TEMPERATURE_IGNORED ? 1.0 : T; }

// One logits row, decoded.
std::vector<double> load_row(int dtype, const void* base, int64_t row, int64_t V) {
  std::vector<double> x((size_t)V);
  for (int64_t v = 0; v < V; ++v) x[(size_t)v] = decode(dtype, base, row * V + v);
  return x;
}

// Largest value, lowest index on ties; NaN never chosen. found=false if no
// entry exceeds -inf.
struct ArgMax { double value; int64_t index; bool found; };
ArgMax argmax_of(const std::vector<double>& x) {
  ArgMax a{-kInf, 0, false};
  for (size_t v = 0; v < x.size(); ++v) {
    if (x[v] > a.value) { a.value = x[v]; a.index = (int64_t)v; a.found = true; }
  }
  return a;
}

// Softmax at temperature T: m = max x, z_v = exp((x_v - m)/T), Z = sum z.
struct Softmax {
  double m = -kInf, Z = 0;
  std::vector<double> z;
  bool ok = false;
  double prob(int64_t v) const { return z[(size_t)v] / Z; }
};
Softmax softmax_of(const std::vector<double>& x, double T) {
  Softmax s;
  T = effective_T(T);
  for (double xv : x) if (xv > s.m) s.m = xv;  // NaN entries compare false
  s.z.resize(x.size());
  double Z = 0;
  for (size_t v = 0; v < x.size(); ++v) {
    s.z[v] = std::exp((x[v] - s.m) / T);
    Z += s.z[v];
  }
  s.Z = Z;
  s.ok = std::isfinite(Z) && Z > 0;
  return s;
}

struct Draw { int64_t y; double lo, hi; };

Draw invcdf(const std::vector<double>& w, double u) {
  double S = 0;
  for (double wv : w) S += wv;
  Draw d{-1, kNaN, kNaN};
  if (!(S > 0) || !std::isfinite(S)) return d;
  const double thr = u * S;
  double C = 0;
  for (size_t v = 0; v < w.size(); ++v) {
    const double prev = C;
    C += w[v];
    const bool hit = (g_mutation == MUT_INVCDF_GE) ? (C >= thr) : (C > thr);
    if (hit) { d.y = (int64_t)v; d.lo = prev / S; d.hi = C / S; return d; }
  }
  // Rounding left no bin: the last index with positive weight.
  int64_t last = -1;
  for (size_t v = 0; v < w.size(); ++v) if (w[v] > 0) last = (int64_t)v;
  double before = 0;
  for (int64_t v = 0; v < last; ++v) before += w[(size_t)v];
  d.y = last;
  d.lo = before / S;
  d.hi = (before + w[(size_t)last]) / S;
  return d;
}

// Whether u lies within eps of either edge of the bin it selected: a draw whose
// outcome rounding could change.
bool near_draw(double u, const Draw& d, double eps) {
  if (g_mutation == MUT_NEAR_LO_ONLY) return std::fabs(u - d.lo) < eps;
  return std::fabs(u - d.lo) < eps || std::fabs(u - d.hi) < eps;
}

}  // namespace

extern "C" {

int orc_commit_linear(int64_t B, int64_t k, const int32_t* accept_len, const int32_t* out_tokens,
                      const int32_t* drafts, int32_t* seq_len, int32_t* history, int64_t capacity,
                      int32_t* shifted, int32_t* next_token, int32_t* err_flags) {
  if (B < 0 || k < 0 || !accept_len || !out_tokens || !seq_len) return -1;
  for (int64_t b = 0; b < B; ++b) {
    const int64_t L = accept_len[b];
    const int64_t len = seq_len[b];
    int32_t err = 0;
    if (L < 0 || L > k) err = 32;
    else if (history && (len < 0 || len + L + 1 > capacity)) err = 16;
    const int32_t* out = out_tokens + b * (k + 1);
    const int32_t y = err ? -1 : out[L];
    if (!err) {
      // the sequence grows by the accepted drafts and the target's token
      if (history)
        for (int64_t j = 0; j <= L; ++j) history[b * capacity + len + j] = out[j];
      if (history && g_mutation == MUT_COMMIT_REJECTED_DRAFT && L < k)
        history[b * capacity + len + L] = drafts[b * k + L];
      seq_len[b] = (int32_t)(len + L + 1);
    }
    if (shifted) {
      // input of the draft at position j: the token that follows position j
      for (int64_t j = 0; j <= k; ++j) {
        int32_t v;
        if (err) v = -1;
        else if (j < L) v = out[j];          // accepted draft x_j
        else if (j == L) v = y;              // the target's token
        else if (j < k) v = drafts[b * k + j];  // not accepted: left as drafted
        else v = y;                          // nothing follows the last position
        shifted[b * (k + 1) + j] = v;
      }
    }
    if (next_token) next_token[b] = y;
    if (err_flags) err_flags[b] = err;
  }
  return 0;
}

int orc_sample(int mode, double T, int64_t rows, int64_t V, int dtype, const void* x,
               const float* uniforms, double tie_eps, int32_t* tokens, int32_t* err_flags,
               int32_t* near_tie) {
  if (rows < 0 || V < 1 || !x || !tokens) return -1;
  if (mode == 1 && (!(T > 0) || !uniforms)) return -1;
  for (int64_t r = 0; r < rows; ++r) {
    const std::vector<double> row = load_row(dtype, x, r, V);
    int64_t y = -1;
    int32_t nt = 0;
    if (mode == 0) {
      const ArgMax a = argmax_of(row);
      if (a.found) y = a.index;
    } else {
      const Softmax s = softmax_of(row, T);
      if (s.ok) {
        const Draw d = invcdf(s.z, (double)uniforms[r]);
        y = d.y;
        nt = near_draw((double)uniforms[r], d, tie_eps) ? NT_FINAL : 0;
      }
    }
    tokens[r] = (int32_t)y;
    if (err_flags) err_flags[r] = y < 0 ? 2 : 0;
    if (near_tie) near_tie[r] = nt;
  }
  return 0;
}

int orc_tree_mask(int64_t n_nodes, const int32_t* parent, uint8_t* dense) {
  if (n_nodes < 1 || !parent || !dense) return -1;
  if (parent[0] != -1) return -1;
  for (int64_t i = 1; i < n_nodes; ++i)
    if (parent[i] < 0 || parent[i] >= i) return -1;
  for (int64_t i = 0; i < n_nodes; ++i) {
    uint8_t* row = dense + i * n_nodes;
    if (i == 0) {
      for (int64_t j = 0; j < n_nodes; ++j) row[j] = 0;
    } else {
      // what the parent sees, the node sees too
      const uint8_t* prow = dense + (int64_t)parent[i] * n_nodes;
      for (int64_t j = 0; j < n_nodes; ++j) row[j] = prow[j];
    }
    row[i] = 1;
  }
  return 0;
}

int64_t orc_tree_build_greedy(int64_t K, int64_t S, const double* acc, int64_t budget,
                              int32_t* parent, int32_t* depth, int32_t* rank, double* expected_len) {
  if (K < 1 || S < 1 || budget < 0 || !acc || !parent) return -1;
  struct Node { double value; int64_t depth, rank, parent; };   // parent: index in `added`
  std::vector<Node> added;
  added.push_back({1.0, 0, 0, -1});
  std::vector<Node> cand;
  for (int64_t r = 1; r <= S; ++r) cand.push_back({acc[r - 1], 1, r, 0});
  while ((int64_t)added.size() < budget + 1 && !cand.empty()) {
    // the candidate that contributes most (ties: shallower, earlier parent, lower rank)
    size_t best = 0;
    for (size_t c = 1; c < cand.size(); ++c) {
      const Node& a = cand[c];
      const Node& b = cand[best];
      bool better;
      if (a.value != b.value) better = a.value > b.value;
      else if (a.depth != b.depth) better = a.depth < b.depth;
      else if (a.parent != b.parent) better = a.parent < b.parent;
      else better = a.rank < b.rank;
      if (better) best = c;
    }
    const Node nd = cand[best];
    cand.erase(cand.begin() + (std::ptrdiff_t)best);
    const int64_t id = (int64_t)added.size();
    added.push_back(nd);
    if (nd.depth < K)
      for (int64_t r = 1; r <= S; ++r) cand.push_back({nd.value * acc[nd.depth * S + r - 1], nd.depth + 1, r, id});
  }
  // breadth-first numbering: a queue from the root, children in rank order
  const int64_t n = (int64_t)added.size();
  std::vector<std::vector<int64_t>> kids((size_t)n);
  for (int64_t i = 1; i < n; ++i) kids[(size_t)added[(size_t)i].parent].push_back(i);
  for (auto& v : kids)
    for (size_t a = 1; a < v.size(); ++a)   // insertion sort by rank
      for (size_t b = a; b > 0 && added[(size_t)v[b]].rank < added[(size_t)v[b - 1]].rank; --b)
        std::swap(v[b], v[b - 1]);
  std::vector<int64_t> queue(1, 0), num((size_t)n, -1);
  num[0] = 0;
  for (size_t h = 0; h < queue.size(); ++h)
    for (int64_t c : kids[(size_t)queue[h]]) {
      num[(size_t)c] = (int64_t)queue.size();
      queue.push_back(c);
    }
  double E = 0;
  for (size_t h = 0; h < queue.size(); ++h) {
    const Node& nd = added[(size_t)queue[h]];
    parent[h] = nd.parent < 0 ? -1 : (int32_t)num[(size_t)nd.parent];
    if (depth) depth[h] = (int32_t)nd.depth;
    if (rank) rank[h] = (int32_t)nd.rank;
    if (h > 0) E += nd.value;
  }
  if (expected_len) *expected_len = E;
  return n;
}

int orc_verify_tree_typical(double T, double epsilon, double delta, int64_t B, int64_t n_nodes,
                            int64_t V, int dtype, const int32_t* parent, int64_t parent_stride,
                            const int32_t* cand, const void* logits, const float* uniforms,
                            int64_t max_depth, double tie_eps, int32_t* accept_len,
                            int32_t* path_nodes, int32_t* out_tokens, int32_t* err_flags,
                            int32_t* near_tie, int32_t* n_eval) {
  if (B < 0 || n_nodes < 1 || V < 1 || !parent || !cand || !logits || !uniforms || max_depth < 0 ||
      !accept_len || !path_nodes || !out_tokens || !(T > 0))
    return -1;
  for (int64_t b = 0; b < B; ++b) {
    const int32_t* par = parent + b * parent_stride;
    const int32_t* cd = cand + b * n_nodes;
    int32_t* pn = path_nodes + b * max_depth;
    int32_t* out = out_tokens + b * (max_depth + 1);
    for (int64_t j = 0; j < max_depth; ++j) pn[j] = -1;
    for (int64_t j = 0; j <= max_depth; ++j) out[j] = -1;
    int32_t err = 0, nt = 0, ne = 0;
    std::vector<int64_t> depth((size_t)n_nodes, 0);
    if (par[0] != -1) err |= 4;
    for (int64_t i = 1; i < n_nodes && !(err & 4); ++i) {
      if (par[i] < 0 || par[i] >= i) { err |= 4; break; }
      depth[(size_t)i] = depth[(size_t)par[i]] + 1;
      if (depth[(size_t)i] > max_depth) err |= 4;
    }
    for (int64_t i = 1; i < n_nodes; ++i)
      if (cd[i] < 0 || cd[i] >= V) err |= 1;
    // every node's distribution and its entropy
    std::vector<Softmax> sm((size_t)n_nodes);
    std::vector<double> H((size_t)n_nodes, 0.0);
    for (int64_t n = 0; n < n_nodes; ++n) {
      sm[(size_t)n] = softmax_of(load_row(dtype, logits, b * n_nodes + n, V), T);
      if (!sm[(size_t)n].ok) { err |= 2; continue; }
      double h = 0;
      for (int64_t v = 0; v < V; ++v) {
        const double pv = sm[(size_t)n].prob(v);
        if (pv > 0) h -= pv * std::log(pv);
      }
      H[(size_t)n] = h;
    }
    if (!err) {
      std::vector<char> acc((size_t)n_nodes, 0), close((size_t)n_nodes, 0);
      acc[0] = 1;
      for (int64_t i = 1; i < n_nodes; ++i) {
        const int64_t p = par[i];
        const double prob = sm[(size_t)p].prob(cd[i]);
        const double tau = std::min(epsilon, delta * std::exp(-H[(size_t)p]));
        close[(size_t)i] = std::fabs(prob - tau) <= tie_eps * tau;
        acc[(size_t)i] = (prob > tau) && acc[(size_t)p];
      }
      int64_t best = 0;
      for (int64_t i = 1; i < n_nodes; ++i)
        if (acc[(size_t)i] && depth[(size_t)i] > depth[(size_t)best]) best = i;
      const int64_t L = depth[(size_t)best];
      accept_len[b] = (int32_t)L;
      int64_t node = best;
      for (int64_t j = L - 1; j >= 0; --j) {
        pn[j] = (int32_t)node;
        out[j] = cd[node];
        node = par[node];
      }
      // the result depends on the test of every child of an accepted node
      for (int64_t i = 1; i < n_nodes; ++i)
        if (acc[(size_t)par[i]] || g_mutation == MUT_NEVAL_ALL) {
          ++ne;
          if (close[(size_t)i] && g_mutation != MUT_ACCEPT_TIE_OFF) nt |= NT_DECISION;
        }
      const double u = (double)uniforms[b * n_nodes + best];
      const Draw d = invcdf(sm[(size_t)best].z, u);
      out[L] = (int32_t)d.y;
      ++ne;
      if (near_draw(u, d, tie_eps)) nt |= NT_FINAL;
    } else {
      accept_len[b] = -1;
    }
    if (err_flags) err_flags[b] = err;
    if (near_tie) near_tie[b] = nt;
    if (n_eval) n_eval[b] = ne;
  }
  return 0;
}

void orc_set_mutation(int which) { g_mutation = which; }

int orc_row_stats(int dtype, double T, int64_t rows, int64_t V, const void* x, double* m,
                  double* lse, int32_t* argmax, int32_t* flags) {
  if (!x || rows < 0 || V < 1 || !(T > 0)) return -1;
  for (int64_t r = 0; r < rows; ++r) {
    const std::vector<double> row = load_row(dtype, x, r, V);
    const ArgMax a = argmax_of(row);
    const Softmax s = softmax_of(row, T);
    const double Te = effective_T(T);
    if (m) m[r] = a.found ? a.value : -kInf;
    if (argmax) argmax[r] = a.found ? (int32_t)a.index : -1;
    if (lse) {
      const double base = (g_mutation == MUT_LSE_WITHOUT_MAX) ? 0.0 : s.m / Te;
      lse[r] = s.ok ? base + std::log(s.Z) : kNaN;
    }
    if (flags) flags[r] = (a.found && s.ok) ? 0 : 2;
  }
  return 0;
}

int64_t orc_invcdf(const double* w, int64_t n, double u, double* lo, double* hi) {
  std::vector<double> ww(w, w + n);
  const Draw d = invcdf(ww, u);
  if (lo) *lo = d.lo;
  if (hi) *hi = d.hi;
  return d.y;
}

int orc_verify_linear(int mode, double T, int64_t B, int64_t k, int64_t V, int dtype,
                      const void* target, const void* draft, const int32_t* draft_tokens,
                      const float* uniforms, double tie_eps, int32_t* accept_len,
                      int32_t* out_tokens, double* p_target, double* p_draft, int32_t* err_flags,
                      int32_t* near_tie, int32_t* n_eval) {
  const bool stochastic = (mode == 1);
  if (B < 0 || k < 0 || V < 1 || !target || (k > 0 && !draft_tokens) || !accept_len ||
      !out_tokens)
    return -1;
  if (stochastic && (!(T > 0) || !uniforms || (k > 0 && !draft))) return -1;

  for (int64_t b = 0; b < B; ++b) {
    int32_t* out = out_tokens + b * (k + 1);
    for (int64_t j = 0; j <= k; ++j) out[j] = -1;
    int32_t err = 0;
    const int32_t* x = draft_tokens + b * k;
    for (int64_t i = 0; i < k; ++i)
      if (x[i] < 0 || x[i] >= V) err |= 1;
    int32_t nt = 0, ne = 0;
    int64_t L = k;
    int64_t y = -1;

    if (!stochastic) {
      // Greedy: a draft token is accepted when it is the target's argmax there;
      // the extra token is the argmax after the accepted prefix.
      std::vector<ArgMax> am((size_t)(k + 1));
      for (int64_t i = 0; i <= k; ++i) {
        am[(size_t)i] = argmax_of(load_row(dtype, target, b * (k + 1) + i, V));
        if (!am[(size_t)i].found) err |= 2;
      }
      if (!err) {
        for (int64_t i = 0; i < k; ++i)
          if (x[i] != am[(size_t)i].index) { L = i; break; }
        y = am[(size_t)L].index;
      }
    } else {
      // Stochastic: softmax(x/T) for every target and draft row.
      std::vector<Softmax> st((size_t)(k + 1)), sd((size_t)k);
      for (int64_t i = 0; i <= k; ++i) {
        st[(size_t)i] = softmax_of(load_row(dtype, target, b * (k + 1) + i, V), T);
        if (!st[(size_t)i].ok) err |= 2;
      }
      for (int64_t i = 0; i < k; ++i) {
        sd[(size_t)i] = softmax_of(load_row(dtype, draft, b * k + i, V), T);
        if (!sd[(size_t)i].ok) err |= 2;
      }
      const float* u = uniforms + b * (k + 1);
      if (!err) {
        std::vector<double> pt((size_t)k), pd((size_t)k);
        for (int64_t i = 0; i < k; ++i) {
          pt[(size_t)i] = st[(size_t)i].prob(x[i]);
          pd[(size_t)i] = sd[(size_t)i].prob(x[i]);
          if (p_target) p_target[b * k + i] = pt[(size_t)i];
          if (p_draft) p_draft[b * k + i] = pd[(size_t)i];
        }
        for (int64_t i = 0; i < k; ++i) {
          double num = pt[(size_t)i], den = pd[(size_t)i];
          if (g_mutation == MUT_SWAPPED_RATIO) std::swap(num, den);
          double q;
          if (den > 0) q = num / den;
          else q = (num > 0) ? kInf : kNaN;
          const double thr = std::fmin(1.0, q);
          const bool accept = (double)u[i] < q;  // NaN ratio: reject
          ++ne;
          if (!std::isnan(q) && std::fabs((double)u[i] - thr) < tie_eps && g_mutation != MUT_ACCEPT_TIE_OFF)
            nt |= NT_DECISION;
          if (!accept) { L = i; break; }
        }
        if (g_mutation == MUT_NEVAL_ALL) ne = (int32_t)k;
        std::vector<double> w((size_t)V);
        const Softmax& tL = st[(size_t)L];
        if (L < k && g_mutation != MUT_RESIDUAL_AS_TARGET) {
          // residual max(0, p_t - p_d); zero total falls back to p_t
          const Softmax& dL = sd[(size_t)L];
          double S = 0;
          for (int64_t v = 0; v < V; ++v) {
            w[(size_t)v] = std::fmax(0.0, tL.prob(v) - dL.prob(v));
            S += w[(size_t)v];
          }
          if (!(S > 0)) w = tL.z;
        } else {
          w = tL.z;
        }
        const Draw d = invcdf(w, (double)u[k]);
        ++ne;
        if (near_draw((double)u[k], d, tie_eps)) nt |= NT_FINAL;
        y = d.y;
        if (y < 0) err |= 2;
      }
    }

    if (err) {
      accept_len[b] = -1;
      if (stochastic) {
        for (int64_t i = 0; i < k; ++i) {
          if (p_target) p_target[b * k + i] = kNaN;
          if (p_draft) p_draft[b * k + i] = kNaN;
        }
      }
      nt = 0;
      ne = 0;
    } else {
      accept_len[b] = (int32_t)L;
      for (int64_t i = 0; i < L; ++i) out[i] = x[i];
      if (!(g_mutation == MUT_NO_BONUS && L == k)) out[L] = (int32_t)y;
    }
    if (err_flags) err_flags[b] = err;
    if (near_tie) near_tie[b] = nt;
    if (n_eval) n_eval[b] = ne;
  }
  return 0;
}

int orc_verify_tree(int mode, double T, int64_t B, int64_t n_nodes, int64_t V, int dtype,
                    const int32_t* parent, int64_t parent_stride, const int32_t* cand,
                    const void* logits, const float* uniforms, int64_t max_depth, double tie_eps,
                    int32_t* accept_len, int32_t* path_nodes, int32_t* out_tokens,
                    int32_t* err_flags, int32_t* near_tie, int32_t* n_eval, int32_t* node_token) {
  const bool stochastic = (mode == 1);
  if (B < 0 || n_nodes < 1 || V < 1 || !parent || !cand || !logits || max_depth < 0 ||
      !accept_len || !path_nodes || !out_tokens)
    return -1;
  if (stochastic && (!(T > 0) || !uniforms)) return -1;

  for (int64_t b = 0; b < B; ++b) {
    const int32_t* par = parent + b * parent_stride;
    const int32_t* cd = cand + b * n_nodes;
    int32_t* pn = path_nodes + b * max_depth;
    int32_t* out = out_tokens + b * (max_depth + 1);
    for (int64_t j = 0; j < max_depth; ++j) pn[j] = -1;
    for (int64_t j = 0; j <= max_depth; ++j) out[j] = -1;
    int32_t err = 0, nt = 0, ne = 0;

    // Structure: parent[0] = -1, 0 <= parent[i] < i, depth within max_depth.
    std::vector<int64_t> depth((size_t)n_nodes, 0);
    if (par[0] != -1) err |= 4;
    for (int64_t i = 1; i < n_nodes && !(err & 4); ++i) {
      if (par[i] < 0 || par[i] >= i) { err |= 4; break; }
      depth[(size_t)i] = depth[(size_t)par[i]] + 1;
      if (depth[(size_t)i] > max_depth) err |= 4;
    }
    for (int64_t i = 1; i < n_nodes; ++i)
      if (cd[i] < 0 || cd[i] >= V) err |= 1;

    // Token chosen at every node from its own logits row.
    std::vector<int64_t> y((size_t)n_nodes, -1);
    std::vector<Draw> draw((size_t)n_nodes);
    for (int64_t n = 0; n < n_nodes; ++n) {
      const std::vector<double> row = load_row(dtype, logits, b * n_nodes + n, V);
      if (!stochastic) {
        const ArgMax a = argmax_of(row);
        if (!a.found) err |= 2;
        y[(size_t)n] = a.index;
      } else {
        const Softmax s = softmax_of(row, T);
        if (!s.ok) { err |= 2; continue; }
        draw[(size_t)n] = invcdf(s.z, (double)uniforms[b * n_nodes + n]);
        y[(size_t)n] = draw[(size_t)n].y;
      }
    }
    if (node_token)
      for (int64_t n = 0; n < n_nodes; ++n) node_token[b * n_nodes + n] = err ? -1 : (int32_t)y[(size_t)n];

    if (!err) {
      // A node is accepted when its token is the one chosen at its parent and
      // its parent is accepted; the root always is.
      std::vector<char> acc((size_t)n_nodes, 0);
      acc[0] = 1;
      for (int64_t i = 1; i < n_nodes; ++i) {
        const bool match = cd[i] == y[(size_t)par[i]];
        acc[(size_t)i] = (g_mutation == MUT_TREE_NO_ANCESTOR) ? match : (match && acc[(size_t)par[i]]);
      }
      // Deepest accepted node, lowest index on ties.
      int64_t best = 0;
      for (int64_t i = 1; i < n_nodes; ++i)
        if (acc[(size_t)i] && depth[(size_t)i] > depth[(size_t)best]) best = i;
      const int64_t L = depth[(size_t)best];
      accept_len[b] = (int32_t)L;
      int64_t node = best;
      for (int64_t j = L - 1; j >= 0; --j) {
        pn[j] = (int32_t)node;
        out[j] = cd[node];
        node = par[node];
      }
      out[L] = (int32_t)y[(size_t)best];
      if (stochastic) {
        // The draw at an accepted node decides which of its children are accepted
        // (so the path's length), and at a leaf on the path only the final token.
        std::vector<char> has_child((size_t)n_nodes, 0);
        for (int64_t i = 1; i < n_nodes; ++i) has_child[(size_t)par[i]] = 1;
        for (int64_t i = 0; i < n_nodes; ++i) {
          if (!acc[(size_t)i] && g_mutation != MUT_NEVAL_ALL) continue;
          ++ne;
          if (near_draw((double)uniforms[b * n_nodes + i], draw[(size_t)i], tie_eps))
            nt |= has_child[(size_t)i] ? NT_DECISION : NT_FINAL;
        }
      }
    } else {
      accept_len[b] = -1;
    }
    if (err_flags) err_flags[b] = err;
    if (near_tie) near_tie[b] = nt;
    if (n_eval) n_eval[b] = ne;
  }
  return 0;
}

double orc_expected_accept_len(int64_t n_nodes, const int32_t* parent, const int32_t* rank,
                               int64_t S, const double* acc) {
  std::vector<int64_t> depth((size_t)n_nodes, 0);
  std::vector<double> pathprob((size_t)n_nodes, 1.0);
  double E = 0;
  for (int64_t i = 1; i < n_nodes; ++i) {
    depth[(size_t)i] = depth[(size_t)parent[i]] + 1;
    pathprob[(size_t)i] =
        pathprob[(size_t)parent[i]] * acc[(depth[(size_t)i] - 1) * S + (rank[i] - 1)];
    E += pathprob[(size_t)i];
  }
  return E;
}

}  // extern "C"

// libspecverify: the steps around verification, for gfx950 — committing the
// verified tokens on the device, sampling a token per row, the tree attention
// mask, and the greedy construction of a sparse candidate tree.
//
// Sources: "Accelerating Sonar through speculation" (sections "MTP" and
// "MTP-Zeitplan für ein einzelnes Token": the draft's input tokens are the
// target's shifted one place left against its hidden states, and a kernel
// inserts the next target token so that no host synchronisation follows the
// acceptance; section "Inferenz mit spekulativem Decoding": the accepted count
// sets each sequence's next length; sections "MTP" and "Ziel-Entwurf": sampling
// and logit processing shared by every scheme); "Speculative-Decoding, LLM推理的加速
// / Medusa 方法阅读" (section 三: the tree attention mask, under which a token sees
// only itself and its ancestors, as a causal mask does in a chain; section 四: the
// greedy tree that adds, one node at a time, the node contributing most to the
// expected accepted length).
#include "../../include/specverify.h"
#include "sv_device.hpp"
#include "sv_host.hpp"
#include "sv_rows.hpp"

#include <hip/hip_runtime.h>
#include <algorithm>
#include <cstdint>
#include <queue>
#include <vector>

using namespace sv;

namespace {

// ------------------------------------------------------------------ commit
struct CommitParams {
  const int32_t* accept_len;
  const int32_t* out_tokens;   // [B][k+1]
  const int32_t* drafts;       // [B][k]
  int32_t* seq_len;            // [B]
  int32_t* history;            // [B][capacity]
  int64_t capacity;
  int32_t* shifted;            // [B][k+1]
  int32_t* next_token;         // [B]
  int32_t* err_flags;          // [B]
  int64_t B, k;
};

// One wave per sequence; lane j handles position j (k <= 31).
__global__ __launch_bounds__(BLOCK) void commit_kernel(CommitParams P) {
  const int64_t b = (int64_t)blockIdx.x * WPB + wave_in_block();
  if (b >= P.B) return;
  const int lane = lane_id();
  const int64_t k = P.k;
  const int L = P.accept_len[b];
  const int len = P.seq_len[b];   // every lane reads it before lane 0 updates it
  int err = 0;
  if (L < 0 || L > k) {
    err = SV_ERR_UNVERIFIED;
  } else if (P.history && (len < 0 || (int64_t)len + L + 1 > P.capacity)) {
    err = SV_ERR_CAPACITY;
  }
  const int y = err ? -1 : P.out_tokens[b * (k + 1) + L];
  if (lane <= k) {
    const int64_t j = lane;
    if (!err && j <= L && P.history) P.history[b * P.capacity + len + j] = P.out_tokens[b * (k + 1) + j];
    if (P.shifted) {
      // the token after position j: the committed x_j while accepted, y at L;
      // later positions keep the stale drafts (work on them is discarded), the
      // last one y
      int v = -1;
      if (!err) {
        if (j < L) v = P.out_tokens[b * (k + 1) + j];
        else if (j == L || j == k) v = y;
        else v = P.drafts[b * k + j];
      }
      P.shifted[b * (k + 1) + j] = v;
    }
  }
  if (lane == 0) {
    if (!err) P.seq_len[b] = len + L + 1;
    if (P.next_token) P.next_token[b] = y;
    if (P.err_flags) P.err_flags[b] = err;
  }
}

// ------------------------------------------------------------------ sampler
struct SampleParams {
  const char* x;
  const float* uniforms;
  int32_t* tokens;
  int32_t* err_flags;
  uint64_t* parts;      // [rows][C] Partial records
  uint32_t* row_cnt;    // [rows]
  int64_t rows, V;
  int C, CP;
  float c0;
  uint32_t tag;
  int64_t n_stream;
};

// One wave per (row, chunk); the last chunk of a row combines it and takes the
// token: argmax (greedy) or the inverse-CDF draw with the row's uniform.
template <int DT, bool STOCH>
__global__ __launch_bounds__(BLOCK) void sample_kernel(SampleParams P) {
  constexpr int E = DTraits<DT>::E;
  const int64_t w = (int64_t)blockIdx.x * WPB + wave_in_block();
  if (w >= P.n_stream) return;
  uint32_t q32, c32;
  stream_coords((uint32_t)w, (uint32_t)P.CP, (uint32_t)P.rows, q32, c32);
  if (c32 >= (uint32_t)P.C) return;   // padding wave
  const int64_t q = q32, c = c32;
  const char* row = P.x + (q * P.V) * E;
  const Partial p = chunk_partial<DT, STOCH, !STOCH>(row, P.V, c, P.c0);
  // the count before the record: a returning atomic also waits for the stores
  // issued before it (the reader polls the record's tag, so the order is free)
  uint32_t old = 0;
  if (lane_id() == 0) {
    old = counter_add(P.row_cnt + q * CSTRIDE, 1u);
    put_rec(P.parts + (q * P.C + c) * PART_WORDS, p, P.tag);
  }
  old = bcast(old);
  if (old + 1 != (uint32_t)P.C) return;
  const RowParts rp = read_parts(P.parts + q * P.C * PART_WORDS, P.C, P.tag);
  double wl[MAX_ROUNDS];
  const RowSums rs = row_sums<STOCH>(rp, P.c0, wl);
  int y = -1, err = 0;
  if (!rp.got) {
    err = SV_ERR_INTERNAL;
  } else if constexpr (STOCH) {
    const bool usable = rs.M > -INFINITY && __builtin_isfinite(rs.Z) && rs.Z > 0.0;
    if (usable) y = softmax_draw<DT>(row, P.V, P.C, P.c0, P.uniforms[q], rp, rs, wl);
    if (y < 0) err = SV_ERR_ROW;
  } else {
    y = rs.argmax;
    if (y < 0) err = SV_ERR_ROW;
  }
  if (lane_id() == 0) {
    P.tokens[q] = y;
    if (P.err_flags) P.err_flags[q] = err;
  }
  clear_parts<Partial>(P.parts + q * P.C * PART_WORDS, P.C, P.row_cnt + q * CSTRIDE);
}

template <int DT, bool STOCH>
struct SampleLauncher {
  static sv_status run(const SampleParams& P, hipStream_t s) {
    hipLaunchKernelGGL((sample_kernel<DT, STOCH>), dim3(blocks_for(P.n_stream)), dim3(BLOCK), 0, s, P);
    return launch_status();
  }
};

Layout sample_layout(int64_t rows, int64_t V, sv_dtype dt) {
  const int64_t C = chunks_per_row(V, dt);
  return make_layout({(size_t)(rows * C) * PART_WORDS * 8, (size_t)(rows * CSTRIDE) * 4});
}

// ------------------------------------------------------------------ tree mask
constexpr int MASK_SLOTS = (SV_MAX_TREE_NODES + 32 * WAVE - 1) / (32 * WAVE);   // words per lane per row

struct MaskParams {
  const int32_t* parent;
  int64_t parent_stride;
  uint32_t* mask;       // [T][n][W]
  int32_t* err_flags;   // [T]
  int64_t T, n, W;
};

// One wave per (tree, node i): the bits of row i are i and its ancestors. Lane l
// holds words l, l + 64, ... of the row in registers while the wave walks the
// chain of parents, then stores them.
__global__ __launch_bounds__(BLOCK) void tree_mask_kernel(MaskParams P) {
  const int64_t w = (int64_t)blockIdx.x * WPB + wave_in_block();
  if (w >= P.T * P.n) return;
  const int64_t t = w / P.n, i = w - t * P.n;
  const int lane = lane_id();
  const int32_t* par = P.parent + t * P.parent_stride;
  uint32_t words[MASK_SLOTS];
#pragma unroll
  for (int s = 0; s < MASK_SLOTS; ++s) words[s] = 0u;
  bool bad = (i == 0) ? (par[0] != -1) : false;
  int64_t j = i;
  while (true) {
    const int64_t word = j >> 5;
    if ((word & (WAVE - 1)) == lane) {
      const int slot = (int)(word >> 6);
#pragma unroll
      for (int s = 0; s < MASK_SLOTS; ++s)
        if (s == slot) words[s] |= 1u << (j & 31);
    }
    if (j == 0) break;
    const int64_t p = par[j];
    if (p < 0 || p >= j) {   // not an earlier node: the chain stops here
      bad = true;
      break;
    }
    j = p;
  }
  uint32_t* row = P.mask + (t * P.n + i) * P.W;
#pragma unroll
  for (int s = 0; s < MASK_SLOTS; ++s) {
    const int64_t word = (int64_t)s * WAVE + lane;
    if (word < P.W) row[word] = words[s];
  }
  if (bad && lane == 0 && P.err_flags)
    __hip_atomic_fetch_or(P.err_flags + t, (int32_t)SV_ERR_TREE, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(BLOCK) void zero_i32_kernel(int32_t* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * BLOCK + threadIdx.x;
  if (i < n) p[i] = 0;
}

// ------------------------------------------------------------------ greedy tree
// A node that may join the tree: the path product of accuracies down to it.
struct Candidate {
  double value;
  int32_t depth;    // 1..K (head)
  int32_t rank;     // 1..S
  int64_t parent;   // selection index of the parent (0 = root)
};

// Priority: larger value; then smaller depth, then earlier parent, then smaller rank.
struct Later {
  bool operator()(const Candidate& a, const Candidate& b) const {
    if (a.value != b.value) return a.value < b.value;
    if (a.depth != b.depth) return a.depth > b.depth;
    if (a.parent != b.parent) return a.parent > b.parent;
    return a.rank > b.rank;
  }
};

}  // namespace

extern "C" {

sv_status spec_commit_linear(int64_t B, int64_t k, const int32_t* accept_len, const int32_t* out_tokens,
                             const int32_t* draft_tokens, int32_t* seq_len, int32_t* history, int64_t capacity,
                             int32_t* shifted, int32_t* next_token, int32_t* err_flags, sv_stream_t stream) {
  if (B < 0 || k < 0 || capacity < 0) return SV_EINVAL;
  if (k > SV_MAX_K) return SV_ELIMIT;
  if (B == 0) return SV_OK;
  if (!accept_len || !out_tokens || !seq_len) return SV_EINVAL;
  if (shifted && k > 0 && !draft_tokens) return SV_EINVAL;
  if (capacity > 0 && !history) return SV_EINVAL;
  CommitParams P{};
  P.accept_len = accept_len;
  P.out_tokens = out_tokens;
  P.drafts = draft_tokens;
  P.seq_len = seq_len;
  P.history = capacity > 0 ? history : nullptr;
  P.capacity = capacity;
  P.shifted = shifted;
  P.next_token = next_token;
  P.err_flags = err_flags;
  P.B = B;
  P.k = k;
  if (B > MAX_WAVES) return SV_ELIMIT;
  hipLaunchKernelGGL(commit_kernel, dim3(blocks_for(B)), dim3(BLOCK), 0, reinterpret_cast<hipStream_t>(stream), P);
  return launch_status();
}

size_t spec_sample_workspace(int64_t rows, int64_t V, sv_dtype dtype) {
  if (rows < 0 || V < 1 || !dtype_ok(dtype)) return 0;
  return sample_layout(rows, V, dtype).total;
}

sv_status spec_sample(sv_mode mode, float temperature, int64_t rows, int64_t V, sv_dtype dtype, const void* logits,
                      const float* uniforms, int32_t* tokens, int32_t* err_flags, void* workspace,
                      size_t workspace_bytes, sv_stream_t stream) {
  if (!dtype_ok(dtype)) return SV_EDTYPE;
  if (mode != SV_GREEDY && mode != SV_STOCHASTIC) return SV_EINVAL;
  const bool stoch = mode == SV_STOCHASTIC;
  if (rows < 0 || V < 1) return SV_EINVAL;
  if (!shape_ok(V, dtype)) return SV_ELIMIT;
  if (rows == 0) return SV_OK;
  if (!logits || !tokens) return SV_EINVAL;
  if (stoch && (!temperature_ok(temperature) || !uniforms)) return SV_EINVAL;
  const Layout lay = sample_layout(rows, V, dtype);
  if (!ws_ok(workspace, workspace_bytes, lay.total)) return SV_EWORKSPACE;
  SampleParams P{};
  P.x = static_cast<const char*>(logits);
  P.uniforms = uniforms;
  P.tokens = tokens;
  P.err_flags = err_flags;
  char* ws = static_cast<char*>(workspace);
  P.parts = reinterpret_cast<uint64_t*>(ws + lay.off[0]);
  P.row_cnt = reinterpret_cast<uint32_t*>(ws + lay.off[1]);
  P.rows = rows;
  P.V = V;
  P.C = (int)chunks_per_row(V, dtype);
  P.CP = (P.C + WPB - 1) / WPB * WPB;
  P.c0 = stoch ? temperature_c0(temperature) : 1.0f;
  P.n_stream = rows * P.CP;
  if (P.n_stream > MAX_WAVES) return SV_ELIMIT;
  P.tag = next_tag();
  return dispatch<SampleLauncher>(dtype, stoch, P, reinterpret_cast<hipStream_t>(stream));
}

sv_status spec_tree_mask(int64_t n_trees, int64_t n_nodes, const int32_t* parent, int64_t parent_batch_stride,
                         uint32_t* mask, int32_t* err_flags, sv_stream_t stream) {
  if (n_trees < 0 || n_nodes < 1 || parent_batch_stride < 0) return SV_EINVAL;
  if (n_nodes > SV_MAX_TREE_NODES) return SV_ELIMIT;
  if (n_trees == 0) return SV_OK;
  if (!parent || !mask) return SV_EINVAL;
  if (n_trees * n_nodes > MAX_WAVES) return SV_ELIMIT;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (err_flags) {
    hipLaunchKernelGGL(zero_i32_kernel, dim3((unsigned)((n_trees + BLOCK - 1) / BLOCK)), dim3(BLOCK), 0, s,
                       err_flags, n_trees);
    if (launch_status() != SV_OK) return SV_EHIP;
  }
  MaskParams P{};
  P.parent = parent;
  P.parent_stride = parent_batch_stride;
  P.mask = mask;
  P.err_flags = err_flags;
  P.T = n_trees;
  P.n = n_nodes;
  P.W = (n_nodes + 31) / 32;
  hipLaunchKernelGGL(tree_mask_kernel, dim3(blocks_for(n_trees * n_nodes)), dim3(BLOCK), 0, s, P);
  return launch_status();
}

int64_t spec_tree_build_greedy(int64_t K, int64_t S, const double* accuracy, int64_t budget, int32_t* parent,
                               int32_t* depth, int32_t* rank, double* expected_len) {
  if (K < 1 || S < 1 || budget < 0 || !accuracy || !parent) return -SV_EINVAL;
  if (budget + 1 > SV_MAX_TREE_NODES) return -SV_ELIMIT;
  for (int64_t i = 0; i < K * S; ++i)
    if (!(accuracy[i] >= 0.0 && accuracy[i] <= 1.0)) return -SV_EINVAL;
  // selection: the candidate of largest contribution joins, its children become
  // candidates (a child never contributes more than its parent, so the chosen set
  // stays a tree)
  std::vector<Candidate> chosen;   // selection order; chosen[0] = root
  chosen.push_back({1.0, 0, 0, -1});
  std::priority_queue<Candidate, std::vector<Candidate>, Later> pq;
  for (int32_t r = 1; r <= S; ++r) pq.push({accuracy[r - 1], 1, r, 0});
  while ((int64_t)chosen.size() < budget + 1 && !pq.empty()) {
    const Candidate c = pq.top();
    pq.pop();
    const int64_t id = (int64_t)chosen.size();
    chosen.push_back(c);
    if (c.depth < K)
      for (int32_t r = 1; r <= S; ++r) pq.push({c.value * accuracy[c.depth * S + r - 1], c.depth + 1, r, id});
  }
  // number the nodes breadth first: by depth, then by the parent's number, then rank
  const int64_t n = (int64_t)chosen.size();
  std::vector<int64_t> order((size_t)n), num((size_t)n);
  for (int64_t i = 0; i < n; ++i) order[(size_t)i] = i;
  std::vector<int64_t> pnum((size_t)n, -1);
  int64_t next = 0;
  // depth by depth, so that a parent's number is known before its children are sorted
  for (int32_t d = 0; d <= K; ++d) {
    std::vector<int64_t> level;
    for (int64_t i = 0; i < n; ++i)
      if (chosen[(size_t)i].depth == d) level.push_back(i);
    std::stable_sort(level.begin(), level.end(), [&](int64_t a, int64_t b) {
      const int64_t pa = d ? num[(size_t)chosen[(size_t)a].parent] : -1;
      const int64_t pb = d ? num[(size_t)chosen[(size_t)b].parent] : -1;
      if (pa != pb) return pa < pb;
      return chosen[(size_t)a].rank < chosen[(size_t)b].rank;
    });
    for (int64_t i : level) num[(size_t)i] = next++;
  }
  double E = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    const Candidate& c = chosen[(size_t)i];
    const int64_t m = num[(size_t)i];
    parent[m] = c.depth ? (int32_t)num[(size_t)c.parent] : -1;
    if (depth) depth[m] = c.depth;
    if (rank) rank[m] = c.rank;
  }
  // expected accepted length: the contributions summed in node order
  std::vector<double> val((size_t)n);
  for (int64_t i = 0; i < n; ++i) val[(size_t)num[(size_t)i]] = chosen[(size_t)i].value;
  for (int64_t m = 1; m < n; ++m) E += val[(size_t)m];
  if (expected_len) *expected_len = E;
  return n;
}

}  // extern "C"

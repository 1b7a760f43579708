// libspecverify: speculative-decoding verification kernels for gfx950 and the C ABI
// declared in include/specverify.h.
//
// Linear drafts (one launch in greedy mode, two in stochastic mode):
//   linear_stats_kernel    one workgroup per (sequence, row, 16 KiB chunk): streams
//                          the chunk once (max / argmax / exp-sum partials). The last
//                          chunk of a row combines the row (max, normaliser, argmax)
//                          and, for target row k in stochastic mode, draws the bonus
//                          token. The last row of a sequence runs the acceptance test
//                          for all k positions at once (one lane per position), the
//                          first-reject scan, and emits the tokens.
//   linear_residual_kernel one workgroup per (sequence, chunk): for sequences that
//                          rejected at L < k, sums max(0, p_t,L - p_d,L) over its chunk;
//                          the last chunk picks the chunk holding u*S and runs the
//                          LDS block scan there (inverse CDF) for the correction token.
// Trees (one launch): tree_kernel streams every node row like the linear pass; the
// last chunk of a node picks the node's token (argmax or inverse-CDF draw); the last
// node of a tree runs the accepted-path search in LDS and emits.
//
// Sources: "Accelerating Sonar through speculation" (sections "Spekulatives
// Decoding", "Ziel-Entwurf", "MTP", "EAGLE"); "Speculative-Decoding, LLM推理的加速 /
// Medusa 方法阅读" (section 三). The acceptance rule is that of the Leviathan et al.
// method the Sonar page cites: accept x_i iff u_i < p_t,i(x_i) / p_d,i(x_i).
#include "../../include/specverify.h"
#include "sv_device.hpp"

#include <hip/hip_runtime.h>
#include <cmath>
#include <cstdint>

using namespace sv;

namespace {

constexpr double LN2 = 0.69314718055994530941723212145818;
constexpr double LOG2E = 1.4426950408889634073599246810019;

// ------------------------------------------------------------------ row finalisation
// Combines the C chunk partials of one row (wave 0), then optionally draws a token
// from softmax(row / T) with uniform u (whole block). Result is valid in all threads.
template <int DT, bool SUM>
__device__ RowStat finalize_row(const char* row, int64_t V, const Partial* parts, int C, float c0,
                                bool draw, float u, BlockScratch& sm, RowStat& sh) {
  if (wave_id() == 0) {
    const int lane = lane_id();
    const int per = (C + 63) / 64;
    const int c_lo = min(C, lane * per), c_hi = min(C, c_lo + per);
    float M = -INFINITY;
    int arg = INT_SENTINEL;
    for (int c = c_lo; c < c_hi; ++c) {
      const Partial p = fetch(parts + c);
      argmax_combine(M, arg, p.m, p.idx);
    }
    wave_argmax(M, arg);
    double Z = 0.0;
    if constexpr (SUM) {
      const double Mc0 = (double)M * (double)c0;
      double local = 0.0;
      for (int c = c_lo; c < c_hi; ++c) {
        const Partial p = fetch(parts + c);
        if (p.m != -INFINITY) local += p.s * exp2((double)chunk_mc0(p.m, c0) - Mc0);
      }
      Z = wave_sum(local);
    }
    if (lane == 0) {
      sh.M = M;
      sh.argmax = (M > -INFINITY && arg != INT_SENTINEL) ? arg : -1;
      sh.Z = Z;
      sh.ok = SUM ? ((M > -INFINITY) && __builtin_isfinite(Z) && Z > 0.0) : (M > -INFINITY);
      sh.y = SUM ? -1 : sh.argmax;
    }
  }
  __syncthreads();
  RowStat st = sh;
  __syncthreads();
  if constexpr (SUM) {
    if (draw && st.ok) {
      const double Mc0 = (double)st.M * (double)c0;
      if (wave_id() == 0) {
        const ChunkPick pk = pick_chunk(C, (double)u, [&](int c) -> double {
          const Partial p = fetch(parts + c);
          return (p.m == -INFINITY) ? 0.0 : p.s * exp2((double)chunk_mc0(p.m, c0) - Mc0);
        });
        if (lane_id() == 0) {
          sm.result = pk.c;
          if (pk.c >= 0) {
            const float mc0 = chunk_mc0(fetch(parts + pk.c).m, c0);
            // threshold in the chunk's own units (weights relative to its mc0)
            sm.theta = pk.fallback ? INFINITY : (pk.theta - pk.before) * exp2(Mc0 - (double)mc0);
          }
        }
      }
      __syncthreads();
      const int cstar = (int)sm.result;
      const double th = sm.theta;
      __syncthreads();
      if (cstar >= 0) {
        SoftmaxWeights<DT> pol{row, V, row_aligned(row), c0, chunk_mc0(fetch(parts + cstar).m, c0)};
        st.y = (int)chunk_invcdf<DT>(pol, cstar, th, sm);
      } else {
        st.y = -1;
      }
    }
  }
  return st;
}

// ------------------------------------------------------------------ linear
struct LinearParams {
  const char* target;
  const char* draft;
  const int32_t* tokens;
  const float* uniforms;
  int32_t* accept_len;
  int32_t* out_tokens;
  float* p_target;
  float* p_draft;
  int32_t* err_flags;
  Partial* parts;       // [B][R][C]
  RowStat* rows;        // [B][R]
  int32_t* seq_state;   // [B][4]: L, residual pending
  double* res_part;     // [B][C]
  unsigned* row_cnt;    // [B][R]   zero between calls
  unsigned* seq_cnt;    // [B]      zero between calls
  unsigned* res_cnt;    // [B]      zero between calls
  int64_t B, k, V;
  int R, C;
  float c0;
  int64_t nblocks;
};

template <int DT>
__device__ inline const char* linear_row(const LinearParams& P, int64_t b, int r) {
  constexpr int E = DTraits<DT>::E;
  if (r <= P.k) return P.target + ((b * (P.k + 1) + r) * P.V) * E;
  return P.draft + ((b * P.k + (r - P.k - 1)) * P.V) * E;
}

// Acceptance test, first-reject scan and emission for sequence b (wave 0).
template <int DT, bool STOCH>
__device__ void linear_decide(const LinearParams& P, int64_t b) {
  const int lane = lane_id();
  const int64_t k = P.k, V = P.V;
  const RowStat* rows = P.rows + b * P.R;
  const bool has = lane < k;
  const int x = has ? P.tokens[b * k + lane] : 0;
  const bool tok_bad = has && (x < 0 || x >= V);
  RowStat ts{}, ds{};
  if (has) ts = fetch(rows + lane);
  if (STOCH && has) ds = fetch(rows + k + 1 + lane);
  const RowStat tk = fetch(rows + k);
  const bool row_bad = (has && !ts.ok) || (STOCH && has && !ds.ok) || !tk.ok;
  int err = 0;
  if (__ballot(tok_bad)) err |= SV_ERR_TOKEN;
  if (__ballot(row_bad)) err |= SV_ERR_ROW;

  int32_t* out = P.out_tokens + b * (k + 1);
  if (err) {
    for (int64_t j = lane; j <= k; j += 64) out[j] = -1;
    if (STOCH && has) {
      if (P.p_target) P.p_target[b * k + lane] = NAN;
      if (P.p_draft) P.p_draft[b * k + lane] = NAN;
    }
    if (lane == 0) {
      P.accept_len[b] = -1;
      if (P.err_flags) P.err_flags[b] = err;
      P.seq_state[b * 4 + 0] = -1;
      P.seq_state[b * 4 + 1] = 0;
    }
    return;
  }
  bool acc = false;
  if constexpr (!STOCH) {
    acc = has && (x == ts.argmax);
  } else {
    if (has) {
      const double c0d = (double)P.c0;
      const float tx = load_elem<DT>(linear_row<DT>(P, b, lane), x);
      const float dx = load_elem<DT>(linear_row<DT>(P, b, (int)(k + 1 + lane)), x);
      const double pt = exp2(((double)tx - (double)ts.M) * c0d) / ts.Z;
      const double pd = exp2(((double)dx - (double)ds.M) * c0d) / ds.Z;
      double q;
      if (pd > 0.0) q = pt / pd;
      else q = (pt > 0.0) ? INFINITY : NAN;
      acc = (double)P.uniforms[b * (k + 1) + lane] < q;  // NaN ratio rejects
      if (P.p_target) P.p_target[b * k + lane] = (float)pt;
      if (P.p_draft) P.p_draft[b * k + lane] = (float)pd;
    }
  }
  const unsigned long long rej = __ballot(has && !acc);
  const int L = rej ? __builtin_ctzll(rej) : (int)k;
  bool pending = false;
  int y;
  if constexpr (!STOCH) {
    const int yl = __shfl(ts.argmax, L & 63);
    y = (L == k) ? tk.argmax : yl;
  } else {
    pending = (L < k);
    y = tk.y;
  }
  for (int64_t j = lane; j <= k; j += 64) {
    if (j < L) out[j] = x;  // j == lane here: lane L-1 < 64 holds x_j
    else if (j == L) { if (!pending) out[j] = y; }
    else out[j] = -1;
  }
  if (lane == 0) {
    P.accept_len[b] = L;
    if (P.err_flags) P.err_flags[b] = 0;
    P.seq_state[b * 4 + 0] = L;
    P.seq_state[b * 4 + 1] = pending ? 1 : 0;
  }
}

template <int DT, bool STOCH>
__global__ __launch_bounds__(BLOCK) void linear_stats_kernel(LinearParams P) {
  __shared__ BlockScratch sm;
  __shared__ RowStat rsh;
  const int64_t lb = xcd_logical_block(blockIdx.x, P.nblocks);
  const int64_t per_seq = (int64_t)P.R * P.C;
  const int64_t b = lb / per_seq;
  const int r = (int)((lb / P.C) % P.R);
  const int64_t c = lb % P.C;
  const char* row = linear_row<DT>(P, b, r);

  const Partial p = chunk_stats<DT, STOCH, !STOCH>(row, P.V, c, P.c0, sm);
  const int64_t rid = b * P.R + r;
  if (threadIdx.x == 0) publish(P.parts + rid * P.C + c, p);
  if (!arrive_last(&P.row_cnt[rid], (unsigned)P.C, sm)) return;

  const bool draw = STOCH && (r == P.k);
  const float u = draw ? P.uniforms[b * (P.k + 1) + P.k] : 0.0f;
  const RowStat st = finalize_row<DT, STOCH>(row, P.V, P.parts + rid * P.C, P.C, P.c0, draw, u, sm, rsh);
  if (threadIdx.x == 0) publish(P.rows + rid, st);
  if (!arrive_last(&P.seq_cnt[b], (unsigned)P.R, sm)) return;
  if (wave_id() == 0) linear_decide<DT, STOCH>(P, b);
}

template <int DT>
__global__ __launch_bounds__(BLOCK) void linear_residual_kernel(LinearParams P, int64_t nblocks) {
  __shared__ BlockScratch sm;
  __shared__ RowStat rsh;
  const int64_t lb = xcd_logical_block(blockIdx.x, nblocks);
  const int64_t b = lb / P.C;
  const int64_t c = lb % P.C;
  if (P.seq_state[b * 4 + 1] == 0) return;  // same for the whole block
  const int L = P.seq_state[b * 4 + 0];
  const int64_t k = P.k;
  const RowStat ts = P.rows[b * P.R + L];
  const RowStat ds = P.rows[b * P.R + k + 1 + L];
  const char* trow = linear_row<DT>(P, b, L);
  const char* drow = linear_row<DT>(P, b, (int)(k + 1 + L));
  const float c0 = P.c0;
  const float mc0t = ts.M * c0, mc0d = ds.M * c0;
  // 1 / sum_v exp2(x_v*c0 - fl32(M*c0)) from Z = sum_v exp2(x_v*c0 - M*c0)
  const float izt = (float)(1.0 / (ts.Z * exp2((double)ts.M * (double)c0 - (double)mc0t)));
  const float izd = (float)(1.0 / (ds.Z * exp2((double)ds.M * (double)c0 - (double)mc0d)));
  ResidualWeights<DT> pol{trow, drow, P.V, row_aligned(trow), row_aligned(drow), c0, mc0t, mc0d, izt, izd};

  const double s = chunk_weight_sum<DT>(pol, c, sm);
  if (threadIdx.x == 0) publish(P.res_part + b * P.C + c, s);
  if (!arrive_last(&P.res_cnt[b], (unsigned)P.C, sm)) return;

  const float u = P.uniforms[b * (k + 1) + k];
  const double* rp = P.res_part + b * P.C;
  if (wave_id() == 0) {
    const ChunkPick pk = pick_chunk(P.C, (double)u, [&](int cc) -> double { return fetch(rp + cc); });
    if (lane_id() == 0) {
      sm.result = pk.c;
      sm.theta = pk.fallback ? INFINITY : pk.theta - pk.before;
    }
  }
  __syncthreads();
  const int cstar = (int)sm.result;
  const double th = sm.theta;
  __syncthreads();
  int y;
  if (cstar >= 0) {
    y = (int)chunk_invcdf<DT>(pol, cstar, th, sm);
  } else {
    // no residual mass (equal rows up to rounding): draw from p_t,L instead
    const RowStat st = finalize_row<DT, true>(trow, P.V, P.parts + (b * P.R + L) * P.C, P.C, c0,
                                              true, u, sm, rsh);
    y = st.y;
  }
  if (threadIdx.x == 0) P.out_tokens[b * (k + 1) + L] = y;
}

// ------------------------------------------------------------------ trees
struct TreeParams {
  const char* logits;
  const int32_t* parent;
  int64_t parent_stride;
  const int32_t* cand;
  const float* uniforms;
  int32_t* accept_len;
  int32_t* path_nodes;
  int32_t* out_tokens;
  int32_t* err_flags;
  Partial* parts;       // [B][N][C]
  int32_t* node_y;      // [B][N]  token chosen at each node, -1 if its row is unusable
  unsigned* row_cnt;    // [B][N]  zero between calls
  unsigned* tree_cnt;   // [B]     zero between calls
  int64_t B, N, V, max_depth;
  int C;
  float c0;
  int64_t nblocks;
};

// Accepted-path search for tree b (whole block). LDS: parent (int16) and match
// flag (uint8) of every node.
__device__ void tree_walk(const TreeParams& P, int64_t b, unsigned char* smem, BlockScratch& sm) {
  const int64_t N = P.N;
  int16_t* par_s = reinterpret_cast<int16_t*>(smem);
  unsigned char* match_s = smem + 2 * N;
  const int32_t* par = P.parent + b * P.parent_stride;
  const int32_t* cand = P.cand + b * N;
  const int32_t* ny = P.node_y + b * N;
  int err = 0;
  for (int64_t i = threadIdx.x; i < N; i += BLOCK) {
    const int p = par[i];
    const bool bad = (i == 0) ? (p != -1) : (p < 0 || p >= i);
    par_s[i] = (int16_t)(bad ? 0 : p);
    if (bad) err |= SV_ERR_TREE;
    if (fetch(ny + i) < 0) err |= SV_ERR_ROW;
    unsigned char m = 0;
    if (i > 0) {
      const int ci = cand[i];
      if (ci < 0 || ci >= P.V) err |= SV_ERR_TOKEN;
      if (!bad) m = (ci == fetch(ny + p)) ? 1 : 0;
    }
    match_s[i] = m;
  }
  // OR of the error bits over the block (each bit separately)
  int all_err = 0;
  for (int bit = 1; bit <= SV_ERR_TREE; bit <<= 1)
    if (__syncthreads_or(err & bit)) all_err |= bit;

  // Depth check and path search (bad parents were replaced by the root above, so
  // every chain ends; the depth bound is checked whatever other error was found).
  unsigned long long best_key = 0ull;
  int too_deep = 0;
  {
    for (int64_t i = threadIdx.x; i < N; i += BLOCK) {
      int64_t j = i, d = 0;
      int acc = 1;
      while (j != 0) {
        if (d >= P.max_depth) { too_deep = 1; break; }
        acc &= match_s[j];
        j = par_s[j];
        ++d;
      }
      if (acc && !too_deep) {
        const unsigned long long key = ((unsigned long long)d << 32) | (0xffffffffull - (unsigned long long)i);
        if (key > best_key) best_key = key;
      }
    }
    if (__syncthreads_or(too_deep)) all_err |= SV_ERR_TREE;
  }
  int32_t* path = P.path_nodes + b * P.max_depth;
  int32_t* out = P.out_tokens + b * (P.max_depth + 1);
  if (all_err) {
    for (int64_t j = threadIdx.x; j < P.max_depth; j += BLOCK) path[j] = -1;
    for (int64_t j = threadIdx.x; j <= P.max_depth; j += BLOCK) out[j] = -1;
    if (threadIdx.x == 0) {
      P.accept_len[b] = -1;
      if (P.err_flags) P.err_flags[b] = all_err;
    }
    return;
  }
  // block max of the (depth, -index) key
  {
    unsigned long long v = best_key;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const unsigned long long t = __shfl_xor(v, o);
      v = t > v ? t : v;
    }
    if (lane_id() == 0) sm.d[wave_id()] = __longlong_as_double((long long)v);
    __syncthreads();
    unsigned long long r = 0ull;
    for (int w = 0; w < NWAVES; ++w) {
      const unsigned long long t = (unsigned long long)__double_as_longlong(sm.d[w]);
      r = t > r ? t : r;
    }
    __syncthreads();
    best_key = r;
  }
  const int L = (int)(best_key >> 32);
  const int best = (int)(0xffffffffull - (best_key & 0xffffffffull));
  for (int64_t j = L + threadIdx.x; j < P.max_depth; j += BLOCK) path[j] = -1;
  for (int64_t j = L + 1 + threadIdx.x; j <= P.max_depth; j += BLOCK) out[j] = -1;
  if (threadIdx.x == 0) {
    int node = best;
    for (int j = L - 1; j >= 0; --j) {
      path[j] = node;
      out[j] = cand[node];
      node = par_s[node];
    }
    out[L] = fetch(ny + best);
    P.accept_len[b] = L;
    if (P.err_flags) P.err_flags[b] = 0;
  }
}

template <int DT, bool STOCH>
__global__ __launch_bounds__(BLOCK) void tree_kernel(TreeParams P) {
  __shared__ BlockScratch sm;
  __shared__ RowStat rsh;
  extern __shared__ unsigned char walk_smem[];
  constexpr int E = DTraits<DT>::E;
  const int64_t lb = xcd_logical_block(blockIdx.x, P.nblocks);
  const int64_t per_tree = P.N * P.C;
  const int64_t b = lb / per_tree;
  const int64_t n = (lb / P.C) % P.N;
  const int64_t c = lb % P.C;
  const int64_t rid = b * P.N + n;
  const char* row = P.logits + (rid * P.V) * E;

  const Partial p = chunk_stats<DT, STOCH, !STOCH>(row, P.V, c, P.c0, sm);
  if (threadIdx.x == 0) publish(P.parts + rid * P.C + c, p);
  if (!arrive_last(&P.row_cnt[rid], (unsigned)P.C, sm)) return;

  const float u = STOCH ? P.uniforms[rid] : 0.0f;
  const RowStat st = finalize_row<DT, STOCH>(row, P.V, P.parts + rid * P.C, P.C, P.c0, STOCH, u, sm, rsh);
  if (threadIdx.x == 0) publish(P.node_y + rid, (int32_t)(st.ok ? st.y : -1));
  if (!arrive_last(&P.tree_cnt[b], (unsigned)P.N, sm)) return;
  tree_walk(P, b, walk_smem, sm);
}

// ------------------------------------------------------------------ row statistics
struct RowStatsParams {
  const char* x;
  float* row_max;
  float* row_lse;
  int32_t* row_argmax;
  int32_t* err_flags;
  Partial* parts;
  unsigned* row_cnt;
  int64_t rows, V;
  int C;
  float c0;
  int64_t nblocks;
};

template <int DT>
__global__ __launch_bounds__(BLOCK) void row_stats_kernel(RowStatsParams P) {
  __shared__ BlockScratch sm;
  __shared__ RowStat rsh;
  constexpr int E = DTraits<DT>::E;
  const int64_t lb = xcd_logical_block(blockIdx.x, P.nblocks);
  const int64_t r = lb / P.C, c = lb % P.C;
  const char* row = P.x + (r * P.V) * E;
  const Partial p = chunk_stats<DT, true, true>(row, P.V, c, P.c0, sm);
  if (threadIdx.x == 0) publish(P.parts + r * P.C + c, p);
  if (!arrive_last(&P.row_cnt[r], (unsigned)P.C, sm)) return;
  // argmax needs the ARG partials, the normaliser the SUM partials: both are kept
  const RowStat st = finalize_row<DT, true>(row, P.V, P.parts + r * P.C, P.C, P.c0, false, 0.0f, sm, rsh);
  if (threadIdx.x == 0) {
    const bool ok = st.ok && st.argmax >= 0;
    if (P.row_max) P.row_max[r] = st.M;
    if (P.row_argmax) P.row_argmax[r] = st.argmax;
    if (P.row_lse) P.row_lse[r] = ok ? (float)((double)st.M * (double)P.c0 * LN2 + log(st.Z)) : NAN;
    if (P.err_flags) P.err_flags[r] = ok ? 0 : SV_ERR_ROW;
  }
}

__global__ __launch_bounds__(BLOCK) void clear_kernel(unsigned char* p, size_t bytes) {
  const size_t n16 = bytes / 16;
  const size_t stride = (size_t)gridDim.x * BLOCK;
  uint4* q = reinterpret_cast<uint4*>(p);
  for (size_t i = (size_t)blockIdx.x * BLOCK + threadIdx.x; i < n16; i += stride) q[i] = make_uint4(0, 0, 0, 0);
  for (size_t i = n16 * 16 + (size_t)blockIdx.x * BLOCK + threadIdx.x; i < bytes; i += stride) p[i] = 0;
}

// ------------------------------------------------------------------ host helpers
int elem_bytes(sv_dtype dt) { return dt == SV_F32 ? 4 : 2; }
bool dtype_ok(int dt) { return dt == SV_F32 || dt == SV_BF16 || dt == SV_F16; }

int64_t chunks_per_row(int64_t V, sv_dtype dt) {
  const int64_t W = 16 / elem_bytes(dt);
  const int64_t units = (V + W - 1) / W;
  return (units + UNITS_PER_CHUNK - 1) / UNITS_PER_CHUNK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Layout {
  size_t off[8];
  size_t total;
};

// Regions laid out back to back, each 256-byte aligned.
Layout make_layout(std::initializer_list<size_t> sizes) {
  Layout L{};
  size_t o = 0;
  int i = 0;
  for (size_t s : sizes) {
    L.off[i++] = o;
    o += align256(s);
  }
  L.total = o;
  return L;
}

Layout linear_layout(int64_t B, int64_t k, int64_t V, sv_dtype dt, sv_mode mode) {
  const int64_t R = (mode == SV_STOCHASTIC) ? 2 * k + 1 : k + 1;
  const int64_t C = chunks_per_row(V, dt);
  return make_layout({(size_t)(B * R * C) * sizeof(Partial), (size_t)(B * R) * sizeof(RowStat),
                      (size_t)B * 16, (size_t)(B * C) * sizeof(double), (size_t)(B * R) * 4,
                      (size_t)B * 4, (size_t)B * 4});
}

Layout tree_layout(int64_t B, int64_t N, int64_t V, sv_dtype dt) {
  const int64_t C = chunks_per_row(V, dt);
  return make_layout({(size_t)(B * N * C) * sizeof(Partial), (size_t)(B * N) * 4,
                      (size_t)(B * N) * 4, (size_t)B * 4});
}

Layout rowstats_layout(int64_t rows, int64_t V, sv_dtype dt) {
  const int64_t C = chunks_per_row(V, dt);
  return make_layout({(size_t)(rows * C) * sizeof(Partial), (size_t)rows * 4});
}

bool temperature_ok(float T) { return std::isfinite(T) && T > 0.0f; }

float temperature_c0(float T) { return (float)(LOG2E / (double)T); }

sv_status launch_status() {
  return hipGetLastError() == hipSuccess ? SV_OK : SV_EHIP;
}

template <template <int, bool> class Launcher, class... Args>
sv_status dispatch(sv_dtype dt, bool stoch, Args&&... args) {
  switch (dt) {
    case SV_F32: return stoch ? Launcher<DT_F32, true>::run(args...) : Launcher<DT_F32, false>::run(args...);
    case SV_BF16: return stoch ? Launcher<DT_BF16, true>::run(args...) : Launcher<DT_BF16, false>::run(args...);
    case SV_F16: return stoch ? Launcher<DT_F16, true>::run(args...) : Launcher<DT_F16, false>::run(args...);
  }
  return SV_EDTYPE;
}

enum LinearPhase { PHASE_ACCEPT = 1, PHASE_CORRECT = 2, PHASE_BOTH = 3 };

template <int DT, bool STOCH>
struct LinearLauncher {
  static sv_status run(const LinearParams& P, int phases, hipStream_t s) {
    if (phases & PHASE_ACCEPT) {
      hipLaunchKernelGGL((linear_stats_kernel<DT, STOCH>), dim3((unsigned)P.nblocks), dim3(BLOCK), 0, s, P);
      if (hipGetLastError() != hipSuccess) return SV_EHIP;
    }
    if ((phases & PHASE_CORRECT) && STOCH && P.k > 0) {
      const int64_t nb = P.B * P.C;
      hipLaunchKernelGGL((linear_residual_kernel<DT>), dim3((unsigned)nb), dim3(BLOCK), 0, s, P, nb);
    }
    return launch_status();
  }
};

template <int DT, bool STOCH>
struct TreeLauncher {
  static sv_status run(const TreeParams& P, size_t smem, hipStream_t s) {
    hipLaunchKernelGGL((tree_kernel<DT, STOCH>), dim3((unsigned)P.nblocks), dim3(BLOCK), smem, s, P);
    return launch_status();
  }
};

template <int DT, bool UNUSED>
struct RowStatsLauncher {
  static sv_status run(const RowStatsParams& P, hipStream_t s) {
    hipLaunchKernelGGL((row_stats_kernel<DT>), dim3((unsigned)P.nblocks), dim3(BLOCK), 0, s, P);
    return launch_status();
  }
};

bool ws_ok(const void* ws, size_t have, size_t need) {
  return ws != nullptr && (reinterpret_cast<uintptr_t>(ws) & 255u) == 0 && have >= need;
}

constexpr int64_t MAX_BLOCKS = 0x7fffffff;

}  // namespace

extern "C" {

const char* spec_verify_status_string(sv_status s) {
  switch (s) {
    case SV_OK: return "ok";
    case SV_EINVAL: return "invalid argument";
    case SV_EDTYPE: return "unknown dtype";
    case SV_EWORKSPACE: return "workspace missing, misaligned or too small";
    case SV_EHIP: return "HIP launch failed";
    case SV_ELIMIT: return "shape beyond a documented limit";
  }
  return "unknown status";
}

size_t spec_verify_linear_workspace(int64_t B, int64_t k, int64_t V, sv_dtype dtype, sv_mode mode) {
  if (B < 0 || k < 0 || V < 1 || !dtype_ok(dtype)) return 0;
  return linear_layout(B, k, V, dtype, mode).total;
}

static sv_status linear_entry(int phases, sv_mode mode, float temperature, int64_t B, int64_t k,
                              int64_t V, sv_dtype dtype, const void* target_logits,
                              const void* draft_logits, const int32_t* draft_tokens,
                              const float* uniforms, int32_t* accept_len, int32_t* out_tokens,
                              float* p_target, float* p_draft, int32_t* err_flags, void* workspace,
                              size_t workspace_bytes, sv_stream_t stream) {
  if (!dtype_ok(dtype)) return SV_EDTYPE;
  if (mode != SV_GREEDY && mode != SV_STOCHASTIC) return SV_EINVAL;
  const bool stoch = (mode == SV_STOCHASTIC);
  if (B < 0 || k < 0 || V < 1) return SV_EINVAL;
  if (k > SV_MAX_K || V > 0x7fffffffLL - 16) return SV_ELIMIT;
  if (chunks_per_row(V, dtype) > MAX_CHUNKS) return SV_ELIMIT;
  if (B == 0) return SV_OK;
  if (!target_logits || !accept_len || !out_tokens || (k > 0 && !draft_tokens)) return SV_EINVAL;
  if (stoch && (!temperature_ok(temperature) || !uniforms || (k > 0 && !draft_logits))) return SV_EINVAL;
  const Layout lay = linear_layout(B, k, V, dtype, mode);
  if (!ws_ok(workspace, workspace_bytes, lay.total)) return SV_EWORKSPACE;

  LinearParams P{};
  P.target = static_cast<const char*>(target_logits);
  P.draft = static_cast<const char*>(draft_logits);
  P.tokens = draft_tokens;
  P.uniforms = uniforms;
  P.accept_len = accept_len;
  P.out_tokens = out_tokens;
  P.p_target = stoch ? p_target : nullptr;
  P.p_draft = stoch ? p_draft : nullptr;
  P.err_flags = err_flags;
  char* ws = static_cast<char*>(workspace);
  P.parts = reinterpret_cast<Partial*>(ws + lay.off[0]);
  P.rows = reinterpret_cast<RowStat*>(ws + lay.off[1]);
  P.seq_state = reinterpret_cast<int32_t*>(ws + lay.off[2]);
  P.res_part = reinterpret_cast<double*>(ws + lay.off[3]);
  P.row_cnt = reinterpret_cast<unsigned*>(ws + lay.off[4]);
  P.seq_cnt = reinterpret_cast<unsigned*>(ws + lay.off[5]);
  P.res_cnt = reinterpret_cast<unsigned*>(ws + lay.off[6]);
  P.B = B;
  P.k = k;
  P.V = V;
  P.R = (int)(stoch ? 2 * k + 1 : k + 1);
  P.C = (int)chunks_per_row(V, dtype);
  P.c0 = stoch ? temperature_c0(temperature) : 1.0f;
  P.nblocks = B * P.R * P.C;
  if (P.nblocks > MAX_BLOCKS) return SV_ELIMIT;
  return dispatch<LinearLauncher>(dtype, stoch, P, phases, reinterpret_cast<hipStream_t>(stream));
}

sv_status spec_verify_linear(sv_mode mode, float temperature, int64_t B, int64_t k, int64_t V,
                             sv_dtype dtype, const void* target_logits, const void* draft_logits,
                             const int32_t* draft_tokens, const float* uniforms, int32_t* accept_len,
                             int32_t* out_tokens, float* p_target, float* p_draft,
                             int32_t* err_flags, void* workspace, size_t workspace_bytes,
                             sv_stream_t stream) {
  return linear_entry(PHASE_BOTH, mode, temperature, B, k, V, dtype, target_logits, draft_logits,
                      draft_tokens, uniforms, accept_len, out_tokens, p_target, p_draft, err_flags,
                      workspace, workspace_bytes, stream);
}

sv_status spec_verify_linear_accept(sv_mode mode, float temperature, int64_t B, int64_t k, int64_t V,
                                    sv_dtype dtype, const void* target_logits,
                                    const void* draft_logits, const int32_t* draft_tokens,
                                    const float* uniforms, int32_t* accept_len, int32_t* out_tokens,
                                    float* p_target, float* p_draft, int32_t* err_flags,
                                    void* workspace, size_t workspace_bytes, sv_stream_t stream) {
  return linear_entry(PHASE_ACCEPT, mode, temperature, B, k, V, dtype, target_logits, draft_logits,
                      draft_tokens, uniforms, accept_len, out_tokens, p_target, p_draft, err_flags,
                      workspace, workspace_bytes, stream);
}

sv_status spec_verify_linear_correct(sv_mode mode, float temperature, int64_t B, int64_t k, int64_t V,
                                     sv_dtype dtype, const void* target_logits,
                                     const void* draft_logits, const int32_t* draft_tokens,
                                     const float* uniforms, int32_t* accept_len, int32_t* out_tokens,
                                     float* p_target, float* p_draft, int32_t* err_flags,
                                     void* workspace, size_t workspace_bytes, sv_stream_t stream) {
  return linear_entry(PHASE_CORRECT, mode, temperature, B, k, V, dtype, target_logits, draft_logits,
                      draft_tokens, uniforms, accept_len, out_tokens, p_target, p_draft, err_flags,
                      workspace, workspace_bytes, stream);
}

size_t spec_verify_tree_workspace(int64_t B, int64_t n_nodes, int64_t V, sv_dtype dtype, sv_mode mode) {
  (void)mode;
  if (B < 0 || n_nodes < 1 || V < 1 || !dtype_ok(dtype)) return 0;
  return tree_layout(B, n_nodes, V, dtype).total;
}

sv_status spec_verify_tree(sv_mode mode, float temperature, int64_t B, int64_t n_nodes, int64_t V,
                           sv_dtype dtype, const int32_t* parent, int64_t parent_batch_stride,
                           const int32_t* cand_tokens, const void* target_logits,
                           const float* uniforms, int64_t max_depth, int32_t* accept_len,
                           int32_t* path_nodes, int32_t* out_tokens, int32_t* err_flags,
                           void* workspace, size_t workspace_bytes, sv_stream_t stream) {
  if (!dtype_ok(dtype)) return SV_EDTYPE;
  if (mode != SV_GREEDY && mode != SV_STOCHASTIC) return SV_EINVAL;
  const bool stoch = (mode == SV_STOCHASTIC);
  if (B < 0 || n_nodes < 1 || V < 1 || max_depth < 0 || parent_batch_stride < 0) return SV_EINVAL;
  if (n_nodes > SV_MAX_TREE_NODES || V > 0x7fffffffLL - 16) return SV_ELIMIT;
  if (chunks_per_row(V, dtype) > MAX_CHUNKS) return SV_ELIMIT;
  if (B == 0) return SV_OK;
  if (!parent || !cand_tokens || !target_logits || !accept_len || !out_tokens) return SV_EINVAL;
  if (max_depth > 0 && !path_nodes) return SV_EINVAL;
  if (stoch && (!temperature_ok(temperature) || !uniforms)) return SV_EINVAL;
  const Layout lay = tree_layout(B, n_nodes, V, dtype);
  if (!ws_ok(workspace, workspace_bytes, lay.total)) return SV_EWORKSPACE;

  TreeParams P{};
  P.logits = static_cast<const char*>(target_logits);
  P.parent = parent;
  P.parent_stride = parent_batch_stride;
  P.cand = cand_tokens;
  P.uniforms = uniforms;
  P.accept_len = accept_len;
  P.path_nodes = path_nodes;
  P.out_tokens = out_tokens;
  P.err_flags = err_flags;
  char* ws = static_cast<char*>(workspace);
  P.parts = reinterpret_cast<Partial*>(ws + lay.off[0]);
  P.node_y = reinterpret_cast<int32_t*>(ws + lay.off[1]);
  P.row_cnt = reinterpret_cast<unsigned*>(ws + lay.off[2]);
  P.tree_cnt = reinterpret_cast<unsigned*>(ws + lay.off[3]);
  P.B = B;
  P.N = n_nodes;
  P.V = V;
  P.max_depth = max_depth;
  P.C = (int)chunks_per_row(V, dtype);
  P.c0 = stoch ? temperature_c0(temperature) : 1.0f;
  P.nblocks = B * n_nodes * P.C;
  if (P.nblocks > MAX_BLOCKS) return SV_ELIMIT;
  const size_t smem = (size_t)n_nodes * 3 + 16;
  return dispatch<TreeLauncher>(dtype, stoch, P, smem, reinterpret_cast<hipStream_t>(stream));
}

size_t spec_row_stats_workspace(int64_t rows, int64_t V, sv_dtype dtype) {
  if (rows < 0 || V < 1 || !dtype_ok(dtype)) return 0;
  return rowstats_layout(rows, V, dtype).total;
}

sv_status spec_row_stats(sv_dtype dtype, float temperature, int64_t rows, int64_t V, const void* x,
                         float* row_max, float* row_lse, int32_t* row_argmax, int32_t* err_flags,
                         void* workspace, size_t workspace_bytes, sv_stream_t stream) {
  if (!dtype_ok(dtype)) return SV_EDTYPE;
  if (rows < 0 || V < 1 || !temperature_ok(temperature)) return SV_EINVAL;
  if (V > 0x7fffffffLL - 16 || chunks_per_row(V, dtype) > MAX_CHUNKS) return SV_ELIMIT;
  if (rows == 0) return SV_OK;
  if (!x) return SV_EINVAL;
  const Layout lay = rowstats_layout(rows, V, dtype);
  if (!ws_ok(workspace, workspace_bytes, lay.total)) return SV_EWORKSPACE;
  RowStatsParams P{};
  P.x = static_cast<const char*>(x);
  P.row_max = row_max;
  P.row_lse = row_lse;
  P.row_argmax = row_argmax;
  P.err_flags = err_flags;
  char* ws = static_cast<char*>(workspace);
  P.parts = reinterpret_cast<Partial*>(ws + lay.off[0]);
  P.row_cnt = reinterpret_cast<unsigned*>(ws + lay.off[1]);
  P.rows = rows;
  P.V = V;
  P.C = (int)chunks_per_row(V, dtype);
  P.c0 = temperature_c0(temperature);
  P.nblocks = rows * P.C;
  if (P.nblocks > MAX_BLOCKS) return SV_ELIMIT;
  return dispatch<RowStatsLauncher>(dtype, false, P, reinterpret_cast<hipStream_t>(stream));
}

sv_status spec_workspace_clear(void* workspace, size_t bytes, sv_stream_t stream) {
  if (bytes == 0) return SV_OK;
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 15u) != 0) return SV_EINVAL;
  size_t blocks = (bytes / 16 + BLOCK - 1) / BLOCK;
  if (blocks < 1) blocks = 1;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(clear_kernel, dim3((unsigned)blocks), dim3(BLOCK), 0,
                     reinterpret_cast<hipStream_t>(stream), static_cast<unsigned char*>(workspace), bytes);
  return launch_status();
}

}  // extern "C"

// libspecverify: speculative-decoding verification kernels for gfx950 and the C ABI
// declared in include/specverify.h.
//
// One launch per call. The grid's workgroups are, in dispatch order:
//  * streaming workgroups, one per (row, 16 KiB chunk), sequence by sequence:
//    each streams its chunk once (max / argmax / exp-sum), writes its partial as a
//    tagged record and is done. The workgroup of a row's last chunk combines the
//    row (max, normaliser, argmax) and, for the bonus row k in stochastic mode,
//    draws the extra token; the one finishing a sequence's last row runs the
//    acceptance test for all k positions at once (one lane per position), the
//    first-reject scan, and emits the tokens;
//  * in stochastic mode, one residual workgroup per (sequence, chunk): for
//    sequences that rejected at L < k it sums max(0, p_t,L - p_d,L) over its chunk;
//    the sequence's last residual workgroup picks the chunk holding u*S and runs the
//    LDS block scan there (inverse CDF) for the correction token;
// Trees and row statistics use the same streaming workgroups; the workgroup
// finishing a tree's last node runs the accepted-path search in LDS.
//
// Workgroups hand results to each other through tagged records in the workspace.
// Every call carries a fresh tag; a record's single reader polls until it sees
// the call's tag and then clears the record, so a workspace is all zeros again
// after every call that completed without an internal error.
//
// Sources: "Accelerating Sonar through speculation" (sections "Spekulatives
// Decoding", "Ziel-Entwurf", "MTP", "EAGLE"); "Speculative-Decoding, LLM推理的加速 /
// Medusa 方法阅读" (section 三). The acceptance rule is that of the Leviathan et al.
// method the Sonar page cites: accept x_i iff u_i < p_t,i(x_i) / p_d,i(x_i).
#include "../../include/specverify.h"
#include "sv_device.hpp"

#include <hip/hip_runtime.h>
#include <atomic>
#include <cmath>
#include <cstdint>

using namespace sv;

namespace {

constexpr double LN2 = 0.69314718055994530941723212145818;
constexpr double LOG2E = 1.4426950408889634073599246810019;

// Record slots (8-byte tagged words) per record type.
constexpr int PART_WORDS = RecWords<Partial>::N;   // 4
constexpr int ROW_WORDS = RecWords<RowStat>::N;    // 8

struct Decision {   // what the residual workgroups of a sequence need
  int L;            // first rejected position
  int pending;      // 1 if the correction token is drawn from the residual
  float Mt, Md;     // row maxima of t_L, d_L
  double Zt, Zd;    // normalisers of t_L, d_L (relative to M*c0)
};
constexpr int DEC_WORDS = RecWords<Decision>::N;    // 8

struct ResPart {
  double s;
};
constexpr int RES_WORDS = RecWords<ResPart>::N;     // 2

// ------------------------------------------------------------------ row finalisation
// Wave 0 waits for the C tagged partials of one row, clears them and combines them; then,
// optionally, the whole workgroup draws a token from softmax(row / T) with
// uniform u. Result valid in all threads; ok = -1 if a wait timed out.
template <int DT, bool SUM>
__device__ __forceinline__ RowStat finalize_row(const char* row, int64_t V, const uint64_t* parts, int C,
                                                float c0, uint32_t tag, bool draw, float u,
                                                BlockScratch& sm, RowStat& sh) {
  if (wave_id() == 0) {
    int c_lo, c_hi;
    lane_chunk_range(C, c_lo, c_hi);
    Partial pl[CHUNKS_PER_LANE];
    bool ok = true;
#pragma unroll
    for (int q = 0; q < CHUNKS_PER_LANE; ++q) {
      pl[q].m = -INFINITY;
      pl[q].idx = INT_SENTINEL;
      pl[q].s = 0.0;
      if (c_lo + q < c_hi) ok = get_rec(parts + (int64_t)(c_lo + q) * PART_WORDS, pl[q], tag) && ok;
    }
#pragma unroll
    for (int q = 0; q < CHUNKS_PER_LANE; ++q)
      if (c_lo + q < c_hi) clear_rec<Partial>(const_cast<uint64_t*>(parts) + (int64_t)(c_lo + q) * PART_WORDS);
    const bool all_ok = __ballot(!ok) == 0ull;
    float M = -INFINITY;
    int arg = INT_SENTINEL;
#pragma unroll
    for (int q = 0; q < CHUNKS_PER_LANE; ++q) argmax_combine(M, arg, pl[q].m, pl[q].idx);
    wave_argmax(M, arg);
    double Z = 0.0;
    double wl[CHUNKS_PER_LANE];
    const double Mc0 = (double)M * (double)c0;
    if constexpr (SUM) {
      double local = 0.0;
#pragma unroll
      for (int q = 0; q < CHUNKS_PER_LANE; ++q) {
        wl[q] = (pl[q].m == -INFINITY) ? 0.0 : pl[q].s * exp2((double)chunk_mc0(pl[q].m, c0) - Mc0);
        local += wl[q];
      }
      Z = wave_sum(local);
    }
    bool rowok = SUM ? ((M > -INFINITY) && __builtin_isfinite(Z) && Z > 0.0) : (M > -INFINITY);
    if (lane_id() == 0) {
      sh.M = M;
      sh.argmax = (M > -INFINITY && arg != INT_SENTINEL) ? arg : -1;
      sh.Z = Z;
      sh.ok = all_ok ? (rowok ? 1 : 0) : -1;
      sh.y = SUM ? -1 : sh.argmax;
    }
    if constexpr (SUM) {
      if (draw && all_ok && rowok) {
        const ChunkPick pk = pick_chunk(C, (double)u, wl);
        // the chosen chunk's max, from the lane holding it
        float mine = 0.0f;
#pragma unroll
        for (int q = 0; q < CHUNKS_PER_LANE; ++q)
          if (c_lo + q == pk.c) mine = pl[q].m;
        const int per = (C + 63) / 64;
        const float mstar = __shfl(mine, (pk.c >= 0 ? pk.c : 0) / per);
        if (lane_id() == 0) {
          sm.result = pk.c;
          const float mc0 = chunk_mc0(mstar, c0);
          sm.f[0] = mc0;
          // threshold in the chunk's own units (weights relative to its mc0)
          sm.theta = (pk.c < 0) ? 0.0 : (pk.fallback ? INFINITY : (pk.theta - pk.before) * exp2(Mc0 - (double)mc0));
        }
      } else if (lane_id() == 0) {
        sm.result = -1;
      }
    }
  }
  __syncthreads();
  RowStat st = sh;
  if constexpr (SUM) {
    if (draw && st.ok == 1) {
      const int cstar = (int)sm.result;
      const double th = sm.theta;
      const float mc0 = sm.f[0];
      __syncthreads();
      if (cstar >= 0) {
        SoftmaxWeights<DT> pol{row, V, row_aligned(row), c0, mc0};
        st.y = (int)chunk_invcdf<DT>(pol, cstar, th, sm);
      } else {
        st.y = -1;
      }
    }
  }
  __syncthreads();
  return st;
}

// Streams one chunk and writes its partial record (thread 0).
template <int DT, bool SUM, bool ARG>
__device__ __forceinline__ void stream_chunk(const char* row, int64_t V, int64_t c, float c0,
                                             uint64_t* part_slot, uint32_t tag, BlockScratch& sm) {
  const int64_t unit0 = c * UNITS_PER_CHUNK;
  const bool aligned = row_aligned(row);
  ChunkRaw raw;
  load_chunk_raw<DT>(row, V, unit0, aligned, raw);
  const Partial p = reduce_chunk<DT, SUM, ARG>(row, V, unit0, aligned, raw, c0, sm);
  if (threadIdx.x == 0) put_rec(part_slot, p, tag);
}

// Inverse-CDF draw from softmax(row / T) that streams the whole row itself (every
// chunk's weight sum relative to the row max, then the scan in the chosen chunk).
// Used only when no partials are at hand (the residual of two rows that are equal
// up to rounding). LDS: up to MAX_CHUNKS doubles in `wsum`.
template <int DT>
__device__ __forceinline__ int draw_row_streamed(const char* row, int64_t V, int C, float M, float c0, float u,
                                                 double* wsum, BlockScratch& sm) {
  SoftmaxWeights<DT> pol{row, V, row_aligned(row), c0, M * c0};
  for (int c = 0; c < C; ++c) {
    const double w = chunk_weight_sum<DT>(pol, c, sm);
    if (threadIdx.x == 0) wsum[c] = w;
  }
  __syncthreads();
  if (wave_id() == 0) {
    int c_lo, c_hi;
    lane_chunk_range(C, c_lo, c_hi);
    double wl[CHUNKS_PER_LANE];
#pragma unroll
    for (int q = 0; q < CHUNKS_PER_LANE; ++q) wl[q] = (c_lo + q < c_hi) ? wsum[c_lo + q] : 0.0;
    const ChunkPick pk = pick_chunk(C, (double)u, wl);
    if (lane_id() == 0) {
      sm.result = pk.c;
      sm.theta = pk.fallback ? INFINITY : pk.theta - pk.before;
    }
  }
  __syncthreads();
  const int cstar = (int)sm.result;
  const double th = sm.theta;
  __syncthreads();
  return cstar >= 0 ? (int)chunk_invcdf<DT>(pol, cstar, th, sm) : -1;
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
  uint64_t* parts;      // [B][R][C] Partial records
  uint64_t* rows;       // [B][R]    RowStat records
  uint64_t* dec;        // [B]       Decision records
  uint64_t* res;        // [B][C]    ResPart records
  int64_t B, k, V;
  int R, C;
  float c0;
  uint32_t tag;         // this call's record tag
  int64_t n_stream;     // streaming workgroups (B * R * C)
  int64_t n_resid;      // residual workgroups (B * C in stochastic mode, else 0)
};

// Row slots per sequence. Stochastic: slot 0 = target row k (bonus), then the
// pairs (t_0, d_0), (t_1, d_1), ...; greedy: slot i = target row i.
template <int DT, bool STOCH>
__device__ __forceinline__ const char* slot_ptr(const LinearParams& P, int64_t b, int slot) {
  constexpr int E = DTraits<DT>::E;
  if (!STOCH) return P.target + ((b * (P.k + 1) + slot) * P.V) * E;
  if (slot == 0) return P.target + ((b * (P.k + 1) + P.k) * P.V) * E;
  const int64_t i = (slot - 1) >> 1;
  if (((slot - 1) & 1) != 0) return P.draft + ((b * P.k + i) * P.V) * E;
  return P.target + ((b * (P.k + 1) + i) * P.V) * E;
}
__device__ __forceinline__ int tslot(bool stoch, int i, int64_t k) { return stoch ? (i == k ? 0 : 1 + 2 * i) : i; }
__device__ __forceinline__ int dslot(int i) { return 2 + 2 * i; }

// Acceptance test, first-reject scan and emission for sequence b (wave 0).
template <int DT, bool STOCH>
__device__ __forceinline__ void linear_decide(const LinearParams& P, int64_t b, uint32_t tag) {
  const int lane = lane_id();
  const int64_t k = P.k, V = P.V;
  const uint64_t* rows = P.rows + b * P.R * ROW_WORDS;
  const bool has = lane < k;
  const int x = has ? P.tokens[b * k + lane] : 0;
  const bool tok_bad = has && (x < 0 || x >= V);
  RowStat ts{}, ds{}, tk{};
  bool got = true;
  if (has) got = get_rec(rows + (int64_t)tslot(STOCH, lane, k) * ROW_WORDS, ts, tag) && got;
  if (STOCH && has) got = get_rec(rows + (int64_t)dslot(lane) * ROW_WORDS, ds, tag) && got;
  got = get_rec(rows + (int64_t)tslot(STOCH, (int)k, k) * ROW_WORDS, tk, tag) && got;
  // every row record of the sequence has been read: clear them
  for (int64_t r = lane; r < P.R; r += 64) clear_rec<RowStat>(const_cast<uint64_t*>(rows) + r * ROW_WORDS);
  const bool row_bad = (has && ts.ok != 1) || (STOCH && has && ds.ok != 1) || tk.ok != 1;
  const bool internal = (has && (ts.ok < 0 || (STOCH && ds.ok < 0))) || tk.ok < 0 || !got;
  int err = 0;
  if (__ballot(tok_bad)) err |= SV_ERR_TOKEN;
  if (__ballot(row_bad)) err |= SV_ERR_ROW;
  if (__ballot(internal)) err |= SV_ERR_INTERNAL;

  int32_t* out = P.out_tokens + b * (k + 1);
  Decision d{};
  if (err) {
    for (int64_t j = lane; j <= k; j += 64) out[j] = -1;
    if (STOCH && has) {
      if (P.p_target) P.p_target[b * k + lane] = NAN;
      if (P.p_draft) P.p_draft[b * k + lane] = NAN;
    }
    if (lane == 0) {
      P.accept_len[b] = -1;
      if (P.err_flags) P.err_flags[b] = err;
      d.L = -1;
      d.pending = 0;
      if (STOCH && P.n_resid > 0) put_rec(P.dec + b * DEC_WORDS, d, tag);
    }
    return;
  }
  bool acc = false;
  if constexpr (!STOCH) {
    acc = has && (x == ts.argmax);
  } else {
    if (has) {
      const double c0d = (double)P.c0;
      const float tx = load_elem<DT>(P.target + ((b * (k + 1) + lane) * V) * DTraits<DT>::E, x);
      const float dx = load_elem<DT>(P.draft + ((b * k + lane) * V) * DTraits<DT>::E, x);
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
    // the residual workgroups need t_L's and d_L's statistics
    d.L = L;
    d.pending = pending ? 1 : 0;
    d.Mt = __shfl(ts.M, L & 63);
    d.Md = __shfl(ds.M, L & 63);
    d.Zt = __shfl(ts.Z, L & 63);
    d.Zd = __shfl(ds.Z, L & 63);
  }
  for (int64_t j = lane; j <= k; j += 64) {
    if (j < L) out[j] = x;  // j == lane here: lane L-1 < 64 holds x_j
    else if (j == L) { if (!pending) out[j] = y; }
    else out[j] = -1;
  }
  if (lane == 0) {
    P.accept_len[b] = L;
    if (P.err_flags) P.err_flags[b] = 0;
    if (STOCH && P.n_resid > 0) put_rec(P.dec + b * DEC_WORDS, d, tag);
  }
}

template <int DT, bool STOCH>
__device__ __forceinline__ void linear_stream_block(const LinearParams& P, uint32_t item,
                                                    BlockScratch& sm, RowStat& rsh) {
  // item < 2^31: 32-bit index arithmetic (64-bit division would be a long scalar loop)
  const uint32_t C = (uint32_t)P.C, R = (uint32_t)P.R;
  const uint32_t rid32 = item / C;
  const int64_t c = item - rid32 * C;
  const int64_t b = rid32 / R;
  const int slot = (int)(rid32 - (uint32_t)b * R);
  const int64_t rid = rid32;
  const char* row = slot_ptr<DT, STOCH>(P, b, slot);
  const uint32_t tag = P.tag;
  stream_chunk<DT, STOCH, !STOCH>(row, P.V, c, P.c0, P.parts + (int64_t)item * PART_WORDS, tag, sm);
  if (c != P.C - 1) return;
  // last chunk of the row: combine it (and draw the bonus token from row k)
  const bool draw = STOCH && slot == 0;
  const float u = draw ? P.uniforms[b * (P.k + 1) + P.k] : 0.0f;
  const RowStat st = finalize_row<DT, STOCH>(row, P.V, P.parts + rid * P.C * PART_WORDS, P.C, P.c0, tag,
                                             draw, u, sm, rsh);
  if (threadIdx.x == 0) put_rec(P.rows + rid * ROW_WORDS, st, tag);
  if (slot != P.R - 1) return;
  // last row of the sequence: decide
  if (wave_id() == 0) linear_decide<DT, STOCH>(P, b, tag);
}

template <int DT>
__device__ __forceinline__ void linear_residual_block(const LinearParams& P, int64_t task, BlockScratch& sm,
                                                      double* wsum) {
  const uint32_t b32 = (uint32_t)task / (uint32_t)P.C;
  const int64_t b = b32;
  const int64_t c = (uint32_t)task - b32 * (uint32_t)P.C;
  const int64_t k = P.k;
  const uint32_t tag = P.tag;
  if (threadIdx.x == 0) {
    Decision d{};
    const bool ok = get_rec(P.dec + b * DEC_WORDS, d, tag);
    sm.i[0] = ok ? d.pending : 0;
    sm.i[1] = d.L;
    sm.i[2] = ok ? 1 : 0;
    sm.f[0] = d.Mt;
    sm.f[1] = d.Md;
    sm.d[0] = d.Zt;
    sm.d[1] = d.Zd;
  }
  __syncthreads();
  const int pending = sm.i[0];
  const int L = sm.i[1];
  const bool got_decision = sm.i[2] != 0;
  const float Mt = sm.f[0], Md = sm.f[1];
  const double Zt = sm.d[0], Zd = sm.d[1];
  __syncthreads();
  constexpr int E = DTraits<DT>::E;
  const char* trow = P.target + ((b * (k + 1) + (pending ? L : 0)) * P.V) * E;
  const char* drow = P.draft + ((b * k + (pending ? L : 0)) * P.V) * E;
  const float c0 = P.c0;
  const float mc0t = Mt * c0, mc0d = Md * c0;
  // 1 / sum_v exp2(x_v*c0 - fl32(M*c0)) from Z = sum_v exp2(x_v*c0 - M*c0)
  const float izt = pending ? (float)(1.0 / (Zt * exp2((double)Mt * (double)c0 - (double)mc0t))) : 0.0f;
  const float izd = pending ? (float)(1.0 / (Zd * exp2((double)Md * (double)c0 - (double)mc0d))) : 0.0f;
  ResidualWeights<DT> pol{trow, drow, P.V, row_aligned(trow), row_aligned(drow), c0, mc0t, mc0d, izt, izd};

  // every residual workgroup answers (0 when there is nothing to draw), so the
  // sequence's last one knows when the decision record may be cleared
  ResPart mine;
  mine.s = pending ? chunk_weight_sum<DT>(pol, c, sm) : 0.0;
  if (c != P.C - 1) {
    if (threadIdx.x == 0) put_rec(P.res + task * RES_WORDS, mine, tag);
    return;
  }

  // last chunk of the sequence's residual: pick the chunk holding u*S, scan it
  const float u = pending ? P.uniforms[b * (k + 1) + k] : 0.0f;
  if (wave_id() == 0) {
    int c_lo, c_hi;
    lane_chunk_range(P.C, c_lo, c_hi);
    double wl[CHUNKS_PER_LANE];
    bool ok = true;
#pragma unroll
    for (int q = 0; q < CHUNKS_PER_LANE; ++q) {
      wl[q] = 0.0;
      ResPart r{};
      const int cc = c_lo + q;
      if (cc >= c_hi) continue;
      if (cc < P.C - 1) {
        const bool g = get_rec(P.res + (b * P.C + cc) * RES_WORDS, r, tag);
        ok = ok && g;
        wl[q] = g ? r.s : 0.0;
        clear_rec<ResPart>(P.res + (b * P.C + cc) * RES_WORDS);
      } else {
        wl[q] = mine.s;
      }
    }
    if (lane_id() == 0) clear_rec<Decision>(P.dec + b * DEC_WORDS);
    const bool all_ok = __ballot(!ok) == 0ull;
    const ChunkPick pk = pick_chunk(P.C, (double)u, wl);
    if (lane_id() == 0) {
      sm.result = (all_ok && got_decision) ? pk.c : -2;
      sm.theta = pk.fallback ? INFINITY : pk.theta - pk.before;
    }
  }
  __syncthreads();
  const int cstar = (int)sm.result;
  const double th = sm.theta;
  __syncthreads();
  if (!pending) {
    if (!got_decision && threadIdx.x == 0) {   // the decision never arrived: flag the sequence
      P.accept_len[b] = -1;
      if (P.err_flags) P.err_flags[b] = SV_ERR_INTERNAL;
    }
    return;
  }
  int y;
  if (cstar >= 0) {
    y = (int)chunk_invcdf<DT>(pol, cstar, th, sm);
  } else if (cstar == -1) {
    // no residual mass (equal rows up to rounding): draw from p_t,L instead
    y = draw_row_streamed<DT>(trow, P.V, P.C, Mt, c0, u, wsum, sm);
  } else {
    y = -1;
    if (threadIdx.x == 0) {
      P.accept_len[b] = -1;
      if (P.err_flags) P.err_flags[b] = SV_ERR_INTERNAL;
    }
  }
  if (threadIdx.x == 0) P.out_tokens[b * (k + 1) + L] = y;
}

template <int DT, bool STOCH>
__global__ __launch_bounds__(BLOCK) void linear_kernel(LinearParams P) {
  __shared__ BlockScratch sm;
  __shared__ RowStat rsh;
  const int64_t hw = blockIdx.x;
  if (hw < P.n_stream) {
    linear_stream_block<DT, STOCH>(P, (uint32_t)xcd_logical_block(hw, P.n_stream), sm, rsh);
  } else {
    if constexpr (STOCH) {
      __shared__ double wsum[MAX_CHUNKS];
      linear_residual_block<DT>(P, hw - P.n_stream, sm, wsum);
    }
  }
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
  uint64_t* parts;      // [B][N][C] Partial records
  uint64_t* node_y;     // [B][N]    token chosen at each node (-1: unusable row, -2: timeout)
  int64_t B, N, V, max_depth;
  int C;
  float c0;
  uint32_t tag;
  int64_t n_stream;
};

// Accepted-path search for tree b (whole workgroup). LDS: parent (int16) and
// match flag (uint8) of every node.
__device__ __forceinline__ void tree_walk(const TreeParams& P, int64_t b, uint32_t tag, unsigned char* smem,
                                          BlockScratch& sm) {
  const int64_t N = P.N;
  int16_t* par_s = reinterpret_cast<int16_t*>(smem);
  unsigned char* match_s = smem + 2 * N;
  const int32_t* par = P.parent + b * P.parent_stride;
  const int32_t* cand = P.cand + b * N;
  const uint64_t* ny = P.node_y + b * N;
  int err = 0;
  for (int64_t i = threadIdx.x; i < N; i += BLOCK) {
    int32_t y;
    if (!get_rec(ny + i, y, tag)) y = -2;
    if (y == -1) err |= SV_ERR_ROW;
    if (y == -2) err |= SV_ERR_INTERNAL;
    const int p = par[i];
    const bool bad = (i == 0) ? (p != -1) : (p < 0 || p >= i);
    par_s[i] = (int16_t)(bad ? 0 : p);
    if (bad) err |= SV_ERR_TREE;
    unsigned char m = 0;
    if (i > 0) {
      const int ci = cand[i];
      if (ci < 0 || ci >= P.V) err |= SV_ERR_TOKEN;
      if (!bad) {
        int32_t yp;
        if (!get_rec(ny + p, yp, tag)) { yp = -2; err |= SV_ERR_INTERNAL; }
        m = (ci == yp) ? 1 : 0;
      }
    }
    match_s[i] = m;
  }
  // OR of the error bits over the workgroup (each bit separately)
  int all_err = 0;
  for (int bit = 1; bit <= SV_ERR_INTERNAL; bit <<= 1)
    if (__syncthreads_or(err & bit)) all_err |= bit;

  // Depth check and path search (bad parents were replaced by the root above, so
  // every chain ends; the depth bound is checked whatever other error was found).
  unsigned long long best_key = 0ull;
  int too_deep = 0;
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
  int32_t* path = P.path_nodes + b * P.max_depth;
  int32_t* out = P.out_tokens + b * (P.max_depth + 1);
  if (all_err) {
    for (int64_t j = threadIdx.x; j < P.max_depth; j += BLOCK) path[j] = -1;
    for (int64_t j = threadIdx.x; j <= P.max_depth; j += BLOCK) out[j] = -1;
    if (threadIdx.x == 0) {
      P.accept_len[b] = -1;
      if (P.err_flags) P.err_flags[b] = all_err;
    }
    __syncthreads();
    for (int64_t i = threadIdx.x; i < N; i += BLOCK) clear_rec<int32_t>(const_cast<uint64_t*>(ny) + i);
    return;
  }
  // workgroup max of the (depth, -index) key
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
    int32_t yb;
    out[L] = get_rec(ny + best, yb, tag) ? yb : -1;
    P.accept_len[b] = L;
    if (P.err_flags) P.err_flags[b] = 0;
  }
  // every node record of the tree has been read: clear them
  __syncthreads();
  for (int64_t i = threadIdx.x; i < N; i += BLOCK) clear_rec<int32_t>(const_cast<uint64_t*>(ny) + i);
}

template <int DT, bool STOCH>
__global__ __launch_bounds__(BLOCK) void tree_kernel(TreeParams P) {
  __shared__ BlockScratch sm;
  __shared__ RowStat rsh;
  extern __shared__ unsigned char walk_smem[];
  constexpr int E = DTraits<DT>::E;
  const int64_t hw = blockIdx.x;
  if (hw < P.n_stream) {
    const uint32_t item = (uint32_t)xcd_logical_block(hw, P.n_stream);
    const uint32_t rid32 = item / (uint32_t)P.C;
    const int64_t rid = rid32;
    const int64_t c = item - rid32 * (uint32_t)P.C;
    const uint32_t b32 = rid32 / (uint32_t)P.N;
    const int64_t b = b32;
    const int64_t n = rid32 - b32 * (uint32_t)P.N;
    const char* row = P.logits + (rid * P.V) * E;
    const uint32_t tag = P.tag;
    stream_chunk<DT, STOCH, !STOCH>(row, P.V, c, P.c0, P.parts + (int64_t)item * PART_WORDS, tag, sm);
    if (c == P.C - 1) {
      const float u = STOCH ? P.uniforms[rid] : 0.0f;
      const RowStat st = finalize_row<DT, STOCH>(row, P.V, P.parts + rid * P.C * PART_WORDS, P.C, P.c0,
                                                 tag, STOCH, u, sm, rsh);
      if (threadIdx.x == 0) {
        const int32_t y = st.ok == 1 ? st.y : (st.ok < 0 ? -2 : -1);
        put_rec(P.node_y + rid, y, tag);
      }
      if (n == P.N - 1) tree_walk(P, b, tag, walk_smem, sm);
    }
  }
}

// ------------------------------------------------------------------ row statistics
struct RowStatsParams {
  const char* x;
  float* row_max;
  float* row_lse;
  int32_t* row_argmax;
  int32_t* err_flags;
  uint64_t* parts;
  int64_t rows, V;
  int C;
  float c0;
  uint32_t tag;
  int64_t n_stream;
};

template <int DT>
__global__ __launch_bounds__(BLOCK) void row_stats_kernel(RowStatsParams P) {
  __shared__ BlockScratch sm;
  __shared__ RowStat rsh;
  constexpr int E = DTraits<DT>::E;
  const int64_t hw = blockIdx.x;
  if (hw < P.n_stream) {
    const uint32_t item = (uint32_t)xcd_logical_block(hw, P.n_stream);
    const uint32_t r32 = item / (uint32_t)P.C;
    const int64_t r = r32, c = item - r32 * (uint32_t)P.C;
    const char* row = P.x + (r * P.V) * E;
    const uint32_t tag = P.tag;
    stream_chunk<DT, true, true>(row, P.V, c, P.c0, P.parts + (int64_t)item * PART_WORDS, tag, sm);
    if (c == P.C - 1) {
      // argmax needs the ARG partials, the normaliser the SUM partials: both are kept
      const RowStat st = finalize_row<DT, true>(row, P.V, P.parts + r * P.C * PART_WORDS, P.C, P.c0, tag,
                                                false, 0.0f, sm, rsh);
      if (threadIdx.x == 0) {
        const bool ok = st.ok == 1 && st.argmax >= 0;
        if (P.row_max) P.row_max[r] = st.M;
        if (P.row_argmax) P.row_argmax[r] = st.argmax;
        if (P.row_lse) P.row_lse[r] = ok ? (float)((double)st.M * (double)P.c0 * LN2 + log(st.Z)) : NAN;
        if (P.err_flags) P.err_flags[r] = ok ? 0 : (st.ok < 0 ? SV_ERR_INTERNAL : SV_ERR_ROW);
      }
    }
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

// Record regions back to back, each 256-byte aligned.
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
  return make_layout({(size_t)(B * R * C) * PART_WORDS * 8, (size_t)(B * R) * ROW_WORDS * 8,
                      (size_t)B * DEC_WORDS * 8, (size_t)(B * C) * RES_WORDS * 8});
}

Layout tree_layout(int64_t B, int64_t N, int64_t V, sv_dtype dt) {
  const int64_t C = chunks_per_row(V, dt);
  return make_layout({(size_t)(B * N * C) * PART_WORDS * 8, (size_t)(B * N) * 8});
}

Layout rowstats_layout(int64_t rows, int64_t V, sv_dtype dt) {
  const int64_t C = chunks_per_row(V, dt);
  return make_layout({(size_t)(rows * C) * PART_WORDS * 8});
}

bool temperature_ok(float T) { return std::isfinite(T) && T > 0.0f; }

float temperature_c0(float T) { return (float)(LOG2E / (double)T); }

sv_status launch_status() {
  return hipGetLastError() == hipSuccess ? SV_OK : SV_EHIP;
}

// A fresh record tag per call: odd (never the cleared value 0), distinct from the
// tags of the last 2^31 calls of this process.
std::atomic<uint32_t> g_tag{0};
uint32_t next_tag() { return (g_tag.fetch_add(1, std::memory_order_relaxed) << 1) | 1u; }

template <template <int, bool> class Launcher, class... Args>
sv_status dispatch(sv_dtype dt, bool stoch, Args&&... args) {
  switch (dt) {
    case SV_F32: return stoch ? Launcher<DT_F32, true>::run(args...) : Launcher<DT_F32, false>::run(args...);
    case SV_BF16: return stoch ? Launcher<DT_BF16, true>::run(args...) : Launcher<DT_BF16, false>::run(args...);
    case SV_F16: return stoch ? Launcher<DT_F16, true>::run(args...) : Launcher<DT_F16, false>::run(args...);
  }
  return SV_EDTYPE;
}

template <int DT, bool STOCH>
struct LinearLauncher {
  static sv_status run(const LinearParams& P, hipStream_t s) {
    const int64_t G = P.n_stream + P.n_resid;
    hipLaunchKernelGGL((linear_kernel<DT, STOCH>), dim3((unsigned)G), dim3(BLOCK), 0, s, P);
    return launch_status();
  }
};

template <int DT, bool STOCH>
struct TreeLauncher {
  static sv_status run(const TreeParams& P, size_t smem, hipStream_t s) {
    hipLaunchKernelGGL((tree_kernel<DT, STOCH>), dim3((unsigned)P.n_stream), dim3(BLOCK), smem, s, P);
    return launch_status();
  }
};

template <int DT, bool UNUSED>
struct RowStatsLauncher {
  static sv_status run(const RowStatsParams& P, hipStream_t s) {
    hipLaunchKernelGGL((row_stats_kernel<DT>), dim3((unsigned)P.n_stream), dim3(BLOCK), 0, s, P);
    return launch_status();
  }
};

bool ws_ok(const void* ws, size_t have, size_t need) {
  return ws != nullptr && (reinterpret_cast<uintptr_t>(ws) & 255u) == 0 && have >= need;
}

constexpr int64_t MAX_BLOCKS = 0x7fffffff - 1;

sv_status linear_entry(sv_mode mode, float temperature, int64_t B, int64_t k, int64_t V,
                       sv_dtype dtype, const void* target_logits, const void* draft_logits,
                       const int32_t* draft_tokens, const float* uniforms, int32_t* accept_len,
                       int32_t* out_tokens, float* p_target, float* p_draft, int32_t* err_flags,
                       void* workspace, size_t workspace_bytes, sv_stream_t stream) {
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
  P.parts = reinterpret_cast<uint64_t*>(ws + lay.off[0]);
  P.rows = reinterpret_cast<uint64_t*>(ws + lay.off[1]);
  P.dec = reinterpret_cast<uint64_t*>(ws + lay.off[2]);
  P.res = reinterpret_cast<uint64_t*>(ws + lay.off[3]);
  P.B = B;
  P.k = k;
  P.V = V;
  P.R = (int)(stoch ? 2 * k + 1 : k + 1);
  P.C = (int)chunks_per_row(V, dtype);
  P.c0 = stoch ? temperature_c0(temperature) : 1.0f;
  P.n_stream = B * P.R * P.C;
  P.n_resid = (stoch && k > 0) ? B * P.C : 0;
  if (P.n_stream + P.n_resid > MAX_BLOCKS) return SV_ELIMIT;
  P.tag = next_tag();
  return dispatch<LinearLauncher>(dtype, stoch, P, reinterpret_cast<hipStream_t>(stream));
}

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

sv_status spec_verify_linear(sv_mode mode, float temperature, int64_t B, int64_t k, int64_t V,
                             sv_dtype dtype, const void* target_logits, const void* draft_logits,
                             const int32_t* draft_tokens, const float* uniforms, int32_t* accept_len,
                             int32_t* out_tokens, float* p_target, float* p_draft,
                             int32_t* err_flags, void* workspace, size_t workspace_bytes,
                             sv_stream_t stream) {
  return linear_entry(mode, temperature, B, k, V, dtype, target_logits, draft_logits,
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
  P.parts = reinterpret_cast<uint64_t*>(ws + lay.off[0]);
  P.node_y = reinterpret_cast<uint64_t*>(ws + lay.off[1]);
  P.B = B;
  P.N = n_nodes;
  P.V = V;
  P.max_depth = max_depth;
  P.C = (int)chunks_per_row(V, dtype);
  P.c0 = stoch ? temperature_c0(temperature) : 1.0f;
  P.n_stream = B * n_nodes * P.C;
  if (P.n_stream > MAX_BLOCKS) return SV_ELIMIT;
  P.tag = next_tag();
  // LDS of the path search: parent (2 B) + match flag (1 B) per node
  const size_t smem = (size_t)((3 * n_nodes + 15) & ~(int64_t)15);
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
  P.parts = reinterpret_cast<uint64_t*>(ws + lay.off[0]);
  P.rows = rows;
  P.V = V;
  P.C = (int)chunks_per_row(V, dtype);
  P.c0 = temperature_c0(temperature);
  P.n_stream = rows * P.C;
  if (P.n_stream > MAX_BLOCKS) return SV_ELIMIT;
  P.tag = next_tag();
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

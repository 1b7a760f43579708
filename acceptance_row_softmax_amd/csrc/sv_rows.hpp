// Row combine and draws shared by the streaming kernels of libspecverify: the
// chunk partials of a row read back and combined (max, argmax, normaliser), and
// inverse-CDF draws from softmax(row / T).
#pragma once

#include "sv_device.hpp"

namespace sv {

constexpr int PART_WORDS = RecWords<Partial>::N;   // 6
// Every atomic counter sits on its own 128-byte line: counters that share a line
// serialise each other's atomics.
constexpr int64_t CSTRIDE = 32;                     // in 32-bit words
constexpr int64_t SSTRIDE = 16;                     // in 64-bit words
constexpr int ROW_WORDS = RecWords<RowStat>::N;    // 8

template <class T>
__device__ __forceinline__ T bcast(T v) { return __shfl(v, 0); }

// ------------------------------------------------------------------ row combine
// Chunk partials of one row, lane-strided (lane l holds chunks l + 64 t).
struct RowParts {
  float m[MAX_ROUNDS];
  int idx[MAX_ROUNDS];
  double s[MAX_ROUNDS];
  bool got;    // every partial arrived (same in every lane)
  bool xin;    // some chunk holds the draft token
  float xv;    // its logit
};

// Reads the C partials of a row (clear_parts zeroes them afterwards).
__device__ __forceinline__ RowParts read_parts(uint64_t* parts, int C, uint32_t tag) {
  const int lane = lane_id();
  RowParts rp;
  bool got = true;
  int xin = 0;
  float xv = 0.0f;
#pragma unroll
  for (int t = 0; t < MAX_ROUNDS; ++t) {
    Partial p;
    p.m = -INFINITY;
    p.idx = INT_SENTINEL;
    p.s = 0.0;
    p.xin = 0;
    p.xv = 0.0f;
    const int c = t * WAVE + lane;
    if (c < C) got = get_rec(parts + (int64_t)c * PART_WORDS, p, tag) && got;
    rp.m[t] = p.m;
    rp.idx[t] = p.idx;
    rp.s[t] = p.s;
    if (p.xin) { xin = 1; xv = p.xv; }
  }
  const unsigned long long xm = __ballot(xin != 0);
  rp.xin = xm != 0ull;
  rp.xv = __shfl(xv, xm ? first_lane(xm) : 0);
  rp.got = __ballot(!got) == 0ull;
  return rp;
}

// Zeroes the C partials of a row, and its arrival counter, for the next call: by
// the wave that read them, once it has nothing left to wait for (a wait for a load
// or a returning atomic also waits for every store the wave issued before it, and
// a device-scope store takes about a microsecond to complete).
template <class T>
__device__ __forceinline__ void clear_parts(uint64_t* parts, int C, uint32_t* cnt) {
  const int lane = lane_id();
  for (int c = lane; c < C; c += WAVE) clear_rec<T>(parts + (int64_t)c * PART_WORDS);
  if (lane == 0) counter_reset(cnt);
}

struct RowSums {
  float M;
  int argmax;   // -1 if no entry exceeds -inf
  double Z;     // relative to 2^(M*c0); 0 if not computed
};

// Combines the partials of a row of C chunks; wl receives each chunk's weight
// relative to 2^(M*c0). Rounds past C (lane-strided chunk groups no lane of which
// holds a chunk) are skipped with a wave-uniform branch. ARG = false: the max only
// (argmax -1).
template <bool SUM, bool ARG = true>
__device__ __forceinline__ RowSums row_sums(const RowParts& rp, float c0, double (&wl)[MAX_ROUNDS],
                                            int C = MAX_CHUNKS) {
  float M = -INFINITY;
  int arg = INT_SENTINEL;
#pragma unroll
  for (int t = 0; t < MAX_ROUNDS; ++t) {
    if (t * WAVE >= C) break;
    if constexpr (ARG) argmax_combine(M, arg, rp.m[t], rp.idx[t]);
    else M = fmaxf(M, rp.m[t]);
  }
  if constexpr (ARG) wave_argmax(M, arg);
  else M = wave_max(M);
  RowSums r;
  r.M = M;
  r.argmax = (ARG && M > -INFINITY && arg != INT_SENTINEL) ? arg : -1;
  r.Z = 0.0;
  if constexpr (SUM) {
    const double Mc0 = (double)M * (double)c0;
    double local = 0.0;
#pragma unroll
    for (int t = 0; t < MAX_ROUNDS; ++t) {
      wl[t] = 0.0;
      if (t * WAVE >= C) continue;
      if (rp.m[t] != -INFINITY) wl[t] = rp.s[t] * pow2_neg((double)chunk_mc0(rp.m[t], c0) - Mc0);
      local += wl[t];
    }
    r.Z = wave_sum(local);
  }
  return r;
}

// Inverse-CDF draw from softmax(row / T) with uniform u, given the row's chunk
// partials: pick the chunk, then scan inside it. -1 if the row has no weight.
template <int DT>
__device__ __forceinline__ int softmax_draw(const char* row, int64_t V, int C, float c0, float u,
                                            const RowParts& rp, const RowSums& rs, const double (&wl)[MAX_ROUNDS]) {
  const ChunkPick pk = pick_chunk(C, (double)u, wl);
  if (pk.c < 0) return -1;
  const int tc = pk.c / WAVE, lc = pk.c % WAVE;
  float mm = rp.m[0];
#pragma unroll
  for (int t = 1; t < MAX_ROUNDS; ++t) if (t == tc) mm = rp.m[t];
  const float mstar = __shfl(mm, lc);
  const float mc0 = chunk_mc0(mstar, c0);
  // threshold in the chunk's own units (weights relative to its mc0)
  const double th = pk.fallback ? (double)INFINITY
                                : (pk.theta - pk.before) * exp2((double)rs.M * (double)c0 - (double)mc0);
  Raw r;
  const Chunk k = load_chunk<DT>(row, V, pk.c, r);
  SoftmaxW sw;
  sw.c0 = c0;
  sw.mc0 = mc0;
  const int64_t y = chunk_invcdf<DT, false>(k, r, r, th, sw);
  return (int)y;
}

}  // namespace sv

// Device building blocks for libspecverify (gfx950, wave64).
//
// Data path: logits rows are streamed in 16-byte units (8 bf16/fp16 or 4 fp32
// values per lane per load). A "chunk" is BLOCK * UNROLL units (16 KiB) handled
// by one 256-thread workgroup; thread t owns units unit0 + j*BLOCK + t, j < UNROLL,
// so every load instruction of a wave reads 1 KiB of contiguous memory.
//
// Arithmetic (all of it the row softmax at temperature T, computed in base 2):
//   c0 = log2(e)/T (fp32).  Chunk max m_c; mc0 = fl32(m_c * c0).
//   element weight  w = exp2(fma(x, c0, -mc0))            (fp32, v_exp_f32)
//   unit sum        pairwise fp32 sum of the unit's W weights
//   chunk sum s_c   per-thread fp64 sum of its unit sums, then a fixed-order
//                   fp64 butterfly across the wave and the 4 waves.
//   row normaliser  Z = sum_c s_c * 2^(mc0_c - M*c0)       (fp64, M = row max)
// Every reduction has a fixed order, so results are bit-identical run to run, and
// any code that recomputes a weight uses the same expression as the pass that
// summed it (the inverse-CDF scan relies on that).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

constexpr int BLOCK = 256;
constexpr int NWAVES = BLOCK / 64;
constexpr int UNROLL = 4;
constexpr int UNITS_PER_CHUNK = BLOCK * UNROLL;
constexpr int INT_SENTINEL = 0x7fffffff;

enum { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2 };

template <int DT> struct DTraits;
template <> struct DTraits<DT_F32>  { static constexpr int W = 4; static constexpr int E = 4; };
template <> struct DTraits<DT_BF16> { static constexpr int W = 8; static constexpr int E = 2; };
template <> struct DTraits<DT_F16>  { static constexpr int W = 8; static constexpr int E = 2; };

// Per-(row, chunk) partial statistics.
struct Partial {
  float m;     // chunk max (-inf if no entry above -inf)
  int idx;     // lowest row index holding m (INT_SENTINEL if none)
  double s;    // sum of exp2(fma(x, c0, -fl32(m*c0))) over the chunk (stochastic only)
};

// Per-row statistics written by the last chunk block of the row.
struct RowStat {
  double Z;    // sum_v 2^(x_v*c0 - M*c0), M*c0 in fp64
  float M;     // row max
  int argmax;  // lowest index of M, -1 if none
  int ok;      // 1 if the row is usable in the current mode
  int y;       // token chosen at this row (argmax, or an inverse-CDF draw), -1 if none
  int pad0, pad1;
};

// ------------------------------------------------------------------ loads
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float f16_lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu)); }
__device__ __forceinline__ float f16_hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }

template <int DT>
__device__ __forceinline__ float load_elem(const char* row, int64_t i) {
  if constexpr (DT == DT_F32) {
    return reinterpret_cast<const float*>(row)[i];
  } else if constexpr (DT == DT_BF16) {
    return __uint_as_float((uint32_t) reinterpret_cast<const uint16_t*>(row)[i] << 16);
  } else {
    return (float)__builtin_bit_cast(_Float16, reinterpret_cast<const uint16_t*>(row)[i]);
  }
}

template <int DT>
__device__ __forceinline__ void decode_unit(const uint4 v, float (&x)[DTraits<DT>::W]) {
  if constexpr (DT == DT_F32) {
    x[0] = __uint_as_float(v.x); x[1] = __uint_as_float(v.y);
    x[2] = __uint_as_float(v.z); x[3] = __uint_as_float(v.w);
  } else if constexpr (DT == DT_BF16) {
    x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x); x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
    x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z); x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
  } else {
    x[0] = f16_lo(v.x); x[1] = f16_hi(v.x); x[2] = f16_lo(v.y); x[3] = f16_hi(v.y);
    x[4] = f16_lo(v.z); x[5] = f16_hi(v.z); x[6] = f16_lo(v.w); x[7] = f16_hi(v.w);
  }
}

// Load unit `unit` of a row: W consecutive elements starting at unit*W.
// Elements at or past V read as -inf (zero weight, never a maximum).
// Used for single units (the scan's final unit); chunks use load_chunk.
template <int DT>
__device__ __forceinline__ void load_unit(const char* row, int64_t V, int64_t unit, bool aligned,
                                 float (&x)[DTraits<DT>::W]) {
  constexpr int W = DTraits<DT>::W;
  constexpr int E = DTraits<DT>::E;
  const int64_t e0 = unit * W;
  if (aligned && e0 + W <= V) {
    const uint4 v = *reinterpret_cast<const uint4*>(row + e0 * E);
    decode_unit<DT>(v, x);
  } else {
#pragma unroll
    for (int e = 0; e < W; ++e) x[e] = (e0 + e < V) ? load_elem<DT>(row, e0 + e) : -INFINITY;
  }
}

// A chunk's raw 16-byte words for one thread (UNROLL units), as loaded.
struct ChunkRaw {
  uint4 v[UNROLL];
};

// Issue this thread's UNROLL vector loads of a chunk (units unit0 + j*BLOCK + tid)
// without waiting: addresses are clamped to units lying entirely inside the row.
// Rows that do not start on a 16-byte boundary load nothing here (decode_chunk
// reads them element by element).
template <int DT>
__device__ __forceinline__ void load_chunk_raw(const char* row, int64_t V, int64_t unit0, bool aligned,
                                               ChunkRaw& raw) {
  constexpr int W = DTraits<DT>::W;
  constexpr int E = DTraits<DT>::E;
  const int64_t nfull = V / W;                 // units lying entirely inside the row
  if (aligned && nfull > 0) {
#pragma unroll
    for (int j = 0; j < UNROLL; ++j) {
      const int64_t u = unit0 + j * BLOCK + threadIdx.x;
      const int64_t uc = (u < nfull) ? u : nfull - 1;
      raw.v[j] = *reinterpret_cast<const uint4*>(row + uc * (W * E));
    }
  }
}

// Decode a chunk loaded by load_chunk_raw; units (partly) past V and rows that do
// not start on a 16-byte boundary are read element by element here (entries past
// V read as -inf).
template <int DT>
__device__ __forceinline__ void decode_chunk(const char* row, int64_t V, int64_t unit0, bool aligned,
                                             const ChunkRaw& raw, float (&x)[UNROLL][DTraits<DT>::W]) {
  constexpr int W = DTraits<DT>::W;
  const int64_t nfull = V / W;
  if (aligned && nfull > 0) {
#pragma unroll
    for (int j = 0; j < UNROLL; ++j) {
      decode_unit<DT>(raw.v[j], x[j]);
      const int64_t u = unit0 + j * BLOCK + threadIdx.x;
      if (u >= nfull) {
#pragma unroll
        for (int e = 0; e < W; ++e) {
          const int64_t i = u * W + e;
          x[j][e] = (i < V) ? load_elem<DT>(row, i) : -INFINITY;
        }
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < UNROLL; ++j) {
      const int64_t u = unit0 + j * BLOCK + threadIdx.x;
#pragma unroll
      for (int e = 0; e < W; ++e) {
        const int64_t i = u * W + e;
        const float v = load_elem<DT>(row, i < V ? i : V - 1);
        x[j][e] = (i < V) ? v : -INFINITY;
      }
    }
  }
}

// Decode unit j of this thread from a raw chunk (see decode_chunk).
template <int DT>
__device__ __forceinline__ void decode_unit_at(const char* row, int64_t V, int64_t unit0, bool aligned,
                                               const ChunkRaw& raw, int j, float (&x)[DTraits<DT>::W]) {
  constexpr int W = DTraits<DT>::W;
  const int64_t nfull = V / W;
  const int64_t u = unit0 + j * BLOCK + threadIdx.x;
  if (aligned && nfull > 0) {
    decode_unit<DT>(raw.v[j], x);
    if (u >= nfull) {
#pragma unroll
      for (int e = 0; e < W; ++e) {
        const int64_t i = u * W + e;
        x[e] = (i < V) ? load_elem<DT>(row, i) : -INFINITY;
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < W; ++e) {
      const int64_t i = u * W + e;
      const float v = load_elem<DT>(row, i < V ? i : V - 1);
      x[e] = (i < V) ? v : -INFINITY;
    }
  }
}

// Load and decode this thread's UNROLL units of a chunk, every vector load issued
// before any result is used.
template <int DT>
__device__ __forceinline__ void load_chunk(const char* row, int64_t V, int64_t unit0, bool aligned,
                                           float (&x)[UNROLL][DTraits<DT>::W]) {
  ChunkRaw raw;
  load_chunk_raw<DT>(row, V, unit0, aligned, raw);
  decode_chunk<DT>(row, V, unit0, aligned, raw, x);
}

__device__ __forceinline__ bool row_aligned(const char* row) { return (reinterpret_cast<uintptr_t>(row) & 15u) == 0; }

// ------------------------------------------------------------------ arithmetic
__device__ __forceinline__ float softmax_weight(float x, float c0, float mc0) {
  return __builtin_amdgcn_exp2f(__builtin_fmaf(x, c0, -mc0));
}

template <int W>
__device__ __forceinline__ float pairwise_sum(const float (&w)[W]) {
  if constexpr (W == 8) {
    return ((w[0] + w[1]) + (w[2] + w[3])) + ((w[4] + w[5]) + (w[6] + w[7]));
  } else {
    return (w[0] + w[1]) + (w[2] + w[3]);
  }
}

// m*c0 in fp32 as used for the chunk's weights; 0 for an empty (-inf) chunk so
// that its -inf entries weigh exp2(-inf) = 0 instead of NaN.
__device__ __forceinline__ float chunk_mc0(float m, float c0) { return (m == -INFINITY) ? 0.0f : m * c0; }

// ------------------------------------------------------------------ reductions
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ int wave_max_int(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
// (value, index): larger value wins, lower index on equal values.
__device__ __forceinline__ void argmax_combine(float& m, int& i, float m2, int i2) {
  if (m2 > m || (m2 == m && i2 < i)) { m = m2; i = i2; }
}
__device__ __forceinline__ void wave_argmax(float& m, int& i) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o);
    const int i2 = __shfl_xor(i, o);
    argmax_combine(m, i, m2, i2);
  }
}

// Inclusive prefix sum over the 64 lanes (lane order), Hillis-Steele.
__device__ __forceinline__ double wave_incl_scan(double v) {
  const int lane = lane_id();
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

struct BlockScratch {
  double d[NWAVES];
  float f[NWAVES];
  int i[NWAVES];
  int flag;
  int64_t result;
  double theta;
};

__device__ __forceinline__ double block_sum(double v, BlockScratch& sm) {
  v = wave_sum(v);
  if (lane_id() == 0) sm.d[wave_id()] = v;
  __syncthreads();
  double r = sm.d[0];
#pragma unroll
  for (int w = 1; w < NWAVES; ++w) r += sm.d[w];
  __syncthreads();
  return r;
}
__device__ __forceinline__ float block_max(float v, BlockScratch& sm) {
  v = wave_max(v);
  if (lane_id() == 0) sm.f[wave_id()] = v;
  __syncthreads();
  float r = sm.f[0];
#pragma unroll
  for (int w = 1; w < NWAVES; ++w) r = fmaxf(r, sm.f[w]);
  __syncthreads();
  return r;
}
__device__ __forceinline__ int block_max_int(int v, BlockScratch& sm) {
  v = wave_max_int(v);
  if (lane_id() == 0) sm.i[wave_id()] = v;
  __syncthreads();
  int r = sm.i[0];
#pragma unroll
  for (int w = 1; w < NWAVES; ++w) r = max(r, sm.i[w]);
  __syncthreads();
  return r;
}
__device__ __forceinline__ int block_sum_int(int v, BlockScratch& sm) {
  v = wave_sum_int(v);
  if (lane_id() == 0) sm.i[wave_id()] = v;
  __syncthreads();
  int r = 0;
#pragma unroll
  for (int w = 0; w < NWAVES; ++w) r += sm.i[w];
  __syncthreads();
  return r;
}
__device__ __forceinline__ void block_argmax(float& m, int& idx, BlockScratch& sm) {
  wave_argmax(m, idx);
  if (lane_id() == 0) { sm.f[wave_id()] = m; sm.i[wave_id()] = idx; }
  __syncthreads();
  float rm = sm.f[0];
  int ri = sm.i[0];
#pragma unroll
  for (int w = 1; w < NWAVES; ++w) argmax_combine(rm, ri, sm.f[w], sm.i[w]);
  __syncthreads();
  m = rm;
  idx = ri;
}
// Block-wide inclusive and exclusive prefix sums in thread order.
__device__ __forceinline__ void block_scan(double v, double& incl, double& excl, BlockScratch& sm) {
  const double wi = wave_incl_scan(v);
  const double prev = __shfl_up(wi, 1);
  if (lane_id() == 63) sm.d[wave_id()] = wi;
  __syncthreads();
  double off = 0.0;
  for (int w = 0; w < wave_id(); ++w) off += sm.d[w];
  __syncthreads();
  incl = off + wi;
  excl = (lane_id() == 0) ? off : off + prev;
}

// ------------------------------------------------------------------ cross-workgroup records
// Workgroups hand data to each other inside one launch without fences and
// without atomics: a record is an array of 8-byte words, each holding a 32-bit
// value and the 32-bit tag of the call that wrote it. The writer stores the words
// with device-coherent 8-byte stores and moves on; the record's one reader polls
// them with device-coherent loads until every word carries the call's tag, then
// clears the words (tag 0). A word is written and read whole, so a matching tag
// means its value is this call's. Every call draws a fresh odd tag, and every
// record is cleared by its reader, so neither an earlier call's words nor those of
// an earlier replay of the same captured graph can ever match.
//
// A workgroup only ever waits for records of workgroups with a lower dispatch
// index, which were dispatched before it and are resident or finished; waits are
// bounded all the same (about 0.2 s), and a timeout is reported as an error.
constexpr int SPIN_LIMIT = 1 << 18;

template <class T>
struct RecWords {
  static_assert(sizeof(T) % 4 == 0, "records are made of 4-byte words");
  static constexpr int N = sizeof(T) / 4;
};

template <class T>
__device__ __forceinline__ void put_rec(uint64_t* dst, const T& v, uint32_t tag) {
  uint32_t w[RecWords<T>::N];
  __builtin_memcpy(w, &v, sizeof(T));
#pragma unroll
  for (int i = 0; i < RecWords<T>::N; ++i)
    __hip_atomic_store(dst + i, ((uint64_t)tag << 32) | w[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Waits until all words of the record carry `tag`; false on timeout (v undefined).
template <class T>
__device__ __forceinline__ bool get_rec(const uint64_t* src, T& v, uint32_t tag) {
  uint32_t w[RecWords<T>::N];
  for (int spin = 0; spin < SPIN_LIMIT; ++spin) {
    bool ok = true;
#pragma unroll
    for (int i = 0; i < RecWords<T>::N; ++i) {
      const uint64_t x = __hip_atomic_load(src + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      ok = ok && ((uint32_t)(x >> 32) == tag);
      w[i] = (uint32_t)x;
    }
    if (ok) {
      __builtin_memcpy(&v, w, sizeof(T));
      return true;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  return false;
}

// Clears a consumed record (its reader does this once it has read it).
template <class T>
__device__ __forceinline__ void clear_rec(uint64_t* dst) {
#pragma unroll
  for (int i = 0; i < RecWords<T>::N; ++i)
    __hip_atomic_store(dst + i, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Logical block index with consecutive indices placed on the same XCD:
// workgroups are dispatched round-robin over the 8 XCDs, so hardware block b runs
// on XCD b % 8. This makes the chunks of one row share that XCD's L2.
__device__ __forceinline__ int64_t xcd_logical_block(int64_t hw, int64_t nblocks) {
  constexpr int64_t NX = 8;
  const int64_t xcd = hw % NX, local = hw / NX;
  const int64_t base = nblocks / NX, rem = nblocks % NX;
  return xcd * base + (xcd < rem ? xcd : rem) + local;
}

// ------------------------------------------------------------------ chunk statistics
// Reduces one chunk, loaded raw by load_chunk_raw, to its partial (same value in
// every thread): max with lowest index (if ARG), and the weight sum relative to
// fl32(m*c0) (if SUM). Units are decoded on the fly in each pass, so only the raw
// words stay live across the block reduction.
template <int DT, bool SUM, bool ARG>
__device__ __forceinline__ Partial reduce_chunk(const char* row, int64_t V, int64_t unit0, bool aligned,
                                                const ChunkRaw& raw, float c0, BlockScratch& sm) {
  constexpr int W = DTraits<DT>::W;
  const int tid = threadIdx.x;
  float best = -INFINITY;
  int pos = INT_SENTINEL;
#pragma unroll
  for (int j = 0; j < UNROLL; ++j) {
    float x[W];
    decode_unit_at<DT>(row, V, unit0, aligned, raw, j, x);
#pragma unroll
    for (int e = 0; e < W; ++e) {
      if constexpr (ARG) {
        if (x[e] > best) { best = x[e]; pos = j * W + e; }
      } else {
        best = fmaxf(best, x[e]);
      }
    }
  }
  Partial p;
  p.s = 0.0;
  if constexpr (ARG) {
    int gidx = INT_SENTINEL;
    if (pos != INT_SENTINEL)
      gidx = (int)((unit0 + (int64_t)(pos / W) * BLOCK + tid) * W + (pos % W));
    block_argmax(best, gidx, sm);
    p.m = best;
    p.idx = gidx;
  } else {
    p.m = block_max(best, sm);
    p.idx = INT_SENTINEL;
  }
  if constexpr (SUM) {
    const float mc0 = chunk_mc0(p.m, c0);
    double acc = 0.0;
#pragma unroll
    for (int j = 0; j < UNROLL; ++j) {
      float w[W];
      decode_unit_at<DT>(row, V, unit0, aligned, raw, j, w);
#pragma unroll
      for (int e = 0; e < W; ++e) w[e] = softmax_weight(w[e], c0, mc0);
      acc += (double)pairwise_sum<W>(w);
    }
    p.s = block_sum(acc, sm);
  }
  return p;
}

// ------------------------------------------------------------------ inverse-CDF scan in one chunk
// Weight policy for one softmax row: w = exp2(fma(x, c0, -mc0)).
template <int DT>
struct SoftmaxWeights {
  const char* row;
  int64_t V;
  bool aligned;
  float c0, mc0;
  __device__ void unit(int64_t u, float (&w)[DTraits<DT>::W]) const {
    float x[DTraits<DT>::W];
    load_unit<DT>(row, V, u, aligned, x);
#pragma unroll
    for (int e = 0; e < DTraits<DT>::W; ++e) w[e] = softmax_weight(x[e], c0, mc0);
  }
  __device__ void chunk(int64_t unit0, float (&w)[UNROLL][DTraits<DT>::W]) const {
    load_chunk<DT>(row, V, unit0, aligned, w);
#pragma unroll
    for (int j = 0; j < UNROLL; ++j)
#pragma unroll
      for (int e = 0; e < DTraits<DT>::W; ++e) w[j][e] = softmax_weight(w[j][e], c0, mc0);
  }
};

// Weight policy for the residual max(0, p_t - p_d) of a target/draft row pair:
// p = exp2(fma(x, c0, -mc0)) * invZ with invZ = 1 / sum_v exp2(x_v*c0 - mc0).
template <int DT>
struct ResidualWeights {
  const char* trow;
  const char* drow;
  int64_t V;
  bool taligned, daligned;
  float c0, mc0t, mc0d, izt, izd;
  __device__ float weight(float xt, float xd) const {
    const float pt = softmax_weight(xt, c0, mc0t);
    const float pd = softmax_weight(xd, c0, mc0d) * izd;
    return fmaxf(0.0f, __builtin_fmaf(pt, izt, -pd));
  }
  __device__ void unit(int64_t u, float (&w)[DTraits<DT>::W]) const {
    float xt[DTraits<DT>::W], xd[DTraits<DT>::W];
    load_unit<DT>(trow, V, u, taligned, xt);
    load_unit<DT>(drow, V, u, daligned, xd);
#pragma unroll
    for (int e = 0; e < DTraits<DT>::W; ++e) w[e] = weight(xt[e], xd[e]);
  }
  __device__ void chunk(int64_t unit0, float (&w)[UNROLL][DTraits<DT>::W]) const {
    float xd[UNROLL][DTraits<DT>::W];
    load_chunk<DT>(trow, V, unit0, taligned, w);
    load_chunk<DT>(drow, V, unit0, daligned, xd);
#pragma unroll
    for (int j = 0; j < UNROLL; ++j)
#pragma unroll
      for (int e = 0; e < DTraits<DT>::W; ++e) w[j][e] = weight(w[j][e], xd[j][e]);
  }
};

// Sum of a policy's weights over chunk c (fixed order, same unit sums as the scan).
template <int DT, class Policy>
__device__ __forceinline__ double chunk_weight_sum(const Policy& pol, int64_t c, BlockScratch& sm) {
  constexpr int W = DTraits<DT>::W;
  const int64_t unit0 = c * UNITS_PER_CHUNK;
  double acc = 0.0;
  float w[UNROLL][W];
  pol.chunk(unit0, w);
#pragma unroll
  for (int j = 0; j < UNROLL; ++j) acc += (double)pairwise_sum<W>(w[j]);
  return block_sum(acc, sm);
}

// Inverse CDF inside chunk c: the row index of the first element whose cumulative
// weight (element order within the chunk) exceeds theta. If rounding leaves no
// such element (theta at or past the chunk total), the last element of positive
// weight. Returns -1 if the chunk has no positive weight. Same value in all threads.
template <int DT, class Policy>
__device__ __forceinline__ int64_t chunk_invcdf(const Policy& pol, int64_t c, double theta, BlockScratch& sm) {
  constexpr int W = DTraits<DT>::W;
  const int tid = threadIdx.x;
  const int64_t unit0 = c * UNITS_PER_CHUNK;
  float us[UNROLL];
  {
    float w[UNROLL][W];
    pol.chunk(unit0, w);
#pragma unroll
    for (int j = 0; j < UNROLL; ++j) us[j] = pairwise_sum<W>(w[j]);
  }

  // 1) which group of BLOCK consecutive units holds the crossing
  double tot[UNROLL];
#pragma unroll
  for (int j = 0; j < UNROLL; ++j) tot[j] = block_sum((double)us[j], sm);
  int js = -1;
  double before = 0.0;
  bool fallback = false;
  {
    double cum = 0.0;
#pragma unroll
    for (int j = 0; j < UNROLL; ++j) {
      if (js < 0 && cum + tot[j] > theta) { js = j; before = cum; }
      cum += tot[j];
    }
    if (js < 0) {
      fallback = true;
#pragma unroll
      for (int j = 0; j < UNROLL; ++j)
        if (tot[j] > 0.0) js = j;
      if (js < 0) return -1;
    }
  }
  // 2) which unit (thread) of that group
  float my = 0.0f;
#pragma unroll
  for (int j = 0; j < UNROLL; ++j) if (j == js) my = us[j];
  double incl, excl;
  block_scan((double)my, incl, excl, sm);
  int tstar = 0;
  const double th = theta - before;
  if (!fallback) {
    const int below = block_sum_int((incl > th) ? 0 : 1, sm);   // incl is non-decreasing
    if (below >= BLOCK) fallback = true;
    tstar = below;
  }
  if (fallback) tstar = block_max_int(my > 0.0f ? tid : -1, sm);
  // 3) which element of that unit: recompute its weights (same expression as above)
  if (tid == tstar) {
    const int64_t u = unit0 + (int64_t)js * BLOCK + tid;
    float w[W];
    pol.unit(u, w);
    int pick = -1;
    if (!fallback) {
      double cum = excl;
#pragma unroll
      for (int e = 0; e < W; ++e) {
        cum += (double)w[e];
        if (pick < 0 && cum > th) pick = e;
      }
    }
    if (pick < 0) {
#pragma unroll
      for (int e = 0; e < W; ++e) if (w[e] > 0.0f) pick = e;
    }
    sm.result = u * W + pick;
  }
  __syncthreads();
  const int64_t r = sm.result;
  __syncthreads();
  return r;
}

// ------------------------------------------------------------------ chunk selection (wave 0)
constexpr int MAX_CHUNKS = 256;            // 4 chunks per lane of wave 0
constexpr int CHUNKS_PER_LANE = MAX_CHUNKS / 64;

// Given per-chunk weights W_c (c < C) held by lane-contiguous ranges, pick the
// first chunk whose inclusive prefix exceeds u * total. Runs in wave 0 only;
// result fields are valid in all lanes of wave 0.
struct ChunkPick {
  int c;          // chosen chunk, -1 if the total is not a positive finite number
  double before;  // sum of weights of the chunks before c
  double total;   // sum of all chunk weights (scan order)
  double theta;   // u * total
  bool fallback;  // no chunk crossed: c is the last chunk of positive weight
};

// Each lane of wave 0 holds the weights of chunks c_lo .. c_lo+CHUNKS_PER_LANE-1
// (c_lo = lane * ceil(C/64); zero past its range), in wl[].
__device__ __forceinline__ void lane_chunk_range(int C, int& c_lo, int& c_hi) {
  const int per = (C + 63) / 64;
  c_lo = min(C, lane_id() * per);
  c_hi = min(C, c_lo + per);
}

__device__ __forceinline__ ChunkPick pick_chunk(int C, double u, const double (&wl)[CHUNKS_PER_LANE]) {
  const int lane = lane_id();
  int c_lo, c_hi;
  lane_chunk_range(C, c_lo, c_hi);
  double local = 0.0;
#pragma unroll
  for (int q = 0; q < CHUNKS_PER_LANE; ++q) local += wl[q];
  const double incl = wave_incl_scan(local);
  const double prev = __shfl_up(incl, 1);
  const double excl = (lane == 0) ? 0.0 : prev;
  const double total = __shfl(incl, 63);
  ChunkPick r;
  r.total = total;
  r.theta = 0.0;
  r.c = -1;
  r.before = 0.0;
  r.fallback = false;
  if (!(total > 0.0) || !__builtin_isfinite(total)) return r;
  const double theta = u * total;
  r.theta = theta;
  int hit = INT_SENTINEL;
  double hit_before = 0.0;
  {
    double cum = excl;
#pragma unroll
    for (int q = 0; q < CHUNKS_PER_LANE; ++q) {
      if (hit == INT_SENTINEL && c_lo + q < c_hi) {
        if (cum + wl[q] > theta) { hit = c_lo + q; hit_before = cum; }
        cum += wl[q];
      }
    }
  }
  // first lane with a hit (hits are monotone in lane order)
  const unsigned long long mask = __ballot(hit != INT_SENTINEL);
  if (mask != 0ull) {
    const int src = __builtin_ctzll(mask);
    r.c = __shfl(hit, src);
    r.before = __shfl(hit_before, src);
    return r;
  }
  // rounding left no crossing: the last chunk with positive weight
  int last = -1;
#pragma unroll
  for (int q = 0; q < CHUNKS_PER_LANE; ++q)
    if (c_lo + q < c_hi && wl[q] > 0.0) last = c_lo + q;
  last = wave_max_int(last);
  r.c = last;
  r.fallback = true;
  return r;
}

}  // namespace sv

// Device building blocks for libspecverify (gfx950, wave64).
//
// Work is split into waves, not workgroups: a 128-thread workgroup holds two
// wave64s that never synchronise with each other, so one wave's arithmetic
// overlaps the others' memory traffic. A wave streams one chunk of one row: lane l
// owns the 16-byte units u0 + j*64 + l (j < CU), so every load instruction reads
// 1 KiB of contiguous memory and a chunk is CU KiB (8 KiB: 4096 bf16/fp16 or 2048
// fp32 logits).
//
// Arithmetic (the row softmax at temperature T, in base 2):
//   c0 = log2(e)/T (fp32).  Chunk max m_c; mc0 = fl32(m_c * c0).
//   element weight  w = exp2(fma(x, c0, -mc0))            (fp32, v_exp_f32)
//   unit sum        pairwise fp32 sum of the unit's W weights
//   chunk sum s_c   per-lane fp64 sum of its unit sums, then a fixed fp64
//                   butterfly across the wave
//   row normaliser  Z = sum_c s_c * 2^(mc0_c - M*c0)       (fp64, M = row max)
// Every reduction has a fixed order, so results are bit-identical run to run, and
// code that recomputes a weight uses the same expression as the pass that summed it.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

constexpr int WAVE = 64;
constexpr int BLOCK = 128;
constexpr int WPB = BLOCK / WAVE;               // independent waves per workgroup
#ifndef SV_CU
#define SV_CU 8
#endif
constexpr int CU = SV_CU;                       // 16-byte units per lane per chunk
constexpr int CHUNK_UNITS = WAVE * CU;          // 512 units = 8 KiB
constexpr int MAX_ROUNDS = 4;                   // chunks per lane in a row combine
constexpr int MAX_CHUNKS = WAVE * MAX_ROUNDS;   // chunks per row
constexpr int INT_SENTINEL = 0x7fffffff;

enum { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2 };

template <int DT> struct DTraits;
template <> struct DTraits<DT_F32>  { static constexpr int W = 4; static constexpr int E = 4; };
template <> struct DTraits<DT_BF16> { static constexpr int W = 8; static constexpr int E = 2; };
template <> struct DTraits<DT_F16>  { static constexpr int W = 8; static constexpr int E = 2; };

// Per-(row, chunk) partial statistics.
struct Partial {
  float m;     // chunk max (-inf if no entry above -inf)
  int idx;     // lowest row index holding m (INT_SENTINEL if none; argmax mode only)
  double s;    // sum of exp2(fma(x, c0, -fl32(m*c0))) over the chunk (softmax mode only)
  float xv;    // the logit at the row's draft token, if this chunk holds it
  int xin;     // 1 if this chunk holds the draft token
};

// Per-row statistics, written by the wave that combines the row.
struct RowStat {
  double Z;    // sum_v 2^(x_v*c0 - M*c0), M*c0 in fp64
  double px;   // softmax probability of the row's draft token (draft/target pair rows)
  float M;     // row max
  int argmax;  // lowest index of M, -1 if none
  int ok;      // 1 usable, 0 data error, -1 a wait timed out
  int y;       // token drawn at this row (bonus row, tree nodes), -1 if none
};

// ------------------------------------------------------------------ lanes and waves
__device__ __forceinline__ int lane_id() { return threadIdx.x & (WAVE - 1); }
// The wave's index in its workgroup, as a wave-uniform (scalar) value: role and
// address arithmetic derived from it then runs on the scalar unit, and pointers
// chosen by it come from scalar kernel-argument loads rather than vector loads.
__device__ __forceinline__ int wave_in_block() { return __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE); }

// Cross-lane steps use DPP row operations (inside rows of 16 lanes: swap
// neighbours, swap pairs, mirror halves, mirror the row), after which every lane
// of a row holds the row's result; the four row results are then combined in
// lane order from lanes 0, 16, 32 and 48. Both orders are fixed, so every lane
// gets the same bits, run after run.
enum : int {
  DPP_XOR1 = 0xB1,          // quad_perm [1,0,3,2]
  DPP_XOR2 = 0x4E,          // quad_perm [2,3,0,1]
  DPP_HALF_MIRROR = 0x141,  // lane i <-> 7-i within 8
  DPP_MIRROR = 0x140,       // lane i <-> 15-i within 16
  DPP_SHR1 = 0x111, DPP_SHR2 = 0x112, DPP_SHR4 = 0x114, DPP_SHR8 = 0x118,
  DPP_BCAST15 = 0x142, DPP_BCAST31 = 0x143
};

template <int CTRL, int ROW_MASK = 0xF, bool BOUND_ZERO = false>
__device__ __forceinline__ int dpp_i(int v, int old = 0) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, ROW_MASK, 0xF, BOUND_ZERO);
}
template <int CTRL, int ROW_MASK = 0xF, bool BOUND_ZERO = false>
__device__ __forceinline__ float dpp_f(float v, float old = 0.0f) {
  return __int_as_float(dpp_i<CTRL, ROW_MASK, BOUND_ZERO>(__float_as_int(v), __float_as_int(old)));
}
template <int CTRL, int ROW_MASK = 0xF, bool BOUND_ZERO = false>
__device__ __forceinline__ double dpp_d(double v, double old = 0.0) {
  const long long x = __double_as_longlong(v), o = __double_as_longlong(old);
  const int lo = dpp_i<CTRL, ROW_MASK, BOUND_ZERO>((int)(x & 0xffffffffll), (int)(o & 0xffffffffll));
  const int hi = dpp_i<CTRL, ROW_MASK, BOUND_ZERO>((int)(x >> 32), (int)(o >> 32));
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}
__device__ __forceinline__ double readlane_d(double v, int l) {
  const long long x = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane((int)(x & 0xffffffffll), l);
  const int hi = __builtin_amdgcn_readlane((int)(x >> 32), l);
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}
__device__ __forceinline__ float readlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ int readlane_i(int v, int l) { return __builtin_amdgcn_readlane(v, l); }

__device__ __forceinline__ double wave_sum(double v) {
  v += dpp_d<DPP_XOR1>(v);
  v += dpp_d<DPP_XOR2>(v);
  v += dpp_d<DPP_HALF_MIRROR>(v);
  v += dpp_d<DPP_MIRROR>(v);
  return ((readlane_d(v, 0) + readlane_d(v, 16)) + readlane_d(v, 32)) + readlane_d(v, 48);
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<DPP_XOR1>(v));
  v = fmaxf(v, dpp_f<DPP_XOR2>(v));
  v = fmaxf(v, dpp_f<DPP_HALF_MIRROR>(v));
  v = fmaxf(v, dpp_f<DPP_MIRROR>(v));
  return fmaxf(fmaxf(readlane_f(v, 0), readlane_f(v, 16)), fmaxf(readlane_f(v, 32), readlane_f(v, 48)));
}
__device__ __forceinline__ int wave_max_int(int v) {
  v = max(v, dpp_i<DPP_XOR1>(v));
  v = max(v, dpp_i<DPP_XOR2>(v));
  v = max(v, dpp_i<DPP_HALF_MIRROR>(v));
  v = max(v, dpp_i<DPP_MIRROR>(v));
  return max(max(readlane_i(v, 0), readlane_i(v, 16)), max(readlane_i(v, 32), readlane_i(v, 48)));
}
// (value, index): larger value wins, lower index on equal values.
__device__ __forceinline__ void argmax_combine(float& m, int& i, float m2, int i2) {
  if (m2 > m || (m2 == m && i2 < i)) { m = m2; i = i2; }
}
template <int CTRL>
__device__ __forceinline__ void argmax_step(float& m, int& i) {
  const float m2 = dpp_f<CTRL>(m);
  const int i2 = dpp_i<CTRL>(i);
  argmax_combine(m, i, m2, i2);
}
__device__ __forceinline__ void wave_argmax(float& m, int& i) {
  argmax_step<DPP_XOR1>(m, i);
  argmax_step<DPP_XOR2>(m, i);
  argmax_step<DPP_HALF_MIRROR>(m, i);
  argmax_step<DPP_MIRROR>(m, i);
  float rm = readlane_f(m, 0);
  int ri = readlane_i(i, 0);
  argmax_combine(rm, ri, readlane_f(m, 16), readlane_i(i, 16));
  argmax_combine(rm, ri, readlane_f(m, 32), readlane_i(i, 32));
  argmax_combine(rm, ri, readlane_f(m, 48), readlane_i(i, 48));
  m = rm;
  i = ri;
}
// Inclusive prefix sum over the 64 lanes in lane order: shifts by 1, 2, 4, 8
// inside each row, then the totals of rows 0 and 2 into rows 1 and 3, then the
// total of rows 0-1 into rows 2-3.
__device__ __forceinline__ double wave_incl_scan(double v) {
  v += dpp_d<DPP_SHR1, 0xF, true>(v);
  v += dpp_d<DPP_SHR2, 0xF, true>(v);
  v += dpp_d<DPP_SHR4, 0xF, true>(v);
  v += dpp_d<DPP_SHR8, 0xF, true>(v);
  v += dpp_d<DPP_BCAST15, 0xA, false>(v, 0.0);
  v += dpp_d<DPP_BCAST31, 0xC, false>(v, 0.0);
  return v;
}
__device__ __forceinline__ int first_lane(unsigned long long mask) { return mask ? __builtin_ctzll(mask) : -1; }

// ------------------------------------------------------------------ element decoding
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

template <int W>
__device__ __forceinline__ float max_of(const float (&x)[W]) {
  if constexpr (W == 8) {
    return fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
  } else {
    return fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
  }
}

// m*c0 in fp32 as used for the chunk's weights; 0 for an empty (-inf) chunk so
// that its -inf entries weigh exp2(-inf) = 0 instead of NaN.
__device__ __forceinline__ float chunk_mc0(float m, float c0) { return (m == -INFINITY) ? 0.0f : m * c0; }

// ------------------------------------------------------------------ chunks
// Chunk c of a row: units [c*CHUNK_UNITS, (c+1)*CHUNK_UNITS). Every chunk is
// brought into the same register layout, a lane's CU units as packed 16-byte
// words: units inside the row of a 16-byte aligned row are vector loads; the unit
// that straddles the row end, and every unit of a row that does not start on a
// 16-byte boundary, are assembled element by element; entries at or past V hold
// -inf (no weight, never a maximum).
struct Chunk {
  const char* row;
  int64_t V;
  int64_t u0;
};

// NU consecutive 16-byte units per lane: a whole chunk (CU) or a part of one.
template <int NU>
struct RawN {
  uint4 v[NU];
};
using Raw = RawN<CU>;

template <int DT>
__device__ __forceinline__ uint32_t neg_inf_bits() {
  if constexpr (DT == DT_F32) return 0xff800000u;
  else if constexpr (DT == DT_BF16) return 0xff80ff80u;
  else return 0xfc00fc00u;
}

// Unit u assembled element by element (entries past V are -inf).
template <int DT>
__device__ __forceinline__ uint4 unit_by_elements(const char* row, int64_t V, int64_t u) {
  constexpr int W = DTraits<DT>::W;
  const uint32_t ninf = neg_inf_bits<DT>();
  uint32_t w[4] = {ninf, ninf, ninf, ninf};
  const int64_t e0 = u * W;
  if constexpr (DT == DT_F32) {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(row);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (e0 + e < V) w[e] = p[e0 + e];
  } else {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(row);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (e0 + e < V) {
        const uint32_t h = p[e0 + e];
        w[e >> 1] = (e & 1) ? ((w[e >> 1] & 0x0000ffffu) | (h << 16)) : ((w[e >> 1] & 0xffff0000u) | h);
      }
    }
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Loads this lane's NU units of the run of NU * WAVE units from unit u0 (this
// lane's unit j is u0 + j * WAVE + lane).
template <int DT, int NU>
__device__ __forceinline__ Chunk load_units(const char* row, int64_t V, int64_t u0, RawN<NU>& r) {
  constexpr int W = DTraits<DT>::W;
  Chunk k;
  k.row = row;
  k.V = V;
  k.u0 = u0;
  const int lane = lane_id();
  const bool aligned = row_aligned(row);
  if (aligned && (k.u0 + NU * WAVE) * W <= V) {
    // the common case: the whole run is inside an aligned row
    const uint4* p = reinterpret_cast<const uint4*>(row) + k.u0 + lane;
#pragma unroll
    for (int j = 0; j < NU; ++j) r.v[j] = p[j * WAVE];
  } else {
    const uint32_t ninf = neg_inf_bits<DT>();
#pragma unroll
    for (int j = 0; j < NU; ++j) {
      const int64_t u = k.u0 + j * WAVE + lane;
      if (aligned && (u + 1) * W <= V) {
        r.v[j] = reinterpret_cast<const uint4*>(row)[u];
      } else if (u * W < V) {
        r.v[j] = unit_by_elements<DT>(row, V, u);
      } else {
        r.v[j] = make_uint4(ninf, ninf, ninf, ninf);
      }
    }
  }
  return k;
}

// Loads this lane's CU units of chunk c.
template <int DT>
__device__ __forceinline__ Chunk load_chunk(const char* row, int64_t V, int64_t c, Raw& r) {
  return load_units<DT, CU>(row, V, c * CHUNK_UNITS, r);
}

// The W values of this lane's unit j.
template <int DT>
__device__ __forceinline__ void unit_values(const Raw& r, int j, float (&x)[DTraits<DT>::W]) {
  decode_unit<DT>(r.v[j], x);
}

// Partial of a chunk (same value in every lane): max, with the lowest index
// holding it if ARG (NaN never chosen), if SUM the weight sum relative to
// fl32(max*c0), and the logit at row index x if the chunk holds it (x < 0: none).
// Makes the compiler take the chunk's raw words as changed, so that logits it
// decoded from them for one pass are not kept in registers for the next (it
// decodes them again: one or two instructions per 32-bit word). fp32 words are the
// logits themselves and need no barrier.
template <int DT, int NU>
__device__ __forceinline__ void decode_barrier(RawN<NU>& r) {
  if constexpr (DT != DT_F32) {
#pragma unroll
    for (int j = 0; j < NU; ++j)
      asm volatile("" : "+v"(r.v[j].x), "+v"(r.v[j].y), "+v"(r.v[j].z), "+v"(r.v[j].w));
  }
}

template <int DT, bool SUM, bool ARG>
__device__ __forceinline__ Partial chunk_reduce(const Chunk& k, Raw r, float c0, int64_t x) {
  constexpr int W = DTraits<DT>::W;
  float best = -INFINITY;
  int pos = INT_SENTINEL;
#pragma unroll
  for (int j = 0; j < CU; ++j) {
    float v[W];
    unit_values<DT>(r, j, v);
    if constexpr (ARG) {
      const int base = (int)((k.u0 + j * WAVE + lane_id()) * W);
#pragma unroll
      for (int e = 0; e < W; ++e)
        if (v[e] > best) { best = v[e]; pos = base + e; }
    } else {
      best = fmaxf(best, max_of<W>(v));
    }
  }
  Partial p;
  if constexpr (ARG) {
    wave_argmax(best, pos);
    p.m = best;
    p.idx = pos;
  } else {
    p.m = wave_max(best);
    p.idx = INT_SENTINEL;
  }
  p.s = 0.0;
  if constexpr (SUM) {
    decode_barrier<DT>(r);   // decode again for the sums rather than hold every logit
    const float mc0 = chunk_mc0(p.m, c0);
    double s = 0.0;
#pragma unroll
    for (int j = 0; j < CU; ++j) {
      // one unit decoded at a time: the compiler would otherwise decode
      // them all ahead of the exponentials and hold the floats
      if (j > 0) decode_barrier<DT>(r);
      float w[W];
      unit_values<DT>(r, j, w);
#pragma unroll
      for (int e = 0; e < W; ++e) w[e] = softmax_weight(w[e], c0, mc0);
      s += (double)pairwise_sum<W>(w);
    }
    p.s = wave_sum(s);
  }
  p.xv = 0.0f;
  p.xin = 0;
  const int64_t ux = x >= 0 ? x / W - k.u0 : -1;   // the unit holding x, relative to the chunk
  if (ux >= 0 && ux < CHUNK_UNITS && x < k.V) {
    const int jx = (int)(ux / WAVE), lx = (int)(ux % WAVE), ex = (int)(x % W);
    float v = 0.0f;
#pragma unroll
    for (int j = 0; j < CU; ++j) {
      if (j == jx) {
        float xs[W];
        unit_values<DT>(r, j, xs);
#pragma unroll
        for (int e = 0; e < W; ++e) if (e == ex) v = xs[e];
      }
    }
    p.xv = __shfl(v, lx);
    p.xin = 1;
  }
  return p;
}

// Partial of a chunk for the entropy of softmax(row / T): the max m, the weight
// sum s relative to fl32(m*c0), and the first moment s1 = sum_v w_v t_v of the
// exponents t_v = x_v*c0 - fl32(m*c0) (base-2 units; divide by c0 for x - m).
struct EntPartial {
  float m;
  int pad;
  double s;
  double s1;
};

template <int DT>
__device__ __forceinline__ EntPartial chunk_reduce_ent(const Raw& r, float c0) {
  constexpr int W = DTraits<DT>::W;
  float best = -INFINITY;
#pragma unroll
  for (int j = 0; j < CU; ++j) {
    float x[W];
    unit_values<DT>(r, j, x);
    best = fmaxf(best, max_of<W>(x));
  }
  EntPartial p;
  p.m = wave_max(best);
  p.pad = 0;
  const float mc0 = chunk_mc0(p.m, c0);
  double s = 0.0, s1 = 0.0;
#pragma unroll
  for (int j = 0; j < CU; ++j) {
    float x[W], w[W], wx[W];
    unit_values<DT>(r, j, x);
#pragma unroll
    for (int e = 0; e < W; ++e) {
      // the weight from the exponent as it is (a NaN entry poisons the sum, as it
      // must); in the moment the exponent is floored at -1000, where the weight is
      // 0 in fp32 anyway, so that -inf entries add 0 * -1000 = 0
      const float t = __builtin_fmaf(x[e], c0, -mc0);
      w[e] = __builtin_amdgcn_exp2f(t);
      wx[e] = w[e] * fmaxf(t, -1000.0f);
    }
    s += (double)pairwise_sum<W>(w);
    s1 += (double)pairwise_sum<W>(wx);
  }
  p.s = wave_sum(s);
  p.s1 = wave_sum(s1);
  return p;
}

// Loads chunk c of a row and reduces it.
template <int DT, bool SUM, bool ARG>
__device__ __forceinline__ Partial chunk_partial(const char* row, int64_t V, int64_t c, float c0, int64_t x = -1) {
  Raw r;
  const Chunk k = load_chunk<DT>(row, V, c, r);
  return chunk_reduce<DT, SUM, ARG>(k, r, c0, x);
}

// 2^d for d <= 0 (fp64), as 2^floor(d) * exp2f(frac(d)): relative error ~1e-7.
__device__ __forceinline__ double pow2_neg(double d) {
  if (!(d > -1000.0)) return (d != d) ? d : 0.0;   // NaN stays NaN; far below: 0
  const double di = floor(d);
  return ldexp((double)__builtin_amdgcn_exp2f((float)(d - di)), (int)di);
}

// Streaming waves of one launch: rows are processed in groups of 8 consecutive
// rows, and every chunk of a row runs on the same XCD (workgroups are dispatched
// round-robin over the 8 XCDs): row q on XCD q % 8. The chunks of a row are
// padded to a multiple of WPB waves (CP) so that no workgroup spans two rows;
// padding waves have c >= C and do nothing. RQ rows.
__device__ __forceinline__ void stream_coords(uint32_t w, uint32_t CP, uint32_t RQ, uint32_t& q, uint32_t& c) {
  const uint32_t bpr = CP / WPB;           // workgroups per row
  const uint32_t h = w / WPB, lw = w % WPB;
  const uint32_t G = 8 * bpr;              // workgroups per group of 8 rows
  const uint32_t g = h / G, hb = h - g * G;
  const uint32_t rows = min(8u, RQ - 8 * g);
  uint32_t r, jb;
  if (rows == 8) {
    r = hb % 8;
    jb = hb / 8;
  } else {
    r = hb / bpr;
    jb = hb - r * bpr;
  }
  q = 8 * g + r;
  c = jb * WPB + lw;
}

// ------------------------------------------------------------------ inverse CDF inside one chunk
// Weight functors: softmax weights of one row, or the residual max(0, p_t - p_d)
// of a (target, draft) row pair.
struct SoftmaxW {
  float c0, mc0;
  __device__ __forceinline__ float operator()(float x, float) const { return softmax_weight(x, c0, mc0); }
};
struct ResidW {
  float c0, mc0t, mc0d, izt, izd;
  __device__ __forceinline__ float operator()(float xt, float xd) const {
    const float pt = softmax_weight(xt, c0, mc0t) * izt;
    const float pd = softmax_weight(xd, c0, mc0d) * izd;
    return fmaxf(pt - pd, 0.0f);
  }
};

// Weights of this lane's unit j (j a compile-time constant after unrolling).
template <int DT, bool PAIR, class WT, int NU>
__device__ __forceinline__ void unit_weights(const RawN<NU>& ra, const RawN<NU>& rb, int j, const WT& wt,
                                             float (&w)[DTraits<DT>::W]) {
  constexpr int W = DTraits<DT>::W;
  float xa[W], xb[W];
  decode_unit<DT>(ra.v[j], xa);
  if constexpr (PAIR) decode_unit<DT>(rb.v[j], xb);
#pragma unroll
  for (int e = 0; e < W; ++e) w[e] = wt(xa[e], PAIR ? xb[e] : 0.0f);
}

// The row index of the first element of the chunk (in row order) whose
// cumulative weight exceeds th, or, if rounding leaves none, of the last element
// of positive weight; -1 if the chunk has no positive weight. Same value in
// every lane. PAIR: weights of the element pairs of ra (target) and rb (draft).
//
// Units in row order are j-major, lane-minor. The search first finds the unit row
// j whose running total crosses th (fp64 wave totals), then the lane inside it
// (one fp64 prefix scan), then the element inside that unit.
template <int DT, bool PAIR, class WT, int NU>
__device__ __forceinline__ void chunk_unit_sums(const RawN<NU>& ra, const RawN<NU>& rb, const WT& wt,
                                                float (&us)[NU]) {
  constexpr int W = DTraits<DT>::W;
#pragma unroll
  for (int j = 0; j < NU; ++j) {
    float w[W];
    unit_weights<DT, PAIR>(ra, rb, j, wt, w);
    us[j] = pairwise_sum<W>(w);
  }
}

// The same search from this lane's unit weight sums us[j] (unit j*64 + lane, as
// chunk_unit_sums forms them), which the caller may already hold.
template <int DT, bool PAIR, class WT, int NU>
__device__ __forceinline__ int64_t chunk_invcdf_us(const Chunk& k, RawN<NU> ra, RawN<NU> rb, const float (&us)[NU],
                                                   double th, const WT& wt) {
  constexpr int W = DTraits<DT>::W;
  const int lane = lane_id();
  double off = 0.0, offj = 0.0;
  int hj = -1;
#pragma unroll
  for (int j = 0; j < NU; ++j) {
    const double t = wave_sum((double)us[j]);
    if (hj < 0 && off + t > th) { hj = j; offj = off; }
    off += t;
  }
  int key = -1;     // (unit row, lane) of the unit holding the answer
  bool scan = false;
  double hexcl = 0.0;
  if (hj >= 0) {
    float uj = us[0];
#pragma unroll
    for (int j = 1; j < NU; ++j) if (j == hj) uj = us[j];
    const double incl = wave_incl_scan((double)uj);
    const unsigned long long hit = __ballot(offj + incl > th);
    if (hit) {
      const int hl = first_lane(hit);
      key = hj * WAVE + hl;
      hexcl = offj + __shfl(incl, hl) - (double)__shfl(uj, hl);
      scan = true;
    } else {
      // rounding between the two sums: the last positive unit of that row
      key = wave_max_int(uj > 0.0f ? hj * WAVE + lane : -1);
    }
  }
  if (key < 0) {
    // no crossing: the last unit of positive weight in the chunk
#pragma unroll
    for (int j = 0; j < NU; ++j) if (us[j] > 0.0f) key = j * WAVE + lane;
    key = wave_max_int(key);
    if (key < 0) return -1;
  }
  const int kj = key / WAVE, kl = key % WAVE;
  // the crossing unit decoded again rather than every unit's logits held since the sums
  decode_barrier<DT>(ra);
  if constexpr (PAIR) decode_barrier<DT>(rb);
  // the unit's weights, selected by a branch per unit row (wave-uniform) so that
  // the register array is never indexed at run time
  float w[W];
#pragma unroll
  for (int e = 0; e < W; ++e) w[e] = 0.0f;
#pragma unroll
  for (int j = 0; j < NU; ++j)
    if (j == kj) unit_weights<DT, PAIR>(ra, rb, j, wt, w);
  int pick = -1;
  if (lane == kl) {
    if (scan) {
      double cum = hexcl;
#pragma unroll
      for (int e = 0; e < W; ++e) {
        cum += (double)w[e];
        if (pick < 0 && cum > th) pick = e;
      }
    }
    if (pick < 0) {   // rounding inside the unit, or no crossing: its last positive element
#pragma unroll
      for (int e = 0; e < W; ++e) if (w[e] > 0.0f) pick = e;
    }
  }
  pick = __shfl(pick, kl);
  return (k.u0 + kj * WAVE + kl) * W + pick;
}

template <int DT, bool PAIR, class WT, int NU>
__device__ __forceinline__ int64_t chunk_invcdf(const Chunk& k, const RawN<NU>& ra, const RawN<NU>& rb, double th,
                                                const WT& wt) {
  float us[NU];
  chunk_unit_sums<DT, PAIR>(ra, rb, wt, us);
  return chunk_invcdf_us<DT, PAIR>(k, ra, rb, us, th, wt);
}

// ------------------------------------------------------------------ chunk selection over a row
// Chunk weights held lane-strided: lane l holds chunks l + 64*t (t < R),
// zero past C. Picks the first chunk (row order) whose inclusive prefix exceeds
// u * total.
struct ChunkPick {
  int c;          // chosen chunk; -1 if the total is not a positive finite number
  double before;  // sum of the weights of the chunks before c
  double theta;   // u * total
  double total;   // the weights' sum
  bool fallback;  // rounding left no crossing: c is the last chunk of positive weight
};

template <int R = MAX_ROUNDS>
__device__ __forceinline__ ChunkPick pick_chunk(int C, double u, const double (&wl)[R]) {
  const int lane = lane_id();
  ChunkPick r;
  r.c = -1;
  r.before = 0.0;
  r.theta = 0.0;
  r.total = 0.0;
  r.fallback = false;
  if (C <= WAVE) {
    // one round: the inclusive scan gives the total (its last lane) and the crossing
    const double w0 = lane < C ? wl[0] : 0.0;
    const double incl = wave_incl_scan(w0);
    const double tot = readlane_d(incl, WAVE - 1);
    r.total = tot;
    if (!(tot > 0.0) || !__builtin_isfinite(tot)) return r;
    const double theta = u * tot;
    r.theta = theta;
    const unsigned long long hit = __ballot(incl > theta && lane < C);
    if (hit) {
      const int l = first_lane(hit);
      r.c = l;
      r.before = __shfl(incl, l) - __shfl(w0, l);
      return r;
    }
    r.c = wave_max_int(lane < C && w0 > 0.0 ? lane : -1);
    r.fallback = true;
    return r;
  }
  // the rounds' totals are formed twice (the same sums in the same order) rather
  // than held, to keep the registers of large R down
  double tot = 0.0;
#pragma unroll
  for (int t = 0; t < R; ++t) tot += (t * WAVE < C) ? wave_sum(wl[t]) : 0.0;
  r.total = tot;
  if (!(tot > 0.0) || !__builtin_isfinite(tot)) return r;
  const double theta = u * tot;
  r.theta = theta;
  double off = 0.0, offt = 0.0;
  int ht = -1;
#pragma unroll
  for (int t = 0; t < R; ++t) {
    const double tr = (t * WAVE < C) ? wave_sum(wl[t]) : 0.0;
    if (ht < 0 && off + tr > theta) { ht = t; offt = off; }
    off += tr;
  }
  if (ht >= 0) {
    double wt = wl[0];
#pragma unroll
    for (int t = 1; t < R; ++t) if (t == ht) wt = wl[t];
    const double incl = wave_incl_scan(wt);
    const unsigned long long hit = __ballot(offt + incl > theta && ht * WAVE + lane < C);
    if (hit) {
      const int l = first_lane(hit);
      r.c = ht * WAVE + l;
      r.before = offt + __shfl(incl, l) - __shfl(wt, l);
      return r;
    }
  }
  int last = -1;
#pragma unroll
  for (int t = 0; t < R; ++t)
    if (t * WAVE + lane < C && wl[t] > 0.0) last = t * WAVE + lane;
  r.c = wave_max_int(last);
  r.fallback = true;
  return r;
}

// ------------------------------------------------------------------ kernel parameters
// A kernel's by-value parameter struct, read in place in the kernel-argument
// segment (the constant address space), field by field where the code uses it.
// Named as a kernel parameter, every field the kernel uses is loaded into scalar
// registers on entry and kept live through every branch, which in kernels of many
// roles spills scalar registers to vector lanes on every wave's path.
template <class T>
__device__ __forceinline__ const T& kernel_args() {
  return *(const T*)(const __attribute__((address_space(4))) T*)__builtin_amdgcn_kernarg_segment_ptr();
}

// ------------------------------------------------------------------ cross-wave records
// Waves hand data to each other inside one launch without fences: a record is an
// array of 8-byte words, each holding a 32-bit value and the 32-bit tag of the
// call that wrote it. The writer stores the words with device-coherent 8-byte
// stores; a reader polls them with device-coherent loads until every word carries
// the call's tag. A word is written and read whole, so a matching tag means its
// value is this call's. Every record is cleared (tag 0) by the last wave that
// reads it, so records of an earlier call, or of an earlier replay of a captured
// graph that carries the same tag, never match.
//
// Which wave is "last" is decided by device-scope atomic counters in the same
// workspace; each is reset to zero by the wave that sees it reach its final count.
// Waits are bounded; a timeout is reported as an error, never a hang.
//
// A wait gives up once the GPU's constant 100 MHz clock has advanced by
// g_wait_ticks since its first unsuccessful poll (a wait whose first poll succeeds
// reads neither the clock nor the limit). The limit is per device; the host sets
// it with spec_set_wait_limit (default 0.25 s).
constexpr uint64_t WAIT_TICKS = 25000000;
static __device__ uint64_t g_wait_ticks = WAIT_TICKS;

struct WaitClock {
  uint64_t end = 0;
  // Called after an unsuccessful poll: false once the wait's time is up.
  __device__ __forceinline__ bool more() {
    const uint64_t now = __builtin_amdgcn_s_memrealtime();
    if (end == 0) {
      end = now + g_wait_ticks + 1;
      return true;
    }
    return now <= end;
  }
};

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

// The same record written by the whole wave with one store instruction: lane i
// stores word i. v must be the same in every lane.
template <class T>
__device__ __forceinline__ void put_rec_wave(uint64_t* dst, const T& v, uint32_t tag) {
  constexpr int N = RecWords<T>::N;
  static_assert(N <= WAVE, "one word per lane");
  uint32_t w[N];
  __builtin_memcpy(w, &v, sizeof(T));
  const int lane = lane_id();
  uint32_t mine = 0;
#pragma unroll
  for (int i = 0; i < N; ++i)
    if (lane == i) mine = w[i];
  if (lane < N) __hip_atomic_store(dst + lane, ((uint64_t)tag << 32) | mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Waits until all words of the record carry `tag`; false on timeout (v undefined).
template <class T>
__device__ __forceinline__ bool get_rec(const uint64_t* src, T& v, uint32_t tag) {
  uint32_t w[RecWords<T>::N];
  WaitClock clk;
  for (;;) {
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
    if (!clk.more()) return false;
    __builtin_amdgcn_s_sleep(2);
  }
}

// Polls a whole record with one load per word, lane i reading word i (one request
// for the record's line), with a longer pause between polls: for waits that may
// last a while. Called by every lane of the wave; the record is returned in every
// lane; false on timeout (v undefined).
template <class T>
__device__ __forceinline__ bool poll_rec(const uint64_t* src, T& v, uint32_t tag) {
  constexpr int N = RecWords<T>::N;
  static_assert(N <= WAVE, "one word per lane");
  const int lane = lane_id();
  WaitClock clk;
  for (;;) {
    uint64_t x = 0;
    if (lane < N) x = __hip_atomic_load(src + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (__ballot(lane < N && (uint32_t)(x >> 32) != tag) == 0ull) {
      uint32_t w[N];
#pragma unroll
      for (int i = 0; i < N; ++i) w[i] = __shfl((uint32_t)x, i);
      __builtin_memcpy(&v, w, sizeof(T));
      return true;
    }
    if (!clk.more()) return false;
    __builtin_amdgcn_s_sleep(8);
  }
}

// Zeroing a record or a counter for the next call. Every caller makes the last
// access its words get in the launch, so the store need not be seen by another
// wave of the same launch: it is a plain store, which completes in its XCD's L2
// (a device-scope store writes through to memory, about a microsecond, and a wave
// whose last stores are still in flight holds its slot). The end of the launch
// writes the L2 back before any later launch can read the word.
__device__ __forceinline__ void store_zero(uint64_t* p) {
  __hip_atomic_store(p, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
}
template <class T>
__device__ __forceinline__ void clear_rec(uint64_t* dst) {
#pragma unroll
  for (int i = 0; i < RecWords<T>::N; ++i) store_zero(dst + i);
}

__device__ __forceinline__ uint32_t counter_add(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// OR of error bits, complete before the wave goes on: the returned value is
// consumed, so the wave waits for it, and the bits are in place before any later
// event count of this wave (the emission, which reads them, follows that count).
__device__ __forceinline__ void error_or(uint32_t* p, uint32_t v) {
  uint32_t prev = __hip_atomic_fetch_or(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  asm volatile("" : "+v"(prev));
}
__device__ __forceinline__ uint64_t state_or(uint64_t* p, uint64_t v) {
  return __hip_atomic_fetch_or(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t state_load(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// (the last access of the counter in the launch; see store_zero)
template <class T>
__device__ __forceinline__ void counter_reset(T* p) {
  __hip_atomic_store(p, (T)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
}

}  // namespace sv

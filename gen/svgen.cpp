// Seeded synthetic workload generator for speculative-decoding verification.
//
// This file produces INPUTS only (logits, uniforms, draft-token draws); it holds
// none of the verification arithmetic. Both the CPU oracle and the HIP library
// consume the bytes it writes.
//
// Random numbers: counter-based SplitMix64 (Steele, Lea, Flood, "Fast splittable
// pseudorandom number generators", OOPSLA 2014; constants as published by Vigna).
// Value i of the stream with key K is mix(K + (i+1)*GAMMA), i.e. the i-th output
// of a SplitMix64 generator seeded with K, so any element can be generated
// independently and the output does not depend on the thread count.
// Normals: Box-Muller in double. Uniforms for the verifier: (r >> 40) * 2^-24.
// Rounding: double -> fp32 (round to nearest even, C cast), then fp32 -> bf16 or
// fp16 with the round-to-nearest-even bit code below.

#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>
#include <algorithm>

namespace {

constexpr uint64_t GAMMA = 0x9E3779B97F4A7C15ull;

inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

inline uint64_t stream_at(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * GAMMA); }

// open interval (0,1): 53-bit mantissa, never 0
inline double unit_open(uint64_t r) { return ((double)(r >> 11) + 0.5) * (1.0 / 9007199254740992.0); }

// Box-Muller: normal number i of stream key uses the counter pair (2j, 2j+1), j = i/2;
// even i takes the cosine branch, odd i the sine branch.
inline double normal_at(uint64_t key, uint64_t i) {
  const uint64_t j = i >> 1;
  const double u1 = unit_open(stream_at(key, 2 * j));
  const double u2 = unit_open(stream_at(key, 2 * j + 1));
  const double rad = std::sqrt(-2.0 * std::log(u1));
  const double ang = 6.283185307179586476925286766559 * u2;
  return (i & 1) ? rad * std::sin(ang) : rad * std::cos(ang);
}

inline uint32_t f32_bits(float f) { uint32_t u; std::memcpy(&u, &f, 4); return u; }
inline float bits_f32(uint32_t u) { float f; std::memcpy(&f, &u, 4); return f; }

// fp32 -> bf16, round to nearest even (finite inputs; NaN kept quiet)
inline uint16_t to_bf16(float f) {
  uint32_t u = f32_bits(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// fp32 -> IEEE binary16, round to nearest even, with subnormals and overflow to inf
inline uint16_t to_f16(float f) {
  const uint32_t u = f32_bits(f);
  const uint32_t sign = (u >> 16) & 0x8000u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return (uint16_t)(sign | 0x7e00u);   // NaN
  if (a >= 0x477ff000u) return (uint16_t)(sign | 0x7c00u);  // rounds to >= 65520: inf
  if (a < 0x38800000u) {                                    // below 2^-14: subnormal or zero
    if (a < 0x33000000u) return (uint16_t)sign;             // below 2^-25: rounds to 0
    const uint32_t e = a >> 23;                              // biased fp32 exponent, 102..112
    const uint32_t mant = (a & 0x7fffffu) | 0x800000u;       // 24-bit significand
    const uint32_t shift = 126 - e;                          // bits to drop to reach 2^-24 units
    uint32_t q = mant >> shift;
    const uint32_t rem = mant & ((1u << shift) - 1u);
    const uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (q & 1u))) q += 1;
    return (uint16_t)(sign | q);
  }
  // normal range: rebias exponent (127 -> 15) and round the 13 dropped bits
  uint32_t v = a - 0x38000000u;                              // exponent - 112
  const uint32_t rem = v & 0x1fffu;
  v >>= 13;
  if (rem > 0x1000u || (rem == 0x1000u && (v & 1u))) v += 1;
  return (uint16_t)(sign | v);
}

inline void store(int dtype, void* out, size_t i, double x) {
  const float f = (float)x;
  switch (dtype) {
    case 0: static_cast<float*>(out)[i] = f; break;
    case 1: static_cast<uint16_t*>(out)[i] = to_bf16(f); break;
    default: static_cast<uint16_t*>(out)[i] = to_f16(f); break;
  }
}

inline double load(int dtype, const void* in, size_t i) {
  switch (dtype) {
    case 0: return static_cast<const float*>(in)[i];
    case 1: return bits_f32((uint32_t) static_cast<const uint16_t*>(in)[i] << 16);
    default: {
      const uint16_t h = static_cast<const uint16_t*>(in)[i];
      const int e = (h >> 10) & 31, m = h & 1023;
      const double s = (h & 0x8000) ? -1.0 : 1.0;
      if (e == 0) return s * std::ldexp((double)m, -24);
      if (e == 31) return m ? NAN : s * INFINITY;
      return s * std::ldexp((double)(m | 1024), e - 25);
    }
  }
}

template <class F>
void parallel_for(size_t n, int nthreads, F&& body) {
  if (nthreads <= 0) {
    nthreads = (int)std::thread::hardware_concurrency();
    if (nthreads <= 0) nthreads = 1;
    nthreads = std::min(nthreads, 16);
  }
  if (n < (1u << 16) || nthreads == 1) { body(size_t(0), n); return; }
  std::vector<std::thread> ts;
  const size_t per = (n + nthreads - 1) / nthreads;
  for (int t = 0; t < nthreads; ++t) {
    const size_t lo = std::min(n, t * per), hi = std::min(n, lo + per);
    if (lo < hi) ts.emplace_back([=, &body] { body(lo, hi); });
  }
  for (auto& th : ts) th.join();
}

}  // namespace

extern "C" {

uint64_t svg_mix64(uint64_t x) { return mix64(x); }
uint64_t svg_stream_at(uint64_t key, uint64_t i) { return stream_at(key, i); }
double svg_normal_at(uint64_t key, uint64_t i) { return normal_at(key, i); }

// Stream key of (config id, seed, purpose): three chained SplitMix64 steps.
uint64_t svg_key(uint64_t cfg, uint64_t seed, uint64_t purpose) {
  return stream_at(stream_at(stream_at(cfg, 0) ^ seed, 0) ^ purpose, 0);
}

// a_i = sig_a * N_a(first+i); if out_b: b_i = a_i + sig_b * N_b(first+i).
// Both are rounded to `dtype` (0 fp32, 1 bf16, 2 fp16) only at the store.
void svg_normal_pair(uint64_t key_a, double sig_a, uint64_t key_b, double sig_b,
                     uint64_t first, uint64_t n, int dtype, void* out_a, void* out_b,
                     int nthreads) {
  parallel_for(n, nthreads, [&](size_t lo, size_t hi) {
    for (size_t i = lo; i < hi; ++i) {
      const double a = sig_a * normal_at(key_a, first + i);
      if (out_a) store(dtype, out_a, i, a);
      if (out_b) store(dtype, out_b, i, a + sig_b * normal_at(key_b, first + i));
    }
  });
}

// Verifier uniforms in [0, 1 - 2^-24]: exactly representable in fp32.
void svg_uniform24(uint64_t key, uint64_t first, uint64_t n, float* out) {
  for (uint64_t i = 0; i < n; ++i)
    out[i] = (float)((double)(stream_at(key, first + i) >> 40) * (1.0 / 16777216.0));
}

// Draw one token per row from softmax(x / T) by the Gumbel-max trick:
// token = argmax_v (x_v / T - log(-log(U_v))), U_v open-uniform from stream
// element row*V + v. Ties (probability zero) go to the lowest index.
void svg_gumbel_rows(uint64_t key, int dtype, int64_t rows, int64_t V, const void* logits,
                     double T, int32_t* out, int nthreads) {
  parallel_for((size_t)rows, nthreads, [&](size_t lo, size_t hi) {
    for (size_t r = lo; r < hi; ++r) {
      double best = -INFINITY;
      int32_t arg = 0;
      for (int64_t v = 0; v < V; ++v) {
        const size_t idx = r * (size_t)V + (size_t)v;
        const double g = -std::log(-std::log(unit_open(stream_at(key, idx))));
        const double s = load(dtype, logits, idx) / T + g;
        if (s > best) { best = s; arg = (int32_t)v; }
      }
      out[r] = arg;
    }
  });
}

// Greedy draft choice: index of the first largest stored value per row.
void svg_argmax_rows(int dtype, int64_t rows, int64_t V, const void* logits, int32_t* out,
                     int nthreads) {
  parallel_for((size_t)rows, nthreads, [&](size_t lo, size_t hi) {
    for (size_t r = lo; r < hi; ++r) {
      double best = -INFINITY;
      int32_t arg = 0;
      for (int64_t v = 0; v < V; ++v) {
        const double x = load(dtype, logits, r * (size_t)V + (size_t)v);
        if (x > best) { best = x; arg = (int32_t)v; }
      }
      out[r] = arg;
    }
  });
}

// Round doubles to a storage dtype (used for crafted test rows).
void svg_round(int dtype, int64_t n, const double* in, void* out) {
  for (int64_t i = 0; i < n; ++i) store(dtype, out, (size_t)i, in[i]);
}

// Decode a storage dtype to double (used by tests to build expectations).
void svg_decode(int dtype, int64_t n, const void* in, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = load(dtype, in, (size_t)i);
}

}  // extern "C"

// Host-side helpers of libspecverify: workspace layouts, argument checks, call
// tags and the dtype dispatch of launches.
#pragma once

#include "../../include/specverify.h"
#include "sv_device.hpp"

#include <hip/hip_runtime.h>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <initializer_list>

namespace sv {

constexpr double LOG2E = 1.4426950408889634073599246810019;

inline int elem_bytes(sv_dtype dt) { return dt == SV_F32 ? 4 : 2; }
inline bool dtype_ok(int dt) { return dt == SV_F32 || dt == SV_BF16 || dt == SV_F16; }

inline int64_t chunks_per_row(int64_t V, sv_dtype dt) {
  const int64_t W = 16 / elem_bytes(dt);
  const int64_t units = (V + W - 1) / W;
  return (units + CHUNK_UNITS - 1) / CHUNK_UNITS;
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Layout {
  size_t off[14];
  size_t total;
};

// Regions back to back, each 256-byte aligned.
inline Layout make_layout(std::initializer_list<size_t> sizes) {
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

inline bool temperature_ok(float T) { return std::isfinite(T) && T > 0.0f; }

inline float temperature_c0(float T) { return (float)(LOG2E / (double)T); }

inline sv_status launch_status() {
  return hipGetLastError() == hipSuccess ? SV_OK : SV_EHIP;
}

// A fresh record tag per call: odd (never the cleared value 0), distinct from the
// tags of the last 2^31 calls of this process.
inline std::atomic<uint32_t> g_tag{0};
inline uint32_t next_tag() { return (g_tag.fetch_add(1, std::memory_order_relaxed) << 1) | 1u; }

inline unsigned blocks_for(int64_t waves) { return (unsigned)((waves + WPB - 1) / WPB); }

template <template <int, bool> class Launcher, class... Args>
inline sv_status dispatch(sv_dtype dt, bool stoch, Args&&... args) {
  switch (dt) {
    case SV_F32: return stoch ? Launcher<DT_F32, true>::run(args...) : Launcher<DT_F32, false>::run(args...);
    case SV_BF16: return stoch ? Launcher<DT_BF16, true>::run(args...) : Launcher<DT_BF16, false>::run(args...);
    case SV_F16: return stoch ? Launcher<DT_F16, true>::run(args...) : Launcher<DT_F16, false>::run(args...);
  }
  return SV_EDTYPE;
}

inline bool ws_ok(const void* ws, size_t have, size_t need) {
  return ws != nullptr && (reinterpret_cast<uintptr_t>(ws) & 255u) == 0 && have >= need;
}

// Waves of one launch, and rows x chunks as 32-bit indices.
constexpr int64_t MAX_WAVES = 0x7fffffffLL;

static_assert((int64_t)MAX_CHUNKS * CHUNK_UNITS * 16 == SV_MAX_ROW_BYTES, "row limit of the header");

inline bool shape_ok(int64_t V, sv_dtype dt) {
  return V <= 0x7fffffffLL - 16 && chunks_per_row(V, dt) <= MAX_CHUNKS;
}

}  // namespace sv

// Wave-level (64-lane) reductions and scans for gfx950, on DPP row operations
// and lane reads: no LDS round trip, so they cost a few cycles instead of the
// LDS latency a shuffle-based butterfly pays at every step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pmqa {

// DPP controls (GFX9 encoding): shift right / rotate right within a 16-lane row.
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowRor1 = 0x121, kRowRor2 = 0x122, kRowRor4 = 0x124, kRowRor8 = 0x128;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  // lanes whose source lies outside their row read 0
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}

__device__ __forceinline__ uint32_t lane_of(uint32_t v, int l) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, l);
}

// Inclusive prefix sum within each 16-lane row.
__device__ __forceinline__ uint32_t row_prefix(uint32_t x) {
  x += dpp<kRowShr1>(x);
  x += dpp<kRowShr2>(x);
  x += dpp<kRowShr4>(x);
  return x + dpp<kRowShr8>(x);
}

// Inclusive prefix sum over the 64 lanes; `total` receives the wave's sum.
__device__ __forceinline__ uint32_t wave_prefix(uint32_t x, int lane, uint32_t& total) {
  x = row_prefix(x);
  const uint32_t r0 = lane_of(x, 15), r1 = lane_of(x, 31), r2 = lane_of(x, 47),
                 r3 = lane_of(x, 63);
  const int row = lane >> 4;
  x += (row > 0 ? r0 : 0u) + (row > 1 ? r1 : 0u) + (row > 2 ? r2 : 0u);
  total = r0 + r1 + r2 + r3;
  return x;
}

// Sum / max / min over the 64 lanes (uniform result).
__device__ __forceinline__ uint32_t wave_sum(uint32_t x) {
  x += dpp<kRowRor1>(x);
  x += dpp<kRowRor2>(x);
  x += dpp<kRowRor4>(x);
  x += dpp<kRowRor8>(x);
  return lane_of(x, 0) + lane_of(x, 16) + lane_of(x, 32) + lane_of(x, 48);
}

__device__ __forceinline__ uint32_t row_max(uint32_t x) {
  x = max(x, dpp<kRowRor1>(x));
  x = max(x, dpp<kRowRor2>(x));
  x = max(x, dpp<kRowRor4>(x));
  return max(x, dpp<kRowRor8>(x));
}

__device__ __forceinline__ uint32_t row_min(uint32_t x) {
  x = min(x, dpp<kRowRor1>(x));
  x = min(x, dpp<kRowRor2>(x));
  x = min(x, dpp<kRowRor4>(x));
  return min(x, dpp<kRowRor8>(x));
}

__device__ __forceinline__ uint32_t wave_max(uint32_t x) {
  x = row_max(x);
  return max(max(lane_of(x, 0), lane_of(x, 16)), max(lane_of(x, 32), lane_of(x, 48)));
}

__device__ __forceinline__ uint32_t wave_min(uint32_t x) {
  x = row_min(x);
  return min(min(lane_of(x, 0), lane_of(x, 16)), min(lane_of(x, 32), lane_of(x, 48)));
}

}  // namespace pmqa

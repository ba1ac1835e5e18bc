// Wavefront-64 primitives for gfx950 (CDNA4).
//
// Prefix sums, sums and maxima across a 64-lane wavefront, used by the
// radix-select kernels for the histogram suffix scan (finding the threshold
// bucket) and for ordered compaction of the selected indices.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mitopk {

constexpr int kWave = 64;

// Inclusive prefix sum over the lanes of one wavefront: lane i gets
// v[0] + ... + v[i].  Within each 16-lane row the sum is built with DPP row
// shifts; the row totals are then read with readlane and added to the rows
// above them.
__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t v) {
  // DPP control codes: row_shr:n is 0x110 + n.  With bound_ctrl set, lanes
  // whose source falls outside their row read 0.
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x111, 0xF, 0xF, true));
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x112, 0xF, 0xF, true));
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x114, 0xF, 0xF, true));
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x118, 0xF, 0xF, true));
  const uint32_t r0 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 15));
  const uint32_t r1 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 31));
  const uint32_t r2 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 47));
  const int row = static_cast<int>(__lane_id()) >> 4;
  uint32_t add = 0;
  add += (row >= 1) ? r0 : 0u;
  add += (row >= 2) ? r1 : 0u;
  add += (row >= 3) ? r2 : 0u;
  return v + add;
}

// Maximum over the lanes of one wavefront (every lane gets it): row maxima
// with DPP row shifts, then the four row results through readlane.
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x111, 0xF, 0xF, true)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x112, 0xF, 0xF, true)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x114, 0xF, 0xF, true)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x118, 0xF, 0xF, true)));
  const uint32_t r0 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 15));
  const uint32_t r1 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 31));
  const uint32_t r2 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 47));
  const uint32_t r3 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
  return max(max(r0, r1), max(r2, r3));
}

// Sum over the lanes of one wavefront (every lane gets it).
__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(wave_inclusive_sum(v)), 63));
}

}  // namespace mitopk

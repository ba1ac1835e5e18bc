// Wavefront-64 and workgroup primitives for gfx950 (CDNA4).
//
// Prefix sums across a 64-lane wavefront and across a workgroup, used by the
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

// LDS words block_inclusive_sum<BLOCK, NV> needs.
template <int BLOCK, int NV>
constexpr int scan_lds_words() {
  return NV * (BLOCK / kWave) + NV;
}

// Inclusive prefix sums of NV independent per-thread values across a
// workgroup of BLOCK threads (BLOCK a multiple of 64, at most 1024).  On
// return v[i] holds the inclusive prefix of value i and tot[i] its workgroup
// total.  Each wavefront scans its lanes; wavefront 0 then scans the
// wavefront totals and leaves each wavefront's offset in LDS, so a thread
// reads one offset per value instead of every wavefront's total.  Contains
// three workgroup barriers; every thread of the workgroup must call it.
template <int BLOCK, int NV>
__device__ __forceinline__ void block_inclusive_sum(uint32_t (&v)[NV], uint32_t (&tot)[NV],
                                                    uint32_t* lds) {
  constexpr int NW = BLOCK / kWave;
  static_assert(NW >= 1 && NW <= kWave, "workgroup of 64..4096 threads");
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    v[i] = wave_inclusive_sum(v[i]);
    if (lane == kWave - 1) lds[i * NW + w] = v[i];
  }
  __syncthreads();
  if (w == 0) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const uint32_t x = lane < NW ? lds[i * NW + lane] : 0u;
      const uint32_t incl = wave_inclusive_sum(x);
      if (lane < NW) lds[i * NW + lane] = incl - x;
      if (lane == NW - 1) lds[NV * NW + i] = incl;
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    v[i] += lds[i * NW + w];
    tot[i] = lds[NV * NW + i];
  }
  __syncthreads();
}

}  // namespace mitopk

// Device-side building blocks of the row-wise top-k radix select (gfx950).
//
// What is selected (the operation the public header states): for a row with
// valid length L and m = min(k, L), every entry strictly above the m-th
// largest value, plus entries equal to it taken lowest index first.  The
// entries strictly above the threshold are always taken and the threshold
// bucket is resolved afterwards, as in TopKCluster::forward on the SGLang
// PR #34167 page; the rows' valid length and memory stride follow the vLLM
// PR #42169 report page.
//
// How.  Each value gets an order-preserving 32-bit key.  Appending the
// reversed column index below the key gives a composite that is distinct for
// every entry and orders entries by (value descending, index ascending), so
// the wanted set is exactly the m largest composites and is unique.  A radix
// select over the composite's digits finds the shortest prefix P with
// "#(composites with that prefix >= P) == m"; the selected entries are then
// those whose prefix is >= P, and no separate tie pass is needed: for untied
// rows the key digits settle it, and the index digits are only reached when
// the threshold value is repeated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wave64.hpp"

namespace mitopk {

constexpr int kFirstBits = 12;  // sign, 8 exponent bits, 3 mantissa bits
constexpr int kFirstBins = 1 << kFirstBits;
constexpr int kNextBits = 10;  // later digits: 10 + 10 complete the key
constexpr int kNextBins = 1 << kNextBits;
// 12 + 10 + 10 key bits, then at most 31 index bits in 10-bit digits.
constexpr int kMaxRounds = 7;

// Order-preserving key: x < y (IEEE) implies key(x) < key(y).  Positive values
// get the sign bit set; negative values map to the two's complement of their
// bit pattern, which reverses their order and puts them below every positive
// value.  -0.0 (0x80000000) maps to 0x80000000, the key of +0.0, so the two
// zeros tie as IEEE says they do.  No value maps to 0 (the smallest image is
// 1, from the all-ones NaN pattern); key 0 marks entries outside the row.
__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t u = __float_as_uint(x);
  return (static_cast<int32_t>(u) >= 0) ? (u | 0x80000000u) : (0u - u);
}
__device__ __forceinline__ uint32_t order_key_bits(uint32_t u) {
  return (static_cast<int32_t>(u) >= 0) ? (u | 0x80000000u) : (0u - u);
}

// A fixed prefix of the composite (key : reversed index).
//   bits <= 32: kp holds the top `bits` bits of the key;
//   bits  > 32: kp is the whole key T and ip the top (bits - 32) bits of the
//               reversed index (ib index bits in all).
struct Prefix {
  int bits;
  uint32_t kp;
  uint32_t ip;
};

__device__ __forceinline__ int digit_bits(int bits, int ib) {
  if (bits == 0) return kFirstBits;
  if (bits < 32) return kNextBits;
  const int left = 32 + ib - bits;
  return left < kNextBits ? left : kNextBits;
}

__device__ __forceinline__ Prefix extend(Prefix p, int d, uint32_t b) {
  if (p.bits < 32) {
    p.kp = (p.kp << d) | b;
  } else {
    p.ip = (p.ip << d) | b;
  }
  p.bits += d;
  return p;
}

// Prefix tests, one type per phase so that the per-entry code has no
// branches on the phase.  Each answers, for an entry (key, column j):
//   ge(): composite prefix >= P (the entry is selected once P is final)
//   eq(): composite prefix == P (the entry is in the current bucket)
// Entries outside the row carry key 0 and fail both.
struct PredKey {    // 0 < bits <= 32, kp != 0
  int sh;
  uint32_t kp;
  __device__ __forceinline__ bool ge(uint32_t key, int32_t) const { return (key >> sh) >= kp; }
  __device__ __forceinline__ bool eq(uint32_t key, int32_t) const { return (key >> sh) == kp; }
};
struct PredKey0 {   // 0 < bits <= 32, kp == 0: the lowest bucket
  int sh;
  __device__ __forceinline__ bool ge(uint32_t key, int32_t) const { return key != 0u; }
  __device__ __forceinline__ bool eq(uint32_t key, int32_t) const {
    return key != 0u && (key >> sh) == 0u;
  }
};
struct PredIdx {    // bits > 32: key == T decided, index digits follow
  uint32_t T;
  int ish;
  uint32_t ip;
  uint32_t rmask;
  __device__ __forceinline__ bool ge(uint32_t key, int32_t j) const {
    return key > T || (key == T && ((rmask - static_cast<uint32_t>(j)) >> ish) >= ip);
  }
  __device__ __forceinline__ bool eq(uint32_t key, int32_t j) const {
    return key == T && ((rmask - static_cast<uint32_t>(j)) >> ish) == ip;
  }
};

// Calls f(pred) with the prefix test for p (a uniform branch).
template <class F>
__device__ __forceinline__ void with_pred(const Prefix& p, int ib, uint32_t rmask, F f) {
  if (p.bits <= 32) {
    const int sh = 32 - p.bits;
    if (p.kp != 0u) {
      f(PredKey{sh, p.kp});
    } else {
      f(PredKey0{sh});
    }
  } else {
    f(PredIdx{p.kp, ib - (p.bits - 32), p.ip, rmask});
  }
}

// Histogram one digit (d bits, below prefix p) of the entries in p's bucket,
// for entries produced by `for_each(f)` calling f(key, j).  p.bits > 0.
template <class ForEach>
__device__ __forceinline__ void count_digit(ForEach for_each, const Prefix& p, int d, int ib,
                                            uint32_t rmask, uint32_t* hist) {
  const uint32_t dmask = (1u << d) - 1u;
  if (p.bits < 32) {
    const int sh = 32 - p.bits;
    const int dsh = sh - d;
    const uint32_t kp = p.kp;
    if (kp != 0u) {
      for_each([&](uint32_t key, int32_t) {
        if ((key >> sh) == kp) atomicAdd(&hist[(key >> dsh) & dmask], 1u);
      });
    } else {
      for_each([&](uint32_t key, int32_t) {
        if (key != 0u && (key >> sh) == 0u) atomicAdd(&hist[(key >> dsh) & dmask], 1u);
      });
    }
  } else {
    const int ish = ib - (p.bits - 32);
    const int dsh = ish - d;
    const uint32_t T = p.kp, ip = p.ip;
    for_each([&](uint32_t key, int32_t j) {
      const uint32_t ridx = rmask - static_cast<uint32_t>(j);
      if (key == T && (ridx >> ish) == ip) atomicAdd(&hist[(ridx >> dsh) & dmask], 1u);
    });
  }
}

// Finds the bucket b holding the need-th largest entry of a histogram of nb
// bins (nb a power of two): the largest b with sum(hist[b..nb)) >= need.
// Thread t owns a group of adjacent bins counted from the top; a workgroup
// prefix sum over the groups gives each group the number of entries above
// it, and the one group where that count crosses `need` walks its bins.
// Result in LDS: res[0] bucket, res[1] entries in higher buckets, res[2]
// entries in the bucket.
template <int BLOCK>
__device__ __forceinline__ void find_bucket(const uint32_t* hist, int nb, uint32_t need,
                                            uint32_t* lds_scan, uint32_t* res) {
  const int tid = threadIdx.x;
  const int bpt = nb >= BLOCK ? nb / BLOCK : 1;
  const int groups = nb / bpt;
  const int top = nb - tid * bpt;  // this thread's bins: [top - bpt, top)
  uint32_t s = 0;
  if (tid < groups) {
    for (int i = 0; i < bpt; ++i) s += hist[top - 1 - i];
  }
  uint32_t v[1] = {s}, tot[1];
  block_inclusive_sum<BLOCK, 1>(v, tot, lds_scan);
  const uint32_t incl = v[0];
  const uint32_t excl = incl - s;
  if (tid < groups && excl < need && incl >= need) {
    uint32_t run = excl;
    for (int i = 0; i < bpt; ++i) {
      const int bin = top - 1 - i;
      const uint32_t h = hist[bin];
      if (run + h >= need) {
        res[0] = static_cast<uint32_t>(bin);
        res[1] = run;
        res[2] = h;
        break;
      }
      run += h;
    }
  }
  __syncthreads();
}

// Radix rounds inside one workgroup.  `src.count(p, d, ib, rmask, hist)`
// histograms digit d below prefix p (p.bits == 0: all entries).  Starting
// from prefix p with `need` entries still to choose among p's bucket, the
// prefix is refined one digit at a time until the bucket holding the need-th
// entry contains exactly `need` entries.  Returns the final prefix: the
// selected entries are those whose composite prefix is >= it.
template <int BLOCK, class Src>
__device__ Prefix rounds_local(const Src& src, Prefix p, uint32_t need, int ib, uint32_t* hist,
                               uint32_t* lds_scan, uint32_t* res) {
  const uint32_t rmask = (1u << ib) - 1u;
  for (int round = 0; round < kMaxRounds + 1; ++round) {
    const int d = digit_bits(p.bits, ib);
    const int nb = 1 << d;
    for (int i = threadIdx.x; i < nb; i += BLOCK) hist[i] = 0;
    __syncthreads();
    src.count(p, d, ib, rmask, hist);
    __syncthreads();
    find_bucket<BLOCK>(hist, nb, need, lds_scan, res);
    const uint32_t b = res[0], gt = res[1], cnt = res[2];
    need -= gt;
    p = extend(p, d, b);
    if (cnt == need) break;
  }
  return p;
}

}  // namespace mitopk

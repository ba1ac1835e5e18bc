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
// Written without a compare and select: with s = all sign bits (0 or ~0),
// (u ^ (s | 2^31)) - s is u | 2^31 for s = 0 and ~u + 1 = -u for s = ~0.
__device__ __forceinline__ uint32_t order_key_bits(uint32_t u) {
  const uint32_t s = static_cast<uint32_t>(static_cast<int32_t>(u) >> 31);
  return (u ^ (s | 0x80000000u)) - s;
}
__device__ __forceinline__ uint32_t order_key(float x) { return order_key_bits(__float_as_uint(x)); }

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
  if (bits < 32) return 32 - bits < kNextBits ? 32 - bits : kNextBits;  // digits end at the key's end
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

// The smallest key an entry selected by prefix p can have.
__device__ __forceinline__ uint32_t prefix_edge(const Prefix& p) {
  return p.bits >= 32 ? p.kp : (p.kp << (32 - p.bits));
}

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
// for entries produced by `for_each(f)` calling f(key, j).
template <class ForEach>
__device__ __forceinline__ void count_digit(ForEach for_each, const Prefix& p, int d, int ib,
                                            uint32_t rmask, uint32_t* hist) {
  const uint32_t dmask = (1u << d) - 1u;
  if (p.bits == 0) {
    const int sh = 32 - d;
    for_each([&](uint32_t key, int32_t) {
      if (key != 0u) atomicAdd(&hist[key >> sh], 1u);
    });
  } else if (p.bits < 32) {
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

// hist[bin] += 1 for the lanes with `take`, as one atomic when every such
// lane of the wavefront has the same bin (the rows of a tied or constant
// input, where per-lane atomics to one address would serialise), else one
// per lane.  Every lane of the wavefront must call it.
__device__ __forceinline__ void hist_add_wave(uint32_t* hist, uint32_t bin, bool take) {
  const uint64_t tm = __ballot(take);
  if (tm == 0) return;
  const int first = __ffsll(static_cast<unsigned long long>(tm)) - 1;
  const uint32_t b0 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(bin), first));
  const uint64_t same = __ballot(take && bin == b0);
  if (same == tm) {
    if (static_cast<int>(__lane_id()) == first) atomicAdd(&hist[b0], static_cast<uint32_t>(__popcll(tm)));
  } else if (take) {
    atomicAdd(&hist[bin], 1u);
  }
}

// count_digit with wavefront-aggregated increments (hist_add_wave); for_each
// must call f for the same number of entries on every lane.
template <class ForEach>
__device__ __forceinline__ void count_digit_agg(ForEach for_each, const Prefix& p, int d, int ib,
                                                uint32_t rmask, uint32_t* hist) {
  const uint32_t dmask = (1u << d) - 1u;
  if (p.bits == 0) {
    const int sh = 32 - d;
    for_each([&](uint32_t key, int32_t) { hist_add_wave(hist, key >> sh, key != 0u); });
  } else if (p.bits < 32) {
    const int sh = 32 - p.bits;
    const int dsh = sh - d;
    const uint32_t kp = p.kp;
    if (kp != 0u) {
      for_each([&](uint32_t key, int32_t) {
        hist_add_wave(hist, (key >> dsh) & dmask, (key >> sh) == kp);
      });
    } else {
      for_each([&](uint32_t key, int32_t) {
        hist_add_wave(hist, (key >> dsh) & dmask, key != 0u && (key >> sh) == 0u);
      });
    }
  } else {
    const int ish = ib - (p.bits - 32);
    const int dsh = ish - d;
    const uint32_t T = p.kp, ip = p.ip;
    for_each([&](uint32_t key, int32_t j) {
      const uint32_t ridx = rmask - static_cast<uint32_t>(j);
      hist_add_wave(hist, (ridx >> dsh) & dmask, key == T && (ridx >> ish) == ip);
    });
  }
}

// Finds the bucket b holding the need-th largest entry of a histogram of NB
// bins (NB a power of two): the largest b with sum(hist[b..NB)) >= need.
// Result in LDS: res[0] bucket, res[1] entries in higher buckets, res[2]
// entries in the bucket.  Done by the calling wavefront alone (the other
// wavefronts of the workgroup need not take part), in two levels: lane l first sums a
// group of NB/64 adjacent bins (group l counted from the top, read with
// 16-byte LDS loads), a wavefront prefix sum finds the group holding the
// need-th entry, and then lane i reads bin i of that group and a second
// prefix sum finds the bin.  need_of(total) gives `need` from the
// histogram's total (so a caller can derive it from the count).  The result
// goes to res[0..2]; the caller synchronises before reading it.  Returns the
// histogram total.
template <int NB, class NeedOf>
__device__ __forceinline__ uint32_t find_bucket_wave_nb(const uint32_t* hist, NeedOf need_of,
                                                        uint32_t* res) {
  static_assert(NB >= 4 && (NB & (NB - 1)) == 0, "power-of-two bin count");
  constexpr int GS = NB >= kWave ? NB / kWave : 1;      // bins per group
  constexpr int GROUPS = NB / GS;
  const int lane = static_cast<int>(__lane_id());
  uint32_t s = 0;
  if (lane < GROUPS) {
    const int lo = NB - (lane + 1) * GS;                 // group [lo, lo + GS)
    if constexpr (GS >= 4) {
      // batches of at most four 16-byte loads in flight (few registers)
      constexpr int NV = GS / 4;
      constexpr int BATCH = NV < 4 ? NV : 4;
      const uint4* h4 = reinterpret_cast<const uint4*>(hist + lo);
#pragma unroll 1
      for (int b = 0; b < NV; b += BATCH) {
        uint4 v[BATCH];
#pragma unroll
        for (int i = 0; i < BATCH; ++i) v[i] = h4[b + i];
#pragma unroll
        for (int i = 0; i < BATCH; ++i) s += v[i].x + v[i].y + v[i].z + v[i].w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < GS; ++i) s += hist[lo + i];
    }
  }
  const uint32_t incl = wave_inclusive_sum(s);
  const uint32_t total = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(incl), 63));
  const uint32_t need = need_of(total);
  if (need == 0u || need > total) return total;
  const uint64_t crossed = __ballot(incl >= need);
  const int g = __ffsll(static_cast<unsigned long long>(crossed)) - 1;   // first group reaching need
  const uint32_t above_g = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(incl - s), g));
  // second level: lane i takes bin i of group g, counted from the group's top
  const int bin = NB - g * GS - 1 - lane;
  const uint32_t h = lane < GS ? hist[bin] : 0u;
  const uint32_t incl2 = above_g + wave_inclusive_sum(h);
  const uint64_t crossed2 = __ballot(lane < GS && incl2 >= need);
  const int c = __ffsll(static_cast<unsigned long long>(crossed2)) - 1;
  if (lane == c) {
    res[0] = static_cast<uint32_t>(bin);
    res[1] = incl2 - h;
    res[2] = h;
  }
  return total;
}

// The same search with every thread of the workgroup and one barrier:
// thread t sums group t of GS = NB/BLOCK adjacent bins counted from the top
// (one bin, for t < NB, when NB < BLOCK; read with 16-byte LDS loads when GS
// is a multiple of 4), a wavefront prefix sum and the wavefronts' totals (in
// wt[0..NW)) give each group the count above it, and the thread whose group
// crosses `need` walks its bins.  need_of(total) gives `need` from the
// histogram's total.  Result in res[0..2]; nothing is written when need is 0
// or above the total.  Every thread must call it; the caller synchronises
// before reading res (and before reusing wt).
template <int BLOCK, int NB, class NeedOf>
__device__ __forceinline__ void find_bucket_block(const uint32_t* hist, NeedOf need_of, uint32_t* res,
                                                  uint32_t* wt) {
  static_assert(NB >= 2 && (NB & (NB - 1)) == 0, "power-of-two bin count");
  constexpr int NW = BLOCK / kWave;
  constexpr int GS = NB >= BLOCK ? NB / BLOCK : 1;
  const int t = static_cast<int>(threadIdx.x);
  const bool live = t * GS < NB;
  const int top = NB - t * GS;  // this thread's bins: [top - GS, top)
  uint32_t h[GS];               // h[i]: bin top - 1 - i
  if constexpr (GS % 4 == 0) {
#pragma unroll
    for (int v = 0; v < GS / 4; ++v) {
      const uint4 q = *reinterpret_cast<const uint4*>(hist + top - 4 * (v + 1));
      h[4 * v + 0] = q.w;
      h[4 * v + 1] = q.z;
      h[4 * v + 2] = q.y;
      h[4 * v + 3] = q.x;
    }
  } else {
#pragma unroll
    for (int i = 0; i < GS; ++i) h[i] = live ? hist[top - 1 - i] : 0u;
  }
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < GS; ++i) s += h[i];
  const uint32_t incl = wave_inclusive_sum(s);
  const int w = t / kWave;
  if ((t & (kWave - 1)) == kWave - 1) wt[w] = incl;
  __syncthreads();
  uint32_t above = 0, total = 0;
#pragma unroll
  for (int v = 0; v < NW; ++v) {
    const uint32_t x = wt[v];
    above += v < w ? x : 0u;
    total += x;
  }
  const uint32_t need = need_of(total);
  if (need == 0u || need > total) return;
  const uint32_t a = above + incl - s;  // entries in the groups above this one
  if (live && a < need && a + s >= need) {
    uint32_t run = a;
    bool found = false;
#pragma unroll
    for (int i = 0; i < GS; ++i) {
      if (!found && run + h[i] >= need) {
        res[0] = static_cast<uint32_t>(top - 1 - i);
        res[1] = run;
        res[2] = h[i];
        found = true;
      }
      run += h[i];
    }
  }
}

// find_bucket_wave_nb for a bin count known only at run time (a power of two
// from 2 to 4096).
__device__ __forceinline__ void find_bucket_wave(const uint32_t* hist, int nb, uint32_t need,
                                                 uint32_t* res) {
  auto fixed = [need](uint32_t) { return need; };
  switch (nb) {
    case 4096: find_bucket_wave_nb<4096>(hist, fixed, res); break;
    case 1024: find_bucket_wave_nb<1024>(hist, fixed, res); break;
    case 512: find_bucket_wave_nb<512>(hist, fixed, res); break;
    case 256: find_bucket_wave_nb<256>(hist, fixed, res); break;
    case 128: find_bucket_wave_nb<128>(hist, fixed, res); break;
    case 64: find_bucket_wave_nb<64>(hist, fixed, res); break;
    case 32: find_bucket_wave_nb<32>(hist, fixed, res); break;
    case 16: find_bucket_wave_nb<16>(hist, fixed, res); break;
    case 8: find_bucket_wave_nb<8>(hist, fixed, res); break;
    case 4: find_bucket_wave_nb<4>(hist, fixed, res); break;
    default: {  // nb == 2
      const int lane = static_cast<int>(__lane_id());
      if (lane == 0) {
        const uint32_t h1 = hist[1], h0 = hist[0];
        if (h1 >= need) {
          res[0] = 1u; res[1] = 0u; res[2] = h1;
        } else {
          res[0] = 0u; res[1] = h1; res[2] = h0;
        }
      }
    }
  }
}

// Radix rounds inside one workgroup (wt: NW words of LDS scratch).
// `src.count(p, d, ib, rmask, hist)`
// histograms digit d below prefix p (p.bits == 0: all entries).  Starting
// from prefix p with `need` entries still to choose among p's bucket, the
// prefix is refined one digit at a time until the bucket holding the need-th
// entry contains exactly `need` entries.  Returns the final prefix: the
// selected entries are those whose composite prefix is >= it.  With
// key_need, the rounds stop once the whole key T is known (32 bits) and its
// bucket still holds more than the entries to take: *key_need is then set to
// the number of entries equal to T to take (the first in column order, for
// an emission that counts them), and the index digits are not visited.
template <int BLOCK, class Src>
__device__ __forceinline__ Prefix rounds_local(const Src& src, Prefix p, uint32_t need, int ib,
                                               uint32_t* hist, uint32_t* res, uint32_t* wt,
                                               uint32_t* key_need = nullptr) {
  const uint32_t rmask = (1u << ib) - 1u;
  for (int round = 0; round < kMaxRounds + 1; ++round) {
    const int d = digit_bits(p.bits, ib);
    const int nb = 1 << d;
    for (int i = threadIdx.x; i < nb; i += BLOCK) hist[i] = 0;
    __syncthreads();
    src.count(p, d, ib, rmask, hist);
    __syncthreads();
    if (threadIdx.x < kWave) find_bucket_wave(hist, nb, need, res);
    __syncthreads();
    const uint32_t b = res[0], gt = res[1], cnt = res[2];
    need -= gt;
    p = extend(p, d, b);
    if (cnt == need) break;
    if (key_need != nullptr && p.bits == 32) {
      *key_need = need;
      break;
    }
  }
  return p;
}

// The last step when the bucket of key prefix kp (the top 32 - sh key bits)
// holds at most 64 entries: they are gathered into LDS (lds[2i] key,
// lds[2i + 1] column, in any order; res[3] counts them and must be zero on
// entry), and the wavefronts rank them against each other by the composite
// (key, then lower column first); the entry of rank need - 1 is the last one
// selected.  Returns the prefix that selects exactly the need entries of the
// bucket: key >= T (32 bits) when no entry with key T falls below it, else
// the whole composite.  Two workgroup barriers; every thread must call it.
template <int BLOCK, class Src>
__device__ __forceinline__ Prefix finish_small(const Src& src, uint32_t kp, int sh, uint32_t need,
                                               int ib, uint32_t* lds, uint32_t* res) {
  src([&](uint32_t key, int32_t j) {
    if (key != 0u && (key >> sh) == kp) {
      const uint32_t at = atomicAdd(&res[3], 1u);
      lds[2 * at] = key;
      lds[2 * at + 1] = static_cast<uint32_t>(j);
    }
  });
  __syncthreads();
  {
    // Every wavefront holds the n entries on its lanes (lane l: entry l) and
    // ranks entries i = w, w + NW, ...: the rank of entry i is the number of
    // entries ordered before it, one ballot.  The wavefront holding rank
    // need - 1 (there is exactly one) reports it.
    const uint32_t n = res[3];
    const uint32_t lane = __lane_id();
    const uint32_t kl = lane < n ? lds[2 * lane] : 0u;
    const uint32_t jl = lane < n ? lds[2 * lane + 1] : 0u;
    constexpr uint32_t nw = BLOCK / kWave;
    const uint32_t w = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x / kWave)));
    for (uint32_t i = w; i < n; i += nw) {
      const uint32_t ki = lds[2 * i], ji = lds[2 * i + 1];
      const uint64_t before = __ballot(lane < n && (kl > ki || (kl == ki && jl < ji)));
      if (static_cast<uint32_t>(__popcll(before)) == need - 1u) {
        // an entry with key T ordered after (T, jt) is left out
        const uint64_t tie_below = __ballot(lane < n && kl == ki && jl > ji);
        if (lane == 0) {
          res[0] = ki;
          res[1] = ji;
          res[2] = tie_below != 0 ? 1u : 0u;
        }
      }
    }
  }
  __syncthreads();
  const uint32_t T = res[0], jt = res[1];
  if (res[2] == 0u) return Prefix{32, T, 0u};
  return Prefix{32 + ib, T, ((1u << ib) - 1u) - jt};
}

// The smallest shift s with (hi >> s) - (lo >> s) < kFirstBins (lo <= hi):
// at least bitlen(hi - lo) - kFirstBits (below it the difference is
// kFirstBins or more) and at most one more than that, since the difference
// falls as s grows.
__device__ __forceinline__ int window_shift(uint32_t lo, uint32_t hi) {
  int s = hi > lo ? max(0, 32 - __clz(hi - lo) - kFirstBits) : 0;
  while ((hi >> s) - (lo >> s) >= static_cast<uint32_t>(kFirstBins)) ++s;
  return s;
}

// Radix rounds for entries whose keys all lie in [lo, hi] (entries outside
// the row carry key 0).  The first round histograms the key bits just below
// the ones every key in [lo, hi] shares: the shift s is the smallest that
// puts hi >> s and lo >> s fewer than kFirstBins apart, and bin i counts keys
// with key >> s == (lo >> s) + i, so its bucket is an ordinary key prefix of
// 32 - s bits.  When the keys are confined to a narrow range (a filtered
// list), that one round resolves as many bits as two or three full-range
// digits and spreads the entries over many bins.  A bucket of at most 64
// entries is then finished by finish_small, a larger one by rounds_local.
// hist_zero: the caller has already zeroed hist[0..kFirstBins) before a
// workgroup barrier.  equal_ok: the caller's emission keeps only the first
// `need` selected entries in column order, so when lo == hi (every key the
// same, nothing above it) the whole key is returned after the one round,
// without rounds over the columns.  res[3] is overwritten.  Returns the
// final prefix.
template <int BLOCK, class Src>
__device__ __forceinline__ Prefix rounds_window(const Src& src, uint32_t lo, uint32_t hi,
                                                uint32_t need, int ib, uint32_t* hist,
                                                uint32_t* res, uint32_t* wt,
                                                bool hist_zero = false, bool equal_ok = false) {
  const int s = window_shift(lo, hi);
  const uint32_t base = lo >> s;
  if (!hist_zero) {  // (uniform) else the caller cleared it before a barrier
    for (int i = threadIdx.x; i < kFirstBins; i += BLOCK) hist[i] = 0;
    __syncthreads();
  }
  src([&](uint32_t key, int32_t) {
    if (key != 0u) atomicAdd(&hist[(key >> s) - base], 1u);
  });
  __syncthreads();
  if (threadIdx.x == 0) res[3] = 0u;  // finish_small's counter (visible after the search's barrier)
  find_bucket_block<BLOCK, kFirstBins>(hist, [need](uint32_t) { return need; }, res, wt);
  __syncthreads();
  const uint32_t b = res[0], gt = res[1], cnt = res[2];
  need -= gt;
  const Prefix p{32 - s, base + b, 0u};
  if (cnt == need || (equal_ok && lo == hi)) return p;
  if (cnt <= static_cast<uint32_t>(kWave)) return finish_small<BLOCK>(src, base + b, s, need, ib, hist, res);
  return rounds_local<BLOCK>(src, p, need, ib, hist, res, wt);
}

}  // namespace mitopk

namespace mitopk {

// ---------------------------------------------------------------------------
// Value order: a row's selected columns ranked from the largest value to the
// smallest, equal values by ascending column.  Each selected entry becomes
// the 64-bit composite (key << 32) | (2^32 - 1 - column), distinct per entry,
// whose descending order is exactly that ranking; the composites of a row
// are sorted in LDS by a bitonic network.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t vo_composite(uint32_t key, int32_t j) {
  return (static_cast<uint64_t>(key) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(j));
}
__device__ __forceinline__ int32_t vo_column(uint64_t c) {
  return static_cast<int32_t>(0xFFFFFFFFu - static_cast<uint32_t>(c));
}

// Sorts a[0..n) descending, n a power of two, every thread of the workgroup
// taking part (the caller synchronises before, so a[] is complete).  Thread t
// handles pairs t, t + BLOCK, ...: pair p of stride s compares elements
// i = 2p - (p mod s) and i + s.  For s <= 64 the pairs of wavefront w lie in
// its own 128-element slices ([128w, 128w + 128) + 2*BLOCK*r), the same
// slices at every such stride, so consecutive stages of stride <= 64 need
// only the wavefront's own ordering; a workgroup barrier separates a stage
// from its neighbours only where one of them has a larger stride.
template <int BLOCK>
__device__ __forceinline__ void bitonic_sort_desc(uint64_t* a, int n) {
  const int tid = static_cast<int>(threadIdx.x);
  bool prev_wide = false;
  for (int size = 2; size <= n; size <<= 1) {
    for (int s = size >> 1; s > 0; s >>= 1) {
      const bool wide = s > 64;
      if (wide || prev_wide) {
        __syncthreads();
      } else {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
      prev_wide = wide;
      for (int p = tid; p < (n >> 1); p += BLOCK) {
        const int i = ((p & ~(s - 1)) << 1) | (p & (s - 1));
        const uint64_t x = a[i], y = a[i + s];
        const bool desc = (i & size) == 0;
        if (desc ? x < y : x > y) {
          a[i] = y;
          a[i + s] = x;
        }
      }
    }
  }
  __syncthreads();
}

// comp[0..m) holds a row's selected composites (in any order): sorts them
// and writes their columns to out[0..m).  comp must hold next_pow2(m)
// entries.
template <int BLOCK>
__device__ __forceinline__ void vo_sort_store(uint64_t* comp, int m, int32_t* out) {
  if (m <= 0) return;
  int n = 1;
  while (n < m) n <<= 1;
  for (int i = m + static_cast<int>(threadIdx.x); i < n; i += BLOCK) comp[i] = 0ull;  // sorts last
  __syncthreads();
  bitonic_sort_desc<BLOCK>(comp, n);
  // (nontemporal stores: the index rows are not read again here)
  for (int i = static_cast<int>(threadIdx.x); i < m; i += BLOCK) __builtin_nontemporal_store(vo_column(comp[i]), out + i);
}

// Ranks by value the m columns this workgroup has just written to out[0..m)
// of a row (its first L entries at `row`): the values are read back from the
// row, which the workgroup has just streamed, so they come from the caches.
template <int BLOCK>
__device__ __forceinline__ void vo_rank_written(const float* row, int L, int m, int32_t* out,
                                                uint64_t* comp) {
  if (m <= 1) return;
  __syncthreads();  // the workgroup's stores to out are visible to its loads
  for (int i = static_cast<int>(threadIdx.x); i < m; i += BLOCK) {
    const int32_t j = out[i];
    const uint32_t key = (j >= 0 && j < L) ? order_key(row[j]) : 0u;
    comp[i] = vo_composite(key, j);
  }
  vo_sort_store<BLOCK>(comp, m, out);
}

}  // namespace mitopk

namespace mitopk {

// The float value of an order-preserving key (the inverse of order_key).
__device__ __forceinline__ float key_value(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : (0u - key));
}

// A monotone map from keys in [lo, hi] to 4096 bins (a larger key never gets
// a smaller bin), spreading the values of a row's selected entries evenly:
// linear in the value, (x - x_lo) * 4096 / (x_hi - x_lo), which rounding
// keeps monotone; NaN keys (above +inf, below -inf) take the end bins.  When
// a bound is infinite or the range overflows, the keys' 12-bit window below
// the bits lo and hi share is used instead (linear in the key).
struct VoBins {
  static constexpr uint32_t kKeyPosInf = 0xFF800000u;  // key of +inf
  static constexpr uint32_t kKeyNegInf = 0x00800000u;  // key of -inf
  bool linear;
  float xlo, scale;
  int s;
  uint32_t base;
  __device__ __forceinline__ VoBins(uint32_t lo, uint32_t hi) {
    xlo = key_value(lo);
    const float xhi = key_value(hi);
    const float span = xhi - xlo;
    linear = lo >= kKeyNegInf && hi <= kKeyPosInf && __builtin_isfinite(xlo) && __builtin_isfinite(xhi) &&
             __builtin_isfinite(span) && span > 0.0f;
    scale = linear ? static_cast<float>(kFirstBins) / span : 0.0f;
    s = window_shift(lo, hi);
    base = lo >> s;
  }
  __device__ __forceinline__ uint32_t operator()(uint32_t key) const {
    if (!linear) return (key >> s) - base;
    if (key > kKeyPosInf) return kFirstBins - 1;
    if (key < kKeyNegInf) return 0u;
    const float v = (key_value(key) - xlo) * scale;
    return static_cast<uint32_t>(fminf(fmaxf(v, 0.0f), static_cast<float>(kFirstBins - 1)));
  }
};

// Value order for m selected entries whose keys all lie in [lo, hi], by
// buckets instead of a sort (VoBins: 4096 bins in key order).  A count per
// bin, a suffix scan (bins from the top: each bin's first rank), a scatter
// of the composites through per-bin cursors, then each entry's rank among
// the few entries of its own bin, by comparing composites.  A bin of more
// than 64 entries (runs of equal or close values) sends the row through the
// bitonic sort of the scattered composites instead.  for_each(f) calls
// f(key, column) for each selected entry this thread holds (every entry
// once in the workgroup; called twice).  word: 4096 LDS words; comp:
// next_pow2(m) LDS composites; wt: BLOCK/64 words; res: 1 word.  Every
// thread must call it; it synchronises first, so the caller may have read
// any of these just before.
template <int BLOCK, class ForEach>
__device__ __forceinline__ void vo_bucket_rank(ForEach for_each, uint32_t lo, uint32_t hi, int m,
                                               int32_t* out, uint32_t* word, uint64_t* comp,
                                               uint32_t* wt, uint32_t* res) {
  constexpr int NB = kFirstBins;
  constexpr int NW = BLOCK / kWave;
  constexpr int GS = NB / BLOCK;  // bins per thread in the scan
  static_assert(GS >= 4 && GS % 4 == 0, "16-byte scan reads");
  const int tid = static_cast<int>(threadIdx.x);
  const VoBins bin_of(lo, hi);
  __syncthreads();
  for (int i = tid; i < NB; i += BLOCK) word[i] = 0u;
  if (tid == 0) res[0] = 0u;
  __syncthreads();
  for_each([&](uint32_t key, int32_t) { atomicAdd(&word[bin_of(key)], 1u); });
  __syncthreads();
  // thread t: bins [NB - GS(t+1), NB - GS t), the top ones first (read
  // twice rather than held, to keep registers free)
  const int top = NB - tid * GS;
  uint32_t sum = 0, mx = 0;
#pragma unroll
  for (int v = 0; v < GS / 4; ++v) {
    const uint4 q = *reinterpret_cast<const uint4*>(word + top - 4 * (v + 1));
    sum += q.x + q.y + q.z + q.w;
    mx = max(max(mx, max(q.x, q.y)), max(q.z, q.w));
  }
  const uint32_t incl = wave_inclusive_sum(sum);
  mx = wave_max(mx);
  const int w = tid / kWave;
  if ((tid & (kWave - 1)) == kWave - 1) wt[w] = incl;
  if ((tid & (kWave - 1)) == 0) atomicMax(res, mx);
  __syncthreads();
  uint32_t run = incl - sum;
#pragma unroll
  for (int v = 0; v < NW; ++v) run += v < w ? wt[v] : 0u;
#pragma unroll
  for (int v = 0; v < GS / 4; ++v) {  // each bin's first rank (bins from the top)
    uint4* at = reinterpret_cast<uint4*>(word + top - 4 * (v + 1));
    const uint4 q = *at;
    uint4 o;
    o.w = run;
    o.z = o.w + q.w;
    o.y = o.z + q.z;
    o.x = o.y + q.y;
    run = o.x + q.x;
    *at = o;
  }
  const bool heavy = res[0] > static_cast<uint32_t>(kWave);
  __syncthreads();
  for_each([&](uint32_t key, int32_t j) {
    comp[atomicAdd(&word[bin_of(key)], 1u)] = vo_composite(key, j);
  });
  if (heavy) {
    vo_sort_store<BLOCK>(comp, m, out);  // (synchronises first)
    return;
  }
  __syncthreads();
  // after the scatter word[b] is the end of bin b and word[b + 1] its start
#pragma unroll 1
  for (int q = tid; q < m; q += BLOCK) {
    const uint64_t c = comp[q];
    const uint32_t b = bin_of(static_cast<uint32_t>(c >> 32));
    const uint32_t start = b + 1 < static_cast<uint32_t>(NB) ? word[b + 1] : 0u;
    const uint32_t end = word[b];
    uint32_t r = start;
    for (uint32_t t = start; t < end; ++t) r += comp[t] > c ? 1u : 0u;
    __builtin_nontemporal_store(vo_column(c), out + r);
  }
}

}  // namespace mitopk

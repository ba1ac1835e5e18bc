// Row-wise top-k index selection kernels for gfx950 (MI355X) and the C ABI
// that launches them.
//
// Paths (chosen on the host from num_rows, row_stride and k; each row then
// branches on its own length on the device):
//   * trivial  — L_i <= k: every index 0..L_i-1, then -1.  No logits are read.
//   * row      — short rows (up to 8192 entries), one workgroup per row: the
//                row in registers as order-preserving keys, radix rounds in
//                LDS, the selected indices written in ascending order.
//   * stream   — rows of 8K-32K entries with enough rows to fill the device,
//                one workgroup per row: a sampled bound filters the row into
//                an ordered LDS list while it streams in (HBM read once), and
//                the rounds run on that list.
//   * chunks   — long rows, or too few rows to fill the device: one
//                workgroup per 16384-entry chunk publishes the chunk's
//                entries above its own sampled bound; the row's last
//                workgroup to arrive selects among them and checks that the
//                result is exact (else streams the row itself).  Ordinary
//                launch, no workgroup waits for another.
//   * split    — the same shapes with k above the chunked path's limit: G
//                workgroups per row merge digit histograms through the row
//                workspace with device-scope atomics and meet at per-row
//                barriers; the launch is cooperative, so every barrier wait
//                ends.
// The intra-row split over an 8-CTA cluster with DSMEM on the SGLang
// PR #34167 page (TopKCluster::forward) is prior art for the multi-workgroup
// paths; here the merge goes through global memory because CDNA has no
// clusters.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "mi_topk.h"
#include "select_device.hpp"
#include "wave64.hpp"

#define MI_TOPK_EXPORT extern "C" __attribute__((visibility("default")))

namespace mitopk {
namespace {

constexpr int kCandCap = 4096;     // candidate list entries (split path)
constexpr int kSortMaxK = 4096;    // largest k of a value-ordered selection (composites in LDS)
constexpr int kMaxChunks = 1024;   // workgroups per row (split path)
constexpr uint32_t kSpinLimit = 1u << 22;

struct Params {
  const float* logits;
  int64_t row_stride;
  const int32_t* lengths;
  int64_t num_rows;
  int32_t* out;
  uint8_t* ws;
  int32_t k;
  int32_t chunk;          // split: elements per chunk, a multiple of 4
  int32_t G;              // split: workgroups per row
  int32_t rows_per_iter;  // split: rows processed per pass of the grid
  // paged output (block_table == nullptr: the columns themselves)
  const int32_t* block_table;  // one row of page numbers per request
  int64_t bt_stride;           // entries between two requests' rows of block_table
  const int32_t* row_req;      // request of each row (nullptr: row i is request i)
  int32_t page;                // columns per page (>= 1)
  int32_t page_log2;           // log2(page) when page is a power of two, else -1
};

// Per-row workspace of the split path.  Every field starts at zero and is
// returned to zero by the last workgroup to leave the row.
struct RowWs {
  uint32_t bar;         // arrivals at the row's barriers
  uint32_t cand_count;  // candidate list fill
  uint32_t pad[62];
  uint32_t hist[kFirstBins + (kMaxRounds - 1) * kNextBins];  // one histogram per round
  uint32_t wg_count[kMaxChunks];                             // published per-workgroup counts
  uint64_t cand[kCandCap];                                   // (key << 32) | column
};
constexpr size_t kWsHeader = 256;  // word 0: sticky error flag
static_assert(sizeof(RowWs) % 256 == 0, "row workspace keeps 256-byte alignment");

__device__ __forceinline__ uint32_t hist_offset(int round) {
  return round == 0 ? 0u : static_cast<uint32_t>(kFirstBins + (round - 1) * kNextBins);
}

// ---- device-scope memory helpers (coherent across the XCDs' L2 caches) ----
__device__ __forceinline__ void g_add(uint32_t* p, uint32_t v) {
  __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t g_load(uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void g_store(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t g_load64(uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void g_store64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Cache-policy operand of the buffer intrinsics that gives sc1, the policy of
// the device-scope relaxed atomic loads and stores above on gfx950.
constexpr int kCoherent = 16;
// Cache-policy operand for rows streamed once: nt, the streaming hint.  A
// 537 MB read of one row per workgroup measured 6.86 TB/s with it against
// 6.12 TB/s with the default policy.  (Paths that read a row again soon
// after, from the caches, keep the default.)
constexpr int kReadOnce = 2;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Barrier among the workgroups of one row (`target` arrivals in all).
// Every access to data shared between the row's workgroups (histograms,
// counts, candidates, this counter) is a device-scope atomic, so it is
// coherent across the XCDs' L2 caches without cache write-back or
// invalidation; what the barrier must guarantee is order.  Each wavefront
// waits until its own atomics and stores have completed, the workgroup
// synchronises, and thread 0 arrives and polls the counter.  The wait is
// bounded: after kSpinLimit polls it sets the sticky error word and gives
// up, so no wave can wait forever.
__device__ __forceinline__ void row_barrier(uint32_t* bar, uint32_t target, uint32_t* err) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_add(bar, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t spins = 0;
    while (__hip_atomic_load(bar, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      __builtin_amdgcn_s_sleep(1);
      if (++spins == kSpinLimit) {
        g_store(err, 1u);
        break;
      }
    }
  }
  __syncthreads();
  asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------
// Register layout of a chunk.
//
// Thread t = 64*w + l (wavefront w, lane l) of a workgroup holds E elements.
// Its element at position u (0 <= u < E) is chunk element
//     e = w*64*E + u*64 + l,
// so every wavefront owns one contiguous stretch of 64*E elements, each of
// its load instructions reads 256 consecutive bytes, and in (wavefront,
// position, lane) order the elements are in column order.  That order is
// what lets the kernels place selected elements with a wavefront ballot and
// still write them in ascending column order.  Element e of the chunk is
// column jbase + e of the row.
// ---------------------------------------------------------------------------
struct Chunk {
  const float* base;  // element 0 of the chunk (the row start minus head, for chunk 0)
  int llo, lhi;       // valid elements [llo, lhi) of the chunk (llo <= 3)
  int32_t jbase;
};

__device__ __forceinline__ Chunk make_chunk(const float* row_ptr, int head, int64_t cbase, int llo,
                                            int lhi) {
  Chunk ch;
  ch.base = row_ptr - head + cbase;
  ch.llo = llo;
  ch.lhi = lhi;
  ch.jbase = static_cast<int32_t>(cbase - head);
  return ch;
}

__device__ __forceinline__ uint32_t wave_id() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
}

// This thread's element at position 0 (w*64*E + l), derived afresh on every
// call through an empty asm statement so that the compiler does not keep one
// position register per element alive across the callers' loops.
template <int E>
__device__ __forceinline__ int thread_elem0() {
  int e = static_cast<int>(wave_id()) * (kWave * E) + static_cast<int>(__lane_id());
  asm volatile("" : "+v"(e));
  return e;
}

// Marks positions outside [llo, lhi): fn(u, e) is called for every position
// u of a wavefront row that holds the chunk's start or end (the test is
// uniform across the wavefront for every other row), and `beyond(u)` for
// rows entirely past the end.
template <int E, class Partial, class Beyond>
__device__ __forceinline__ void for_boundary_positions(const Chunk& ch, Partial partial,
                                                       Beyond beyond) {
  const int e_wave = static_cast<int>(wave_id()) * (kWave * E);
  const int e0 = thread_elem0<E>();
#pragma unroll
  for (int u = 0; u < E; ++u) {
    const int e_first = e_wave + u * kWave;
    if (e_first >= ch.lhi) {
      beyond(u);
    } else if (e_first + kWave > ch.lhi || e_first < ch.llo) {
      partial(u, e0 + u * kWave);
    }
  }
}

// Raw float bits of entries outside the row: a negative NaN pattern whose
// key (1) is below every filter bound used here.
constexpr uint32_t kOutsideBits = 0xFFFFFFFFu;

// Loads the chunk's raw float bits.  All loads are issued before any is
// consumed (no branch between them), through a buffer resource whose bound
// is the chunk's last valid element: lanes past it read zeros without
// touching memory (the byte offset is in the range-checked vector offset).
// Positions outside [llo, lhi) then get kOutsideBits.
template <int BLOCK, int E>
__device__ __forceinline__ void load_raw(uint32_t (&raw)[E], const Chunk& ch) {
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(ch.base), 0, ch.lhi * 4, 0x00020000);
  const int e0 = static_cast<int>(wave_id()) * (kWave * E) + static_cast<int>(__lane_id());
#pragma unroll
  for (int u = 0; u < E; ++u)
    raw[u] = __builtin_amdgcn_raw_buffer_load_b32(rsrc, (e0 + u * kWave) * 4, 0, 0);
  for_boundary_positions<E>(
      ch,
      [&](int u, int e) { raw[u] = (e >= ch.llo && e < ch.lhi) ? raw[u] : kOutsideBits; },
      [&](int u) { raw[u] = kOutsideBits; });
}

// Replaces raw bits by their order-preserving keys, in place; entries
// outside the row get key 0 (decided by position, so a row value equal to
// kOutsideBits stays valid).
template <int BLOCK, int E>
__device__ __forceinline__ void keys_in_place(uint32_t (&v)[E], const Chunk& ch) {
#pragma unroll
  for (int u = 0; u < E; ++u) v[u] = order_key_bits(v[u]);
  for_boundary_positions<E>(
      ch, [&](int u, int e) { v[u] = (e >= ch.llo && e < ch.lhi) ? v[u] : 0u; },
      [&](int u) { v[u] = 0u; });
}

// The register-held chunk (keys) as a source of (key, column) entries.
// Entries outside the row hold key 0, which no prefix test accepts.
template <int BLOCK, int E>
struct RegSource {
  const uint32_t (&key)[E];
  const Chunk& ch;

  template <class F>
  __device__ __forceinline__ void operator()(F f) const {
    const int32_t j0 = ch.jbase + thread_elem0<E>();
#pragma unroll
    for (int u = 0; u < E; ++u) f(key[u], j0 + u * kWave);
  }

  // Histogram of digit d below prefix p; the first digit is counted without
  // a per-entry test on rows of the wavefront that are entirely inside the
  // chunk's valid range.
  __device__ __forceinline__ void count(const Prefix& p, int d, int ib, uint32_t rmask,
                                        uint32_t* hist) const {
    if (p.bits != 0) {
      count_digit(*this, p, d, ib, rmask, hist);
      return;
    }
    const int sh = 32 - d;
    const int e_wave = static_cast<int>(wave_id()) * (kWave * E);
#pragma unroll
    for (int u = 0; u < E; ++u) {
      const int e_first = e_wave + u * kWave;
      if (e_first >= ch.llo && e_first + kWave <= ch.lhi) {
        atomicAdd(&hist[key[u] >> sh], 1u);
      } else if (e_first < ch.lhi) {
        if (key[u] != 0u) atomicAdd(&hist[key[u] >> sh], 1u);
      }
    }
  }
};

// The n entries of an LDS candidate list, visited thread-strided.
template <int BLOCK>
struct ListSource {
  const uint64_t* list;
  int n;
  template <class F>
  __device__ __forceinline__ void operator()(F f) const {
    for (int i = threadIdx.x; i < n; i += BLOCK) {
      const uint64_t e = list[i];
      f(static_cast<uint32_t>(e >> 32), static_cast<int32_t>(static_cast<uint32_t>(e)));
    }
  }
  __device__ __forceinline__ void count(const Prefix& p, int d, int ib, uint32_t rmask,
                                        uint32_t* hist) const {
    count_digit(*this, p, d, ib, rmask, hist);
  }
};

// Per-thread selected count over the register-held chunk.
template <int BLOCK, int E, class Pred>
__device__ __forceinline__ uint32_t count_ge(const uint32_t (&key)[E], const Chunk& ch,
                                             const Pred& pred) {
  uint32_t n = 0;
  RegSource<BLOCK, E>{key, ch}([&](uint32_t kk, int32_t j) { n += pred.ge(kk, j) ? 1u : 0u; });
  return n;
}

// Offset of this wavefront's output: sum of the earlier wavefronts' counts
// (wtot: one LDS word per wavefront; contains a workgroup barrier).
template <int BLOCK>
__device__ __forceinline__ uint32_t wave_offset(uint32_t wave_count, uint32_t* wtot) {
  constexpr int NW = BLOCK / kWave;
  const uint32_t w = wave_id();
  if (__lane_id() == 0) wtot[w] = wave_count;
  __syncthreads();
  uint32_t off = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) off += (static_cast<uint32_t>(i) < w) ? wtot[i] : 0u;
  return off;
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
}

// One output row.  Slot `at` receives column j, or -1; with a page table
// (the index transform that follows the selection) column j of the row's
// request is written as its KV-cache slot table[j / page] * page + j % page,
// and -1 stays -1.
struct OutRow {
  int32_t* p;
  const int32_t* table;  // the row's request's page numbers, or nullptr
  int32_t page;
  int32_t page_log2;
  __device__ __forceinline__ int32_t map(int32_t j) const {
    if (table == nullptr || j < 0) return j;
    if (page_log2 >= 0) return (table[j >> page_log2] << page_log2) | (j & (page - 1));
    return table[j / page] * page + j % page;
  }
  __device__ __forceinline__ void put(uint32_t at, int32_t j) const { p[at] = map(j); }
};

// Writes columns staged in LDS, cols[0..n), to out_row[0..n) in order: 16
// bytes a lane when the row is 16-byte aligned and n a multiple of 4, else
// 4, with the nontemporal (streaming) store policy: interleaved with a read
// stream of the whole device, the index rows of a 4096-row batch measured
// 13.3 us of writing with the default policy against 8.3 us with this one.
// Every thread of the workgroup takes part; the caller synchronises before
// (the staging is complete).
template <int BLOCK>
__device__ __forceinline__ void write_staged(const OutRow& out_row, const int32_t* cols, uint32_t n) {
  typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
  const uint32_t tid = threadIdx.x;
  if ((reinterpret_cast<uintptr_t>(out_row.p) & 15u) == 0 && (n & 3u) == 0) {
    for (uint32_t i = 4u * tid; i < n; i += 4u * BLOCK) {
      const int4 v = *reinterpret_cast<const int4*>(cols + i);
      const i32x4 o{out_row.map(v.x), out_row.map(v.y), out_row.map(v.z), out_row.map(v.w)};
      __builtin_nontemporal_store(o, reinterpret_cast<i32x4*>(out_row.p + i));
    }
  } else {
    for (uint32_t i = tid; i < n; i += BLOCK) __builtin_nontemporal_store(out_row.map(cols[i]), out_row.p + i);
  }
}

// Writes the chunk's selected elements (pred.ge) to out_row[base ...] in
// ascending column order: a first pass counts each wavefront's selections,
// then each position's selected lanes are placed with a ballot.
template <int BLOCK, int E, class Pred>
__device__ __forceinline__ void emit_regs(const uint32_t (&key)[E], const Chunk& ch,
                                          const Pred& pred, const OutRow& out_row, uint32_t base,
                                          uint32_t limit, uint32_t* wtot) {
  const uint32_t n = count_ge<BLOCK, E>(key, ch, pred);
  uint32_t pos_wave = base + wave_offset<BLOCK>(wave_sum(n), wtot);
  const int32_t j0 = ch.jbase + thread_elem0<E>();
#pragma unroll
  for (int u = 0; u < E; ++u) {
    const int32_t j = j0 + u * kWave;
    const bool sel = pred.ge(key[u], j);
    const uint64_t m = __ballot(sel);
    const uint32_t pos = pos_wave + lanes_below(m);
    if (sel && pos < limit) out_row.put(pos, j);
    pos_wave += static_cast<uint32_t>(__popcll(m));
  }
}

// Ordered emission when the threshold key T is known but its ties are not
// resolved by index digits: every entry with key above T, and of those equal
// to T the first `ties` in column order, counted through the ballots (the
// wavefronts' counts of both kinds packed in one word, each below 2^16).
template <int BLOCK, int E>
__device__ __forceinline__ void emit_ordered_ties(const uint32_t (&key)[E], const Chunk& ch, uint32_t T,
                                                  uint32_t ties, const OutRow& out_row, uint32_t* wtot) {
  static_assert(BLOCK * E < (1 << 16), "packed counts");
  uint32_t n = 0;
#pragma unroll
  for (int u = 0; u < E; ++u) n += (key[u] > T ? 1u : 0u) + (key[u] == T ? 0x10000u : 0u);
  const uint32_t off = wave_offset<BLOCK>(wave_sum(n), wtot);
  uint32_t eq_seen = off >> 16;
  uint32_t pos = (off & 0xFFFFu) + min(eq_seen, ties);
  const int32_t j0 = ch.jbase + thread_elem0<E>();
#pragma unroll
  for (int u = 0; u < E; ++u) {
    const bool eq = key[u] == T;
    const uint64_t meq = __ballot(eq);
    const bool sel = key[u] > T || (eq && eq_seen + lanes_below(meq) < ties);
    const uint64_t m = __ballot(sel);
    if (sel) out_row.put(pos + lanes_below(m), j0 + u * kWave);
    pos += static_cast<uint32_t>(__popcll(m));
    eq_seen += static_cast<uint32_t>(__popcll(meq));
  }
}

template <int BLOCK, int E>
__device__ __forceinline__ void emit_ordered(const uint32_t (&key)[E], const Chunk& ch,
                                             const Prefix& p, int ib, const OutRow& out_row,
                                             uint32_t base, uint32_t limit, uint32_t* wtot) {
  const uint32_t rmask = (1u << ib) - 1u;
  with_pred(p, ib, rmask, [&](const auto& pred) {
    emit_regs<BLOCK, E>(key, ch, pred, out_row, base, limit, wtot);
  });
}

__device__ __forceinline__ void write_trivial(const OutRow& out_row, int L, int k, int nthreads) {
  for (int t = threadIdx.x; t < k; t += nthreads) out_row.put(static_cast<uint32_t>(t), t < L ? t : -1);
}

__device__ __forceinline__ OutRow out_row_of(const Params& p, int64_t row) {
  OutRow o;
  o.p = p.out + row * static_cast<int64_t>(p.k);
  o.table = nullptr;
  if (p.block_table != nullptr) {
    const int64_t req = p.row_req != nullptr ? static_cast<int64_t>(p.row_req[row]) : row;
    o.table = p.block_table + req * p.bt_stride;
  }
  o.page = p.page;
  o.page_log2 = p.page_log2;
  return o;
}

// ceil(a * b / c) for the sample shares of k below (c >= 1).  The product
// fits 32 bits whenever k is below about 170000, and a 32-bit division on
// the scalar unit takes a tenth of the instructions of a 64-bit one, which
// every wavefront would otherwise run on the way to its bound.
__device__ __forceinline__ uint32_t ceil_mul_div(uint32_t a, uint32_t b, uint32_t c) {
  const uint64_t num = static_cast<uint64_t>(a) * b;
  if ((num >> 32) == 0u) {
    const uint32_t n = static_cast<uint32_t>(num);
    const uint32_t q = n / c;
    return q + (q * c != n ? 1u : 0u);
  }
  return static_cast<uint32_t>((num + c - 1) / c);
}

__device__ __forceinline__ int index_bits(int L) {
  // bits needed for column indices 0..L-1 (L >= 2 here)
  return 32 - __clz(static_cast<uint32_t>(L - 1));
}

__device__ __forceinline__ int row_length(const Params& p, int64_t row) {
  const int64_t L = p.lengths[row];
  return static_cast<int>(L < 0 ? 0 : (L > p.row_stride ? p.row_stride : L));
}

// ---------------------------------------------------------------------------
// Whole row in one workgroup: sampled filter, then exact selection on the
// filtered list.
//
// Only entries at or above the m-th largest can be selected.  A sample of
// the row (4 entries per thread, spread over the row) gives a key bound LB
// such that, with a wide margin, at least k entries of the row are >= LB.
// One pass over the raw bits then copies the entries >= LB (typically
// 10-15 % of a long row) into an LDS list in column order, and the key
// transform, every radix round and the ordered emission run on that list
// instead of on the whole row.  If fewer than k entries are >= LB, or more
// than the list holds, the row is selected from the registers instead
// (always exact; only slower).
// ---------------------------------------------------------------------------
constexpr int kListPerThread = 12;

// LDS list: wavefront w's region is [w*kRegionStride, ... + count_w); each
// region is followed by one spare slot per lane, where lanes with nothing to
// store write instead (so the copy needs no branch).
constexpr int kRegion = kWave * kListPerThread;
constexpr int kRegionStride = kRegion + kWave;

template <int BLOCK>
struct __attribute__((aligned(16))) RowLds {
  uint32_t hist[kFirstBins];
  uint32_t lraw[(BLOCK / kWave) * kRegionStride];
  uint16_t lcol[(BLOCK / kWave) * kRegionStride];
  uint32_t wtot[BLOCK / kWave];
  uint32_t res[4];
};

// The filtered list, N entries per thread in registers: thread t holds list
// entries [t*per, t*per + per) (column order, per <= N); unused entries have
// key 0.
template <int N = kListPerThread>
struct RegList {
  uint32_t key[N];
  int32_t col[N];
  template <class F>
  __device__ __forceinline__ void operator()(F f) const {
#pragma unroll
    for (int u = 0; u < N; ++u) f(key[u], col[u]);
  }
  __device__ __forceinline__ void count(const Prefix& p, int d, int ib, uint32_t rmask,
                                        uint32_t* hist) const {
    count_digit(*this, p, d, ib, rmask, hist);
  }
};

// Sample-based bound.  Each thread contributes 4 entries (one from each
// quarter of its positions); the bound is the lower edge of the first-digit
// bin where the sample's count from the top reaches 5/4 of its share of k
// plus 8.  Returns a key >= 2.
template <int BLOCK, int E>
__device__ __forceinline__ uint32_t sample_bound(const uint32_t (&raw)[E], int L, int k,
                                                 RowLds<BLOCK>& lds) {
  const int tid = threadIdx.x;
  for (int i = tid; i < kFirstBins; i += BLOCK) lds.hist[i] = 0;
  __syncthreads();
#pragma unroll
  for (int qd = 0; qd < 4; ++qd) {
    const uint32_t key = order_key_bits(raw[qd * E / 4]);
    if (key > 1u) atomicAdd(&lds.hist[key >> (32 - kFirstBits)], 1u);
  }
  __syncthreads();
  if (tid < kWave) {
    if (tid == 0) lds.res[0] = 0u;  // no bound unless the sample is large enough
    // from the sample size ns, need_s = ceil(5 k ns / 4 L) + 8
    find_bucket_wave_nb<kFirstBins>(
        lds.hist,
        [&](uint32_t ns) {
          return ceil_mul_div(5u * static_cast<uint32_t>(k), ns, 4u * static_cast<uint32_t>(L)) + 8u;
        },
        lds.res);
  }
  __syncthreads();
  const uint32_t lb = lds.res[0] << (32 - kFirstBits);
  return lb < 2u ? 2u : lb;
}

// Copies the entries whose key is >= lb (tested on the raw bits) into
// wavefront w's region of the LDS list, in column order, and returns the
// wavefront's count (entries past the region's size are counted, not
// stored).  For lb <= 0x80000000 a value passes iff its bits, unsigned, are
// <= 2^32 - lb; above that, iff its bits, signed, are >= the bound's bits.
template <int BLOCK, int E, bool kPositiveBound>
__device__ __forceinline__ uint32_t filter_wave(const uint32_t (&raw)[E], const Chunk& ch,
                                                uint32_t lb, RowLds<BLOCK>& lds) {
  const uint32_t w = wave_id();
  uint32_t* rraw = lds.lraw + w * kRegionStride;
  uint16_t* rcol = lds.lcol + w * kRegionStride;
  const uint32_t spare = kRegion + __lane_id();
  const uint32_t ulim = 0u - lb;
  const int32_t slim = static_cast<int32_t>(lb & 0x7FFFFFFFu);
  const int32_t j0 = ch.jbase + thread_elem0<E>();
  uint32_t cnt = 0;
#pragma unroll
  for (int u = 0; u < E; ++u) {
    const uint32_t x = raw[u];
    const bool hit = kPositiveBound ? static_cast<int32_t>(x) >= slim : x <= ulim;
    const uint64_t m = __ballot(hit);
    const uint32_t pos = cnt + lanes_below(m);
    const uint32_t a = (hit && pos < static_cast<uint32_t>(kRegion)) ? pos : spare;
    rraw[a] = x;
    rcol[a] = static_cast<uint16_t>(j0 + u * kWave);
    cnt += static_cast<uint32_t>(__popcll(m));
  }
  return cnt;
}

// Exact selection of a whole row held by this workgroup (L > k), with the
// selected columns written to out_row in ascending order.
template <int BLOCK, int E>
__device__ __forceinline__ void select_row(uint32_t (&raw)[E], const Chunk& ch, int L, int k,
                                           const OutRow& out_row, RowLds<BLOCK>& lds) {
  constexpr int NW = BLOCK / kWave;
  const int ib = index_bits(L);
  const uint32_t rmask = (1u << ib) - 1u;
  const uint32_t kk = static_cast<uint32_t>(k);
  bool done = false;
  const bool sampled = L >= 4 * k;
  if (sampled) {
    const uint32_t lb = sample_bound<BLOCK, E>(raw, L, k, lds);
    const uint32_t cw = lb > 0x80000000u ? filter_wave<BLOCK, E, true>(raw, ch, lb, lds)
                                         : filter_wave<BLOCK, E, false>(raw, ch, lb, lds);
    if (__lane_id() == 0) lds.wtot[wave_id()] = cw;
    __syncthreads();
    uint32_t total = 0, over = 0;
    uint32_t pre[NW];
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const uint32_t c = lds.wtot[i];
      pre[i] = total;
      total += c;
      over |= c > static_cast<uint32_t>(kRegion) ? 1u : 0u;
    }
    if (!over && total >= kk) {
      // the list in registers: entry i of the concatenated regions is at
      // region w(i), offset i - pre[w(i)]
      const uint32_t per = (total + BLOCK - 1) / BLOCK;
      const uint32_t first = threadIdx.x * per;
      RegList<> lst;
#pragma unroll
      for (int u = 0; u < kListPerThread; ++u) {
        const uint32_t i = first + u;
        uint32_t rw = 0, rp = 0;
#pragma unroll
        for (int r = 1; r < NW; ++r) {
          if (i >= pre[r]) {
            rw = r;
            rp = pre[r];
          }
        }
        const bool ok = static_cast<uint32_t>(u) < per && i < total;
        const uint32_t a = rw * kRegionStride + (i - rp);
        lst.key[u] = ok ? order_key_bits(lds.lraw[a]) : 0u;
        lst.col[u] = ok ? static_cast<int32_t>(lds.lcol[a]) : 0;
      }
      const Prefix pf = rounds_local<BLOCK>(lst, Prefix{0, 0u, 0u}, kk, ib, lds.hist, lds.res, lds.wtot);
      with_pred(pf, ib, rmask, [&](const auto& pred) {
        uint32_t n = 0;
#pragma unroll
        for (int u = 0; u < kListPerThread; ++u) n += pred.ge(lst.key[u], lst.col[u]) ? 1u : 0u;
        const uint32_t incl = wave_inclusive_sum(n);
        const uint32_t wtotal =
            static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(incl), 63));
        uint32_t pos = wave_offset<BLOCK>(wtotal, lds.wtot) + incl - n;
#pragma unroll
        for (int u = 0; u < kListPerThread; ++u) {
          if (pred.ge(lst.key[u], lst.col[u])) {
            if (pos < kk) out_row.put(pos, lst.col[u]);
            ++pos;
          }
        }
      });
      done = true;
    }
    __syncthreads();  // LDS is reused below
  }
  if (!done) {
    // the row is read again rather than kept in registers through the list
    // phase, which would otherwise spill
    if (sampled) load_raw<BLOCK, E>(raw, ch);
    keys_in_place<BLOCK, E>(raw, ch);
    const Prefix pf =
        rounds_local<BLOCK>(RegSource<BLOCK, E>{raw, ch}, Prefix{0, 0u, 0u}, kk, ib, lds.hist, lds.res, lds.wtot);
    emit_ordered<BLOCK, E>(raw, ch, pf, ib, out_row, 0u, kk, lds.wtot);
  }
}

// ---------------------------------------------------------------------------
// Local path: one workgroup per row, whole row in registers.
// ---------------------------------------------------------------------------
// Two workgroups per CU (4 wavefronts per SIMD) let one workgroup's loads
// overlap the other's selection.
// VO: the selected columns leave ranked by value (their composites sorted in
// LDS) instead of in ascending column order.
template <int BLOCK, int E, bool VO>
__device__ __forceinline__ void row_item(const Params& p, int64_t row) {
  __shared__ RowLds<BLOCK> lds;
  static_assert(sizeof(RowLds<BLOCK>) >= 8 * kSortMaxK, "composites of a row fit the LDS");
  const int L = row_length(p, row);
  const OutRow out_row = out_row_of(p, row);
  const float* row_ptr = p.logits + row * p.row_stride;
  uint64_t* comp = reinterpret_cast<uint64_t*>(&lds);
  if (L <= p.k) {
    write_trivial(out_row, L, p.k, BLOCK);
    if constexpr (VO) vo_rank_written<BLOCK>(row_ptr, L, L, out_row.p, comp);
    return;
  }
  const int head = static_cast<int>((reinterpret_cast<uintptr_t>(row_ptr) >> 2) & 3u);
  const Chunk ch = make_chunk(row_ptr, head, 0, head, head + L);
  uint32_t raw[E];
  load_raw<BLOCK, E>(raw, ch);
  select_row<BLOCK, E>(raw, ch, L, p.k, out_row, lds);
  if constexpr (VO) vo_rank_written<BLOCK>(row_ptr, L, p.k, out_row.p, comp);
}

// One workgroup per row; PERSIST: a fixed grid whose workgroups take rows
// blockIdx.x, blockIdx.x + gridDim.x, ... (the launch does not depend on the
// batch).
template <int BLOCK, int E, bool VO, bool PERSIST>
__global__ void __launch_bounds__(BLOCK) __attribute__((amdgpu_waves_per_eu(4)))
topk_row_kernel(Params p) {
  if constexpr (PERSIST) {
    for (int64_t row = blockIdx.x; row < p.num_rows; row += gridDim.x) {
      row_item<BLOCK, E, VO>(p, row);
      __syncthreads();  // the LDS is reused by the next row
    }
  } else {
    row_item<BLOCK, E, VO>(p, blockIdx.x);
  }
}

// ---------------------------------------------------------------------------
// Streaming row kernel: one workgroup per row, the row streamed through
// registers instead of held in them.
//
// Wavefront w owns the contiguous stretch [w*S, (w+1)*S) of the row's span
// (S = 64*NP elements) and reads it in chunks of 16 positions (lane l's
// position u is element w*S + u*64 + l, so each load instruction reads 256
// consecutive bytes), alternating between two 16-word register buffers so
// that the next chunk is in flight while the current one is filtered.  The
// sample that fixes the filter bound is read first (one word at the start of
// each quarter of the stretch), and its histogram search runs while the
// first two chunks arrive.  Each wavefront then filters its own stretch into
// its own LDS region, in column order, with no workgroup barrier until the
// stretch is done.  80 registers and a 48 KB LDS footprint (the histogram
// shares memory with the list) let three workgroups share a CU.
//
// Rows that the sample does not settle (fewer than k entries pass, or a
// region overflows), rows shorter than 4k, and rows too short to be worth
// sampling are selected exactly by radix rounds that read the row again from
// memory (or, for a row of at most 16 positions per thread, from registers).
// ---------------------------------------------------------------------------
constexpr int kChunkPos = 16;     // positions per chunk, per thread
constexpr int kStreamBufs = 2;    // chunks in flight per wavefront
constexpr int kStreamRegion = 768;  // list entries per wavefront

// List entry i of wavefront w: raw bits at list[w*kStreamRegion + i], column
// at list[kListCols + w*kStreamRegion + i] (one address, two constant offsets).
template <int BLOCK>
struct __attribute__((aligned(16))) StreamLds {
  static constexpr int kListCols = (BLOCK / kWave) * kStreamRegion;
  union {
    uint32_t hist[kFirstBins];
    uint32_t list[2 * kListCols];
  } u;
  uint32_t wtot[BLOCK / kWave];
  uint32_t res[4];
};

// The row as read from memory in the streaming layout (NP positions per
// thread); entries outside the row carry key 0.
template <int BLOCK, int NP>
struct StreamGeom {
  __amdgpu_buffer_rsrc_t rsrc;
  int llo, lhi;
  int32_t jbase;

  static constexpr int kStretch = kWave * NP;
  static constexpr int kChunks = NP / kChunkPos;

  __device__ __forceinline__ StreamGeom(const Chunk& ch)
      : rsrc(__builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(ch.base), 0, ch.lhi * 4,
                                               0x00020000)),
        llo(ch.llo), lhi(ch.lhi), jbase(ch.jbase) {}

  // first element of this wavefront's chunk c (uniform)
  __device__ __forceinline__ int chunk_first(int c) const {
    return static_cast<int>(wave_id()) * kStretch + c * (kChunkPos * kWave);
  }
  __device__ __forceinline__ bool chunk_live(int c) const { return chunk_first(c) < lhi; }

  // this thread's element at position 0 of chunk c
  __device__ __forceinline__ int elem(int c) const {
    int e = chunk_first(c) + static_cast<int>(__lane_id());
    asm volatile("" : "+v"(e));
    return e;
  }

  // Issues the loads of chunk c (positions past lhi read zeros, no memory access).
  __device__ __forceinline__ void load(uint32_t (&buf)[kChunkPos], int c) const {
    const int e = elem(c);
#pragma unroll
    for (int u = 0; u < kChunkPos; ++u)
      buf[u] = __builtin_amdgcn_raw_buffer_load_b32(rsrc, (e + u * kWave) * 4, 0, kReadOnce);
  }

  // True if every position of chunk c lies inside [llo, lhi) (uniform).
  __device__ __forceinline__ bool chunk_inside(int c) const {
    const int first = chunk_first(c);
    return first >= llo && first + kChunkPos * kWave <= lhi;
  }

  // Replaces the words of positions outside [llo, lhi) by `outside`; only
  // chunks that hold the row's start or end are touched (a uniform branch).
  __device__ __forceinline__ void mask_edges(uint32_t (&buf)[kChunkPos], int c,
                                             uint32_t outside) const {
    if (chunk_inside(c)) return;
    const int e = elem(c);
#pragma unroll
    for (int u = 0; u < kChunkPos; ++u) {
      const int eu = e + u * kWave;
      buf[u] = (eu >= llo && eu < lhi) ? buf[u] : outside;
    }
  }

  // (key, column) source over the whole row, read from memory chunk by chunk.
  template <class F>
  __device__ __forceinline__ void operator()(F f) const {
#pragma unroll 1
    for (int c = 0; c < kChunks; ++c) {
      if (!chunk_live(c)) break;
      uint32_t buf[kChunkPos];
      load(buf, c);
#pragma unroll
      for (int u = 0; u < kChunkPos; ++u) buf[u] = order_key_bits(buf[u]);
      mask_edges(buf, c, 0u);
      const int32_t j0 = jbase + elem(c);
#pragma unroll
      for (int u = 0; u < kChunkPos; ++u) f(buf[u], j0 + u * kWave);
    }
  }
  __device__ __forceinline__ void count(const Prefix& p, int d, int ib, uint32_t rmask,
                                        uint32_t* hist) const {
    count_digit(*this, p, d, ib, rmask, hist);
  }
};

// Exact selection over the row read from memory: radix rounds, then an
// ordered emission (a counting pass for each wavefront's offset, then one
// ballot per position).
template <int BLOCK, int NP>
__device__ __forceinline__ void select_stream_exact(const StreamGeom<BLOCK, NP>& g, int L, int k,
                                                    const OutRow& out_row, StreamLds<BLOCK>& lds) {
  const int ib = index_bits(L);
  const uint32_t rmask = (1u << ib) - 1u;
  const uint32_t kk = static_cast<uint32_t>(k);
  const Prefix pf = rounds_local<BLOCK>(g, Prefix{0, 0u, 0u}, kk, ib, lds.u.hist, lds.res, lds.wtot);
  with_pred(pf, ib, rmask, [&](const auto& pred) {
    uint32_t n = 0;
    g([&](uint32_t key, int32_t j) { n += pred.ge(key, j) ? 1u : 0u; });
    uint32_t pos_wave = wave_offset<BLOCK>(wave_sum(n), lds.wtot);
#pragma unroll 1
    for (int c = 0; c < StreamGeom<BLOCK, NP>::kChunks; ++c) {
      if (!g.chunk_live(c)) break;
      uint32_t buf[kChunkPos];
      g.load(buf, c);
#pragma unroll
      for (int u = 0; u < kChunkPos; ++u) buf[u] = order_key_bits(buf[u]);
      g.mask_edges(buf, c, 0u);
      const int32_t j0 = g.jbase + g.elem(c);
#pragma unroll
      for (int u = 0; u < kChunkPos; ++u) {
        const int32_t j = j0 + u * kWave;
        const bool sel = pred.ge(buf[u], j);
        const uint64_t m = __ballot(sel);
        const uint32_t pos = pos_wave + lanes_below(m);
        if (sel && pos < kk) out_row.put(pos, j);
        pos_wave += static_cast<uint32_t>(__popcll(m));
      }
    }
  });
}

// Filters one chunk into this wavefront's LDS region; cnt counts every
// entry that passed.  A position's hits are stored only if all of them fit
// (a uniform test), so a region that overflows ends with cnt above its size.
// kEdge: the chunk holds the row's end; positions past it are read as
// kOutsideBits (the buffer itself is not modified).
template <int BLOCK, int NP, bool kPositiveBound, bool kEdge>
__device__ __forceinline__ void filter_chunk(const StreamGeom<BLOCK, NP>& g,
                                             const uint32_t (&buf)[kChunkPos], int c, uint32_t lb,
                                             uint32_t* region, uint32_t& cnt) {
  constexpr int kCols = StreamLds<BLOCK>::kListCols;
  const uint32_t ulim = 0u - lb;
  const int32_t slim = static_cast<int32_t>(lb & 0x7FFFFFFFu);
  const int32_t j0 = g.jbase + g.elem(c);
#pragma unroll
  for (int u = 0; u < kChunkPos; ++u) {
    const uint32_t x = !kEdge || j0 + u * kWave < g.jbase + g.lhi ? buf[u] : kOutsideBits;
    const bool hit = kPositiveBound ? static_cast<int32_t>(x) >= slim : x <= ulim;
    const uint64_t m = __ballot(hit);
    const uint32_t n = static_cast<uint32_t>(__popcll(m));
    if (cnt + n <= static_cast<uint32_t>(kStreamRegion)) {
      if (hit) {
        const uint32_t pos = __builtin_amdgcn_mbcnt_hi(
            static_cast<uint32_t>(m >> 32), __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), cnt));
        region[pos] = x;
        region[kCols + pos] = static_cast<uint32_t>(j0 + u * kWave);
      }
    }
    cnt += n;
  }
}

// Streams the wavefront's stretch through kStreamBufs register buffers:
// chunk c + kStreamBufs is loaded into the buffer that chunk c has just been
// filtered from.  The first kStreamBufs chunks were issued by the caller.
template <int BLOCK, int NP, bool kPositiveBound>
__device__ __forceinline__ uint32_t filter_stream(const StreamGeom<BLOCK, NP>& g,
                                                  uint32_t (&bufs)[kStreamBufs][kChunkPos],
                                                  uint32_t lb, StreamLds<BLOCK>& lds) {
  constexpr int NCH = StreamGeom<BLOCK, NP>::kChunks;
  uint32_t* region = lds.u.list + wave_id() * kStreamRegion;
  uint32_t cnt = 0;
  // the row starts at element 0, so only the chunk holding its end is partial
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    if (g.chunk_inside(c)) {
      filter_chunk<BLOCK, NP, kPositiveBound, false>(g, bufs[c % kStreamBufs], c, lb, region, cnt);
    } else if (g.chunk_live(c)) {
      filter_chunk<BLOCK, NP, kPositiveBound, true>(g, bufs[c % kStreamBufs], c, lb, region, cnt);
    }
    // issued even for chunks past the row's end (they read nothing): a load
    // behind a branch makes every later wait for the buffers conservative
    if (c + kStreamBufs < NCH) g.load(bufs[c % kStreamBufs], c + kStreamBufs);
  }
  return cnt;
}

// The streaming kernel's selection from its filtered list (each wavefront's
// cw entries in its LDS region, keys in [lb, ...]): the list in registers, N
// entries a thread, a windowed radix round, and the ordered emission.
template <int BLOCK, int N, bool VO>
__device__ __forceinline__ void stream_list_select(const Params& p, StreamLds<BLOCK>& lds, uint32_t cw,
                                                   uint32_t lb, int L, const OutRow& out_row,
                                                   const float* row_ptr, uint64_t* comp) {
  static_assert(N % 4 == 0 && N <= kListPerThread, "16-byte LDS reads");
  const int tid = threadIdx.x;
  const uint32_t w = wave_id();
  const uint32_t kk = static_cast<uint32_t>(p.k);
  const int ib = index_bits(L);
  const uint32_t rmask = (1u << ib) - 1u;
  // lane l takes entries [l*per, l*per+per) of its wavefront's region, per a
  // multiple of 4 (16-byte LDS reads)
  RegList<N> lst;
  {
    constexpr int kCols = StreamLds<BLOCK>::kListCols;
    const uint32_t per = (((cw + kWave - 1) / kWave) + 3u) & ~3u;
    const uint32_t first = __lane_id() * per;
    const uint32_t* region = lds.u.list + w * kStreamRegion;
#pragma unroll
    for (int q = 0; q < N / 4; ++q) {
      const uint32_t i0 = first + 4u * q;
      uint4 r = make_uint4(0u, 0u, 0u, 0u), c = make_uint4(0u, 0u, 0u, 0u);
      if (4u * q < per) {
        r = *reinterpret_cast<const uint4*>(region + i0);
        c = *reinterpret_cast<const uint4*>(region + kCols + i0);
      }
      const uint32_t rv[4] = {r.x, r.y, r.z, r.w};
      const uint32_t cv[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const bool ok = 4u * q + t < per && i0 + t < cw;
        lst.key[4 * q + t] = ok ? order_key_bits(rv[t]) : 0u;
        lst.col[4 * q + t] = static_cast<int32_t>(cv[t]);
      }
    }
    uint32_t mx = 0;
#pragma unroll
    for (int u = 0; u < N; ++u) mx = max(mx, lst.key[u]);
    mx = wave_max(mx);
    if (__lane_id() == 0) atomicMax(&lds.res[3], mx);
  }
  __syncthreads();  // the list's LDS becomes the histogram
  // every listed key lies in [lb, largest]
  const uint32_t kmax = lds.res[3];
  const Prefix pf = rounds_window<BLOCK>(lst, lb, kmax, kk, ib, lds.u.hist, lds.res, lds.wtot);
  // VO: with k <= 2048 the selected composites are staged in LDS at their
  // column-order ranks (the list's registers end here) and ranked by value
  // from there: union words [0, 16 KB) bins, [16, 32) staging, [32, 48) the
  // scattered composites.  A larger k ranks the written row instead.
  constexpr int kVoStage = kFirstBins / 2;
  uint64_t* const stage = comp + kVoStage;
  const bool vo_lds = VO && p.k <= kVoStage;
  // Otherwise the selected columns are staged in LDS at their ranks and
  // written out in order: a lane's selected entries are a run of ranks, so
  // storing them directly would spread each store instruction's 64 lanes
  // over the whole output row.  (The list holds at most 6144 entries, so k
  // fits the union's 12288 words.)
  int32_t* const cols = reinterpret_cast<int32_t*>(lds.u.list);
  with_pred(pf, ib, rmask, [&](const auto& pred) {
    uint32_t n = 0;
#pragma unroll
    for (int u = 0; u < N; ++u) n += pred.ge(lst.key[u], lst.col[u]) ? 1u : 0u;
    const uint32_t incl = wave_inclusive_sum(n);
    const uint32_t wtotal =
        static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(incl), 63));
    uint32_t pos = wave_offset<BLOCK>(wtotal, lds.wtot) + incl - n;
#pragma unroll
    for (int u = 0; u < N; ++u) {
      if (pred.ge(lst.key[u], lst.col[u])) {
        if (pos < kk) {
          if (vo_lds) {
            stage[pos] = vo_composite(lst.key[u], lst.col[u]);
          } else {
            cols[pos] = lst.col[u];
          }
        }
        ++pos;
      }
    }
  });
  if (!vo_lds) {
    __syncthreads();  // the staged columns are complete
    write_staged<BLOCK>(out_row, cols, kk);
  }
  if constexpr (VO) {
    if (vo_lds) {
      __syncthreads();  // the staged composites are complete
      const int m = p.k;
      vo_bucket_rank<BLOCK>(
          [&](auto f) {
#pragma unroll 1
            for (int i = tid; i < m; i += BLOCK) {
              const uint64_t c = stage[i];
              f(static_cast<uint32_t>(c >> 32), vo_column(c));
            }
          },
          prefix_edge(pf), kmax, m, out_row.p, lds.u.hist, comp + 2 * kVoStage, lds.wtot, lds.res);
    } else {
      vo_rank_written<BLOCK>(row_ptr, L, p.k, out_row.p, comp);
    }
  }
}

template <int BLOCK, int NP, bool VO>
__device__ __forceinline__ void stream_item(const Params& p, int64_t row) {
  constexpr int NW = BLOCK / kWave;
  __shared__ StreamLds<BLOCK> lds;
  // composites of a row; their bucket ranking: bins, staging, scatter (16 KB each)
  static_assert(sizeof(lds.u) >= 8 * kSortMaxK && sizeof(lds.u) >= 12 * kFirstBins,
                "composites of a row fit the LDS");
  uint64_t* comp = reinterpret_cast<uint64_t*>(lds.u.list);
  const int L = row_length(p, row);
  const OutRow out_row = out_row_of(p, row);
  const float* row_ptr = p.logits + row * p.row_stride;
  if (L <= p.k) {
    write_trivial(out_row, L, p.k, BLOCK);
    if constexpr (VO) vo_rank_written<BLOCK>(row_ptr, L, L, out_row.p, comp);
    return;
  }
  // word loads need no 16-byte alignment, so the row starts at element 0
  const Chunk ch = make_chunk(row_ptr, 0, 0, 0, L);
  const int ib = index_bits(L);
  const uint32_t kk = static_cast<uint32_t>(p.k);
  const int tid = threadIdx.x;

  if (ch.lhi <= BLOCK * kChunkPos) {
    // the whole row in 16 registers per thread
    uint32_t key[kChunkPos];
    load_raw<BLOCK, kChunkPos>(key, ch);
    keys_in_place<BLOCK, kChunkPos>(key, ch);
    const Prefix pf = rounds_local<BLOCK>(RegSource<BLOCK, kChunkPos>{key, ch}, Prefix{0, 0u, 0u},
                                          kk, ib, lds.u.hist, lds.res, lds.wtot);
    emit_ordered<BLOCK, kChunkPos>(key, ch, pf, ib, out_row, 0u, kk, lds.wtot);
    if constexpr (VO) vo_rank_written<BLOCK>(row_ptr, L, p.k, out_row.p, comp);
    return;
  }
  const StreamGeom<BLOCK, NP> g(ch);
  if (L < 4 * p.k) {
    select_stream_exact<BLOCK, NP>(g, L, p.k, out_row, lds);
    if constexpr (VO) vo_rank_written<BLOCK>(row_ptr, L, p.k, out_row.p, comp);
    return;
  }

  // sample (one word at the start of each quarter of the stretch), then the
  // first two chunks
  constexpr int QS = NP / 4;
  uint32_t smp[4];
  {
    const int e = g.elem(0);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      smp[q] = __builtin_amdgcn_raw_buffer_load_b32(g.rsrc, (e + q * QS * kWave) * 4, 0, kReadOnce);
  }
  uint32_t bufs[kStreamBufs][kChunkPos];
#pragma unroll
  for (int c = 0; c < kStreamBufs; ++c)
    if (c < StreamGeom<BLOCK, NP>::kChunks) g.load(bufs[c], c);

  for (int i = tid; i < kFirstBins; i += BLOCK) lds.u.hist[i] = 0;
  __syncthreads();
  {
    const int e = g.elem(0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int eq = e + q * QS * kWave;
      const uint32_t key = order_key_bits(smp[q]);
      if (eq >= g.llo && eq < g.lhi && key > 1u) atomicAdd(&lds.u.hist[key >> (32 - kFirstBits)], 1u);
    }
  }
  __syncthreads();
  if (tid == 0) lds.res[0] = 0u;
  find_bucket_block<BLOCK, kFirstBins>(
      lds.u.hist,
      [&](uint32_t ns) {
        return ceil_mul_div(5u * kk, ns, 4u * static_cast<uint32_t>(L)) + 8u;
      },
      lds.res, lds.wtot);
  __syncthreads();
  uint32_t lb = lds.res[0] << (32 - kFirstBits);
  lb = lb < 2u ? 2u : lb;

  const uint32_t cw = lb > 0x80000000u ? filter_stream<BLOCK, NP, true>(g, bufs, lb, lds)
                                       : filter_stream<BLOCK, NP, false>(g, bufs, lb, lds);
  const uint32_t w = wave_id();
  if (__lane_id() == 0) lds.wtot[w] = cw;
  if (tid == 0) lds.res[3] = 0u;  // the list's largest key, below
  __syncthreads();
  uint32_t total = 0, over = 0, maxcw = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const uint32_t c = lds.wtot[i];
    total += c;
    maxcw = max(maxcw, c);
    over |= c > static_cast<uint32_t>(kStreamRegion) ? 1u : 0u;
  }
  if (over || total < kk) {
    __syncthreads();  // wtot is reused
    select_stream_exact<BLOCK, NP>(g, L, p.k, out_row, lds);
    if constexpr (VO) vo_rank_written<BLOCK>(row_ptr, L, p.k, out_row.p, comp);
    return;
  }

  // the lists in registers: N entries a thread, the fewest that hold the
  // longest wavefront list (a lane takes a multiple of 4 entries)
  if (maxcw <= 8u * kWave) {
    stream_list_select<BLOCK, 8, VO>(p, lds, cw, lb, L, out_row, row_ptr, comp);
  } else {
    stream_list_select<BLOCK, kListPerThread, VO>(p, lds, cw, lb, L, out_row, row_ptr, comp);
  }
}

template <int BLOCK, int NP, bool VO, bool PERSIST>
__global__ void __launch_bounds__(BLOCK) __attribute__((amdgpu_waves_per_eu(6)))
topk_stream_kernel(Params p) {
  if constexpr (PERSIST) {
    for (int64_t row = blockIdx.x; row < p.num_rows; row += gridDim.x) {
      stream_item<BLOCK, NP, VO>(p, row);
      __syncthreads();  // the LDS is reused by the next row
    }
  } else {
    stream_item<BLOCK, NP, VO>(p, blockIdx.x);
  }
}

// ---------------------------------------------------------------------------
// Split path: G workgroups per row, merged through the row workspace.
// ---------------------------------------------------------------------------

// Sum over the workgroup of one value per thread (every thread gets it).
template <int BLOCK>
__device__ __forceinline__ uint32_t block_sum(uint32_t x, uint32_t* wtot) {
  const uint32_t ws = wave_sum(x);
  const uint32_t w = wave_id();
  if (__lane_id() == 0) wtot[w] = ws;
  __syncthreads();
  uint32_t t = 0;
#pragma unroll
  for (int i = 0; i < BLOCK / kWave; ++i) t += wtot[i];
  __syncthreads();
  return t;
}

template <int BLOCK, int E>
__device__ __forceinline__ void select_chunk_whole_row(const uint32_t (&key)[E], const Chunk& ch,
                                                       int L, int k, const OutRow& out_row,
                                                       uint32_t* hist, uint32_t* wtot,
                                                       uint32_t* res) {
  const int ib = index_bits(L);
  const uint32_t kk = static_cast<uint32_t>(k);
  uint32_t ties = 0xFFFFFFFFu;  // set when the key is known and its ties are left to the emission
  const Prefix pf = rounds_local<BLOCK>(RegSource<BLOCK, E>{key, ch}, Prefix{0, 0u, 0u}, kk, ib, hist, res,
                                        wtot, &ties);
  if (ties != 0xFFFFFFFFu) {
    emit_ordered_ties<BLOCK, E>(key, ch, pf.kp, ties, out_row, wtot);
  } else {
    emit_ordered<BLOCK, E>(key, ch, pf, ib, out_row, 0u, kk, wtot);
  }
}

// Two 512-thread workgroups per CU, so that up to 512 chunks are co-resident.
template <int BLOCK, int E>
__global__ void __launch_bounds__(BLOCK) __attribute__((amdgpu_waves_per_eu(4)))
topk_split_kernel(Params p) {
  __shared__ __attribute__((aligned(16))) uint32_t hist[kFirstBins];
  __shared__ uint64_t cand[kCandCap];
  __shared__ uint32_t csel[kMaxChunks];
  __shared__ uint32_t wtot[BLOCK / kWave];
  __shared__ uint32_t res[4];
  const int tid = threadIdx.x;
  const int G = p.G;
  uint32_t* err = reinterpret_cast<uint32_t*>(p.ws);
  RowWs* ws_rows = reinterpret_cast<RowWs*>(p.ws + kWsHeader);

  for (int64_t row0 = 0; row0 < p.num_rows; row0 += p.rows_per_iter) {
    __syncthreads();  // LDS is reused from the previous row
    const int64_t row = row0 + blockIdx.x / G;
    if (row >= p.num_rows) break;
    const int g = blockIdx.x % G;
    const int L = row_length(p, row);
    const OutRow out_row = out_row_of(p, row);
    if (L <= p.k) {
      if (g == 0) write_trivial(out_row, L, p.k, BLOCK);
      continue;
    }
    const float* row_ptr = p.logits + row * p.row_stride;
    const int head = static_cast<int>((reinterpret_cast<uintptr_t>(row_ptr) >> 2) & 3u);
    const int64_t span = static_cast<int64_t>(head) + L;
    const int Gr = static_cast<int>((span + p.chunk - 1) / p.chunk);
    if (g >= Gr) continue;
    const int64_t cbase = static_cast<int64_t>(g) * p.chunk;
    const Chunk ch = make_chunk(row_ptr, head, cbase, g == 0 ? head : 0,
                                static_cast<int>(span - cbase < p.chunk ? span - cbase : p.chunk));
    uint32_t key[E];
    load_raw<BLOCK, E>(key, ch);
    keys_in_place<BLOCK, E>(key, ch);
    if (Gr == 1) {
      select_chunk_whole_row<BLOCK, E>(key, ch, L, p.k, out_row, hist, wtot, res);
      continue;
    }

    RowWs* ws = ws_rows + row;
    const int ib = index_bits(L);
    const uint32_t rmask = (1u << ib) - 1u;
    const RegSource<BLOCK, E> regs{key, ch};
    const uint32_t nwg = static_cast<uint32_t>(Gr);
    uint32_t need = static_cast<uint32_t>(p.k);
    Prefix pr{0, 0u, 0u};
    uint32_t nbar = 0;
    int round = 0;
    bool use_cand = false;
    uint32_t cnt = 0;
    // Global rounds: histogram the chunk, merge, wait for the row, search.
    for (; round < kMaxRounds; ++round) {
      const int d = digit_bits(pr.bits, ib);
      const int nb = 1 << d;
      for (int i = tid; i < nb; i += BLOCK) hist[i] = 0;
      __syncthreads();
      regs.count(pr, d, ib, rmask, hist);
      __syncthreads();
      uint32_t* gh = ws->hist + hist_offset(round);
      for (int i = tid; i < nb; i += BLOCK) {
        const uint32_t h = hist[i];
        if (h != 0) g_add(&gh[i], h);
      }
      row_barrier(&ws->bar, ++nbar * nwg, err);
      for (int i = tid; i < nb; i += BLOCK) hist[i] = g_load(&gh[i]);
      __syncthreads();
      if (tid < kWave) find_bucket_wave(hist, nb, need, res);
      __syncthreads();
      const uint32_t b = res[0], gt = res[1];
      cnt = res[2];
      need -= gt;
      pr = extend(pr, d, b);
      if (cnt == need) break;
      if (cnt <= static_cast<uint32_t>(kCandCap)) {
        use_cand = true;
        break;
      }
    }
    const int rounds_used = round + 1;

    Prefix pf = pr;
    uint32_t off = 0;
    if (!use_cand) {
      // The prefix alone decides the set; publish counts for the output offsets.
      uint32_t n = 0;
      with_pred(pf, ib, rmask, [&](const auto& pred) { n = count_ge<BLOCK, E>(key, ch, pred); });
      const uint32_t total = block_sum<BLOCK>(n, wtot);
      if (tid == 0) g_store(&ws->wg_count[g], total);
      row_barrier(&ws->bar, ++nbar * nwg, err);
      uint32_t part = 0;
      for (int i = tid; i < g; i += BLOCK) part += g_load(&ws->wg_count[i]);
      off = block_sum<BLOCK>(part, wtot);
    } else {
      // Entries above the bucket are taken; the bucket's entries go to the
      // row's candidate list, which every workgroup then finishes locally.
      uint32_t n_sel = 0, n_cand = 0;
      with_pred(pr, ib, rmask, [&](const auto& pred) {
        regs([&](uint32_t kk, int32_t j) {
          n_sel += pred.ge(kk, j) ? 1u : 0u;
          n_cand += pred.eq(kk, j) ? 1u : 0u;
        });
      });
      const uint32_t above = block_sum<BLOCK>(n_sel - n_cand, wtot);
      const uint32_t cw = wave_sum(n_cand);
      const uint32_t wave_base = wave_offset<BLOCK>(cw, wtot);
      uint32_t ctot = 0;
#pragma unroll
      for (int i = 0; i < BLOCK / kWave; ++i) ctot += wtot[i];
      if (tid == 0) {
        res[3] = ctot ? __hip_atomic_fetch_add(&ws->cand_count, ctot, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT)
                      : 0u;
        g_store(&ws->wg_count[g], above);
      }
      __syncthreads();
      uint32_t pos = res[3] + wave_base + wave_inclusive_sum(n_cand) - n_cand;
      with_pred(pr, ib, rmask, [&](const auto& pred) {
        regs([&](uint32_t kk, int32_t j) {
          if (pred.eq(kk, j)) {
            if (pos < static_cast<uint32_t>(kCandCap))
              g_store64(&ws->cand[pos], (static_cast<uint64_t>(kk) << 32) | static_cast<uint32_t>(j));
            ++pos;
          }
        });
      });
      row_barrier(&ws->bar, ++nbar * nwg, err);
      const int nc = static_cast<int>(cnt);
      for (int i = tid; i < nc; i += BLOCK) cand[i] = g_load64(&ws->cand[i]);
      __syncthreads();
      pf = rounds_local<BLOCK>(ListSource<BLOCK>{cand, nc}, pr, need, ib, hist, res, wtot);
      for (int i = tid; i < Gr; i += BLOCK) csel[i] = 0;
      __syncthreads();
      with_pred(pf, ib, rmask, [&](const auto& pred) {
        for (int i = tid; i < nc; i += BLOCK) {
          const uint64_t e = cand[i];
          const uint32_t kk = static_cast<uint32_t>(e >> 32);
          const int32_t j = static_cast<int32_t>(static_cast<uint32_t>(e));
          if (pred.ge(kk, j)) atomicAdd(&csel[(j + head) / p.chunk], 1u);
        }
      });
      __syncthreads();
      uint32_t part = 0;
      for (int i = tid; i < g; i += BLOCK) part += g_load(&ws->wg_count[i]) + csel[i];
      off = block_sum<BLOCK>(part, wtot);
    }
    emit_ordered<BLOCK, E>(key, ch, pf, ib, out_row, off, static_cast<uint32_t>(p.k), wtot);

    // Leave the row; the last workgroup out returns its workspace to zero.
    // Every read of the row's shared data happened before this arrival.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) {
      const uint32_t old = __hip_atomic_fetch_add(&ws->bar, 1u, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
      res[3] = old == (nbar + 1) * nwg - 1u ? 1u : 0u;
    }
    __syncthreads();
    if (res[3]) {
      for (int r = 0; r < rounds_used; ++r) {
        const int nbins = r == 0 ? kFirstBins : kNextBins;
        uint32_t* gh = ws->hist + hist_offset(r);
        for (int i = tid; i < nbins; i += BLOCK) g_store(&gh[i], 0u);
      }
      // published counts and candidates too: the workspace is left all zero,
      // whichever path uses it next
      for (int i = tid; i < Gr; i += BLOCK) g_store(&ws->wg_count[i], 0u);
      if (use_cand) {
        const uint32_t nc = cnt < static_cast<uint32_t>(kCandCap) ? cnt : kCandCap;
        for (uint32_t i = tid; i < nc; i += BLOCK) g_store64(&ws->cand[i], 0ull);
      }
      if (tid == 0) g_store(&ws->cand_count, 0u);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (tid == 0) g_store(&ws->bar, 0u);
    }
  }
}

// ---------------------------------------------------------------------------
// Chunked path: G workgroups per row and no grid-wide synchronisation.
//
// Each workgroup holds one chunk of a row (BLOCK*E entries) in registers and
// estimates, from a sample of its own chunk, a bound below which no entry of
// the row's top k is expected: with ns sample entries of a chunk of a row of
// length L, k*ns/L of them are expected at or above the row's threshold, and
// the bound is the sample entry (to 22 key bits) where the sample's count from
// the top reaches ceil(3 k ns / 2L) + 16, far beyond that expectation.  The chunk's
// entries at or above its bound go to the row's workspace in column order,
// with the chunk's count and bound.  The last workgroup of the row to arrive
// (a device-scope counter, which it then resets) gathers the chunks'
// candidates into registers and selects the top k among them.  The result is
// the row's top k whenever every chunk's bound lies at or below the smallest
// selected key: an entry a chunk did not publish is below that chunk's bound,
// hence below every selected entry.  This is checked; a row that fails it,
// or whose candidates overflow, is selected exactly by the same workgroup
// with radix rounds that stream the row from memory.
//
// A chunk publishes keys and column offsets in two lists.  The final
// workgroup reads chunk c's keys into union entries [c*W, c*W + count_c),
// W = 4 * floor(BLOCK*kUnionPerThread / 4G) (whole 16-byte groups): the
// slots past a chunk's count hold zero (key 0, never selected), so these
// loads need no counts and go out with the loads of the counts and bounds.
// When some chunk published more than W, the union is packed instead, by
// offsets from the counts.  The selected columns are staged in LDS at their
// ranks and written out in order.
// ---------------------------------------------------------------------------
constexpr int kChunkCap = 4096;       // candidates one chunk may publish
constexpr int kUnionPerThread = 16;   // candidates per thread in the final selection
constexpr int kChunkSamples = 16;     // sample positions per thread (the first half)

// Row r's block in the workspace (after the header) starts at
// r * chunk_row_bytes(G): a 256-byte head whose word 0 counts the row's
// arrived workgroups, then count[G], bound[G] and the largest published key
// kmax[G] (rounded to 256 bytes), then the candidates' keys (u32, G lists of
// kChunkCap) and their column offsets within the chunk (u16, G lists of
// kChunkCap).
__host__ __device__ constexpr size_t chunk_row_bytes(int G) {
  return 256 + ((12 * static_cast<size_t>(G) + 255) / 256) * 256 +
         static_cast<size_t>(G) * kChunkCap * 6;
}

// The union of the chunks' candidates in registers: thread t holds four
// groups of four consecutive union entries, group q being union entries
// 4*(q*BLOCK + t) .. +3, so entry u = 4q + j of the thread is union entry
// 4*(q*BLOCK + t) + j (the union is in column order); unused entries have
// key 0.  An entry's column is its chunk's first column plus the 16-bit
// offset published with it, which is read only where a column is used.
template <int CHUNK>
struct UnionList {
  uint32_t key[kUnionPerThread];
  uint32_t sat[kUnionPerThread];      // candidate slot: chunk << 12 | offset in the chunk's list
  u32x2 offw[kUnionPerThread / 4];    // column offsets within the chunk, 16 bits each (loaded late)
  __device__ __forceinline__ int32_t col(int u) const {
    const uint32_t w2 = (u & 2) ? offw[u >> 2].y : offw[u >> 2].x;
    const uint32_t off = (u & 1) ? (w2 >> 16) : (w2 & 0xFFFFu);
    return static_cast<int32_t>((sat[u] >> 12) * static_cast<uint32_t>(CHUNK) + off);
  }
  template <class F>
  __device__ __forceinline__ void operator()(F f) const {
#pragma unroll
    for (int u = 0; u < kUnionPerThread; ++u) f(key[u], col(u));
  }
  __device__ __forceinline__ void count(const Prefix& p, int d, int ib, uint32_t rmask,
                                        uint32_t* hist) const {
    count_digit(*this, p, d, ib, rmask, hist);
  }
};

// A whole row read from memory in blocks of BLOCK*16 entries (position u of
// thread (w, l) in block b is entry b*BLOCK*16 + w*1024 + u*64 + l, so the
// visiting order is column order); entries past the row carry key 0.
// Adds n to hist[bin] for each lane with n != 0 (n the same on all such
// lanes): one atomic when those lanes share a bin.
__device__ __forceinline__ void hist_add_lanes(uint32_t* hist, uint32_t bin, uint32_t n) {
  const uint64_t tm = __ballot(n != 0u);
  if (tm == 0u) return;
  const int first = __ffsll(static_cast<unsigned long long>(tm)) - 1;
  const uint32_t b0 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(bin), first));
  if (__ballot(n != 0u && bin != b0) == 0u) {
    if (static_cast<int>(__lane_id()) == first) atomicAdd(&hist[b0], n * static_cast<uint32_t>(__popcll(tm)));
  } else if (n != 0u) {
    atomicAdd(&hist[bin], n);
  }
}

// Smallest and largest of a lane's keys of a block.
__device__ __forceinline__ void lane_range(const uint32_t (&buf)[kChunkPos], uint32_t& mn, uint32_t& mx) {
  mn = buf[0];
  mx = buf[0];
#pragma unroll
  for (int u = 1; u < kChunkPos; ++u) {
    mn = min(mn, buf[u]);
    mx = max(mx, buf[u]);
  }
}

// One workgroup streaming a row of L entries in blocks of BLOCK x kChunkPos:
// wavefront w's part of a block is kChunkPos positions of 64 consecutive
// columns, so a block's column order is (wavefront, position, lane).  A
// pass over the row costs one CU's vector issue rate per operation on each
// entry, so the passes below summarise each lane's 16 keys by their range
// and do per-entry work only where the range leaves the answer open.
template <int BLOCK>
struct RowStream {
  __amdgpu_buffer_rsrc_t rsrc;
  int L;
  static constexpr int kBlockElems = BLOCK * kChunkPos;
  static constexpr int kRowBufs = 3;  // blocks in flight

  __device__ __forceinline__ RowStream(const float* row, int len)
      : rsrc(__builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(row), 0, len * 4, 0x00020000)),
        L(len) {}

  __device__ __forceinline__ int elem0(int base) const {
    int e = base + static_cast<int>(wave_id()) * (kWave * kChunkPos) +
            static_cast<int>(__lane_id());
    asm volatile("" : "+v"(e));
    return e;
  }
  // Loads block `base` (positions past the row read nothing).
  __device__ __forceinline__ void load(uint32_t (&buf)[kChunkPos], int e0) const {
#pragma unroll
    for (int u = 0; u < kChunkPos; ++u)
      buf[u] = __builtin_amdgcn_raw_buffer_load_b32(rsrc, (e0 + u * kWave) * 4, 0, 0);
  }
  // The block's keys; positions past the row get key 0, below every real
  // key (which is at least 1).  full: the block lies inside the row.
  __device__ __forceinline__ void keys(uint32_t (&buf)[kChunkPos], int e0, bool full) const {
    if (full) {
#pragma unroll
      for (int u = 0; u < kChunkPos; ++u) buf[u] = order_key_bits(buf[u]);
    } else {
#pragma unroll
      for (int u = 0; u < kChunkPos; ++u) buf[u] = e0 + u * kWave < L ? order_key_bits(buf[u]) : 0u;
    }
  }
  // Visits the row's blocks in order, block b+kRowBufs-1 loading while
  // block b is visited: visit(buf, e0, full) gets a block's keys and returns
  // whether to go on (the same answer on every thread of the workgroup; the
  // blocks after a false are skipped).  The loads are issued
  // unconditionally (past the row they read nothing), so the compiler's
  // waits stay exact.
  template <class V>
  __device__ __forceinline__ void blocks(V visit) const {
    uint32_t buf[kRowBufs][kChunkPos];
#pragma unroll
    for (int i = 0; i < kRowBufs - 1; ++i) load(buf[i], elem0(i * kBlockElems));
    bool go = true;
#pragma unroll 1
    for (int base = 0; go && base < L; base += kRowBufs * kBlockElems) {
#pragma unroll
      for (int i = 0; i < kRowBufs; ++i) {
        const int bb = base + i * kBlockElems;
        load(buf[(i + kRowBufs - 1) % kRowBufs], elem0(bb + (kRowBufs - 1) * kBlockElems));
        const int e0 = elem0(bb);
        const bool full = bb + kBlockElems <= L;
        keys(buf[i], e0, full);
        if (go) go = visit(buf[i], e0, full);
      }
    }
  }
  // Histogram of key digit d below the key prefix p (p.bits < 32; 0: every
  // entry of the row).  A wavefront whose lanes each have their 16 keys
  // outside the prefix or in one bin adds per lane (one atomic when the
  // lanes share the bin); other blocks add entry by entry (see below).
  // With `tally`, also the row's keys above x and equal to x, added to
  // gt_eq[0] and gt_eq[1] (x >= 1).
  __device__ __forceinline__ void count(const Prefix& p, int d, uint32_t* hist, bool tally,
                                        uint32_t x, uint32_t* gt_eq) const {
    const int sh = 32 - p.bits;  // bits below the prefix
    const uint32_t plo = p.bits == 0 ? 1u : max(p.kp << sh, 1u);
    const uint32_t phi = p.bits == 0 ? 0xFFFFFFFFu : (p.kp << sh) | ((1u << sh) - 1u);
    const uint32_t span = phi - plo;
    const int dsh = sh - d;
    const uint32_t dmask = (1u << d) - 1u;
    auto bin = [&](uint32_t key) { return (key >> dsh) & dmask; };
    auto take = [&](uint32_t key) { return key - plo <= span; };
    uint32_t gt = 0, eq = 0;
    blocks([&](const uint32_t (&buf)[kChunkPos], int, bool full) {
      if (full) {
        uint32_t mn, mx;
        lane_range(buf, mn, mx);
        if (tally) {
          gt += mn > x ? static_cast<uint32_t>(kChunkPos) : 0u;
          eq += mn == mx && mn == x ? static_cast<uint32_t>(kChunkPos) : 0u;
          if (!(mn > x || mx < x || mn == mx)) {
#pragma unroll
            for (int u = 0; u < kChunkPos; ++u) {
              gt += buf[u] > x ? 1u : 0u;
              eq += buf[u] == x ? 1u : 0u;
            }
          }
        }
        const bool none = mx < plo || mn > phi;
        const bool one = mn >= plo && mx <= phi && bin(mn) == bin(mx);
        if (__ballot(!none && !one) == 0u) {
          hist_add_lanes(hist, bin(mn), one ? static_cast<uint32_t>(kChunkPos) : 0u);
          return true;
        }
      } else if (tally) {
#pragma unroll
        for (int u = 0; u < kChunkPos; ++u) {
          gt += buf[u] > x ? 1u : 0u;
          eq += buf[u] == x ? 1u : 0u;
        }
      }
      // entry by entry: aggregated per position where the first position's
      // 64 entries share a bin (runs of equal or nearby values), else each
      // alone (scattered values, whose adds rarely meet in one bin)
      const uint32_t b00 = bin(buf[0]);
      if (__ballot(b00 != static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(b00)))) == 0u) {
#pragma unroll
        for (int u = 0; u < kChunkPos; ++u) hist_add_wave(hist, bin(buf[u]), take(buf[u]));
      } else {
#pragma unroll
        for (int u = 0; u < kChunkPos; ++u)
          if (take(buf[u])) atomicAdd(&hist[bin(buf[u])], 1u);
      }
      return true;
    });
    if (tally) {
      gt = wave_sum(gt);
      eq = wave_sum(eq);
      if (__lane_id() == 0) {
        atomicAdd(&gt_eq[0], gt);
        atomicAdd(&gt_eq[1], eq);
      }
    }
  }
};

// Exact selection of a whole row streamed from memory by one workgroup,
// given keys lo <= hi with lo <= T <= hi for the row's threshold key T (the
// k-th largest; lo = 0, hi = 2^32 - 1 when nothing is known).  Radix rounds
// over key digits (12, 10, 10 bits; those lo and hi share are skipped) run
// until the bucket holding the k-th entry is taken whole or T is known.  With lo >= 1 the first round also counts the keys
// above lo and equal to lo: fewer than k above and at least k at or above
// make T = lo.  Then, block by block, an ordered emission, which stops once
// k columns are out.  When only part of T's bucket is taken, the emission
// takes every entry above T and the first `need` entries equal to T in
// column order (the lowest columns among the ties), counting the ties
// before each entry as it goes, so ties cost no rounds over index digits.
template <int BLOCK>
__device__ __forceinline__ void select_row_streamed(const float* row, int L, int k, const OutRow& out_row,
                                                 uint32_t* hist, uint32_t* wtot, uint32_t* res,
                                                 uint32_t lo, uint32_t hi) {
  constexpr int NW = BLOCK / kWave;
  const RowStream<BLOCK> src(row, L);
  const int ib = index_bits(L);
  const uint32_t kk = static_cast<uint32_t>(k);
  const int tid = static_cast<int>(threadIdx.x);
  uint32_t need = kk;
  // T's leading bits are those lo and hi share, and no key is above hi, so
  // no entry lies in a bucket above that prefix: the rounds start at the
  // last digit boundary within it (moving the digits instead would make
  // them finer than the row's runs of nearby values, whose lanes the
  // histogram adds at once).
  if (lo > hi) {  // (not a bound pair: nothing is known)
    lo = 0u;
    hi = 0xFFFFFFFFu;
  }
  const int shared = lo == hi ? 32 : __clz(lo ^ hi);
  const int start = shared == 32 ? 32
                    : shared >= kFirstBits + kNextBits ? kFirstBits + kNextBits
                    : shared >= kFirstBits ? kFirstBits : 0;
  Prefix pf{start, start == 0 ? 0u : hi >> (32 - start), 0u};
  bool whole = false;  // the last bucket is taken whole
  bool first = true;
  while (pf.bits < 32) {
    const int d = digit_bits(pf.bits, ib);
    const bool wide = d > kNextBits;
    const int nb = wide ? kFirstBins : kNextBins;  // the bins the search reads
    for (int i = tid; i < nb; i += BLOCK) hist[i] = 0;
    if (tid == 0) {
      res[7] = 0u;
      res[8] = 0u;
    }
    __syncthreads();
    const bool tally = first && lo != 0u;
    src.count(pf, d, hist, tally, lo, res + 7);
    __syncthreads();
    if (tally) {
      const uint32_t above = res[7], at = res[8];
      if (above < kk && above + at >= kk) {
        pf = Prefix{32, lo, 0u};
        need = kk - above;
        break;
      }
    }
    first = false;
    const auto fixed = [need](uint32_t) { return need; };
    if (wide) {
      find_bucket_block<BLOCK, kFirstBins>(hist, fixed, res, wtot);
    } else {
      find_bucket_block<BLOCK, kNextBins>(hist, fixed, res, wtot);
    }
    __syncthreads();
    const uint32_t b = res[0], gt = res[1], cnt = res[2];
    need -= gt;
    pf = extend(pf, d, b);
    if (cnt == need) {
      whole = true;
      break;
    }
  }
  // The emission's wavefront counts alternate between two LDS arrays (wtot
  // and, free by now, the histogram's first words), so that one barrier
  // per count suffices: a wavefront writes an array again only after a
  // later barrier that every reader of its last contents has passed.
  uint32_t out_base = 0;
  if (whole) {
    // the selected entries are those with a key at or above the bucket's
    // edge: exactly k of them
    const uint32_t edge = prefix_edge(pf);
    bool odd = false;
    src.blocks([&](const uint32_t (&buf)[kChunkPos], int e0, bool) {
      uint32_t* const wc = odd ? hist : wtot;
      odd = !odd;
      uint32_t mn, mx;
      lane_range(buf, mn, mx);
      uint32_t n = mn >= edge ? static_cast<uint32_t>(kChunkPos) : 0u;
      if (!(mn >= edge || mx < edge)) {
#pragma unroll
        for (int u = 0; u < kChunkPos; ++u) n += buf[u] >= edge ? 1u : 0u;
      }
      const uint32_t wn = wave_sum(n);
      uint32_t pos = out_base + wave_offset<BLOCK>(wn, wc);
      uint32_t block_total = 0;
#pragma unroll
      for (int i = 0; i < NW; ++i) block_total += wc[i];
      if (wn != 0u) {
#pragma unroll
        for (int u = 0; u < kChunkPos; ++u) {
          const bool sel = buf[u] >= edge;
          const uint64_t m = __ballot(sel);
          const uint32_t at = pos + lanes_below(m);
          if (sel && at < kk) out_row.put(at, e0 + u * kWave);
          pos += static_cast<uint32_t>(__popcll(m));
        }
      }
      out_base += block_total;
      return out_base < kk;
    });
    __syncthreads();  // the output and the LDS are complete for the caller
    return;
  }
  // T = pf.kp (the whole key); `need` entries equal to T are taken.
  const uint32_t T = pf.kp;
  uint32_t tie_run = 0;  // entries equal to T in the earlier blocks
  src.blocks([&](const uint32_t (&buf)[kChunkPos], int e0, bool) {
    uint32_t mn, mx;
    lane_range(buf, mn, mx);
    const bool any = __ballot(mx >= T) != 0u;                 // keys at or above T
    const bool ties = __ballot(mn <= T && T <= mx) != 0u;     // keys that may equal T
    uint32_t tw = 0;
    if (ties) {
#pragma unroll
      for (int u = 0; u < kChunkPos; ++u) tw += static_cast<uint32_t>(__popcll(__ballot(buf[u] == T)));
    }
    uint32_t tr = tie_run + wave_offset<BLOCK>(tw, wtot);
    uint32_t tie_block = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) tie_block += wtot[i];
    uint32_t n = 0, selm = 0;
    if (ties) {
#pragma unroll
      for (int u = 0; u < kChunkPos; ++u) {
        const bool tie = buf[u] == T;
        const uint64_t m = __ballot(tie);
        const bool sel = buf[u] > T || (tie && tr + lanes_below(m) < need);
        selm |= sel ? (1u << u) : 0u;
        n += sel ? 1u : 0u;
        tr += static_cast<uint32_t>(__popcll(m));
      }
      n = wave_sum(n);
    } else if (any) {
#pragma unroll
      for (int u = 0; u < kChunkPos; ++u) {
        const bool sel = buf[u] > T;
        selm |= sel ? (1u << u) : 0u;
        n += sel ? 1u : 0u;
      }
      n = wave_sum(n);
    }
    uint32_t pos = out_base + wave_offset<BLOCK>(n, hist);
    uint32_t block_total = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) block_total += hist[i];
    if (n != 0u) {
#pragma unroll
      for (int u = 0; u < kChunkPos; ++u) {
        const bool sel = ((selm >> u) & 1u) != 0u;
        const uint64_t m = __ballot(sel);
        const uint32_t at = pos + lanes_below(m);
        if (sel && at < kk) out_row.put(at, e0 + u * kWave);
        pos += static_cast<uint32_t>(__popcll(m));
      }
    }
    out_base += block_total;
    tie_run += tie_block;
    return out_base < kk;
  });
  __syncthreads();  // the output and the LDS are complete for the caller
}

// Adds N entries per lane of a wavefront to an LDS histogram: one atomic
// for the wavefront when every entry is taken and falls in one bin (a run of
// equal values: constant rows, -inf tails), else one atomic per taken entry
// (a wavefront-aggregated add per entry costs a chain of lane reads and
// ballots; plain adds to mostly distinct bins are a few instructions).
template <int N, class BinOf, class TakeOf>
__device__ __forceinline__ void hist_add_entries(uint32_t* hist, BinOf bin_of, TakeOf take_of) {
  const uint32_t b0 = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(bin_of(0))));
  bool uni = true;
#pragma unroll
  for (int q = 0; q < N; ++q) uni = uni && take_of(q) && bin_of(q) == b0;
  if (__ballot(!uni) == 0u) {
    if (__lane_id() == 0) atomicAdd(&hist[b0], static_cast<uint32_t>(N * kWave));
  } else {
#pragma unroll
    for (int q = 0; q < N; ++q)
      if (take_of(q)) atomicAdd(&hist[bin_of(q)], 1u);
  }
}

// The J largest of v[0, N) in t, largest first (insertion: each value is
// carried down the list, swapping with every smaller entry).
template <int J, int N, int E>
__device__ __forceinline__ void largest_of(const uint32_t (&v)[E], uint32_t (&t)[J]) {
#pragma unroll
  for (int j = 0; j < J; ++j) t[j] = 0u;
#pragma unroll
  for (int u = 0; u < N; ++u) {
    uint32_t x = v[u];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const uint32_t m = max(t[j], x);
      x = min(t[j], x);
      t[j] = m;
    }
  }
}

template <int BLOCK, int E, bool VO>
__device__ __forceinline__ void chunks_item(const Params& p, int64_t item) {
  constexpr int NW = BLOCK / kWave;
  // the histogram's words; with VO also the composites of the row (32 KB)
  // behind them
  __shared__ __attribute__((aligned(16))) uint64_t hist_words[kFirstBins / 2 + (VO ? kSortMaxK : 0)];
  uint32_t* const hist = reinterpret_cast<uint32_t*>(hist_words);
  uint64_t* const comp = hist_words + kFirstBins / 2;
  __shared__ uint32_t coff[kMaxChunks + 1];
  __shared__ uint16_t scol[kChunkCap];
  __shared__ uint32_t wq[4 * NW];
  __shared__ uint32_t wtot[NW];
  __shared__ uint32_t res[13];
  const int tid = threadIdx.x;
  const int G = p.G;
  // Item i is chunk i / R of row i % R: the rows' chunks interleave in
  // dispatch order, so each row has its share of the first workgroups to
  // start (alone on their CU, their loads first in line) and of the later
  // ones.  Row after row, the last rows' chunks all started second on their
  // CU (long rows: those rows ended 3-4 us after the others), and a batch's
  // later rows, whose selection may stream the row itself, started it late.
  const int64_t row = item % p.num_rows;
  const int g = static_cast<int>(item / p.num_rows);
  const int L = row_length(p, row);
  const OutRow out_row = out_row_of(p, row);
  const float* row_ptr = p.logits + row * p.row_stride;
  if (L <= p.k) {
    if (g == 0) {
      write_trivial(out_row, L, p.k, BLOCK);
      if constexpr (VO) vo_rank_written<BLOCK>(row_ptr, L, L, out_row.p, comp);
    }
    return;
  }
  const int chunk = BLOCK * E;
  const int Gr = (L + chunk - 1) / chunk;
  if (g >= Gr) return;
  const int64_t cbase = static_cast<int64_t>(g) * chunk;
  const int clen = static_cast<int>(L - cbase < chunk ? L - cbase : chunk);
  const Chunk ch = make_chunk(row_ptr, 0, cbase, 0, clen);
  const uint32_t kk = static_cast<uint32_t>(p.k);
  const int ib = index_bits(L);
  const uint32_t rmask = (1u << ib) - 1u;
  if (Gr == 1) {
    // (the chunk is loaded inside each branch: a load before it kept the
    // registers of one branch live through the other)
    uint32_t raw1[E];
    load_raw<BLOCK, E>(raw1, ch);
    keys_in_place<BLOCK, E>(raw1, ch);
    select_chunk_whole_row<BLOCK, E>(raw1, ch, L, p.k, out_row, hist, wtot, res);
    if constexpr (VO) vo_rank_written<BLOCK>(row_ptr, L, p.k, out_row.p, comp);
    return;
  }
  // The chunk's raw bits, every load issued at once (past the row they read
  // nothing).  They become keys in place; positions past the row get key 1,
  // below every bound and skipped by the sample.  The sample is the thread's
  // first kChunkSamples positions (the first half of each wavefront's
  // stretch of the chunk), so it is taken while the second half is still
  // arriving; that half becomes keys after the bound.  (No branch touches a
  // loaded word before its conversion: a register copy where two paths
  // join would make the wave wait for every load issued before it.)
  static_assert(2 * kChunkSamples == E, "the sample is the first half");
  uint32_t kv[E];
  const int e0 = thread_elem0<E>();
  {
    const __amdgpu_buffer_rsrc_t rrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(ch.base), 0, clen * 4, 0x00020000);
#pragma unroll
    for (int u = 0; u < E; ++u)
      kv[u] = __builtin_amdgcn_raw_buffer_load_b32(rrs, (e0 + u * kWave) * 4, 0, 0);
  }
  const bool whole = clen == chunk;
  auto to_keys = [&](auto first, auto last) {
    if (whole) {
#pragma unroll
      for (int u = decltype(first)::value; u < decltype(last)::value; ++u) kv[u] = order_key_bits(kv[u]);
    } else {
#pragma unroll
      for (int u = decltype(first)::value; u < decltype(last)::value; ++u)
        kv[u] = e0 + u * kWave < clen ? order_key_bits(kv[u]) : 1u;
    }
  };
  to_keys(std::integral_constant<int, 0>{}, std::integral_constant<int, kChunkSamples>{});

  uint8_t* rb = p.ws + kWsHeader + static_cast<size_t>(row) * chunk_row_bytes(G);
  uint32_t* arrived = reinterpret_cast<uint32_t*>(rb);
  uint32_t* counts = reinterpret_cast<uint32_t*>(rb + 256);
  uint32_t* bounds = counts + G;
  uint32_t* kmaxs = bounds + G;
  uint8_t* ckeys = rb + 256 + ((12 * static_cast<size_t>(G) + 255) / 256) * 256;  // u32 [G][kChunkCap]
  uint8_t* ccols = ckeys + static_cast<size_t>(G) * kChunkCap * 4;                 // u16 [G][kChunkCap]

  // sample: the first kChunkSamples positions of each thread, ns entries
  // (the first 64*kChunkSamples elements of each wavefront's stretch that
  // lie inside the chunk); the bound is the nd-th largest of them.
  int ns = 0;
#pragma unroll
  for (int v = 0; v < NW; ++v) ns += min(max(clen - v * kWave * E, 0), kWave * kChunkSamples);
  const uint32_t nd = ceil_mul_div(3u * kk, static_cast<uint32_t>(ns), 2u * static_cast<uint32_t>(L)) + 16u;
  // When nd is small against the 512 threads, each thread contributes only
  // the largest of its samples (nd <= 64), or its two (nd <= 256) or four
  // (nd <= 1024) largest: the nd largest samples then lie in nearly nd
  // different threads, or few threads hold more of them than they
  // contribute, so the nd-th largest contribution is a bound just below the
  // nd-th largest sample (never above it: contributions are samples), found
  // from 512 to 2048 entries instead of 8192.  On smooth data the samples
  // crowd into few first-digit bins, whose LDS atomics then serialise.
  const bool by_max = nd <= 64u;
  const bool by_two = nd <= 256u;
  const bool by_four = nd <= 1024u;
  uint32_t smax = 0;
  uint32_t more[3] = {0u, 0u, 0u};  // (nd > 64) the next largest samples after smax
#pragma unroll
  for (int u = 0; u < kChunkSamples; ++u) smax = max(smax, kv[u]);  // positions past the row: key 1
  for (int i = tid; i < kFirstBins; i += BLOCK) hist[i] = 0;
  if (tid == 0) res[0] = 0u;
  __syncthreads();
  if (by_four) {
    if (smax > 1u) atomicAdd(&hist[smax >> (32 - kFirstBits)], 1u);
    if (!by_max) {  // (uniform: these passes cost the nd <= 64 rows nothing)
      if (by_two) {
        uint32_t t[2];
        largest_of<2, kChunkSamples>(kv, t);
        more[0] = t[1];
      } else {
        uint32_t t[4];
        largest_of<4, kChunkSamples>(kv, t);
        more[0] = t[1];
        more[1] = t[2];
        more[2] = t[3];
      }
#pragma unroll
      for (int j = 0; j < 3; ++j)
        if (more[j] > 1u) atomicAdd(&hist[more[j] >> (32 - kFirstBits)], 1u);
    }
  } else {
    hist_add_entries<kChunkSamples>(
        hist, [&](int q) { return kv[q] >> (32 - kFirstBits); },
        [&](int q) { return kv[q] > 1u; });
  }
  __syncthreads();
  find_bucket_block<BLOCK, kFirstBins>(hist, [nd](uint32_t) { return nd; }, res, wtot);
  __syncthreads();
  // The first-digit bin holding the need-th sample is refined by the next
  // digit, so the bound sits at that sample (to 22 bits) rather than at the
  // bin's lower edge, which on smooth data is up to twice as many entries
  // further down.  Bin 0 (also: too few samples) leaves the bound at 2.
  uint32_t lb = 2u;
  const uint32_t b0 = res[0];
  if (b0 != 0u) {
    const uint32_t need2 = nd - res[1];
    __syncthreads();  // res and hist are reused
    for (int i = tid; i < kNextBins; i += BLOCK) hist[i] = 0;
    __syncthreads();
    if (by_four) {
      if ((smax >> (32 - kFirstBits)) == b0)
        atomicAdd(&hist[(smax >> (32 - kFirstBits - kNextBits)) & (kNextBins - 1)], 1u);
      if (!by_max) {
#pragma unroll
        for (int j = 0; j < 3; ++j)
          if ((more[j] >> (32 - kFirstBits)) == b0)
            atomicAdd(&hist[(more[j] >> (32 - kFirstBits - kNextBits)) & (kNextBins - 1)], 1u);
      }
    } else {
      hist_add_entries<kChunkSamples>(
          hist, [&](int q) { return (kv[q] >> (32 - kFirstBits - kNextBits)) & (kNextBins - 1); },
          [&](int q) { return (kv[q] >> (32 - kFirstBits)) == b0; });
    }
    __syncthreads();
    find_bucket_block<BLOCK, kNextBins>(hist, [need2](uint32_t) { return need2; }, res, wtot);
    __syncthreads();
    lb = (b0 << (32 - kFirstBits)) | (res[0] << (32 - kFirstBits - kNextBits));
  }

  // The second half stays raw bits and is tested against the bound on them
  // (key >= lb: for lb <= 2^31 the bits, unsigned, are <= 2^32 - lb; above
  // that the bits, signed, are >= lb's low 31 bits); a key is formed only at
  // positions where some lane passes.  Positions past the row read as
  // kOutsideBits, whose key (1) is below every bound.
  if (!whole) {
#pragma unroll
    for (int u = kChunkSamples; u < E; ++u) kv[u] = e0 + u * kWave < clen ? kv[u] : kOutsideBits;
  }
  const uint32_t ulim = 0u - lb;
  const int32_t slim = static_cast<int32_t>(lb & 0x7FFFFFFFu);
  const bool pos_bound = lb > 0x80000000u;
  auto hit_of = [&](int u) -> bool {
    if (u < kChunkSamples) return kv[u] >= lb;
    return pos_bound ? static_cast<int32_t>(kv[u]) >= slim : kv[u] <= ulim;
  };
  auto key_of = [&](int u) -> uint32_t { return u < kChunkSamples ? kv[u] : order_key_bits(kv[u]); };

  // Publish the chunk's entries with key >= lb, in column order.  Each
  // wavefront stages its candidates in its own region of kWaveStage LDS
  // entries (keys in the histogram's words, column offsets in scol) while
  // counting them; the wavefronts' counts then place the regions one after
  // another, and consecutive threads write the list out.  A chunk whose
  // ties at the bound are cut (below), or a wavefront with more candidates
  // than its region holds, goes through the same steps with positions
  // counted first.
  constexpr uint32_t kWaveStage = kChunkCap / NW;
  const uint32_t wv = wave_id();
  uint32_t pos = 0;  // this wavefront's candidates so far (uniform)
  uint32_t tw = 0;   // ... and those equal to the bound
  uint32_t cm = 0;   // the largest key of this thread's candidates
#pragma unroll
  for (int u = 0; u < E; ++u) {
    const bool hit = hit_of(u);
    const uint64_t m = __ballot(hit);
    if (m != 0u) {  // most positions of a wavefront have no candidate
      const uint32_t key = key_of(u);
      cm = hit ? max(cm, key) : cm;
      const uint32_t at = pos + lanes_below(m);
      if (hit && at < kWaveStage) {
        hist[wv * kWaveStage + at] = key;
        scol[wv * kWaveStage + at] = static_cast<uint16_t>(e0 + u * kWave);
      }
      pos += static_cast<uint32_t>(__popcll(m));
      tw += static_cast<uint32_t>(__popcll(__ballot(key == lb)));
    }
  }
  cm = wave_max(cm);
  if (__lane_id() == 0) {
    wtot[wv] = pos;
    wq[wv] = tw;
    wq[NW + wv] = cm;
  }
  __syncthreads();
  uint32_t woff[NW + 1];
  woff[0] = 0;
  bool spill = false;
#pragma unroll
  for (int v = 0; v < NW; ++v) {
    const uint32_t c = wtot[v];
    woff[v + 1] = woff[v] + c;
    spill |= c > kWaveStage;
  }
  uint32_t total = woff[NW];
  // Of the chunk's entries equal to its bound, only the first k - A in
  // column order (A: its entries above the bound) can be selected: ties are
  // taken lowest column first and k entries at most, and if the row's
  // threshold is below the bound all of the chunk's entries at or above it
  // are selected, so there are at most k of them.  Long runs of ties (more
  // than a wavefront's worth) beyond that allowance are cut.
  uint32_t ties = 0;
#pragma unroll
  for (int v = 0; v < NW; ++v) ties += wq[v];
  const uint32_t above = total - ties;
  const uint32_t allowed = above < kk ? min(ties, kk - above) : 0u;
  const bool cut = allowed < ties && ties > static_cast<uint32_t>(kWave);
  const uint32_t limit = cut ? allowed : ties;
  const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
      ckeys + static_cast<size_t>(g) * kChunkCap * 4, 0, kChunkCap * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t pcs = __builtin_amdgcn_make_buffer_rsrc(
      ccols + static_cast<size_t>(g) * kChunkCap * 2, 0, kChunkCap * 2, 0x00020000);
  if (!spill && !cut) {
    if (total <= static_cast<uint32_t>(kChunkCap)) {  // else the row falls back: publish the count only
      for (uint32_t i = static_cast<uint32_t>(tid); i < total; i += BLOCK) {
        uint32_t v = 0, base = 0;  // the region holding list entry i
#pragma unroll
        for (int x = 1; x < NW; ++x) {
          const bool in = i >= woff[x];
          v = in ? static_cast<uint32_t>(x) : v;
          base = in ? woff[x] : base;
        }
        const uint32_t at = v * kWaveStage + (i - base);
        __builtin_amdgcn_raw_buffer_store_b32(hist[at], prs, i * 4, 0, kCoherent);
        __builtin_amdgcn_raw_buffer_store_b16(static_cast<unsigned short>(scol[at]), pcs, i * 2, 0, kCoherent);
      }
    }
  } else {
    // positions counted first: the entries above the bound and the first
    // `limit` ties, one list for the whole chunk
    uint32_t tp = 0, kp = 0, my_tp = 0, my_kp = 0;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      const uint32_t t_v = wq[v];
      const uint32_t keep_t = tp >= limit ? 0u : min(t_v, limit - tp);
      if (static_cast<uint32_t>(v) == wv) {
        my_tp = tp;
        my_kp = kp;
      }
      tp += t_v;
      kp += wtot[v] - t_v + keep_t;
    }
    total = kp;
    if (total <= static_cast<uint32_t>(kChunkCap)) {  // else the row falls back: publish the count only
      __syncthreads();  // the regions are rewritten
      uint32_t at = my_kp, tr = my_tp;
#pragma unroll
      for (int u = 0; u < E; ++u) {
        const uint32_t key = key_of(u);
        const bool tie = key == lb;
        const uint64_t mt = __ballot(tie);
        const bool keep = key >= lb && (!tie || tr + lanes_below(mt) < limit);
        const uint64_t mk = __ballot(keep);
        if (mk != 0u) {
          const uint32_t a2 = at + lanes_below(mk);
          if (keep) {
            hist[a2] = key;
            scol[a2] = static_cast<uint16_t>(e0 + u * kWave);
          }
          at += static_cast<uint32_t>(__popcll(mk));
        }
        tr += static_cast<uint32_t>(__popcll(mt));
      }
      __syncthreads();
      for (uint32_t i = static_cast<uint32_t>(tid); i < total; i += BLOCK) {
        __builtin_amdgcn_raw_buffer_store_b32(hist[i], prs, i * 4, 0, kCoherent);
        __builtin_amdgcn_raw_buffer_store_b16(static_cast<unsigned short>(scol[i]), pcs, i * 2, 0, kCoherent);
      }
    }
  }
  if (tid == 0) {
    uint32_t km = 0;
#pragma unroll
    for (int v = 0; v < NW; ++v) km = max(km, wq[NW + v]);
    g_store(&counts[g], total);
    g_store(&bounds[g], lb);
    g_store(&kmaxs[g], km);
  }
  // arrive; every store above has completed before the counter moves
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0) {
    const uint32_t old = __hip_atomic_fetch_add(arrived, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    res[4] = old == static_cast<uint32_t>(Gr) - 1u ? 1u : 0u;
  }
  __syncthreads();
  if (res[4] == 0u) return;

  // ---- the row's last workgroup: select among the chunks' candidates ----
  if (tid == 0) g_store(arrived, 0u);  // every workgroup of the row has arrived
  // Union layout: thread t holds groups q = 0..3 of four consecutive union
  // entries, group gi = q*BLOCK + t being union entries 4*gi .. 4*gi + 3;
  // the thread's entry u = 4q + j is union entry 4*gi + j.  Each entry
  // keeps its candidate slot (chunk << 12 | offset in the chunk's list).
  // Slotted: chunk c's list fills groups [c*Wg, (c+1)*Wg) with
  // Wg = 2048 / G (>= 2 since G <= kMaxChunks), so a group's keys are 16
  // consecutive bytes, loaded at once, before the counts are known; the
  // quotient by the reciprocal ceil(2^32 / Wg) is exact for gi, Wg < 2^16.
  // The groups past G*Wg (fewer than G) all read group Wg of the last
  // chunk, at entries below kChunkCap, which hold zero whenever this union
  // is used.  The column offsets (8 bytes per group) load right behind
  // the keys and arrive during the radix rounds, which need them only for
  // ties at the threshold.
  static_assert(kChunkCap == 4096, "slot = chunk << 12 | offset");
  static_assert(kUnionPerThread == 16, "four groups of four entries per thread");
  constexpr int kGroups = kUnionPerThread / 4;
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc(ckeys, 0, Gr * kChunkCap * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t crs =
      __builtin_amdgcn_make_buffer_rsrc(ccols, 0, Gr * kChunkCap * 2, 0x00020000);
  const uint32_t Wg = static_cast<uint32_t>(BLOCK * kGroups / Gr);
  const uint32_t Wgr = static_cast<uint32_t>((0x100000000ull + Wg - 1) / Wg);
  uint32_t gslot[kGroups];
  uint32_t sk[kUnionPerThread];
#pragma unroll
  for (int q = 0; q < kGroups; ++q) {
    const uint32_t gi = static_cast<uint32_t>(q * BLOCK + tid);
    const uint32_t c = min(__umulhi(gi, Wgr), static_cast<uint32_t>(Gr - 1));
    gslot[q] = c * static_cast<uint32_t>(kChunkCap) + 4u * min(gi - c * Wg, Wg);
  }
#pragma unroll
  for (int q = 0; q < kGroups; ++q) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(krs, gslot[q] * 4, 0, kCoherent);
    sk[4 * q + 0] = v.x;
    sk[4 * q + 1] = v.y;
    sk[4 * q + 2] = v.z;
    sk[4 * q + 3] = v.w;
  }
  // the slotted layout's column offsets go out right behind the keys (one
  // round trip for both; waiting for the keys leaves these in flight); the
  // packed layout loads its own instead
  UnionList<BLOCK * E> un;
#pragma unroll
  for (int q = 0; q < kGroups; ++q)
    un.offw[q] = __builtin_amdgcn_raw_buffer_load_b64(crs, gslot[q] * 2, 0, kCoherent);
  // the first window round's histogram is cleared while the keys arrive
  for (int i = tid; i < kFirstBins; i += BLOCK) hist[i] = 0;
  if (tid < kWave) {
    // offsets of the chunks' candidates in the packed union, total, bounds,
    // largest key
    uint32_t run = 0, lo = 0xFFFFFFFFu, hi = 0u, bad = 0u, mc = 0u, km = 0u;
    uint32_t cnt0 = 0u, km0 = 0u;  // this lane's chunk of the first 64
    for (int b0 = 0; b0 < Gr; b0 += kWave) {
      const int c = b0 + tid;
      const uint32_t cnt = c < Gr ? g_load(&counts[c]) : 0u;
      const uint32_t bnd = c < Gr ? g_load(&bounds[c]) : 0u;
      const uint32_t kmc = c < Gr ? g_load(&kmaxs[c]) : 0u;
      km = max(km, kmc);
      if (b0 == 0) {
        cnt0 = cnt;
        km0 = kmc;
      }
      const uint32_t incl = wave_inclusive_sum(cnt);
      if (c < Gr) coff[c] = run + incl - cnt;
      run += static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(incl), 63));
      if (c < Gr) {
        lo = bnd < lo ? bnd : lo;
        hi = bnd > hi ? bnd : hi;
        bad |= cnt > static_cast<uint32_t>(kChunkCap) ? 1u : 0u;
        mc = cnt > mc ? cnt : mc;
      }
    }
    hi = wave_max(hi);
    lo = ~wave_max(~lo);
    bad = wave_max(bad);
    mc = wave_max(mc);
    km = wave_max(km);
    // Union entries at or above the largest bound come only from chunks
    // whose largest key reaches it: with fewer than k of those the union's
    // k-th largest lies below that bound and the union cannot be exact
    // (counted when each lane holds one chunk).
    const uint32_t reach = wave_sum(km0 >= hi ? cnt0 : 0u);
    if (tid == 0) {
      coff[Gr] = run;
      res[5] = run;
      res[6] = lo;
      res[7] = hi;
      res[8] = bad;
      res[10] = mc;
      res[11] = km;
      res[12] = Gr <= kWave && reach < kk ? 1u : 0u;
    }
  }
  __syncthreads();
  // the counts, bounds and largest keys have been read (into coff and res)
  for (int c = tid; c < Gr; c += BLOCK) {
    g_store(&counts[c], 0u);
    g_store(&bounds[c], 0u);
    g_store(&kmaxs[c], 0u);
  }
  const uint32_t utotal = res[5], min_lb = res[6], max_lb = res[7];
  const bool fits = res[8] == 0u && utotal >= kk;
  const bool slotted = fits && res[10] <= 4u * Wg;
  const bool exact_ok =
      fits && (slotted || utotal <= static_cast<uint32_t>(BLOCK * kUnionPerThread)) && res[12] == 0u;
  bool done = false;
  if (exact_ok) {
    if (slotted) {
#pragma unroll
      for (int u = 0; u < kUnionPerThread; ++u) un.sat[u] = gslot[u / 4] + static_cast<uint32_t>(u % 4);
    } else {
      // packed union: the same entry order over the chunks' lists laid end
      // to end; a map from union entry to chunk (16-bit, in the histogram's
      // LDS; wavefront w fills the chunks c = w mod NW) gives each slot
      uint16_t* chunk_of = reinterpret_cast<uint16_t*>(hist);
      for (int c = static_cast<int>(wave_id()); c < Gr; c += NW)
        for (uint32_t i = coff[c] + __lane_id(); i < coff[c + 1]; i += kWave)
          chunk_of[i] = static_cast<uint16_t>(c);
      __syncthreads();
#pragma unroll
      for (int u = 0; u < kUnionPerThread; ++u) {
        const uint32_t i = 4u * static_cast<uint32_t>((u / 4) * BLOCK + tid) + static_cast<uint32_t>(u % 4);
        const bool ok = i < utotal;
        const uint32_t c = ok ? chunk_of[i] : 0u;
        un.sat[u] = ok ? c * static_cast<uint32_t>(kChunkCap) + (i - coff[c]) : 0xFFFFFFFFu;
      }
#pragma unroll
      for (int u = 0; u < kUnionPerThread; ++u)
        sk[u] = un.sat[u] != 0xFFFFFFFFu
                    ? __builtin_amdgcn_raw_buffer_load_b32(krs, un.sat[u] * 4, 0, kCoherent)
                    : 0u;
      __syncthreads();  // chunk_of (the histogram's words) is reused
    }
    uint32_t nz = 0;
#pragma unroll
    for (int u = 0; u < kUnionPerThread; ++u) {
      un.key[u] = sk[u];
      nz |= sk[u];
    }
    // the keys are consumed before the packed layout's column loads go
    // out, so no wait for those loads comes before the emission needs them
    asm volatile("" : : "v"(nz) : "memory");
    if (slotted) {
      // every slot of the union has been read (keys here, column offsets
      // once they have arrived): return them to zero now, so that the stores
      // drain during the rounds rather than after the output
      uint32_t oz = 0;
#pragma unroll
      for (int q = 0; q < kGroups; ++q) oz |= un.offw[q].x | un.offw[q].y;
      asm volatile("" : : "v"(oz) : "memory");
#pragma unroll
      for (int q = 0; q < kGroups; ++q) {
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{0u, 0u, 0u, 0u}, krs, gslot[q] * 4, 0, kCoherent);
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{0u, 0u}, crs, gslot[q] * 2, 0, kCoherent);
      }
    }
    if (!slotted) {
      uint32_t o[kUnionPerThread];
#pragma unroll
      for (int u = 0; u < kUnionPerThread; ++u)
        o[u] = un.key[u] != 0u ? __builtin_amdgcn_raw_buffer_load_b16(crs, un.sat[u] * 2, 0, kCoherent) : 0u;
#pragma unroll
      for (int q = 0; q < kGroups; ++q)
        un.offw[q] = u32x2{o[4 * q] | (o[4 * q + 1] << 16), o[4 * q + 2] | (o[4 * q + 3] << 16)};
    }
    const uint32_t kmax = res[11];
    // slotted: the histogram was cleared before the counts' barrier; packed:
    // its words held the chunk map, rounds_window clears them
    // Every candidate key lies in [min_lb, kmax].  When the two meet, every
    // candidate equals the row's largest key T, nothing lies above T, and the
    // first k candidates in the union's (column) order are the selection:
    // "key >= T" with the emission's cap at k, no rounds over the columns
    // (a chunk publishes its first k ties at most, in column order).  The
    // value-order emission ranks exactly k entries, so it takes the rounds.
    const Prefix pf = rounds_window<BLOCK>(un, min_lb, kmax, kk, ib, hist, res, wtot, slotted, !VO);
    // every selected key is at least the selected bucket's lower edge
    const uint32_t edge = prefix_edge(pf);
    if (edge >= max_lb) {
      // ordered emission.  The union's order is (group q, wavefront, lane,
      // j), so a selected entry's rank is: the selected entries of the
      // (q, wavefront) pairs before its own (an exclusive prefix over the
      // 4*NW pair totals, which every wavefront takes itself), plus those
      // of the lanes below in its wavefront's group q, plus those of its
      // own group before j.  The columns go to LDS at their ranks, then out
      // in order.
      uint32_t* stage = hist;  // k <= kChunkCap columns
      const uint32_t w = wave_id();
      const uint32_t lane = __lane_id();
      with_pred(pf, ib, rmask, [&](const auto& pred) {
        uint32_t sel = 0;
#pragma unroll
        for (int u = 0; u < kUnionPerThread; ++u)
          sel |= pred.ge(un.key[u], un.col(u)) ? (1u << u) : 0u;
        if constexpr (VO) {
          // the selected keys are on chip: ranked by buckets of the union's window
          vo_bucket_rank<BLOCK>(
              [&](auto f) {
#pragma unroll
                for (int u = 0; u < kUnionPerThread; ++u)
                  if ((sel >> u) & 1u) f(un.key[u], un.col(u));
              },
              prefix_edge(pf), kmax, static_cast<int>(kk), out_row.p, hist, comp, wtot, res);
          return;  // (from this lambda: what follows stores the column order)
        }
        uint32_t below[kGroups];
#pragma unroll
        for (int q = 0; q < kGroups; ++q) {
          const uint32_t c = static_cast<uint32_t>(__builtin_popcount((sel >> (4 * q)) & 15u));
          const uint32_t incl = wave_inclusive_sum(c);
          below[q] = incl - c;
          if (lane == kWave - 1) wq[q * NW + w] = incl;
        }
        __syncthreads();
        const uint32_t v = lane < static_cast<uint32_t>(kGroups * NW) ? wq[lane] : 0u;
        const uint32_t ex = wave_inclusive_sum(v) - v;
#pragma unroll
        for (int q = 0; q < kGroups; ++q) {
          uint32_t r = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(ex), q * NW + static_cast<int>(w))) +
                       below[q];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int u = 4 * q + j;
            if ((sel >> u) & 1u) {
              if (r < kk) stage[r] = static_cast<uint32_t>(un.col(u));
              ++r;
            }
          }
        }
        __syncthreads();
        // (the stores of write_staged, kept inline: calling the helper here
        // changed this kernel's code layout and measured 1% slower on rows
        // that go on to the streamed selection)
        if ((reinterpret_cast<uintptr_t>(out_row.p) & 15u) == 0 && (kk & 3u) == 0) {
          for (uint32_t i = 4u * static_cast<uint32_t>(tid); i < kk; i += 4u * BLOCK) {
            const uint4 v = *reinterpret_cast<const uint4*>(stage + i);
            *reinterpret_cast<int4*>(out_row.p + i) =
                int4{out_row.map(static_cast<int32_t>(v.x)), out_row.map(static_cast<int32_t>(v.y)),
                     out_row.map(static_cast<int32_t>(v.z)), out_row.map(static_cast<int32_t>(v.w))};
          }
        } else {
          for (uint32_t i = static_cast<uint32_t>(tid); i < kk; i += BLOCK)
            out_row.put(i, static_cast<int32_t>(stage[i]));
        }
      });
    }
    done = edge >= max_lb;
    if (tid == 0) res[9] = edge;  // (for the streamed selection: at most the row's threshold)
    // the slots read return to zero (other paths may use the workspace next;
    // the slotted union's were cleared as soon as they were read)
    if (!slotted) {
#pragma unroll
      for (int u = 0; u < kUnionPerThread; ++u)
        if (un.key[u] != 0u) {
          __builtin_amdgcn_raw_buffer_store_b32(0u, krs, un.sat[u] * 4, 0, kCoherent);
          __builtin_amdgcn_raw_buffer_store_b16(static_cast<unsigned short>(0), crs, un.sat[u] * 2, 0, kCoherent);
        }
    }
    if (!done) __syncthreads();  // the streamed selection reuses the LDS
  }
  if (!done) {
    // Bounds on the row's threshold key T.  Below: the union is part of
    // the row, so its k-th largest key (at least the edge of its bucket) is
    // at most T; without the union, at least k candidates lie at or above
    // the smallest chunk bound.  Above: every chunk's largest key is among
    // its candidates (a bound is at most one of the chunk's own samples),
    // except in a chunk of keys 1 alone, below every bound.
    const uint32_t t_lo = exact_ok ? res[9] : (res[5] >= kk ? res[6] : 0u);
    select_row_streamed<BLOCK>(row_ptr, L, p.k, out_row, hist, wtot, res, t_lo, max(res[11], 1u));
    if constexpr (VO) vo_rank_written<BLOCK>(row_ptr, L, p.k, out_row.p, comp);
  }
  if (!exact_ok) {
    for (int c = 0; c < Gr; ++c) {
      const uint32_t cnt = coff[c + 1] - coff[c];
      const uint32_t used = cnt <= static_cast<uint32_t>(kChunkCap) ? cnt : 0u;  // see the publish
      for (uint32_t j = static_cast<uint32_t>(tid); j < used; j += BLOCK) {
        const uint32_t at = static_cast<uint32_t>(c) * kChunkCap + j;
        __builtin_amdgcn_raw_buffer_store_b32(0u, krs, at * 4, 0, kCoherent);
        __builtin_amdgcn_raw_buffer_store_b16(static_cast<unsigned short>(0), crs, at * 2, 0, kCoherent);
      }
    }
  }
}

// One workgroup per chunk of a row; PERSIST: a fixed grid whose workgroups
// take chunks blockIdx.x, blockIdx.x + gridDim.x, ... in (row, chunk)
// order.  No workgroup ever waits for another, so any grid drains.
template <int BLOCK, int E, bool VO, bool PERSIST>
__global__ void __launch_bounds__(BLOCK) __attribute__((amdgpu_waves_per_eu(4)))
topk_chunks_kernel(Params p) {
  if constexpr (PERSIST) {
    const int64_t items = p.num_rows * p.G;
    for (int64_t item = blockIdx.x; item < items; item += gridDim.x) {
      chunks_item<BLOCK, E, VO>(p, item);
      __syncthreads();  // the LDS is reused by the next chunk
    }
  } else {
    chunks_item<BLOCK, E, VO>(p, blockIdx.x);
  }
}

__global__ void debug_keys_kernel(const float* in, uint32_t* out, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) out[i] = order_key(in[i]);
}

// Zero-fills n 16-byte words with vector stores (a kernel rather than a
// memset, so that a call captured in a graph records a kernel node).
__global__ void __launch_bounds__(256) fill_zero_kernel(uint4* p, int64_t n) {
  const int64_t step = static_cast<int64_t>(gridDim.x) * 256;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n; i += step)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// ---------------------------------------------------------------------------
// Value order as a pass over an existing selection: the selected columns of
// a row reordered by value (largest first, equal values by ascending
// column).  One workgroup per row gathers the m = min(k, L_i) selected
// values from the row and sorts their composites in LDS; slots [m, k) keep
// -1.  The selection kernels rank in their own emission instead (VO); this
// pass serves the cooperative split kernel and callers with an existing
// selection.
// ---------------------------------------------------------------------------

template <int BLOCK>
__global__ void __launch_bounds__(BLOCK) topk_value_order_kernel(const float* logits, int64_t row_stride,
                                                              const int32_t* lengths, int32_t k,
                                                              int32_t* idx) {
  __shared__ uint64_t comp[kSortMaxK];
  const int64_t row = blockIdx.x;
  int64_t L = lengths[row];
  L = L < 0 ? 0 : (L > row_stride ? row_stride : L);
  const int m = static_cast<int>(L < k ? L : k);
  if (m <= 1) return;
  const float* row_ptr = logits + row * row_stride;
  int32_t* out = idx + row * static_cast<int64_t>(k);
  for (int i = threadIdx.x; i < m; i += BLOCK) {
    const int32_t j = out[i];
    // a column outside the row (not a selection's output) reads nothing
    const bool ok = j >= 0 && j < L;
    comp[i] = vo_composite(ok ? order_key(row_ptr[j]) : 0u, j);
  }
  vo_sort_store<BLOCK>(comp, m, out);
}

// ---------------------------------------------------------------------------
// Host side: planning and launch.
// ---------------------------------------------------------------------------
enum Kind { kRow256x16, kRow512x16, kSplit512x32, kStream512x32, kStream512x64, kChunks512x32,
            kNumKinds };

// Largest k the chunked path takes; above it the candidates of a row would
// crowd the final selection, and the cooperative split path is used.
constexpr int32_t kChunksMaxK = 4096;
// One-workgroup-per-row kernels in increasing row capacity.
constexpr int kLocalKinds[] = {kRow256x16, kRow512x16, kStream512x32, kStream512x64};
constexpr int kNumLocalKinds = sizeof(kLocalKinds) / sizeof(kLocalKinds[0]);
constexpr int kLargestLocal = kLocalKinds[kNumLocalKinds - 1];

enum Mode { kModeRow, kModeSplit, kModeChunks };

struct KindInfo {
  int block, e;
  Mode mode;     // one workgroup per row; cooperative split; chunked
  bool aligned;  // the kernel starts a row's span at the 16-byte boundary below it
  const void* fn;
  const void* fn_vo;       // the same kernel writing value order (nullptr: a separate pass does)
  const void* fn_persist;  // the same kernel on a fixed grid (nullptr: none)
  int resident_per_cu;     // co-resident workgroups per CU on gfx950 (registers, LDS)
};

#define MI_TOPK_KERNEL_PTR(...) reinterpret_cast<const void*>(&__VA_ARGS__)
const KindInfo kKinds[kNumKinds] = {
    {256, 16, kModeRow, true, MI_TOPK_KERNEL_PTR(topk_row_kernel<256, 16, false, false>),
     MI_TOPK_KERNEL_PTR(topk_row_kernel<256, 16, true, false>),
     MI_TOPK_KERNEL_PTR(topk_row_kernel<256, 16, false, true>), 4},
    {512, 16, kModeRow, true, MI_TOPK_KERNEL_PTR(topk_row_kernel<512, 16, false, false>),
     MI_TOPK_KERNEL_PTR(topk_row_kernel<512, 16, true, false>),
     MI_TOPK_KERNEL_PTR(topk_row_kernel<512, 16, false, true>), 2},
    {512, 32, kModeSplit, true, MI_TOPK_KERNEL_PTR(topk_split_kernel<512, 32>), nullptr, nullptr, 2},
    {512, 32, kModeRow, false, MI_TOPK_KERNEL_PTR(topk_stream_kernel<512, 32, false, false>),
     MI_TOPK_KERNEL_PTR(topk_stream_kernel<512, 32, true, false>),
     MI_TOPK_KERNEL_PTR(topk_stream_kernel<512, 32, false, true>), 3},
    {512, 64, kModeRow, false, MI_TOPK_KERNEL_PTR(topk_stream_kernel<512, 64, false, false>),
     MI_TOPK_KERNEL_PTR(topk_stream_kernel<512, 64, true, false>),
     MI_TOPK_KERNEL_PTR(topk_stream_kernel<512, 64, false, true>), 3},
    {512, 32, kModeChunks, false, MI_TOPK_KERNEL_PTR(topk_chunks_kernel<512, 32, false, false>),
     MI_TOPK_KERNEL_PTR(topk_chunks_kernel<512, 32, true, false>),
     MI_TOPK_KERNEL_PTR(topk_chunks_kernel<512, 32, false, true>), 2},
};
#undef MI_TOPK_KERNEL_PTR

struct DeviceInfo {
  int cus = 0;
  int coop = 0;
  int split_per_cu = 0;  // co-resident split workgroups per CU
  int per_cu[kNumKinds] = {};  // co-resident workgroups per CU of each kernel on its fixed grid
  hipError_t status = hipSuccess;
};

constexpr int kMaxDevices = 64;
std::once_flag g_dev_once[kMaxDevices];
DeviceInfo g_dev[kMaxDevices];

hipError_t device_info(DeviceInfo* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_dev_once[dev], [dev]() {
    DeviceInfo d;
    d.status = hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (d.status == hipSuccess)
      d.status = hipDeviceGetAttribute(&d.coop, hipDeviceAttributeCooperativeLaunch, dev);
    if (d.status == hipSuccess)
      d.status = hipOccupancyMaxActiveBlocksPerMultiprocessor(&d.split_per_cu, kKinds[kSplit512x32].fn,
                                                              kKinds[kSplit512x32].block, 0);
    for (int i = 0; i < kNumKinds && d.status == hipSuccess; ++i)
      if (kKinds[i].fn_persist != nullptr)
        d.status = hipOccupancyMaxActiveBlocksPerMultiprocessor(&d.per_cu[i], kKinds[i].fn_persist,
                                                                kKinds[i].block, 0);

    g_dev[dev] = d;
  });
  *out = g_dev[dev];
  return out->status;
}

struct Plan {
  int kind = kRow256x16;
  int64_t chunk = 0;
  int G = 1;
  int rows_per_iter = 0;
  int64_t grid = 0;
  size_t ws_bytes = 0;
  bool persist = false;  // the kernel's fixed-grid form
};

int64_t cap_of(int kind) { return static_cast<int64_t>(kKinds[kind].block) * kKinds[kind].e; }

// Elements a row can span in `kind`'s layout: the stride, plus the
// misalignment below a 16-byte boundary for kernels that align row starts.
int64_t span_of(int kind, int64_t row_stride, int head_max) {
  return row_stride + (kKinds[kind].aligned ? head_max : 0);
}

// head_max: largest misalignment (in elements) of a row start below a 16-byte
// boundary: 0 when logits is 16-byte aligned and row_stride % 4 == 0, else 3.
int make_plan_kernel(int64_t num_rows, int64_t row_stride, int32_t k, int path, int chunks, int head_max,
                     const DeviceInfo& dev, Plan* pl);

// MI_TOPK_PATH_PERSIST: the kernel the automatic choice takes, on a fixed
// grid of the workgroups the device holds at once (its compute units times
// the kernel's residency), whatever the batch; the cooperative split kernel
// already runs on a grid of co-resident workgroups.
int make_plan(int64_t num_rows, int64_t row_stride, int32_t k, int path, int chunks, int head_max,
              const DeviceInfo& dev, Plan* pl) {
  const bool persist = path == MI_TOPK_PATH_PERSIST;
  const int st = make_plan_kernel(num_rows, row_stride, k, persist ? MI_TOPK_PATH_AUTO : path, chunks,
                                  head_max, dev, pl);
  if (st != MI_TOPK_OK || !persist || kKinds[pl->kind].fn_persist == nullptr) return st;
  const int per_cu = dev.per_cu[pl->kind];
  if (per_cu < 1) return MI_TOPK_ELAUNCH;
  pl->persist = true;
  pl->grid = static_cast<int64_t>(per_cu) * dev.cus;
  return MI_TOPK_OK;
}

int make_plan_kernel(int64_t num_rows, int64_t row_stride, int32_t k, int path, int chunks, int head_max,
                     const DeviceInfo& dev, Plan* pl) {
  const int64_t need = row_stride + head_max;  // elements a row can span from its aligned start
  const bool fits_local = span_of(kLargestLocal, row_stride, head_max) <= cap_of(kLargestLocal);
  bool split;
  if (path == MI_TOPK_PATH_LOCAL) {
    if (!fits_local) return MI_TOPK_ETOOLONG;
    split = false;
  } else if (path == MI_TOPK_PATH_SPLIT || path == MI_TOPK_PATH_CHUNKS) {
    split = true;
  } else {
    // Few long rows cannot fill the device with one workgroup each.
    split = !fits_local || (row_stride > 8192 && num_rows < 2 * static_cast<int64_t>(dev.cus));
  }
  if (!split) {
    int i = 0;
    while (cap_of(kLocalKinds[i]) < span_of(kLocalKinds[i], row_stride, head_max)) ++i;
    const int kind = kLocalKinds[i];
    pl->kind = kind;
    pl->chunk = cap_of(kind);
    pl->G = 1;
    pl->grid = num_rows;

    pl->rows_per_iter = static_cast<int>(num_rows);
    pl->ws_bytes = 0;
    return MI_TOPK_OK;
  }
  if (path == MI_TOPK_PATH_CHUNKS || (path == MI_TOPK_PATH_AUTO && k <= kChunksMaxK)) {
    // G chunks of BLOCK*E entries per row, one workgroup each, rows starting
    // at element 0; the last workgroup of a row selects among the chunks'
    // candidates
    const int64_t cap = cap_of(kChunks512x32);
    const int64_t G = (row_stride + cap - 1) / cap;
    if (G > kMaxChunks || num_rows * G > INT32_MAX) return MI_TOPK_ETOOLONG;
    if (k > kChunksMaxK) return MI_TOPK_EINVAL;
    pl->kind = kChunks512x32;
    pl->chunk = cap;
    pl->G = static_cast<int>(G);
    pl->rows_per_iter = static_cast<int>(num_rows);
    pl->grid = num_rows * G;
    pl->ws_bytes = kWsHeader + static_cast<size_t>(num_rows) * chunk_row_bytes(static_cast<int>(G));
    return MI_TOPK_OK;
  }
  if (!dev.coop || dev.split_per_cu < 1) return MI_TOPK_ELAUNCH;
  const int64_t cap = cap_of(kSplit512x32);
  const int64_t max_res = static_cast<int64_t>(dev.split_per_cu) * dev.cus;
  const int64_t g_min = (need + cap - 1) / cap;
  int64_t G;
  if (chunks > 0) {
    G = chunks;
  } else {
    const int64_t g_fill = (max_res + num_rows - 1) / num_rows;
    const int64_t g_most = std::max<int64_t>(1, (need + 4095) / 4096);  // chunks of >= 4096
    G = std::max(g_min, std::min(g_fill, g_most));
  }
  if (G < g_min) return MI_TOPK_EINVAL;
  int64_t chunk = ((need + G - 1) / G + 3) & ~int64_t(3);
  G = (need + chunk - 1) / chunk;
  if (G > kMaxChunks || G > max_res) return MI_TOPK_ETOOLONG;
  const int64_t rows_per_iter = std::min<int64_t>(num_rows, max_res / G);
  pl->kind = kSplit512x32;
  pl->chunk = chunk;
  pl->G = static_cast<int>(G);
  pl->rows_per_iter = static_cast<int>(rows_per_iter);
  pl->grid = rows_per_iter * G;
  pl->ws_bytes = kWsHeader + static_cast<size_t>(num_rows) * sizeof(RowWs);
  return MI_TOPK_OK;
}

int check_shape(int64_t num_rows, int64_t row_stride, int32_t k) {
  if (num_rows < 0 || num_rows > INT32_MAX) return MI_TOPK_EINVAL;
  if (row_stride < 1 || row_stride > INT32_MAX - 8) return MI_TOPK_EINVAL;
  if (k < 1 || k > MI_TOPK_MAX_K) return MI_TOPK_EINVAL;
  return MI_TOPK_OK;
}

size_t workspace_size_impl(int64_t num_rows, int64_t row_stride, int32_t k, int path, int chunks) {
  if (check_shape(num_rows, row_stride, k) != MI_TOPK_OK || num_rows == 0) return 0;
  DeviceInfo dev;
  if (device_info(&dev) != hipSuccess) return 0;
  Plan pl;
  if (make_plan(num_rows, row_stride, k, path, chunks, 3, dev, &pl) != MI_TOPK_OK) return 0;
  return pl.ws_bytes;
}

int value_order_launch(const Params& prm, hipStream_t stream);

// vo: the output in value order, by the kernel's own value-order variant or,
// for a kernel without one, by the value-order pass after it.
int launch(const Plan& pl, Params prm, hipStream_t stream, bool vo = false) {
  const KindInfo& ki = kKinds[pl.kind];
  void* args[] = {&prm};
  const bool vo_pass = vo && (ki.fn_vo == nullptr || pl.persist);  // value order by the separate pass
  const void* fn = pl.persist ? ki.fn_persist : (vo && !vo_pass ? ki.fn_vo : ki.fn);
  hipError_t e;
  if (ki.mode == kModeSplit) {
    e = hipLaunchCooperativeKernel(fn, dim3(static_cast<unsigned>(pl.grid)), dim3(ki.block), args, 0,
                                   stream);
  } else {
    e = hipLaunchKernel(fn, dim3(static_cast<unsigned>(pl.grid)), dim3(ki.block), args, 0, stream);
  }
  if (e != hipSuccess) return MI_TOPK_ELAUNCH;
  if (vo_pass) return value_order_launch(prm, stream);
  return MI_TOPK_OK;
}

// Paged output: the page table, its row stride, page size and row-to-request
// map of a topk_indices_paged call (table == nullptr: plain columns).
struct Paging {
  const int32_t* table = nullptr;
  int64_t stride = 0;
  int32_t page = 1;
  const int32_t* row_req = nullptr;
};

int topk_impl(const float* logits, int64_t row_stride, const int32_t* lengths, int64_t num_rows,
              int32_t k, int32_t* out, void* workspace, size_t workspace_bytes, int path, int chunks,
              hipStream_t stream, const Paging& pg = Paging{}, bool vo = false) {
  int st = check_shape(num_rows, row_stride, k);
  if (st != MI_TOPK_OK) return st;
  if (vo && (k > kSortMaxK || pg.table != nullptr)) return MI_TOPK_EINVAL;
  if (path < MI_TOPK_PATH_AUTO || path > MI_TOPK_PATH_PERSIST || chunks < 0) return MI_TOPK_EINVAL;
  if (num_rows == 0) return MI_TOPK_OK;
  if (!logits || !lengths || !out) return MI_TOPK_EINVAL;
  if ((reinterpret_cast<uintptr_t>(logits) & 3u) || (reinterpret_cast<uintptr_t>(lengths) & 3u) ||
      (reinterpret_cast<uintptr_t>(out) & 3u))
    return MI_TOPK_EINVAL;
  if (pg.table != nullptr &&
      (pg.page < 1 || pg.stride < 0 || (reinterpret_cast<uintptr_t>(pg.table) & 3u) ||
       (reinterpret_cast<uintptr_t>(pg.row_req) & 3u)))
    return MI_TOPK_EINVAL;
  DeviceInfo dev;
  if (device_info(&dev) != hipSuccess) return MI_TOPK_ELAUNCH;
  const int head_max = ((reinterpret_cast<uintptr_t>(logits) & 15u) == 0 && (row_stride & 3) == 0) ? 0 : 3;
  Plan pl;
  st = make_plan(num_rows, row_stride, k, path, chunks, head_max, dev, &pl);
  if (st != MI_TOPK_OK) return st;
  if (pl.ws_bytes > 0 && (workspace == nullptr || workspace_bytes < pl.ws_bytes)) return MI_TOPK_EWORKSPACE;
  Params prm;
  prm.logits = logits;
  prm.row_stride = row_stride;
  prm.lengths = lengths;
  prm.num_rows = num_rows;
  prm.out = out;
  prm.ws = static_cast<uint8_t*>(workspace);
  prm.k = k;
  prm.chunk = static_cast<int32_t>(pl.chunk);
  prm.G = pl.G;
  prm.rows_per_iter = pl.rows_per_iter;
  prm.block_table = pg.table;
  prm.bt_stride = pg.stride;
  prm.row_req = pg.row_req;
  prm.page = pg.page;
  prm.page_log2 = (pg.page & (pg.page - 1)) == 0 ? __builtin_ctz(static_cast<unsigned>(pg.page)) : -1;
  return launch(pl, prm, stream, vo);
}

}  // namespace
}  // namespace mitopk

using namespace mitopk;

MI_TOPK_EXPORT size_t topk_workspace_size(int64_t num_rows, int64_t row_stride, int32_t k) {
  return workspace_size_impl(num_rows, row_stride, k, MI_TOPK_PATH_AUTO, 0);
}

MI_TOPK_EXPORT size_t topk_workspace_size_path(int64_t num_rows, int64_t row_stride, int32_t k,
                                               int32_t path, int32_t chunks) {
  if (path < MI_TOPK_PATH_AUTO || path > MI_TOPK_PATH_PERSIST || chunks < 0) return 0;
  return workspace_size_impl(num_rows, row_stride, k, path, chunks);
}

MI_TOPK_EXPORT int topk_indices(const float* logits, int64_t row_stride, const int32_t* lengths,
                                int64_t num_rows, int32_t k, int32_t* out, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  return topk_impl(logits, row_stride, lengths, num_rows, k, out, workspace, workspace_bytes,
                   MI_TOPK_PATH_AUTO, 0, stream);
}

MI_TOPK_EXPORT int topk_indices_path(const float* logits, int64_t row_stride, const int32_t* lengths,
                                     int64_t num_rows, int32_t k, int32_t* out, void* workspace,
                                     size_t workspace_bytes, int32_t path, int32_t chunks,
                                     hipStream_t stream) {
  return topk_impl(logits, row_stride, lengths, num_rows, k, out, workspace, workspace_bytes, path,
                   chunks, stream);
}

MI_TOPK_EXPORT int topk_indices_paged_path(const float* logits, int64_t row_stride,
                                           const int32_t* lengths, int64_t num_rows, int32_t k,
                                           int32_t* out, void* workspace, size_t workspace_bytes,
                                           const int32_t* block_table, int64_t block_table_stride,
                                           int32_t page_size, const int32_t* row_to_req,
                                           int32_t path, int32_t chunks, hipStream_t stream) {
  if (block_table == nullptr) return MI_TOPK_EINVAL;
  Paging pg;
  pg.table = block_table;
  pg.stride = block_table_stride;
  pg.page = page_size;
  pg.row_req = row_to_req;
  return topk_impl(logits, row_stride, lengths, num_rows, k, out, workspace, workspace_bytes, path,
                   chunks, stream, pg);
}

MI_TOPK_EXPORT int topk_indices_paged(const float* logits, int64_t row_stride, const int32_t* lengths,
                                      int64_t num_rows, int32_t k, int32_t* out, void* workspace,
                                      size_t workspace_bytes, const int32_t* block_table,
                                      int64_t block_table_stride, int32_t page_size,
                                      const int32_t* row_to_req, hipStream_t stream) {
  return topk_indices_paged_path(logits, row_stride, lengths, num_rows, k, out, workspace,
                                 workspace_bytes, block_table, block_table_stride, page_size,
                                 row_to_req, MI_TOPK_PATH_AUTO, 0, stream);
}

namespace mitopk {
namespace {
int describe(int64_t num_rows, int64_t row_stride, int32_t k, int32_t path, int32_t chunks,
             const DeviceInfo& dev, int64_t* info) {
  Plan pl;
  const int head_max = (row_stride & 3) == 0 ? 0 : 3;
  const int st = make_plan(num_rows, row_stride, k, path, chunks, head_max, dev, &pl);
  if (st != MI_TOPK_OK) return st;
  const KindInfo& ki = kKinds[pl.kind];
  info[0] = ki.mode == kModeSplit ? MI_TOPK_PATH_SPLIT
            : ki.mode == kModeChunks ? MI_TOPK_PATH_CHUNKS
                                     : MI_TOPK_PATH_LOCAL;
  if (pl.persist) info[0] |= MI_TOPK_PLAN_PERSIST;
  info[1] = ki.block;
  info[2] = ki.e;
  info[3] = pl.chunk;
  info[4] = pl.G;
  info[5] = pl.grid;
  info[6] = static_cast<int64_t>(pl.ws_bytes);
  return MI_TOPK_OK;
}
}  // namespace
}  // namespace mitopk

MI_TOPK_EXPORT int topk_plan_describe(int64_t num_rows, int64_t row_stride, int32_t k, int32_t path,
                                      int32_t chunks, int64_t* info) {
  const int st = check_shape(num_rows, row_stride, k);
  if (st != MI_TOPK_OK) return st;
  if (!info || path < MI_TOPK_PATH_AUTO || path > MI_TOPK_PATH_PERSIST || chunks < 0) return MI_TOPK_EINVAL;
  DeviceInfo dev;
  if (device_info(&dev) != hipSuccess) return MI_TOPK_ELAUNCH;
  return describe(num_rows, row_stride, k, path, chunks, dev, info);
}

MI_TOPK_EXPORT int topk_plan_describe_for(int64_t num_rows, int64_t row_stride, int32_t k,
                                          int32_t path, int32_t chunks, int32_t cus, int32_t coop,
                                          int32_t split_per_cu, int64_t* info) {
  const int st = check_shape(num_rows, row_stride, k);
  if (st != MI_TOPK_OK) return st;
  if (!info || path < MI_TOPK_PATH_AUTO || path > MI_TOPK_PATH_PERSIST || chunks < 0 || cus < 1 ||
      split_per_cu < 0)
    return MI_TOPK_EINVAL;
  DeviceInfo dev;
  dev.cus = cus;
  dev.coop = coop;
  dev.split_per_cu = split_per_cu;
  for (int i = 0; i < kNumKinds; ++i) dev.per_cu[i] = kKinds[i].resident_per_cu;
  return describe(num_rows, row_stride, k, path, chunks, dev, info);
}

MI_TOPK_EXPORT const char* topk_status_string(int status) {
  switch (status) {
    case MI_TOPK_OK: return "ok";
    case MI_TOPK_EINVAL: return "invalid argument";
    case MI_TOPK_EWORKSPACE: return "workspace too small";
    case MI_TOPK_ELAUNCH: return "HIP launch or device query failed";
    case MI_TOPK_ETOOLONG: return "rows too long for the device";
    case MI_TOPK_ESCRATCH: return "batch needs more workspace than the no-allocation entry point holds";
    default: return "unknown status";
  }
}

namespace mitopk {
namespace {
int value_order_launch(const Params& prm, hipStream_t stream) {
  hipLaunchKernelGGL(topk_value_order_kernel<512>, dim3(static_cast<unsigned>(prm.num_rows)), dim3(512), 0,
                     stream, prm.logits, prm.row_stride, prm.lengths, prm.k, prm.out);
  return hipGetLastError() == hipSuccess ? MI_TOPK_OK : MI_TOPK_ELAUNCH;
}
}  // namespace
}  // namespace mitopk

MI_TOPK_EXPORT int topk_value_order(const float* logits, int64_t row_stride, const int32_t* lengths,
                                    int64_t num_rows, int32_t k, int32_t* idx, hipStream_t stream) {
  if (num_rows < 0 || num_rows > INT32_MAX || row_stride < 1 || k < 1 || k > kSortMaxK)
    return MI_TOPK_EINVAL;
  if (num_rows == 0) return MI_TOPK_OK;
  if (!logits || !lengths || !idx) return MI_TOPK_EINVAL;
  Params prm{};
  prm.logits = logits;
  prm.row_stride = row_stride;
  prm.lengths = lengths;
  prm.num_rows = num_rows;
  prm.k = k;
  prm.out = idx;
  return value_order_launch(prm, stream);
}

MI_TOPK_EXPORT int topk_indices_sorted_path(const float* logits, int64_t row_stride,
                                            const int32_t* lengths, int64_t num_rows, int32_t k,
                                            int32_t* out, void* workspace, size_t workspace_bytes,
                                            int32_t path, int32_t chunks, hipStream_t stream) {
  return topk_impl(logits, row_stride, lengths, num_rows, k, out, workspace, workspace_bytes, path,
                   chunks, stream, Paging{}, true);
}

MI_TOPK_EXPORT int topk_indices_sorted(const float* logits, int64_t row_stride, const int32_t* lengths,
                                       int64_t num_rows, int32_t k, int32_t* out, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream) {
  return topk_impl(logits, row_stride, lengths, num_rows, k, out, workspace, workspace_bytes,
                   MI_TOPK_PATH_AUTO, 0, stream, Paging{}, true);
}

MI_TOPK_EXPORT int topk_debug_keys(const float* in, uint32_t* out, int64_t n, hipStream_t stream) {
  if (n < 0 || n > (int64_t(1) << 40)) return MI_TOPK_EINVAL;
  if (n == 0) return MI_TOPK_OK;
  if (!in || !out) return MI_TOPK_EINVAL;
  const int64_t blocks = (n + 255) / 256;
  if (blocks > INT32_MAX) return MI_TOPK_EINVAL;
  hipLaunchKernelGGL(debug_keys_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, in, out, n);
  return hipGetLastError() == hipSuccess ? MI_TOPK_OK : MI_TOPK_ELAUNCH;
}

// ---------------------------------------------------------------------------
// The no-allocation entry point: topk_indices() with its workspace in a
// fixed device array instead of a caller's buffer.
// ---------------------------------------------------------------------------
namespace {
constexpr size_t kScratchBytes = MI_TOPK_NOALLOC_WORKSPACE;
}  // namespace

// One copy per device, held until the process ends.  In host code this name
// stands for the array but is not its device address: the address is taken
// once per device with hipGetSymbolAddress (scratch_of below) and only that
// pointer is ever passed to a kernel.
static __device__ __attribute__((aligned(256))) uint8_t scratch[kScratchBytes];

namespace mitopk {
namespace {

std::once_flag g_scratch_once[kMaxDevices];
uint8_t* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_status[kMaxDevices];
std::once_flag g_scratch_clear_once[kMaxDevices];
hipError_t g_scratch_clear_status[kMaxDevices];

int fill_zero(uint8_t* p, size_t bytes, hipStream_t stream) {
  const int64_t n = static_cast<int64_t>((bytes + 15) / 16);
  if (n == 0) return MI_TOPK_OK;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(fill_zero_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                     reinterpret_cast<uint4*>(p), n);
  return hipGetLastError() == hipSuccess ? MI_TOPK_OK : MI_TOPK_ELAUNCH;
}

// The current device's scratch address, taken on the first call on that
// device (with it current), and the scratch zero-filled on the stream of
// that first call (the kernels need it zero before their first use and
// leave it zero after every call).
int scratch_of(hipStream_t stream, uint8_t** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MI_TOPK_ELAUNCH;
  std::call_once(g_scratch_once[dev], [dev]() {
    void* ptr = nullptr;
    g_scratch_status[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = static_cast<uint8_t*>(ptr);
  });
  if (g_scratch_status[dev] != hipSuccess || g_scratch_ptr[dev] == nullptr) return MI_TOPK_ELAUNCH;
  std::call_once(g_scratch_clear_once[dev], [dev, stream]() {
    g_scratch_clear_status[dev] =
        fill_zero(g_scratch_ptr[dev], kScratchBytes, stream) == MI_TOPK_OK ? hipSuccess : hipErrorLaunchFailure;
  });
  if (g_scratch_clear_status[dev] != hipSuccess) return MI_TOPK_ELAUNCH;
  *out = g_scratch_ptr[dev];
  return MI_TOPK_OK;
}

}  // namespace
}  // namespace mitopk

MI_TOPK_EXPORT int topk_indices_noalloc(const float* logits, int64_t row_stride, const int32_t* lengths,
                                        int64_t num_rows, int32_t k, int32_t* out, hipStream_t stream) {
  int st = check_shape(num_rows, row_stride, k);
  if (st != MI_TOPK_OK) return st;
  if (num_rows == 0) return MI_TOPK_OK;
  if (!logits || !lengths || !out) return MI_TOPK_EINVAL;
  DeviceInfo dev;
  if (device_info(&dev) != hipSuccess) return MI_TOPK_ELAUNCH;
  if ((reinterpret_cast<uintptr_t>(logits) & 3u) || (reinterpret_cast<uintptr_t>(lengths) & 3u) ||
      (reinterpret_cast<uintptr_t>(out) & 3u))
    return MI_TOPK_EINVAL;
  const int head_max = ((reinterpret_cast<uintptr_t>(logits) & 15u) == 0 && (row_stride & 3) == 0) ? 0 : 3;
  Plan pl;
  st = make_plan(num_rows, row_stride, k, MI_TOPK_PATH_AUTO, 0, head_max, dev, &pl);
  if (st != MI_TOPK_OK) return st;
  if (pl.ws_bytes > kScratchBytes) return MI_TOPK_ESCRATCH;
  uint8_t* ws = nullptr;
  st = scratch_of(stream, &ws);
  if (st != MI_TOPK_OK) return st;
  // The split path's cross-workgroup waits are bounded; one that gives up
  // leaves its row's counters behind, so that path starts from a cleared
  // region.  The other paths leave the scratch zero whatever the data.
  if (kKinds[pl.kind].mode == kModeSplit) {
    st = fill_zero(ws, pl.ws_bytes, stream);
    if (st != MI_TOPK_OK) return st;
  }
  return topk_impl(logits, row_stride, lengths, num_rows, k, out, ws, kScratchBytes,
                   MI_TOPK_PATH_AUTO, 0, stream);
}

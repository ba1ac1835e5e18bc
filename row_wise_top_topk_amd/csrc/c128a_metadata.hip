// Adaptive-width C128A top-k metadata for DeepSeek-V4-style compressed
// attention, for gfx950 (MI355X).
//
// Every query token of C128A attention (keys compressed 128 to 1) attends to
// all the compressed entries it can see, so its index list is those entries,
// written as int32 rows into buffers whose row stride is a fixed capacity.
// The adaptive width writes only the first `width` entries of each row
// (max(next_pow2(context / ratio), 128) of them) and keeps the capacity
// stride, instead of filling the whole capacity ("[DSv4 Perf] Adaptive topk
// width for dsv4, making #50004 back", sections Test/Perf and Acc).  What a
// row holds, as read here:
//   n = (position + 1) / ratio entries are visible (an entry becomes visible
//   when the last of its `ratio` tokens has been seen); a decode token's row
//   holds their KV-cache slots through its request's block table, a prefill
//   token's row the entry numbers 0..n-1; -1 fills the row up to the width.
//
// The kernel is a pure write stream: per row, one position (and, for decode
// tokens, one request id) is read and `width` int32 are written.  A block
// first reads its rows' positions with one coalesced load into LDS; then each
// wavefront writes whole rows with 16-byte stores (64 lanes x 16 B = 1 KB per
// instruction), so no global load sits between two stores of the write loop.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mi_c128a.h"

#define MI_C128A_EXPORT extern "C" __attribute__((visibility("default")))

namespace mic128a {
namespace {

constexpr int kBlock = 256;
constexpr int kWaves = kBlock / 64;
constexpr int kMaxRowsPerWave = 64;

struct Params {
  const int64_t* positions;
  int64_t num_tokens;
  int64_t num_decode;
  int64_t ratio;
  const int32_t* token_to_req;
  const int32_t* block_table;
  int64_t bt_stride;
  int32_t block_size;
  int32_t bs_log2;  // log2(block_size) when a power of two, else -1
  int32_t* decode_buf;
  int64_t decode_stride;
  int32_t* decode_lens;
  int32_t* prefill_buf;
  int64_t prefill_stride;
  int32_t width;
  int32_t rows_per_wave;
};

// Entry c of a decode row: the KV-cache slot of compressed entry c of the
// request whose block-table row is `table`.
__device__ __forceinline__ int32_t slot_of(const Params& p, const int32_t* table, int32_t c) {
  if (p.bs_log2 >= 0) return (table[c >> p.bs_log2] << p.bs_log2) | (c & (p.block_size - 1));
  return table[c / p.block_size] * p.block_size + c % p.block_size;
}

template <bool kVec>
__global__ void __launch_bounds__(kBlock) c128a_metadata_kernel(Params p) {
  __shared__ int32_t s_shown[kWaves * kMaxRowsPerWave];
  __shared__ int32_t s_req[kWaves * kMaxRowsPerWave];
  const int rows = kWaves * p.rows_per_wave;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * rows;
  for (int i = threadIdx.x; i < rows; i += kBlock) {
    const int64_t t = t0 + i;
    int32_t shown = 0, req = 0;
    if (t < p.num_tokens) {
      const int64_t pos = p.positions[t];
      const int64_t n = pos < 0 ? 0 : (pos + 1) / p.ratio;
      shown = static_cast<int32_t>(n < p.width ? n : p.width);
      if (t < p.num_decode) {
        req = p.token_to_req[t];
        p.decode_lens[t] = shown;
      }
    }
    s_shown[i] = shown;
    s_req[i] = req;
  }
  __syncthreads();
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const int lane = static_cast<int>(__lane_id());
  for (int j = 0; j < p.rows_per_wave; ++j) {
    const int i = w * p.rows_per_wave + j;
    const int64_t t = t0 + i;
    if (t >= p.num_tokens) break;
    const int32_t shown = s_shown[i];
    const bool decode = t < p.num_decode;
    int32_t* row = decode ? p.decode_buf + t * p.decode_stride
                          : p.prefill_buf + (t - p.num_decode) * p.prefill_stride;
    if (!decode) {
      if constexpr (kVec) {
        for (int c = 4 * lane; c < p.width; c += 4 * 64) {
          const int4 v{c < shown ? c : -1, c + 1 < shown ? c + 1 : -1, c + 2 < shown ? c + 2 : -1,
                       c + 3 < shown ? c + 3 : -1};
          *reinterpret_cast<int4*>(row + c) = v;
        }
      } else {
        for (int c = lane; c < p.width; c += 64) row[c] = c < shown ? c : -1;
      }
    } else {
      const int32_t* table = p.block_table + static_cast<int64_t>(s_req[i]) * p.bt_stride;
      if constexpr (kVec) {
        for (int c = 4 * lane; c < p.width; c += 4 * 64) {
          const int4 v{c < shown ? slot_of(p, table, c) : -1, c + 1 < shown ? slot_of(p, table, c + 1) : -1,
                       c + 2 < shown ? slot_of(p, table, c + 2) : -1,
                       c + 3 < shown ? slot_of(p, table, c + 3) : -1};
          *reinterpret_cast<int4*>(row + c) = v;
        }
      } else {
        for (int c = lane; c < p.width; c += 64) row[c] = c < shown ? slot_of(p, table, c) : -1;
      }
    }
  }
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

}  // namespace
}  // namespace mic128a

using namespace mic128a;

MI_C128A_EXPORT int32_t c128a_active_width(int64_t context_len, int32_t compress_ratio) {
  if (context_len < 0 || compress_ratio < 1) return -1;
  const int64_t q = context_len / compress_ratio;
  int64_t w = 1;
  while (w < q) w <<= 1;
  if (w < 128) w = 128;
  return w > INT32_MAX ? -1 : static_cast<int32_t>(w);
}

MI_C128A_EXPORT int c128a_topk_metadata(const int64_t* positions, int64_t num_tokens,
                                        int32_t compress_ratio, int64_t num_decode_tokens,
                                        const int32_t* token_to_req, const int32_t* block_table,
                                        int64_t block_table_stride, int32_t block_size,
                                        int32_t* decode_buf, int64_t decode_stride,
                                        int32_t* decode_lens, int32_t* prefill_buf,
                                        int64_t prefill_stride, int32_t width, hipStream_t stream) {
  if (num_tokens < 0 || compress_ratio < 1 || width < 1 || num_decode_tokens < 0 ||
      num_decode_tokens > num_tokens)
    return MI_C128A_EINVAL;
  if (num_tokens == 0) return MI_C128A_OK;
  if (positions == nullptr || (reinterpret_cast<uintptr_t>(positions) & 7u)) return MI_C128A_EINVAL;
  const bool has_decode = num_decode_tokens > 0;
  const bool has_prefill = num_tokens > num_decode_tokens;
  if (has_prefill && (prefill_buf == nullptr || prefill_stride < width ||
                      (reinterpret_cast<uintptr_t>(prefill_buf) & 3u)))
    return MI_C128A_EINVAL;
  if (has_decode && (decode_buf == nullptr || decode_lens == nullptr || token_to_req == nullptr ||
                     block_table == nullptr || block_size < 1 || block_table_stride < 0 ||
                     decode_stride < width || (reinterpret_cast<uintptr_t>(decode_buf) & 3u) ||
                     (reinterpret_cast<uintptr_t>(decode_lens) & 3u) ||
                     (reinterpret_cast<uintptr_t>(token_to_req) & 3u) ||
                     (reinterpret_cast<uintptr_t>(block_table) & 3u)))
    return MI_C128A_EINVAL;
  Params p;
  p.positions = positions;
  p.num_tokens = num_tokens;
  p.num_decode = num_decode_tokens;
  p.ratio = compress_ratio;
  p.token_to_req = token_to_req;
  p.block_table = block_table;
  p.bt_stride = block_table_stride;
  p.block_size = block_size < 1 ? 1 : block_size;
  p.bs_log2 = (p.block_size & (p.block_size - 1)) == 0 ? __builtin_ctz(static_cast<unsigned>(p.block_size)) : -1;
  p.decode_buf = decode_buf;
  p.decode_stride = decode_stride;
  p.decode_lens = decode_lens;
  p.prefill_buf = prefill_buf;
  p.prefill_stride = prefill_stride;
  p.width = width;
  // about 16 KB of stores per wavefront: one row of 4096 or more entries,
  // else several narrower rows
  int rpw = 4096 / width;
  p.rows_per_wave = rpw < 1 ? 1 : (rpw > kMaxRowsPerWave ? kMaxRowsPerWave : rpw);
  const int64_t rows_per_block = static_cast<int64_t>(kWaves) * p.rows_per_wave;
  const int64_t blocks = (num_tokens + rows_per_block - 1) / rows_per_block;
  if (blocks > INT32_MAX) return MI_C128A_EINVAL;
  const bool vec = (width & 3) == 0 &&
                   (!has_prefill || (aligned16(prefill_buf) && (prefill_stride & 3) == 0)) &&
                   (!has_decode || (aligned16(decode_buf) && (decode_stride & 3) == 0));
  if (vec) {
    hipLaunchKernelGGL(c128a_metadata_kernel<true>, dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0,
                       stream, p);
  } else {
    hipLaunchKernelGGL(c128a_metadata_kernel<false>, dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0,
                       stream, p);
  }
  return hipGetLastError() == hipSuccess ? MI_C128A_OK : MI_C128A_ELAUNCH;
}

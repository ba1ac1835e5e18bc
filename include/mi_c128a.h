/*
 * mi_c128a — adaptive-width C128A top-k metadata for DeepSeek-V4-style
 * compressed attention, for gfx950 (MI355X).  Part of libmi_topk.so.
 *
 * Source: the page "[DSv4 Perf] Adaptive topk width for dsv4, making #50004
 * back".  Section Test/Perf times `build_c128a_topk_metadata(positions,
 * ratio, 0, token_to_req_indices, block_table, 2, slot_mapping,
 * global_decode_buffer, decode_lens_buffer, prefill_buffer,
 * max_compressed_tokens=width)` with width = the capacity (8192) against
 * width = ACTIVE_WIDTH = max(next_pow2(context // ratio), 128) (256 at
 * context 32768); section Acc runs a logical width of 128 inside a capacity
 * row stride of 640.  The page gives the call, the width rule and that the
 * capacity stride is kept; what a row holds is read as follows:
 *
 *   Token t at position p sees n_t = (p + 1) / ratio compressed entries
 *   (entry c covers tokens [c*ratio, (c+1)*ratio) and is visible once its
 *   last token has been seen; n_t = 0 for p < 0).  The first
 *   num_decode_tokens tokens are decode tokens: row t of decode_buf holds the
 *   KV-cache slots of entries 0..n_t-1 of request r = token_to_req[t],
 *       block_table[r * block_table_stride + c / block_size] * block_size
 *         + c % block_size,
 *   and decode_lens[t] = min(n_t, width).  The other tokens are prefill
 *   tokens: row t - num_decode_tokens of prefill_buf holds the entry
 *   numbers 0..n_t-1.  Entries [n_t, width) are -1; a row whose n_t exceeds
 *   the width keeps its first `width` entries (the width rule prevents it).
 *   Entries [width, stride) of every row are never written.
 *
 * All pointers are device pointers owned by the caller; nothing is
 * allocated, freed or synchronised; the work is one kernel on `stream`.
 */
#ifndef MI_C128A_H
#define MI_C128A_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MI_C128A_OK 0
#define MI_C128A_EINVAL 1  /* bad argument; nothing was launched */
#define MI_C128A_ELAUNCH 3 /* the kernel launch failed            */

/*
 * The adaptive width: max(next_pow2(context_len / compress_ratio), 128).
 * Returns -1 for context_len < 0, compress_ratio < 1 or a result above
 * INT32_MAX.  Host only.
 */
int32_t c128a_active_width(int64_t context_len, int32_t compress_ratio);

/*
 * Writes the C128A index rows described above.
 *
 *   positions           int64 [num_tokens], 8-byte aligned.
 *   num_tokens          >= 0 (0 is a no-op).
 *   compress_ratio      >= 1 (128 for C128A).
 *   num_decode_tokens   0 <= num_decode_tokens <= num_tokens.
 *   token_to_req        int32 [num_tokens] (read for decode tokens only).
 *   block_table         int32, a row of page numbers per request, each row
 *                       holding ceil(n_t / block_size) valid entries for its
 *                       decode tokens (not checked).
 *   block_table_stride  entries between two requests' rows, >= 0.
 *   block_size          compressed entries per KV-cache block, >= 1.
 *   decode_buf          int32 [num_decode_tokens, decode_stride].
 *   decode_lens         int32 [num_decode_tokens].
 *   prefill_buf         int32 [num_tokens - num_decode_tokens, prefill_stride].
 *   decode_stride, prefill_stride  the capacity: row stride in entries,
 *                       >= width.
 *   width               entries written per row (max_compressed_tokens), >= 1.
 *
 * The decode arguments may be NULL when num_decode_tokens is 0, prefill_buf
 * when every token is a decode token.  Buffers are 4-byte aligned; 16-byte
 * aligned buffers with width and strides multiple of 4 are written with
 * 16-byte stores.  Returns MI_C128A_OK, MI_C128A_EINVAL (nothing enqueued)
 * or MI_C128A_ELAUNCH.
 */
int c128a_topk_metadata(const int64_t* positions, int64_t num_tokens, int32_t compress_ratio,
                        int64_t num_decode_tokens, const int32_t* token_to_req,
                        const int32_t* block_table, int64_t block_table_stride, int32_t block_size,
                        int32_t* decode_buf, int64_t decode_stride, int32_t* decode_lens,
                        int32_t* prefill_buf, int64_t prefill_stride, int32_t width,
                        hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MI_C128A_H */

/*
 * mi_topk — batched, row-wise, stride-correct top-k index selection over fp32
 * logits, for gfx950 (MI355X).
 *
 * The operation.  For every row i of a batch of fp32 logits, return the column
 * indices of the k largest values among the row's first L_i entries:
 *
 *   - Row i starts i * row_stride elements after `logits`.  row_stride is the
 *     memory stride between rows (torch `stride(0)`), which may exceed the
 *     logical width: the logits producer of the DeepSeek-V4 indexer pads its
 *     max-model-len axis to a multiple of 256 and then slices it, and taking
 *     the width as the stride selects from the wrong memory (vLLM PR #42169
 *     report, "Implementation breakdown" and the csrc/topk.cu excerpt).
 *   - Only entries [0, L_i) of a row are candidates; entries [L_i, row_stride)
 *     are never selected and their contents are irrelevant (SGLang PR #34167
 *     page, TopKCluster::forward excerpt: the scan covers problem.seq_len).
 *   - m_i = min(k, L_i) indices are returned.  Every entry strictly above the
 *     m_i-th largest value v* is included; the remaining slots are taken from
 *     the entries equal to v*, lowest index first (same excerpt: values at or
 *     above the upper bucket bound are always emitted, the threshold bucket is
 *     resolved separately).  Values are compared in IEEE order: -0.0 equals
 *     +0.0 and -inf is an ordinary value.  NaN inside [0, L_i) is outside the
 *     contract: the output is then still m_i distinct indices in [0, L_i).
 *   - Output row i holds the m_i selected indices in ascending order in slots
 *     [0, m_i) and -1 in slots [m_i, k).  Every slot is written.
 *
 * Memory and ownership.  The caller owns every buffer; the library never
 * allocates, frees or synchronises on the call path, and enqueues all work on
 * `stream`.  All pointers passed to topk_indices are device pointers.
 *
 * Workspace.  topk_workspace_size() gives the bytes of device workspace a call
 * needs (0 for batches that one workgroup per row handles).  The workspace
 * must be zero-filled before its first use.  Its counters and histograms are
 * returned to zero by the kernels of every call that returns MI_TOPK_OK (the
 * rest of it is scratch), so one buffer can be reused by consecutive calls on
 * one stream without clearing it again.  Calls that run concurrently
 * (different streams) must use different workspaces.
 * The first 4 bytes of the workspace are a sticky error word: nonzero after a
 * kernel gave up waiting at a cross-workgroup barrier (that call's output is
 * then invalid and the workspace must be zero-filled again).
 */
#ifndef MI_TOPK_H
#define MI_TOPK_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define MI_TOPK_OK 0
#define MI_TOPK_EINVAL 1     /* bad argument; nothing was launched, out untouched */
#define MI_TOPK_EWORKSPACE 2 /* workspace_bytes below topk_workspace_size()       */
#define MI_TOPK_ELAUNCH 3    /* a HIP call failed (launch or device query)         */
#define MI_TOPK_ETOOLONG 4   /* rows too long to keep on chip across the device    */
#define MI_TOPK_ESCRATCH 5   /* batch needs more than MI_TOPK_NOALLOC_WORKSPACE    */

/* Largest k accepted. */
#define MI_TOPK_MAX_K (1 << 24)

/*
 * Bytes of device workspace topk_indices() needs for this batch shape on the
 * current HIP device, for any alignment of `logits`.  Returns 0 when no
 * workspace is needed, and also for arguments topk_indices() would reject.
 */
size_t topk_workspace_size(int64_t num_rows, int64_t row_stride, int32_t k);

/*
 * Row-wise top-k index selection (the operation described above).
 *
 *   logits      device fp32, at least (num_rows-1)*row_stride + max L_i
 *               elements, 4-byte aligned (any 16-byte misalignment is fine).
 *   row_stride  elements between the starts of consecutive rows, >= 1.
 *   lengths     device int32 [num_rows]: L_i.  Values are clamped into
 *               [0, row_stride] on the device; the host never reads them.
 *   num_rows    rows in the batch, 0 <= num_rows <= INT32_MAX; 0 is a no-op.
 *   k           1 <= k <= MI_TOPK_MAX_K.
 *   out         device int32 [num_rows, k], contiguous (row stride k).
 *   workspace   device buffer of workspace_bytes, zero-filled before first use
 *               (see above); may be NULL when topk_workspace_size() is 0.
 *   stream      HIP stream the kernels are enqueued on.
 *
 * Returns MI_TOPK_OK, or a status code above.  On MI_TOPK_EINVAL,
 * MI_TOPK_EWORKSPACE and MI_TOPK_ETOOLONG nothing is enqueued.
 */
int topk_indices(const float* logits, int64_t row_stride, const int32_t* lengths,
                 int64_t num_rows, int32_t k, int32_t* out, void* workspace,
                 size_t workspace_bytes, hipStream_t stream);

/* Static text for a status code. */
const char* topk_status_string(int status);

/*
 * Path control, for cross-checking the kernels' paths against each other on
 * the same input.  `path`:
 *   MI_TOPK_PATH_AUTO   the choice topk_indices() makes;
 *   MI_TOPK_PATH_LOCAL  one workgroup per row holds the whole row on chip
 *                       (rows up to 32768 entries);
 *   MI_TOPK_PATH_SPLIT  `chunks` workgroups per row (0 = automatic) hold one
 *                       chunk each and merge their histograms in workspace
 *                       (a cooperative launch; any k);
 *   MI_TOPK_PATH_CHUNKS one workgroup per 16384-entry chunk of a row; each
 *                       publishes the entries above a bound estimated from
 *                       its own chunk, and the row's last workgroup selects
 *                       among them (an ordinary launch; k <= 4096, `chunks`
 *                       ignored).
 *   MI_TOPK_PATH_PERSIST the kernel MI_TOPK_PATH_AUTO takes, launched on a
 *                       fixed grid of as many workgroups as the device holds
 *                       at once (compute units x the kernel's residency),
 *                       whatever the batch: each workgroup loops over rows
 *                       (or chunks).  The pages' serving paths pair such a
 *                       persistent pool for large batches with a per-row
 *                       cluster for small ones (vLLM PR #42169 report,
 *                       实现拆解: persistent_topk; SGLang PR #34167 page,
 *                       风险与影响 item 5: the persistent-pool path).  The
 *                       cooperative split kernel is launched as usual.
 * topk_workspace_size_path() and topk_indices_path() otherwise behave like
 * topk_workspace_size() and topk_indices().
 */
#define MI_TOPK_PATH_AUTO 0
#define MI_TOPK_PATH_LOCAL 1
#define MI_TOPK_PATH_SPLIT 2
#define MI_TOPK_PATH_CHUNKS 3
#define MI_TOPK_PATH_PERSIST 4

size_t topk_workspace_size_path(int64_t num_rows, int64_t row_stride, int32_t k,
                                int32_t path, int32_t chunks);

int topk_indices_path(const float* logits, int64_t row_stride, const int32_t* lengths,
                      int64_t num_rows, int32_t k, int32_t* out, void* workspace,
                      size_t workspace_bytes, int32_t path, int32_t chunks,
                      hipStream_t stream);

/*
 * topk_indices() with the index transform that follows the selection on a
 * paged KV cache applied as the output is written (the pages' kernels pass
 * their output through a transform as they store it: the report on SGLang
 * PR #34167, section 关键源码片段, `problem_transform`; the page table and
 * block size are those the C128A metadata builder takes: "[DSv4 Perf]
 * Adaptive topk width for dsv4, making #50004 back", section Test/Perf).
 * A selected column j of row i is written as the KV-cache slot
 *     block_table[r * block_table_stride + j / page_size] * page_size
 *       + j % page_size,    r = row_to_req ? row_to_req[i] : i;
 * -1 padding stays -1, and the slots keep the columns' ascending order.
 *   block_table         device int32, a row of page numbers per request; row
 *                       r must hold ceil(L_i / page_size) valid entries for
 *                       every row i of request r (not checked); 4-byte aligned.
 *   block_table_stride  entries between two requests' rows (>= 0).
 *   page_size           columns per page (>= 1; powers of two take shifts).
 *   row_to_req          device int32 [num_rows], or NULL for row i = request i.
 * The slot values must fit int32.  Everything else, the workspace included,
 * as topk_indices() / topk_indices_path().  Returns a status code
 * (MI_TOPK_EINVAL also for a NULL block_table, page_size < 1, a negative
 * stride or a misaligned table or map).
 */
int topk_indices_paged(const float* logits, int64_t row_stride, const int32_t* lengths,
                       int64_t num_rows, int32_t k, int32_t* out, void* workspace,
                       size_t workspace_bytes, const int32_t* block_table,
                       int64_t block_table_stride, int32_t page_size,
                       const int32_t* row_to_req, hipStream_t stream);

int topk_indices_paged_path(const float* logits, int64_t row_stride, const int32_t* lengths,
                            int64_t num_rows, int32_t k, int32_t* out, void* workspace,
                            size_t workspace_bytes, const int32_t* block_table,
                            int64_t block_table_stride, int32_t page_size,
                            const int32_t* row_to_req, int32_t path, int32_t chunks,
                            hipStream_t stream);

/*
 * Value order for a selection: reorders the first m = min(k, L_i) entries of
 * each row of `idx` (the output of topk_indices() for the same logits,
 * row_stride, lengths and k) so that they run from the largest value to the
 * smallest, equal values by ascending column; slots [m, k) are left as they
 * are (-1).  The pages leave the order of the k indices open (their kernels
 * take output slots with atomics); a caller that wants the indices ranked,
 * as a sorted top-k returns them, asks for this order.
 *
 *   logits, row_stride, lengths, num_rows  as for topk_indices().
 *   k           1 <= k <= 4096.
 *   idx         device int32 [num_rows, k], contiguous, read and rewritten in
 *               place; entries of [0, m) outside [0, L_i) are kept (ordered
 *               last) and never dereferenced.
 *   stream      HIP stream the kernel is enqueued on.
 *
 * One kernel launch, no workspace, no allocation.  Returns MI_TOPK_OK,
 * MI_TOPK_EINVAL (nothing enqueued: bad sizes, k above 4096, a NULL
 * pointer with num_rows > 0) or MI_TOPK_ELAUNCH.
 */
int topk_value_order(const float* logits, int64_t row_stride, const int32_t* lengths,
                     int64_t num_rows, int32_t k, int32_t* idx, hipStream_t stream);

/*
 * topk_indices() / topk_indices_path() with the output in value order: the
 * first m = min(k, L_i) entries of each row run from the largest value to
 * the smallest, equal values by ascending column (the set is the same);
 * slots [m, k) hold -1.  The register, streaming and chunked kernels rank the
 * selected entries in their own emission (their keys are on chip, or the row
 * was just read): the composites (key, reversed column) of a row are sorted
 * in LDS.  The cooperative split kernel is followed by the topk_value_order
 * pass.  1 <= k <= 4096; no page table.  Everything else as topk_indices().
 */
int topk_indices_sorted(const float* logits, int64_t row_stride, const int32_t* lengths,
                        int64_t num_rows, int32_t k, int32_t* out, void* workspace,
                        size_t workspace_bytes, hipStream_t stream);

int topk_indices_sorted_path(const float* logits, int64_t row_stride, const int32_t* lengths,
                             int64_t num_rows, int32_t k, int32_t* out, void* workspace,
                             size_t workspace_bytes, int32_t path, int32_t chunks,
                             hipStream_t stream);

/*
 * Describe the launch topk_indices_path() would make, without launching:
 * writes up to 7 int64 values to `info` (path, block threads, elements per
 * thread, chunk elements, chunks per row, grid workgroups, workspace bytes)
 * for a 16-byte-aligned `logits`.  The path is MI_TOPK_PATH_LOCAL, _SPLIT or
 * _CHUNKS, with MI_TOPK_PLAN_PERSIST set for a fixed-grid launch.  Returns a
 * status code.
 */
#define MI_TOPK_PLAN_PERSIST 16
int topk_plan_describe(int64_t num_rows, int64_t row_stride, int32_t k, int32_t path,
                       int32_t chunks, int64_t* info);

/*
 * The same description for a device given by its properties instead of the
 * current one: `cus` compute units, `coop` nonzero if it supports cooperative
 * launches, `split_per_cu` co-resident workgroups of the cooperative split
 * kernel per compute unit (the fixed grids take the other kernels'
 * residencies on gfx950).  Makes no HIP call (the host planning alone, e.g.
 * for tests on a machine without a GPU).  Returns a status code, as
 * topk_plan_describe() (MI_TOPK_EINVAL also for cus < 1 or split_per_cu < 0).
 */
int topk_plan_describe_for(int64_t num_rows, int64_t row_stride, int32_t k, int32_t path,
                           int32_t chunks, int32_t cus, int32_t coop, int32_t split_per_cu,
                           int64_t* info);

/*
 * topk_indices() for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments and result as topk_indices() without the workspace pair:
 * the workspace is a fixed array of MI_TOPK_NOALLOC_WORKSPACE bytes that the
 * library holds on every device it runs on until the process ends.  The call
 * allocates nothing and frees nothing.  On the first call on a device the
 * array's address is looked up and the array is zero-filled (a kernel on
 * `stream`; make that first call outside graph capture, or the fill becomes
 * part of the graph).  Every call on a device shares that device's array:
 * calls that may overlap in time on one device (different streams, or
 * threads without ordering) race and give wrong results; calls ordered on
 * one stream are fine.  Returns MI_TOPK_ESCRATCH, with nothing enqueued,
 * when the batch needs more workspace than the array holds (one 900K-entry
 * row of the chunked path needs about 1.35 MB; topk_workspace_size() gives
 * the need), else as topk_indices().
 */
#define MI_TOPK_NOALLOC_WORKSPACE ((size_t)64 << 20)

int topk_indices_noalloc(const float* logits, int64_t row_stride, const int32_t* lengths,
                         int64_t num_rows, int32_t k, int32_t* out, hipStream_t stream);

/*
 * Diagnostic: the order-preserving key the kernels give each fp32 value
 * (x < y implies key(x) < key(y); -0.0 and +0.0 share a key; every value,
 * NaN included, maps to a key >= 1).  in and out are device arrays of n
 * elements.  Returns a status code.
 */
int topk_debug_keys(const float* in, uint32_t* out, int64_t n, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MI_TOPK_H */

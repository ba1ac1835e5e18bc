"""Python binding of ``libmi_topk.so``: row-wise top-k index selection on gfx950.

Argument marshalling only: every step of the selection runs in the library's
HIP kernels.  PyTorch provides device memory and the stream.  The functions
raise if the library has not been built (``python -m row_wise_top_topk_amd.build``);
there is no fallback implementation.
"""

from __future__ import annotations

import ctypes
import os
import threading

import torch

__all__ = [
    "PATH_AUTO", "PATH_LOCAL", "PATH_SPLIT", "PATH_CHUNKS", "PATH_PERSIST", "PLAN_PERSIST",
    "library_path", "load_library", "topk_indices", "workspace_size",
    "plan_describe", "debug_keys", "workspace_error", "status_string",
    "c128a_active_width", "c128a_topk_metadata",
]

PATH_AUTO, PATH_LOCAL, PATH_SPLIT, PATH_CHUNKS, PATH_PERSIST = 0, 1, 2, 3, 4
PLAN_PERSIST = 16   # set in plan_describe()["path"] for a fixed-grid launch
_PATHS = {"auto": PATH_AUTO, "local": PATH_LOCAL, "split": PATH_SPLIT, "chunks": PATH_CHUNKS,
          "persist": PATH_PERSIST}
MAX_K = 1 << 24

_HERE = os.path.dirname(os.path.abspath(__file__))
_libs: dict = {}
_lib_lock = threading.Lock()
_ws_cache: dict = {}


def library_path() -> str:
    return os.environ.get("MI_TOPK_LIB", os.path.join(_HERE, "libmi_topk.so"))


def _declare(lib: ctypes.CDLL) -> ctypes.CDLL:
    """Argument and result types of every exported function."""
    i64, i32, vp, sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
    lib.topk_workspace_size.argtypes = [i64, i64, i32]
    lib.topk_workspace_size.restype = sz
    lib.topk_workspace_size_path.argtypes = [i64, i64, i32, i32, i32]
    lib.topk_workspace_size_path.restype = sz
    lib.topk_indices.argtypes = [vp, i64, vp, i64, i32, vp, vp, sz, vp]
    lib.topk_indices.restype = ctypes.c_int
    lib.topk_indices_path.argtypes = [vp, i64, vp, i64, i32, vp, vp, sz, i32, i32, vp]
    lib.topk_indices_path.restype = ctypes.c_int
    lib.topk_indices_paged.argtypes = [vp, i64, vp, i64, i32, vp, vp, sz, vp, i64, i32, vp, vp]
    lib.topk_indices_paged.restype = ctypes.c_int
    lib.topk_indices_paged_path.argtypes = [vp, i64, vp, i64, i32, vp, vp, sz, vp, i64, i32, vp,
                                            i32, i32, vp]
    lib.topk_indices_paged_path.restype = ctypes.c_int
    lib.topk_plan_describe.argtypes = [i64, i64, i32, i32, i32, ctypes.POINTER(i64)]
    lib.topk_plan_describe.restype = ctypes.c_int
    lib.topk_plan_describe_for.argtypes = [i64, i64, i32, i32, i32, i32, i32, i32, ctypes.POINTER(i64)]
    lib.topk_plan_describe_for.restype = ctypes.c_int
    lib.topk_status_string.argtypes = [ctypes.c_int]
    lib.topk_status_string.restype = ctypes.c_char_p
    lib.topk_value_order.argtypes = [vp, i64, vp, i64, i32, vp, vp]
    lib.topk_value_order.restype = ctypes.c_int
    lib.topk_debug_keys.argtypes = [vp, vp, i64, vp]
    lib.topk_debug_keys.restype = ctypes.c_int
    lib.topk_indices_sorted.argtypes = [vp, i64, vp, i64, i32, vp, vp, sz, vp]
    lib.topk_indices_sorted.restype = ctypes.c_int
    lib.topk_indices_sorted_path.argtypes = [vp, i64, vp, i64, i32, vp, vp, sz, i32, i32, vp]
    lib.topk_indices_sorted_path.restype = ctypes.c_int
    lib.topk_indices_noalloc.argtypes = [vp, i64, vp, i64, i32, vp, vp]
    lib.topk_indices_noalloc.restype = ctypes.c_int
    lib.c128a_active_width.argtypes = [i64, i32]
    lib.c128a_active_width.restype = i32
    lib.c128a_topk_metadata.argtypes = [vp, i64, i32, i64, vp, vp, i64, i32, vp, i64, vp, vp, i64, i32, vp]
    lib.c128a_topk_metadata.restype = ctypes.c_int
    return lib


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load a build of the library once (default: ``library_path()``); raise
    if it is missing.  Other paths (e.g. a build at another optimisation
    level) are loaded side by side."""
    path = library_path() if path is None else os.path.abspath(path)
    with _lib_lock:
        lib = _libs.get(path)
        if lib is not None:
            return lib
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: build it with `python -m row_wise_top_topk_amd.build`")
        lib = _declare(ctypes.CDLL(path))
        _libs[path] = lib
        return lib


def status_string(status: int) -> str:
    return load_library().topk_status_string(int(status)).decode()


def _check(status: int, what: str) -> None:
    if status != 0:
        raise RuntimeError(f"{what} failed: {status_string(status)} (status {status})")


def _path_id(path) -> int:
    if isinstance(path, str):
        return _PATHS[path]
    return int(path)


def workspace_size(num_rows: int, row_stride: int, k: int, path="auto", chunks: int = 0) -> int:
    """Bytes of zero-filled device workspace a call with this shape needs."""
    return int(load_library().topk_workspace_size_path(
        int(num_rows), int(row_stride), int(k), _path_id(path), int(chunks)))


def plan_describe(num_rows: int, row_stride: int, k: int, path="auto", chunks: int = 0) -> dict:
    """The launch the library makes for this shape (16-byte-aligned logits)."""
    info = (ctypes.c_int64 * 7)()
    _check(load_library().topk_plan_describe(int(num_rows), int(row_stride), int(k),
                                             _path_id(path), int(chunks), info), "topk_plan_describe")
    keys = ("path", "block", "elems_per_thread", "chunk", "chunks_per_row", "grid", "workspace_bytes")
    return dict(zip(keys, (int(v) for v in info)))


def plan_describe_for(num_rows: int, row_stride: int, k: int, path="auto", chunks: int = 0,
                      cus: int = 256, coop: bool = True, split_per_cu: int = 2) -> dict:
    """plan_describe for a device given by its properties (MI355X: 256 CUs);
    host planning only, no device is touched."""
    info = (ctypes.c_int64 * 7)()
    _check(load_library().topk_plan_describe_for(int(num_rows), int(row_stride), int(k),
                                                 _path_id(path), int(chunks), int(cus),
                                                 int(bool(coop)), int(split_per_cu), info),
           "topk_plan_describe_for")
    keys = ("path", "block", "elems_per_thread", "chunk", "chunks_per_row", "grid", "workspace_bytes")
    return dict(zip(keys, (int(v) for v in info)))


def _cached_workspace(device: torch.device, stream: int, nbytes: int) -> torch.Tensor:
    key = (device.index, stream)
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < nbytes:
        if torch.cuda.is_current_stream_capturing():
            raise RuntimeError(
                "topk_indices needs a workspace for this shape and is called under stream "
                "capture, where it allocates nothing: pass workspace= (zero-filled, "
                "workspace_size() bytes) allocated before the capture")
        ws = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
        _ws_cache[key] = ws
    return ws


def topk_indices(logits: torch.Tensor, lengths: torch.Tensor, k: int, out: torch.Tensor = None,
                 workspace: torch.Tensor = None, path="auto", chunks: int = 0,
                 block_table: torch.Tensor = None, page_size: int = 1,
                 row_to_req: torch.Tensor = None, order: str = "column",
                 library: str | None = None, check_workspace: bool = False) -> torch.Tensor:
    """Indices of the k largest of ``logits[i, :L_i]`` for every row i, where
    ``L_i = lengths[i]`` clamped into ``[0, logits.stride(0)]``.

    ``logits``: float32 device tensor, 2-D, ``stride(1) == 1``; ``stride(0)``
    is passed as the row stride (it may exceed the width: a view sliced from
    a padded buffer).  ``lengths``: int32 device tensor ``[rows]``.  Lengths
    are clamped to the row stride, not to ``logits.shape[1]``: entries between
    the width and the stride of a sliced view are read when a length exceeds
    the width, so keep ``lengths <= logits.shape[1]`` unless that memory is
    yours (on the last row it may lie past the tensor's storage).  Returns
    int32 ``[rows, k]``: selected indices in ascending order, then -1.

    ``workspace`` (uint8, zero-filled before its first use, at least
    ``workspace_size()`` bytes) is allocated and cached per stream when not
    given; under stream capture nothing is allocated, and a call that needs a
    workspace and has none raises.  The workspace's first word is a sticky
    error flag (a cross-workgroup wait of the cooperative split path gave up);
    ``check_workspace=True`` reads it after the call (a synchronisation), and
    on a set flag zero-fills the workspace and raises.

    With ``block_table`` (int32 device tensor ``[requests, pages]``, unit
    stride along its last axis) each selected column j of row i is written as
    the KV-cache slot ``block_table[r, j // page_size] * page_size + j %
    page_size``, ``r = row_to_req[i]`` (int32 ``[rows]``; default ``i``), and
    -1 stays -1 (topk_indices_paged).

    ``order="value"`` returns each row's selected columns from the largest
    value to the smallest (equal values by ascending column) instead of in
    ascending column order, ranked inside the selection kernels
    (topk_indices_sorted_path; k <= 4096, not with a page table).

    ``library``: path of another build of the library to call (default: the
    in-tree ``libmi_topk.so``).
    """
    lib = load_library(library)
    if not isinstance(logits, torch.Tensor) or logits.dtype != torch.float32 or logits.dim() != 2:
        raise ValueError("logits must be a 2-D float32 tensor")
    if not logits.is_cuda:
        raise ValueError("logits must be on a GPU")
    if logits.shape[0] > 0 and logits.shape[1] > 1 and logits.stride(1) != 1:
        raise ValueError("logits must have unit stride along its last axis")
    if lengths.dtype != torch.int32 or lengths.dim() != 1 or lengths.device != logits.device:
        raise ValueError("lengths must be a 1-D int32 tensor on the logits' device")
    if not lengths.is_contiguous():
        raise ValueError("lengths must be contiguous")
    rows = int(logits.shape[0])
    if lengths.shape[0] != rows:
        raise ValueError("lengths must have one entry per row")
    k = int(k)
    if not 1 <= k <= MAX_K:
        raise ValueError(f"k must be in [1, {MAX_K}]")
    row_stride = int(logits.stride(0)) if rows > 1 else max(int(logits.stride(0)), int(logits.shape[1]), 1)
    device = logits.device
    if out is None:
        out = torch.empty((rows, k), dtype=torch.int32, device=device)
    elif (out.dtype != torch.int32 or tuple(out.shape) != (rows, k) or not out.is_contiguous()
          or out.device != device):
        raise ValueError("out must be a contiguous int32 [rows, k] tensor on the logits' device")
    if order not in ("column", "value"):
        raise ValueError("order must be 'column' or 'value'")
    if order == "value" and (k > 4096 or block_table is not None):
        raise ValueError("order='value' takes k <= 4096 and no page table")
    if rows == 0:
        return out
    pid = _path_id(path)
    stream = torch.cuda.current_stream(device).cuda_stream
    need = int(lib.topk_workspace_size_path(rows, row_stride, k, pid, int(chunks)))
    ws_ptr, ws_bytes = None, 0
    if need > 0:
        if workspace is None:
            workspace = _cached_workspace(device, stream, need)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    if block_table is None:
        fn = lib.topk_indices_sorted_path if order == "value" else lib.topk_indices_path
        with torch.cuda.device(device):
            st = fn(logits.data_ptr(), row_stride, lengths.data_ptr(), rows, k,
                    out.data_ptr(), ws_ptr, ws_bytes, pid, int(chunks), stream)
        _check(st, "topk_indices")
    else:
        if (block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.device != device
                or (block_table.shape[1] > 1 and block_table.stride(1) != 1)):
            raise ValueError("block_table must be a 2-D int32 tensor on the logits' device with unit "
                             "stride along its last axis")
        req_ptr = None
        if row_to_req is not None:
            if (row_to_req.dtype != torch.int32 or row_to_req.dim() != 1 or row_to_req.shape[0] != rows
                    or not row_to_req.is_contiguous() or row_to_req.device != device):
                raise ValueError("row_to_req must be a contiguous 1-D int32 tensor with one entry per row")
            req_ptr = row_to_req.data_ptr()
        with torch.cuda.device(device):
            st = lib.topk_indices_paged_path(logits.data_ptr(), row_stride, lengths.data_ptr(), rows, k,
                                             out.data_ptr(), ws_ptr, ws_bytes, block_table.data_ptr(),
                                             int(block_table.stride(0)), int(page_size), req_ptr, pid,
                                             int(chunks), stream)
        _check(st, "topk_indices_paged")
    if check_workspace and workspace is not None and need > 0 and workspace_error(workspace):
        workspace.zero_()
        raise RuntimeError("a cross-workgroup wait of the split path gave up: this call's output "
                           "is invalid (the workspace has been zero-filled again)")
    return out


def workspace_error(workspace: torch.Tensor) -> int:
    """The sticky error word of a workspace (nonzero: a barrier wait gave up)."""
    return int(workspace[:4].view(torch.int32).item())


def debug_keys(x: torch.Tensor) -> torch.Tensor:
    """The kernels' order-preserving uint32 key of each float32 value (as int32 bits)."""
    if x.dtype != torch.float32 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous float32 GPU tensor")
    out = torch.empty(x.shape, dtype=torch.int32, device=x.device)
    stream = torch.cuda.current_stream(x.device).cuda_stream
    with torch.cuda.device(x.device):
        _check(load_library().topk_debug_keys(x.data_ptr(), out.data_ptr(), x.numel(), stream),
               "topk_debug_keys")
    return out


def c128a_active_width(context_len: int, compress_ratio: int = 128) -> int:
    """The adaptive C128A width, max(next_pow2(context_len // compress_ratio), 128)."""
    w = int(load_library().c128a_active_width(int(context_len), int(compress_ratio)))
    if w < 0:
        raise ValueError("context_len must be >= 0 and compress_ratio >= 1")
    return w


def c128a_topk_metadata(positions: torch.Tensor, compress_ratio: int, num_decode_tokens: int,
                        token_to_req: torch.Tensor, block_table: torch.Tensor, block_size: int,
                        decode_buf: torch.Tensor, decode_lens: torch.Tensor,
                        prefill_buf: torch.Tensor, width: int) -> None:
    """The C128A index rows (c128a_topk_metadata in mi_c128a.h): writes the
    first ``width`` entries of every row of ``decode_buf`` (the first
    ``num_decode_tokens`` tokens: KV-cache slots through ``block_table``) and
    ``prefill_buf`` (the other tokens: entry numbers), and ``decode_lens``;
    the buffers' row strides (the capacity) are kept.  ``positions`` int64
    [tokens]; ``token_to_req`` int32 [tokens]; ``block_table`` int32
    [requests, pages]; the buffers int32 2-D with unit stride along their
    last axis.  Decode arguments may be None when there are no decode tokens."""
    lib = load_library()
    dev = positions.device
    if positions.dtype != torch.int64 or positions.dim() != 1 or not positions.is_contiguous():
        raise ValueError("positions must be a contiguous 1-D int64 tensor")
    T = int(positions.shape[0])
    nd = int(num_decode_tokens)

    def ptr(t, dtype, what, dims):
        if t is None:
            return None, 0
        if t.dtype != dtype or t.dim() != dims or t.device != dev:
            raise ValueError(f"{what} must be a {dims}-D {dtype} tensor on the positions' device")
        if dims == 2 and t.shape[1] > 1 and t.stride(1) != 1:
            raise ValueError(f"{what} must have unit stride along its last axis")
        if dims == 1 and not t.is_contiguous():
            raise ValueError(f"{what} must be contiguous")
        return t.data_ptr(), (int(t.stride(0)) if dims == 2 else 0)

    tr, _ = ptr(token_to_req, torch.int32, "token_to_req", 1)
    bt, bts = ptr(block_table, torch.int32, "block_table", 2)
    db, ds = ptr(decode_buf, torch.int32, "decode_buf", 2)
    dl, _ = ptr(decode_lens, torch.int32, "decode_lens", 1)
    pb, ps = ptr(prefill_buf, torch.int32, "prefill_buf", 2)
    if nd > 0 and None not in (decode_buf, decode_lens, token_to_req) and (
            decode_buf.shape[0] < nd or decode_lens.shape[0] < nd or token_to_req.shape[0] < nd):
        raise ValueError("decode buffers must have a row per decode token")
    if T > nd and prefill_buf.shape[0] < T - nd:
        raise ValueError("prefill_buf must have a row per prefill token")
    stream = torch.cuda.current_stream(dev).cuda_stream
    with torch.cuda.device(dev):
        st = lib.c128a_topk_metadata(positions.data_ptr(), T, int(compress_ratio), nd, tr, bt, bts,
                                     int(block_size), db, ds, dl, pb, ps, int(width), stream)
    if st != 0:
        raise RuntimeError(f"c128a_topk_metadata failed (status {st})")


def value_order(logits: torch.Tensor, lengths: torch.Tensor, idx: torch.Tensor) -> torch.Tensor:
    """Reorder an existing selection ``idx`` (int32 [rows, k], the output of
    topk_indices for the same logits and lengths) by value, in place
    (topk_value_order: a separate pass that reads the selected values back)."""
    rows, k = int(idx.shape[0]), int(idx.shape[1])
    row_stride = int(logits.stride(0)) if rows > 1 else max(int(logits.stride(0)), int(logits.shape[1]), 1)
    stream = torch.cuda.current_stream(logits.device).cuda_stream
    with torch.cuda.device(logits.device):
        _check(load_library().topk_value_order(logits.data_ptr(), row_stride, lengths.data_ptr(), rows, k,
                                               idx.data_ptr(), stream), "topk_value_order")
    return idx

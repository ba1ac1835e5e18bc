"""Shared helpers for the GPU parity tests (inputs come from ``workloads``;
expected values from the CPU oracle only)."""

import numpy as np
import torch

import row_wise_top_topk_amd as mt
from oracle import check_row, oracle_topk, row_view

SENTINEL = 0x7F7F7F7F


def device_view(w, dev="cuda:0", offset=0):
    """Copy a workload's flat buffer to the GPU, optionally shifted by
    ``offset`` elements, and return the [rows, row_stride] strided view the
    library reads (stride(0) == row_stride)."""
    flat = torch.empty(w.flat.numel() + offset + 8, dtype=torch.float32, device=dev)
    flat[offset:offset + w.flat.numel()].copy_(w.flat)
    width = max(1, w.row_stride)
    logits = flat.as_strided((w.num_rows, width), (w.row_stride, 1), storage_offset=offset)
    lengths = w.lengths.to(dev)
    return logits, lengths


def run_gpu(w, path="auto", chunks=0, offset=0, k=None, dev="cuda:0"):
    k = w.k if k is None else k
    logits, lengths = device_view(w, dev, offset)
    out = torch.full((w.num_rows, k), SENTINEL, dtype=torch.int32, device=dev)
    mt.topk_indices(logits, lengths, k, out=out, path=path, chunks=chunks)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def expected(w, k=None, rows=None):
    k = w.k if k is None else k
    return oracle_topk(w.flat.numpy(), w.row_stride, w.lengths.numpy(), w.num_rows, k, rows=rows)


def assert_parity(w, got, k=None, rows=None, label=""):
    """Element-by-element equality with the oracle on every (listed) row;
    on mismatch also report whether the GPU row is at least a valid top-k."""
    k = w.k if k is None else k
    rows = list(range(w.num_rows)) if rows is None else list(rows)
    exp = expected(w, k, rows)
    sub = got[rows] if len(rows) != got.shape[0] else got
    bad = np.nonzero(np.any(sub != exp, axis=1))[0]
    if bad.size:
        r = rows[int(bad[0])]
        x = row_view(w.flat.numpy(), w.row_stride, int(w.lengths[r]), r)
        why = check_row(x, k, got[r])
        raise AssertionError(
            f"{label}: {bad.size} rows differ from the oracle; first row {r} "
            f"(L={int(w.lengths[r])}, k={k}) invariants: {why or 'valid but different'}; "
            f"got[:8]={got[r][:8].tolist()} exp[:8]={exp[int(bad[0])][:8].tolist()}")
    assert not np.any(got == SENTINEL), f"{label}: unwritten output slots"

"""CPU oracle for batched, row-wise, stride-correct top-k index selection.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite, the package smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code, constants or helpers
with the HIP kernels; it is written from the definition of the result, not from
the kernels' algorithm.

What it computes (the plain definition, no radix rounds, no blocking):

* Row addressing.  Row ``i`` starts ``i * row_stride`` elements into the flat
  buffer, where ``row_stride`` is the memory stride between rows and not the
  logical width.  This is the fix described on the vLLM PR #42169 report page
  (section "Implementation breakdown", items 1-2, and the ``csrc/topk.cu``
  excerpt): the logits coming out of the paged MQA-logits producer are padded
  to a multiple of 256 and then sliced, so ``stride(0)`` can exceed
  ``size(1)``; using the width as the stride reads the wrong rows.
* Valid length.  Only the first ``L_i`` entries of row ``i`` are candidates
  (the SGLang PR #34167 page, ``TopKCluster::forward`` excerpt: the loop runs
  over ``problem.seq_len`` / ``local_seq_len`` entries of ``problem.in``).
  ``L_i`` is clamped into ``[0, row_stride]``.
* Selection.  ``m = min(k, L_i)`` indices are returned: every entry strictly
  above the m-th largest value ``v*`` is in the set, and the remaining slots
  are filled from the entries equal to ``v*`` (same excerpt: entries with
  ``val >= v_hi`` are always emitted, the threshold bucket is resolved
  separately by the tie handler).  Among equal values this oracle takes the
  lowest indices first.  Values are compared with IEEE order, so -0.0 and
  +0.0 are equal and -inf is a selectable value.
* Output.  Slots ``[0, m)`` hold the selected indices in ascending order,
  slots ``[m, k)`` hold -1.

Readings where the pages are silent: output order is free (set semantics;
ascending order is used here only to give one canonical form); ties are broken
by lowest index; NaN inside ``L_i`` is outside the contract.

Paged output (``oracle_page_slots``).  On the pages the selection's output
passes through a transform as it is stored (the SGLang PR #34167 page,
section 关键源码片段: ``problem_transform`` on the output pointer; v1's
``topk_transform_kernel``), and the DeepSeek-V4 metadata builder on the
"[DSv4 Perf] Adaptive topk width" page (section Test/Perf) takes a
``block_table`` and a block size.  The transform's formula is not printed;
the reading taken is the ordinary paged-cache lookup: column ``j`` of
request ``r`` lives in page ``block_table[r][j // page_size]`` at offset
``j % page_size``, i.e. slot ``page * page_size + offset``; -1 stays -1.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "oracle_topk_row",
    "oracle_topk",
    "oracle_page_slots",
    "row_view",
    "check_row",
    "is_untied",
]


def _clamp_length(length: int, row_stride: int) -> int:
    """Valid length of a row, clamped into ``[0, row_stride]``."""
    return int(min(max(int(length), 0), int(row_stride)))


def row_view(flat: np.ndarray, row_stride: int, length: int, row: int) -> np.ndarray:
    """The valid prefix of row ``row``: ``flat[row*row_stride : row*row_stride + L]``.

    The stride is in elements (torch ``stride(0)``), never the logical width
    (vLLM PR #42169 report, "Implementation breakdown").
    """
    n = _clamp_length(length, row_stride)
    start = int(row) * int(row_stride)
    return flat[start:start + n]


def oracle_topk_row(x: np.ndarray, k: int, order: str = "column") -> np.ndarray:
    """Top-k indices of one row's valid prefix ``x``; returns int32 of length k.

    A stable sort of ``-x`` orders values from largest to smallest and keeps
    equal values in index order, so its first ``m`` entries are the m largest
    values with ties taken lowest-index first.  ``order="column"`` lists them
    in ascending index order; ``order="value"`` keeps the sort's order (values
    descending, equal values by ascending index), the order of a ranked top-k.
    """
    x = np.asarray(x, dtype=np.float32)
    k = int(k)
    m = min(k, x.shape[0])
    out = np.full(k, -1, dtype=np.int32)
    if m == 0:
        return out
    ranked = np.argsort(-x, kind="stable")[:m]
    if order == "column":
        out[:m] = np.sort(ranked).astype(np.int32)
    elif order == "value":
        out[:m] = ranked.astype(np.int32)
    else:
        raise ValueError(f"unknown order {order!r}")
    return out


def oracle_topk(flat: np.ndarray, row_stride: int, lengths: np.ndarray,
                num_rows: int, k: int, rows=None, order: str = "column") -> np.ndarray:
    """Oracle for a whole batch: int32 ``[len(rows), k]`` (all rows by default)."""
    flat = np.asarray(flat, dtype=np.float32).reshape(-1)
    lengths = np.asarray(lengths).reshape(-1)
    if rows is None:
        rows = range(int(num_rows))
    rows = list(rows)
    out = np.empty((len(rows), int(k)), dtype=np.int32)
    for t, r in enumerate(rows):
        out[t] = oracle_topk_row(row_view(flat, row_stride, lengths[r], r), k, order)
    return out


def oracle_page_slots(indices: np.ndarray, table_row: np.ndarray, page_size: int) -> np.ndarray:
    """One output row's columns written as KV-cache slots through the page
    table row of its request: ``table_row[j // page_size] * page_size +
    j % page_size`` for ``j >= 0``; -1 stays -1 (see the module notes)."""
    out = []
    for j in np.asarray(indices).reshape(-1):
        j = int(j)
        if j < 0:
            out.append(-1)
        else:
            page, offset = divmod(j, int(page_size))
            out.append(int(table_row[page]) * int(page_size) + offset)
    return np.asarray(out, dtype=np.int32)


def _kth_largest(x: np.ndarray, m: int) -> float:
    """The m-th largest value of x counted with multiplicity (m >= 1)."""
    return float(np.sort(x)[x.shape[0] - m])


def is_untied(x: np.ndarray, k: int) -> bool:
    """True when the valid top-k set is unique.

    That holds when ``#{j : x_j >= v*} == m`` (which includes ``L <= k``).
    """
    x = np.asarray(x, dtype=np.float32)
    m = min(int(k), x.shape[0])
    if m == 0 or m == x.shape[0]:
        return True
    v = _kth_largest(x, m)
    return int(np.count_nonzero(x >= v)) == m


def check_row(x: np.ndarray, k: int, o: np.ndarray) -> list:
    """Invariants every valid output row satisfies; returns a list of violations.

    1. slots ``[m, k)`` are -1;
    2. slots ``[0, m)`` are m distinct integers in ``[0, L)``;
    3. every index whose value is strictly above ``v*`` is present;
    4. every selected value is ``>= v*``.
    Order inside ``[0, m)`` is not checked (set semantics).
    """
    x = np.asarray(x, dtype=np.float32)
    o = np.asarray(o).astype(np.int64).reshape(-1)
    k = int(k)
    L = x.shape[0]
    m = min(k, L)
    bad = []
    if o.shape[0] != k:
        return [f"row has {o.shape[0]} slots, expected {k}"]
    if np.any(o[m:] != -1):
        bad.append("padding slots [m, k) are not all -1")
    sel = o[:m]
    if np.any((sel < 0) | (sel >= L)):
        bad.append("selected index outside [0, L)")
        return bad
    if np.unique(sel).shape[0] != m:
        bad.append("selected indices are not distinct")
    if m == 0:
        return bad
    v = _kth_largest(x, m)
    above = np.nonzero(x > v)[0]
    if not np.all(np.isin(above, sel)):
        bad.append("an index with value strictly above the k-th value is missing")
    if np.any(x[sel] < v):
        bad.append("a selected value is below the k-th value")
    return bad

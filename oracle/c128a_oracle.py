"""CPU oracle for the adaptive-width C128A top-k metadata build.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite and the benchmark's CPU-baseline leg
use it.  It shares no code with the HIP kernels.

Source: the page "[DSv4 Perf] Adaptive topk width for dsv4, making #50004
back", sections Test/Perf (the benchmark script: the call of
``build_c128a_topk_metadata`` and the ``ACTIVE_WIDTH`` rule; the timing
table) and Acc (a logical width of 128 inside a capacity row stride of 640).
For DeepSeek-V4's C128A attention (keys compressed 128 to 1) every query
token attends to all compressed entries it can see, so its "top-k" list is
simply those entries, written into int32 rows of a capacity-wide buffer.

What the page states:

* the width rule: ``ACTIVE_WIDTH = max(next_pow2(context // ratio), 128)``,
  which the page prints as 256 for context 32768 and ratio 128, and which the
  Acc run reports as a logical width of 128 for sequences of at most 9037
  tokens;
* only ``width`` entries of each row are written (``max_compressed_tokens``),
  and the row stride stays the capacity (8192 in the benchmark, 640 in the
  Acc run): the entries ``[width, capacity)`` of a row are not written;
* the call takes the tokens' positions, the compress ratio, a count (0 in
  the benchmark), the token-to-request map, a block table and a block size
  (2 in the benchmark), a slot mapping, a decode buffer with a lengths
  buffer, and the prefill buffer.

Readings taken where the page gives only the call (parity unpinned: no
value on the page fixes them):

* R1 visible compressed entries.  Compressed entry c covers tokens
  ``[c*ratio, (c+1)*ratio)`` and is visible to a token at position p once
  complete, i.e. when ``(c+1)*ratio - 1 <= p``: the token sees
  ``n = (p + 1) // ratio`` entries (0 for p < 0).
* R2 the count argument is the number of decode tokens, which come first:
  tokens ``[0, num_decode)`` fill the decode buffer and its lengths, tokens
  ``[num_decode, T)`` fill the prefill buffer (row ``t - num_decode``).
* R3 prefill rows hold the request-local entry numbers ``0 .. n-1``; decode
  rows hold global KV-cache slots through the request's block table:
  ``block_table[r][c // block_size] * block_size + c % block_size`` with
  ``r = token_to_req[t]`` (the benchmark passes a 1 x 1 table with no decode
  tokens, which only works if prefill rows do not use the table).
* R4 entries ``[n, width)`` of a row are -1; a row keeps only its first
  ``width`` entries if ``n`` exceeds the width (the width rule prevents
  that); the decode length is ``min(n, width)``.
* R5 the slot mapping (where each token's own KV is written) does not enter
  the indices under R1-R4 and is not taken.
"""

from __future__ import annotations

import numpy as np

__all__ = ["next_pow2", "active_width", "visible_entries", "oracle_c128a_metadata"]


def next_pow2(n: int) -> int:
    """Smallest power of two >= n (1 for n <= 1)."""
    n = int(n)
    p = 1
    while p < n:
        p *= 2
    return p


def active_width(context_len: int, compress_ratio: int = 128, floor: int = 128) -> int:
    """The adaptive width: max(next_pow2(context_len // compress_ratio), floor)."""
    return max(next_pow2(int(context_len) // int(compress_ratio)), int(floor))


def visible_entries(position: int, compress_ratio: int) -> int:
    """Compressed entries a token at ``position`` sees (reading R1): the
    entries c whose last token ``(c+1)*ratio - 1`` is at or before it."""
    p = int(position)
    if p < 0:
        return 0
    return (p + 1) // int(compress_ratio)


def oracle_c128a_metadata(positions, compress_ratio: int, num_decode: int, token_to_req,
                          block_table, block_size: int, width: int):
    """(decode rows int32 [num_decode, width], decode lengths int32
    [num_decode], prefill rows int32 [T - num_decode, width]), per readings
    R1-R5.  Only the first ``width`` entries of a row are produced: the
    buffers' entries beyond them are never written."""
    positions = np.asarray(positions, dtype=np.int64).reshape(-1)
    T = positions.shape[0]
    num_decode = int(num_decode)
    width = int(width)
    decode = np.full((num_decode, width), -1, dtype=np.int32)
    lens = np.zeros(num_decode, dtype=np.int32)
    prefill = np.full((T - num_decode, width), -1, dtype=np.int32)
    for t in range(T):
        n = visible_entries(positions[t], compress_ratio)
        shown = min(n, width)
        if t < num_decode:
            r = int(np.asarray(token_to_req)[t])
            for c in range(shown):
                page, offset = divmod(c, int(block_size))
                decode[t, c] = int(np.asarray(block_table)[r, page]) * int(block_size) + offset
            lens[t] = shown
        else:
            prefill[t - num_decode, :shown] = np.arange(shown, dtype=np.int32)
    return decode, lens, prefill

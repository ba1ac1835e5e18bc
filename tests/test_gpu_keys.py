"""The kernels' order-preserving key, over every float32 bit pattern.

Walks all non-NaN patterns in increasing IEEE order (-inf, negatives of
decreasing magnitude, -0, +0, positives of increasing magnitude, +inf) and
checks that the device keys strictly increase, except that -0.0 and +0.0
share one key; NaN patterns must map to nonzero keys.
"""

import pytest
import torch

import row_wise_top_topk_amd as mt

pytestmark = pytest.mark.gpu

CHUNK = 1 << 27


def _keys(bits_i64):
    x = bits_i64.to(torch.int32).view(torch.float32).contiguous()
    return mt.debug_keys(x).to(torch.int64) & 0xFFFFFFFF


def test_keys_strictly_increase_over_all_patterns():
    dev = torch.device("cuda:0")
    prev_last = None
    # negatives from -inf (0xFF800000) up to -0.0 (0x80000000): bit patterns descending
    segments = [(0xFF800000, 0x80000000, -1), (0x00000000, 0x7F800000, +1)]
    for first, last, step in segments:
        n_total = (last - first) * step + 1
        for start in range(0, n_total, CHUNK):
            n = min(CHUNK, n_total - start)
            bits = first + step * (start + torch.arange(n, dtype=torch.int64, device=dev))
            k = _keys(bits)
            d = k[1:] - k[:-1]
            if first == 0 and start == 0 and prev_last is not None:
                # +0.0 shares the key of -0.0
                assert int(k[0]) == prev_last
            elif prev_last is not None:
                assert int(k[0]) > prev_last
            assert bool(torch.all(d > 0)), f"not increasing in chunk at {first:#x}+{start}"
            assert bool(torch.all(k > 0))
            prev_last = int(k[-1])


def test_nan_patterns_have_nonzero_keys():
    dev = torch.device("cuda:0")
    for lo, hi in ((0x7F800001, 0x80000000), (0xFF800001, 0x100000000)):
        for start in range(lo, hi, CHUNK):
            n = min(CHUNK, hi - start)
            k = _keys(start + torch.arange(n, dtype=torch.int64, device=dev))
            assert bool(torch.all(k > 0))

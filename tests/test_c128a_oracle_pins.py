"""Pins of the C128A metadata oracle (CPU).

What pins it, against something other than itself:

* the width rule against the values the page prints ("[DSv4 Perf] Adaptive
  topk width for dsv4, making #50004 back": Test/Perf prints active width 256
  for context 32768, compress ratio 128; Acc reports a logical width of 128
  for sequences of at most 9037 tokens, the prompt being 6543);
* next_pow2 against Python's int.bit_length;
* the visibility count against brute force (count the entries c whose last
  token (c+1)*ratio - 1 is at or before the position);
* a hand-worked fixture (tests/golden/c128a_example.json) with decode rows
  through a block table, prefill rows, the -1 tail and a row cut at the
  width;
* spot values, worked by hand, at the page's sizes: capacity 8192 / width
  256 at context 32768, and capacity 640 / width 128 at 9037 tokens;
* planted mistakes (visibility off by one, a width taken from the capacity)
  that the fixture must reject.
"""

import json
import os

import numpy as np
import pytest

from oracle import active_width, next_pow2, oracle_c128a_metadata, visible_entries
import oracle.c128a_oracle as C

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "c128a_example.json")


def test_width_rule_matches_the_page():
    assert active_width(32768, 128) == 256          # Test/Perf: context=32768 ... active=256
    assert active_width(9037, 128) == 128           # Acc: logical width 128 at <= 9037 tokens
    assert active_width(6543, 128) == 128           # Acc: the prompt alone


@pytest.mark.parametrize("ctx,ratio,want", [
    (65536, 128, 512), (100, 128, 128), (16384 + 127, 128, 128), (16384 + 128, 128, 256),
    (32768 + 128, 128, 512), (1 << 20, 128, 8192), (4096, 4, 1024), (0, 128, 128),
])
def test_width_rule_hand_values(ctx, ratio, want):
    assert active_width(ctx, ratio) == want


def test_next_pow2_brute_force():
    assert next_pow2(0) == 1 and next_pow2(1) == 1
    for n in range(2, 5000):
        assert next_pow2(n) == 1 << (n - 1).bit_length()


@pytest.mark.parametrize("ratio", [1, 2, 3, 4, 128])
def test_visible_entries_brute_force(ratio):
    for p in range(-3, 1500):
        brute = sum(1 for c in range(1500) if (c + 1) * ratio - 1 <= p)
        assert visible_entries(p, ratio) == brute, (p, ratio)


def _golden():
    return json.load(open(GOLDEN))


def _run(d, fn=oracle_c128a_metadata):
    return fn(np.array(d["positions"]), d["compress_ratio"], d["num_decode"],
              np.array(d["token_to_req"]), np.array(d["block_table"]), d["block_size"], d["width"])


def test_hand_worked_fixture():
    d = _golden()
    dec, lens, pre = _run(d)
    assert dec.tolist() == d["expected_decode"]
    assert lens.tolist() == d["expected_decode_lens"]
    assert pre.tolist() == d["expected_prefill"]


def test_page_sizes_spot_values():
    # capacity 8192 / width 256 at context 32768, the benchmark's 512 tokens
    # (positions 32256 .. 32767): every row fits the width
    w = active_width(32768, 128)
    pos = np.arange(32768 - 512, 32768)
    _, _, pre = oracle_c128a_metadata(pos, 128, 0, np.zeros(512, np.int32), np.zeros((1, 1), np.int32), 2, w)
    assert pre.shape == (512, 256)
    last = pre[-1]                       # p = 32767 sees 32768 // 128 = 256 entries
    assert last[0] == 0 and last[255] == 255 and np.all(last == np.arange(256))
    assert pre[-2][254] == 254 and pre[-2][255] == -1     # p = 32766: 255 entries
    assert pre[0][251] == 251 and pre[0][252] == -1       # p = 32256: 32257 // 128 = 252
    # capacity 640 / width 128 (the Acc run's shape): p = 9036 sees 70 entries
    _, _, pre2 = oracle_c128a_metadata([9036, 6542, 126, 127], 128, 0, np.zeros(4, np.int32),
                                       np.zeros((1, 1), np.int32), 2, active_width(9037, 128))
    assert pre2.shape == (4, 128)
    assert pre2[0][69] == 69 and pre2[0][70] == -1
    assert pre2[1][50] == 50 and pre2[1][51] == -1        # 6543 // 128 = 51
    assert np.all(pre2[2] == -1)                           # p = 126: no complete entry
    assert pre2[3][0] == 0 and pre2[3][1] == -1            # p = 127: the first one


def test_planted_mistakes_fail_the_fixture(monkeypatch):
    d = _golden()
    # visibility off by one: p // ratio instead of (p + 1) // ratio
    monkeypatch.setattr(C, "visible_entries", lambda p, r: max(int(p), 0) // int(r))
    _, _, pre = _run(d, C.oracle_c128a_metadata)
    assert pre.tolist() != d["expected_prefill"]
    monkeypatch.undo()
    # rows of the capacity instead of the width: not the fixture's shape
    _, _, pre = C.oracle_c128a_metadata(np.array(d["positions"]), d["compress_ratio"], d["num_decode"],
                                        np.array(d["token_to_req"]), np.array(d["block_table"]),
                                        d["block_size"], d["capacity"])
    assert pre.tolist() != d["expected_prefill"]

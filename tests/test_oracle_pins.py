"""Pins of the CPU oracle to things other than itself (no GPU needed).

Each test ties the oracle to an independent source: a hand-worked strided
example checked again by subset enumeration, brute force over every subset of
tiny rows, closed forms (argmax, ramps, L <= k, all-equal, few levels), a
library sort of the values, and planted mistakes that must fail.
"""

import itertools
import json
import os

import numpy as np
import pytest

from oracle import check_row, is_untied, oracle_page_slots, oracle_topk, oracle_topk_row
import oracle.topk_oracle as ot

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "strided_example.json")


def _load_golden():
    with open(GOLDEN) as f:
        d = json.load(f)
    flat = np.array([float(v) for row in d["rows"] for v in row], dtype=np.float32)
    return d, flat


def _valid_sets(x, k):
    """All index sets a correct top-k may return, by enumeration."""
    L = x.shape[0]
    m = min(k, L)
    out = []
    for S in itertools.combinations(range(L), m):
        rest = [j for j in range(L) if j not in S]
        if not rest or min(x[list(S)]) >= max(x[rest]):
            out.append(tuple(S))
    return out


def test_golden_strided_example():
    d, flat = _load_golden()
    got = oracle_topk(flat, d["row_stride"], np.array(d["lengths"]), 3, d["k"])
    assert got.tolist() == d["expected"]
    # the fixture's valid sets are exactly what subset enumeration gives
    for r, L in enumerate(d["lengths"]):
        x = flat[r * d["row_stride"]: r * d["row_stride"] + L]
        assert sorted(_valid_sets(x, d["k"])) == sorted(tuple(s) for s in d["valid_sets"][r])


def test_golden_catches_width_as_stride_and_ignored_length():
    d, flat = _load_golden()
    wrong = oracle_topk(flat, d["width_as_stride_bug"]["wrong_stride"],
                        np.array(d["lengths"]), 3, d["k"])
    assert wrong.tolist() == d["width_as_stride_bug"]["expected_wrong"]
    assert wrong.tolist() != d["expected"]
    full = oracle_topk(flat, d["row_stride"], np.array([8, 8, 8]), 3, d["k"])
    assert full.tolist() == d["length_ignored_bug"]["expected_wrong"]
    assert full.tolist() != d["expected"]


@pytest.mark.parametrize("seed", range(40))
def test_brute_force_tiny_rows(seed):
    rng = np.random.default_rng(seed)
    L = int(rng.integers(0, 9))
    x = rng.integers(-3, 4, size=L).astype(np.float32)   # small integers: many ties
    for k in range(1, L + 2):
        valid = _valid_sets(x, k)
        o = oracle_topk_row(x, k)
        m = min(k, L)
        S = tuple(int(v) for v in o[:m])
        assert S in valid
        # lowest-index tie break == the lexicographically smallest valid set
        assert S == min(valid)
        assert np.all(o[m:] == -1)
        # the checker accepts exactly the valid sets
        for T in itertools.combinations(range(L), m):
            row = np.array(list(T) + [-1] * (k - m), dtype=np.int32)
            assert (check_row(x, k, row) == []) == (T in valid)
        # untied <=> exactly one valid set
        assert is_untied(x, k) == (len(valid) == 1)


def test_k_equals_one_is_argmax():
    rng = np.random.default_rng(7)
    for _ in range(50):
        x = rng.integers(-5, 5, size=int(rng.integers(1, 200))).astype(np.float32)
        assert oracle_topk_row(x, 1)[0] == np.argmax(x)    # first occurrence of the max


def test_short_rows_return_every_index():
    rng = np.random.default_rng(8)
    for L in range(0, 12):
        x = rng.standard_normal(L).astype(np.float32)
        o = oracle_topk_row(x, 12)
        assert o[:L].tolist() == list(range(L))
        assert np.all(o[L:] == -1)


def test_ramps_and_all_equal():
    L, k = 5000, 777
    up = np.arange(L, dtype=np.float32)
    assert oracle_topk_row(up, k).tolist() == list(range(L - k, L))
    down = -np.arange(L, dtype=np.float32)
    assert oracle_topk_row(down, k).tolist() == list(range(k))
    eq = np.full(L, 0.5, dtype=np.float32)
    assert oracle_topk_row(eq, k).tolist() == list(range(k))
    plateau = np.floor(np.arange(L) / 100.0).astype(np.float32)
    o = oracle_topk_row(plateau, k)
    # values 49..43 fill 700 slots; the remaining 77 come from the plateau at
    # value 42, lowest indices first
    need = k - 700
    sel = [j for j in range(L) if plateau[j] >= 43] + \
          [j for j in range(L) if plateau[j] == 42][:need]
    assert o.tolist() == sorted(sel)


def test_levels_by_counts():
    rng = np.random.default_rng(9)
    L, k = 20000, 1500
    x = (rng.integers(0, 16, size=L) - 7.5).astype(np.float32)
    o = oracle_topk_row(x, k)
    levels = np.sort(np.unique(x))[::-1]
    sel, need = [], k
    for v in levels:
        idx = np.nonzero(x == v)[0]
        if idx.size <= need:
            sel.extend(idx.tolist())
            need -= idx.size
        else:
            sel.extend(idx[:need].tolist())
            need = 0
        if need == 0:
            break
    assert o.tolist() == sorted(sel)


@pytest.mark.parametrize("seed", range(10))
def test_selected_values_are_library_top_values(seed):
    rng = np.random.default_rng(100 + seed)
    L = int(rng.integers(1, 5000))
    k = int(rng.integers(1, 3000))
    x = rng.standard_normal(L).astype(np.float32)
    if seed % 2:
        x = np.round(x * 4) / 4          # ties
    o = oracle_topk_row(x, k)
    m = min(k, L)
    assert np.array_equal(np.sort(x[o[:m]]), np.sort(x)[L - m:])
    assert check_row(x, k, o) == []


def test_signed_zero_and_infinity():
    x = np.array([0.0, -0.0, -1.0], dtype=np.float32)
    assert oracle_topk_row(x, 1).tolist() == [0]
    x = np.array([-0.0, -1.0, 0.0, -0.0], dtype=np.float32)
    assert oracle_topk_row(x, 2).tolist() == [0, 2]
    # -inf inside L is a value like any other
    x = np.array([1.0, 2.0] + [-np.inf] * 10, dtype=np.float32)
    assert oracle_topk_row(x, 5).tolist() == [0, 1, 2, 3, 4]


def test_length_is_clamped():
    flat = np.arange(12, dtype=np.float32)
    got = oracle_topk(flat, 4, np.array([-3, 99, 2]), 3, 2)
    assert got.tolist() == [[-1, -1], [2, 3], [0, 1]]


def test_checker_flags_mutations():
    rng = np.random.default_rng(11)
    x = rng.standard_normal(300).astype(np.float32)
    k = 40
    good = oracle_topk_row(x, k)
    assert check_row(x, k, good) == []
    dup = good.copy(); dup[1] = dup[0]
    assert check_row(x, k, dup)
    oob = good.copy(); oob[3] = 300
    assert check_row(x, k, oob)
    neg = good.copy(); neg[3] = -1
    assert check_row(x, k, neg)
    order = np.argsort(-x, kind="stable")
    miss = good.copy(); miss[np.nonzero(good == order[0])[0][0]] = order[k]
    assert check_row(x, k, miss)                    # drops the maximum
    short = oracle_topk_row(x[:10], k)
    pad = short.copy(); pad[15] = 3
    assert check_row(x[:10], k, pad)                # value in a padding slot
    assert check_row(x[:10], k, short[:-1])         # wrong slot count


def _planted_highest_index_ties(x, k, order="column"):
    """A plausible mistake: reversing an ascending sort (highest index on ties)."""
    x = np.asarray(x, dtype=np.float32)
    m = min(k, x.shape[0])
    out = np.full(k, -1, dtype=np.int32)
    out[:m] = np.sort(np.argsort(x, kind="stable")[::-1][:m])
    return out


def _planted_no_padding(x, k, order="column"):
    """A plausible mistake: short rows not padded with -1."""
    x = np.asarray(x, dtype=np.float32)
    m = min(k, x.shape[0])
    out = np.zeros(k, dtype=np.int32)
    out[:m] = np.sort(np.argsort(-x, kind="stable")[:m])
    return out


@pytest.mark.parametrize("planted", [_planted_highest_index_ties, _planted_no_padding])
def test_planted_mistakes_fail_the_pins(monkeypatch, planted):
    monkeypatch.setattr(ot, "oracle_topk_row", planted)
    failed = False
    d, flat = _load_golden()
    got = ot.oracle_topk(flat, d["row_stride"], np.array(d["lengths"]), 3, d["k"])
    failed |= got.tolist() != d["expected"]
    assert failed


# ---- paged output: columns written as KV-cache slots through a page table

def test_page_slots_hand_example():
    # page size 4, the request's pages [7, 2, 11]: column 0 -> page 7, offset 0
    # -> slot 28; 5 -> page 2 (second), offset 1 -> 9; 9 -> page 11, offset 1
    # -> 45; 11 -> page 11, offset 3 -> 47; -1 stays -1
    got = oracle_page_slots(np.array([0, 5, 9, 11, -1]), np.array([7, 2, 11]), 4)
    assert got.tolist() == [28, 9, 45, 47, -1]


@pytest.mark.parametrize("page_size", [1, 3, 16])
def test_page_slots_identity_table_keeps_columns(page_size):
    # pages numbered 0, 1, 2, ... in order: every column maps to itself
    cols = np.array([0, 1, 2, 17, 40, 63, -1, -1])
    table = np.arange(64)
    assert oracle_page_slots(cols, table, page_size).tolist() == cols.tolist()


def test_page_slots_unit_pages_are_a_lookup():
    # one column per page: the slot is the table entry itself
    table = np.array([50, 3, 99, 7, 12])
    cols = np.array([4, 0, 2, -1])
    assert oracle_page_slots(cols, table, 1).tolist() == [12, 50, 99, -1]


# ---- value order: the selected columns ranked by value

def _ranked_by_definition(x, k):
    """Brute force: every index sorted by (value descending, index ascending)
    with Python's own sort, cut to m, then -1."""
    x = [float(v) for v in x]
    m = min(k, len(x))
    ranked = sorted(range(len(x)), key=lambda j: (-x[j], j))[:m]
    return ranked + [-1] * (k - m)


def test_value_order_hand_examples():
    # 7.0 (column 4), then the two 2.0 values in column order, then 0.5 and -0.0
    x = [0.5, -1.0, 2.0, 2.0, 7.0, -0.0]
    assert ot.oracle_topk_row(np.array(x, dtype=np.float32), 3, "value").tolist() == [4, 2, 3]
    assert ot.oracle_topk_row(np.array(x, dtype=np.float32), 5, "value").tolist() == [4, 2, 3, 0, 5]
    # +0.0 and -0.0 are equal values: the lower column first
    assert ot.oracle_topk_row(np.array([0.0, -0.0, -1.0], dtype=np.float32), 2, "value").tolist() == [0, 1]
    assert ot.oracle_topk_row(np.array([-0.0, 0.0, -1.0], dtype=np.float32), 2, "value").tolist() == [0, 1]
    # -inf is a value; a short row is padded
    assert ot.oracle_topk_row(np.array([-np.inf, 1.0], dtype=np.float32), 4, "value").tolist() == [1, 0, -1, -1]


def test_value_order_matches_brute_force_and_the_column_set():
    rng = np.random.default_rng(11)
    for _ in range(300):
        L = int(rng.integers(0, 12))
        k = int(rng.integers(1, 14))
        x = rng.integers(-3, 4, size=L).astype(np.float32)  # many ties
        got = ot.oracle_topk_row(x, k, "value")
        assert got.tolist() == _ranked_by_definition(x, k)
        col = ot.oracle_topk_row(x, k, "column")
        assert sorted(got.tolist()) == sorted(col.tolist())
        m = min(k, L)
        vals = x[got[:m]]
        assert np.all(vals[:-1] >= vals[1:])


def test_value_order_batch_uses_the_row_layout():
    d, flat = _load_golden()
    got = ot.oracle_topk(flat, d["row_stride"], np.array(d["lengths"]), 3, d["k"], order="value")
    col = ot.oracle_topk(flat, d["row_stride"], np.array(d["lengths"]), 3, d["k"])
    assert [sorted(r) for r in got.tolist()] == [sorted(r) for r in col.tolist()]
    with pytest.raises(ValueError):
        ot.oracle_topk_row(np.zeros(3, dtype=np.float32), 2, "random")

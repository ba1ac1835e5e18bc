"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every comparison is element by element on the selected indices (the kernels
emit ascending order and break ties by lowest index, as the oracle does).
Outputs are prefilled with a sentinel so unwritten slots show up.
"""

import json
import os

import numpy as np
import pytest
import torch

import row_wise_top_topk_amd as mt
from oracle import oracle_page_slots, oracle_topk
import workloads
from gpu_util import SENTINEL, assert_parity, device_view, expected, run_gpu

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "strided_example.json")


def test_golden_strided_example():
    d = json.load(open(GOLDEN))
    flat = torch.tensor([float(v) for r in d["rows"] for v in r], dtype=torch.float32)
    w = workloads.Workload("golden", flat, d["row_stride"], torch.tensor(d["lengths"], dtype=torch.int32),
                           len(d["lengths"]), d["k"])
    for path in ("auto", "local", "split"):
        got = run_gpu(w, path=path)
        assert got.tolist() == d["expected"], path


@pytest.mark.parametrize("name", ["tiny", "decode", "long", "prefill", "adversarial"])
def test_named_workloads_match_oracle(name):
    w = workloads.make(name)
    got = run_gpu(w)
    assert_parity(w, got, label=name)


@pytest.mark.parametrize("offset", [1, 2, 3])
@pytest.mark.parametrize("stride", [4097, 5003, 30001])
def test_misaligned_base_and_odd_stride(offset, stride):
    lengths = [1, 5, 511, 512, 513, stride - 3, stride, stride - 1]
    w = workloads.make_custom(len(lengths), stride, lengths, 512, seed=stride + offset, kind="normal")
    for path in ("auto", "split", "chunks"):
        got = run_gpu(w, path=path, offset=offset)
        assert_parity(w, got, label=f"{path} off={offset} stride={stride}")


@pytest.mark.parametrize("kind", ["normal", "bf16", "levels", "equal", "ramp", "outliers"])
def test_local_and_split_agree_with_oracle(kind):
    stride = 20000
    lengths = [20000, 19999, 17, 2048, 2049, 12345, 4096, 16384]
    w = workloads.make_custom(len(lengths), stride, lengths, 2048, seed=7, kind=kind)
    ref = expected(w)
    for path, chunks in (("local", 0), ("split", 0), ("split", 2), ("split", 3), ("split", 7),
                         ("chunks", 0)):
        got = run_gpu(w, path=path, chunks=chunks)
        assert np.array_equal(got, ref), f"{kind} {path} chunks={chunks}"


@pytest.mark.parametrize("k", [1, 31, 255, 512, 1023, 1024, 2048, 4096, 9000])
def test_k_sweep_in_one_process(k):
    lengths = [30000, 8000, 5000, 1, k, k + 1, max(k - 1, 0), 29999]
    w = workloads.make_custom(len(lengths), 30016, lengths, k, seed=k, kind="bf16")
    got = run_gpu(w)
    assert_parity(w, got, label=f"k={k}")
    got = run_gpu(w, path="split", chunks=4)
    assert_parity(w, got, label=f"k={k} split")
    if k <= 4096:
        got = run_gpu(w, path="chunks")
        assert_parity(w, got, label=f"k={k} chunks")


def test_lengths_are_clamped_and_empty_rows_padded():
    w = workloads.make_custom(6, 1000, [0, -5, 3000, 1000, 999, 1], 64, seed=3)
    got = run_gpu(w)
    w.lengths = w.lengths.clamp(0, 1000)       # what the oracle's definition does
    assert_parity(w, got, label="clamp")
    assert np.all(got[0] == -1) and np.all(got[1] == -1)


def test_empty_batch_is_a_noop():
    logits = torch.zeros((0, 128), dtype=torch.float32, device="cuda:0")
    lengths = torch.zeros((0,), dtype=torch.int32, device="cuda:0")
    out = mt.topk_indices(logits, lengths, 8)
    assert out.shape == (0, 8)


def test_special_values():
    stride = 4096
    rows = []
    neg0 = np.zeros(stride, dtype=np.float32); neg0[1::2] = -0.0
    rows.append(neg0)
    infs = np.full(stride, -np.inf, dtype=np.float32); infs[:5] = [1, 2, 3, 4, 5]
    rows.append(infs)
    mixed = np.random.default_rng(5).standard_normal(stride).astype(np.float32)
    mixed[::7] = 0.0; mixed[3::7] = -0.0; mixed[5::11] = np.inf
    rows.append(mixed)
    sub = (np.random.default_rng(6).integers(1, 1 << 23, size=stride, dtype=np.int64)
           | (np.random.default_rng(7).integers(0, 2, size=stride, dtype=np.int64) << 31))
    rows.append(sub.astype(np.uint32).view(np.float32))
    flat = torch.from_numpy(np.concatenate(rows))
    w = workloads.Workload("special", flat, stride, torch.full((4,), stride, dtype=torch.int32), 4, 300)
    for path in ("local", "split", "chunks"):
        assert_parity(w, run_gpu(w, path=path), label=f"special {path}")


def test_random_stress():
    rng = np.random.default_rng(1234)
    for trial in range(60):
        rows = int(rng.integers(1, 40))
        stride = int(rng.integers(1, 70000))
        k = int(rng.integers(1, 3000))
        lengths = rng.integers(-2, stride + 3, size=rows)
        kind = ["normal", "bf16", "levels", "equal", "outliers"][trial % 5]
        w = workloads.make_custom(rows, stride, lengths, k, seed=trial, kind=kind)
        got = run_gpu(w, offset=trial % 4)
        w.lengths = w.lengths.clamp(0, stride)
        assert_parity(w, got, label=f"trial {trial} rows={rows} stride={stride} k={k} {kind}")


def test_random_stress_chunked_path():
    # the chunked path on random long-row shapes (2 to 25 chunks a row),
    # random lengths and k, smooth and tied kinds; one workspace for every
    # call, left all zero each time
    rng = np.random.default_rng(4321)
    kinds = ["normal", "bf16", "levels", "equal", "outliers", "ramp", "tail", "plateau", "fineramp",
             "descending"]
    ws = None
    for trial in range(60):
        rows = int(rng.integers(1, 9))
        stride = int(rng.integers(16385, 400001))
        k = int(rng.integers(1, 4097))
        lengths = rng.integers(-2, stride + 3, size=rows)
        kind = kinds[trial % len(kinds)]
        w = workloads.make_custom(rows, stride, lengths, k, seed=100 + trial, kind=kind)
        need = mt.workspace_size(rows, stride, k, path="chunks")
        if ws is None or ws.numel() < need:
            ws = torch.zeros(need, dtype=torch.uint8, device="cuda:0")
        logits, lens = device_view(w)
        out = mt.topk_indices(logits, lens, k, workspace=ws, path="chunks")
        torch.cuda.synchronize()
        w.lengths = w.lengths.clamp(0, stride)
        label = f"trial {trial} rows={rows} stride={stride} k={k} {kind}"
        assert_parity(w, out.cpu().numpy(), label=label)
        assert int(ws.count_nonzero()) == 0, label


def test_workspace_reuse_across_calls():
    w = workloads.make_custom(16, 50000, 50000, 1024, seed=9, kind="bf16")
    logits, lengths = device_view(w)
    need = mt.workspace_size(16, 50000, 1024, path="split", chunks=5)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda:0")
    ref = expected(w)
    for _ in range(5):
        out = mt.topk_indices(logits, lengths, 1024, workspace=ws, path="split", chunks=5)
        assert np.array_equal(out.cpu().numpy(), ref)
    torch.cuda.synchronize()
    assert mt.workspace_error(ws) == 0


@pytest.mark.parametrize("kind", ["outliers", "normal", "bf16", "equal", "ramp", "levels"])
def test_chunks_long_rows(kind):
    # rows of 19 chunks: sampled bounds, the last-workgroup merge, and (for
    # tied or ordered rows) the streamed exact fallback; lengths cut chunks
    # at odd places
    stride = 300032
    lengths = [300000, 300032, 16385, 45000, 131071]
    w = workloads.make_custom(len(lengths), stride, lengths, 2048, seed=21, kind=kind)
    ref = expected(w)
    for path in ("auto", "chunks"):
        got = run_gpu(w, path=path)
        assert np.array_equal(got, ref), f"{kind} {path}"


@pytest.mark.parametrize("k", [1024, 2048])
@pytest.mark.parametrize("kind", ["normal", "bf16", "ramp", "descending", "fineramp", "plateau"])
def test_chunk_bound_tiers(kind, k):
    # lengths that put a chunk's sample need nd = ceil(3 k n_s / 2L) + 16 in
    # every tier of the sampled bound: each thread's largest sample
    # (nd <= 64), its two largest (<= 256), its four largest (<= 1024), all
    # of them; in ordered rows many of a chunk's largest samples share a
    # thread, which lowers the bound of the first three
    stride = 300032
    lengths = [300000, 131072, 60000, 40000, 20000, 16385]
    w = workloads.make_custom(len(lengths), stride, lengths, k, seed=29, kind=kind)
    ref = expected(w)
    for path in ("auto", "chunks"):
        got = run_gpu(w, path=path)
        assert np.array_equal(got, ref), f"{kind} k={k} {path}"


def test_chunks_path_is_chosen_for_long_rows():
    plan = mt.plan_describe(8, 900096, 2048)
    assert plan["path"] == mt.PATH_CHUNKS
    assert plan["chunks_per_row"] == (900096 + 16383) // 16384
    assert mt.plan_describe(8, 900096, 5000)["path"] == mt.PATH_SPLIT


def test_paths_share_one_workspace():
    # every path returns the workspace to zero, so the paths can alternate
    # on one buffer; tied rows send the chunked path through its fallback
    stride, k = 60000, 1024
    lengths = [60000, 59999, 20000, 16385, 3, 40000]
    w = workloads.make_custom(len(lengths), stride, lengths, k, seed=31, kind="bf16")
    w2 = workloads.make_custom(len(lengths), stride, lengths, k, seed=32, kind="levels")
    need = max(mt.workspace_size(len(lengths), stride, k, path=p) for p in ("split", "chunks"))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda:0")
    for wl in (w, w2):
        logits, lens = device_view(wl)
        ref = expected(wl)
        for path in ("chunks", "split", "chunks", "chunks", "split"):
            out = mt.topk_indices(logits, lens, k, workspace=ws, path=path)
            torch.cuda.synchronize()
            assert np.array_equal(out.cpu().numpy(), ref), path
            assert int(ws.count_nonzero()) == 0, path


def test_chunks_long_workload_leaves_workspace_zero():
    # the small-batch long-context shape (55 chunks per row: the final
    # workgroup reads the chunks' keys in whole 16-byte groups), then tied
    # levels on the same shape (chunks overflow their groups or the union):
    # repeated calls on one workspace, each exact and each leaving it zero
    base = workloads.make("long")
    lengths = base.lengths.tolist()
    wls = [base, workloads.make_custom(base.num_rows, base.row_stride, lengths, base.k,
                                       seed=43, kind="levels")]
    need = mt.workspace_size(base.num_rows, base.row_stride, base.k, path="chunks")
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda:0")
    for wl in wls:
        logits, lens = device_view(wl)
        ref = expected(wl)
        for _ in range(3):
            out = mt.topk_indices(logits, lens, wl.k, workspace=ws, path="chunks")
            torch.cuda.synchronize()
            assert np.array_equal(out.cpu().numpy(), ref)
            assert int(ws.count_nonzero()) == 0


@pytest.mark.parametrize("ties", [3, 10, 40, 200])
@pytest.mark.parametrize("stride,k,path", [(32768, 2048, "auto"), (300032, 2048, "chunks"),
                                           (60000, 1024, "chunks"), (20000, 512, "auto"),
                                           (16384, 1024, "chunks"), (9000, 512, "chunks")])
def test_ties_straddle_the_threshold(stride, k, path, ties):
    # `ties` entries ranked around the k-th all take the k-th value, so the
    # threshold key is tied across the cut: the lowest columns among the
    # ties are selected.  Few ties stay inside a small last bucket (finished
    # by one wavefront), many go through further radix rounds; on the
    # chunked path a row of one chunk (16384 entries or fewer) stops its
    # rounds at the key and counts the ties in its emission.
    rows = 4
    rng = np.random.default_rng(stride * 7 + ties)
    x = rng.standard_normal((rows, stride)).astype(np.float32)
    for r in range(rows):
        order = np.argsort(-x[r], kind="stable")
        v = x[r, order[k - 1]]
        lo = k - 1 - ties // 2
        x[r, order[lo:lo + ties]] = v
    flat = torch.from_numpy(x.reshape(-1))
    lengths = torch.full((rows,), stride, dtype=torch.int32)
    w = workloads.Workload("ties", flat, stride, lengths, rows, k)
    ref = expected(w)
    got = run_gpu(w, path=path)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("page_size", [1, 16, 3])
@pytest.mark.parametrize("path,stride,lengths,k,kind", [
    ("local", 4096, [4096, 100, 1, 3000], 512, "normal"),        # register row kernel, trivial rows
    ("local", 32768, [32768, 30000, 5, 2049], 2048, "normal"),   # streaming row kernel
    ("chunks", 60000, [60000, 17000, 3, 40000], 1024, "bf16"),   # chunked, 16-byte output stores
    ("chunks", 60000, [60000, 17000, 3, 40000], 1023, "normal"), # chunked, scalar output stores
    ("chunks", 131072, [131072, 90000], 1024, "ramp"),           # chunked, streamed fallback
    ("split", 60000, [60000, 17000, 3, 40000], 1024, "normal"),  # cooperative split
])
def test_paged_output(path, stride, lengths, k, kind, page_size):
    # each selected column goes out as its KV-cache slot through the row's
    # request's page table (rows share requests; the table's row stride
    # exceeds its width); -1 padding stays -1
    rows = len(lengths)
    w = workloads.make_custom(rows, stride, lengths, k, seed=stride + k + page_size, kind=kind)
    rng = np.random.default_rng(stride * 3 + page_size)
    row_to_req = np.array([2, 0, 2, 1][:rows], dtype=np.int32)
    n_req, pages = 3, -(-stride // page_size)
    table = np.zeros((n_req, pages + 5), dtype=np.int32)
    for r in range(n_req):
        table[r, :pages] = rng.permutation(n_req * pages)[:pages]
    ref = expected(w)
    want = np.stack([oracle_page_slots(ref[i], table[row_to_req[i]], page_size) for i in range(rows)])
    logits, lens = device_view(w)
    got = mt.topk_indices(logits, lens, k, path=path, block_table=torch.from_numpy(table).cuda(),
                          page_size=page_size, row_to_req=torch.from_numpy(row_to_req).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), want)


def test_paged_output_rejects_bad_arguments():
    w = workloads.make_custom(2, 4096, 4096, 64, seed=1)
    logits, lens = device_view(w)
    table = torch.zeros((2, 4096), dtype=torch.int32, device="cuda:0")
    with pytest.raises(RuntimeError, match="status 1"):
        mt.topk_indices(logits, lens, 64, block_table=table, page_size=0)


def test_chunks_cluster_in_one_chunk():
    # one chunk holds a block of 3000 equal high values: its count exceeds the
    # last workgroup's fixed window, so the union is gathered through the
    # chunk offsets, and the threshold value is tied 3000 ways
    rows, stride, k = 4, 100000, 2048
    rng = np.random.default_rng(41)
    x = rng.standard_normal((rows, stride)).astype(np.float32)
    for r in range(rows):
        start = 16384 + 1000 * r
        x[r, start:start + 3000] = 5.0
    flat = torch.from_numpy(x.reshape(-1))
    lengths = torch.tensor([stride, stride - 7, 99000, 70001], dtype=torch.int32)
    w = workloads.Workload("cluster", flat, stride, lengths, rows, k)
    ref = expected(w)
    for path in ("chunks", "split"):
        got = run_gpu(w, path=path)
        assert np.array_equal(got, ref), path


def _fallback_rows(stride, k):
    """Rows whose chunked union cannot be exact, so the last workgroup
    selects by streaming the row: finite heads followed by -inf (the
    threshold is -inf when fewer than k values are finite), ramps whose top
    k sit in one chunk, plateaus and fine ramps (runs of equal values)."""
    j = np.arange(stride, dtype=np.float64)
    rows = []
    rng = np.random.default_rng(stride + k)
    for f in (0, 1, 100, k // 2, k - 1, k, k + 1, 3 * k, stride // 2):
        x = np.full(stride, -np.inf, dtype=np.float32)
        x[:f] = rng.standard_normal(f).astype(np.float32)
        rows.append(x)
    rows.append(j.astype(np.float32))                          # ascending ramp
    rows.append((-j).astype(np.float32))                       # descending ramp
    rows.append(np.floor(j / 100.0).astype(np.float32))        # plateaus of 100
    rows.append(np.floor(j / 37.0).astype(np.float32))         # plateaus of 37
    rows.append((1.0 + j * 2.0 ** -30).astype(np.float32))     # runs of 128 equal values
    rows.append((1.0 - j * 2.0 ** -30).astype(np.float32))     # the same, descending
    x = np.ones(stride, dtype=np.float32)
    x[stride // 3:] = 2.0                                      # two levels, the top one tied
    rows.append(x)
    x = np.full(stride, 0.25, dtype=np.float32)
    x[::1000] = 3.0                                            # sparse maxima above a constant
    rows.append(x)
    return np.stack(rows)


@pytest.mark.parametrize("stride,k", [(131072, 1024), (131072, 4096), (300032, 2048)])
def test_streamed_fallback_shortcuts(stride, k):
    # the streamed selection starts from what the chunks' union proved: a
    # threshold fixed outright (lower bound equal to the row's largest key),
    # a threshold equal to the lower bound (fewer than k entries above it),
    # or a first round over the key bits below those the bounds share
    x = _fallback_rows(stride, k)
    rows = x.shape[0]
    flat = torch.from_numpy(x.reshape(-1).copy())
    lengths = torch.full((rows,), stride, dtype=torch.int32)
    lengths[1] = stride - 5
    w = workloads.Workload("fallback", flat, stride, lengths, rows, k)
    ref = expected(w)
    for path in ("auto", "chunks"):
        got = run_gpu(w, path=path)
        assert_parity(w, got, label=f"{path} stride {stride} k {k}")


def _structured_rows(rng, rows, stride):
    """Rows built from runs: plateaus of random lengths and levels, ramps of
    random slope (some within one float binade, so that many keys share
    their leading bits), -inf or constant tails at random columns, and
    mixtures, so that the streamed selection meets blocks whose lanes lie
    in one histogram bin, outside the round's prefix, or straddle it."""
    out = np.empty((rows, stride), dtype=np.float32)
    j = np.arange(stride, dtype=np.float64)
    for r in range(rows):
        kind = r % 6
        if kind == 0:    # plateaus
            run = int(rng.integers(1, 400))
            out[r] = np.floor(j / run).astype(np.float32) * np.float32(rng.choice([1.0, -1.0, 0.5]))
        elif kind == 1:  # fine ramp: runs of equal values inside one binade
            out[r] = (1.0 + j * 2.0 ** -int(rng.integers(24, 34))).astype(np.float32)
        elif kind == 2:  # ramp with a random sign and offset
            out[r] = (rng.uniform(-1e4, 1e4) + rng.choice([1.0, -1.0]) * j).astype(np.float32)
        elif kind == 3:  # finite head, then a constant or -inf tail
            f = int(rng.integers(0, stride))
            out[r] = rng.choice([-np.inf, -7.0, 0.0])
            out[r, :f] = rng.standard_normal(f).astype(np.float32)
        elif kind == 4:  # few levels in long runs
            lv = rng.standard_normal(int(rng.integers(2, 9))).astype(np.float32)
            cuts = np.sort(rng.integers(0, stride, size=len(lv) - 1))
            out[r] = lv[np.searchsorted(cuts, np.arange(stride), side="right")]
        else:            # noise on one half, a plateau on the other
            h = stride // 2
            out[r, :h] = rng.standard_normal(h).astype(np.float32)
            out[r, h:] = np.float32(rng.uniform(-3, 3))
            if rng.random() < 0.5:
                out[r] = out[r, ::-1]
    return out


@pytest.mark.parametrize("stride,k", [(131072, 1), (131072, 1024), (131072, 4096), (65536, 2048), (200000, 333)])
def test_streamed_fallback_structured_rows(stride, k):
    # rows of runs, ramps and tails, many of which the chunked path hands to
    # its streamed selection; lengths random, some not a multiple of the
    # streamed block
    rng = np.random.default_rng(stride * 7 + k)
    rows = 36
    x = _structured_rows(rng, rows, stride)
    flat = torch.from_numpy(x.reshape(-1).copy())
    lengths = torch.from_numpy(rng.integers(k + 1, stride + 1, size=rows).astype(np.int32))
    lengths[::4] = stride
    w = workloads.Workload("structured", flat, stride, lengths, rows, k)
    for path in ("auto", "chunks"):
        got = run_gpu(w, path=path)
        assert_parity(w, got, label=f"{path} stride {stride} k {k}")


@pytest.mark.parametrize("name", ["tiny", "decode", "long", "prefill", "adversarial"])
def test_value_order_named_workloads(name):
    # the selected columns ranked by value (descending, ties by column), on
    # the kernel each batch shape takes
    w = workloads.make(name)
    logits, lengths = device_view(w)
    out = torch.full((w.num_rows, w.k), SENTINEL, dtype=torch.int32, device="cuda:0")
    mt.topk_indices(logits, lengths, w.k, out=out, order="value")
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    exp = oracle_topk(w.flat.numpy(), w.row_stride, w.lengths.numpy(), w.num_rows, w.k, order="value")
    bad = np.nonzero(np.any(got != exp, axis=1))[0]
    assert bad.size == 0, f"{name}: {bad.size} rows differ, first {int(bad[0])}"


@pytest.mark.parametrize("k", [1, 2, 3, 64, 65, 1000, 4096])
@pytest.mark.parametrize("kind", ["normal", "bf16", "levels", "equal"])
def test_value_order_k_and_ties(k, kind):
    stride = 6007  # odd stride, ragged lengths, some rows shorter than k
    lengths = [6007, 5000, 4097, 4096, 100, 1, 0, 3000]
    w = workloads.make_custom(len(lengths), stride, lengths, k, seed=90 + k, kind=kind)
    logits, lens = device_view(w, offset=1)
    out = mt.topk_indices(logits, lens, k, order="value")
    torch.cuda.synchronize()
    exp = oracle_topk(w.flat.numpy(), stride, w.lengths.numpy(), w.num_rows, k, order="value")
    assert np.array_equal(out.cpu().numpy(), exp)


@pytest.mark.parametrize("order", ["column", "value"])
@pytest.mark.parametrize("k", [2049, 2500, 3000, 4096])
def test_streaming_list_large_k(k, order):
    # the streaming kernel's filtered list with k above the value-order
    # staging limit (2048): the columns are staged in LDS and written in
    # order, with and without 16-byte rows (k odd or a multiple of 4), and in
    # value order ranked from the written row
    stride = 32768
    lengths = [32768, 32767, 30001, 20000, 16385, 12289, 9000, k, 5]
    assert mt.plan_describe_for(len(lengths), stride, k, path="local")["elems_per_thread"] == 64
    for kind in ("normal", "bf16"):
        w = workloads.make_custom(len(lengths), stride, lengths, k, seed=k + len(kind), kind=kind)
        logits, lens = device_view(w)
        out = torch.full((w.num_rows, k), SENTINEL, dtype=torch.int32, device="cuda:0")
        mt.topk_indices(logits, lens, k, out=out, path="local", order=order)
        torch.cuda.synchronize()
        exp = oracle_topk(w.flat.numpy(), stride, w.lengths.numpy(), w.num_rows, k, order=order)
        got = out.cpu().numpy()
        bad = np.nonzero(np.any(got != exp, axis=1))[0]
        assert bad.size == 0, f"k={k} {order} {kind}: rows {bad.tolist()} differ"


def test_value_order_rejects_bad_arguments():
    w = workloads.make_custom(2, 8192, [8192, 100], 4097, seed=5)
    logits, lens = device_view(w)
    with pytest.raises(ValueError):
        mt.topk_indices(logits, lens, 4097, order="value")
    with pytest.raises(ValueError):
        mt.topk_indices(logits, lens, 16, order="random")


@pytest.mark.parametrize("path", ["local", "chunks", "split", "auto"])
@pytest.mark.parametrize("kind", ["normal", "bf16", "levels", "equal", "ramp"])
def test_value_order_every_path(path, kind):
    # value order ranked inside each emission site: trivial rows (L <= k),
    # rows held in registers, the streaming kernel's list and its exact
    # fallback, the chunked merge, its streamed fallback and one-chunk rows;
    # the cooperative split kernel is followed by the value-order pass
    k = 1024
    stride = 32768 if path == "local" else 131072
    lengths = [stride, stride - 1, 1000, 5000, 8192, 9000, 16385, 3, 4095]
    w = workloads.make_custom(len(lengths), stride, lengths, k, seed=len(kind) + stride, kind=kind)
    logits, lens = device_view(w, offset=1 if path == "split" else 0)
    out = torch.full((w.num_rows, k), SENTINEL, dtype=torch.int32, device="cuda:0")
    mt.topk_indices(logits, lens, k, out=out, path=path, order="value")
    torch.cuda.synchronize()
    exp = oracle_topk(w.flat.numpy(), stride, w.lengths.numpy(), w.num_rows, k, order="value")
    got = out.cpu().numpy()
    bad = np.nonzero(np.any(got != exp, axis=1))[0]
    assert bad.size == 0, f"{path} {kind}: rows {bad.tolist()} differ"


def test_value_order_pass_on_an_existing_selection():
    # topk_value_order: a separate pass that ranks an existing selection
    w = workloads.make_custom(6, 50000, [50000, 20000, 100, 3000, 49999, 1], 2048, seed=4, kind="bf16")
    logits, lens = device_view(w)
    out = mt.topk_indices(logits, lens, 2048)
    mt.value_order(logits, lens, out)
    torch.cuda.synchronize()
    exp = oracle_topk(w.flat.numpy(), 50000, w.lengths.numpy(), 6, 2048, order="value")
    assert np.array_equal(out.cpu().numpy(), exp)


@pytest.mark.parametrize("name", ["tiny", "decode", "long", "prefill", "adversarial"])
def test_persistent_grid_matches_oracle(name):
    # the kernels on their fixed grids: workgroups loop over rows or chunks
    w = workloads.make(name)
    got = run_gpu(w, path="persist")
    assert_parity(w, got, label=f"persist {name}")


def test_persistent_grid_residency_matches_the_host_table():
    # the fixed grid the device reports equals the one host planning derives
    # from the kernels' gfx950 residency (the table topk_plan_describe_for uses)
    import torch as _t
    cus = _t.cuda.get_device_properties(0).multi_processor_count
    for shape in ((4096, 32768, 2048), (4, 4096, 512), (4096, 6000, 64), (8, 900096, 2048)):
        dev = mt.plan_describe(*shape, path="persist")
        host = mt.plan_describe_for(*shape, path="persist", cus=cus)
        assert dev == host, (shape, dev, host)


def test_persistent_grid_random_shapes_and_value_order():
    rng = np.random.default_rng(77)
    for trial in range(40):
        rows = int(rng.integers(1, 700))
        stride = int(rng.integers(100, 40000)) if rows > 64 else int(rng.integers(100, 300000))
        stride = min(stride, 3_000_000 // rows)     # keeps the oracle fast
        k = int(rng.integers(1, 2049))
        lengths = rng.integers(0, stride + 1, size=rows)
        w = workloads.make_custom(rows, stride, lengths, k, seed=500 + trial,
                                  kind=["normal", "bf16", "levels"][trial % 3])
        got = run_gpu(w, path="persist")
        assert_parity(w, got, label=f"persist trial {trial} rows={rows} stride={stride} k={k}")
    w = workloads.make_custom(600, 9000, [9000, 8000, 100, 4097] * 150, 1024, seed=9, kind="bf16")
    logits, lens = device_view(w)
    out = mt.topk_indices(logits, lens, 1024, path="persist", order="value")
    torch.cuda.synchronize()
    exp = oracle_topk(w.flat.numpy(), 9000, w.lengths.numpy(), 600, 1024, order="value")
    assert np.array_equal(out.cpu().numpy(), exp)

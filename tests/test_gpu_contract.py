"""GPU: contract items beyond the named workloads.

* Row offsets past 2^31 elements (byte offsets past 2^33): every kernel
  family addresses rows with 64-bit offsets.  A few rows at both ends of a
  batch whose footprint exceeds 2^31 elements carry data (the rest have
  L_i = 0 and must come back all -1); each data row is compared with the
  oracle.  Addressing mistakes are the class of bug the vLLM PR #42169 report
  is about (执行摘要, 实现拆解).
* NaN inside [0, L_i): outside the value contract, but the output must still
  be m_i distinct columns in [0, L_i) followed by -1 (invariants 1-2).
* The same workloads through the -O1 build of the library: a result that
  depends on the compiler's optimisation choices is the failure the SGLang
  PR #34167 page reports (风险与影响, item 1).
* Width-sliced views: lengths are clamped to the row stride, not the width.
* The cooperative split path under HIP graph capture.
"""

import os

import numpy as np
import pytest
import torch

import row_wise_top_topk_amd as mt
import workloads
from gpu_util import SENTINEL, assert_parity, device_view, expected
from oracle import check_row, oracle_topk, oracle_topk_row

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TWO31 = 1 << 31
O1_LIB = os.path.join(os.path.dirname(mt.__file__), "libmi_topk_O1.so")


def _far_rows(stride, k, kind, path, order="column", seed=0):
    rows = TWO31 // stride + 3
    assert rows * stride > TWO31
    cross = TWO31 // stride                       # the row holding element 2^31
    data = sorted({0, 1, cross - 1, cross, cross + 1, rows - 2, rows - 1})
    print(f"far rows: stride={stride} rows={rows} k={k} path={path} order={order} data={data}",
          flush=True)
    flat = torch.full((rows * stride,), float("nan"), dtype=torch.float32, device=DEV)
    lengths = torch.zeros(rows, dtype=torch.int32)
    host = {}
    for i, r in enumerate(data):
        L = [stride, stride - 5, max(k + 1, stride // 3), stride - 1][i % 4]
        w = workloads.make_custom(1, stride, [L], k, seed=seed + 17 * i, kind=kind)
        flat[r * stride:(r + 1) * stride].copy_(w.flat)
        lengths[r] = L
        host[r] = w.flat[:L].numpy().copy()
    logits = flat.as_strided((rows, stride), (stride, 1))
    out = torch.full((rows, k), SENTINEL, dtype=torch.int32, device=DEV)
    mt.topk_indices(logits, lengths.to(DEV), k, out=out, path=path, order=order)
    torch.cuda.synchronize()
    empty = torch.ones(rows, dtype=torch.bool, device=DEV)
    empty[data] = False
    assert bool((out[empty] == -1).all()), "rows with L_i = 0 must be all -1"
    got = out[data].cpu().numpy()
    for t, r in enumerate(data):
        exp = oracle_topk_row(host[r], k, order=order)
        assert np.array_equal(got[t], exp), f"row {r} (element offset {r * stride})"
    del flat, out, logits
    torch.cuda.empty_cache()


@pytest.mark.parametrize("stride,k,kind,path", [
    (4096, 512, "normal", "auto"),        # register row kernel, 524291 rows
    (32768, 2048, "outliers", "auto"),    # streaming row kernel, 65539 rows
    (2097152, 2048, "outliers", "auto"),  # chunked kernel, 1027 rows of 128 chunks
    (2097152, 5000, "bf16", "auto"),      # cooperative split kernel (k > 4096)
])
def test_row_offsets_beyond_2_31_elements(stride, k, kind, path):
    _far_rows(stride, k, kind, path)


def test_value_order_row_offsets_beyond_2_31_elements():
    _far_rows(32768, 2048, "normal", "auto", order="value", seed=5)


def _nan_rows(stride, k):
    rng = np.random.default_rng(stride + k)
    pos_nan = np.uint32(0x7FC00000)
    neg_nan = np.uint32(0xFFFFFFFF)
    sig_nan = np.uint32(0x7F800001)
    rows = []
    for pattern in (pos_nan, neg_nan, sig_nan):
        x = rng.standard_normal(stride).astype(np.float32)
        at = rng.choice(stride, size=max(1, stride // 100), replace=False)
        x.view(np.uint32)[at] = pattern
        rows.append(x)
    rows.append(np.full(stride, pos_nan, dtype=np.uint32).view(np.float32))   # all NaN
    rows.append(np.full(stride, neg_nan, dtype=np.uint32).view(np.float32))   # all NaN, key 1
    x = np.full(stride, -np.inf, dtype=np.float32)                            # NaN among -inf
    x.view(np.uint32)[::7] = neg_nan
    x[:3] = 1.0
    rows.append(x)
    x = rng.standard_normal(stride).astype(np.float32)                        # mixed signs of NaN
    x.view(np.uint32)[rng.choice(stride, size=3 * k, replace=False)] = np.where(
        rng.random(3 * k) < 0.5, pos_nan, neg_nan).astype(np.uint32)
    rows.append(x)
    return np.stack(rows)


@pytest.mark.parametrize("stride,k,paths", [
    (4096, 512, ("local", "split", "chunks")),     # register row kernel
    (32768, 2048, ("local", "split", "chunks")),   # streaming row kernel
    (200000, 2048, ("auto", "chunks", "split")),   # chunked and split kernels
    (200000, 5000, ("auto",)),                     # split (k > 4096)
])
def test_nan_inside_valid_length_keeps_invariants(stride, k, paths):
    x = _nan_rows(stride, k)
    rows = x.shape[0]
    lengths = np.array([stride, stride - 3, stride // 2, stride, stride - 1, stride, stride][:rows],
                       dtype=np.int32)
    flat = torch.from_numpy(x.reshape(-1).copy())
    w = workloads.Workload("nan", flat, stride, torch.from_numpy(lengths), rows, k)
    for path in paths:
        print(f"nan rows: stride={stride} k={k} path={path}", flush=True)
        logits, lens = device_view(w)
        out = torch.full((rows, k), SENTINEL, dtype=torch.int32, device=DEV)
        mt.topk_indices(logits, lens, k, out=out, path=path)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        for r in range(rows):
            L = int(lengths[r])
            bad = [v for v in check_row(x[r, :L], k, got[r])
                   if "padding" in v or "outside" in v or "distinct" in v or "slots" in v]
            assert not bad, f"{path} row {r}: {bad}"


@pytest.mark.parametrize("name", ["tiny", "decode", "long", "prefill", "adversarial"])
def test_O1_build_matches_oracle(name):
    assert os.path.exists(O1_LIB), "build both libraries first (python -m row_wise_top_topk_amd.build)"
    w = workloads.make(name)
    logits, lengths = device_view(w)
    out = torch.full((w.num_rows, w.k), SENTINEL, dtype=torch.int32, device=DEV)
    mt.topk_indices(logits, lengths, w.k, out=out, library=O1_LIB)
    torch.cuda.synchronize()
    assert_parity(w, out.cpu().numpy(), label=f"-O1 {name}")


@pytest.mark.parametrize("kind", ["normal", "bf16", "levels", "ramp"])
def test_O1_build_every_path(kind):
    stride = 60000
    lengths = [60000, 59999, 17, 2048, 2049, 16385, 40000, 3]
    w = workloads.make_custom(len(lengths), stride, lengths, 1024, seed=11, kind=kind)
    ref = expected(w)
    logits, lens = device_view(w, offset=1)
    for path, k in (("auto", 1024), ("chunks", 1024), ("split", 1024), ("split", 5000)):
        out = torch.full((w.num_rows, k), SENTINEL, dtype=torch.int32, device=DEV)
        mt.topk_indices(logits, lens, k, out=out, path=path, library=O1_LIB)
        torch.cuda.synchronize()
        want = ref if k == 1024 else expected(w, k=k)
        assert np.array_equal(out.cpu().numpy(), want), f"-O1 {kind} {path} k={k}"
    w2 = workloads.make_custom(6, 30000, [30000, 29000, 100, 8000, 4097, 30000], 512, seed=12, kind=kind)
    logits, lens = device_view(w2)
    out = mt.topk_indices(logits, lens, 512, path="local", library=O1_LIB, order="value")
    torch.cuda.synchronize()
    exp = oracle_topk(w2.flat.numpy(), 30000, w2.lengths.numpy(), 6, 512, order="value")
    assert np.array_equal(out.cpu().numpy(), exp)


def test_width_sliced_view_clamps_lengths_to_the_stride():
    # a [rows, 4000] view of a [rows, 5000] buffer: lengths up to the width
    # select inside it; lengths past the width (here inside the allocation,
    # which covers every row's full stride) are clamped to the stride, as
    # the C ABI states, and so read the padding columns
    stride, width, k = 5000, 4000, 256
    lengths = [4000, 3999, 4800, 5000, 7000, 100]
    w = workloads.make_custom(len(lengths), stride, lengths, k, seed=3, kind="normal")
    buf = w.flat.to(DEV)
    view = buf.view(len(lengths), stride)[:, :width]
    assert view.stride(0) == stride and view.shape[1] == width
    out = mt.topk_indices(view, w.lengths.to(DEV), k)
    torch.cuda.synchronize()
    w.lengths = w.lengths.clamp(0, stride)
    assert_parity(w, out.cpu().numpy(), label="width-sliced view")


def test_split_path_under_graph_capture():
    # k > 4096 on rows longer than 32768 takes the cooperative split kernel;
    # a captured call is replayed over new inputs and each replay is checked
    stride, k = 60000, 5000
    lengths = [60000, 41000, 4999, 30000]
    rows = len(lengths)
    assert mt.plan_describe(rows, stride, k)["path"] == mt.PATH_SPLIT
    ins = [workloads.make_custom(rows, stride, lengths, k, seed=80 + i, kind=kind)
           for i, kind in enumerate(("normal", "bf16", "levels"))]
    flat = torch.empty(rows * stride, dtype=torch.float32, device=DEV)
    logits = flat.as_strided((rows, stride), (stride, 1))
    lens = torch.empty(rows, dtype=torch.int32, device=DEV)
    out = torch.full((rows, k), SENTINEL, dtype=torch.int32, device=DEV)
    ws = torch.zeros(mt.workspace_size(rows, stride, k), dtype=torch.uint8, device=DEV)
    flat.copy_(ins[0].flat)
    lens.copy_(ins[0].lengths)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        mt.topk_indices(logits, lens, k, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        mt.topk_indices(logits, lens, k, out=out, workspace=ws)
    torch.cuda.synchronize()
    for rep in range(3):
        for w in ins:
            flat.copy_(w.flat)
            lens.copy_(w.lengths)
            out.fill_(SENTINEL)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            assert_parity(w, out.cpu().numpy(), label=f"split replay {rep} {w.name}")
            assert mt.workspace_error(ws) == 0
            assert int(ws.count_nonzero()) == 0

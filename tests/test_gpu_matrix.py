"""GPU: the validation matrix at scale.

The SGLang PR #34167 page (实现拆解, item 4) validates its kernels with
1500 random stress shapes, 500 CUDA-graph replays and a sweep over k.  Here:
3000 random shapes (20 parts of 150), each run on the automatic path and on
one forced path, and 500+ graph replays over fresh inputs on every kernel,
every result compared element by element with the CPU oracle.  Each part
stops at its first mismatch and names the case.
"""

import numpy as np
import pytest
import torch

import row_wise_top_topk_amd as mt
import workloads
from gpu_util import SENTINEL, assert_parity, device_view, expected

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
KINDS = ["normal", "bf16", "levels", "equal", "outliers", "ramp", "tail", "plateau", "fineramp",
         "descending"]
MAX_ELEMS = 1_500_000       # per case, so that the oracle stays fast


def _case(rng, trial):
    rows = int(rng.integers(1, 25))
    stride = int(np.exp(rng.uniform(0.0, np.log(400_000))))
    stride = max(1, min(stride, MAX_ELEMS // rows))
    if rng.random() < 0.15:
        k = int(rng.integers(4097, 9001))
    else:
        k = max(1, int(np.exp(rng.uniform(0.0, np.log(4096)))))
    lengths = rng.integers(-2, stride + 3, size=rows)
    for i in range(rows):          # lengths at the interesting places
        u = rng.random()
        if u < 0.1:
            lengths[i] = k
        elif u < 0.2:
            lengths[i] = k + 1
        elif u < 0.3:
            lengths[i] = stride
        elif u < 0.35:
            lengths[i] = 0
    kind = KINDS[trial % len(KINDS)]
    offset = int(rng.integers(0, 4))
    return rows, stride, k, lengths, kind, offset


def _forced_path(rng, stride, k):
    choices = ["split"]
    if stride <= 32768:
        choices.append("local")
    if k <= 4096:
        choices.append("chunks")
    return choices[int(rng.integers(0, len(choices)))]


@pytest.mark.parametrize("part", range(20))
def test_random_matrix(part):
    rng = np.random.default_rng(10_000 + part)
    ws = None
    for i in range(150):
        trial = part * 150 + i
        rows, stride, k, lengths, kind, offset = _case(rng, trial)
        w = workloads.make_custom(rows, stride, lengths, k, seed=trial, kind=kind)
        forced = _forced_path(rng, stride, k)
        logits, lens = device_view(w, offset=offset)
        need = max(mt.workspace_size(rows, stride, k), mt.workspace_size(rows, stride, k, path=forced))
        if need and (ws is None or ws.numel() < need):
            ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
        clamped = workloads.Workload(w.name, w.flat, stride, w.lengths.clamp(0, stride), rows, k)
        for path in ("auto", forced):
            out = torch.full((rows, k), SENTINEL, dtype=torch.int32, device=DEV)
            mt.topk_indices(logits, lens, k, out=out, path=path, workspace=ws if need else None)
            torch.cuda.synchronize()
            assert_parity(clamped, out.cpu().numpy(),
                          label=f"trial {trial} {path} rows={rows} stride={stride} k={k} {kind} "
                                f"offset={offset}")
        if ws is not None and i % 25 == 0:
            assert int(ws.count_nonzero()) == 0, f"trial {trial}: workspace left nonzero"


GRAPH_CASES = [
    # (id, rows, stride, lengths, k, replays, page_size)
    ("row", 600, 4096, [4096, 4000, 513, 4096, 100, 0], 512, 100, 0),
    ("stream", 512, 9000, [9000, 8999, 8193, 2048, 2049, 0, 7000], 2048, 60, 0),
    ("chunks", 4, 200000, [200000, 131071, 40000, 3], 2048, 150, 0),
    ("chunks-paged", 6, 60160, [60000, 5000, 1000, 37000, 17000, 60160], 1024, 100, 16),
    ("split", 4, 60000, [60000, 41000, 4999, 30000], 5000, 100, 0),
]


@pytest.mark.parametrize("case", GRAPH_CASES, ids=[c[0] for c in GRAPH_CASES])
def test_graph_replay_matrix(case):
    name, rows, stride, lens_pattern, k, replays, page = case
    lengths = (lens_pattern * (rows // len(lens_pattern) + 1))[:rows]
    flat = torch.empty(rows * stride, dtype=torch.float32, device=DEV)
    logits = flat.as_strided((rows, stride), (stride, 1))
    lens = torch.empty(rows, dtype=torch.int32, device=DEV)
    out = torch.full((rows, k), SENTINEL, dtype=torch.int32, device=DEV)
    need = mt.workspace_size(rows, stride, k)
    ws = torch.zeros(max(need, 1), dtype=torch.uint8, device=DEV)
    paging = {}
    table = None
    if page:
        rng = np.random.default_rng(5)
        pages = -(-stride // page)
        table = rng.permutation(3 * pages)[:pages].astype(np.int32).reshape(1, pages)
        paging = dict(block_table=torch.from_numpy(table).to(DEV), page_size=page,
                      row_to_req=torch.zeros(rows, dtype=torch.int32, device=DEV))

    def call():
        mt.topk_indices(logits, lens, k, out=out, workspace=ws, **paging)

    w0 = workloads.make_custom(rows, stride, lengths, k, seed=1, kind="normal")
    flat.copy_(w0.flat)
    lens.copy_(w0.lengths)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    for rep in range(replays):
        kind = KINDS[rep % len(KINDS)]
        w = workloads.make_custom(rows, stride, lengths, k, seed=1000 + rep, kind=kind)
        flat.copy_(w.flat)
        lens.copy_(w.lengths)
        out.fill_(SENTINEL)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        if page:
            from oracle import oracle_page_slots
            ref = expected(w)
            want = np.stack([oracle_page_slots(ref[i], table[0], page) for i in range(rows)])
            assert np.array_equal(got, want), f"{name} replay {rep} {kind}"
        else:
            assert_parity(w, got, label=f"{name} replay {rep} {kind}")
        if rep % 10 == 0:
            # the program's own eager call on the same buffers between replays
            eager = torch.full_like(out, SENTINEL)
            mt.topk_indices(logits, lens, k, out=eager, workspace=ws, **paging)
            torch.cuda.synchronize()
            assert np.array_equal(eager.cpu().numpy(), got), f"{name} eager after replay {rep}"
    assert int(ws.count_nonzero()) == 0

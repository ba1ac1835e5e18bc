"""GPU: one top-k call captured in a HIP graph and replayed.

The library makes its launch decisions on the host from scalars only
(num_rows, row_stride, k), writes nothing but kernels into the stream and
leaves its workspace zero after every call, so a captured call can be
replayed over new contents of the same buffers.  Each replay is checked
against the CPU oracle element by element, with the test's own eager work
(copies, fills, an eager call) and synchronisations between replays.
"""

import numpy as np
import pytest
import torch

import row_wise_top_topk_amd as mt
import workloads
from gpu_util import SENTINEL, assert_parity

pytestmark = pytest.mark.gpu

CASES = [
    # (row_stride, lengths, k, kinds of the replayed inputs)
    (32768, [32768, 30001, 28673, 16385, 2048, 0] * 100, 2048, ("normal", "bf16", "levels")),
    (300032, [300000, 131071, 40000], 2048, ("outliers", "ramp", "normal")),
    (60160, [60000, 5000, 1000, 37000, 17000], 1024, ("bf16", "equal", "normal")),
    (4096, [4096, 4000, 513, 4096] * 150, 512, ("normal", "levels", "bf16")),
]


@pytest.mark.parametrize("stride,lengths,k,kinds", CASES)
def test_captured_call_replays(stride, lengths, k, kinds):
    dev = torch.device("cuda:0")
    rows = len(lengths)
    ins = [workloads.make_custom(rows, stride, lengths, k, seed=70 + i, kind=kind)
           for i, kind in enumerate(kinds)]
    flat = torch.empty(rows * stride, dtype=torch.float32, device=dev)
    logits = flat.as_strided((rows, stride), (stride, 1))
    lens = torch.empty(rows, dtype=torch.int32, device=dev)
    out = torch.full((rows, k), SENTINEL, dtype=torch.int32, device=dev)
    need = mt.workspace_size(rows, stride, k)
    ws = torch.zeros(max(need, 1), dtype=torch.uint8, device=dev)

    # eager warm-up on a side stream (library set-up happens outside the capture)
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

    for rep in range(2):
        for w in ins:
            flat.copy_(w.flat)
            lens.copy_(w.lengths)
            out.fill_(SENTINEL)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            got = out.cpu().numpy()
            assert_parity(w, got, label=f"replay {rep} {w.name}")
            # an eager call on the same buffers between replays agrees
            eager = mt.topk_indices(logits, lens, k, workspace=ws)
            torch.cuda.synchronize()
            assert np.array_equal(eager.cpu().numpy(), got)
            assert int(ws.count_nonzero()) == 0

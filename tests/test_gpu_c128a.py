"""GPU parity of the C128A metadata kernel against its CPU oracle.

Shapes from the page "[DSv4 Perf] Adaptive topk width for dsv4, making
#50004 back": Test/Perf times 512, 2048, 8192 and 32768 prefill tokens at
positions CONTEXT - T .. CONTEXT - 1 (context 32768, ratio 128), capacity
8192, at the fixed width (8192) and the adaptive width (256); Acc runs
width 128 inside a capacity of 640.  Every written entry is compared with
the oracle; the entries between the width and the capacity must be left as
they were (the buffers are prefilled with a sentinel).
"""

import numpy as np
import pytest
import torch

import row_wise_top_topk_amd as mt
from oracle import active_width, oracle_c128a_metadata

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SENT = 0x5A5A5A5A


def _run(positions, ratio, num_decode, token_to_req, table, block_size, width, capacity,
         buf_offset=0):
    T = len(positions)
    nd = num_decode
    pos = torch.as_tensor(np.asarray(positions, dtype=np.int64)).to(DEV)
    tr = torch.as_tensor(np.asarray(token_to_req, dtype=np.int32)).to(DEV)
    bt = torch.as_tensor(np.asarray(table, dtype=np.int32)).to(DEV)
    dstore = torch.full((max(nd, 1) * capacity + buf_offset,), SENT, dtype=torch.int32, device=DEV)
    pstore = torch.full((max(T - nd, 1) * capacity + buf_offset,), SENT, dtype=torch.int32, device=DEV)
    dbuf = dstore[buf_offset:].view(max(nd, 1), capacity)
    pbuf = pstore[buf_offset:].view(max(T - nd, 1), capacity)
    dlens = torch.full((max(nd, 1),), SENT, dtype=torch.int32, device=DEV)
    mt.c128a_topk_metadata(pos, ratio, nd, tr, bt, block_size, dbuf, dlens, pbuf, width)
    torch.cuda.synchronize()
    return dbuf.cpu().numpy(), dlens.cpu().numpy(), pbuf.cpu().numpy()


def _check(positions, ratio, num_decode, token_to_req, table, block_size, width, capacity, **kw):
    T = len(positions)
    dbuf, dlens, pbuf = _run(positions, ratio, num_decode, token_to_req, table, block_size, width,
                             capacity, **kw)
    dec, lens, pre = oracle_c128a_metadata(positions, ratio, num_decode, token_to_req, table,
                                           block_size, width)
    nd = num_decode
    if nd:
        assert np.array_equal(dbuf[:nd, :width], dec), "decode rows"
        assert np.array_equal(dlens[:nd], lens), "decode lengths"
        assert np.all(dbuf[:nd, width:] == SENT), "decode entries past the width were written"
    if T > nd:
        for r0 in range(0, T - nd, 4096):       # compare in slices (the fixed width is 1 GB)
            sl = slice(r0, min(T - nd, r0 + 4096))
            assert np.array_equal(pbuf[sl, :width], pre[sl]), f"prefill rows {r0}+"
            assert np.all(pbuf[sl, width:] == SENT), "prefill entries past the width were written"


@pytest.mark.parametrize("tokens", [512, 2048, 8192, 32768])
@pytest.mark.parametrize("fixed", [False, True], ids=["adaptive", "fixed"])
def test_page_benchmark_shapes(tokens, fixed):
    context, ratio, capacity = 32768, 128, 8192
    width = capacity if fixed else mt.c128a_active_width(context, ratio)
    assert mt.c128a_active_width(context, ratio) == active_width(context, ratio) == 256
    positions = np.arange(context - tokens, context)
    _check(positions, ratio, 0, np.zeros(tokens, np.int32), np.zeros((1, 1), np.int32), 2,
           width, capacity)


def test_acc_run_shape():
    # width 128 inside a capacity of 640; sequences up to 9037 tokens
    rng = np.random.default_rng(1)
    positions = rng.integers(0, 9037, size=3000)
    width = mt.c128a_active_width(9037, 128)
    assert width == 128
    _check(positions, 128, 0, np.zeros(3000, np.int32), np.zeros((1, 1), np.int32), 2, width, 640)


@pytest.mark.parametrize("block_size", [2, 3, 64])
@pytest.mark.parametrize("width,capacity,offset", [(256, 300, 0), (130, 131, 0), (256, 260, 1)])
def test_decode_and_prefill_tokens(block_size, width, capacity, offset):
    # decode tokens (KV-cache slots through per-request block tables) then
    # prefill tokens; widths that are and are not a multiple of 4, and a
    # buffer that is not 16-byte aligned (4-byte stores)
    rng = np.random.default_rng(block_size * 1000 + width)
    ratio, reqs = 4, 5
    T, nd = 700, 37
    positions = rng.integers(-3, width * ratio + 40, size=T)     # some rows cut at the width
    token_to_req = rng.integers(0, reqs, size=T).astype(np.int32)
    pages = -(-(width + 16) // block_size)
    table = np.stack([rng.permutation(reqs * pages)[:pages] for _ in range(reqs)]).astype(np.int32)
    table = np.concatenate([table, np.full((reqs, 7), -7, np.int32)], axis=1)   # stride > width
    _check(positions, ratio, nd, token_to_req, table, block_size, width, capacity, buf_offset=offset)


def test_only_decode_tokens_and_ratio_one():
    rng = np.random.default_rng(9)
    positions = rng.integers(0, 200, size=64)
    table = rng.permutation(4096)[:256].astype(np.int32).reshape(2, 128)
    tr = rng.integers(0, 2, size=64).astype(np.int32)
    _check(positions, 1, 64, tr, table, 2, 256, 256)


def test_empty_and_bad_arguments():
    pos = torch.zeros(0, dtype=torch.int64, device=DEV)
    buf = torch.zeros((1, 8), dtype=torch.int32, device=DEV)
    mt.c128a_topk_metadata(pos, 128, 0, None, None, 2, None, None, buf, 8)   # no tokens: no-op
    pos = torch.arange(4, dtype=torch.int64, device=DEV)
    narrow = torch.zeros((4, 4), dtype=torch.int32, device=DEV)
    wide = torch.zeros((4, 8), dtype=torch.int32, device=DEV)
    with pytest.raises(RuntimeError):
        mt.c128a_topk_metadata(pos, 128, 0, None, None, 2, None, None, narrow, 8)  # stride < width
    with pytest.raises(RuntimeError):
        mt.c128a_topk_metadata(pos, 0, 0, None, None, 2, None, None, wide, 8)      # ratio 0
    with pytest.raises(RuntimeError):
        mt.c128a_topk_metadata(pos, 128, 2, None, None, 2, None, None, wide, 8)    # decode without buffers

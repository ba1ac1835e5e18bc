"""Host planning (which kernel takes a shape, its grid and workspace), checked
on the CPU through topk_plan_describe_for for an MI355X-like device (256
compute units, cooperative launches, two co-resident split workgroups per
compute unit).  The expected values are derived by hand from the launch
layouts: chunked rows of G = ceil(stride / 16384) workgroups with a per-row
workspace block of 256 + round256(12 G) + G * 4096 * 6 bytes, the split path's
78080-byte row block, and one workgroup per row for short rows.
"""
import pytest

import row_wise_top_topk_amd as mt

HEADER = 256


def chunk_row_bytes(G: int) -> int:
    # arrival counter head; counts, bounds and largest keys; key lists (u32) and
    # column-offset lists (u16)
    return 256 + ((12 * G + 255) // 256) * 256 + G * 4096 * 4 + G * 4096 * 2


SPLIT_ROW_BYTES = (2 + 62) * 4 + (4096 + 6 * 1024) * 4 + 1024 * 4 + 4096 * 8


@pytest.mark.parametrize("shape,expect", [
    # tiny: 4096 entries fit the 256 x 16 register kernel
    ((4, 4096, 512), dict(path=mt.PATH_LOCAL, block=256, elems_per_thread=16, grid=4, workspace_bytes=0)),
    # prefill: many rows of 32768 -> one 512 x 64 streaming workgroup per row
    ((4096, 32768, 2048), dict(path=mt.PATH_LOCAL, block=512, elems_per_thread=64, grid=4096,
                               workspace_bytes=0)),
    # decode, long, adversarial: too few rows to fill 256 CUs -> chunked
    ((64, 60160, 1024), dict(path=mt.PATH_CHUNKS, chunks_per_row=4, grid=256,
                             workspace_bytes=HEADER + 64 * chunk_row_bytes(4))),
    ((8, 900096, 2048), dict(path=mt.PATH_CHUNKS, chunks_per_row=55, grid=440,
                             workspace_bytes=HEADER + 8 * chunk_row_bytes(55))),
    ((256, 131072, 1024), dict(path=mt.PATH_CHUNKS, chunks_per_row=8, grid=2048,
                               workspace_bytes=HEADER + 256 * chunk_row_bytes(8))),
])
def test_named_shapes(shape, expect):
    d = mt.plan_describe_for(*shape)
    for key, v in expect.items():
        assert d[key] == v, (key, d)


def test_long_rows_with_large_k_take_the_cooperative_split_path():
    # k above 4096: G = max(55 chunks of <= 16384, min(512 co-resident / 8 rows, 900096 / 4096))
    # = 64 chunks of 14064, 8 rows per pass
    d = mt.plan_describe_for(8, 900096, 4097)
    assert d["path"] == mt.PATH_SPLIT
    assert (d["chunks_per_row"], d["chunk"], d["grid"]) == (64, 14064, 512)
    assert d["workspace_bytes"] == HEADER + 8 * SPLIT_ROW_BYTES
    with pytest.raises(RuntimeError, match="status 3"):  # no cooperative launches
        mt.plan_describe_for(8, 900096, 4097, coop=False)


def test_misaligned_stride_widens_aligned_kernels():
    # rows of 4095 may start 3 elements past a 16-byte boundary: 4098 > 4096
    assert mt.plan_describe_for(4096, 4095, 64)["block"] == 512
    assert mt.plan_describe_for(4096, 4096, 64)["block"] == 256


def test_few_rows_of_moderate_length_go_chunked():
    d = mt.plan_describe_for(100, 16385, 64)
    assert (d["path"], d["chunks_per_row"]) == (mt.PATH_CHUNKS, 2)
    assert d["workspace_bytes"] == HEADER + 100 * chunk_row_bytes(2)
    # enough rows to fill the device: one workgroup per row
    assert mt.plan_describe_for(600, 16385, 64)["path"] == mt.PATH_LOCAL


def test_forced_paths_and_limits():
    with pytest.raises(RuntimeError, match="status 4"):      # too long for one workgroup
        mt.plan_describe_for(8, 900096, 2048, path="local")
    with pytest.raises(RuntimeError, match="status 1"):      # chunked path takes k <= 4096
        mt.plan_describe_for(8, 900096, 5000, path="chunks")
    with pytest.raises(RuntimeError, match="status 4"):      # more than 1024 chunks per row
        mt.plan_describe_for(1, 1024 * 16384 + 1, 16, path="chunks")
    with pytest.raises(RuntimeError, match="status 1"):      # no compute units
        mt.plan_describe_for(8, 900096, 2048, cus=0)
    assert mt.plan_describe_for(1, 1024 * 16384, 16, path="chunks")["chunks_per_row"] == 1024


@pytest.mark.parametrize("shape,path,grid", [
    ((4096, 32768, 2048), mt.PATH_LOCAL, 3 * 256),   # streaming kernel: 3 workgroups per CU
    ((4, 4096, 512), mt.PATH_LOCAL, 4 * 256),        # register kernel 256 x 16: 4 per CU
    ((4096, 6000, 64), mt.PATH_LOCAL, 2 * 256),      # register kernel 512 x 16: 2 per CU
    ((8, 900096, 2048), mt.PATH_CHUNKS, 2 * 256),    # chunked kernel: 2 per CU
    ((256, 131072, 1024), mt.PATH_CHUNKS, 2 * 256),
])
def test_persistent_grid_is_fixed_by_the_device(shape, path, grid):
    # the fixed grid: the device's compute units times the kernel's residency,
    # whatever the batch; the kernel is the automatic choice
    d = mt.plan_describe_for(*shape, path="persist")
    assert d["path"] == path | mt.PLAN_PERSIST
    assert d["grid"] == grid
    auto = mt.plan_describe_for(*shape)
    assert (d["block"], d["elems_per_thread"], d["chunks_per_row"], d["workspace_bytes"]) == (
        auto["block"], auto["elems_per_thread"], auto["chunks_per_row"], auto["workspace_bytes"])
    half = mt.plan_describe_for(max(1, shape[0] // 2), shape[1], shape[2], path="persist")
    assert half["grid"] == grid


def test_persistent_path_keeps_the_cooperative_split_launch():
    d = mt.plan_describe_for(8, 900096, 4097, path="persist")
    assert d["path"] == mt.PATH_SPLIT and d["grid"] == 512

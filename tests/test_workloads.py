"""The seeded input generators: determinism, shapes and poisoned padding."""

import numpy as np
import pytest
import torch

import workloads


def test_tiny_is_deterministic():
    a = workloads.make("tiny")
    b = workloads.make("tiny")
    assert torch.equal(a.flat, b.flat)
    assert a.num_rows == 4 and a.row_stride == 4096 and a.k == 512
    assert a.flat.numel() == 4 * 4096


@pytest.mark.parametrize("name", ["decode", "long"])
def test_shapes_and_poison(name):
    w = workloads.make(name)
    assert w.flat.dtype == torch.float32
    assert w.flat.numel() == w.num_rows * w.row_stride
    rows = w.flat.view(w.num_rows, w.row_stride)
    for r in range(w.num_rows):
        L = int(w.lengths[r])
        assert 1 <= L <= w.row_stride
        pad = rows[r, L:]
        if r % 2 == 0:
            assert bool(torch.all(pad == 3.0e38))
        else:
            assert bool(torch.all(torch.isnan(pad)))
        assert bool(torch.all(torch.isfinite(rows[r, :L])))
    if name == "decode":
        assert w.row_stride == 60160 and w.k == 1024
        # bf16-rounded values: low 16 bits of every valid value are zero
        bits = rows[0, : int(w.lengths[0])].view(torch.int32)
        assert bool(torch.all((bits & 0xFFFF) == 0))
    else:
        assert w.row_stride == 900096 and int(w.lengths[0]) == 900000
        assert int((rows[0, :900000] > 2.5).sum()) > 3000      # the outliers


def test_custom_lengths_broadcast():
    w = workloads.make_custom(5, 100, 37, 8, seed=1, kind="bf16")
    assert w.lengths.tolist() == [37] * 5
    assert np.isnan(w.flat.view(5, 100)[1, 37:].numpy()).all()

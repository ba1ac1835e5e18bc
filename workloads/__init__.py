"""Seeded synthetic inputs for row-wise top-k selection.

This module only draws data: it holds none of the selection arithmetic and is
shared by the tests, the benchmark and the smoke check as the common source of
inputs for both the HIP path and the CPU oracle.

Every workload is a flat fp32 buffer of ``num_rows * row_stride`` elements,
int32 valid lengths ``L_i`` and a k.  Columns ``[L_i, row_stride)`` are
poisoned (+3.0e38 on even rows, NaN on odd rows) so that any read past the
valid length, or any use of the width as the stride, shows up in the result.

The five named workloads follow the decode, long-context and prefill shapes
that the pages describe (a max-model-len of 900000 padded to 900096 on the
vLLM PR #42169 report page; small-batch decode above the 32K cluster floor and
k in {512, 1024, 2048} on the SGLang PR #34167 page; causal prefill at context
32768 in the benchmark script on the vLLM PR #52823 page).
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

__all__ = ["Workload", "NAMES", "make", "make_custom", "poison_padding"]


@dataclass
class Workload:
    name: str
    flat: torch.Tensor        # float32, CPU, num_rows * row_stride elements
    row_stride: int
    lengths: torch.Tensor     # int32, CPU, [num_rows]
    num_rows: int
    k: int

    @property
    def valid_elements(self) -> int:
        return int(self.lengths.clamp(0, self.row_stride).to(torch.int64).sum())

    def algorithmic_bytes(self) -> int:
        """Valid logits read once + k int32 written + one int32 length, per row."""
        return 4 * self.valid_elements + 4 * self.k * self.num_rows + 4 * self.num_rows


NAMES = ("tiny", "decode", "long", "prefill", "adversarial")


def poison_padding(flat: torch.Tensor, row_stride: int, lengths: torch.Tensor) -> None:
    """Fill columns ``[L_i, row_stride)``: +3.0e38 on even rows, NaN on odd rows."""
    rows = flat.view(-1, row_stride)
    col = torch.arange(row_stride).unsqueeze(0)
    pad = col >= lengths.to(torch.int64).clamp(0, row_stride).unsqueeze(1)
    even = (torch.arange(rows.shape[0]) % 2 == 0).unsqueeze(1)
    rows.masked_fill_(pad & even, 3.0e38)
    rows.masked_fill_(pad & ~even, float("nan"))


def _bf16_round(t: torch.Tensor) -> torch.Tensor:
    return t.to(torch.bfloat16).to(torch.float32)


def _tiny(seed: int) -> Workload:
    g = torch.Generator().manual_seed(seed)
    R, S = 4, 4096
    flat = torch.randn(R * S, generator=g, dtype=torch.float32)
    lengths = torch.full((R,), S, dtype=torch.int32)
    return Workload("tiny", flat, S, lengths, R, 512)


def _decode(seed: int) -> Workload:
    g = torch.Generator().manual_seed(seed)
    R, S = 64, 60160          # 60000 rounded up to a multiple of 256
    lengths = torch.randint(1, 60001, (R,), generator=g, dtype=torch.int32)
    flat = _bf16_round(torch.randn(R * S, generator=g, dtype=torch.float32))
    poison_padding(flat, S, lengths)
    return Workload("decode", flat, S, lengths, R, 1024)


def _long(seed: int) -> Workload:
    g = torch.Generator().manual_seed(seed)
    R, S, L = 8, 900096, 900000
    lengths = torch.full((R,), L, dtype=torch.int32)
    rows = torch.randn(R, S, generator=g, dtype=torch.float32)
    n_out = L // 200          # 0.5 % outliers per row
    for r in range(R):
        pos = torch.randperm(L, generator=g)[:n_out]
        rows[r, pos] = 4.0 + torch.randn(n_out, generator=g, dtype=torch.float32)
    flat = rows.reshape(-1)
    poison_padding(flat, S, lengths)
    return Workload("long", flat, S, lengths, R, 2048)


def _prefill(seed: int) -> Workload:
    g = torch.Generator().manual_seed(seed)
    R, S = 4096, 32768
    lengths = (28672 + torch.arange(R, dtype=torch.int32) + 1).to(torch.int32)
    offsets = torch.rand(R, 1, generator=g, dtype=torch.float32) * 6.0 - 3.0
    rows = torch.randn(R, S, generator=g, dtype=torch.float32)
    rows.add_(offsets)
    flat = rows.reshape(-1)
    poison_padding(flat, S, lengths)
    return Workload("prefill", flat, S, lengths, R, 2048)


def _adversarial(seed: int) -> Workload:
    g = torch.Generator().manual_seed(seed)
    R, S, k = 256, 131072, 1024
    rows = torch.empty(R, S, dtype=torch.float32)
    lengths = torch.full((R,), S, dtype=torch.int32)
    j = torch.arange(S, dtype=torch.float64)
    for r in range(R):
        cls, i = divmod(r, 32)
        if cls == 0:      # A: all-equal rows
            c = i % 4
            if c == 0:
                rows[r] = 1.0
            elif c == 1:
                rows[r] = -2.5
            elif c == 2:
                rows[r] = float("-inf")
            else:
                rows[r] = 0.0
                rows[r, 1::2] = -0.0
        elif cls == 1:    # B: 16 levels
            lvl = torch.randint(0, 16, (S,), generator=g)
            rows[r] = lvl.to(torch.float32) - 7.5
        elif cls == 2:    # C: -inf tails
            f = (0, 1, 512, 1023, 1024, 1025, 2048, 65536)[i % 8]
            rows[r] = float("-inf")
            rows[r, :f] = torch.randn(f, generator=g, dtype=torch.float32)
        elif cls == 3:    # D: ramps
            c = i % 4
            if c == 0:
                rows[r] = j.to(torch.float32)
            elif c == 1:
                rows[r] = (-j).to(torch.float32)
            elif c == 2:
                rows[r] = torch.floor(j / 100.0).to(torch.float32)
            else:
                rows[r] = (1.0 + j * 2.0 ** -30).to(torch.float32)
        elif cls == 4:    # E: lengths around k, N(0,1)
            lengths[r] = (1, k - 1, k, k + 1)[i % 4]
            rows[r] = torch.randn(S, generator=g, dtype=torch.float32)
        elif cls == 5:    # F: lengths around k, all-equal 0.5
            lengths[r] = (1, k - 1, k, k + 1)[i % 4]
            rows[r] = 0.5
        elif cls == 6:    # G: bf16-rounded N(0,1)
            rows[r] = _bf16_round(torch.randn(S, generator=g, dtype=torch.float32))
        else:             # H: random length, N(0,1) with signed zeros and subnormals
            lengths[r] = int(torch.randint(1, S + 1, (1,), generator=g))
            x = torch.randn(S, generator=g, dtype=torch.float32)
            n = S // 100
            pz = torch.randperm(S, generator=g)[: 2 * n]
            zs = torch.where(torch.rand(n, generator=g) < 0.5, 0.0, -0.0)
            x[pz[:n]] = zs.to(torch.float32)
            bits = torch.randint(1, 1 << 23, (n,), generator=g, dtype=torch.int32)
            sign = (torch.rand(n, generator=g) < 0.5).to(torch.int32) << 31
            x[pz[n:]] = (bits | sign).view(torch.float32)
            rows[r] = x
    flat = rows.reshape(-1)
    poison_padding(flat, S, lengths)
    return Workload("adversarial", flat, S, lengths, R, k)


_BUILDERS = {
    "tiny": (_tiny, 0),
    "decode": (_decode, 1),
    "long": (_long, 2),
    "prefill": (_prefill, 3),
    "adversarial": (_adversarial, 4),
}


def make(name: str, seed: int | None = None) -> Workload:
    """One of the five named workloads (``NAMES``), seeded as documented."""
    fn, default_seed = _BUILDERS[name]
    return fn(default_seed if seed is None else seed)


def make_custom(num_rows: int, row_stride: int, lengths, k: int, seed: int,
                kind: str = "normal", levels: int = 16) -> Workload:
    """A smaller workload for parity cases.

    ``kind``: ``normal`` (N(0,1)), ``bf16`` (N(0,1) rounded to bf16, many ties),
    ``levels`` (``levels`` distinct values), ``equal`` (one value), ``ramp``
    (ascending ``x_j = j``), ``outliers`` (N(0,1) with 0.5 % N(4,1)),
    ``tail`` (an N(0,1) head of random length per row, then ``-inf``),
    ``plateau`` (``floor(j / run)`` with a random run per row), ``fineramp``
    (``1 + j * 2**-30``: runs of 128 equal values inside one binade),
    ``descending`` (``x_j = -j``).
    """
    g = torch.Generator().manual_seed(seed)
    lengths = torch.as_tensor(lengths, dtype=torch.int32).reshape(-1)
    if lengths.numel() == 1 and num_rows > 1:
        lengths = lengths.repeat(num_rows)
    rows = torch.randn(num_rows, row_stride, generator=g, dtype=torch.float32)
    if kind == "bf16":
        rows = _bf16_round(rows)
    elif kind == "levels":
        lvl = torch.randint(0, levels, (num_rows, row_stride), generator=g)
        rows = lvl.to(torch.float32) - levels / 2.0
    elif kind == "equal":
        rows.fill_(0.75)
    elif kind == "ramp":
        rows = torch.arange(row_stride, dtype=torch.float32).repeat(num_rows, 1)
    elif kind == "outliers":
        mask = torch.rand(num_rows, row_stride, generator=g) < 0.005
        rows[mask] = 4.0 + torch.randn(int(mask.sum()), generator=g, dtype=torch.float32)
    elif kind == "tail":
        heads = torch.randint(0, row_stride + 1, (num_rows,), generator=g)
        col = torch.arange(row_stride).unsqueeze(0)
        rows.masked_fill_(col >= heads.unsqueeze(1), float("-inf"))
    elif kind == "plateau":
        runs = torch.randint(1, 300, (num_rows, 1), generator=g).to(torch.float64)
        j = torch.arange(row_stride, dtype=torch.float64).unsqueeze(0)
        rows = torch.floor(j / runs).to(torch.float32)
    elif kind == "fineramp":
        j = torch.arange(row_stride, dtype=torch.float64)
        rows = (1.0 + j * 2.0 ** -30).to(torch.float32).repeat(num_rows, 1)
    elif kind == "descending":
        rows = (-torch.arange(row_stride, dtype=torch.float32)).repeat(num_rows, 1)
    elif kind != "normal":
        raise ValueError(f"unknown kind {kind!r}")
    flat = rows.reshape(-1).contiguous()
    poison_padding(flat, row_stride, lengths)
    return Workload(f"custom-{kind}", flat, row_stride, lengths, num_rows, k)


def to_numpy(w: Workload):
    """(flat float32, lengths int32) as NumPy arrays, for the CPU oracle."""
    return w.flat.numpy(), w.lengths.numpy().astype(np.int32)

"""The C-ABI library loads and exports every symbol its header declares.

No GPU needed: only calls that return before touching a device are made.
"""

import ctypes
import glob
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("mi_topk.h", "mi_c128a.h")]
PREFIXES = ("topk_", "c128a_")


def _declared_functions():
    names = []
    for h in HEADERS:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)
    keep = [n for n in names if n.startswith(PREFIXES)]
    return sorted(set(keep))


@pytest.fixture(scope="module")
def lib():
    import row_wise_top_topk_amd as m
    path = m.library_path()
    if not os.path.exists(path):
        pytest.fail(f"{path} not built: run `python -m row_wise_top_topk_amd.build`")
    return m.load_library()


def test_header_declares_the_boundary():
    names = _declared_functions()
    for n in ("topk_indices", "topk_workspace_size", "topk_status_string"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    import row_wise_top_topk_amd as m
    out = subprocess.run(["nm", "-D", "--defined-only", m.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for n in _declared_functions():
        assert n in exported, n
        assert getattr(lib, n) is not None
    # nothing else with C linkage leaks out under the library's prefixes
    assert {e for e in exported if e.startswith(PREFIXES)} == set(_declared_functions())
    assert set(glob.glob(os.path.join(ROOT, "include", "*.h"))) == set(HEADERS)


def test_status_strings(lib):
    import row_wise_top_topk_amd as m
    assert m.status_string(0) == "ok"
    assert "invalid" in m.status_string(1)
    assert "workspace" in m.status_string(2)
    assert m.status_string(99) == "unknown status"


def test_invalid_arguments_rejected_before_any_device_call(lib):
    vp = ctypes.c_void_p
    fake = vp(0x1000)       # never dereferenced: validation fails first
    call = lib.topk_indices
    assert call(fake, 8, fake, -1, 4, fake, None, 0, None) == 1          # num_rows < 0
    assert call(fake, 8, fake, 3, 0, fake, None, 0, None) == 1           # k == 0
    assert call(fake, 8, fake, 3, (1 << 24) + 1, fake, None, 0, None) == 1
    assert call(fake, 0, fake, 3, 4, fake, None, 0, None) == 1           # row_stride < 1
    assert call(None, 8, fake, 3, 4, fake, None, 0, None) == 1           # NULL logits
    assert call(fake, 8, None, 3, 4, fake, None, 0, None) == 1           # NULL lengths
    assert call(fake, 8, fake, 3, 4, None, None, 0, None) == 1           # NULL out
    assert call(vp(0x1002), 8, fake, 3, 4, fake, None, 0, None) == 1     # misaligned logits
    assert call(fake, 8, fake, 0, 4, fake, None, 0, None) == 0           # empty batch: no-op
    assert lib.topk_indices_path(fake, 8, fake, 3, 4, fake, None, 0, 7, 0, None) == 1
    assert lib.topk_workspace_size(-1, 8, 4) == 0
    assert lib.topk_workspace_size(3, 8, 0) == 0
    assert lib.topk_debug_keys(None, None, -1, None) == 1
    vo = lib.topk_value_order
    assert vo(fake, 8, fake, 3, 4097, fake, None) == 1                   # k above 4096
    assert vo(fake, 8, fake, 3, 0, fake, None) == 1                      # k == 0
    assert vo(fake, 0, fake, 3, 4, fake, None) == 1                      # row_stride < 1
    assert vo(fake, 8, fake, -1, 4, fake, None) == 1                     # num_rows < 0
    assert vo(None, 8, fake, 3, 4, fake, None) == 1                      # NULL logits
    assert vo(fake, 8, fake, 3, 4, None, None) == 1                      # NULL idx
    assert vo(fake, 8, fake, 0, 4, fake, None) == 0                      # empty batch: no-op


def test_c128a_width_rule_and_argument_checks(lib):
    # host-only: the width rule, and calls rejected before anything is enqueued
    assert lib.c128a_active_width(32768, 128) == 256
    assert lib.c128a_active_width(9037, 128) == 128
    assert lib.c128a_active_width(65536, 128) == 512
    assert lib.c128a_active_width(-1, 128) == -1
    assert lib.c128a_active_width(100, 0) == -1
    vp = ctypes.c_void_p
    fake = vp(0x1000)
    call = lib.c128a_topk_metadata
    args = lambda **kw: [kw.get(n, d) for n, d in (
        ("pos", fake), ("T", 4), ("ratio", 128), ("nd", 0), ("tr", None), ("bt", None), ("bts", 0),
        ("bs", 2), ("db", None), ("ds", 0), ("dl", None), ("pb", fake), ("ps", 8), ("w", 8), ("s", None))]
    assert call(*args(T=0)) == 0                 # no tokens: no-op
    assert call(*args(T=-1)) == 1
    assert call(*args(ratio=0)) == 1
    assert call(*args(w=0)) == 1
    assert call(*args(ps=7)) == 1                # stride below the width
    assert call(*args(nd=5)) == 1                # more decode tokens than tokens
    assert call(*args(nd=2)) == 1                # decode tokens without decode buffers
    assert call(*args(pos=None)) == 1
    assert call(*args(pos=vp(0x1004))) == 1      # positions not 8-byte aligned
    assert call(*args(pb=None)) == 1

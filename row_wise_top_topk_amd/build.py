"""Build libmi_topk.so (the C-ABI library with the gfx950 kernels) in-tree.

Two builds of the same sources: ``libmi_topk.so`` at -O3 (the library the
binding loads) and ``libmi_topk_O1.so`` at -O1, which the parity tests run
as well, since a top-k kernel whose result depended on the compiler's
optimisation choices is the failure the SGLang PR #34167 page reports
(section 风险与影响, item 1).

Usage: python -m row_wise_top_topk_amd.build [--opt O3] [--out PATH] [--save-temps DIR]
"""

from __future__ import annotations

import argparse
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SOURCES = [os.path.join(CSRC, "topk_kernels.hip"), os.path.join(CSRC, "c128a_metadata.hip")]
LIB = os.path.join(PKG, "libmi_topk.so")
LIB_O1 = os.path.join(PKG, "libmi_topk_O1.so")
ARCH = "gfx950"


def hipcc_command(out: str = LIB, opt: str = "O3", extra=()) -> list:
    return [
        os.environ.get("HIPCC", "/opt/rocm/bin/hipcc"),
        f"-{opt}", "-std=c++17", f"--offload-arch={ARCH}",
        "-fPIC", "-shared", "-fvisibility=hidden", "-fvisibility-inlines-hidden",
        # no packed-fp32 instructions in the device code (the host pass warns
        # that it does not know the feature; the gfx950 pass honours it)
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-command-line-argument",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        *extra,
        "-o", out, *SOURCES,
    ]


def _start(out: str, opt: str, extra, verbose: bool):
    cmd = hipcc_command(out, opt, extra)
    if verbose:
        print(" ".join(cmd), flush=True)
    tmp = out + ".tmp"
    cmd[cmd.index("-o") + 1] = tmp
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True), tmp


def _finish(proc, tmp: str, out: str) -> str:
    text, _ = proc.communicate()
    if proc.returncode != 0:
        sys.stderr.write(text)
        raise RuntimeError(f"hipcc failed with status {proc.returncode} building {out}")
    os.replace(tmp, out)
    return out


def build(out: str = LIB, opt: str = "O3", extra=(), verbose: bool = False) -> str:
    """One build of the library."""
    proc, tmp = _start(out, opt, extra, verbose)
    return _finish(proc, tmp, out)


def build_all(verbose: bool = False) -> list:
    """The -O3 library and its -O1 twin, compiled side by side."""
    jobs = [(_start(o, opt, (), verbose), o) for o, opt in ((LIB, "O3"), (LIB_O1, "O1"))]
    return [_finish(proc, tmp, o) for (proc, tmp), o in jobs]


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--opt", default=None, help="one build at this level (default: both builds)")
    ap.add_argument("--out", default=None)
    ap.add_argument("--save-temps", default=None,
                    help="directory for the device assembly of this build")
    args = ap.parse_args()
    extra = []
    if args.save_temps:
        os.makedirs(args.save_temps, exist_ok=True)
        extra = [f"-save-temps={'obj'}", "-Rpass-analysis=kernel-resource-usage"]
        os.chdir(args.save_temps)
    if args.opt is None and args.out is None and not extra:
        print("\n".join(build_all(verbose=True)))
    else:
        print(build(args.out or LIB, args.opt or "O3", extra, verbose=True))


if __name__ == "__main__":
    main()

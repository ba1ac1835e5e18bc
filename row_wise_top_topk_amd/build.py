"""Build libmi_topk.so (the C-ABI library with the gfx950 kernels) in-tree.

Usage: python -m row_wise_top_topk_amd.build [--opt O3] [--save-temps DIR]
"""

from __future__ import annotations

import argparse
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SOURCES = [os.path.join(CSRC, "topk_kernels.hip")]
LIB = os.path.join(PKG, "libmi_topk.so")
ARCH = "gfx950"


def hipcc_command(out: str = LIB, opt: str = "O3", extra=()) -> list:
    return [
        os.environ.get("HIPCC", "/opt/rocm/bin/hipcc"),
        f"-{opt}", "-std=c++17", f"--offload-arch={ARCH}",
        "-fPIC", "-shared", "-fvisibility=hidden", "-fvisibility-inlines-hidden",
        # keep the compiler from forming packed-fp32 instructions
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-command-line-argument",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        *extra,
        "-o", out, *SOURCES,
    ]


def build(out: str = LIB, opt: str = "O3", extra=(), verbose: bool = False) -> str:
    cmd = hipcc_command(out, opt, extra)
    if verbose:
        print(" ".join(cmd), flush=True)
    tmp = out + ".tmp"
    cmd[cmd.index("-o") + 1] = tmp
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with status {res.returncode}")
    os.replace(tmp, out)
    return out


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--opt", default="O3")
    ap.add_argument("--out", default=LIB)
    ap.add_argument("--save-temps", default=None,
                    help="directory for the device assembly of this build")
    args = ap.parse_args()
    extra = []
    if args.save_temps:
        os.makedirs(args.save_temps, exist_ok=True)
        extra = [f"-save-temps={'obj'}", "-Rpass-analysis=kernel-resource-usage"]
        os.chdir(args.save_temps)
    print(build(args.out, args.opt, extra, verbose=True))


if __name__ == "__main__":
    main()

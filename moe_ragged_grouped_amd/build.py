"""Compile the gfx950 HIP libraries in-tree with hipcc.

    python -m moe_ragged_grouped_amd.build

produces moe_ragged_grouped_amd/libmoe_ragged_grouped_amd.so from csrc/, and
libmoe_ragged_grouped_amd_trace.so, the same sources built with GG_TILE_TRACE
(the per-tile timeline of include/grouped_gemm_trace.h; a diagnostic the
product library does not contain).
"""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe_ragged_grouped_amd.so")
TRACE_LIB = os.path.join(HERE, "libmoe_ragged_grouped_amd_trace.so")
SOURCES = [os.path.join(CSRC, "grouped_gemm.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # hipcc -O3 forms packed fp32 ops from plain float code; keep it from doing so
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose: bool = False, extra=(), out: str = LIB) -> str:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, *extra, "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if noise not in ln]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, out)
    return out


def build_trace(verbose: bool = False) -> str:
    return build(verbose, extra=("-DGG_TILE_TRACE",), out=TRACE_LIB)


if __name__ == "__main__":
    print(build(verbose=True, extra=sys.argv[1:]))
    print(build_trace(verbose=True))

"""Build libspax.so in-tree with hipcc for gfx950.

    python -m activation_sparse_decode_token_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libspax.so")

SOURCES = ["plan.hip", "select.hip", "gemv.hip", "layer.hip", "aux.hip", "static_ws.hip", "api.cpp",
           "trellis_pack.cpp"]
# per-source flags: the trellis encoder's fp32 error arithmetic is defined
# operation by operation (no contraction into fused multiply-adds)
EXTRA = {
    "trellis_pack.cpp": ["-ffp-contract=off"],
    # the layer kernel reads its argument struct (736 bytes, in the kernel
    # argument segment) from many places; past LLVM's default limit of 300
    # users the compiler keeps a private copy of it in scratch, whose loads
    # then wait for every global load in flight
    "layer.hip": ["-mllvm", "-instcombine-max-copied-from-constant-users=100000"],
}

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 instructions are kept out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libspax.so")


def build(verbose: bool = False) -> str:
    """Compile every source to an object (in parallel), then link."""
    import concurrent.futures
    import tempfile
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    with tempfile.TemporaryDirectory(prefix="spax_build_") as tmpdir:
        objs = [os.path.join(tmpdir, s + ".o") for s in SOURCES]
        cmds = [[HIPCC, *FLAGS, *EXTRA.get(s, []), *inc, "-c", os.path.join(CSRC, s), "-o", o]
                for s, o in zip(SOURCES, objs)]
        workers = max(1, min(len(cmds), os.cpu_count() or 1, 8))
        with concurrent.futures.ThreadPoolExecutor(workers) as ex:
            list(ex.map(lambda c: _run(c, verbose), cmds))
        tmp = LIB + ".tmp"
        _run([HIPCC, *FLAGS, *objs, "-o", tmp], verbose)
        os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

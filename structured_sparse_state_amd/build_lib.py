"""Compile the HIP library ``libpdssm.so`` for gfx950 with hipcc (in-tree).

Two test builds of the same sources sit beside it, loaded only by the GPU
tests (structured_sparse_state_amd.variant):

* ``libpdssm_w5.so``: five chunk waves per scan workgroup instead of seven,
  so tiles of 80 steps at N = 64 (chunk-size invariance of the results);
* ``libpdssm_remap.so``: PDSSM_TEST_TICKET_REMAP, the sequences of each tile
  row handed out in reverse order and the heads of the per-head ticket
  streams served by the workgroups in reverse (order invariance of the
  look-back).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(HERE, "libpdssm.so")
VARIANTS = {
    "w5": ["-DPDSSM_SCAN_W=5"],
    "remap": ["-DPDSSM_TEST_TICKET_REMAP"],
}
SOURCES = [os.path.join(CSRC, f) for f in ("pdssm_scan.hip", "pdssm_bwd.hip", "pdssm_aux.hip",
                                            "pdssm_router.hip")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # Keep the compiler from emitting packed-fp32 VALU instructions.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def variant_path(name: str) -> str:
    return os.path.join(HERE, f"libpdssm_{name}.so")


def build(out: str = LIBRARY, extra=(), verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    cmd = [hipcc, *HIPCC_FLAGS, *extra, "-I", INCLUDE, "-I", CSRC, "-o", out + ".tmp", *SOURCES]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def build_all(verbose: bool = False) -> None:
    """The library and its test builds, compiled side by side."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    jobs = [(LIBRARY, [])] + [(variant_path(k), v) for k, v in VARIANTS.items()]
    procs = []
    for out, extra in jobs:
        cmd = [hipcc, *HIPCC_FLAGS, *extra, "-I", INCLUDE, "-I", CSRC, "-o", out + ".tmp", *SOURCES]
        if verbose:
            print(" ".join(cmd), file=sys.stderr)
        procs.append((out, subprocess.Popen(cmd)))
    failed = [out for out, p in procs if p.wait() != 0]
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    for out, _ in procs:
        os.replace(out + ".tmp", out)


if __name__ == "__main__":
    build_all(verbose=True)

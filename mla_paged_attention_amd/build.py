"""Build libmla_mi355x.so in-tree with hipcc for gfx950.

The library is plain C ABI (include/mla.h); the Python binding loads it with
ctypes. Run ``python -m mla_paged_attention_amd.build`` or call ``build()``.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SOURCES = [os.path.join(CSRC, f)
           for f in ("mla_kernels.hip", "gemm_fp8.hip", "absorb.hip", "mla_api.hip")]
LIBRARY = os.path.join(HERE, "libmla_mi355x.so")
# Calibration kernels (measured HBM and matrix-core peaks), a library of
# their own: the decode library does not contain them.
PEAKS_SOURCES = [os.path.join(CSRC, "peaks.hip")]
PEAKS_LIBRARY = os.path.join(HERE, "libmla_peaks.so")
# Bounds-check build of the decode library: every clamp of a corrupt input
# (block id, seq_len) is also reported in an error word of the workspace.
CHECKED_LIBRARY = os.path.join(HERE, "libmla_mi355x_checked.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # Keep hipcc from forming packed fp32 instructions.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _hipcc(sources, library, verbose, extra_flags):
    tmp = library + ".tmp"
    cmd = [HIPCC, *FLAGS, *(extra_flags or []), "-o", tmp, *sources]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if noise not in ln]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, library)
    return library


def build(verbose: bool = False, extra_flags=None) -> str:
    """Build the decode library, its bounds-check build and the calibration
    library; returns the decode library's path."""
    _hipcc(PEAKS_SOURCES, PEAKS_LIBRARY, verbose, extra_flags)
    _hipcc(SOURCES, CHECKED_LIBRARY, verbose, [*(extra_flags or []), "-DMLA_BOUNDS_CHECK=1"])
    return _hipcc(SOURCES, LIBRARY, verbose, extra_flags)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

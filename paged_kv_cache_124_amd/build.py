"""Build libpa.so (HIP kernels for gfx950 + C ABI + host block manager) in-tree.

    python paged_kv_cache_124_amd/build.py

(run as a file: importing the package loads the library this builds)

Produces ``paged_kv_cache_124_amd/libpa.so``.  hipcc cross-compiles gfx950
code objects without a GPU, so this runs on any machine with ROCm.
"""

from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpa.so")

HIP_SOURCES = ["decode.hip", "decode_stream.hip", "decode_stream_i8.hip", "decode_shared.hip", "kv_ops.hip", "probe.hip"]
HOST_SOURCES = ["block_manager.cpp", "status.cpp"]

# -packed-fp32-ops: keep hipcc from forming packed fp32 VALU ops on its own.
# atomic optimizer off: it turns the decode kernel's lane-0 work claim into a
# wave-aggregated atomic whose result is waited for at once, which would stall
# the tile pipeline; the claim's result is only needed one worker later.
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose: bool = False, extra_flags=None) -> str:
    srcs = [os.path.join(CSRC, s) for s in HIP_SOURCES + HOST_SOURCES]
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, *(extra_flags or []), "-I", INCLUDE, "-I", CSRC, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the gfx feature above; that warning is noise
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        sys.stderr.write("\n".join(msgs) + "\n")
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

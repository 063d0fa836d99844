"""Build the libraries in-tree.

    python paged_kv_cache_124_amd/build.py [-v]

(run as a file: importing the package loads the library this builds)

Produces, in ``paged_kv_cache_124_amd/``:
  libpa.so            HIP kernels for gfx950 + C ABI (include/pa.h) + host block manager
  libpa_probe.so      the HBM read-rate probe (include/pa_probe.h), loaded by bench.py only
  libpa_host.so       the host block manager and status strings alone (g++, no HIP)
  libpa_host_asan.so  the same built with AddressSanitizer and UBSan, for the CPU tests
hipcc cross-compiles gfx950 code objects without a GPU, so this runs on any
machine with ROCm.
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
PROBE_LIB = os.path.join(PKG, "libpa_probe.so")
HOST_LIB = os.path.join(PKG, "libpa_host.so")
HOST_ASAN_LIB = os.path.join(PKG, "libpa_host_asan.so")
# test build: the block manager with a 2-bit chain hash, so the prefix cache's exact chain comparison is
# exercised on every lookup (tests/test_block_manager_collide.py)
HOST_COLLIDE_LIB = os.path.join(PKG, "libpa_host_collide.so")

HIP_SOURCES = ["decode.hip", "decode_stream.hip", "decode_stream_i8.hip", "decode_shared.hip", "kv_ops.hip",
               "check.hip"]
PROBE_SOURCES = ["probe.hip"]
HOST_SOURCES = ["block_manager.cpp", "status.cpp"]
HOST_FLAGS = ["-O2", "-g", "-std=c++17", "-fPIC", "-shared", "-Wall", "-Wextra", "-Wno-unused-parameter"]
SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]

# -packed-fp32-ops: keep hipcc from forming packed fp32 VALU ops on its own.
# atomic optimizer off: it folds a wave's atomics on one address into a scan and
# one atomic; the library's atomics are per-lane LDS updates (the batch checks'
# bitmaps, the shared-prefix kernel's row claims) whose results are used at once.
# MFMA in VGPR form: the matrix-core accumulators of the decode kernels are
# loop-carried and rescaled by VALU code, and with the accumulator-register form
# every tile copied them into AGPRs and back (64 moves per tile in the bf16
# kernel; none in this form, and fewer registers).
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _run(cmd, out, verbose):
    tmp = out + ".tmp"
    cmd = [*cmd, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the gfx feature above; that warning is noise
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        sys.stderr.write("\n".join(msgs) + "\n")
        raise RuntimeError(f"{cmd[0]} failed with exit code {res.returncode}")
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, out)
    return out


def build_host(verbose: bool = False, sanitize: bool = False, collide: bool = False) -> str:
    """The block manager without HIP (g++), optionally with AddressSanitizer and UBSan, or with a 2-bit chain hash."""
    srcs = [os.path.join(CSRC, s) for s in HOST_SOURCES]
    flags = HOST_FLAGS + (SANITIZE_FLAGS if sanitize else []) + (["-DPA_CHAIN_HASH_BITS=2"] if collide else [])
    out = HOST_COLLIDE_LIB if collide else (HOST_ASAN_LIB if sanitize else HOST_LIB)
    return _run(["g++", *flags, "-I", INCLUDE, *srcs], out, verbose)


def build(verbose: bool = False, extra_flags=None) -> str:
    # one hipcc per source, in parallel, then one link
    from concurrent.futures import ThreadPoolExecutor
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    compile_flags = [f for f in HIP_FLAGS if f != "-shared"] + ["-c", *(extra_flags or []), "-I", INCLUDE, "-I", CSRC]
    srcs = HIP_SOURCES + HOST_SOURCES
    objs = [os.path.join(objdir, os.path.splitext(s)[0] + ".o") for s in srcs]
    with ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 1)) as ex:
        list(ex.map(lambda so: _run([hipcc(), *compile_flags, os.path.join(CSRC, so[0])], so[1], verbose),
                    zip(srcs, objs)))
    _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs], LIB, verbose)
    _run([hipcc(), *HIP_FLAGS, "-I", INCLUDE, *[os.path.join(CSRC, s) for s in PROBE_SOURCES]], PROBE_LIB, verbose)
    build_host(verbose)
    build_host(verbose, sanitize=True)
    build_host(verbose, collide=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

"""Build libmxfa.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m mxfp8_block_scaled_flash_amd.build

Compiles every csrc/*.hip file with hipcc into objects under _build/ and links
them into mxfp8_block_scaled_flash_amd/libmxfa.so.  Always rebuilds.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmxfa.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed-fp32 VALU instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


# Per-file additions.  The MX attention kernels take maxima of MFMA results and of lane-swapped
# values, which in the default IEEE mode each cost an extra max(x, x) to quiet signalling NaNs;
# these kernels test for no NaN (infinities, which stay honoured, mark masked scores), so they are
# built without NaN semantics: the same codes and outputs, 16 fewer VALU instructions per forward
# tile, 1.4% less forward time (measured).
FILE_FLAGS = {
    "attn_fwd.hip": ["-fno-honor-nans"],
    "attn_bwd.hip": ["-fno-honor-nans"],
}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link of libmxfa.so failed")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    _build_test_probe(verbose)
    return LIB


def _build_test_probe(verbose: bool = False) -> None:
    """tests/hw/libmfmaprobe.so: runs the scaled-MFMA instruction alone, for the
    GPU tests that measure the instruction against the oracle's stated product bound;
    tests/hw/libldsprobe.so: times LDS read patterns (test and measurement infrastructure)."""
    for name, lib in (("mfma_probe.hip", "libmfmaprobe.so"), ("lds_probe.hip", "libldsprobe.so")):
        src = os.path.join(ROOT, "tests", "hw", name)
        if not os.path.exists(src):
            continue
        out = os.path.join(ROOT, "tests", "hw", lib)
        cmd = [HIPCC, *FLAGS, "-shared", src, "-o", out + ".tmp"]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError(f"build of {name} failed")
        os.replace(out + ".tmp", out)
        if verbose:
            print("built", out)


if __name__ == "__main__":
    build(verbose=True)

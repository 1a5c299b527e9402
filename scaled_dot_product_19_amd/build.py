"""Build libsdpa.so (HIP, gfx950) in-tree with hipcc.

Every translation unit is compiled for gfx950 only, then linked into one
shared library next to this file.  Packed-FP32 VALU instructions are disabled
for all HIP code (``-Xclang -target-feature -Xclang -packed-fp32-ops``).
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libsdpa.so")
ARCH = "gfx950"

SOURCES = ["sdpa_api.cpp", "prefill_bf16.hip", "prefill_f32.hip", "decode_paged.hip",
           "decode_small.hip", "decode_wide.hip", "combine.hip", "decode_noalloc.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libsdpa.so)")


def common_flags():
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-I" + INCLUDE, "-I" + CSRC,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


# Per-source extra flags.  The persistent kernels fetch their next work item
# with a one-lane atomicAdd while the current one runs; the wave-level atomic
# optimizer would turn it into a scan that waits for the result on the spot.
_NO_ATOMIC_OPT = ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]
EXTRA_FLAGS = {"prefill_bf16.hip": _NO_ATOMIC_OPT, "decode_small.hip": _NO_ATOMIC_OPT}


def _compile(cc, src, obj):
    cmd = [cc] + common_flags() + EXTRA_FLAGS.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature; that warning is harmless
    noise = [l for l in r.stderr.splitlines() if "is not a recognized feature" not in l]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, "\n".join(noise)))
    return obj


def build(verbose: bool = False) -> str:
    cc = hipcc()
    tmp = tempfile.mkdtemp(prefix="sdpa_build_")
    try:
        objs = [os.path.join(tmp, os.path.splitext(s)[0] + ".o") for s in SOURCES]
        workers = min(len(SOURCES), max(1, min(8, os.cpu_count() or 1)))
        with concurrent.futures.ThreadPoolExecutor(workers) as ex:
            list(ex.map(lambda p: _compile(cc, *p), zip(SOURCES, objs)))
        out_tmp = LIB + ".tmp%d" % os.getpid()
        cmd = [cc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", out_tmp] + objs
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n" + r.stderr)
        os.replace(out_tmp, LIB)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

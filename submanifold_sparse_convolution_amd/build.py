"""Compile the HIP sources for gfx950 into lib/libsubmconv.so (in-tree).

    python -m submanifold_sparse_convolution_amd.build

Each .hip file is compiled to an object under _build/ in parallel, then linked
into one shared library.  The library is written to a temporary name and
renamed, so a process that has the old one loaded never sees a partial file.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libsubmconv.so")
SOURCES = ["submconv_api.hip", "indice_map.hip", "conv.hip", "conv_pool.hip", "conv_offsets.hip", "structure.hip",
           "norm.hip", "sort_scan.hip", "row_order.hip", "peak.hip"]

ARCH = "gfx950"
COMMON = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # Code object v5 loads under both the ROCm 7.0 runtime bundled with torch and ROCm 7.2.
    "-mcode-object-version=5",
    # Packed fp32 VALU ops stay off: the compiler must not form v_pk_{add,mul,fma}_f32.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
    f"-I{os.path.join(ROOT, 'include')}",
    f"-I{CSRC}",
]


def hipcc() -> str:
    return os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # The host pass does not know the packed-fp32 feature and says so; that line is noise.
    out = "\n".join(l for l in proc.stdout.splitlines() if "packed-fp32-ops" not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"command failed ({proc.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    cc = hipcc()
    jobs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        jobs.append((obj, [cc, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 1)) as ex:
        for out in ex.map(lambda j: _run(j[1]), jobs):
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    out = _run([cc, f"--offload-arch={ARCH}", "-mcode-object-version=5", "-shared", "-fPIC", *[o for o, _ in jobs], "-o", tmp])
    if verbose and out.strip():
        print(out)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)

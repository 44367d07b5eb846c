"""Build ``libkvstream.so`` in-tree with hipcc for gfx950.

Usage: ``python -m bounded_kv_cache_stream_amd.build`` (or ``build()``).
Every HIP source is compiled with packed fp32 instructions disabled; the
host-only runtime is compiled with g++ against the HIP runtime headers.

``python -m bounded_kv_cache_stream_amd.build --host-sanitize`` also builds
``_build/libkvstream_hostsan.so``: the host runtime (kvstream.cpp with the
page policy) compiled by g++ with AddressSanitizer and UndefinedBehaviorSanitizer,
linked with the unchanged kernel objects.  It is for CPU runs of the host
tests only; load it with gcc's ASan runtime first:

    KVSTREAM_LIB=_build/libkvstream_hostsan.so LD_PRELOAD=$(g++ -print-file-name=libasan.so) \
        ASAN_OPTIONS=detect_leaks=0 python -m pytest tests/test_lib_host.py
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libkvstream.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ARCH = "gfx950"

HIP_SOURCES = ["attend.hip", "pages.hip", "clces.hip", "diversity.hip"]
# per-file extra flags: keep MFMA accumulators in architectural VGPRs (the
# softmax reads every score accumulator; AGPR copies would cost VALU slots)
EXTRA_FLAGS = {"attend.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
HOST_SOURCES = ["kvstream.cpp"]

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]
GXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
             f"-I{ROCM}/include", f"-I{INCLUDE}", f"-I{CSRC}"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops" not in l and "argument unused during compilation" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    hipcc = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
    jobs = []
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append([hipcc, *HIPCC_FLAGS, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append(["g++", *GXX_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        for out in ex.map(_run, jobs):
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


SAN_LIB = os.path.join(BUILD, "libkvstream_hostsan.so")
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def build_host_sanitized() -> str:
    """The host runtime with ASan + UBSan (g++ only; the kernel objects of build() are linked as they are)."""
    build()
    obj = os.path.join(BUILD, "kvstream.cpp.san.o")
    flags = [f if f != "-O2" else "-O1" for f in GXX_FLAGS] + ["-g", *SAN_FLAGS]
    _run(["g++", *flags, "-c", os.path.join(CSRC, "kvstream.cpp"), "-o", obj])
    objs = [obj] + [os.path.join(BUILD, src + ".o") for src in HIP_SOURCES]
    _run(["g++", "-shared", *SAN_FLAGS, "-o", SAN_LIB, *objs, f"-L{ROCM}/lib", "-lamdhip64",
          f"-Wl,-rpath,{ROCM}/lib"])
    return SAN_LIB


if __name__ == "__main__":
    if "--host-sanitize" in sys.argv:
        print(build_host_sanitized())
    else:
        print(build(verbose="-v" in sys.argv))

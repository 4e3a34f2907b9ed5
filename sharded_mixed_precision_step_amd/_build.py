"""Build of libzerostep.so (the gfx950 kernels and the C-ABI host layer), of
libzerotwin.so (the benchmark's measurement aids, zero_twin.h) and of
workloads/libzerogen.so (the device side of the seeded input generators).

hipcc cross-compiles for gfx950 on any host, so this runs without a GPU.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
INCLUDE = os.path.join(ROOT, "include")
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libzerostep.so")
SOURCES = [os.path.join(CSRC, "zero_kernels.hip"), os.path.join(CSRC, "zero_abi.cpp")]
TWIN_LIB = os.path.join(HERE, "libzerotwin.so")
TWIN_SOURCES = [os.path.join(CSRC, "zero_twin.hip")]
# the device side of the seeded input generators (workloads/), test and
# benchmark infrastructure
GEN_DIR = os.path.join(ROOT, "workloads", "csrc")
GEN_LIB = os.path.join(ROOT, "workloads", "libzerogen.so")
GEN_SOURCES = [os.path.join(GEN_DIR, "zero_gen.hip")]
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # every fp32 operation separately rounded, as the step is defined
    "-ffp-contract=off",
    # no packed fp32 arithmetic in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def code_text(src: str) -> str:
    """C/C++ source with its comments removed and each run of whitespace
    collapsed to one space: what the compiler sees, so that editing a comment
    does not change a digest.  String and character literals are kept as
    they are."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            out.append(" ")
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_digest() -> str:
    """SHA-256 over the code of the sources that fix the kernels' code and
    launch shapes (the device source and the internal header), comments and
    layout aside.  Hardware counters taken on one digest do not describe
    kernels built from another."""
    import hashlib
    h = hashlib.sha256()
    for p in (os.path.join(CSRC, "zero_kernels.hip"), os.path.join(CSRC, "zero_internal.h")):
        with open(p, encoding="utf-8") as f:
            h.update(os.path.basename(p).encode())
            h.update(code_text(f.read()).encode())
    return h.hexdigest()


def build(verbose: bool = False) -> str:
    """Compile the three libraries for gfx950 (hipcc processes side by side),
    each written atomically."""
    jobs = []
    for lib, sources in ((LIB, SOURCES), (TWIN_LIB, TWIN_SOURCES), (GEN_LIB, GEN_SOURCES)):
        name = os.path.basename(lib)
        fd, tmp = tempfile.mkstemp(prefix=f".{name}.", suffix=".tmp", dir=os.path.dirname(lib))
        os.close(fd)
        cmd = [hipcc(), *FLAGS, "-I", INCLUDE, "-I", CSRC, "-I", GEN_DIR, *sources, "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        proc = subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
        jobs.append((lib, tmp, proc))
    errors = []
    try:
        for lib, tmp, proc in jobs:
            out, err = proc.communicate()
            if proc.returncode != 0:
                errors.append(f"hipcc failed ({proc.returncode}) for {os.path.basename(lib)}:"
                              f"\n{out}\n{err}")
                continue
            if verbose and err.strip():
                print(err, flush=True)
            os.replace(tmp, lib)
    finally:
        for _, tmp, proc in jobs:
            if proc.poll() is None:
                proc.kill()
            if os.path.exists(tmp):
                os.unlink(tmp)
    if errors:
        raise RuntimeError("\n".join(errors))
    return LIB


def ensure_built() -> str:
    """Build only if a library is missing."""
    if not all(os.path.exists(p) for p in (LIB, TWIN_LIB, GEN_LIB)):
        build()
    return LIB

"""Build libasp.so in-tree: HIP kernels for gfx950 with hipcc, the host packer with g++.

Usage: ``python -m wam_asp_w4a4_amd.build`` (or ``__graft_entry__.build()``).
Always recompiles.  No fast-math anywhere: the NVFP4 quantiser relies on
IEEE float32 division and exact comparisons.
"""

from __future__ import annotations

import hashlib
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libasp.so")

ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
ARCH = "gfx950"

HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # keep the compiler from forming packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in ordinary VGPRs (no copies through the accumulation registers)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", INCLUDE, "-I", CSRC,
]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-ffp-contract=off", "-pthread",
              "-Wall", "-Wextra", "-I", INCLUDE, "-I", CSRC]


def source_digest() -> str:
    """sha256 (first 16 hex digits) of every source the library is built from:
    the files of csrc/ and include/ in name order.  Compiled into the library
    (asp_source_digest) so that a stale build can be told from a fresh one."""
    h = hashlib.sha256()
    for d in (CSRC, INCLUDE):
        for name in sorted(os.listdir(d)):
            if name.endswith((".hip", ".cpp", ".h")):
                h.update(name.encode())
                with open(os.path.join(d, name), "rb") as f:
                    h.update(f.read())
    return h.hexdigest()[:16]


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if proc.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + proc.stdout)
    return proc.stdout


def build(verbose: bool = False) -> str:
    """Compile every source and link libasp.so next to this file; returns its path."""
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    digest = [f"-DASP_SOURCE_DIGEST=\"{source_digest()}\""]
    with tempfile.TemporaryDirectory(prefix="asp_build_") as tmp:
        objs = []
        jobs = []
        for name in sorted(os.listdir(CSRC)):
            src = os.path.join(CSRC, name)
            obj = os.path.join(tmp, name + ".o")
            if name.endswith(".hip"):
                jobs.append([HIPCC, *HIP_FLAGS, "-c", src, "-o", obj])
            elif name.endswith(".cpp"):
                jobs.append(["g++", *HOST_FLAGS, *digest, "-c", src, "-o", obj])
            else:
                continue
            objs.append(obj)
        with ThreadPoolExecutor(len(jobs)) as ex:
            outs = list(ex.map(_run, jobs))
        if verbose:
            for o in outs:
                if o.strip():
                    print(o, file=sys.stderr)
        tmp_lib = os.path.join(tmp, "libasp.so")
        _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-pthread", *objs,
              "-o", tmp_lib])
        shutil.move(tmp_lib, LIB + ".new")
        os.replace(LIB + ".new", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

"""Build the HIP library libvda.so in-tree for gfx950.

Usage: python -m frame_wise_delta_gram_amd.build   (or call build()).
Compiles each csrc/*.hip file with hipcc in parallel, then links one shared
library next to this file.  hipcc cross-compiles for gfx950 without a GPU.
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
LIB_PATH = os.path.join(PKG, "libvda.so")
SOURCES = ["k_stats.hip", "k_solve.hip", "k_scan.hip", "k_readout.hip", "k_prep.hip",
           "vda_api.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed fp32 VALU ops are disabled for every device compile.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Wno-unused-function"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the device-only feature flag; that note is harmless
    out = "\n".join(ln for ln in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in ln)
    if r.returncode != 0:
        raise RuntimeError("command failed (%d): %s\n%s" % (r.returncode, " ".join(cmd), out))
    return out


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every HIP source and link libvda.so; returns the library path."""
    if not os.path.exists(HIPCC):
        raise RuntimeError("hipcc not found at %s" % HIPCC)
    tmp = tempfile.mkdtemp(prefix="vda_build_")
    try:
        objs = []
        cmds = []
        for src in SOURCES:
            obj = os.path.join(tmp, src.replace(".hip", ".o"))
            objs.append(obj)
            cmds.append([HIPCC] + COMMON + DEVICE_FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj])
        jobs = jobs or min(len(cmds), max(1, os.cpu_count() or 1))
        with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
            for out in ex.map(_run, cmds):
                if verbose and out.strip():
                    print(out)
        tmp_lib = os.path.join(tmp, "libvda.so")
        _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp_lib] + objs)
        shutil.move(tmp_lib, LIB_PATH)  # atomic replace within one filesystem is not
        # guaranteed across tmp and the tree, so move then return the final path
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    build_c_demo()
    return LIB_PATH


C_DEMO_SRC = os.path.join(ROOT, "tests", "c_abi", "forward_demo.c")
C_DEMO = os.path.join(ROOT, "tests", "c_abi", "forward_demo")


def build_c_demo() -> str | None:
    """The plain-C consumer of the ABI that a GPU test runs (tests/c_abi):
    gcc, C99, warnings as errors, linked against libvda.so (found next to the
    package through an $ORIGIN-relative rpath) and the HIP runtime.  Returns
    the executable's path, or None when no C compiler is installed."""
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None or not os.path.exists(C_DEMO_SRC):
        return None
    rocm = os.path.dirname(os.path.dirname(HIPCC))
    _run([cc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-O2",
          "-D__HIP_PLATFORM_AMD__", "-isystem", os.path.join(rocm, "include"), "-I", INCLUDE,
          C_DEMO_SRC, "-o", C_DEMO, "-L", PKG, "-lvda", "-L", os.path.join(rocm, "lib"),
          "-lamdhip64", "-lm", "-Wl,-rpath,$ORIGIN/../../frame_wise_delta_gram_amd",
          "-Wl,-rpath," + os.path.join(rocm, "lib")])
    return C_DEMO


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only; nothing is enqueued).  Every HIP source is compiled with the
sanitizers on its host pass only (the device code is built as usual and never
runs here), linked with two plain-C programs of the C ABI: the host-only checks
of tests/c_abi/abi_check.c and the descriptor fuzzing of
tests/c_abi/desc_fuzz.c (200,000 descriptors through the descriptor checks,
workspace sizing and the entry points' argument refusals).  Any out-of-bounds
access, signed overflow in the size arithmetic or other undefined behaviour
stops the run with a non-zero status."""
import concurrent.futures
import os
import shutil
import subprocess

import pytest

from frame_wise_delta_gram_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CABI = os.path.join(ROOT, "tests", "c_abi")
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]


@pytest.fixture(scope="module")
def san_objects(tmp_path_factory):
    if not os.path.exists(B.HIPCC):
        pytest.skip("hipcc not installed")
    clang = os.path.join(os.path.dirname(os.path.dirname(B.HIPCC)), "llvm", "bin", "clang")
    if not os.path.exists(clang):
        pytest.skip("ROCm clang not installed")
    tmp = tmp_path_factory.mktemp("san")
    cmds = []
    objs = []
    for src in B.SOURCES:
        obj = str(tmp / src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([B.HIPCC, "--offload-arch=" + B.ARCH, "-O1", "-g", "-fno-omit-frame-pointer",
                     "-std=c++17", "-fPIC", "-I", B.INCLUDE, "-I", B.CSRC] + B.DEVICE_FLAGS
                    + HOST_SAN + ["-c", os.path.join(B.CSRC, src), "-o", obj])
    with concurrent.futures.ThreadPoolExecutor(min(len(cmds), os.cpu_count() or 1)) as ex:
        list(ex.map(B._run, cmds))
    return tmp, clang, objs


@pytest.mark.parametrize("prog", ["abi_check", "desc_fuzz"])
def test_host_code_under_sanitizers(san_objects, prog):
    tmp, clang, objs = san_objects
    cobj = str(tmp / (prog + ".o"))
    exe = str(tmp / (prog + "_san"))
    subprocess.run([clang, "-std=c99", "-g", "-O1", "-Wall", "-Wextra", "-Werror",
                    "-fsanitize=address,undefined", "-I", B.INCLUDE, "-c",
                    os.path.join(CABI, prog + ".c"), "-o", cobj], check=True)
    B._run([B.HIPCC, "--offload-arch=" + B.ARCH] + HOST_SAN + ["-o", exe, cobj] + objs + ["-lm"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "runtime error" not in r.stderr, r.stderr[-4000:]
    assert r.stdout.strip() == "ok"

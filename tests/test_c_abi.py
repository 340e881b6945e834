"""The C ABI from a plain C99 program (no C++, no Python): the header compiles
as C with every warning an error, and a program linked against libvda.so
checks the host-only entry points (descriptor checks, workspace sizing, status
strings, argument errors).  CPU only: nothing is enqueued."""
import os
import shutil
import subprocess

import pytest

import frame_wise_delta_gram_amd as vda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_abi", "abi_check.c")


def test_c_program_against_the_library(tmp_path):
    if not os.path.exists(vda.LIB_PATH):
        pytest.skip("libvda.so not built")
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    exe = str(tmp_path / "abi_check")
    libdir = os.path.dirname(vda.LIB_PATH)
    subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                    "-I", os.path.join(ROOT, "include"), SRC, "-o", exe,
                    "-L", libdir, "-lvda", "-Wl,-rpath," + libdir], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "ok"

"""One forward pass driven from the plain-C program tests/c_abi/forward_demo.c
(built with the library: C99 against include/vda.h and the HIP runtime's C
API, no Python in the process): its bf16 inputs and output, written to a file,
against the fp64 oracle at the bf16 bar."""
import os
import subprocess

import numpy as np
import pytest

import workloads as W
from gpu_helpers import TOL_OUT, require_gpu, row_rel_err, say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c_abi", "forward_demo")


def _read(path):
    raw = open(path, "rb").read()
    dims = np.frombuffer(raw[:32], dtype=np.int32)
    units, F, U, T, dk, dv, chunk, radius = (int(x) for x in dims)
    off = 32

    def take(n, dt):
        nonlocal off
        a = np.frombuffer(raw[off:off + n * np.dtype(dt).itemsize], dtype=dt)
        off += n * np.dtype(dt).itemsize
        return a

    bf = lambda n, shape: W.bf16_bits_to_f64(take(n, np.uint16)).reshape(shape)
    x = {"q": bf(units * F * U * dk, (units, F, U, dk)),
         "k": bf(units * F * U * dk, (units, F, U, dk)),
         "v": bf(units * F * U * dv, (units, F, U, dv)),
         "gate": bf(units * F * U * dv, (units, F, U, dv)),
         "beta": take(units * F * U, np.float32).astype(np.float64).reshape(units, F, U),
         "text_k": bf(units * T * dk, (units, T, dk)),
         "text_v": bf(units * T * dv, (units, T, dv)),
         "text_beta": take(units * T, np.float32).astype(np.float64).reshape(units, T),
         "rms_weight": take(dv, np.float32).astype(np.float64)}
    out = bf(units * F * U * dv, (units, F, U, dv))
    assert off == len(raw)
    return x, out, chunk, radius


def test_forward_from_c(tmp_path):
    require_gpu()
    if not os.path.exists(EXE):
        pytest.skip("tests/c_abi/forward_demo not built (python -m frame_wise_delta_gram_amd.build)")
    from oracle import vda_oracle
    path = str(tmp_path / "forward.bin")
    say("[c abi] forward_demo")
    r = subprocess.run([EXE, path], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    x, got, chunk, radius = _read(path)
    ref = vda_oracle.forward(x["q"], x["k"], x["v"], x["beta"], x["gate"], x["text_k"],
                             x["text_v"], x["text_beta"], x["rms_weight"], chunk=chunk,
                             radius=radius, eps=1e-6)
    err = row_rel_err(got, ref)
    say(f"  max row-rel err {err:.3e}")
    assert np.all(np.isfinite(got)) and err <= TOL_OUT["bf16"]

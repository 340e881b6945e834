"""Each stage of the HIP path (through the C ABI's debug taps) against the fp64
oracle on the same seeded inputs.

Stage tolerances (relative Frobenius error per matrix, max over matrices):
fp32 features: 1e-5 for the statistics, 1e-4 for everything after them (fp32
Cholesky and products, error growth bounded by the conditioning of I + A,
whose eigenvalues are all >= 1).  bf16 features: 4e-3 for the statistics
(beta*k is rounded to bf16 before the MFMA: <= 2^-9 relative per term), 1e-2
after them.  The end-to-end tolerances are in test_gpu_parity.py.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_helpers import (desc_for, mat_rel_err, oracle_forward, require_gpu, say, to_device,
                         to_f64, workspace_for)

pytestmark = pytest.mark.gpu

CASES = {
    "tiny-fp32": W.CONFIGS[1],
    "small-bf16": W.CONFIGS[2],
    "d128-partial-bf16": W.custom_config(cfg_id=201, units=2, frames=12, tokens=200, d_k=128,
                                         d_v=128, text_tokens=33, dtype="bf16"),
    "dk64-dv32-fp32": W.custom_config(cfg_id=202, units=2, frames=9, tokens=50, d_k=64, d_v=32,
                                      text_tokens=5, dtype="f32", chunk=2),
    "dk32-dv96-bf16": W.custom_config(cfg_id=203, units=3, frames=11, tokens=70, d_k=32, d_v=96,
                                      text_tokens=0, dtype="bf16", chunk=3, radius=2),
    # frames without tokens: statistics exactly zero, every state the seed
    "no-video-tokens-bf16": W.custom_config(cfg_id=204, units=2, frames=7, tokens=0, d_k=32,
                                            d_v=48, text_tokens=9, dtype="bf16", chunk=2),
    "no-tokens-bf16": W.custom_config(cfg_id=205, units=2, frames=7, tokens=0, d_k=128, d_v=128,
                                      text_tokens=0, dtype="bf16"),
    "no-video-tokens-f32": W.custom_config(cfg_id=206, units=1, frames=6, tokens=0, d_k=16,
                                           d_v=32, text_tokens=5, dtype="f32"),
}


def tol(cfg, stage):
    if cfg.dtype == "f32":
        return 1e-5 if stage == "stats" else 1e-4
    return 4e-3 if stage == "stats" else 1e-2


@pytest.fixture(scope="module", params=sorted(CASES))
def case(request):
    vda = require_gpu()
    import torch
    name = request.param
    cfg = CASES[name]
    h = W.host_inputs(cfg)
    return name, cfg, h, to_device(h, cfg), to_f64(h, cfg), vda, torch


@pytest.mark.parametrize("seed_mode", [0, 1])
def test_stats_and_solve(case, seed_mode):
    name, cfg, h, d, x, vda, torch = case
    say(f"[stages] {name} seed_mode={seed_mode}: stats, solve")
    desc = desc_for(cfg, seed_mode)
    ws = workspace_for(desc)
    U, F, dk, dv = cfg.units, cfg.frames, cfg.d_k, cfg.d_v
    A = torch.empty((U, F + 1, dk, dk), device="cuda")
    B = torch.empty((U, F + 1, dv, dk), device="cuda")
    vda.vda_debug_stats(desc, d["k"], d["v"], d["beta"], d["text_k"], d["text_v"], d["text_beta"],
                        A, B, ws)
    M = torch.empty((U, F + 1, dk, dk), device="cuda")
    seed = torch.empty((U, dv, dk), device="cuda")
    vda.vda_debug_solve(desc, d["k"], d["v"], d["beta"], d["text_k"], d["text_v"], d["text_beta"],
                        M, seed, ws)
    torch.cuda.synchronize()
    A, B, M, seed = (t.cpu().numpy().astype(np.float64) for t in (A, B, M, seed))
    _, tap = oracle_forward(x, cfg, seed_mode, taps=True)
    tscale = 0.5 if seed_mode == 1 else 1.0
    for u in range(U):
        At, Bt = oracle.frame_statistics(x["text_k"][u], x["text_v"][u], tscale * x["text_beta"][u])
        if cfg.text_tokens:
            assert mat_rel_err(A[u, 0], At) <= tol(cfg, "stats")
            assert mat_rel_err(B[u, 0], Bt) <= tol(cfg, "stats")
        else:
            assert np.all(A[u, 0] == 0) and np.all(B[u, 0] == 0)
        np.testing.assert_allclose(M[u, 0], oracle.transition(At), rtol=0, atol=tol(cfg, "M"))
    e_a = mat_rel_err(A[:, 1:], tap["A"])
    e_b = mat_rel_err(B[:, 1:], tap["B"])
    e_m = mat_rel_err(M[:, 1:], tap["M"])
    e_s = mat_rel_err(seed, tap["seed"]) if cfg.text_tokens else float(np.abs(seed).max())
    say(f"  A {e_a:.2e}  B {e_b:.2e}  M {e_m:.2e}  seed {e_s:.2e}")
    assert e_a <= tol(cfg, "stats") and e_b <= tol(cfg, "stats")
    assert e_m <= tol(cfg, "M")
    assert e_s <= tol(cfg, "seed")
    # Prop. 1 on the GPU's own transitions: symmetric, spectral norm <= 1
    Ms = M.reshape(-1, dk, dk)
    assert np.max(np.abs(Ms - Ms.transpose(0, 2, 1))) <= 1e-5
    assert np.max(np.linalg.norm(Ms, 2, axis=(1, 2))) <= 1.0 + 1e-5


def test_chunks_and_states(case):
    name, cfg, h, d, x, vda, torch = case
    say(f"[stages] {name}: chunk maps, boundary states")
    desc = desc_for(cfg, 0)
    ws = workspace_for(desc)
    U, F, dk, dv, C = cfg.units, cfg.frames, cfg.d_k, cfg.d_v, cfg.chunk
    n = cfg.n_chunks
    Mc = torch.empty((U, n, dk, dk), device="cuda")
    Jf = torch.empty((U, n, dv, dk), device="cuda")
    Jr = torch.empty((U, n, dv, dk), device="cuda")
    vda.vda_debug_chunks(desc, d["k"], d["v"], d["beta"], d["text_k"], d["text_v"],
                         d["text_beta"], Mc, Jf, Jr, ws)
    P = torch.empty((U, n + 1, dv, dk), device="cuda")
    R = torch.empty((U, n + 1, dv, dk), device="cuda")
    vda.vda_debug_states(desc, d["k"], d["v"], d["beta"], d["text_k"], d["text_v"],
                         d["text_beta"], P, R, ws)
    torch.cuda.synchronize()
    Mc, Jf, Jr, P, R = (t.cpu().numpy().astype(np.float64) for t in (Mc, Jf, Jr, P, R))
    _, tap = oracle_forward(x, cfg, 0, taps=True)
    # expected chunk maps: the oracle's per-frame maps composed (associativity,
    # pinned in the oracle suite by pin_chunk_composition)
    for u in range(U):
        for j in range(n):
            lo, hi = j * C, min(j * C + C, F)
            m = np.eye(dk)
            jf = np.zeros((dv, dk))
            for f in range(lo, hi):
                m = m @ tap["M"][u, f]
                jf = (jf + tap["B"][u, f]) @ tap["M"][u, f]
            jr = np.zeros((dv, dk))
            for f in range(hi - 1, lo - 1, -1):
                jr = (jr + tap["B"][u, f]) @ tap["M"][u, f]
            assert mat_rel_err(Mc[u, j], m) <= tol(cfg, "Mc"), (u, j)
            assert mat_rel_err(Jf[u, j], jf) <= tol(cfg, "J"), (u, j)
            assert mat_rel_err(Jr[u, j], jr) <= tol(cfg, "J"), (u, j)
    e_p = mat_rel_err(P, tap["P"])
    e_r = mat_rel_err(R, tap["R"])
    say(f"  P {e_p:.2e}  R {e_r:.2e}")
    assert e_p <= tol(cfg, "P") and e_r <= tol(cfg, "R")
    # exactly once (Eq. (1b)): the two seeds are equal halves
    assert np.array_equal(P[:, 0], R[:, n])


def frame_maps(d, cfg, vda, torch, solver=0):
    """vda_debug_frame_maps: (M, J, flag), M and J as fp64 host arrays."""
    U, F, dk, dv = cfg.units, cfg.frames, cfg.d_k, cfg.d_v
    desc = desc_for(cfg, 0, 0, solver)
    ws = workspace_for(desc)
    M = torch.empty((U, F + 1, dk, dk), device="cuda")
    J = torch.empty((U, F + 1, dv, dk), device="cuda")
    flag = torch.full((1,), vda.VDA_OK, dtype=torch.int32, device="cuda")
    vda.vda_debug_frame_maps(desc, d["k"], d["v"], d["beta"], d["text_k"], d["text_v"],
                             d["text_beta"], M, J, flag, ws)
    torch.cuda.synchronize()
    return (M.cpu().numpy().astype(np.float64), J.cpu().numpy().astype(np.float64),
            int(flag.item()))


def test_frame_maps(case):
    """Per-frame J_t = B_t M_t (App. A.1 Eq. (A.1)): against the fp64 product of
    the GPU's own B_t and M_t (the tap's product alone, fp32 dot products of d_k
    terms: 1e-5), and against the oracle's per-frame maps (the stage bar); the
    not-SPD flag stays clear."""
    name, cfg, h, d, x, vda, torch = case
    say(f"[stages] {name}: per-frame maps")
    U, F, dk, dv = cfg.units, cfg.frames, cfg.d_k, cfg.d_v
    M, J, flag = frame_maps(d, cfg, vda, torch)
    assert flag == vda.VDA_OK
    desc = desc_for(cfg, 0)
    ws = workspace_for(desc)
    A = torch.empty((U, F + 1, dk, dk), device="cuda")
    B = torch.empty((U, F + 1, dv, dk), device="cuda")
    vda.vda_debug_stats(desc, d["k"], d["v"], d["beta"], d["text_k"], d["text_v"], d["text_beta"],
                        A, B, ws)
    torch.cuda.synchronize()
    B = B.cpu().numpy().astype(np.float64)
    e_own = mat_rel_err(J, B @ M)
    _, tap = oracle_forward(x, cfg, 0, taps=True)
    e_j = mat_rel_err(J[:, 1:], tap["B"] @ tap["M"])
    e_m = mat_rel_err(M[:, 1:], tap["M"])
    say(f"  J vs own B M {e_own:.2e}, J vs oracle {e_j:.2e}, M vs oracle {e_m:.2e}")
    assert e_own <= 1e-5
    assert e_j <= tol(cfg, "J") and e_m <= tol(cfg, "M")
    for u in range(U):  # the text frame
        At, Bt = oracle.frame_statistics(x["text_k"][u], x["text_v"][u], x["text_beta"][u])
        Jt = Bt @ oracle.transition(At)
        if cfg.text_tokens:
            assert mat_rel_err(J[u, 0], Jt) <= tol(cfg, "J")
        else:
            assert np.all(J[u, 0] == 0)


@pytest.mark.parametrize("solver", [0, 1])
def test_not_spd_flag(solver):
    """A negative beta breaks the precondition of the frame statistics (sqrt(beta)
    is NaN, so is a pivot): the tap's flag reads VDA_ERR_NOT_SPD; on the same
    inputs with beta >= 0 it stays VDA_OK."""
    vda = require_gpu()
    import torch
    cfg = CASES["small-bf16"]
    h = W.host_inputs(cfg)
    d = to_device(h, cfg)
    _, _, flag = frame_maps(d, cfg, vda, torch, solver)
    assert flag == vda.VDA_OK
    bad = dict(d)
    bad["beta"] = d["beta"].clone()
    bad["beta"][1, 3, :5] = -1.0  # unit 1, latent frame 3
    M, J, flag = frame_maps(bad, cfg, vda, torch, solver)
    say(f"[stages] negative beta, solver {solver}: flag {flag}")
    assert flag == vda.VDA_ERR_NOT_SPD
    assert np.all(np.isfinite(M[0]))  # other units untouched

"""The descriptor's two arithmetic options against the fp64 oracle.

solver = 1 (blocked Cholesky I + A_t = L L^T, M_t = L^-T L^-1, the
factor-and-solve form of the frame-wise transition, "Video DeltaNet" Sec. 3.2
Eq. (5)): the transitions against the fp64 inverse of the same statistics the
GPU produced (so only the solve's own rounding is measured), with the default
sweep's error beside them, then the whole output against the oracle, on the
stage cases and on the full-size 768p share.

fp32_products = 1 (the composition and the scan with exact fp32 products,
the fp32 state updates of Sec. 5): the boundary states P and R and the output
against the oracle on small cases and on every unit of the full-size stress
workload, with the split-bf16 path's errors reported beside them and the
distance between the two paths' states (the split products' own error, both
sharing the same statistics and transitions).

Bars.  A transition: relative Frobenius error <= 4 d_k u kappa(I + A_t) (the
usual backward-stable bound gamma_n kappa for an SPD inverse in fp32,
u = 2^-24) and <= 2e-3 absolute cap-free check of symmetry (exact: both
kernels write one triangle mirrored).  States and outputs: the stage and
end-to-end tolerances of the default path."""
import dataclasses

import numpy as np
import pytest

import workloads as W
from gpu_helpers import (TOL_OUT, desc_for, device_to_host_f64, gpu_forward, mat_rel_err,
                         oracle_forward, out_to_f64, require_gpu, row_rel_err, say, to_device,
                         to_f64, workspace_for)

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24

CASES = {
    "tiny-fp32": W.CONFIGS[1],
    "small-bf16": W.CONFIGS[2],
    "d128-partial-bf16": W.custom_config(cfg_id=201, units=2, frames=12, tokens=200, d_k=128,
                                         d_v=128, text_tokens=33, dtype="bf16"),
    "dk64-dv32-fp32": W.custom_config(cfg_id=202, units=2, frames=9, tokens=50, d_k=64, d_v=32,
                                      text_tokens=5, dtype="f32", chunk=2),
    "dk96-stress-bf16": W.custom_config(cfg_id=207, units=2, frames=8, tokens=300, d_k=96,
                                        d_v=64, text_tokens=40, dtype="bf16", beta_mu=2.0,
                                        stress=True, chunk=3),
    "dk48-ragged-f32": W.custom_config(cfg_id=208, units=3, frames=7, tokens=37, d_k=48, d_v=80,
                                       text_tokens=0, dtype="f32", chunk=4, radius=2),
    "dk16-f32": W.custom_config(cfg_id=209, units=1, frames=5, tokens=9, d_k=16, d_v=16,
                                text_tokens=3, dtype="f32", chunk=1),
    "no-video-tokens-bf16": W.custom_config(cfg_id=204, units=2, frames=7, tokens=0, d_k=32,
                                            d_v=48, text_tokens=9, dtype="bf16", chunk=2),
}


def stats_and_solves(d, cfg, vda, torch):
    """The GPU's frame statistics A and its transitions from both solvers."""
    U, F, dk, dv = cfg.units, cfg.frames, cfg.d_k, cfg.d_v
    res = {}
    for solver in (0, 1):
        desc = desc_for(cfg, 0, 0, solver)
        ws = workspace_for(desc)
        if solver == 0:
            A = torch.empty((U, F + 1, dk, dk), device="cuda")
            B = torch.empty((U, F + 1, dv, dk), device="cuda")
            vda.vda_debug_stats(desc, d["k"], d["v"], d["beta"], d["text_k"], d["text_v"],
                                d["text_beta"], A, B, ws)
            res["A"] = A
        M = torch.empty((U, F + 1, dk, dk), device="cuda")
        seed = torch.empty((U, dv, dk), device="cuda")
        vda.vda_debug_solve(desc, d["k"], d["v"], d["beta"], d["text_k"], d["text_v"],
                            d["text_beta"], M, seed, ws)
        res[solver] = M
    torch.cuda.synchronize()
    return res


def check_transitions(A, M_sweep, M_chol, dk):
    """Both solvers against the fp64 inverse of the same I + A; returns the
    worst errors and asserts the bound."""
    worst = {0: 0.0, 1: 0.0}
    for a, ms, mc in zip(A.reshape(-1, dk, dk), M_sweep.reshape(-1, dk, dk),
                         M_chol.reshape(-1, dk, dk)):
        # the statistics kernel may leave the blocks above the diagonal unset:
        # the matrix is the symmetric completion of its lower triangle
        lo = np.tril(a)
        g = np.eye(dk) + lo + np.tril(a, -1).T
        exact = np.linalg.inv(g)
        kappa = np.linalg.cond(g)
        bar = 4 * dk * U32 * kappa
        for s, m in ((0, ms), (1, mc)):
            e = np.linalg.norm(m - exact) / np.linalg.norm(exact)
            worst[s] = max(worst[s], e)
            assert e <= bar, (s, e, bar, kappa)
        assert np.array_equal(mc, mc.T)
    return worst


@pytest.fixture(scope="module", params=sorted(CASES))
def case(request):
    vda = require_gpu()
    import torch
    name = request.param
    cfg = CASES[name]
    h = W.host_inputs(cfg)
    return name, cfg, to_device(h, cfg), to_f64(h, cfg), vda, torch


def test_cholesky_transitions_and_output(case):
    name, cfg, d, x, vda, torch = case
    say(f"[solver] {name}: transitions of both solvers, then the output with solver 1")
    r = stats_and_solves(d, cfg, vda, torch)
    A = r["A"].cpu().numpy().astype(np.float64)
    Ms = r[0].cpu().numpy().astype(np.float64)
    Mc = r[1].cpu().numpy().astype(np.float64)
    worst = check_transitions(A, Ms, Mc, cfg.d_k)
    say(f"  M rel err vs fp64 inverse: sweep {worst[0]:.2e}  cholesky {worst[1]:.2e}")
    for seed_mode in (0, 1):
        out = gpu_forward(d, cfg, seed_mode, solver=1)
        ref = oracle_forward(x, cfg, seed_mode)
        err = row_rel_err(out_to_f64(out, cfg), ref)
        say(f"  seed_mode {seed_mode}: output max row-rel err {err:.3e}")
        assert err <= TOL_OUT[cfg.dtype]
    # the decay form shares the solve
    cfg_a = dataclasses.replace(cfg, alpha_mu=3.0)
    h = W.host_inputs(cfg_a)
    out = gpu_forward(to_device(h, cfg_a), cfg_a, solver=1)
    err = row_rel_err(out_to_f64(out, cfg_a), oracle_forward(to_f64(h, cfg_a), cfg_a))
    say(f"  decay: output max row-rel err {err:.3e}")
    assert err <= TOL_OUT[cfg.dtype]


def state_errors(d, x, cfg, vda, torch, fp32_products, units=None):
    U, dk, dv, n = cfg.units, cfg.d_k, cfg.d_v, cfg.n_chunks
    desc = desc_for(cfg, 0, fp32_products)
    ws = workspace_for(desc)
    P = torch.empty((U, n + 1, dv, dk), device="cuda")
    R = torch.empty((U, n + 1, dv, dk), device="cuda")
    vda.vda_debug_states(desc, d["k"], d["v"], d["beta"], d["text_k"], d["text_v"],
                         d["text_beta"], P, R, ws)
    torch.cuda.synchronize()
    return P.cpu().numpy().astype(np.float64), R.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("name", ["small-bf16", "d128-partial-bf16", "dk96-stress-bf16",
                                  "no-video-tokens-bf16"])
def test_fp32_products_small(name):
    vda = require_gpu()
    import torch
    cfg = CASES[name]
    h = W.host_inputs(cfg)
    d, x = to_device(h, cfg), to_f64(h, cfg)
    say(f"[products] {name}: states and output, split-bf16 and fp32 products")
    _, tap = oracle_forward(x, cfg, 0, taps=True)
    Pf, Rf = state_errors(d, x, cfg, vda, torch, 1)
    Ps, Rs = state_errors(d, x, cfg, vda, torch, 0)
    ef = max(mat_rel_err(Pf, tap["P"]), mat_rel_err(Rf, tap["R"]))
    es = max(mat_rel_err(Ps, tap["P"]), mat_rel_err(Rs, tap["R"]))
    split = max(mat_rel_err(Ps, Pf), mat_rel_err(Rs, Rf))
    say(f"  P/R vs oracle: fp32 products {ef:.2e}, split {es:.2e}; split vs fp32 {split:.2e}")
    assert ef <= 1e-2 and es <= 1e-2
    assert split <= 1e-3
    assert np.array_equal(Pf[:, 0], Rf[:, cfg.n_chunks])
    for seed_mode in (0, 1):
        out = gpu_forward(d, cfg, seed_mode, fp32_products=1)
        err = row_rel_err(out_to_f64(out, cfg), oracle_forward(x, cfg, seed_mode))
        say(f"  seed_mode {seed_mode}: output max row-rel err {err:.3e}")
        assert err <= TOL_OUT[cfg.dtype]


def test_fp32_input_ignores_products_flag():
    """fp32 features always take the fp32 products: the flag changes nothing."""
    vda = require_gpu()
    import torch
    cfg = CASES["dk64-dv32-fp32"]
    d = to_device(W.host_inputs(cfg), cfg)
    a = gpu_forward(d, cfg, fp32_products=0)
    b = gpu_forward(d, cfg, fp32_products=1)
    assert torch.equal(a, b)


@pytest.mark.slow
def test_fp32_products_stress_fullsize():
    """Every unit of the full-size stress workload (kappa(I + A_t) in the
    hundreds): P, R and the output with fp32 products, the split path's
    errors beside them."""
    vda = require_gpu()
    import torch
    cfg = W.CONFIGS[5]
    say(f"[products] {cfg.name}: generating inputs")
    d = W.device_inputs(cfg)
    Pf, Rf = state_errors(d, None, cfg, vda, torch, 1)
    Ps, Rs = state_errors(d, None, cfg, vda, torch, 0)
    out_f = gpu_forward(d, cfg, fp32_products=1)
    out_s = gpu_forward(d, cfg, fp32_products=0)
    worst = dict(pf=0.0, ps=0.0, of=0.0, os=0.0)
    for u in range(cfg.units):
        xu = device_to_host_f64(d, cfg, [u])
        ref, tap = oracle_forward(xu, cfg, 0, taps=True)
        pf = max(mat_rel_err(Pf[u:u + 1], tap["P"]), mat_rel_err(Rf[u:u + 1], tap["R"]))
        ps = max(mat_rel_err(Ps[u:u + 1], tap["P"]), mat_rel_err(Rs[u:u + 1], tap["R"]))
        of = row_rel_err(out_to_f64(out_f[u:u + 1], cfg), ref)
        os_ = row_rel_err(out_to_f64(out_s[u:u + 1], cfg), ref)
        say(f"  unit {u}: P/R fp32 {pf:.3e} split {ps:.3e}; out fp32 {of:.3e} split {os_:.3e}")
        for k, v in (("pf", pf), ("ps", ps), ("of", of), ("os", os_)):
            worst[k] = max(worst[k], v)
    split = max(mat_rel_err(Ps, Pf), mat_rel_err(Rs, Rf))
    say(f"[products] {cfg.name}: worst P/R fp32 {worst['pf']:.3e} split {worst['ps']:.3e}; "
        f"out fp32 {worst['of']:.3e} split {worst['os']:.3e}; split vs fp32 states {split:.3e}")
    assert worst["pf"] <= 1e-2 and worst["ps"] <= 1e-2
    assert worst["of"] <= TOL_OUT["bf16"] and worst["os"] <= TOL_OUT["bf16"]
    assert split <= 1e-3


@pytest.mark.slow
def test_cholesky_768p_fullsize():
    """The full-size 768p share with solver 1: transitions of two units
    against the fp64 inverse of the GPU's statistics, the output of four units
    across the XCD ranges against the oracle, and every unit against the
    default solver's output."""
    vda = require_gpu()
    import torch
    cfg = W.CONFIGS[4]
    say(f"[solver] {cfg.name}: generating inputs")
    d = W.device_inputs(cfg)
    r = stats_and_solves(d, cfg, vda, torch)
    for u in (0, 15):
        worst = check_transitions(r["A"][u].cpu().numpy().astype(np.float64),
                                  r[0][u].cpu().numpy().astype(np.float64),
                                  r[1][u].cpu().numpy().astype(np.float64), cfg.d_k)
        say(f"  unit {u}: M rel err sweep {worst[0]:.2e} cholesky {worst[1]:.2e}")
    del r
    out_c = gpu_forward(d, cfg, solver=1)
    out_c2 = gpu_forward(d, cfg, solver=1)
    assert torch.equal(out_c.view(torch.int16), out_c2.view(torch.int16)), "not deterministic"
    del out_c2
    out_s = gpu_forward(d, cfg, solver=0)
    diff = row_rel_err(out_to_f64(out_c, cfg), out_to_f64(out_s, cfg))
    say(f"  cholesky vs sweep output, every unit: max row-rel diff {diff:.3e}")
    assert diff <= TOL_OUT["bf16"]
    for u in (0, 5, 10, 15):
        ref = oracle_forward(device_to_host_f64(d, cfg, [u]), cfg, 0)
        err = row_rel_err(out_to_f64(out_c[u:u + 1], cfg), ref)
        say(f"  unit {u}: max row-rel err {err:.3e}")
        assert err <= TOL_OUT["bf16"]

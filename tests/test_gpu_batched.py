"""The batched comparison rules ("Video DeltaNet", Sec. 3.1 Eq. (3a)/(3c) and
App. A.2: SANA-WM's frozen-state update S_t = S_{t-1} (I - A_t) + B_t, rule 1,
and with its frame-size key scaling, rule 2) on the HIP path, through the C ABI
with desc.rule, against the fp64 oracle.

Stages: the per-frame factor I - s A (vda_debug_solve), the chunk maps and the
boundary states.  End to end: the usual row-relative bars.  Rule 1 runs on
shapes where A stays below 2 (few tokens per frame against d_k): past that its
factor expands, the states grow geometrically and the bf16 rounding of the
inputs is amplified with them (App. A.2), which the contraction test shows
on purpose with a growth factor the pages predict.
"""
import numpy as np
import pytest

import workloads as W
from gpu_helpers import (TOL_OUT, desc_for, gpu_forward, mat_rel_err, oracle_forward,
                         out_to_f64, require_gpu, row_rel_err, say, to_device, to_f64,
                         workspace_for)

pytestmark = pytest.mark.gpu

C = W.custom_config

STAGE_CASES = {
    "rule1-d32-bf16": C(cfg_id=601, units=2, frames=12, tokens=16, d_k=32, d_v=32,
                        text_tokens=5, dtype="bf16", rule=1),
    "rule2-d128-bf16": C(cfg_id=602, units=2, frames=13, tokens=300, d_k=128, d_v=128,
                         text_tokens=33, dtype="bf16", rule=2),
    "rule2-dk48-dv80-f32": C(cfg_id=603, units=2, frames=11, tokens=70, d_k=48, d_v=80,
                             text_tokens=6, dtype="f32", chunk=3, rule=2),
    "rule1-f32": C(cfg_id=604, units=1, frames=9, tokens=8, d_k=16, d_v=16, text_tokens=3,
                   dtype="f32", chunk=2, rule=1),
}

PARITY_CASES = {
    "rule2-small-bf16": C(cfg_id=611, units=4, frames=40, tokens=256, d_k=64, d_v=64,
                          text_tokens=64, dtype="bf16", rule=2),
    "rule2-medium-bf16": C(cfg_id=612, units=2, frames=60, tokens=1024, d_k=128, d_v=128,
                           text_tokens=256, dtype="bf16", rule=2),
    "rule2-tiny-f32": C(cfg_id=613, units=1, frames=20, tokens=16, d_k=16, d_v=16,
                        text_tokens=8, dtype="f32", rule=2),
    "rule2-anchors-bf16": C(cfg_id=614, units=2, frames=16, tokens=100, d_k=64, d_v=64,
                            text_tokens=9, dtype="bf16", rule=2, anchors=True),
    "rule2-partial-chunk-one-frame-bf16": C(cfg_id=615, units=2, frames=11, tokens=48,
                                            d_k=128, d_v=128, text_tokens=9, dtype="bf16",
                                            rule=2),
    "rule2-chunk1-f32": C(cfg_id=616, units=1, frames=7, tokens=12, d_k=32, d_v=16,
                          text_tokens=2, dtype="f32", chunk=1, radius=1, rule=2),
    "rule2-no-text-bf16": C(cfg_id=617, units=2, frames=10, tokens=64, d_k=64, d_v=64,
                            text_tokens=0, dtype="bf16", rule=2),
    "rule1-d64-bf16": C(cfg_id=618, units=2, frames=15, tokens=24, d_k=64, d_v=64,
                        text_tokens=8, dtype="bf16", rule=1),
    "rule1-tiny-f32": C(cfg_id=619, units=1, frames=20, tokens=16, d_k=16, d_v=16,
                        text_tokens=8, dtype="f32", rule=1),
    "rule1-d128-bf16": C(cfg_id=620, units=2, frames=16, tokens=64, d_k=128, d_v=128,
                         text_tokens=16, dtype="bf16", rule=1),
}


@pytest.fixture(scope="module", params=sorted(STAGE_CASES))
def stage_case(request):
    vda = require_gpu()
    import torch
    name = request.param
    cfg = STAGE_CASES[name]
    h = W.host_inputs(cfg)
    return name, cfg, h, to_device(h, cfg), to_f64(h, cfg), vda, torch


@pytest.mark.parametrize("seed_mode", [0, 1])
def test_batched_stages(stage_case, seed_mode):
    name, cfg, h, d, x, vda, torch = stage_case
    say(f"[batched stages] {name} seed_mode={seed_mode}")
    desc = desc_for(cfg, seed_mode)
    ws = workspace_for(desc)
    U, F, dk, dv, Cn = cfg.units, cfg.frames, cfg.d_k, cfg.d_v, cfg.chunk
    n = cfg.n_chunks
    M = torch.empty((U, F + 1, dk, dk), device="cuda")
    seed = torch.empty((U, dv, dk), device="cuda")
    vda.vda_debug_solve(desc, d["k"], d["v"], d["beta"], d["text_k"], d["text_v"],
                        d["text_beta"], M, seed, ws)
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
    M, seed, Mc, Jf, Jr, P, R = (t.cpu().numpy().astype(np.float64)
                                 for t in (M, seed, Mc, Jf, Jr, P, R))
    _, tap = oracle_forward(x, cfg, seed_mode, taps=True)
    tol = 1e-4 if cfg.dtype == "f32" else 1e-2
    # the factor I - s A of every latent frame, and the seed
    assert mat_rel_err(M[:, 1:], tap["M"]) <= tol
    assert mat_rel_err(seed, tap["seed"]) <= tol if cfg.text_tokens else np.all(seed == 0)
    # chunk maps: S -> S M + B composed frame by frame (oracle taps, rule 2 scaled)
    for u in range(U):
        for j in range(n):
            lo, hi = j * Cn, min(j * Cn + Cn, F)
            mc = np.eye(dk)
            jf = np.zeros((dv, dk))
            for f in range(lo, hi):
                mc = mc @ tap["M"][u, f]
                jf = jf @ tap["M"][u, f] + tap["B"][u, f]
            jr = np.zeros((dv, dk))
            for f in range(hi - 1, lo - 1, -1):
                jr = jr @ tap["M"][u, f] + tap["B"][u, f]
            assert mat_rel_err(Mc[u, j], mc) <= tol, (u, j)
            assert mat_rel_err(Jf[u, j], jf) <= tol, (u, j)
            assert mat_rel_err(Jr[u, j], jr) <= tol, (u, j)
    e_p, e_r = mat_rel_err(P, tap["P"]), mat_rel_err(R, tap["R"])
    say(f"  P {e_p:.2e}  R {e_r:.2e}")
    assert e_p <= tol and e_r <= tol


@pytest.mark.parametrize("name", sorted(PARITY_CASES))
@pytest.mark.parametrize("seed_mode", [0, 1])
def test_batched_parity(name, seed_mode):
    cfg = PARITY_CASES[name]
    require_gpu()
    say(f"[batched parity] {name} seed_mode={seed_mode}")
    h = W.host_inputs(cfg)
    got = out_to_f64(gpu_forward(to_device(h, cfg), cfg, seed_mode), cfg)
    ref = oracle_forward(to_f64(h, cfg), cfg, seed_mode)
    err = row_rel_err(got, ref)
    say(f"  max row-rel err {err:.3e} (bar {TOL_OUT[cfg.dtype]:.0e})")
    assert np.all(np.isfinite(got))
    assert err <= TOL_OUT[cfg.dtype]


@pytest.mark.parametrize("rule", [0, 1, 2])
def test_contraction_of_each_rule(rule):
    """App. A.2 on the GPU: every frame holds U copies of one unit key k with a
    common beta and zero values, the text holds k too; the k-component of the
    forward boundary state is multiplied per chunk (of one frame) by
    1 / (1 + U beta) (rule 0), 1 - U beta (rule 1: |.| > 1 since U beta > 2)
    or 1 - beta (rule 2)."""
    vda = require_gpu()
    import torch
    U, F, dk, dv, b = 16, 6, 32, 32, 0.25  # U b = 4
    cfg = C(cfg_id=630, units=1, frames=F, tokens=U, d_k=dk, d_v=dv, text_tokens=1,
            dtype="f32", chunk=1, radius=0, rule=rule)
    say(f"[batched] contraction, rule {rule}")
    rng = np.random.default_rng(7)
    k = rng.standard_normal(dk)
    k /= np.linalg.norm(k)
    h = W.host_inputs(cfg)
    h["k"][:] = k.astype(np.float32)
    h["v"][:] = 0.0
    h["beta"][:] = b
    h["text_k"][:] = k.astype(np.float32)
    d = to_device(h, cfg)
    desc = desc_for(cfg)
    ws = workspace_for(desc)
    P = torch.empty((1, F + 1, dv, dk), device="cuda")
    R = torch.empty((1, F + 1, dv, dk), device="cuda")
    vda.vda_debug_states(desc, d["k"], d["v"], d["beta"], d["text_k"], d["text_v"],
                         d["text_beta"], P, R, ws)
    torch.cuda.synchronize()
    Pk = P.cpu().numpy().astype(np.float64)[0] @ k
    factor = {0: 1 / (1 + U * b), 1: 1 - U * b, 2: 1 - b}[rule]
    for j in range(F):
        np.testing.assert_allclose(Pk[j + 1], factor * Pk[j], rtol=1e-4,
                                   atol=1e-6 * np.abs(Pk[j]).max())
    growth = np.linalg.norm(Pk[F]) / np.linalg.norm(Pk[0])
    say(f"  |P_F k| / |P_0 k| = {growth:.3e}")
    assert (growth > 1) == (rule == 1)

"""Boundary anchors ("Video DeltaNet", Sec. 2.1, Sec. 2.2, App. A.3 and
Algorithm 1 steps 2 and 7) on the HIP path, through the C ABI with
desc.anchors = 1, against the fp64 oracle (which follows the pages' interior
frame indexing, not the identity-frame shortcut the kernels take).

Stages: the statistics of the anchor frames are exactly zero (their tokens
are never read), and the chunk-boundary states P[j], R[j] equal the oracle's
interior-indexed states through frame min(jC - 1, F - 2) and from frame
max(jC, 1); tolerances as for the plain stages.  End to end: the same
row-relative bar as the plain forward (1e-4 fp32, 2e-2 bf16), with and without
decay, both seed modes; anchor rows and bypassed rows are exactly zero (also
with rms_eps = 0, where a computed zero readout would give NaN).
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
    "anchors-d128-bf16": C(cfg_id=501, units=2, frames=13, tokens=200, d_k=128, d_v=128,
                           text_tokens=33, dtype="bf16", anchors=True),
    "anchors-decay-dk48-bf16": C(cfg_id=502, units=2, frames=11, tokens=70, d_k=48, d_v=80,
                                 text_tokens=6, dtype="bf16", chunk=3, radius=1, alpha_mu=1.0,
                                 anchors=True),
    "anchors-decay-f32": C(cfg_id=503, units=2, frames=9, tokens=50, d_k=64, d_v=32,
                           text_tokens=5, dtype="f32", chunk=2, alpha_mu=2.0, anchors=True),
}

PARITY_CASES = {
    "anchors-small-bf16": C(cfg_id=511, units=4, frames=40, tokens=256, d_k=64, d_v=64,
                            text_tokens=64, dtype="bf16", anchors=True),
    "anchors-medium-decay-bf16": C(cfg_id=512, units=2, frames=60, tokens=1024, d_k=128,
                                   d_v=128, text_tokens=256, dtype="bf16", alpha_mu=3.0,
                                   anchors=True),
    "anchors-tiny-f32": C(cfg_id=513, units=1, frames=20, tokens=16, d_k=16, d_v=16,
                          text_tokens=8, dtype="f32", anchors=True),
    "anchors-decay-f32": C(cfg_id=514, units=2, frames=13, tokens=20, d_k=32, d_v=48,
                           text_tokens=3, dtype="f32", alpha_mu=2.0, anchors=True),
    # chunk 1's window spans the clip: frames 5..9 bypassed
    "anchors-bypass-chunk-bf16": C(cfg_id=515, units=2, frames=11, tokens=48, d_k=64, d_v=64,
                                   text_tokens=9, dtype="bf16", anchors=True),
    "anchors-bypass-decay-bf16": C(cfg_id=516, units=1, frames=11, tokens=48, d_k=128,
                                   d_v=128, text_tokens=9, dtype="bf16", alpha_mu=1.0,
                                   anchors=True),
    # every window spans the clip
    "anchors-all-bypassed": C(cfg_id=517, units=1, frames=10, tokens=32, d_k=32, d_v=32,
                              text_tokens=5, dtype="bf16", anchors=True),
    "anchors-one-frame": C(cfg_id=518, units=2, frames=1, tokens=32, d_k=32, d_v=32,
                           text_tokens=5, dtype="bf16", anchors=True),
    "anchors-two-frames-decay": C(cfg_id=519, units=2, frames=2, tokens=32, d_k=32, d_v=32,
                                  text_tokens=5, dtype="bf16", alpha_mu=1.0, anchors=True),
    "anchors-three-frames-f32": C(cfg_id=520, units=1, frames=3, tokens=8, d_k=16, d_v=16,
                                  text_tokens=2, dtype="f32", chunk=1, radius=0,
                                  anchors=True),
    "anchors-chunk1-radius0-decay": C(cfg_id=521, units=1, frames=8, tokens=32, d_k=32,
                                      d_v=32, text_tokens=5, dtype="bf16", chunk=1, radius=0,
                                      alpha_mu=1.0, anchors=True),
    "anchors-ragged-tokens": C(cfg_id=522, units=2, frames=16, tokens=1027, d_k=128,
                               d_v=128, text_tokens=100, dtype="bf16", anchors=True),
    "anchors-eps-zero-f32": C(cfg_id=523, units=1, frames=11, tokens=16, d_k=16, d_v=16,
                              text_tokens=8, dtype="f32", rms_eps=0.0, anchors=True),
    "anchors-eps-zero-bf16": C(cfg_id=524, units=1, frames=16, tokens=16, d_k=32, d_v=32,
                               text_tokens=8, dtype="bf16", rms_eps=0.0, anchors=True),
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
def test_anchor_stats_and_states(stage_case, seed_mode):
    name, cfg, h, d, x, vda, torch = stage_case
    say(f"[anchor stages] {name} seed_mode={seed_mode}")
    desc = desc_for(cfg, seed_mode)
    ws = workspace_for(desc)
    U, F, dk, dv, Cn = cfg.units, cfg.frames, cfg.d_k, cfg.d_v, cfg.chunk
    n = cfg.n_chunks
    A = torch.empty((U, F + 1, dk, dk), device="cuda")
    B = torch.empty((U, F + 1, dv, dk), device="cuda")
    vda.vda_debug_stats(desc, d["k"], d["v"], d["beta"], d["text_k"], d["text_v"],
                        d["text_beta"], A, B, ws)
    P = torch.empty((U, n + 1, dv, dk), device="cuda")
    R = torch.empty((U, n + 1, dv, dk), device="cuda")
    if "alpha" in d:
        vda.vda_debug_states_decay(desc, d["k"], d["v"], d["beta"], d["alpha"], d["text_k"],
                                   d["text_v"], d["text_beta"], P, R, ws)
    else:
        vda.vda_debug_states(desc, d["k"], d["v"], d["beta"], d["text_k"], d["text_v"],
                             d["text_beta"], P, R, ws)
    torch.cuda.synchronize()
    A, B, P, R = (t.cpu().numpy().astype(np.float64) for t in (A, B, P, R))
    # anchor frames (workspace frames 1 and F) are never read: exactly zero
    assert np.all(A[:, 1] == 0) and np.all(A[:, F] == 0)
    assert np.all(B[:, 1] == 0) and np.all(B[:, F] == 0)
    _, tap = oracle_forward(x, cfg, seed_mode, taps=True)
    tol = 1e-4 if cfg.dtype == "f32" else 1e-2
    assert mat_rel_err(A[:, 2:F], tap["A"][:, 1:F - 1]) <= (1e-5 if cfg.dtype == "f32" else 4e-3)
    # chunk boundary j: forward through frame jC - 1 (clipped to the interior,
    # P_0 = seed below it), reverse from frame jC (R_{F-1} = seed at j = n)
    Pm = np.stack([tap["P"][:, max(min(j * Cn - 1, F - 2), 0)] for j in range(n + 1)], axis=1)
    Rm = np.stack([tap["R"][:, min(max(j * Cn, 1), F - 1) - 1] for j in range(n + 1)], axis=1)
    e_p, e_r = mat_rel_err(P, Pm), mat_rel_err(R, Rm)
    say(f"  P {e_p:.2e}  R {e_r:.2e}")
    assert e_p <= tol and e_r <= tol


def run_case(cfg, seed_mode=0):
    require_gpu()
    h = W.host_inputs(cfg)
    d = to_device(h, cfg)
    got = out_to_f64(gpu_forward(d, cfg, seed_mode), cfg)
    ref = oracle_forward(to_f64(h, cfg), cfg, seed_mode)
    return got, ref


def zero_rows(cfg):
    """Frames whose rows the linear path leaves at zero (anchors, bypass)."""
    F, Cn, r = cfg.frames, cfg.chunk, cfg.radius
    z = set()
    for t in range(F):
        c = t // Cn
        if t in (0, F - 1) or (c - r <= 0 and Cn * (c + r + 1) >= F):
            z.add(t)
    return z


@pytest.mark.parametrize("name", sorted(PARITY_CASES))
@pytest.mark.parametrize("seed_mode", [0, 1])
def test_anchor_parity(name, seed_mode):
    cfg = PARITY_CASES[name]
    say(f"[anchor parity] {name} seed_mode={seed_mode}")
    got, ref = run_case(cfg, seed_mode)
    err = row_rel_err(got, ref)
    say(f"  max row-rel err {err:.3e} (bar {TOL_OUT[cfg.dtype]:.0e})")
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got))
    for t in zero_rows(cfg):
        assert np.all(got[:, t] == 0.0), t
    assert err <= TOL_OUT[cfg.dtype]


def test_anchor_inputs_never_read():
    """Redrawing the anchor frames' k, v, beta, q, gate and gates leaves every
    output bit unchanged (their rows are removed from the linear inputs)."""
    require_gpu()
    cfg = C(cfg_id=530, units=2, frames=16, tokens=40, d_k=64, d_v=64, text_tokens=9,
            dtype="bf16", alpha_mu=2.0, anchors=True)
    say("[anchors] anchor inputs never read")
    h = W.host_inputs(cfg)
    h2 = W.host_inputs(C(cfg_id=531, units=2, frames=16, tokens=40, d_k=64, d_v=64,
                         text_tokens=9, dtype="bf16", alpha_mu=2.0, anchors=True))
    a = out_to_f64(gpu_forward(to_device(h, cfg), cfg), cfg)
    hp = {k: v.copy() for k, v in h.items()}
    for key in ("q", "k", "v", "beta", "gate", "alpha"):
        hp[key][:, 0] = h2[key][:, 0]
        hp[key][:, -1] = h2[key][:, -1]
    b = out_to_f64(gpu_forward(to_device(hp, cfg), cfg), cfg)
    assert np.array_equal(a, b)

"""Channel-wise decay ("Video DeltaNet", Sec. 3.1 Eq. (2), App. A.1 Eq. (A.1),
App. A.3 Eq. (A.4)) on the HIP path, through the C ABI's decay entry points,
against the fp64 oracle on the same seeded inputs.

Stages: the chunk maps (Mc, the reverse map Mr as Mr^T, Jf, Jr) against the
oracle's per-frame maps composed, and the boundary states P, R against the
oracle's scans; tolerances as for the plain stages (relative Frobenius error
per matrix: 1e-4 fp32, 1e-2 bf16).  End to end: the same row-relative bar as
the plain forward (1e-4 fp32, 2e-2 bf16), plus three properties that hold at
any size: gates of one reproduce the plain forward, gates of zero read a zero
state (the bridge product includes the query's own frame), and frames whose
gates are zero cut the forward and reverse memories at that frame.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_helpers import (TOL_OUT, desc_for, gpu_forward, mat_rel_err, oracle_forward,
                         out_to_f64, require_gpu, row_rel_err, say, timed_forward_matches,
                         to_device, to_f64, workspace_for)

pytestmark = pytest.mark.gpu

C = W.custom_config

STAGE_CASES = {
    "d128-decay-bf16": C(cfg_id=401, units=2, frames=12, tokens=200, d_k=128, d_v=128,
                         text_tokens=33, dtype="bf16", alpha_mu=3.0),
    "dk48-dv80-decay-bf16": C(cfg_id=402, units=2, frames=11, tokens=70, d_k=48, d_v=80,
                              text_tokens=6, dtype="bf16", chunk=3, radius=2, alpha_mu=1.0),
    "dk64-dv32-decay-f32": C(cfg_id=403, units=2, frames=9, tokens=50, d_k=64, d_v=32,
                             text_tokens=5, dtype="f32", chunk=2, alpha_mu=2.0),
    "no-video-tokens-decay-bf16": C(cfg_id=404, units=2, frames=7, tokens=0, d_k=32, d_v=48,
                                    text_tokens=9, dtype="bf16", chunk=2, alpha_mu=0.5),
}

PARITY_CASES = {
    "small-decay-bf16": C(cfg_id=411, units=4, frames=40, tokens=256, d_k=64, d_v=64,
                          text_tokens=64, dtype="bf16", alpha_mu=3.0),
    "medium-decay-bf16": C(cfg_id=412, units=2, frames=60, tokens=1024, d_k=128, d_v=128,
                           text_tokens=256, dtype="bf16", alpha_mu=3.0),
    "tiny-decay-f32": C(cfg_id=413, units=1, frames=20, tokens=16, d_k=16, d_v=16,
                        text_tokens=8, dtype="f32", alpha_mu=1.0),
    "partial-chunk-decay-f32": C(cfg_id=414, units=2, frames=13, tokens=20, d_k=32, d_v=48,
                                 text_tokens=3, dtype="f32", alpha_mu=2.0),
    "partial-chunk-decay-bf16": C(cfg_id=415, units=2, frames=7, tokens=48, d_k=64, d_v=64,
                                  text_tokens=9, dtype="bf16", alpha_mu=2.0),
    "one-token-decay": C(cfg_id=416, units=3, frames=15, tokens=1, d_k=128, d_v=128,
                         text_tokens=2, dtype="bf16", alpha_mu=3.0),
    "ragged-tokens-decay": C(cfg_id=417, units=2, frames=10, tokens=1027, d_k=128, d_v=128,
                             text_tokens=100, dtype="bf16", alpha_mu=3.0),
    "dk-ne-dv-decay": C(cfg_id=418, units=2, frames=10, tokens=77, d_k=48, d_v=112,
                        text_tokens=13, dtype="bf16", alpha_mu=1.0),
    "chunk1-radius0-decay": C(cfg_id=419, units=1, frames=6, tokens=32, d_k=32, d_v=32,
                              text_tokens=5, dtype="bf16", chunk=1, radius=0, alpha_mu=1.0),
    "radius-covers-clip-decay": C(cfg_id=420, units=1, frames=10, tokens=32, d_k=32, d_v=32,
                                  text_tokens=5, dtype="bf16", radius=3, alpha_mu=2.0),
    "long-window-decay": C(cfg_id=421, units=1, frames=40, tokens=16, d_k=16, d_v=16,
                           text_tokens=4, dtype="f32", chunk=4, radius=2, alpha_mu=4.0),
    "no-text-decay": C(cfg_id=422, units=2, frames=10, tokens=64, d_k=64, d_v=64,
                       text_tokens=0, dtype="bf16", alpha_mu=1.0),
}


@pytest.fixture(scope="module", params=sorted(STAGE_CASES))
def stage_case(request):
    vda = require_gpu()
    import torch
    name = request.param
    cfg = STAGE_CASES[name]
    h = W.host_inputs(cfg)
    return name, cfg, h, to_device(h, cfg), to_f64(h, cfg), vda, torch


def stage_tol(cfg):
    return 1e-4 if cfg.dtype == "f32" else 1e-2


@pytest.mark.parametrize("seed_mode", [0, 1])
def test_decay_chunks_and_states(stage_case, seed_mode):
    name, cfg, h, d, x, vda, torch = stage_case
    say(f"[decay stages] {name} seed_mode={seed_mode}: chunk maps, boundary states")
    desc = desc_for(cfg, seed_mode)
    ws = workspace_for(desc)
    U, F, dk, dv, Cn = cfg.units, cfg.frames, cfg.d_k, cfg.d_v, cfg.chunk
    n = cfg.n_chunks
    Mc = torch.empty((U, n, dk, dk), device="cuda")
    MrT = torch.empty((U, n, dk, dk), device="cuda")
    Jf = torch.empty((U, n, dv, dk), device="cuda")
    Jr = torch.empty((U, n, dv, dk), device="cuda")
    vda.vda_debug_chunks_decay(desc, d["k"], d["v"], d["beta"], d["alpha"], d["text_k"],
                               d["text_v"], d["text_beta"], Mc, MrT, Jf, Jr, ws)
    P = torch.empty((U, n + 1, dv, dk), device="cuda")
    R = torch.empty((U, n + 1, dv, dk), device="cuda")
    vda.vda_debug_states_decay(desc, d["k"], d["v"], d["beta"], d["alpha"], d["text_k"],
                               d["text_v"], d["text_beta"], P, R, ws)
    torch.cuda.synchronize()
    Mc, MrT, Jf, Jr, P, R = (t.cpu().numpy().astype(np.float64)
                             for t in (Mc, MrT, Jf, Jr, P, R))
    _, tap = oracle_forward(x, cfg, seed_mode, taps=True)
    a = x["alpha"]
    tol = stage_tol(cfg)
    # expected chunk maps: the oracle's per-frame maps S -> (S D_f + B_f) inv_f
    # composed over the chunk (pinned in the oracle suite by
    # pin_decay_chunk_composition); tap["M"] is the decayed transition D_f inv_f
    for u in range(U):
        inv = [oracle.transition(tap["A"][u, f]) for f in range(F)]
        for j in range(n):
            lo, hi = j * Cn, min(j * Cn + Cn, F)
            mc = np.eye(dk)
            jf = np.zeros((dv, dk))
            for f in range(lo, hi):
                mc = mc @ tap["M"][u, f]
                jf = (oracle.decay(jf, a[u, f]) + tap["B"][u, f]) @ inv[f]
            mr = np.eye(dk)
            jr = np.zeros((dv, dk))
            for f in range(hi - 1, lo - 1, -1):
                mr = mr @ tap["M"][u, f]
                jr = (oracle.decay(jr, a[u, f]) + tap["B"][u, f]) @ inv[f]
            assert mat_rel_err(Mc[u, j], mc) <= tol, (u, j)
            assert mat_rel_err(MrT[u, j], mr.T) <= tol, (u, j)
            assert mat_rel_err(Jf[u, j], jf) <= tol, (u, j)
            assert mat_rel_err(Jr[u, j], jr) <= tol, (u, j)
    e_p = mat_rel_err(P, tap["P"])
    e_r = mat_rel_err(R, tap["R"])
    say(f"  P {e_p:.2e}  R {e_r:.2e}")
    assert e_p <= tol and e_r <= tol
    assert np.array_equal(P[:, 0], R[:, n])


def run_case(cfg, seed_mode=0, mutate=None):
    require_gpu()
    h = W.host_inputs(cfg)
    if mutate:
        mutate(h)
    d = to_device(h, cfg)
    got = out_to_f64(gpu_forward(d, cfg, seed_mode), cfg)
    ref = oracle_forward(to_f64(h, cfg), cfg, seed_mode)
    return got, ref


@pytest.mark.parametrize("name", sorted(PARITY_CASES))
@pytest.mark.parametrize("seed_mode", [0, 1])
def test_decay_parity(name, seed_mode):
    cfg = PARITY_CASES[name]
    say(f"[decay parity] {name} seed_mode={seed_mode}")
    got, ref = run_case(cfg, seed_mode)
    err = row_rel_err(got, ref)
    say(f"  max row-rel err {err:.3e} (bar {TOL_OUT[cfg.dtype]:.0e})")
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got))
    assert err <= TOL_OUT[cfg.dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gates_of_one_reproduce_the_plain_forward(dtype):
    """alpha = 1 everywhere: the decay path (its own reverse-transition chain,
    per-frame readout segments) must agree with vda_forward."""
    require_gpu()
    cfg = C(cfg_id=430, units=2, frames=13, tokens=100, d_k=64, d_v=64, text_tokens=9,
            dtype=dtype, alpha_mu=0.0)
    say(f"[decay] alpha = 1 vs plain forward ({dtype})")
    h = W.host_inputs(cfg)
    h["alpha"][:] = 1.0
    d = to_device(h, cfg)
    got = out_to_f64(gpu_forward(d, cfg), cfg)
    plain = dict(d)
    del plain["alpha"]
    ref = out_to_f64(gpu_forward(plain, cfg), cfg)
    err = row_rel_err(got, ref)
    say(f"  max row-rel err {err:.3e}")
    # fp32: both are fp32 paths that differ only in rounding order; bf16: the
    # outputs are rounded to bf16, so allow a few bf16 ulps
    assert err <= (1e-5 if dtype == "f32" else 2e-2)


def test_gates_of_zero_read_a_zero_state():
    """alpha = 0 everywhere: each frame's bridge product includes its own gate,
    so every query reads S~ = 0 and the output is exactly zero."""
    cfg = C(cfg_id=431, units=2, frames=12, tokens=40, d_k=64, d_v=64, text_tokens=9,
            dtype="bf16", alpha_mu=0.0)
    say("[decay] alpha = 0")

    def zero(h):
        h["alpha"][:] = 0.0
    got, ref = run_case(cfg, mutate=zero)
    assert np.all(got == 0.0) and np.all(ref == 0.0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_zero_gate_frame_cuts_the_memories(dtype):
    """Frame g = 14 with all gates zero (chunks of 5, radius 1, no text).
    Entering g, either scan forgets what it carried, and every bridge product
    over a window that holds g is zero on g's side.  So (i) frames 5..9 (window
    0..14: forward seed zero, reverse cut at g) and g itself read a zero state;
    (ii) frames 20..29 read only what frames >= g wrote, bit for bit: redrawing
    the writes of frames 0..13 leaves their outputs unchanged."""
    require_gpu()
    cfg = C(cfg_id=432, units=1, frames=30, tokens=16, d_k=32, d_v=32, text_tokens=0,
            dtype=dtype, alpha_mu=2.0)
    say(f"[decay] a frame of zero gates ({dtype})")
    h = W.host_inputs(cfg)
    h["alpha"][0, 14] = 0.0
    d = to_device(h, cfg)
    got = out_to_f64(gpu_forward(d, cfg), cfg)
    ref = oracle_forward(to_f64(h, cfg), cfg)
    assert row_rel_err(got, ref) <= TOL_OUT[dtype]
    assert np.all(got[0, 5:10] == 0.0) and np.all(got[0, 14] == 0.0)
    assert np.all(np.abs(got[0, 20:]).max(axis=-1) > 0)
    h2 = W.host_inputs(C(cfg_id=433, units=1, frames=30, tokens=16, d_k=32, d_v=32,
                         text_tokens=0, dtype=dtype, alpha_mu=2.0))
    hp = {k: v.copy() for k, v in h.items()}
    for key in ("k", "v", "beta"):
        hp[key][:, :14] = h2[key][:, :14]
    got2 = out_to_f64(gpu_forward(to_device(hp, cfg), cfg), cfg)
    assert np.array_equal(got2[0, 20:], got[0, 20:])
    assert not np.array_equal(got2[0, 10:14], got[0, 10:14])


def test_timed_entry_point_matches_decay():
    require_gpu()
    cfg = PARITY_CASES["small-decay-bf16"]
    say("[decay] vda_forward_timed with gates vs vda_forward_decay")
    assert timed_forward_matches(to_device(W.host_inputs(cfg), cfg), cfg)

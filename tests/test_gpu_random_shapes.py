"""A seeded sweep over random small shapes and options: the HIP path through the
C ABI against the fp64 oracle, end to end, at the usual row-relative bars (1e-4
fp32, 2e-2 bf16).

Each case draws units, frames, tokens per frame, d_k, d_v, text tokens, chunk
length, radius, input dtype, seed mode, write-strength level, clustered keys,
and one of: the frame-wise rule, with decay gates, with boundary anchors, with
both, or the batched comparison rule with frame-size scaling (rule 2).  The
draws come from a fixed generator, so the list of cases is the same on every
run; the shapes are small enough for the oracle to finish each in well under a
second, and they hit what fixed cases tend to miss: d_k != d_v, partial chunks,
chunk lengths 1..7, radii that cover the clip, frames of one token, empty text.

Random shapes also produce rank-deficient gathered states (one text token and a
window that covers the clip leave S~ = S_T of rank one), and for such a state
some queries fall almost into its null space: o = S~ q is then a small
difference of large terms, and no fixed-precision evaluation keeps a relative
error of 1e-4 on it.  The state is fp32 on both paths (the text frame's
statistics are fp32 too), so representing S~ in fp32 alone perturbs o by up to
about u ||S~||_2 ||q|| (u = 2^-24), i.e. by u * kappa relative to ||S~ q||, with
kappa = ||S~||_2 ||q|| / ||S~ q|| the row's condition number (from the
oracle's gathered state).  A row's bar is therefore
    max(tol, min(C_KAPPA * u * kappa, 2e-2)),   C_KAPPA = 4,
the usual bar unless the round-off of fp32 states, amplified by the row's
condition number, is larger; never looser than the bf16 bar.  C_KAPPA leaves
room for the few fp32 roundings the state goes through after the statistics
(solve, composition, scans, readout sum) beyond the single rounding of its
representation.  For every row that gets a relaxed bar the test also forms
o = fl32(S~) q from the oracle's state rounded to fp32 (an fp32 evaluation of
the same product, epilogue in fp64) and logs its error next to the GPU's, and
requires the GPU's worst relaxed-row error to be within C_EVAL = 16 times the
fp32 evaluation's (or within the usual bar).  The fixed-shape tests keep the
plain bar everywhere.
"""
import numpy as np
import pytest

import workloads as W
from gpu_helpers import (TOL_OUT, gpu_forward, oracle_forward, out_to_f64, require_gpu, say,
                         to_device, to_f64)

pytestmark = pytest.mark.gpu

DIMS = (16, 32, 48, 64, 80, 96, 112, 128)
MODES = ("plain", "decay", "anchors", "anchors+decay", "rule2")


def _cases(n=80, seed=2026):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        mode = MODES[i % len(MODES)]
        frames = int(rng.integers(1, 25))
        if "anchors" in mode:
            frames = max(frames, 3)
        tokens = int(rng.choice([1, 2, 7, 16, 33, 64, 100, 257]))
        cfg = W.custom_config(
            cfg_id=900 + i,
            units=int(rng.integers(1, 4)),
            frames=frames,
            tokens=tokens,
            d_k=int(rng.choice(DIMS)),
            d_v=int(rng.choice(DIMS)),
            text_tokens=int(rng.choice([0, 1, 5, 17, 64])),
            dtype=str(rng.choice(["f32", "bf16"])),
            chunk=int(rng.integers(1, 8)),
            radius=int(rng.integers(0, 4)),
            beta_mu=float(rng.choice([-1.0, 0.0, 2.0])),
            stress=bool(rng.random() < 0.2),
            alpha_mu=float(rng.choice([0.5, 2.0, 4.0])) if "decay" in mode else None,
            anchors="anchors" in mode,
            rule=2 if mode == "rule2" else 0,
        )
        cases.append((f"{i:02d}-{mode}-{cfg.dtype}-U{cfg.units}F{cfg.frames}T{cfg.tokens}"
                      f"-dk{cfg.d_k}dv{cfg.d_v}-C{cfg.chunk}r{cfg.radius}-txt{cfg.text_tokens}",
                      cfg, int(rng.integers(0, 2))))
    return cases


CASES = _cases()


def row_condition(x, St):
    """kappa per output row: ||S~||_2 ||q|| / ||S~ q|| (1 where S~ q = 0 exactly
    because S~ = 0 or q = 0: the row must then be exactly zero)."""
    q = x["q"]                                              # units x F x U x d_k
    o = np.einsum("nfvk,nfuk->nfuv", St, q)
    s2 = np.linalg.norm(St, ord=2, axis=(-2, -1))[..., None]  # units x F x 1
    num = s2 * np.linalg.norm(q, axis=-1)
    den = np.linalg.norm(o, axis=-1)
    return np.where(num == 0, 1.0, num / np.where(den == 0, np.inf, den))


U32 = 2.0 ** -24
C_KAPPA = 4.0
C_EVAL = 16.0


def fp32_evaluation(x, St, cfg):
    """out from the oracle's gathered state rounded to fp32, S~ q formed in
    fp32 (q as given to the GPU), RMSNorm and gate in fp64."""
    o = np.einsum("nfvk,nfuk->nfuv", St.astype(np.float32), x["q"].astype(np.float32),
                  dtype=np.float32).astype(np.float64)
    ms = np.mean(o * o, axis=-1, keepdims=True)
    y = x["rms_weight"] * o / np.sqrt(ms + cfg.rms_eps)
    return y / (1.0 + np.exp(-x["gate"]))


@pytest.mark.parametrize("name,cfg,seed_mode", CASES, ids=[c[0] for c in CASES])
def test_random_shape_parity(name, cfg, seed_mode):
    require_gpu()
    say(f"[random shapes] {name} seed_mode={seed_mode}")
    h = W.host_inputs(cfg)
    got = out_to_f64(gpu_forward(to_device(h, cfg), cfg, seed_mode), cfg)
    x = to_f64(h, cfg)
    ref, tap = oracle_forward(x, cfg, seed_mode, taps=True)
    assert got.shape == ref.shape and np.all(np.isfinite(got))
    tol = TOL_OUT[cfg.dtype]
    r = np.abs(ref).max(axis=-1)
    r = np.where(r == 0, 1.0, r)
    err = np.abs(got - ref).max(axis=-1) / r
    kappa = row_condition(x, tap["St"])
    bar = np.maximum(tol, np.minimum(C_KAPPA * U32 * kappa, 2e-2))
    relaxed = bar > tol
    say(f"  max row-rel err {err.max():.3e} (bar {tol:.0e}); max kappa {kappa.max():.3g}; "
        f"rows on a relaxed bar: {int(relaxed.sum())} of {relaxed.size}"
        + (f", their max err / (u kappa) {np.max(err[relaxed] / (U32 * kappa[relaxed])):.3g}"
           if relaxed.any() else ""))
    bad = err > bar
    assert not bad.any(), (f"{bad.sum()} rows over the bar; worst err {err[bad].max():.3e} "
                           f"at kappa {kappa[bad][np.argmax(err[bad])]:.3g}")
    if relaxed.any():
        ev = fp32_evaluation(x, tap["St"], cfg)
        ev_err = np.abs(ev - ref).max(axis=-1) / r
        worst_gpu, worst_ev = err[relaxed].max(), ev_err[relaxed].max()
        say(f"  relaxed rows: GPU worst {worst_gpu:.3e}, fp32 evaluation of S~ q worst "
            f"{worst_ev:.3e}")
        assert worst_gpu <= max(tol, C_EVAL * worst_ev), (worst_gpu, worst_ev)

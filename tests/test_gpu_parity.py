"""vda_forward (HIP path, through the C ABI) against the fp64 oracle.

Bar: max over output rows (unit, frame, token) of ||gpu - oracle||_inf /
||oracle||_inf <= 1e-4 for fp32 features and <= 2e-2 for bf16 features (bf16
in, fp32 accumulation and state, bf16 out).  Every unit and every row is
compared.
"""
import numpy as np
import pytest

import workloads as W
from gpu_helpers import (TOL_OUT, gpu_forward, oracle_forward, out_to_f64, require_gpu,
                         row_rel_err, say, timed_forward_matches, to_device, to_f64)

pytestmark = pytest.mark.gpu

C = W.custom_config
EDGE = {
    # name: config (cfg_id keys the random streams)
    "no-text": C(cfg_id=301, units=2, frames=10, tokens=64, d_k=64, d_v=64, text_tokens=0,
                 dtype="bf16"),
    "one-chunk": C(cfg_id=302, units=2, frames=5, tokens=48, d_k=64, d_v=64, text_tokens=9,
                   dtype="bf16"),
    "partial-chunk": C(cfg_id=303, units=2, frames=7, tokens=48, d_k=64, d_v=64, text_tokens=9,
                       dtype="bf16"),
    "partial-chunk-f32": C(cfg_id=304, units=1, frames=13, tokens=20, d_k=32, d_v=32,
                           text_tokens=3, dtype="f32"),
    "one-token": C(cfg_id=305, units=3, frames=15, tokens=1, d_k=128, d_v=128, text_tokens=2,
                   dtype="bf16"),
    "d16": C(cfg_id=306, units=2, frames=20, tokens=40, d_k=16, d_v=16, text_tokens=4,
             dtype="bf16"),
    "d128-ragged-tokens": C(cfg_id=307, units=2, frames=10, tokens=4032 // 16 + 3, d_k=128,
                            d_v=128, text_tokens=100, dtype="bf16"),
    "dk-ne-dv": C(cfg_id=308, units=2, frames=10, tokens=77, d_k=48, d_v=112, text_tokens=13,
                  dtype="bf16"),
    "dk-ne-dv-f32": C(cfg_id=309, units=2, frames=10, tokens=37, d_k=112, d_v=48,
                      text_tokens=13, dtype="f32"),
    "chunk1-radius0": C(cfg_id=310, units=1, frames=6, tokens=32, d_k=32, d_v=32,
                        text_tokens=5, dtype="bf16", chunk=1, radius=0),
    "radius-covers-clip": C(cfg_id=311, units=1, frames=10, tokens=32, d_k=32, d_v=32,
                            text_tokens=5, dtype="bf16", radius=3),
    "stress-small": C(cfg_id=312, units=2, frames=15, tokens=512, d_k=128, d_v=128,
                      text_tokens=64, dtype="bf16", beta_mu=2.0, stress=True),
    "no-video-tokens": C(cfg_id=314, units=2, frames=7, tokens=0, d_k=64, d_v=64, text_tokens=9,
                         dtype="bf16"),
    "no-tokens-f32": C(cfg_id=315, units=1, frames=4, tokens=0, d_k=16, d_v=16, text_tokens=0,
                       dtype="f32"),
    "eps-zero-f32": C(cfg_id=313, units=1, frames=10, tokens=16, d_k=16, d_v=16, text_tokens=8,
                      dtype="f32", rms_eps=0.0),
    # d_k = d_v = 128 (the scans on the composition's pre-split operand images): a one-frame
    # last chunk, and every chunk one frame
    "d128-one-frame-last-chunk": C(cfg_id=316, units=2, frames=11, tokens=40, d_k=128, d_v=128,
                                   text_tokens=5, dtype="bf16"),
    "d128-chunk1": C(cfg_id=317, units=2, frames=6, tokens=24, d_k=128, d_v=128, text_tokens=3,
                     dtype="bf16", chunk=1, radius=1),
}


def run_case(cfg, seed_mode=0, mutate=None):
    require_gpu()
    h = W.host_inputs(cfg)
    if mutate:
        mutate(h)
    d = to_device(h, cfg)
    got = out_to_f64(gpu_forward(d, cfg, seed_mode), cfg)
    ref = oracle_forward(to_f64(h, cfg), cfg, seed_mode)
    return got, ref


@pytest.mark.parametrize("cfg_id", [1, 2, 3])
@pytest.mark.parametrize("seed_mode", [0, 1])
def test_configs(cfg_id, seed_mode):
    cfg = W.CONFIGS[cfg_id]
    say(f"[parity] {cfg.name} seed_mode={seed_mode}")
    got, ref = run_case(cfg, seed_mode)
    err = row_rel_err(got, ref)
    say(f"  max row-rel err {err:.3e} (bar {TOL_OUT[cfg.dtype]:.0e})")
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got))
    assert err <= TOL_OUT[cfg.dtype]


@pytest.mark.parametrize("name", sorted(EDGE))
@pytest.mark.parametrize("seed_mode", [0, 1])
def test_edge_cases(name, seed_mode):
    cfg = EDGE[name]
    say(f"[parity] edge {name} seed_mode={seed_mode}")
    got, ref = run_case(cfg, seed_mode)
    err = row_rel_err(got, ref)
    say(f"  max row-rel err {err:.3e}")
    assert np.all(np.isfinite(got))
    assert err <= TOL_OUT[cfg.dtype]


def test_all_beta_zero_reads_text_state():
    cfg = C(cfg_id=320, units=2, frames=10, tokens=32, d_k=64, d_v=64, text_tokens=16,
            dtype="bf16")
    say("[parity] all video beta = 0")

    def zero_beta(h):
        h["beta"][:] = 0.0
    got, ref = run_case(cfg, mutate=zero_beta)
    assert row_rel_err(got, ref) <= TOL_OUT["bf16"]


def test_no_text_no_writes_gives_zero():
    cfg = C(cfg_id=321, units=1, frames=10, tokens=32, d_k=32, d_v=32, text_tokens=0,
            dtype="bf16")
    say("[parity] zero state everywhere")

    def zero_beta(h):
        h["beta"][:] = 0.0
    got, ref = run_case(cfg, mutate=zero_beta)
    assert np.all(got == 0.0) and np.all(ref == 0.0)


def test_disjointness_probe():
    """One writing frame, no text: chunks whose window holds that frame read
    exactly zero; all others read it (Sec. 2.2 / Eq. (A.4))."""
    cfg = C(cfg_id=322, units=1, frames=30, tokens=16, d_k=32, d_v=32, text_tokens=0,
            dtype="bf16")
    say("[parity] disjointness probe")
    for fstar in (0, 7, 14, 29):
        def one_frame(h, fstar=fstar):
            b = h["beta"][0, fstar].copy()
            h["beta"][:] = 0.0
            h["beta"][0, fstar] = b
        got, ref = run_case(cfg, mutate=one_frame)
        cs = fstar // cfg.chunk
        for f in range(cfg.frames):
            c = f // cfg.chunk
            zero = (c - cfg.radius <= cs <= c + cfg.radius)
            assert np.all(got[0, f] == 0.0) == zero, (fstar, f)
        assert row_rel_err(got, ref) <= TOL_OUT["bf16"]


def test_time_reversal():
    cfg = C(cfg_id=323, units=2, frames=20, tokens=64, d_k=64, d_v=64, text_tokens=8,
            dtype="f32")
    require_gpu()
    say("[parity] time reversal")
    h = W.host_inputs(cfg)
    hr = dict(h)
    for key in ("q", "k", "v", "beta", "gate"):
        hr[key] = np.ascontiguousarray(h[key][:, ::-1])
    a = out_to_f64(gpu_forward(to_device(h, cfg), cfg), cfg)
    b = out_to_f64(gpu_forward(to_device(hr, cfg), cfg), cfg)
    assert row_rel_err(b[:, ::-1], a) <= 1e-4


def test_token_permutation():
    cfg = C(cfg_id=324, units=1, frames=10, tokens=100, d_k=64, d_v=64, text_tokens=8,
            dtype="bf16")
    require_gpu()
    say("[parity] token permutation")
    h = W.host_inputs(cfg)
    rng = np.random.default_rng(5)
    perm = rng.permutation(cfg.tokens)
    hp = dict(h)
    for key in ("q", "k", "v", "beta", "gate"):
        hp[key] = np.ascontiguousarray(h[key][:, :, perm])
    a = out_to_f64(gpu_forward(to_device(h, cfg), cfg), cfg)
    b = out_to_f64(gpu_forward(to_device(hp, cfg), cfg), cfg)
    assert row_rel_err(b, a[:, :, perm]) <= 2e-2


def test_bitwise_deterministic():
    require_gpu()
    cfg = W.CONFIGS[3]
    say("[parity] determinism medium-bf16")
    d = to_device(W.host_inputs(cfg), cfg)
    a = gpu_forward(d, cfg).clone()
    b = gpu_forward(d, cfg)
    import torch
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_timed_entry_point_matches():
    require_gpu()
    cfg = W.CONFIGS[2]
    say("[parity] vda_forward_timed vs vda_forward")
    assert timed_forward_matches(to_device(W.host_inputs(cfg), cfg), cfg)

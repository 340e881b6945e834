"""The seeded input generators (CPU only)."""
import numpy as np
import pytest

import workloads as W


def test_host_generator_is_deterministic_and_per_unit():
    cfg = W.CONFIGS[2]
    a = W.host_inputs(cfg, units=[1, 3])
    b = W.host_inputs(cfg, units=[3])
    assert np.array_equal(a["k"][1], b["k"][0])
    assert np.array_equal(a["beta"][1], b["beta"][0])
    c = W.host_inputs(cfg, units=[1])
    assert np.array_equal(a["q"][0], c["q"][0])
    assert not np.array_equal(a["q"][0], a["q"][1])


def test_bf16_round_to_nearest_even_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(10000) * 10.0 ** rng.integers(-8, 8, 10000),
                        [0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.0e38, -7.5e-39]])
    ours = W.bf16_bits_from_f64(x)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16)
    assert np.array_equal(ours, ref.numpy().view(np.uint16))
    # ties go to even: 1 + 2^-8 is halfway between 1 and 1 + 2^-7
    assert W.bf16_bits_to_f64(W.bf16_bits_from_f64(np.array([1.0 + 2.0 ** -8])))[0] == 1.0
    assert np.array_equal(W.bf16_bits_to_f64(ours), ref.view(torch.bfloat16).float().numpy())


def test_shapes_dtypes_and_distributions():
    cfg = W.CONFIGS[2]
    h = W.host_inputs(cfg, units=[0])
    F, U, d = cfg.frames, cfg.tokens, cfg.d_k
    assert h["q"].shape == (1, F, U, d) and h["q"].dtype == np.uint16
    assert h["beta"].shape == (1, F, U) and h["beta"].dtype == np.float32
    assert h["text_k"].shape == (1, cfg.text_tokens, d)
    k = W.bf16_bits_to_f64(h["k"])
    nk = np.linalg.norm(k, axis=-1)
    assert np.max(np.abs(nk - 1.0)) < 1e-2  # unit keys up to bf16 rounding
    beta = h["beta"]
    assert 0.0 < beta.min() and beta.max() < 1.0 and abs(beta.mean() - 0.5) < 0.02
    tiny = W.host_inputs(W.CONFIGS[1])
    assert tiny["q"].dtype == np.float32 and tiny["q"].shape == (1, 20, 16, 16)


def test_stress_keys_cluster_near_e1():
    cfg = W.custom_config(cfg_id=55, frames=3, tokens=200, d_k=32, d_v=32, dtype="bf16",
                          beta_mu=2.0, stress=True)
    h = W.host_inputs(cfg, units=[0])
    k = W.bf16_bits_to_f64(h["k"])[0]
    for f in range(3):
        close = np.abs(k[f, :, 0]) > 0.99
        assert close.sum() == round(0.9 * 200)
    # near rank-1 Gram: the top eigenvalue holds most of the trace
    beta = h["beta"][0].astype(np.float64)
    A = k[0].T @ (beta[0][:, None] * k[0])
    ev = np.linalg.eigvalsh(A)
    assert ev[-1] > 0.85 * ev.sum()
    assert beta.mean() > 0.8

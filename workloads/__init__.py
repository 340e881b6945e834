"""Seeded synthetic workloads for Video Delta Attention (VDA) forward.

This module only makes inputs: it holds none of the method's arithmetic.  Both
the fp64 oracle (through the tests and the bench) and the HIP library consume
what it produces; neither side imports the other.

Shapes follow the pages' 768p workload (Video DeltaNet, Sec. 6.1: latents of
48x84 spatial positions, so U = 4032 tokens per latent frame; Sec. 5 and
Sec. 6.4: heads are sharded per GPU), with five concrete sizes:

  tiny-fp32    1 unit,  20 frames, U=16,   d=16,  8 text tokens,   fp32
  small-bf16   4 units, 40 frames, U=256,  d=64,  64 text tokens,  bf16
  medium-bf16  8 units, 60 frames, U=1024, d=128, 256 text tokens, bf16
  768p-bf16    16 units, 90 frames, U=4032, d=128, 512 text tokens, bf16
  stress-bf16  16 units, 75 frames, U=4032, d=128, 512 text tokens, bf16,
               90% of each frame's keys clustered around e_1 (near rank-1 Gram),
               write strengths near 1
  768p-decay-bf16  the 768p workload with per-frame channel-wise decay gates

Custom configs (custom_config) add boundary anchors (anchors=True) or the
batched comparison rules (rule=1, 2) to any shape.  Feature-map workloads
(PrepConfig / PREP_CONFIGS) hold the projection outputs q, k, v in the layout
[batch][frames][height][width][heads][d] and depthwise filters; the 768p one is
the same head share as 2 x 8 heads of 48 x 84 latents.

Recipe (every tensor has its own seeded stream, so any unit can be regenerated
alone):
  q, v, gate logits ~ N(0, 1)
  k: N(0, I_d) rows, L2-normalised ("unit keys")
  beta = sigmoid(N(mu, 1)), mu = 0 (mu = 2 for the stress workload)
  text_k unit keys, text_v ~ N(0, 1), text_beta as beta
  stress keys: round(0.9 U) positions per frame (seeded) get e_1 + 0.01 N(0, I),
  renormalised; the rest are unit keys
  rms weight = 1
  decay gates (only when the config has alpha_mu): alpha = sigmoid(N(alpha_mu, 1))
  per (unit, frame, key channel), fp32 (alpha_mu = 3: mean about 0.95)

Two generators implement that recipe:
  * ``host_inputs``   numpy PCG64, fp64 draws, rounded fp64 -> fp32 -> bf16 with
                      round-to-nearest-even.  Used for the small sizes and every
                      CPU test.
  * ``device_inputs`` torch's device generator, fp32 draws, rounded to bf16 by
                      torch (round-to-nearest-even).  Same distributions; used
                      where host generation of several GB would dominate the run
                      (the two full-size workloads).  Not bit-identical to the
                      host generator; whatever it draws is copied back to the
                      host when the oracle needs it.

bf16 tensors live on the host as ``numpy.uint16`` bit patterns.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = [
    "Config", "CONFIGS", "TENSOR_IDS", "bf16_bits_from_f64", "bf16_bits_to_f64",
    "host_inputs", "device_inputs", "to_f64", "custom_config", "PrepConfig", "PREP_CONFIGS",
    "host_prep_inputs", "device_prep_inputs",
]


@dataclasses.dataclass(frozen=True)
class Config:
    cfg_id: int
    name: str
    units: int
    frames: int
    tokens: int
    d_k: int
    d_v: int
    text_tokens: int
    dtype: str            # "f32" or "bf16" for q, k, v, gate, text_k, text_v, out
    beta_mu: float = 0.0  # beta = sigmoid(N(beta_mu, 1))
    stress: bool = False  # clustered keys
    alpha_mu: float | None = None  # decay gates alpha = sigmoid(N(alpha_mu, 1)); None: no decay
    anchors: bool = False  # boundary anchors: frames 0 and F - 1 out of the linear states
    rule: int = 0  # 0: frame-wise delta rule; 1, 2: batched comparison rules (SANA-WM)
    chunk: int = 5
    radius: int = 1
    rms_eps: float = 1e-6

    @property
    def n_chunks(self) -> int:
        return -(-self.frames // self.chunk) if self.frames > 0 else 0

    @property
    def token_heads(self) -> int:
        return self.units * self.frames * self.tokens


CONFIGS = {
    1: Config(1, "tiny-fp32", 1, 20, 16, 16, 16, 8, "f32"),
    2: Config(2, "small-bf16", 4, 40, 256, 64, 64, 64, "bf16"),
    3: Config(3, "medium-bf16", 8, 60, 1024, 128, 128, 256, "bf16"),
    4: Config(4, "768p-bf16", 16, 90, 4032, 128, 128, 512, "bf16"),
    5: Config(5, "stress-bf16", 16, 75, 4032, 128, 128, 512, "bf16", beta_mu=2.0, stress=True),
    6: Config(6, "768p-decay-bf16", 16, 90, 4032, 128, 128, 512, "bf16", alpha_mu=3.0),
}

# one independent stream per (config, unit, tensor)
TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "beta": 3, "gate": 4,
              "text_k": 5, "text_v": 6, "text_beta": 7, "stress_pos": 8, "alpha": 9,
              "q_raw": 10, "k_raw": 11, "v_raw": 12, "wk_s": 13, "wk_t": 14, "wv_s": 15,
              "wv_t": 16}


# ----------------------------------------------------------------------------- feature map
@dataclasses.dataclass(frozen=True)
class PrepConfig:
    """A feature-map (VDA-Prep) workload: projection outputs q, k, v in the layout
    [batch][frames][height][width][heads][d] and the depthwise filters.

    Recipe: q, k, v ~ N(0, 1); spatial taps ~ U(-1/5, 1/5) and temporal taps
    ~ U(-1/sqrt(5), 1/sqrt(5)) per (head, channel) (bound 1/sqrt(fan-in), the
    usual initial scale of a depthwise convolution: the pages' trained filters
    are not available)."""
    cfg_id: int
    name: str
    batch: int
    heads: int
    frames: int
    height: int
    width: int
    d_k: int
    d_v: int
    dtype: str
    eps: float = 1e-6

    @property
    def units(self) -> int:
        return self.batch * self.heads

    @property
    def tokens(self) -> int:
        return self.height * self.width


PREP_CONFIGS = {
    1: PrepConfig(701, "tiny-prep-f32", 1, 2, 6, 5, 7, 16, 32, "f32"),
    2: PrepConfig(702, "small-prep-bf16", 2, 2, 12, 12, 20, 64, 64, "bf16"),
    # the 768p head share: 48 x 84 latents, 16 heads as 2 x 8, 90 frames
    3: PrepConfig(703, "768p-prep-bf16", 2, 8, 90, 48, 84, 128, 128, "bf16"),
}


def host_prep_inputs(cfg: PrepConfig) -> dict:
    """Feature-map inputs of ``cfg`` as host arrays (features in storage format:
    fp32, or uint16 bf16 bits; filters fp32).  One stream per (config, batch
    index, tensor) for the features, per config for the filters."""
    Bt, F, Hl, Wl, H = cfg.batch, cfg.frames, cfg.height, cfg.width, cfg.heads
    res = {}
    for name, d in (("q", cfg.d_k), ("k", cfg.d_k), ("v", cfg.d_v)):
        x = np.stack([_rng(cfg.cfg_id, b, name + "_raw").standard_normal((F, Hl, Wl, H, d))
                      for b in range(Bt)]) if Bt else np.zeros((0, F, Hl, Wl, H, d))
        res[name] = bf16_bits_from_f64(x) if cfg.dtype == "bf16" else x.astype(np.float32)
    for name, d in (("wk", cfg.d_k), ("wv", cfg.d_v)):
        res[name + "_s"] = _rng(cfg.cfg_id, 0, name + "_s").uniform(
            -0.2, 0.2, (H, d, 5, 5)).astype(np.float32)
        res[name + "_t"] = _rng(cfg.cfg_id, 0, name + "_t").uniform(
            -1 / math.sqrt(5), 1 / math.sqrt(5), (H, d, 5)).astype(np.float32)
    return res


def device_prep_inputs(cfg: PrepConfig, device="cuda", seed: int = 0) -> dict:
    """The same recipe drawn with torch's device generator (full-size runs)."""
    import torch

    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    Bt, F, Hl, Wl, H = cfg.batch, cfg.frames, cfg.height, cfg.width, cfg.heads

    def gen(tensor):
        g = torch.Generator(device=device)
        g.manual_seed(((seed * 131 + cfg.cfg_id) * 1009 + TENSOR_IDS[tensor]) & 0x7FFFFFFFFFFF)
        return g

    res = {}
    for name, d in (("q", cfg.d_k), ("k", cfg.d_k), ("v", cfg.d_v)):
        res[name] = torch.randn((Bt, F, Hl, Wl, H, d), generator=gen(name + "_raw"),
                                device=device, dtype=torch.float32).to(dt)
    for name, d in (("wk", cfg.d_k), ("wv", cfg.d_v)):
        u = torch.rand((H, d, 5, 5), generator=gen(name + "_s"), device=device)
        res[name + "_s"] = (u * 0.4 - 0.2).contiguous()
        u = torch.rand((H, d, 5), generator=gen(name + "_t"), device=device)
        res[name + "_t"] = ((u * 2 - 1) / math.sqrt(5)).contiguous()
    return res


def custom_config(cfg_id=100, **kw) -> Config:
    """A config with explicit sizes (edge cases); cfg_id keys its random streams."""
    base = dict(name=f"custom-{cfg_id}", units=1, frames=5, tokens=16, d_k=16, d_v=16,
                text_tokens=0, dtype="f32")
    base.update(kw)
    return Config(cfg_id=cfg_id, **base)


# ----------------------------------------------------------------------------- bf16 bits
def bf16_bits_from_f64(x: np.ndarray) -> np.ndarray:
    """fp64 -> fp32 -> bf16 (round to nearest, ties to even); returns uint16 bits."""
    f = np.ascontiguousarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """uint16 bf16 bits -> fp64 (exact)."""
    u = np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Host tensor in the config's storage format -> fp64 values."""
    if dtype == "bf16":
        return bf16_bits_to_f64(x)
    return np.asarray(x, dtype=np.float64)


def _rng(cfg_id: int, unit: int, tensor: str) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([0, cfg_id, unit, TENSOR_IDS[tensor]])))


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _unit_rows(x):
    n = np.linalg.norm(x, axis=-1, keepdims=True)
    n[n == 0] = 1.0
    return x / n


def _host_unit(cfg: Config, u: int):
    F, U, T, dk, dv = cfg.frames, cfg.tokens, cfg.text_tokens, cfg.d_k, cfg.d_v
    out = {}
    out["q"] = _rng(cfg.cfg_id, u, "q").standard_normal((F, U, dk))
    k = _unit_rows(_rng(cfg.cfg_id, u, "k").standard_normal((F, U, dk)))
    if cfg.stress and U > 0:
        n_clustered = int(round(0.9 * U))
        prng = _rng(cfg.cfg_id, u, "stress_pos")
        e1 = np.zeros(dk)
        e1[0] = 1.0
        for f in range(F):
            pos = prng.permutation(U)[:n_clustered]
            noise = prng.standard_normal((n_clustered, dk))
            k[f, pos] = _unit_rows(e1[None, :] + 0.01 * noise)
    out["k"] = k
    out["v"] = _rng(cfg.cfg_id, u, "v").standard_normal((F, U, dv))
    out["beta"] = _sigmoid(_rng(cfg.cfg_id, u, "beta").standard_normal((F, U)) + cfg.beta_mu)
    out["gate"] = _rng(cfg.cfg_id, u, "gate").standard_normal((F, U, dv))
    out["text_k"] = _unit_rows(_rng(cfg.cfg_id, u, "text_k").standard_normal((T, dk)))
    out["text_v"] = _rng(cfg.cfg_id, u, "text_v").standard_normal((T, dv))
    out["text_beta"] = _sigmoid(_rng(cfg.cfg_id, u, "text_beta").standard_normal(T) + cfg.beta_mu)
    if cfg.alpha_mu is not None:
        out["alpha"] = _sigmoid(_rng(cfg.cfg_id, u, "alpha").standard_normal((F, dk)) + cfg.alpha_mu)
    return out


def host_inputs(cfg: Config, units=None) -> dict:
    """Inputs of ``cfg`` as host arrays in storage format.

    Returns a dict with q, k, v, gate, text_k, text_v (float32 arrays, or uint16
    bf16 bits when cfg.dtype == "bf16"), beta and text_beta (float32),
    rms_weight (float32, ones) and, for configs with decay, alpha (float32).
    Leading axis is the unit.  ``units`` selects a subset of unit indices
    (default: all).
    """
    units = range(cfg.units) if units is None else list(units)
    per = [_host_unit(cfg, u) for u in units]
    res = {}
    for name in ("q", "k", "v", "gate", "text_k", "text_v"):
        x = np.stack([p[name] for p in per]) if per else np.zeros((0,))
        res[name] = bf16_bits_from_f64(x) if cfg.dtype == "bf16" else x.astype(np.float32)
    for name in ("beta", "text_beta") + (("alpha",) if cfg.alpha_mu is not None else ()):
        x = np.stack([p[name] for p in per]) if per else np.zeros((0,))
        res[name] = x.astype(np.float32)
    res["rms_weight"] = np.ones(cfg.d_v, dtype=np.float32)
    return res


def host_inputs_f64(cfg: Config, units=None) -> dict:
    """host_inputs converted to fp64 values (what the oracle consumes)."""
    h = host_inputs(cfg, units)
    return {k: (to_f64(v, cfg.dtype) if k in ("q", "k", "v", "gate", "text_k", "text_v")
                else v.astype(np.float64)) for k, v in h.items()}


def device_inputs(cfg: Config, device="cuda", seed: int = 0) -> dict:
    """Inputs of ``cfg`` drawn on ``device`` with torch's generator.

    Same recipe as ``host_inputs``; returns torch tensors (bf16 or fp32 for the
    feature tensors, fp32 for beta, text_beta and rms_weight).
    """
    import torch

    F, U, T, dk, dv, N = cfg.frames, cfg.tokens, cfg.text_tokens, cfg.d_k, cfg.d_v, cfg.units
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32

    def gen(tensor):
        g = torch.Generator(device=device)
        g.manual_seed(((seed * 131 + cfg.cfg_id) * 1009 + TENSOR_IDS[tensor]) & 0x7FFFFFFFFFFF)
        return g

    def normal(shape, tensor):
        return torch.randn(shape, generator=gen(tensor), device=device, dtype=torch.float32)

    def unit_rows(x):
        return x / x.norm(dim=-1, keepdim=True).clamp_min(1e-30)

    res = {}
    res["q"] = normal((N, F, U, dk), "q").to(dt)
    k = unit_rows(normal((N, F, U, dk), "k"))
    if cfg.stress and U > 0:
        n_clustered = int(round(0.9 * U))
        scores = torch.rand((N, F, U), generator=gen("stress_pos"), device=device)
        clustered = scores.argsort(dim=-1)[..., :n_clustered]
        noise = normal((N, F, n_clustered, dk), "stress_pos")
        e1 = torch.zeros(dk, device=device)
        e1[0] = 1.0
        ck = unit_rows(e1 + 0.01 * noise)
        k.scatter_(2, clustered[..., None].expand(-1, -1, -1, dk), ck)
    res["k"] = k.to(dt)
    del k
    res["v"] = normal((N, F, U, dv), "v").to(dt)
    res["beta"] = torch.sigmoid(normal((N, F, U), "beta") + cfg.beta_mu).contiguous()
    res["gate"] = normal((N, F, U, dv), "gate").to(dt)
    res["text_k"] = unit_rows(normal((N, T, dk), "text_k")).to(dt)
    res["text_v"] = normal((N, T, dv), "text_v").to(dt)
    res["text_beta"] = torch.sigmoid(normal((N, T), "text_beta") + cfg.beta_mu).contiguous()
    res["rms_weight"] = torch.ones(dv, device=device, dtype=torch.float32)
    if cfg.alpha_mu is not None:
        res["alpha"] = torch.sigmoid(normal((N, F, dk), "alpha") + cfg.alpha_mu).contiguous()
    return res


def tensor_to_host(x) -> np.ndarray:
    """torch tensor (bf16 or fp32, any device) -> host storage format."""
    import torch

    x = x.detach().cpu().contiguous()
    if x.dtype == torch.bfloat16:
        return x.view(torch.int16).numpy().view(np.uint16)
    return x.numpy()


def host_to_tensor(x: np.ndarray, dtype: str, device):
    """Host storage format -> torch tensor on ``device``."""
    import torch

    x = np.ascontiguousarray(x)
    if dtype == "bf16" and x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(x).to(device)


def rms_of(x):
    return math.sqrt(float(np.mean(np.square(x)))) if np.size(x) else 0.0

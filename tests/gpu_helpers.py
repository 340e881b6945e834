"""Shared plumbing of the GPU tests: inputs to the device, calls through the C
ABI, the oracle on the same inputs, and the error metrics."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import workloads as W

FEATURES = ("q", "k", "v", "gate", "text_k", "text_v")


def require_gpu():
    """Skip on a machine without a GPU; on a GPU machine a missing library is an error."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import frame_wise_delta_gram_amd as vda
    vda.load_library()  # raises when libvda.so is missing
    return vda


def say(*a):
    print(*a, flush=True, file=sys.stderr)


def to_device(h: dict, cfg: W.Config, device="cuda") -> dict:
    out = {}
    for name, x in h.items():
        dt = cfg.dtype if name in FEATURES else "f32"
        out[name] = W.host_to_tensor(x, dt, device)
    return out


def to_f64(h: dict, cfg: W.Config) -> dict:
    return {name: (W.to_f64(x, cfg.dtype) if name in FEATURES else np.asarray(x, np.float64))
            for name, x in h.items()}


def device_to_host_f64(d: dict, cfg: W.Config, units=None) -> dict:
    res = {}
    for name, x in d.items():
        if units is not None and name != "rms_weight":
            x = x[list(units)]
        res[name] = W.to_f64(W.tensor_to_host(x), cfg.dtype) if name in FEATURES else \
            W.tensor_to_host(x).astype(np.float64)
    return res


def desc_for(cfg: W.Config, seed_mode=0, fp32_products=0, solver=0):
    import frame_wise_delta_gram_amd as vda
    dt = vda.VDA_DTYPE_BF16 if cfg.dtype == "bf16" else vda.VDA_DTYPE_F32
    return vda.make_desc(cfg.units, cfg.frames, cfg.tokens, cfg.text_tokens, cfg.d_k, cfg.d_v,
                         cfg.chunk, cfg.radius, cfg.rms_eps, seed_mode, dt, int(cfg.anchors),
                         cfg.rule, fp32_products, solver)


def workspace_for(desc):
    import torch
    import frame_wise_delta_gram_amd as vda
    return torch.empty(max(vda.vda_workspace_bytes(desc), 1), dtype=torch.uint8, device="cuda")


def gpu_forward(d: dict, cfg: W.Config, seed_mode=0, ws=None, out=None, fp32_products=0,
                solver=0):
    """vda_forward, or vda_forward_decay when the inputs hold decay gates."""
    import torch
    import frame_wise_delta_gram_amd as vda
    desc = desc_for(cfg, seed_mode, fp32_products, solver)
    ws = workspace_for(desc) if ws is None else ws
    if out is None:
        out = torch.empty((cfg.units, cfg.frames, cfg.tokens, cfg.d_v), device="cuda",
                          dtype=torch.bfloat16 if cfg.dtype == "bf16" else torch.float32)
    if "alpha" in d:
        vda.vda_forward_decay(desc, d["q"], d["k"], d["v"], d["beta"], d["alpha"], d["gate"],
                              d["text_k"], d["text_v"], d["text_beta"], d["rms_weight"], out, ws)
    else:
        vda.vda_forward(desc, d["q"], d["k"], d["v"], d["beta"], d["gate"], d["text_k"],
                        d["text_v"], d["text_beta"], d["rms_weight"], out, ws)
    torch.cuda.synchronize()
    return out


def out_to_f64(out, cfg):
    return W.to_f64(W.tensor_to_host(out), cfg.dtype)


def oracle_forward(x: dict, cfg: W.Config, seed_mode=0, taps=False, units=None):
    import oracle
    return oracle.forward(x["q"], x["k"], x["v"], x["beta"], x["gate"], x["text_k"], x["text_v"],
                          x["text_beta"], x["rms_weight"], chunk=cfg.chunk, radius=cfg.radius,
                          eps=cfg.rms_eps, seed_mode=seed_mode, taps=taps, units=units,
                          alpha=x.get("alpha"), anchors=cfg.anchors, rule=cfg.rule)


def row_rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max over rows of ||got - ref||_inf / ||ref||_inf (rows = last axis)."""
    if ref.size == 0:
        return 0.0
    d = np.abs(got - ref).max(axis=-1)
    r = np.abs(ref).max(axis=-1)
    r = np.where(r == 0, 1.0, r)
    return float((d / r).max())


def mat_rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max over matrices (last two axes) of ||got - ref||_F / ||ref||_F."""
    if ref.size == 0:
        return 0.0
    g = got.reshape(-1, got.shape[-2] * got.shape[-1])
    r = ref.reshape(-1, ref.shape[-2] * ref.shape[-1])
    num = np.linalg.norm(g - r, axis=-1)
    den = np.linalg.norm(r, axis=-1)
    den = np.where(den == 0, 1.0, den)
    return float((num / den).max())


TOL_OUT = {"f32": 1e-4, "bf16": 2e-2}


def timed_forward_matches(d: dict, cfg: W.Config):
    """vda_forward_timed (with decay gates when d holds them) gives bit-identical
    output to the untimed entry point and records six completed events; with
    four of them (two NULL entries) the same output and the four recorded."""
    import ctypes
    import os
    import torch
    import frame_wise_delta_gram_amd as vda
    ref = gpu_forward(d, cfg)
    hip = ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                        ctypes.c_void_p]
    ev = []
    for _ in range(6):
        e = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
        ev.append(e.value)
    try:
        desc = desc_for(cfg)
        ws = workspace_for(desc)
        out = torch.empty_like(ref)
        vda.vda_forward_timed(desc, d["q"], d["k"], d["v"], d["beta"], d.get("alpha"), d["gate"],
                              d["text_k"], d["text_v"], d["text_beta"], d["rms_weight"], out,
                              ws, ev)
        torch.cuda.synchronize()
        total = 0.0
        for i in range(5):
            ms = ctypes.c_float()
            assert hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(ev[i]),
                                           ctypes.c_void_p(ev[i + 1])) == 0
            assert ms.value >= 0.0
            total += ms.value
        assert total > 0.0
        same = lambda x: torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x,
                                     ref.view(torch.int16) if ref.dtype == torch.bfloat16 else ref)
        if not same(out):
            return False
        # NULL entries skip their boundaries; the others are still recorded
        out2 = torch.empty_like(ref)
        part = [ev[0], ev[1], None, None, ev[4], ev[5]]
        vda.vda_forward_timed(desc, d["q"], d["k"], d["v"], d["beta"], d.get("alpha"), d["gate"],
                              d["text_k"], d["text_v"], d["text_beta"], d["rms_weight"], out2,
                              ws, part)
        torch.cuda.synchronize()
        for a, b in ((0, 1), (4, 5)):
            ms = ctypes.c_float()
            assert hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(ev[a]),
                                           ctypes.c_void_p(ev[b])) == 0
            assert ms.value >= 0.0
        return same(out2)
    finally:
        for e in ev:
            hip.hipEventDestroy(ctypes.c_void_p(e))

"""vda_forward_noalloc, the entry point for callers that cannot allocate, through
the C ABI against vda_forward on the same inputs: three calls in a row on one
GPU (a bf16 problem, then a smaller bf16 problem with other channel counts,
then a tiny fp32 one), each bit-identical to vda_forward's output and within
the oracle's bar; its fixed scratch keeps the previous call's contents, so the
smaller calls also show that nothing stale is read."""
import numpy as np
import pytest

import workloads as W
from gpu_helpers import (TOL_OUT, desc_for, gpu_forward, oracle_forward, out_to_f64, require_gpu,
                         row_rel_err, say, to_device, to_f64)

pytestmark = pytest.mark.gpu

CASES = [
    W.custom_config(cfg_id=950, units=3, frames=23, tokens=300, d_k=128, d_v=128,
                    text_tokens=40, dtype="bf16"),
    W.custom_config(cfg_id=951, units=2, frames=9, tokens=37, d_k=64, d_v=48, text_tokens=5,
                    dtype="bf16"),
    W.custom_config(cfg_id=952, units=1, frames=7, tokens=16, d_k=16, d_v=32, text_tokens=3,
                    dtype="f32"),
]


def test_noalloc_matches_forward_on_consecutive_calls():
    vda = require_gpu()
    import torch
    for cfg in CASES:
        desc = desc_for(cfg)
        assert vda.vda_workspace_bytes(desc) <= vda.VDA_NOALLOC_MAX_BYTES
        h = W.host_inputs(cfg)
        d = to_device(h, cfg)
        say(f"[noalloc] {cfg.name}: {cfg.units}x{cfg.frames}x{cfg.tokens} "
            f"d_k={cfg.d_k} d_v={cfg.d_v} {cfg.dtype}")
        ref = gpu_forward(d, cfg)
        out = torch.full_like(ref, float("nan"))  # every row must be written
        vda.vda_forward_noalloc(desc, d["q"], d["k"], d["v"], d["beta"], d["gate"], d["text_k"],
                                d["text_v"], d["text_beta"], d["rms_weight"], out)
        torch.cuda.synchronize()
        bits = torch.int16 if cfg.dtype == "bf16" else torch.int32
        assert torch.equal(out.view(bits), ref.view(bits)), cfg.name
        err = row_rel_err(out_to_f64(out, cfg), oracle_forward(to_f64(h, cfg), cfg))
        say(f"[noalloc] {cfg.name}: bit-identical to vda_forward, row-rel err {err:.3e}")
        assert err <= TOL_OUT[cfg.dtype]


def test_noalloc_refuses_what_its_scratch_cannot_hold():
    vda = require_gpu()
    import torch
    cfg = W.custom_config(cfg_id=953, units=16, frames=90, tokens=8, d_k=128, d_v=128,
                          text_tokens=0, dtype="bf16")
    desc = desc_for(cfg)
    assert vda.vda_workspace_bytes(desc) > vda.VDA_NOALLOC_MAX_BYTES
    d = to_device(W.host_inputs(cfg), cfg)
    out = torch.zeros((cfg.units, cfg.frames, cfg.tokens, cfg.d_v), dtype=torch.bfloat16,
                      device="cuda")
    with pytest.raises(vda.VdaError) as e:
        vda.vda_forward_noalloc(desc, d["q"], d["k"], d["v"], d["beta"], d["gate"], None, None,
                                None, d["rms_weight"], out)
    assert e.value.status == vda.VDA_ERR_SCRATCH_TOO_SMALL
    torch.cuda.synchronize()
    assert not bool(out.view(torch.int16).any())  # nothing was enqueued

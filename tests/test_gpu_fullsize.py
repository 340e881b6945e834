"""The full-size workloads (768p-shaped head share, the ill-conditioned stress
workload and the 768p share with channel-wise decay) in the launch
configuration bench.py times, checked against
the fp64 oracle on whole sampled units (first and last unit: every frame and
every token of those units), plus bitwise run-to-run determinism.
Inputs come from the device generator (workloads.device_inputs); the sampled
units are copied back for the oracle."""
import numpy as np
import pytest

import workloads as W
from gpu_helpers import (TOL_OUT, device_to_host_f64, gpu_forward, oracle_forward, out_to_f64,
                         require_gpu, row_rel_err, say)

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.mark.parametrize("cfg_id", [4, 5, 6])
def test_fullsize_sampled_units(cfg_id):
    require_gpu()
    import torch
    cfg = W.CONFIGS[cfg_id]
    say(f"[fullsize] {cfg.name}: generating inputs")
    d = W.device_inputs(cfg)
    say(f"[fullsize] {cfg.name}: vda_forward")
    out = gpu_forward(d, cfg)
    out2 = gpu_forward(d, cfg)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16)), "not deterministic"
    units = [0, cfg.units - 1]
    got = out_to_f64(out[units], cfg)
    assert np.all(np.isfinite(got))
    say(f"[fullsize] {cfg.name}: oracle on units {units}")
    x = device_to_host_f64(d, cfg, units)
    ref = oracle_forward(x, cfg)
    err = row_rel_err(got, ref)
    say(f"[fullsize] {cfg.name}: max row-rel err {err:.3e}")
    assert err <= TOL_OUT[cfg.dtype]


VARIANTS = {
    "768p-rule2": (4, dict(rule=2), 0),
    "768p-anchors": (4, dict(anchors=True), 0),
    "768p-decay-anchors": (6, dict(anchors=True), 0),
    "768p-seed-mode-1": (4, {}, 1),
}


@pytest.mark.parametrize("name", sorted(VARIANTS))
def test_fullsize_variants(name):
    """The 768p share under the batched rule with frame-size scaling, with
    boundary anchors (with and without decay) and with the text written at
    beta / 2: the same sampled-unit check at full size."""
    require_gpu()
    import dataclasses
    base, kw, seed_mode = VARIANTS[name]
    cfg = dataclasses.replace(W.CONFIGS[base], name=name, **kw)
    say(f"[fullsize] {name}: generating inputs")
    d = W.device_inputs(cfg)
    out = gpu_forward(d, cfg, seed_mode)
    units = [0, cfg.units - 1]
    got = out_to_f64(out[units], cfg)
    assert np.all(np.isfinite(got))
    say(f"[fullsize] {name}: oracle on units {units}")
    ref = oracle_forward(device_to_host_f64(d, cfg, units), cfg, seed_mode)
    err = row_rel_err(got, ref)
    say(f"[fullsize] {name}: max row-rel err {err:.3e}")
    assert err <= TOL_OUT[cfg.dtype]

"""The full-size workloads (768p-shaped head share, the ill-conditioned stress
workload and the 768p share with channel-wise decay) in the launch
configuration bench.py times, checked against the fp64 oracle on every unit
(every frame and every token), plus bitwise run-to-run determinism; the same
whole-workload check for the 768p share under the batched rule, with anchors
(with and without decay), and for the 768p and stress workloads in seed mode 1.
Inputs come from the device generator (workloads.device_inputs); each unit is
copied back and checked on its own, so host memory stays at one unit's fp64
inputs."""
import numpy as np
import pytest

import workloads as W
from gpu_helpers import (TOL_OUT, device_to_host_f64, gpu_forward, oracle_forward, out_to_f64,
                         require_gpu, row_rel_err, say, timed_forward_matches)

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def check_every_unit(d, cfg, out, seed_mode=0):
    """max row-relative error of out against the oracle over all units."""
    worst = 0.0
    for u in range(cfg.units):
        got = out_to_f64(out[u:u + 1], cfg)
        assert np.all(np.isfinite(got)), u
        ref = oracle_forward(device_to_host_f64(d, cfg, [u]), cfg, seed_mode)
        err = row_rel_err(got, ref)
        worst = max(worst, err)
        say(f"  unit {u}: max row-rel err {err:.3e}")
    return worst


@pytest.mark.parametrize("cfg_id", [4, 5, 6])
def test_fullsize_every_unit(cfg_id):
    require_gpu()
    import torch
    cfg = W.CONFIGS[cfg_id]
    say(f"[fullsize] {cfg.name}: generating inputs")
    d = W.device_inputs(cfg)
    say(f"[fullsize] {cfg.name}: vda_forward")
    out = gpu_forward(d, cfg)
    out2 = gpu_forward(d, cfg)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16)), "not deterministic"
    del out2
    # the overlapped schedule (two unit groups) against the stage-by-stage one
    assert timed_forward_matches(d, cfg)
    say(f"[fullsize] {cfg.name}: oracle on all {cfg.units} units")
    err = check_every_unit(d, cfg, out)
    say(f"[fullsize] {cfg.name}: max row-rel err over every unit {err:.3e}")
    assert err <= TOL_OUT[cfg.dtype]


VARIANTS = {
    "768p-rule2": (4, dict(rule=2), 0),
    "768p-anchors": (4, dict(anchors=True), 0),
    "768p-decay-anchors": (6, dict(anchors=True), 0),
    "768p-seed-mode-1": (4, {}, 1),
    "stress-seed-mode-1": (5, {}, 1),
}


@pytest.mark.parametrize("name", sorted(VARIANTS))
def test_fullsize_variants(name):
    """The 768p share under the batched rule with frame-size scaling, with
    boundary anchors (with and without decay), and the 768p and stress
    workloads with the text written at beta / 2: every unit at full size."""
    require_gpu()
    import dataclasses
    base, kw, seed_mode = VARIANTS[name]
    cfg = dataclasses.replace(W.CONFIGS[base], name=name, **kw)
    say(f"[fullsize] {name}: generating inputs")
    d = W.device_inputs(cfg)
    out = gpu_forward(d, cfg, seed_mode)
    say(f"[fullsize] {name}: oracle on all {cfg.units} units")
    err = check_every_unit(d, cfg, out, seed_mode)
    say(f"[fullsize] {name}: max row-rel err over every unit {err:.3e}")
    assert err <= TOL_OUT[cfg.dtype]

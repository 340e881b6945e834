"""The feature map (VDA-Prep: "Video DeltaNet" Sec. 2.3, fused as in Sec. 5) on
the HIP path through vda_prep, against the fp64 oracle (oracle/prep_oracle.py).

Bar: per output row (unit, frame, token) ||gpu - oracle||_inf / ||oracle||_inf
<= 1e-4 for fp32 features and 2e-2 for bf16 (bf16 in, fp32 arithmetic, bf16
out).  Every row of every unit on the small shapes; at the 768p share, whole
units of q' and sampled units of k' and v' over the first and last six frames
(the oracle's clip prefix / suffix gives those frames exactly: an output frame
reads input frames t - 2 .. t + 2).
"""
import dataclasses

import numpy as np
import pytest

import workloads as W
from gpu_helpers import require_gpu, row_rel_err, say

pytestmark = pytest.mark.gpu

P = W.PrepConfig
SHAPES = {
    "tiny-f32": W.PREP_CONFIGS[1],
    "small-bf16": W.PREP_CONFIGS[2],
    "partial-tiles-bf16": P(711, "partial-tiles-bf16", 1, 2, 9, 11, 13, 128, 128, "bf16"),
    "smaller-than-tile-bf16": P(712, "smaller-than-tile-bf16", 2, 1, 4, 3, 5, 32, 48, "bf16"),
    "one-frame-bf16": P(713, "one-frame-bf16", 1, 3, 1, 9, 9, 64, 64, "bf16"),
    "two-frames-f32": P(714, "two-frames-f32", 1, 1, 2, 10, 6, 16, 16, "f32"),
    "dk16-dv128-bf16": P(715, "dk16-dv128-bf16", 2, 2, 6, 8, 16, 16, 128, "bf16"),
    "dk128-f32": P(716, "dk128-f32", 1, 2, 7, 9, 17, 128, 64, "f32"),
    # last tile column 3 wide (a half tile: one output column block) over 6 units,
    # so that the launch's queues reorder full and half tiles across XCD ranges
    "half-tiles-bf16": P(717, "half-tiles-bf16", 2, 3, 5, 9, 19, 64, 32, "bf16"),
}

TOL = {"f32": 1e-4, "bf16": 2e-2}


def _run(cfg, h):
    import torch
    import frame_wise_delta_gram_amd as vda
    dt = vda.VDA_DTYPE_BF16 if cfg.dtype == "bf16" else vda.VDA_DTYPE_F32
    desc = vda.make_prep_desc(cfg.batch, cfg.heads, cfg.frames, cfg.height, cfg.width,
                              cfg.d_k, cfg.d_v, cfg.eps, dt)
    d = {name: (W.host_to_tensor(x, cfg.dtype if name in ("q", "k", "v") else "f32", "cuda")
                if isinstance(x, np.ndarray) else x) for name, x in h.items()}
    tdt = d["q"].dtype
    N, F, Uq = cfg.units, cfg.frames, cfg.tokens
    qo = torch.empty((N, F, Uq, cfg.d_k), dtype=tdt, device="cuda")
    ko = torch.empty_like(qo)
    vo = torch.empty((N, F, Uq, cfg.d_v), dtype=tdt, device="cuda")
    vda.vda_prep(desc, d["q"], d["k"], d["v"], d["wk_s"], d["wk_t"], d["wv_s"], d["wv_t"],
                 qo, ko, vo)
    torch.cuda.synchronize()
    return [W.to_f64(W.tensor_to_host(t), cfg.dtype) for t in (qo, ko, vo)]


def _f64(cfg, h):
    return {k: (W.to_f64(v, cfg.dtype) if k in ("q", "k", "v") else v.astype(np.float64))
            for k, v in h.items()}


@pytest.mark.parametrize("name", sorted(SHAPES))
def test_prep_parity(name):
    require_gpu()
    from oracle import prep_oracle
    cfg = SHAPES[name]
    say(f"[prep parity] {name}")
    h = W.host_prep_inputs(cfg)
    got = _run(cfg, h)
    x = _f64(cfg, h)
    ref = prep_oracle.prep(x["q"], x["k"], x["v"], x["wk_s"], x["wk_t"], x["wv_s"], x["wv_t"],
                           cfg.eps)
    for label, g, r in zip(("q", "k", "v"), got, ref):
        err = row_rel_err(g, r)
        say(f"  {label}' max row-rel err {err:.3e}")
        assert g.shape == r.shape and np.all(np.isfinite(g))
        assert err <= TOL[cfg.dtype], label


def test_prep_zero_rows_stay_zero():
    """An all-zero query row, and a key row whose convolution is zero, are
    normalised to zero (x / max(||x||, eps)), not to NaN."""
    require_gpu()
    cfg = P(720, "zeros-bf16", 1, 2, 5, 6, 6, 64, 64, "bf16")
    say("[prep] zero rows")
    h = W.host_prep_inputs(cfg)
    h["q"][:, 1] = 0
    h["k"][:] = 0
    got = _run(cfg, h)
    assert np.all(got[0][:, 1] == 0) and np.all(np.isfinite(got[0]))
    assert np.all(got[1] == 0)
    # SiLU(0) = 0 for v when the filters are zero
    h = W.host_prep_inputs(cfg)
    h["wv_s"][:] = 0
    got = _run(cfg, h)
    assert np.all(got[2] == 0)


# units of the 768p share checked at full size: every frame of two of them,
# and the first and last frames of one unit in each eighth of the units (the
# convolution's work items run in unit order over the eight XCDs, one eighth
# of the units on each)
FULL_UNITS = (3, 12)
EDGE_UNITS = (0, 4, 7, 8, 11, 15)


def _oracle_blocks(jobs, d, cfg):
    """The prep oracle on frame blocks, in parallel threads (numpy releases the
    GIL in its array loops).  jobs: (unit, lo, hi) output frame ranges; the
    oracle sees input frames [lo - 2, hi + 2) clipped to the clip, which gives
    output frames [lo, hi) exactly (five temporal taps, zero padding only at the
    clip's own borders).  Returns {(unit, lo, hi): (q', k', v') of those frames}."""
    import concurrent.futures
    import os
    from oracle import prep_oracle
    one = dataclasses.replace(cfg, batch=1, heads=1)
    F = cfg.frames
    subs = {}
    for (u, lo, hi) in jobs:
        b, hh = divmod(u, cfg.heads)
        a, z = max(lo - 2, 0), min(hi + 2, F)
        sub = {name: W.tensor_to_host(d[name][b:b + 1, a:z, :, :, hh:hh + 1])
               for name in ("q", "k", "v")}
        for name in ("wk_s", "wk_t", "wv_s", "wv_t"):
            sub[name] = W.tensor_to_host(d[name][hh:hh + 1])
        subs[(u, lo, hi)] = (sub, lo - a, hi - a)

    def run(key):
        sub, s0, s1 = subs[key]
        x = _f64(one, sub)
        ref = prep_oracle.prep(x["q"], x["k"], x["v"], x["wk_s"], x["wk_t"], x["wv_s"],
                               x["wv_t"], cfg.eps)
        return key, tuple(r[0][s0:s1] for r in ref)

    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        return dict(ex.map(run, list(subs)))


@pytest.mark.slow
def test_prep_fullsize():
    """The 768p share (2 x 8 heads, 90 frames of 48 x 84): every frame of units
    FULL_UNITS and the first and last six frames of EDGE_UNITS against the prep
    oracle at the bf16 bar, plus run-to-run determinism."""
    require_gpu()
    import torch
    import frame_wise_delta_gram_amd as vda
    cfg = W.PREP_CONFIGS[3]
    say(f"[prep fullsize] {cfg.name}: generating inputs")
    d = W.device_prep_inputs(cfg)
    desc = vda.make_prep_desc(cfg.batch, cfg.heads, cfg.frames, cfg.height, cfg.width,
                              cfg.d_k, cfg.d_v, cfg.eps, vda.VDA_DTYPE_BF16)
    N, F, Uq = cfg.units, cfg.frames, cfg.tokens
    qo = torch.empty((N, F, Uq, cfg.d_k), dtype=torch.bfloat16, device="cuda")
    ko = torch.empty_like(qo)
    vo = torch.empty((N, F, Uq, cfg.d_v), dtype=torch.bfloat16, device="cuda")
    say("[prep fullsize] vda_prep")
    vda.vda_prep(desc, d["q"], d["k"], d["v"], d["wk_s"], d["wk_t"], d["wv_s"], d["wv_t"],
                 qo, ko, vo)
    torch.cuda.synchronize()
    ko2 = torch.empty_like(ko)
    vo2 = torch.empty_like(vo)
    vda.vda_prep(desc, d["q"], d["k"], d["v"], d["wk_s"], d["wk_t"], d["wv_s"], d["wv_t"],
                 qo, ko2, vo2)
    torch.cuda.synchronize()
    assert torch.equal(ko.view(torch.int16), ko2.view(torch.int16)), "not deterministic"
    assert torch.equal(vo.view(torch.int16), vo2.view(torch.int16)), "not deterministic"
    del ko2, vo2
    jobs = [(u, lo, min(lo + 10, F)) for u in FULL_UNITS for lo in range(0, F, 10)]
    jobs += [(u, lo, hi) for u in EDGE_UNITS for lo, hi in ((0, 6), (F - 6, F))]
    say(f"[prep fullsize] oracle on {len(jobs)} frame blocks")
    refs = _oracle_blocks(jobs, d, cfg)
    worst = {}
    for (u, lo, hi), ref in sorted(refs.items()):
        for label, out, r in (("q", qo, ref[0]), ("k", ko, ref[1]), ("v", vo, ref[2])):
            g = W.to_f64(W.tensor_to_host(out[u, lo:hi]), "bf16")
            err = row_rel_err(g, r)
            worst[(u, label)] = max(worst.get((u, label), 0.0), err)
            assert err <= TOL["bf16"], (u, lo, hi, label, err)
    for u in FULL_UNITS + EDGE_UNITS:
        say(f"  unit {u} ({'every frame' if u in FULL_UNITS else 'frames 0-5, 84-89'}): "
            + ", ".join(f"{lb}' {worst[(u, lb)]:.3e}" for lb in "qkv"))


def _random_prep_shapes(n=24, seed=2027):
    rng = np.random.default_rng(seed)
    dims = (16, 32, 48, 64, 80, 96, 112, 128)
    out = []
    for i in range(n):
        cfg = P(740 + i, f"random-{i}", int(rng.integers(1, 3)), int(rng.integers(1, 4)),
                int(rng.integers(1, 9)), int(rng.integers(1, 20)), int(rng.integers(1, 20)),
                int(rng.choice(dims)), int(rng.choice(dims)), str(rng.choice(["f32", "bf16"])))
        out.append((f"{i:02d}-{cfg.dtype}-B{cfg.batch}H{cfg.heads}F{cfg.frames}"
                    f"-{cfg.height}x{cfg.width}-dk{cfg.d_k}dv{cfg.d_v}", cfg))
    return out


RANDOM = _random_prep_shapes()


@pytest.mark.parametrize("name,cfg", RANDOM, ids=[r[0] for r in RANDOM])
def test_prep_random_shapes(name, cfg):
    """24 shapes from a fixed generator: batch 1-2, heads 1-3, frames 1-8, latent
    grids from 1 x 1 to 19 x 19 (partial 8 x 8 tiles on both axes), d_k and d_v
    independently from 16 to 128, fp32 or bf16; every row at the usual bars."""
    require_gpu()
    from oracle import prep_oracle
    say(f"[prep random] {name}")
    h = W.host_prep_inputs(cfg)
    got = _run(cfg, h)
    x = _f64(cfg, h)
    ref = prep_oracle.prep(x["q"], x["k"], x["v"], x["wk_s"], x["wk_t"], x["wv_s"], x["wv_t"],
                           cfg.eps)
    for label, g, r in zip(("q", "k", "v"), got, ref):
        err = row_rel_err(g, r)
        say(f"  {label}' max row-rel err {err:.3e}")
        assert g.shape == r.shape and np.all(np.isfinite(g))
        assert err <= TOL[cfg.dtype], label


@pytest.mark.parametrize("name", ["small-bf16", "partial-tiles-bf16", "dk128-f32"])
def test_prep_without_query_pass(name):
    """q = q_out = NULL (the query map left to the forward's readout): k' and v'
    are bitwise those of the full call, and nothing is written for q."""
    require_gpu()
    import torch
    import frame_wise_delta_gram_amd as vda
    cfg = SHAPES[name]
    say(f"[prep] {name} without the query pass")
    h = W.host_prep_inputs(cfg)
    dt = vda.VDA_DTYPE_BF16 if cfg.dtype == "bf16" else vda.VDA_DTYPE_F32
    desc = vda.make_prep_desc(cfg.batch, cfg.heads, cfg.frames, cfg.height, cfg.width,
                              cfg.d_k, cfg.d_v, cfg.eps, dt)
    d = {name: (W.host_to_tensor(x, cfg.dtype if name in ("q", "k", "v") else "f32", "cuda")
                if isinstance(x, np.ndarray) else x) for name, x in h.items()}
    tdt = d["q"].dtype
    N, F, Uq = cfg.units, cfg.frames, cfg.tokens
    outs = []
    for with_q in (True, False):
        qo = torch.full((N, F, Uq, cfg.d_k), 7.0, dtype=tdt, device="cuda")
        ko = torch.empty_like(qo)
        vo = torch.empty((N, F, Uq, cfg.d_v), dtype=tdt, device="cuda")
        vda.vda_prep(desc, d["q"] if with_q else None, d["k"], d["v"], d["wk_s"], d["wk_t"],
                     d["wv_s"], d["wv_t"], qo if with_q else None, ko, vo)
        torch.cuda.synchronize()
        outs.append((qo, ko, vo))
    bits = (lambda t: t.view(torch.int16)) if tdt == torch.bfloat16 else (lambda t: t)
    assert torch.equal(bits(outs[0][1]), bits(outs[1][1]))
    assert torch.equal(bits(outs[0][2]), bits(outs[1][2]))
    assert torch.all(outs[1][0] == 7.0)

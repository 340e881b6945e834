"""The feature map's query map inside the readout (descriptor fields q_heads
and q_l2_eps) against the fp64 oracle.

The forward reads raw queries, in the unit layout or in the projection layout
(heads interleaved per token, vda_prep's input order), and L2-normalises each
query row inside its epilogue; the oracle runs the plain forward on the
normalised queries x / max(||x||_2, eps) in the unit layout ("Video
DeltaNet", Sec. 2.3 for the query map, Eq. (1c) for the RMSNorm it folds
into).  Query rows are rescaled by random factors spanning four orders of
magnitude, and a few are set to zero (the floor's case), so that a missing,
misplaced or wrongly scaled normalisation fails.  Every readout kernel is
covered: bf16 with d_k = d_v = 128 (chunk and per-frame images), bf16 at other
shapes (with and without decay), fp32, and boundary anchors.  Bars as in the
plain parity tests; the full-size case checks every unit of the 768p share."""
import dataclasses

import numpy as np
import pytest

import workloads as W
from gpu_helpers import (TOL_OUT, device_to_host_f64, oracle_forward, out_to_f64, require_gpu,
                         row_rel_err, say, to_device, to_f64, workspace_for)

pytestmark = pytest.mark.gpu

C = W.custom_config
EPS_Q = 1e-6
CASES = {
    "c128": C(cfg_id=401, units=4, frames=12, tokens=200, d_k=128, d_v=128, text_tokens=16,
              dtype="bf16"),
    "c128-decay": C(cfg_id=402, units=4, frames=11, tokens=150, d_k=128, d_v=128,
                    text_tokens=16, dtype="bf16", alpha_mu=3.0),
    "c128-anchors": C(cfg_id=403, units=4, frames=13, tokens=96, d_k=128, d_v=128,
                      text_tokens=8, dtype="bf16", anchors=True),
    "bf16-64x48": C(cfg_id=404, units=4, frames=11, tokens=77, d_k=64, d_v=48, text_tokens=9,
                    dtype="bf16"),
    "bf16-48x112-decay": C(cfg_id=405, units=4, frames=9, tokens=65, d_k=48, d_v=112,
                           text_tokens=5, dtype="bf16", alpha_mu=2.0),
    "f32": C(cfg_id=406, units=4, frames=9, tokens=33, d_k=32, d_v=48, text_tokens=4,
             dtype="f32"),
    "f32-decay-anchors": C(cfg_id=407, units=4, frames=10, tokens=21, d_k=64, d_v=32,
                           text_tokens=3, dtype="f32", alpha_mu=2.0, anchors=True),
}


def l2_rows(x, eps):
    """The query map of the feature map's oracle (x / max(||x||_2, eps) per row)."""
    from oracle.prep_oracle import l2_normalize
    return l2_normalize(x, eps)


def rescale_queries(h, cfg, seed):
    """Query rows times exp(N(0, 1.5)) (about 1e-2 .. 1e2), about 2% of them zero;
    rounded back to the storage format, so both sides read the same raw q."""
    rng = np.random.default_rng(seed)
    q = W.to_f64(h["q"], cfg.dtype)
    s = np.exp(rng.normal(0.0, 1.5, size=q.shape[:-1] + (1,)))
    s[rng.random(s.shape) < 0.02] = 0.0
    q = q * s
    h["q"] = W.bf16_bits_from_f64(q) if cfg.dtype == "bf16" else q.astype(np.float32)


def to_projection(q, H):
    """[units][F][U][d] -> [units / H][F][U][H][d] (unit u = b H + h)."""
    units, F, U, d = q.shape
    return np.ascontiguousarray(q.reshape(units // H, H, F, U, d).transpose(0, 2, 3, 1, 4))


def fused_forward(dev, cfg, H, q_dev, eps=EPS_Q):
    import torch
    import frame_wise_delta_gram_amd as vda
    dt = vda.VDA_DTYPE_BF16 if cfg.dtype == "bf16" else vda.VDA_DTYPE_F32
    desc = vda.make_desc(cfg.units, cfg.frames, cfg.tokens, cfg.text_tokens, cfg.d_k, cfg.d_v,
                         cfg.chunk, cfg.radius, cfg.rms_eps, 0, dt, int(cfg.anchors), cfg.rule,
                         q_heads=H, q_l2_eps=eps)
    ws = workspace_for(desc)
    out = torch.empty((cfg.units, cfg.frames, cfg.tokens, cfg.d_v), device="cuda",
                      dtype=torch.bfloat16 if cfg.dtype == "bf16" else torch.float32)
    if "alpha" in dev:
        vda.vda_forward_decay(desc, q_dev, dev["k"], dev["v"], dev["beta"], dev["alpha"],
                              dev["gate"], dev["text_k"], dev["text_v"], dev["text_beta"],
                              dev["rms_weight"], out, ws)
    else:
        vda.vda_forward(desc, q_dev, dev["k"], dev["v"], dev["beta"], dev["gate"],
                        dev["text_k"], dev["text_v"], dev["text_beta"], dev["rms_weight"], out, ws)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("H", [1, 2, 4])
@pytest.mark.parametrize("name", sorted(CASES))
def test_query_map_every_kernel(name, H):
    require_gpu()
    cfg = CASES[name]
    say(f"[query map] {name}, q_heads={H}")
    h = W.host_inputs(cfg)
    rescale_queries(h, cfg, seed=cfg.cfg_id)
    dev = to_device(h, cfg)
    q_dev = W.host_to_tensor(to_projection(h["q"], H) if H > 1 else h["q"], cfg.dtype, "cuda")
    got = out_to_f64(fused_forward(dev, cfg, H, q_dev), cfg)
    x = to_f64(h, cfg)
    x["q"] = l2_rows(x["q"], EPS_Q)
    ref = oracle_forward(x, cfg)
    err = row_rel_err(got, ref)
    say(f"  max row-rel err {err:.3e} (bar {TOL_OUT[cfg.dtype]:.0e})")
    assert np.all(np.isfinite(got))
    assert err <= TOL_OUT[cfg.dtype]


def test_query_map_768p_every_unit():
    """The 768p share (2 entries x 8 heads) with the raw, rescaled queries in
    the projection layout: every unit against the oracle on normalised queries."""
    require_gpu()
    import torch
    cfg = W.CONFIGS[4]
    H = 8
    say("[query map] 768p: generating inputs")
    d = W.device_inputs(cfg)
    g = torch.Generator(device="cuda")
    g.manual_seed(4242)
    s = torch.exp(1.5 * torch.randn(d["q"].shape[:-1] + (1,), generator=g, device="cuda"))
    s = torch.where(torch.rand(s.shape, generator=g, device="cuda") < 0.02, 0.0, s)
    d["q"] = (d["q"].float() * s).to(torch.bfloat16)
    del s
    q_proj = d["q"].view(cfg.units // H, H, cfg.frames, cfg.tokens, cfg.d_k).permute(
        0, 2, 3, 1, 4).contiguous()
    say("[query map] 768p: forward on projection-layout queries")
    out = fused_forward(d, cfg, H, q_proj)
    del q_proj
    worst = 0.0
    for u in range(cfg.units):
        x = device_to_host_f64(d, cfg, [u])
        x["q"] = l2_rows(x["q"], EPS_Q)
        err = row_rel_err(out_to_f64(out[u:u + 1], cfg), oracle_forward(x, cfg))
        worst = max(worst, err)
        say(f"  unit {u}: max row-rel err {err:.3e}")
    assert worst <= TOL_OUT["bf16"]


def test_query_layout_alone_is_bitwise():
    """q_heads alone (no normalisation) only moves where q is read: bitwise the
    same output as the unit layout."""
    require_gpu()
    import torch
    import frame_wise_delta_gram_amd as vda
    cfg = dataclasses.replace(CASES["c128"], cfg_id=408)
    h = W.host_inputs(cfg)
    dev = to_device(h, cfg)
    outs = []
    for H in (1, 4):
        desc = vda.make_desc(cfg.units, cfg.frames, cfg.tokens, cfg.text_tokens, cfg.d_k,
                             cfg.d_v, cfg.chunk, cfg.radius, cfg.rms_eps, 0, vda.VDA_DTYPE_BF16,
                             q_heads=H)
        q = W.host_to_tensor(to_projection(h["q"], H) if H > 1 else h["q"], cfg.dtype, "cuda")
        out = torch.empty((cfg.units, cfg.frames, cfg.tokens, cfg.d_v), device="cuda",
                          dtype=torch.bfloat16)
        vda.vda_forward(desc, q, dev["k"], dev["v"], dev["beta"], dev["gate"], dev["text_k"],
                        dev["text_v"], dev["text_beta"], dev["rms_weight"], out,
                        workspace_for(desc))
        torch.cuda.synchronize()
        outs.append(out)
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))


@pytest.mark.parametrize("prep_id", [1, 2])
def test_feature_map_then_forward(prep_id):
    """The linear branch from projection outputs: vda_prep on k and v alone, then
    vda_forward on the raw projection q (q_heads = heads, q_l2_eps = the feature
    map's eps) and the prepared k', v'; against the two oracles chained
    (prep_oracle.prep, then the forward oracle on its q', k', v')."""
    require_gpu()
    import torch
    import frame_wise_delta_gram_amd as vda
    from oracle.prep_oracle import prep as prep_oracle
    pc = W.PREP_CONFIGS[prep_id]
    cfg = C(cfg_id=410 + prep_id, units=pc.units, frames=pc.frames, tokens=pc.tokens,
            d_k=pc.d_k, d_v=pc.d_v, text_tokens=11, dtype=pc.dtype)
    say(f"[query map] {pc.name}: vda_prep (k, v) then vda_forward (raw q)")
    hp = W.host_prep_inputs(pc)
    h = W.host_inputs(cfg)  # beta, gate, text, weights of the forward
    dp = {n: W.host_to_tensor(x, pc.dtype if n in ("q", "k", "v") else "f32", "cuda")
          for n, x in hp.items()}
    tdt = dp["q"].dtype
    ko = torch.empty((cfg.units, cfg.frames, cfg.tokens, cfg.d_k), dtype=tdt, device="cuda")
    vo = torch.empty((cfg.units, cfg.frames, cfg.tokens, cfg.d_v), dtype=tdt, device="cuda")
    pdesc = vda.make_prep_desc(pc.batch, pc.heads, pc.frames, pc.height, pc.width, pc.d_k,
                               pc.d_v, pc.eps, vda.VDA_DTYPE_BF16 if pc.dtype == "bf16"
                               else vda.VDA_DTYPE_F32)
    vda.vda_prep(pdesc, None, dp["k"], dp["v"], dp["wk_s"], dp["wk_t"], dp["wv_s"], dp["wv_t"],
                 None, ko, vo)
    dev = to_device(h, cfg)
    dev["k"], dev["v"] = ko, vo
    q_proj = dp["q"].view(pc.batch, pc.frames, pc.tokens, pc.heads, pc.d_k)
    out = fused_forward(dev, cfg, pc.heads, q_proj, pc.eps)
    got = out_to_f64(out, cfg)
    f64 = {n: (W.to_f64(x, pc.dtype) if n in ("q", "k", "v") else np.asarray(x, np.float64))
           for n, x in hp.items()}
    q1, k1, v1 = prep_oracle(f64["q"], f64["k"], f64["v"], f64["wk_s"], f64["wk_t"],
                             f64["wv_s"], f64["wv_t"], pc.eps)
    # k' and v' are stored in the features' dtype (vda_prep's output contract),
    # so the chained oracle rounds its own k', v' to that dtype; q' is not
    # stored on the fused path and stays unrounded
    def stored(a):
        return (W.to_f64(W.bf16_bits_from_f64(a), "bf16") if pc.dtype == "bf16"
                else a.astype(np.float32).astype(np.float64))
    x = to_f64(h, cfg)
    x["q"], x["k"], x["v"] = q1, stored(k1), stored(v1)
    ref = oracle_forward(x, cfg)
    err = row_rel_err(got, ref)
    say(f"  max row-rel err {err:.3e} (bar {TOL_OUT[cfg.dtype]:.0e})")
    assert np.all(np.isfinite(got))
    assert err <= TOL_OUT[cfg.dtype]


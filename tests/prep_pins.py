"""Pins of the VDA-Prep oracle (oracle/prep_oracle.py) against what the pages
and the mathematics fix ([VDN] Sec. 2.3: a depthwise 5 x 5 spatial and a
five-tap temporal filter on K and V, SiLU, L2 normalisation of Q and K).

Each ``pin_*`` takes the prep oracle module and raises AssertionError on
disagreement.  The convolution is checked against scipy's n-dimensional
correlation (an independent library routine), against the two 1-D/2-D passes
applied in either order (separability with zero padding), against closed forms
(a delta filter, an all-ones filter on an all-ones clip, a single-voxel input)
and the layout against an index-by-index loop.
"""
from __future__ import annotations

import numpy as np
import scipy.ndimage as ndi


def _rng(seed):
    return np.random.default_rng(seed)


def _filters(rng, ch):
    return rng.standard_normal((ch, 5, 5)), rng.standard_normal((ch, 5))


def pin_prep_scipy(p):
    """The 3-D depthwise correlation equals scipy.ndimage.correlate with the
    outer-product kernel w_t (x) w_s, zero padding (mode='constant')."""
    rng = _rng(1)
    for F, Hl, Wl, ch in ((7, 6, 9, 3), (3, 4, 4, 2), (1, 5, 3, 1), (9, 2, 1, 2)):
        x = rng.standard_normal((F, Hl, Wl, ch))
        ws, wt = _filters(rng, ch)
        y = p.depthwise_conv3d(x, ws, wt)
        for c in range(ch):
            kern = wt[c][:, None, None] * ws[c][None, :, :]
            ref = ndi.correlate(x[..., c], kern, mode="constant", cval=0.0)
            assert np.max(np.abs(y[..., c] - ref)) <= 1e-12, (F, Hl, Wl, c)


def pin_prep_separable(p):
    """Separability with zero padding: the 5 x 5 spatial pass per frame and the
    five-tap temporal pass, in either order, give the 3-D result."""
    rng = _rng(2)
    F, Hl, Wl, ch = 8, 7, 6, 2
    x = rng.standard_normal((F, Hl, Wl, ch))
    ws, wt = _filters(rng, ch)
    y = p.depthwise_conv3d(x, ws, wt)
    for c in range(ch):
        s = np.stack([ndi.correlate(x[t, :, :, c], ws[c], mode="constant") for t in range(F)])
        st = ndi.correlate1d(s, wt[c], axis=0, mode="constant")
        t1 = ndi.correlate1d(x[..., c], wt[c], axis=0, mode="constant")
        ts = np.stack([ndi.correlate(t1[t], ws[c], mode="constant") for t in range(F)])
        assert np.max(np.abs(y[..., c] - st)) <= 1e-12
        assert np.max(np.abs(y[..., c] - ts)) <= 1e-12


def pin_prep_delta_filter(p):
    """Centred delta filters make the convolution the identity."""
    rng = _rng(3)
    x = rng.standard_normal((5, 4, 6, 3))
    ws = np.zeros((3, 5, 5))
    ws[:, 2, 2] = 1.0
    wt = np.zeros((3, 5))
    wt[:, 2] = 1.0
    assert np.array_equal(p.depthwise_conv3d(x, ws, wt), x)


def pin_prep_box_counts(p):
    """All-ones filters on an all-ones clip count the in-clip neighbours:
    y[t, i, j] = n(t, F) n(i, Hl) n(j, Wl), n(i, N) = #{a in -2..2 : 0 <= i + a < N}."""
    F, Hl, Wl = 6, 7, 3
    y = p.depthwise_conv3d(np.ones((F, Hl, Wl, 1)), np.ones((1, 5, 5)), np.ones((1, 5)))

    def cnt(i, N):
        return sum(1 for a in range(-2, 3) if 0 <= i + a < N)
    for t in range(F):
        for i in range(Hl):
            for j in range(Wl):
                assert y[t, i, j, 0] == cnt(t, F) * cnt(i, Hl) * cnt(j, Wl)


def pin_prep_single_voxel(p):
    """Correlation direction: one unit input at (t0, i0, j0) produces
    y[t, i, j] = w_t[t0 - t + 2] w_s[i0 - i + 2, j0 - j + 2] inside the 5 x 5 x 5
    neighbourhood and zero elsewhere."""
    rng = _rng(4)
    F, Hl, Wl = 9, 8, 7
    ws, wt = _filters(rng, 1)
    t0, i0, j0 = 4, 3, 5
    x = np.zeros((F, Hl, Wl, 1))
    x[t0, i0, j0, 0] = 1.0
    y = p.depthwise_conv3d(x, ws, wt)
    for t in range(F):
        for i in range(Hl):
            for j in range(Wl):
                a, b, c = t0 - t + 2, i0 - i + 2, j0 - j + 2
                want = wt[0, a] * ws[0, b, c] if 0 <= a < 5 and 0 <= b < 5 and 0 <= c < 5 else 0.0
                assert abs(y[t, i, j, 0] - want) <= 1e-15, (t, i, j)


def pin_prep_silu_l2(p):
    """SiLU: 0 at 0, x sigma(x) at hand points, silu(x) - silu(-x) = x; the L2
    normalisation gives unit rows, is scale invariant, keeps zero rows zero."""
    xs = np.array([-3.0, -0.5, 0.0, 0.7, 4.0])
    want = xs / (1.0 + np.exp(-xs))
    assert np.max(np.abs(p.silu(xs) - want)) <= 1e-15
    assert np.max(np.abs(p.silu(xs) - p.silu(-xs) - xs)) <= 1e-14
    rng = _rng(5)
    x = rng.standard_normal((6, 8))
    n = p.l2_normalize(x)
    assert np.max(np.abs(np.linalg.norm(n, axis=-1) - 1.0)) <= 1e-14
    assert np.max(np.abs(p.l2_normalize(3.5 * x) - n)) <= 1e-14
    z = np.zeros((2, 8))
    assert np.array_equal(p.l2_normalize(z), z)


def pin_prep_layout(p):
    """to_units: element [b, t, i, j, h, c] lands at [b H + h, t, i Wl + j, c]."""
    Bt, F, Hl, Wl, H, d = 2, 3, 2, 4, 3, 2
    x = np.arange(Bt * F * Hl * Wl * H * d).reshape(Bt, F, Hl, Wl, H, d)
    y = p.to_units(x)
    assert y.shape == (Bt * H, F, Hl * Wl, d)
    for b in range(Bt):
        for t in range(F):
            for i in range(Hl):
                for j in range(Wl):
                    for h in range(H):
                        for c in range(d):
                            assert y[b * H + h, t, i * Wl + j, c] == x[b, t, i, j, h, c]


def pin_prep_pipeline(p):
    """[VDN] Sec. 2.3 end to end on a small clip, rebuilt from scipy's
    correlation: k' = l2(silu(conv(k))), v' = silu(conv(v)), q' = l2(q), per
    (batch, head), in the unit layout."""
    rng = _rng(6)
    Bt, F, Hl, Wl, H, dk, dv = 2, 4, 3, 5, 2, 3, 2
    q = rng.standard_normal((Bt, F, Hl, Wl, H, dk))
    k = rng.standard_normal((Bt, F, Hl, Wl, H, dk))
    v = rng.standard_normal((Bt, F, Hl, Wl, H, dv))
    wk_s, wk_t = rng.standard_normal((H, dk, 5, 5)), rng.standard_normal((H, dk, 5))
    wv_s, wv_t = rng.standard_normal((H, dv, 5, 5)), rng.standard_normal((H, dv, 5))
    qo, ko, vo = p.prep(q, k, v, wk_s, wk_t, wv_s, wv_t)

    def conv(x, ws, wt):
        return ndi.correlate(x, wt[:, None, None] * ws[None], mode="constant")
    for b in range(Bt):
        for h in range(H):
            u = b * H + h
            kc = np.stack([conv(k[b, :, :, :, h, c], wk_s[h, c], wk_t[h, c]) for c in range(dk)],
                          axis=-1).reshape(F, Hl * Wl, dk)
            vc = np.stack([conv(v[b, :, :, :, h, c], wv_s[h, c], wv_t[h, c]) for c in range(dv)],
                          axis=-1).reshape(F, Hl * Wl, dv)
            ks = kc / (1.0 + np.exp(-kc))
            kn = ks / np.linalg.norm(ks, axis=-1, keepdims=True)
            vs = vc / (1.0 + np.exp(-vc))
            qq = q[b, :, :, :, h, :].reshape(F, Hl * Wl, dk)
            qn = qq / np.linalg.norm(qq, axis=-1, keepdims=True)
            assert np.max(np.abs(ko[u] - kn)) <= 1e-12
            assert np.max(np.abs(vo[u] - vs)) <= 1e-12
            assert np.max(np.abs(qo[u] - qn)) <= 1e-12


PREP_PINS = [pin_prep_scipy, pin_prep_separable, pin_prep_delta_filter, pin_prep_box_counts,
             pin_prep_single_voxel, pin_prep_silu_l2, pin_prep_layout, pin_prep_pipeline]

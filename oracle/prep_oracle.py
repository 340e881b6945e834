"""fp64 CPU oracle for the linear branch's feature map (VDA-Prep).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the bench's
CPU-baseline leg may import it; the library never calls it and shares no code
with it.

"Video DeltaNet" (arXiv 2609.20744, cited as [VDN]), Sec. 2.3.  What is
computed: K and V each pass through a short convolution that is separable
into a 5 x 5 spatial filter and a 5-tap temporal filter, both depthwise, and
then through SiLU; Q and the convolved K are then normalised to unit L2 norm.
The linear branch has no rotary embedding.  Sec. 5 ("Fused VDA kernels")
puts this map and the change to the frame-major layout into one kernel.

Readings taken where the pages leave a step open (also listed in the design
notes):
  * input layout: the projection output [batch][F][H_l][W_l][heads][d] (tokens
    in frame, row, column order, heads interleaved); output layout: one unit
    per (batch, head), [batch * heads][F][H_l * W_l][d], the layout the VDA
    forward takes;
  * depthwise: one filter per (head, channel); the two filters combine into
    the 3-D correlation kernel w_t[tau] * w_s[a][b] over (frame, row, column)
    offsets -2..2, centred, with zero padding at the clip's and the frame's
    borders (cross-correlation, as deep-learning convolutions are); no bias;
  * order: convolution, then SiLU, then (K only) L2 normalisation over the d
    channels of one (token, head); Q is only L2-normalised; V gets convolution
    and SiLU;
  * L2 normalisation x / max(||x||_2, eps), eps = 1e-6 by default.
"""
from __future__ import annotations

import numpy as np

__all__ = ["depthwise_conv3d", "silu", "l2_normalize", "to_units", "prep"]

f64 = np.float64


def depthwise_conv3d(x, w_s, w_t):
    """Separable depthwise short convolution of [VDN] Sec. 2.3, written as the
    plain 3-D correlation with the kernel w_t[tau] w_s[a, b]:

      y[t, i, j, c] = sum_{tau, a, b} w_t[c, tau] w_s[c, a, b] x[t + tau - 2, i + a - 2, j + b - 2, c]

    with x = 0 outside the clip.  x: F x Hl x Wl x Ch; w_s: Ch x 5 x 5; w_t: Ch x 5.
    """
    x = np.asarray(x, f64)
    w_s = np.asarray(w_s, f64)
    w_t = np.asarray(w_t, f64)
    F, Hl, Wl, Ch = x.shape
    xp = np.zeros((F + 4, Hl + 4, Wl + 4, Ch))
    xp[2:F + 2, 2:Hl + 2, 2:Wl + 2] = x
    y = np.zeros_like(x)
    for tau in range(5):
        for a in range(5):
            for b in range(5):
                w = w_t[:, tau] * w_s[:, a, b]  # one weight per channel
                y += w * xp[tau:tau + F, a:a + Hl, b:b + Wl]
    return y


def silu(x):
    """SiLU, x * sigmoid(x)."""
    x = np.asarray(x, f64)
    return x / (1.0 + np.exp(-x))


def l2_normalize(x, eps=1e-6):
    """x / max(||x||_2, eps) over the last axis."""
    x = np.asarray(x, f64)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / np.maximum(n, eps)


def to_units(x):
    """[batch][F][Hl][Wl][heads][d] -> [batch * heads][F][Hl * Wl][d]."""
    x = np.asarray(x)
    Bt, F, Hl, Wl, H, d = x.shape
    return x.transpose(0, 4, 1, 2, 3, 5).reshape(Bt * H, F, Hl * Wl, d)


def prep(q, k, v, wk_s, wk_t, wv_s, wv_t, eps=1e-6):
    """The feature map of [VDN] Sec. 2.3 on projection outputs q, k
    ([batch][F][Hl][Wl][heads][d_k]) and v (... [d_v]); filters wk_s
    [heads][d_k][5][5], wk_t [heads][d_k][5] and wv_s, wv_t likewise for v.
    Returns (q', k', v') in the unit layout [batch * heads][F][Hl * Wl][d]."""
    q = np.asarray(q, f64)
    k = np.asarray(k, f64)
    v = np.asarray(v, f64)
    Bt, F, Hl, Wl, H, dk = k.shape
    dv = v.shape[-1]
    kc = np.zeros_like(k)
    vc = np.zeros_like(v)
    for b in range(Bt):
        kc[b] = depthwise_conv3d(k[b].reshape(F, Hl, Wl, H * dk),
                                 np.asarray(wk_s).reshape(H * dk, 5, 5),
                                 np.asarray(wk_t).reshape(H * dk, 5)).reshape(F, Hl, Wl, H, dk)
        vc[b] = depthwise_conv3d(v[b].reshape(F, Hl, Wl, H * dv),
                                 np.asarray(wv_s).reshape(H * dv, 5, 5),
                                 np.asarray(wv_t).reshape(H * dv, 5)).reshape(F, Hl, Wl, H, dv)
    qn = l2_normalize(q, eps)
    kn = l2_normalize(silu(kc), eps)
    vn = silu(vc)
    return to_units(qn), to_units(kn), to_units(vn)

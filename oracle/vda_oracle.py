"""fp64 CPU oracle for the Video Delta Attention (VDA) forward pass.

TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously-correct
statement of what the VDA forward pass computes.  Only the tests, the smoke
check and the bench's CPU-baseline leg may import it; the library never calls it
and shares no code with it.

Every function follows "Video DeltaNet: A Video-Native Hybrid Attention for
Livestream Video Generation" (arXiv 2609.20744), cited below as [VDN] with the
section or equation it restates.  All arithmetic is numpy fp64; a library
routine (matmul, dense solve, inverse) serves as a single step, with no blocking,
fusion or reordering beyond what the cited definition states.

Notation: one "unit" is one (batch, head) pair; all units are independent.
F latent frames of U tokens each; keys k in R^{d_k}, values v in R^{d_v};
states S in R^{d_v x d_k}; chunk length C (5 in [VDN] Sec. 2.1); window radius r
in chunks (1 in [VDN] Sec. 2.1); n = ceil(F / C) chunks; T text tokens.

Readings taken where the pages leave a step open (each is also listed in the
design notes):
  * decay: alpha = 1 by default (no channel-wise decay, no decay bridge).  With
    a per-frame decay alpha_t in [0, 1]^{d_k} ([VDN] Sec. 3.1 Eq. (2)), the
    inherited state is S Diag(alpha_t) in BOTH scans, each frame decaying the
    state it enters with its own gate, and a query of frame t reads the bridged
    boundary states of App. A.3 Eq. (A.4) (the decay products run over the
    window frames up to and including t on each side);
  * no boundary anchors by default: every frame enters both scans.  With
    anchors ([VDN] Sec. 2.1, Sec. 2.2, App. A.3, Algorithm 1 steps 2 and 7),
    frames 0 and F - 1 are excluded from both scans, states are indexed by
    interior frame, windows are clipped to the interior frames, the anchor rows
    get zero output, and a query whose (unclipped) window covers the whole clip
    bypasses the linear path (zero output), as does every row of a clip with no
    interior frame;
  * text seed, mode 0 (default): S_T is ONE frame-wise update from S = 0 over all
    T text tokens (the prompt treated as one extra frame before frame 0, [VDN] Sec. 5) and each
    scan starts at S_T / 2 ([VDN] Eq. (1b)).  Mode 1: the text tokens are written
    from S = 0 at beta / 2 ("written at beta/2" reading);
  * chunk j = frames [C j, min(C j + C, F)); a short last chunk is allowed;
  * the forward state a query in chunk c reads ends before chunk c - r, the
    reverse state starts after chunk c + r (the window's outside, [VDN] Sec. 2.2
    and Eq. (A.4)); a missing side reads the text seed;
  * RMSNorm over the d_v channels of one (unit, frame, token) row with weight
    w in R^{d_v} and epsilon eps, then an element-wise sigmoid gate
    ([VDN] Eq. (1c));
  * comparison rules (rule 1, 2): the frozen-state batched update of SANA-WM,
    S = S_bar (I - A) + B ([VDN] Sec. 3.1 Eq. (3a)/(3c)), replaces Eq. (5)
    everywhere the frame-wise update is used (both scans and the text frame);
    rule 2 adds SANA-WM's frame-size key scaling (every key of a frame of N
    tokens scaled by 1/sqrt(N), [VDN] App. A.2: A -> A / N, B -> B / sqrt(N));
    the text frame is scaled by its own token count T.  Both run with alpha = 1.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "frame_statistics", "frame_update", "batched_update", "scaled_statistics", "update_rule",
    "decay", "transition", "text_state", "chunk_bounds",
    "directional_states", "gather", "window_frames", "bridge", "anchored_states",
    "anchored_state_read", "rms_norm", "sigmoid", "readout", "forward_unit", "forward",
]

f64 = np.float64


def frame_statistics(K, V, beta):
    """Frame statistics, [VDN] Sec. 3.1 Eq. (3b).

    A = sum_u beta_u k_u k_u^T = K^T Diag(beta) K   (d_k x d_k)
    B = sum_u beta_u v_u k_u^T = V^T Diag(beta) K   (d_v x d_k)
    K: U x d_k, V: U x d_v, beta: U (beta >= 0, [VDN] Sec. 3.1).
    """
    K = np.asarray(K, f64)
    V = np.asarray(V, f64)
    beta = np.asarray(beta, f64)
    if np.any(beta < 0):
        raise ValueError("write strengths must be non-negative")
    DK = beta[:, None] * K  # Diag(beta) K: row u of K scaled by beta_u
    A = K.T @ DK
    B = V.T @ DK
    return A, B


def frame_update(S_bar, A, B):
    """Frame-wise delta rule, [VDN] Sec. 3.2 Eq. (5).

    The new state solves the normal equation S (I + A) = S_bar + B; it is
    obtained with a dense solve (no explicit inverse).  S_bar is the inherited
    state (alpha = 1: S_bar = S_{t-1}).
    """
    S_bar = np.asarray(S_bar, f64)
    G = np.eye(A.shape[0]) + A
    # S G = R  <=>  G^T S^T = R^T
    return np.linalg.solve(G.T, (S_bar + B).T).T


def batched_update(S_bar, A, B):
    """Frozen-state batched update of SANA-WM, [VDN] Sec. 3.1 Eq. (3c):
    S = S_bar (I - A) + B, every token correction evaluated at the same S_bar
    (Eq. (3a))."""
    S_bar = np.asarray(S_bar, f64)
    return S_bar @ (np.eye(A.shape[0]) - A) + B


def scaled_statistics(A, B, n_tokens):
    """SANA-WM's frame-size key scaling, [VDN] App. A.2: every key of a frame of
    n_tokens tokens scaled by 1/sqrt(n_tokens), so A -> A / n_tokens and
    B -> B / sqrt(n_tokens) (no change for an empty frame)."""
    if n_tokens == 0:
        return A, B
    return A / n_tokens, B / np.sqrt(n_tokens)


def update_rule(rule):
    """The state update of a rule: 0 the frame-wise delta rule (Eq. (5)), 1 and 2
    the frozen-state batched rule (Eq. (3c); 2 with scaled statistics).  Looked
    up at call time."""
    if rule == 0:
        return frame_update
    if rule in (1, 2):
        return batched_update
    raise ValueError("rule must be 0, 1 or 2")


def decay(S, alpha):
    """Channel-wise decay of an inherited state, [VDN] Sec. 3.1 Eq. (2):
    S_bar = S Diag(alpha) (column j of S, key channel j, scaled by alpha_j)."""
    return np.asarray(S, f64) * np.asarray(alpha, f64)[None, :]


def transition(A, alpha=None):
    """Inherited-state transition, [VDN] App. A.1 Eq. (A.1):
    M = Diag(alpha) (I + A)^{-1}, i.e. (I + A)^{-1} when alpha = 1 (None)."""
    M = np.linalg.inv(np.eye(A.shape[0]) + A)
    if alpha is None:
        return M
    return np.asarray(alpha, f64)[:, None] * M


def text_state(text_k, text_v, text_beta, d_k, d_v, seed_mode=0, rule=0):
    """Initial state of each directional scan, [VDN] Sec. 2.2 Eq. (1b).

    mode 0: S_T = one frame-wise update (Eq. (5)) from S = 0 over all text
            tokens; the seed is S_T / 2, so that the forward and reverse seeds
            together read S_T q exactly once.
    mode 1: the text tokens are written from S = 0 at half write strength.
    No text tokens gives a zero seed.  rule: the update used (update_rule;
    rule 2 scales the text frame's statistics by its token count).
    """
    text_k = np.asarray(text_k, f64).reshape(-1, d_k)
    text_v = np.asarray(text_v, f64).reshape(-1, d_v)
    text_beta = np.asarray(text_beta, f64).reshape(-1)
    zero = np.zeros((d_v, d_k))
    if text_k.shape[0] == 0:
        return zero
    T = text_k.shape[0]
    if seed_mode == 0:
        A, B = frame_statistics(text_k, text_v, text_beta)
        if rule == 2:
            A, B = scaled_statistics(A, B, T)
        return 0.5 * update_rule(rule)(zero, A, B)
    if seed_mode == 1:
        A, B = frame_statistics(text_k, text_v, 0.5 * text_beta)
        if rule == 2:
            A, B = scaled_statistics(A, B, T)
        return update_rule(rule)(zero, A, B)
    raise ValueError("seed_mode must be 0 or 1")


def chunk_bounds(F, C):
    """Chunks of C consecutive latent frames from frame 0 ([VDN] Sec. 2.1); the last may be short."""
    return [(s, min(s + C, F)) for s in range(0, F, C)]


def directional_states(stats, seed, C, alpha=None, update=None):
    """Both directional scans of [VDN] Sec. 2.2 / App. A.3 (no anchors).

    stats: list of (A_f, B_f) for f = 0..F-1; alpha: F x d_k decay gates or None
    (alpha = 1).  Entering frame f, the inherited state is decayed by alpha_f
    (Eq. (2)) and updated by Eq. (5) (or ``update``), in either direction.
    Forward: start at the seed and apply frames 0, 1, ..., F-1;
      P[0] = seed, P[j+1] = the state after the last frame of chunk j.
    Reverse: start at the seed and apply frames F-1, ..., 0;
      R[n] = seed, R[j] = the state after the first frame of chunk j.
    Returns (P, R), each of shape (n + 1, d_v, d_k).
    """
    F = len(stats)
    bounds = chunk_bounds(F, C)
    n = len(bounds)
    P = np.zeros((n + 1,) + seed.shape)
    R = np.zeros((n + 1,) + seed.shape)

    def enter(S, f):
        S_bar = S if alpha is None else decay(S, alpha[f])
        return (update or frame_update)(S_bar, *stats[f])

    S = seed.copy()
    P[0] = S
    for j, (lo, hi) in enumerate(bounds):
        for f in range(lo, hi):
            S = enter(S, f)
        P[j + 1] = S
    S = seed.copy()
    R[n] = S
    for j in range(n - 1, -1, -1):
        lo, hi = bounds[j]
        for f in range(hi - 1, lo - 1, -1):
            S = enter(S, f)
        R[j] = S
    return P, R


def gather(P, R, c, radius):
    """State read by queries of chunk c, [VDN] Eq. (A.4) with alpha = 1 and no anchors.

    The forward state covers the chunks before the window [c - r, c + r], the
    reverse state those after it; an empty side reads the seed (P[0] or R[n]).
    """
    n = P.shape[0] - 1
    return P[max(c - radius, 0)] + R[min(c + radius + 1, n)]


def window_frames(c, C, radius, F):
    """First and last frame of the local window [c - r, c + r] (in chunks) of chunk c,
    clipped to the clip: [l, h] with l = C max(c - r, 0), h = min(C (c + r + 1), F) - 1."""
    return C * max(c - radius, 0), min(C * (c + radius + 1), F) - 1


def bridge(P, R, f, C, radius, alpha):
    """State read by the queries of frame f with decay, [VDN] App. A.3 Eq. (A.4)
    (no anchors):

      P_{l-1} Diag(prod_{s=l}^{f} alpha_s) + R_{h+1} Diag(prod_{s=f}^{h} alpha_s),

    [l, h] the frames of the window of f's chunk (window_frames), P_{l-1} the
    forward state through frame l - 1 (the seed when l = 0), R_{h+1} the reverse
    state from the last frame down to h + 1 (the seed when h = F - 1).  The
    products are channel-wise over the key channels.
    """
    alpha = np.asarray(alpha, f64)
    F = alpha.shape[0]
    n = P.shape[0] - 1
    c = f // C
    lo, hi = window_frames(c, C, radius, F)
    d_f = np.prod(alpha[lo:f + 1], axis=0)
    d_r = np.prod(alpha[f:hi + 1], axis=0)
    return decay(P[max(c - radius, 0)], d_f) + decay(R[min(c + radius + 1, n)], d_r)


def anchored_states(stats, seed, alpha=None, update=None):
    """Both directional scans with boundary anchors, [VDN] Sec. 2.2 and App. A.3.

    stats: list of (A_f, B_f) for f = 0..F-1 (the anchors' entries are never
    read).  Frames 0 and F - 1 are anchors and enter neither scan.  P[j] holds
    what the forward scan has absorbed after the interior frames 1..j (P[0] =
    seed, before any frame); R[j] holds what the reverse scan has absorbed
    after the interior frames F - 2 down to j (R[F - 1] = seed).  Returns dicts
    P (keys 0..F-2) and R (keys 1..F-1); empty for F < 2.
    """
    F = len(stats)
    if F < 2:
        return {}, {}

    def enter(S, f):
        S_bar = S if alpha is None else decay(S, alpha[f])
        return (update or frame_update)(S_bar, *stats[f])

    P = {0: seed.copy()}
    for j in range(1, F - 1):
        P[j] = enter(P[j - 1], j)
    R = {F - 1: seed.copy()}
    for j in range(F - 2, 0, -1):
        R[j] = enter(R[j + 1], j)
    return P, R


def anchored_state_read(P, R, t, C, radius, F, alpha=None):
    """State read by the queries of frame t with anchors, [VDN] App. A.3 Eq. (A.4);
    None where the linear path gives no output (anchor rows, Algorithm 1 step 7;
    a window covering the clip, App. A.3 bypass).

    [l, h] is the window of t's chunk clipped to the interior frames 1..F-2:
      S~ = P[l - 1] Diag(prod_{s=l}^{t} alpha_s) + R[h + 1] Diag(prod_{s=t}^{h} alpha_s)
    (alpha = 1: P[l - 1] + R[h + 1]).
    """
    if t == 0 or t == F - 1:
        return None
    lo, hi = window_frames(t // C, C, radius, F)
    if lo == 0 and hi == F - 1:
        return None
    l, h = max(lo, 1), min(hi, F - 2)
    if alpha is None:
        return P[l - 1] + R[h + 1]
    alpha = np.asarray(alpha, f64)
    return (decay(P[l - 1], np.prod(alpha[l:t + 1], axis=0))
            + decay(R[h + 1], np.prod(alpha[t:h + 1], axis=0)))


def rms_norm(O, w, eps):
    """RMSNorm of each row of O over its d_v channels, scaled by w ([VDN] Eq. (1c))."""
    O = np.asarray(O, f64)
    ms = np.mean(O * O, axis=-1, keepdims=True)
    return np.asarray(w, f64) * O / np.sqrt(ms + eps)


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-np.asarray(x, f64)))


def readout(S_tilde, Q, G, w, eps):
    """Linear-branch readout of [VDN] Eq. (1a), (A.4) and (1c).

    o = S_tilde q for every query row q of Q (tokens x d_k); the output row is
    sigmoid(g) * RMSNorm(o).
    """
    O = np.asarray(Q, f64) @ np.asarray(S_tilde, f64).T
    return sigmoid(G) * rms_norm(O, w, eps)


def forward_unit(q, k, v, beta, gate, text_k, text_v, text_beta, rms_weight,
                 chunk=5, radius=1, eps=1e-6, seed_mode=0, taps=False, alpha=None,
                 anchors=False, rule=0):
    """VDA forward for one unit.

    q: F x U x d_k, k: F x U x d_k, v: F x U x d_v, beta: F x U,
    gate: F x U x d_v (gate logits), text_k: T x d_k, text_v: T x d_v,
    text_beta: T, rms_weight: d_v, alpha: F x d_k decay gates in [0, 1] or None
    (alpha = 1), anchors: boundary anchors (frames 0 and F - 1), rule: 0 the
    frame-wise delta rule, 1 / 2 the batched comparison rules (alpha = 1 only;
    see the module notes).  Returns out
    (F x U x d_v), plus a dict of intermediates when taps=True: A, B (per
    frame; scaled under rule 2), M (per frame: the inherited-state factor,
    Eq. (A.1), or I - A for the batched rules), seed, P, R, and the state St read
    by each frame (F x d_v x d_k; zero where nothing is read).
    With anchors P and R are (F - 1) x d_v x d_k arrays: P[j] after the
    interior frames 1..j (P[0] = seed), R[j - 1] after the interior frames
    F - 2 down to j (R[F - 2] = seed, index F - 1 in App. A.3's numbering).
    """
    q = np.asarray(q, f64)
    k = np.asarray(k, f64)
    v = np.asarray(v, f64)
    beta = np.asarray(beta, f64)
    F, U, d_k = k.shape
    d_v = v.shape[-1]
    if alpha is not None:
        alpha = np.asarray(alpha, f64).reshape(F, d_k)
        if np.any(alpha < 0) or np.any(alpha > 1):
            raise ValueError("decay gates must lie in [0, 1]")
    if rule != 0 and alpha is not None:
        raise ValueError("the batched comparison rules run without decay")
    seed = text_state(text_k, text_v, text_beta, d_k, d_v, seed_mode, rule)
    if anchors:
        return _forward_unit_anchored(q, k, v, beta, gate, rms_weight, seed, chunk, radius,
                                      eps, taps, alpha, rule)
    stats = [_stats(k[f], v[f], beta[f], rule) for f in range(F)]
    P, R = directional_states(stats, seed, chunk, alpha, update_rule(rule))
    out = np.zeros((F, U, d_v))
    St = np.zeros((F, d_v, d_k))
    for c, (lo, hi) in enumerate(chunk_bounds(F, chunk)):
        S_tilde = gather(P, R, c, radius)
        for f in range(lo, hi):
            if alpha is not None:
                S_tilde = bridge(P, R, f, chunk, radius, alpha)
            St[f] = S_tilde
            out[f] = readout(S_tilde, q[f], gate[f], rms_weight, eps)
    if not taps:
        return out
    tap = {
        "A": np.array([s[0] for s in stats]).reshape(F, d_k, d_k),
        "B": np.array([s[1] for s in stats]).reshape(F, d_v, d_k),
        "M": np.array([_factor(stats[f][0], None if alpha is None else alpha[f], rule)
                       for f in range(F)]).reshape(F, d_k, d_k),
        "seed": seed, "P": P, "R": R, "St": St,
    }
    return out, tap


def _stats(K, V, beta, rule):
    """A frame's statistics under a rule (rule 2: scaled by the frame's size)."""
    A, B = frame_statistics(K, V, beta)
    return scaled_statistics(A, B, np.shape(K)[0]) if rule == 2 else (A, B)


def _factor(A, alpha, rule):
    """Inherited-state factor of a frame: Eq. (A.1), or I - A (Eq. (3c))."""
    return transition(A, alpha) if rule == 0 else np.eye(A.shape[0]) - A


def _forward_unit_anchored(q, k, v, beta, gate, rms_weight, seed, chunk, radius, eps, taps,
                           alpha, rule=0):
    """forward_unit with boundary anchors ([VDN] Algorithm 1 steps 2-7): the
    anchor frames' rows are removed from the linear inputs (their statistics
    are never formed), the interior frames are scanned, and each interior,
    non-bypassed query reads anchored_state_read."""
    F, U, d_k = k.shape
    d_v = v.shape[-1]
    stats = [None] * F
    for f in range(1, F - 1):
        stats[f] = _stats(k[f], v[f], beta[f], rule)
    P, R = anchored_states(stats, seed, alpha, update_rule(rule))
    out = np.zeros((F, U, d_v))
    St = np.zeros((F, d_v, d_k))
    for t in range(F):
        S_tilde = anchored_state_read(P, R, t, chunk, radius, F, alpha)
        if S_tilde is None:
            continue  # zero output row
        St[t] = S_tilde
        out[t] = readout(S_tilde, q[t], gate[t], rms_weight, eps)
    if not taps:
        return out
    zero_a, zero_b = np.zeros((d_k, d_k)), np.zeros((d_v, d_k))
    A = np.array([s[0] if s is not None else zero_a for s in stats]).reshape(F, d_k, d_k)
    B = np.array([s[1] if s is not None else zero_b for s in stats]).reshape(F, d_v, d_k)
    Mt = [_factor(A[f], None if alpha is None or stats[f] is None else alpha[f], rule)
          for f in range(F)]
    tap = {"A": A, "B": B, "M": np.array(Mt).reshape(F, d_k, d_k), "seed": seed, "St": St,
           "P": np.array([P[j] for j in range(F - 1)]).reshape(max(F - 1, 0), d_v, d_k),
           "R": np.array([R[j] for j in range(1, F)]).reshape(max(F - 1, 0), d_v, d_k)}
    return out, tap


def forward(q, k, v, beta, gate, text_k, text_v, text_beta, rms_weight,
            chunk=5, radius=1, eps=1e-6, seed_mode=0, taps=False, units=None, alpha=None,
            anchors=False, rule=0):
    """VDA forward over all units (leading axis of every per-unit tensor;
    alpha: units x F x d_k decay gates, or None for alpha = 1; anchors: boundary
    anchors, see forward_unit; rule: the update rule, see forward_unit).

    ``units`` restricts the work to a subset of unit indices; the result then
    holds only those units, in that order.
    """
    idx = range(np.shape(k)[0]) if units is None else list(units)
    outs, tapl = [], []
    for u in idx:
        r = forward_unit(q[u], k[u], v[u], beta[u], gate[u], text_k[u], text_v[u],
                         text_beta[u], rms_weight, chunk, radius, eps, seed_mode, taps,
                         None if alpha is None else alpha[u], anchors, rule)
        if taps:
            outs.append(r[0])
            tapl.append(r[1])
        else:
            outs.append(r)
    out = np.stack(outs) if outs else np.zeros((0,))
    if not taps:
        return out
    merged = {key: np.stack([t[key] for t in tapl]) for key in tapl[0]} if tapl else {}
    return out, merged

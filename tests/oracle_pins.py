"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each ``pin_*`` function takes the oracle module, raises AssertionError when the
oracle disagrees with the fact it checks, and returns nothing otherwise.  The
facts come from "Video DeltaNet" (arXiv 2609.20744), cited as [VDN]:

  * Eq. (3b): the frame statistics are sums of per-token outer products;
  * Eq. (4)-(5): the update is the unique minimiser of a strictly convex
    objective, so its gradient vanishes and an independent least-squares solver
    finds the same state;
  * the classical one-token delta rule ([VDN] Eq. (2)) is the single-key case of
    Eq. (5) with write strength beta / (1 + beta ||k||^2) (Sherman-Morrison);
  * App. A.2 Eq. (A.3): repeated keys get the saturating weight U b / (1 + U b),
    orthogonal keys b / (1 + b) each;
  * Prop. 1 / App. A.1: ||(I + A)^{-1}||_2 <= 1 and state differences never grow;
  * Eq. (1b): the two seeds together read the text state exactly once;
  * Sec. 2.2 and Eq. (A.4): forward and reverse regions are disjoint from the
    local window and from each other;
  * Sec. 3.1 Eq. (2), App. A.1 and A.3: with channel-wise decay the inherited
    state is S Diag(alpha), Prop. 1 still holds, and with no writes the decay
    bridge telescopes to a closed form;
  * Eq. (1c): RMSNorm then an element-wise sigmoid gate;
  * Sec. 2.1, Sec. 2.2, App. A.3 and Algorithm 1: boundary anchors (frames 0 and
    F - 1) are left out of both states, get no linear output, and a window that
    covers the clip bypasses the linear path;
  * Sec. 3.1 Eq. (3a)/(3c) and App. A.2: the frozen-state batched rule of
    SANA-WM is the token-wise correction sum at a shared state, its factor
    I - A stops being non-expansive once an eigenvalue of A passes 2, and the
    frame-size key scaling restores it and assigns the weights A.2 states.

None of these re-types the oracle's own formula: gradients and objectives are
evaluated token by token, least squares goes through numpy's SVD-based solver,
and the scan wiring is checked through symmetries (time reversal, a one-frame
probe) rather than re-implemented.
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _frame(rng, U=7, dk=5, dv=3, unit_keys=False):
    K = rng.standard_normal((U, dk))
    if unit_keys:
        K = _unit(K)
    V = rng.standard_normal((U, dv))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal(U)))
    S_bar = rng.standard_normal((dv, dk))
    return S_bar, K, V, beta


def _update(o, S_bar, K, V, beta):
    A, B = o.frame_statistics(K, V, beta)
    return o.frame_update(S_bar, A, B)


def _objective(S, S_bar, K, V, beta):
    """[VDN] Eq. (4), evaluated token by token."""
    val = 0.5 * np.sum((S - S_bar) ** 2)
    for u in range(K.shape[0]):
        r = S @ K[u] - V[u]
        val += 0.5 * beta[u] * float(r @ r)
    return val


def _gradient(S, S_bar, K, V, beta):
    """Gradient of Eq. (4) w.r.t. S, token by token."""
    G = S - S_bar
    for u in range(K.shape[0]):
        G = G + beta[u] * np.outer(S @ K[u] - V[u], K[u])
    return G


# ----------------------------------------------------------------------------- a2: stats
def pin_stats_hand_loop(o):
    """Eq. (3b) entry by entry with plain Python loops."""
    rng = _rng(1)
    U, dk, dv = 6, 4, 3
    K = rng.standard_normal((U, dk))
    V = rng.standard_normal((U, dv))
    beta = rng.uniform(0, 1, U)
    A, B = o.frame_statistics(K, V, beta)
    assert A.shape == (dk, dk) and B.shape == (dv, dk)
    for i in range(dk):
        for j in range(dk):
            s = 0.0
            for u in range(U):
                s += beta[u] * K[u, i] * K[u, j]
            assert abs(A[i, j] - s) <= 1e-13 * max(1.0, abs(s)), (i, j)
    for i in range(dv):
        for j in range(dk):
            s = 0.0
            for u in range(U):
                s += beta[u] * V[u, i] * K[u, j]
            assert abs(B[i, j] - s) <= 1e-13 * max(1.0, abs(s)), (i, j)


def pin_stats_invariants(o):
    """A is symmetric PSD, tr A = sum_u beta_u ||k_u||^2 ([VDN] App. A.2), and
    standard-basis keys give A = Diag(beta), B = V^T Diag(beta) columns."""
    rng = _rng(2)
    S_bar, K, V, beta = _frame(rng, U=9, dk=6, dv=4)
    A, B = o.frame_statistics(K, V, beta)
    assert np.allclose(A, A.T, atol=1e-14, rtol=0)
    assert np.min(np.linalg.eigvalsh(A)) > -1e-12
    assert abs(np.trace(A) - sum(beta[u] * K[u] @ K[u] for u in range(9))) < 1e-12
    dk = 5
    Ke = np.eye(dk)
    Ve = rng.standard_normal((dk, 3))
    be = rng.uniform(0.1, 1, dk)
    A, B = o.frame_statistics(Ke, Ve, be)
    assert np.allclose(A, np.diag(be), atol=1e-15, rtol=0)
    assert np.allclose(B, (Ve * be[:, None]).T, atol=1e-15, rtol=0)


# ----------------------------------------------------------------------------- a3: update
def pin_gradient_zero(o):
    """Eq. (4)-(5): the update zeroes the gradient of the frame objective."""
    rng = _rng(3)
    for trial in range(5):
        S_bar, K, V, beta = _frame(rng, U=7 + trial, dk=5, dv=3)
        S = _update(o, S_bar, K, V, beta)
        G = _gradient(S, S_bar, K, V, beta)
        A, B = o.frame_statistics(K, V, beta)
        assert np.linalg.norm(G) <= 1e-12 * np.linalg.norm(S_bar + B), trial
        # strictly convex: any perturbation raises the objective
        f0 = _objective(S, S_bar, K, V, beta)
        for _ in range(3):
            D = rng.standard_normal(S.shape) * 1e-3
            assert _objective(S + D, S_bar, K, V, beta) > f0


def pin_lstsq_bruteforce(o):
    """Eq. (4) as stacked least squares per state row, solved by numpy's SVD solver."""
    rng = _rng(4)
    for U, dk, dv in ((1, 3, 2), (5, 4, 4), (16, 16, 16), (3, 8, 2)):
        S_bar, K, V, beta = _frame(rng, U=U, dk=dk, dv=dv)
        S = _update(o, S_bar, K, V, beta)
        sb = np.sqrt(beta)[:, None]
        Mtx = np.vstack([np.eye(dk), sb * K])
        for i in range(dv):
            rhs = np.concatenate([S_bar[i], sb[:, 0] * V[:, i]])
            x = np.linalg.lstsq(Mtx, rhs, rcond=None)[0]
            assert np.max(np.abs(x - S[i])) <= 1e-10 * max(1.0, np.max(np.abs(x))), (U, dk, dv, i)


def pin_sherman_morrison(o):
    """One token: S = S_bar + b' (v - S_bar k) k^T with b' = beta / (1 + beta ||k||^2),
    i.e. the classical delta rule of [VDN] Eq. (2) with an effective strength."""
    rng = _rng(5)
    for trial in range(5):
        dk, dv = 6, 4
        k = rng.standard_normal(dk) * (0.5 + trial)   # not unit on purpose
        v = rng.standard_normal(dv)
        beta = rng.uniform(0.05, 2.0)
        S_bar = rng.standard_normal((dv, dk))
        S = _update(o, S_bar, k[None, :], v[None, :], np.array([beta]))
        bprime = beta / (1.0 + beta * (k @ k))
        expect = S_bar + bprime * np.outer(v - S_bar @ k, k)
        assert np.max(np.abs(S - expect)) <= 1e-12 * max(1.0, np.max(np.abs(expect))), trial


def pin_repeated_keys(o):
    """[VDN] Eq. (A.3): U copies of a unit key k with common beta give
    S k = s / (1 + U beta) + U beta / (1 + U beta) * mean(v); the weight rises
    with U towards, but never reaches, 1."""
    rng = _rng(6)
    dk, dv = 8, 5
    k = _unit(rng.standard_normal(dk))
    S_bar = rng.standard_normal((dv, dk))
    beta = 0.37
    prev = 0.0
    for U in (1, 2, 3, 7, 64, 4032):
        V = rng.standard_normal((U, dv))
        K = np.repeat(k[None, :], U, axis=0)
        S = _update(o, S_bar, K, V, np.full(U, beta))
        w = U * beta / (1.0 + U * beta)
        expect = (S_bar @ k) / (1.0 + U * beta) + w * V.mean(axis=0)
        assert np.max(np.abs(S @ k - expect)) <= 1e-12 * max(1.0, np.max(np.abs(expect))), U
        # directions orthogonal to k keep the inherited state; fp64 rounding of the
        # U-term sum in A leaves O(eps ||A||) off the k direction, ||A|| = U beta
        x = rng.standard_normal(dk)
        x -= (x @ k) * k
        A, B = o.frame_statistics(K, V, np.full(U, beta))
        tol = 1e-14 * dk * (1.0 + U * beta) * max(1.0, np.max(np.abs(S_bar + B)))
        assert np.max(np.abs(S @ x - S_bar @ x)) <= tol, U
        assert prev < w < 1.0
        prev = w


def pin_orthonormal_keys(o):
    """[VDN] App. A.2: orthonormal keys are written independently, each with
    weight beta_u / (1 + beta_u)."""
    rng = _rng(7)
    dk, dv, U = 9, 4, 6
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    K = Qm[:, :U].T
    V = rng.standard_normal((U, dv))
    beta = rng.uniform(0.1, 3.0, U)
    S_bar = rng.standard_normal((dv, dk))
    S = _update(o, S_bar, K, V, beta)
    for u in range(U):
        expect = (S_bar @ K[u] + beta[u] * V[u]) / (1.0 + beta[u])
        assert np.max(np.abs(S @ K[u] - expect)) <= 1e-12, u
    for x in Qm[:, U:].T:
        assert np.max(np.abs(S @ x - S_bar @ x)) <= 1e-12


def pin_beta_zero(o):
    """beta = 0 writes nothing: A = B = 0 and S = S_bar exactly."""
    rng = _rng(8)
    S_bar, K, V, _ = _frame(rng, U=11, dk=6, dv=5)
    S = _update(o, S_bar, K, V, np.zeros(11))
    assert np.array_equal(S, S_bar)


def pin_non_expansive(o):
    """[VDN] Prop. 1 (App. A.1, Eq. (A.2)) with alpha = 1: the transition
    (I + A)^{-1} has spectral norm <= 1, also when lambda_max(A) > 2 (aligned
    keys, App. A.2), and the difference of two entering states never grows."""
    rng = _rng(9)
    for trial in range(4):
        dk, dv, U = 8, 4, 50
        K = _unit(rng.standard_normal((U, dk)))
        if trial % 2:
            K = _unit(np.ones((U, dk)) + 0.05 * rng.standard_normal((U, dk)))
        beta = 1.0 / (1.0 + np.exp(-rng.standard_normal(U)))
        V = rng.standard_normal((U, dv))
        A, B = o.frame_statistics(K, V, beta)
        if trial % 2:
            assert np.max(np.linalg.eigvalsh(A)) > 2.0
        M = o.transition(A)
        ev = np.linalg.eigvalsh((M + M.T) / 2)
        assert np.max(np.abs(M - M.T)) <= 1e-12
        assert 0.0 < np.min(ev) and np.max(ev) <= 1.0 + 1e-12
        assert np.linalg.norm(M, 2) <= 1.0 + 1e-12
        S1 = rng.standard_normal((dv, dk))
        S2 = rng.standard_normal((dv, dk))
        d0 = np.linalg.norm(S1 - S2)
        d1 = np.linalg.norm(o.frame_update(S1, A, B) - o.frame_update(S2, A, B))
        assert d1 <= d0 * (1.0 + 1e-12)
        # the carried contribution is exactly Delta S M (Eq. (A.1))
        D = o.frame_update(S1, A, B) - o.frame_update(S2, A, B)
        assert np.max(np.abs(D - (S1 - S2) @ M)) <= 1e-12


def pin_scalar_case(o):
    """d_k = d_v = 1: Eq. (5) is s_t = (s_{t-1} + b_t) / (1 + a_t); checked against
    the hand-derived fractions in golden/scalar_two_frames.json."""
    with open(os.path.join(GOLDEN, "scalar_two_frames.json")) as fh:
        g = json.load(fh)
    s = np.zeros((1, 1))
    for fr, want in zip(g["frames"], g["states"]):
        K = np.array(fr["k"], float)[:, None]
        V = np.array(fr["v"], float)[:, None]
        beta = np.array([float(Fraction(b)) for b in fr["beta"]])
        A, B = o.frame_statistics(K, V, beta)
        s = o.frame_update(s, A, B)
        assert abs(s[0, 0] - float(Fraction(want))) <= 1e-15, want


def pin_orthonormal_golden(o):
    """golden/orthonormal_d2.json: a 2x2 frame worked by hand (App. A.2)."""
    with open(os.path.join(GOLDEN, "orthonormal_d2.json")) as fh:
        g = json.load(fh)
    fr = lambda m: np.array([[float(Fraction(x)) for x in row] for row in m])  # noqa: E731
    S_bar = fr(g["S_bar"])
    K = fr(g["k"])
    V = fr(g["v"])
    beta = np.array([float(Fraction(b)) for b in g["beta"]])
    S = _update(o, S_bar, K, V, beta)
    assert np.max(np.abs(S - fr(g["S"]))) <= 1e-15


# ----------------------------------------------------------------------------- a1: seed
def pin_exactly_once(o):
    """[VDN] Eq. (1b): P[0] + R[n] equals the text state S_T, found here by
    least squares over the text tokens (mode 0)."""
    rng = _rng(10)
    dk, dv, T = 6, 5, 9
    tk = _unit(rng.standard_normal((T, dk)))
    tv = rng.standard_normal((T, dv))
    tb = rng.uniform(0.1, 1, T)
    F, U = 6, 4
    q = rng.standard_normal((F, U, dk))
    k = _unit(rng.standard_normal((F, U, dk)))
    v = rng.standard_normal((F, U, dv))
    beta = rng.uniform(0, 1, (F, U))
    g = rng.standard_normal((F, U, dv))
    _, tap = o.forward_unit(q, k, v, beta, g, tk, tv, tb, np.ones(dv), chunk=2, radius=1,
                            taps=True)
    sb = np.sqrt(tb)[:, None]
    Mtx = np.vstack([np.eye(dk), sb * tk])
    S_T = np.stack([np.linalg.lstsq(Mtx, np.concatenate([np.zeros(dk), sb[:, 0] * tv[:, i]]),
                                    rcond=None)[0] for i in range(dv)])
    P, R = tap["P"], tap["R"]
    n = P.shape[0] - 1
    assert np.max(np.abs(P[0] + R[n] - S_T)) <= 1e-13
    assert np.max(np.abs(P[0] - R[n])) == 0.0
    # mode 1: the text written from zero at half strength (least squares with beta/2)
    _, tap1 = o.forward_unit(q, k, v, beta, g, tk, tv, tb, np.ones(dv), chunk=2, radius=1,
                             seed_mode=1, taps=True)
    sb = np.sqrt(0.5 * tb)[:, None]
    Mtx = np.vstack([np.eye(dk), sb * tk])
    S_h = np.stack([np.linalg.lstsq(Mtx, np.concatenate([np.zeros(dk), sb[:, 0] * tv[:, i]]),
                                    rcond=None)[0] for i in range(dv)])
    assert np.max(np.abs(tap1["P"][0] - S_h)) <= 1e-13
    # no text tokens: zero seed
    _, tap0 = o.forward_unit(q, k, v, beta, g, tk[:0], tv[:0], tb[:0], np.ones(dv), chunk=2,
                             radius=1, taps=True)
    assert np.array_equal(tap0["P"][0], np.zeros((dv, dk)))


# ----------------------------------------------------------------------------- a4-a6: scans
def _random_unit(rng, F, U, dk, dv, T):
    return dict(
        q=rng.standard_normal((F, U, dk)), k=_unit(rng.standard_normal((F, U, dk))),
        v=rng.standard_normal((F, U, dv)), beta=rng.uniform(0, 1, (F, U)),
        gate=rng.standard_normal((F, U, dv)), text_k=_unit(rng.standard_normal((T, dk))),
        text_v=rng.standard_normal((T, dv)), text_beta=rng.uniform(0, 1, T),
        rms_weight=rng.uniform(0.5, 1.5, dv))


def _call(o, x, **kw):
    return o.forward_unit(x["q"], x["k"], x["v"], x["beta"], x["gate"], x["text_k"],
                          x["text_v"], x["text_beta"], x["rms_weight"], **kw)


def pin_time_reversal(o):
    """[VDN] Sec. 2.2: the two scans are mirror images.  Reversing the frame order
    (F a multiple of C) maps the output of frame f to frame F-1-f."""
    rng = _rng(11)
    for C, r, F in ((5, 1, 20), (2, 1, 8), (3, 2, 15), (1, 1, 6)):
        x = _random_unit(rng, F, 4, 5, 3, 3)
        out = _call(o, x, chunk=C, radius=r)
        xr = dict(x)
        for key in ("q", "k", "v", "beta", "gate"):
            xr[key] = x[key][::-1].copy()
        out_r = _call(o, xr, chunk=C, radius=r)
        assert np.max(np.abs(out_r[::-1] - out)) <= 1e-12, (C, r, F)


def pin_disjointness(o):
    """[VDN] Sec. 2.2 / Eq. (A.4): with a single writing frame f* and no text, a
    query in chunk c sees f* iff chunk(f*) lies outside the window [c-r, c+r];
    otherwise its state and output are exactly zero."""
    rng = _rng(12)
    for C, r, F in ((5, 1, 30), (5, 1, 27), (2, 2, 13), (3, 0, 9)):
        n = -(-F // C)
        for fstar in range(F):
            x = _random_unit(rng, F, 3, 4, 3, 0)
            x["beta"][:] = 0.0
            x["beta"][fstar] = rng.uniform(0.3, 1.0, 3)
            out = _call(o, x, chunk=C, radius=r)
            cs = fstar // C
            for c in range(n):
                frames = range(c * C, min(c * C + C, F))
                seen = not (c - r <= cs <= c + r)
                for f in frames:
                    if seen:
                        assert np.all(np.abs(out[f]).max(axis=-1) > 0), (C, r, F, fstar, c)
                    else:
                        assert np.all(out[f] == 0.0), (C, r, F, fstar, c)


def pin_forward_reverse_regions(o):
    """The forward state read by chunk c depends only on frames before chunk c-r and
    the reverse state only on frames after chunk c+r: changing any other frame's
    inputs leaves P[max(c-r,0)] and R[min(c+r+1,n)] unchanged."""
    rng = _rng(13)
    C, r, F = 3, 1, 14
    n = -(-F // C)
    x = _random_unit(rng, F, 3, 4, 3, 2)
    _, t0 = _call(o, x, chunk=C, radius=r, taps=True)
    for f in range(F):
        y = {key: val.copy() for key, val in x.items()}
        y["v"][f] += 1.0
        _, t1 = _call(o, y, chunk=C, radius=r, taps=True)
        for j in range(n + 1):
            p_dep = f < j * C                 # P[j] covers frames [0, jC)
            r_dep = f >= j * C                # R[j] covers frames [jC, F)
            assert (np.max(np.abs(t1["P"][j] - t0["P"][j])) > 0) == p_dep, (f, j)
            assert (np.max(np.abs(t1["R"][j] - t0["R"][j])) > 0) == r_dep, (f, j)


def pin_chunk_composition(o):
    """[VDN] Sec. 5 and Eq. (A.1): per-frame maps S -> S M_t + J_t compose per
    chunk into one affine map; applying the chunk maps reproduces the per-frame
    scan, and the reverse chunk transition is the transpose of the forward one
    because each M_t is symmetric when alpha = 1."""
    rng = _rng(14)
    F, C, U, dk, dv = 13, 5, 6, 5, 4
    x = _random_unit(rng, F, U, dk, dv, 3)
    _, tap = _call(o, x, chunk=C, radius=1, taps=True)
    n = -(-F // C)
    I = np.eye(dk)
    Ms = [np.linalg.inv(I + tap["A"][f]) for f in range(F)]
    Js = [tap["B"][f] @ Ms[f] for f in range(F)]
    P = [tap["P"][0]]
    R = [None] * (n + 1)
    R[n] = tap["R"][n]
    chunks = [(s, min(s + C, F)) for s in range(0, F, C)]
    maps = []
    for lo, hi in chunks:
        Mf, Jf = I.copy(), np.zeros((dv, dk))
        for f in range(lo, hi):
            Mf, Jf = Mf @ Ms[f], Jf @ Ms[f] + Js[f]
        Mr, Jr = I.copy(), np.zeros((dv, dk))
        for f in range(hi - 1, lo - 1, -1):
            Mr, Jr = Mr @ Ms[f], Jr @ Ms[f] + Js[f]
        assert np.max(np.abs(Mr - Mf.T)) <= 1e-12
        maps.append((Mf, Jf, Mr, Jr))
    for j in range(n):
        P.append(P[j] @ maps[j][0] + maps[j][1])
    for j in range(n - 1, -1, -1):
        R[j] = R[j + 1] @ maps[j][2] + maps[j][3]
    assert np.max(np.abs(np.array(P) - tap["P"])) <= 1e-12
    assert np.max(np.abs(np.array(R) - tap["R"])) <= 1e-12
    # M per frame matches the oracle's tap
    assert np.max(np.abs(np.array(Ms) - tap["M"])) <= 1e-12


def pin_golden_scan(o):
    """golden/scan_scalar.json: d_k = d_v = 1, chunk 1, radius 1, four frames and one
    text token, worked by hand (states P, R and the gathered states)."""
    with open(os.path.join(GOLDEN, "scan_scalar.json")) as fh:
        g = json.load(fh)
    fr = lambda xs: np.array([float(Fraction(v)) for v in xs])  # noqa: E731
    F = len(g["beta"])
    k = np.ones((F, 1, 1))
    v = fr(g["v"]).reshape(F, 1, 1)
    beta = fr(g["beta"]).reshape(F, 1)
    q = np.ones((F, 1, 1))
    gate = np.zeros((F, 1, 1))
    _, tap = o.forward_unit(q, k, v, beta, gate, np.ones((1, 1)), fr(g["text_v"]).reshape(1, 1),
                            fr(g["text_beta"]), np.ones(1), chunk=1, radius=1, taps=True)
    assert np.max(np.abs(tap["seed"].ravel() - float(Fraction(g["seed"])))) <= 1e-15
    assert np.max(np.abs(tap["P"].ravel() - fr(g["P"]))) <= 1e-15
    assert np.max(np.abs(tap["R"].ravel() - fr(g["R"]))) <= 1e-15
    for c, want in enumerate(g["gathered"]):
        St = o.gather(tap["P"], tap["R"], c, 1)
        assert abs(St[0, 0] - float(Fraction(want))) <= 1e-15, c


def pin_token_permutation(o):
    """Frame-wise writes have no token order ([VDN] Sec. 3.1): permuting the tokens
    of every frame permutes the output rows and leaves every state unchanged."""
    rng = _rng(15)
    F, U = 10, 8
    x = _random_unit(rng, F, U, 5, 4, 3)
    out, t0 = _call(o, x, chunk=5, radius=1, taps=True)
    y = {key: val.copy() for key, val in x.items()}
    perms = [rng.permutation(U) for _ in range(F)]
    for f in range(F):
        for key in ("q", "k", "v", "beta", "gate"):
            y[key][f] = x[key][f][perms[f]]
    out2, t1 = _call(o, y, chunk=5, radius=1, taps=True)
    assert np.max(np.abs(t1["P"] - t0["P"])) <= 1e-12
    assert np.max(np.abs(t1["R"] - t0["R"])) <= 1e-12
    for f in range(F):
        assert np.max(np.abs(out2[f] - out[f][perms[f]])) <= 1e-12


def pin_all_beta_zero(o):
    """No video writes: every state stays the seed exactly, so every chunk reads
    seed + seed = S_T (Eq. (1b)); equal query rows in different chunks give
    equal outputs."""
    rng = _rng(16)
    F, U, dk, dv = 12, 5, 4, 6
    x = _random_unit(rng, F, U, dk, dv, 4)
    x["beta"][:] = 0.0
    x["q"][:] = x["q"][0]
    x["gate"][:] = x["gate"][0]
    out, tap = _call(o, x, chunk=5, radius=1, taps=True)
    for j in range(tap["P"].shape[0]):
        assert np.array_equal(tap["P"][j], tap["seed"])
        assert np.array_equal(tap["R"][j], tap["seed"])
    for f in range(1, F):
        assert np.max(np.abs(out[f] - out[0])) <= 1e-14


# ----------------------------------------------------------------------------- a7: epilogue
def pin_rmsnorm_gate(o):
    """Eq. (1c): RMSNorm makes each row's mean square ms/(ms + eps) (~1), is
    invariant to rescaling the row (exactly with eps = 0), and sigmoid(0) = 1/2."""
    rng = _rng(17)
    Oq = rng.standard_normal((7, 12)) * 3.0
    w = np.ones(12)
    y = o.rms_norm(Oq, w, 0.0)
    assert np.max(np.abs(np.mean(y * y, axis=-1) - 1.0)) <= 1e-13
    assert np.max(np.abs(o.rms_norm(5.5 * Oq, w, 0.0) - y)) <= 1e-13
    ye = o.rms_norm(Oq, w, 1e-6)
    ms = np.mean(Oq * Oq, axis=-1)
    assert np.max(np.abs(np.mean(ye * ye, axis=-1) - ms / (ms + 1e-6))) <= 1e-13
    w2 = rng.uniform(0.5, 2.0, 12)
    assert np.max(np.abs(o.rms_norm(Oq, w2, 0.0) - w2 * y)) <= 1e-13
    assert abs(o.sigmoid(0.0) - 0.5) == 0.0
    assert abs(o.sigmoid(np.log(3.0)) - 0.75) <= 1e-15
    # readout: o = S q (hand loop); a saturated gate (sigmoid(40) == 1 in fp64)
    # leaves the normalised o, a zero gate halves it.  A square, non-symmetric
    # state makes a transposed operand visible.
    for dv, dk in ((12, 5), (6, 6)):
        S = rng.standard_normal((dv, dk))
        Q = rng.standard_normal((7, dk))
        O = np.zeros((7, dv))
        for t in range(7):
            for i in range(dv):
                O[t, i] = sum(S[i, kk] * Q[t, kk] for kk in range(dk))
        full = o.readout(S, Q, np.full((7, dv), 40.0), np.ones(dv), 0.0)
        assert np.max(np.abs(np.mean(full * full, axis=-1) - 1.0)) <= 1e-13
        for t in range(7):
            cos = full[t] @ O[t] / (np.linalg.norm(full[t]) * np.linalg.norm(O[t]))
            assert abs(cos - 1.0) <= 1e-13
        half = o.readout(S, Q, np.zeros((7, dv)), np.ones(dv), 0.0)
        assert np.max(np.abs(half - 0.5 * full)) <= 1e-13


# ----------------------------------------------------------------------------- decay (NEXT-1)
def _random_alpha(rng, F, dk, lo=0.3):
    return rng.uniform(lo, 1.0, (F, dk))


def pin_decay_update(o):
    """[VDN] Sec. 3.1 Eq. (2) and App. A.1 Eq. (A.1): entering a frame with decay
    alpha, the inherited state S Diag(alpha) (scaled channel by channel in a hand
    loop) is updated by Eq. (5): the gradient of Eq. (4) around that inherited
    state vanishes, and the result equals S M + J with M = Diag(alpha)(I + A)^{-1},
    J = B (I + A)^{-1}."""
    rng = _rng(31)
    for _ in range(5):
        S_prev, K, V, beta = _frame(rng, U=9, dk=6, dv=4)
        alpha = rng.uniform(0, 1, 6)
        S_bar = S_prev.copy()
        for i in range(S_bar.shape[0]):
            for j in range(S_bar.shape[1]):
                S_bar[i, j] = S_prev[i, j] * alpha[j]
        assert np.max(np.abs(o.decay(S_prev, alpha) - S_bar)) <= 1e-15
        A, B = o.frame_statistics(K, V, beta)
        S = o.frame_update(o.decay(S_prev, alpha), A, B)
        g = _gradient(S, S_bar, K, V, beta)
        assert np.linalg.norm(g) <= 1e-12 * max(1.0, np.linalg.norm(S_bar))
        inv = np.linalg.solve(np.eye(6) + A, np.eye(6))
        assert np.max(np.abs(S - (S_prev @ o.transition(A, alpha) + B @ inv))) <= 1e-12


def pin_decay_one(o):
    """alpha = 1 everywhere is no decay: identical states and outputs to the
    undecayed definition (the bridge products are all one)."""
    rng = _rng(32)
    x = _random_unit(rng, 11, 5, 6, 4, 3)
    out0, t0 = _call(o, x, chunk=3, radius=1, taps=True)
    out1, t1 = _call(o, x, chunk=3, radius=1, taps=True, alpha=np.ones((11, 6)))
    assert np.array_equal(out0, out1)
    assert np.array_equal(t0["P"], t1["P"]) and np.array_equal(t0["R"], t1["R"])


def pin_decay_pure_bridge(o):
    """No video writes (beta = 0) and a text seed s: each scan only decays, so
    P[j] = s Diag(prod_{g < Cj} alpha_g), R[j] = s Diag(prod_{g >= Cj} alpha_g),
    and the bridge of App. A.3 telescopes: frame f reads
    s Diag(prod_{g <= f} alpha_g + prod_{g >= f} alpha_g), whatever the chunk
    length and radius (cumulative products computed here with a running loop)."""
    rng = _rng(33)
    for C, r, F in ((5, 1, 17), (2, 2, 9), (3, 0, 10), (1, 1, 6), (4, 3, 8)):
        x = _random_unit(rng, F, 3, 5, 4, 4)
        x["beta"][:] = 0.0
        alpha = _random_alpha(rng, F, 5, lo=0.0)
        _, t = _call(o, x, chunk=C, radius=r, taps=True, alpha=alpha)
        s = t["seed"]
        fwd = np.ones((F + 1, 5))   # fwd[f] = prod_{g < f} alpha_g
        for f in range(F):
            fwd[f + 1] = fwd[f] * alpha[f]
        bwd = np.ones((F + 1, 5))   # bwd[f] = prod_{g >= f} alpha_g
        for f in range(F - 1, -1, -1):
            bwd[f] = bwd[f + 1] * alpha[f]
        n = -(-F // C)
        for j in range(n + 1):
            e = min(C * j, F)
            assert np.max(np.abs(t["P"][j] - s * fwd[e][None, :])) <= 1e-14, (C, r, j)
            assert np.max(np.abs(t["R"][j] - s * bwd[e][None, :])) <= 1e-14, (C, r, j)
        for f in range(F):
            want = s * (fwd[f + 1] + bwd[f])[None, :]
            assert np.max(np.abs(t["St"][f] - want)) <= 1e-14, (C, r, f)


def pin_decay_zero(o):
    """alpha = 0 erases every inherited state: a frame's state is its own write
    alone, the state after chunk j comes from its last frame only, and every
    bridged state is exactly zero (each product contains alpha_f = 0), so every
    output is zero."""
    rng = _rng(34)
    F, C = 8, 3
    x = _random_unit(rng, F, 4, 5, 3, 2)
    out, t = _call(o, x, chunk=C, radius=1, taps=True, alpha=np.zeros((F, 5)))
    assert np.all(out == 0.0) and np.all(t["St"] == 0.0)
    for j, (lo, hi) in enumerate(o.chunk_bounds(F, C)):
        A, B = o.frame_statistics(x["k"][hi - 1], x["v"][hi - 1], x["beta"][hi - 1])
        S_last = _update(o, np.zeros((3, 5)), x["k"][hi - 1], x["v"][hi - 1], x["beta"][hi - 1])
        assert np.max(np.abs(t["P"][j + 1] - S_last)) <= 1e-14
        S_first = _update(o, np.zeros((3, 5)), x["k"][lo], x["v"][lo], x["beta"][lo])
        assert np.max(np.abs(t["R"][j] - S_first)) <= 1e-14


def pin_decay_scalar(o):
    """d_k = d_v = 1, chunk 1, radius 1, exact rational arithmetic: each frame maps
    s -> (alpha s + b) / (1 + a); the forward and reverse scans and the bridged
    states follow by hand from that rule (Fractions, no numpy)."""
    Fr = Fraction
    v = [Fr(1), Fr(-2), Fr(3), Fr(1, 2), Fr(-1)]
    beta = [Fr(1, 2), Fr(1), Fr(1, 4), Fr(2), Fr(1, 3)]
    alpha = [Fr(1, 2), Fr(3, 4), Fr(1), Fr(1, 5), Fr(2, 3)]
    tv, tb = Fr(2), Fr(1)
    F = len(v)
    seed = tb * tv / (1 + tb) / 2
    step = lambda s, f: (alpha[f] * s + beta[f] * v[f]) / (1 + beta[f])  # noqa: E731
    P = [seed]
    for f in range(F):
        P.append(step(P[-1], f))
    R = [None] * (F + 1)
    R[F] = seed
    for f in range(F - 1, -1, -1):
        R[f] = step(R[f + 1], f)

    def prod(a, b):
        out = Fr(1)
        for g in range(a, b + 1):
            out *= alpha[g]
        return out
    St = []
    for f in range(F):
        lo, hi = max(f - 1, 0), min(f + 1, F - 1)
        St.append(P[lo] * prod(lo, f) + R[hi + 1] * prod(f, hi))
    k = np.ones((F, 1, 1))
    q = np.ones((F, 1, 1))
    _, t = o.forward_unit(q, k, np.array([float(x) for x in v]).reshape(F, 1, 1),
                          np.array([float(x) for x in beta]).reshape(F, 1), np.zeros((F, 1, 1)),
                          np.ones((1, 1)), np.array([[float(tv)]]), np.array([float(tb)]),
                          np.ones(1), chunk=1, radius=1, taps=True,
                          alpha=np.array([float(x) for x in alpha]).reshape(F, 1))
    assert np.max(np.abs(t["P"].ravel() - np.array([float(x) for x in P]))) <= 1e-15
    assert np.max(np.abs(t["R"].ravel() - np.array([float(x) for x in R]))) <= 1e-15
    assert np.max(np.abs(t["St"].ravel() - np.array([float(x) for x in St]))) <= 1e-15


def pin_decay_non_expansive(o):
    """Prop. 1 / App. A.1 with decay: ||Diag(alpha)(I + A)^{-1}||_2 <= 1 for
    alpha in [0, 1] (also for lambda_max(A) > 2), and the difference of two
    entering states never grows through a decayed frame sequence."""
    rng = _rng(35)
    for scale in (0.1, 1.0, 30.0):
        for _ in range(4):
            K = rng.standard_normal((12, 6))
            A, _ = o.frame_statistics(K, np.zeros((12, 1)), scale * rng.uniform(0, 1, 12))
            M = o.transition(A, rng.uniform(0, 1, 6))
            assert np.linalg.norm(M, 2) <= 1.0 + 1e-12
    S1, S2 = rng.standard_normal((2, 4, 6))
    d0 = np.linalg.norm(S1 - S2)
    for _ in range(8):
        _, K, V, beta = _frame(rng, U=10, dk=6, dv=4)
        alpha = rng.uniform(0, 1, 6)
        A, B = o.frame_statistics(K, V, beta)
        S1 = o.frame_update(o.decay(S1, alpha), A, B)
        S2 = o.frame_update(o.decay(S2, alpha), A, B)
        d1 = np.linalg.norm(S1 - S2)
        assert d1 <= d0 * (1 + 1e-12)
        d0 = d1


def pin_decay_time_reversal(o):
    """The two scans stay mirror images with decay: reversing the frame order (and
    the gates with it; F a multiple of C) maps the output of frame f to frame
    F-1-f, which holds only if each direction decays with the gate of the frame it
    enters and the bridge products are taken symmetrically."""
    rng = _rng(36)
    for C, r, F in ((5, 1, 20), (2, 1, 8), (3, 2, 15), (1, 1, 6)):
        x = _random_unit(rng, F, 4, 5, 3, 3)
        alpha = _random_alpha(rng, F, 5)
        out = _call(o, x, chunk=C, radius=r, alpha=alpha)
        xr = dict(x)
        for key in ("q", "k", "v", "beta", "gate"):
            xr[key] = x[key][::-1].copy()
        out_r = _call(o, xr, chunk=C, radius=r, alpha=alpha[::-1].copy())
        assert np.max(np.abs(out_r[::-1] - out)) <= 1e-12, (C, r, F)


def pin_decay_chunk_composition(o):
    """With decay each frame is the affine map S -> S Diag(alpha) (I+A)^{-1} + J;
    composing per chunk in each direction reproduces both scans, and the reverse
    chunk transition is no longer the transpose of the forward one."""
    rng = _rng(37)
    F, C, U, dk, dv = 13, 5, 6, 5, 4
    x = _random_unit(rng, F, U, dk, dv, 3)
    alpha = _random_alpha(rng, F, dk)
    _, tap = _call(o, x, chunk=C, radius=1, taps=True, alpha=alpha)
    n = -(-F // C)
    I = np.eye(dk)
    Ms = [np.diag(alpha[f]) @ np.linalg.inv(I + tap["A"][f]) for f in range(F)]
    Js = [tap["B"][f] @ np.linalg.inv(I + tap["A"][f]) for f in range(F)]
    assert np.max(np.abs(np.array(Ms) - tap["M"])) <= 1e-12
    P = [tap["P"][0]]
    R = [None] * (n + 1)
    R[n] = tap["R"][n]
    maps = []
    asym = 0.0
    for lo, hi in [(s, min(s + C, F)) for s in range(0, F, C)]:
        Mf, Jf = I.copy(), np.zeros((dv, dk))
        for f in range(lo, hi):
            Mf, Jf = Mf @ Ms[f], Jf @ Ms[f] + Js[f]
        Mr, Jr = I.copy(), np.zeros((dv, dk))
        for f in range(hi - 1, lo - 1, -1):
            Mr, Jr = Mr @ Ms[f], Jr @ Ms[f] + Js[f]
        asym = max(asym, np.max(np.abs(Mr - Mf.T)))
        maps.append((Mf, Jf, Mr, Jr))
    for j in range(n):
        P.append(P[j] @ maps[j][0] + maps[j][1])
    for j in range(n - 1, -1, -1):
        R[j] = R[j + 1] @ maps[j][2] + maps[j][3]
    assert np.max(np.abs(np.array(P) - tap["P"])) <= 1e-12
    assert np.max(np.abs(np.array(R) - tap["R"])) <= 1e-12
    assert asym > 1e-3


# ----------------------------------------------------------------------------- NEXT-2: anchors
def _anchor_cases():
    # (F, C, r): interior chunks, clipped windows on both sides, a short last chunk
    return ((13, 5, 1), (16, 5, 1), (9, 2, 1), (12, 3, 0), (11, 1, 2), (21, 5, 1))


def pin_anchor_rows_zero(o):
    """Algorithm 1 step 7 and App. A.3: the anchor rows (frames 0 and F - 1) get
    no linear output, and a clip made only of anchors (F <= 2) gets none at all."""
    rng = _rng(41)
    for F, C, r in _anchor_cases():
        x = _random_unit(rng, F, 3, 4, 3, 2)
        for alpha in (None, _random_alpha(rng, F, 4)):
            out = _call(o, x, chunk=C, radius=r, alpha=alpha, anchors=True)
            assert np.all(out[0] == 0.0) and np.all(out[F - 1] == 0.0), (F, C, r)
    for F in (1, 2):
        x = _random_unit(rng, F, 3, 4, 3, 2)
        out = _call(o, x, chunk=5, radius=1, anchors=True)
        assert out.shape == (F, 3, 3) and np.all(out == 0.0)


def pin_anchor_inputs_ignored(o):
    """Sec. 2.2 / Algorithm 1 step 2: the anchor frames' rows are removed from the
    linear inputs, so redrawing their keys, values, write strengths, queries,
    gate logits and decay gates changes no output at all (bit for bit)."""
    rng = _rng(42)
    for F, C, r in _anchor_cases():
        x = _random_unit(rng, F, 3, 4, 3, 2)
        alpha = _random_alpha(rng, F, 4)
        out = _call(o, x, chunk=C, radius=r, alpha=alpha, anchors=True)
        y = {key: val.copy() for key, val in x.items()}
        a2 = alpha.copy()
        other = _random_unit(rng, F, 3, 4, 3, 2)
        for key in ("q", "k", "v", "beta", "gate"):
            y[key][0] = other[key][0]
            y[key][F - 1] = other[key][F - 1]
        a2[0] = rng.uniform(0, 1, 4)
        a2[F - 1] = rng.uniform(0, 1, 4)
        out2 = _call(o, y, chunk=C, radius=r, alpha=a2, anchors=True)
        assert np.array_equal(out, out2), (F, C, r)


def pin_anchor_identity_frames(o):
    """An anchor left out of both scans is the identity map S -> S: with anchors,
    every interior, non-bypassed row equals the anchor-free forward pass whose
    anchor frames write nothing (beta = 0: Eq. (5) gives S (I + 0) = S_bar) and
    do not decay (alpha = 1), because clipping the window to the interior frames
    then only drops identity factors from the bridge (App. A.3)."""
    rng = _rng(43)
    for F, C, r in _anchor_cases():
        x = _random_unit(rng, F, 4, 5, 3, 3)
        for alpha in (None, _random_alpha(rng, F, 5)):
            out = _call(o, x, chunk=C, radius=r, alpha=alpha, anchors=True)
            y = {key: val.copy() for key, val in x.items()}
            y["beta"][0] = 0.0
            y["beta"][F - 1] = 0.0
            a2 = None
            if alpha is not None:
                a2 = alpha.copy()
                a2[0] = 1.0
                a2[F - 1] = 1.0
            ref = _call(o, y, chunk=C, radius=r, alpha=a2)
            live = [t for t in range(1, F - 1) if np.any(out[t] != 0.0)]
            assert live, (F, C, r)
            for t in live:
                assert np.max(np.abs(out[t] - ref[t])) <= 1e-12, (F, C, r, t)


def pin_anchor_bypass(o):
    """App. A.3: a query whose window (chunks c - r .. c + r) covers the whole clip
    bypasses the linear path.  Hand-enumerated zero rows for four clips."""
    rng = _rng(44)
    cases = {  # (F, C, r): frames with zero output (anchors included)
        (10, 5, 1): set(range(10)),         # both chunks' windows span frames 0..9
        (11, 5, 1): {0, 5, 6, 7, 8, 9, 10},  # chunk 1's window spans 0..10
        (16, 5, 1): {0, 15},                 # no window spans the clip
        (3, 1, 1): {0, 1, 2},                # frame 1's window spans 0..2
    }
    for (F, C, r), zero in cases.items():
        x = _random_unit(rng, F, 3, 4, 3, 2)
        out = _call(o, x, chunk=C, radius=r, anchors=True)
        for t in range(F):
            if t in zero:
                assert np.all(out[t] == 0.0), (F, C, r, t)
            else:
                assert np.all(np.abs(out[t]).max(axis=-1) > 0), (F, C, r, t)


def pin_anchor_scalar(o):
    """d_k = d_v = 1, exact rational arithmetic, App. A.3 written out by hand: the
    interior frames 1..F-2 map s -> (alpha s + b) / (1 + a); P_0 = R_{F-1} = seed;
    P_j through interior frame j, R_j from frame F-2 down to j; frame t reads
    P_{l-1} prod_{l..t} alpha + R_{h+1} prod_{t..h} alpha over its window [l, h]
    clipped to 1..F-2 (F = 7, chunks of 2, radius 0)."""
    Fr = Fraction
    v = [Fr(5), Fr(1), Fr(-2), Fr(3), Fr(1, 2), Fr(-1), Fr(7)]
    beta = [Fr(3), Fr(1, 2), Fr(1), Fr(1, 4), Fr(2), Fr(1, 3), Fr(4)]
    alpha = [Fr(1, 9), Fr(1, 2), Fr(3, 4), Fr(1), Fr(1, 5), Fr(2, 3), Fr(1, 7)]
    tv, tb = Fr(2), Fr(1)
    F, C = 7, 2
    seed = tb * tv / (1 + tb) / 2
    step = lambda s, f: (alpha[f] * s + beta[f] * v[f]) / (1 + beta[f])  # noqa: E731
    P = {0: seed}
    for j in range(1, F - 1):
        P[j] = step(P[j - 1], j)
    R = {F - 1: seed}
    for j in range(F - 2, 0, -1):
        R[j] = step(R[j + 1], j)

    def prod(a, b):
        out = Fr(1)
        for g in range(a, b + 1):
            out *= alpha[g]
        return out
    windows = {1: (1, 1), 2: (2, 3), 3: (2, 3), 4: (4, 5), 5: (4, 5)}  # chunk [2c, 2c+1] clipped
    St = [Fr(0)] * F
    for t, (lo, hi) in windows.items():
        St[t] = P[lo - 1] * prod(lo, t) + R[hi + 1] * prod(t, hi)
    k = np.ones((F, 1, 1))
    q = np.ones((F, 1, 1))
    _, tap = o.forward_unit(q, k, np.array([float(x) for x in v]).reshape(F, 1, 1),
                            np.array([float(x) for x in beta]).reshape(F, 1),
                            np.zeros((F, 1, 1)), np.ones((1, 1)), np.array([[float(tv)]]),
                            np.array([float(tb)]), np.ones(1), chunk=C, radius=0, taps=True,
                            alpha=np.array([float(x) for x in alpha]).reshape(F, 1),
                            anchors=True)
    assert np.max(np.abs(tap["St"].ravel() - np.array([float(x) for x in St]))) <= 1e-15
    assert np.max(np.abs(tap["P"].ravel() - np.array([float(P[j]) for j in range(F - 1)]))) \
        <= 1e-15
    assert np.max(np.abs(tap["R"].ravel() - np.array([float(R[j]) for j in range(1, F)]))) \
        <= 1e-15


def pin_anchor_disjointness(o):
    """Sec. 2.2 with anchors: one writing interior frame f*, no text.  A live query
    frame t (interior, not bypassed) reads f* iff f* lies outside t's window; an
    anchor's write is never read."""
    rng = _rng(45)
    for F, C, r in ((16, 5, 1), (13, 3, 1), (9, 2, 0)):
        for fstar in range(F):
            x = _random_unit(rng, F, 3, 4, 3, 0)
            x["beta"][:] = 0.0
            x["beta"][fstar] = rng.uniform(0.3, 1.0, 3)
            out = _call(o, x, chunk=C, radius=r, anchors=True)
            for t in range(1, F - 1):
                c = t // C
                lo, hi = C * max(c - r, 0), min(C * (c + r + 1), F) - 1
                if lo == 0 and hi == F - 1:
                    continue
                seen = 0 < fstar < F - 1 and not (lo <= fstar <= hi)
                if seen:
                    assert np.all(np.abs(out[t]).max(axis=-1) > 0), (F, C, r, fstar, t)
                else:
                    assert np.all(out[t] == 0.0), (F, C, r, fstar, t)


# ----------------------------------------------------------------------------- NEXT-4: batched rule
def pin_batched_token_sum(o):
    """[VDN] Eq. (3a) with plain loops: every token's correction
    beta_u (v_u - S_bar k_u) k_u^T is evaluated at the same S_bar and added; the
    oracle's Eq. (3c) form S_bar (I - A) + B must agree."""
    rng = _rng(51)
    for _ in range(5):
        S_bar, K, V, beta = _frame(rng, U=8, dk=5, dv=3)
        S = S_bar.copy()
        for u in range(K.shape[0]):
            r = V[u] - S_bar @ K[u]
            for i in range(S.shape[0]):
                for j in range(S.shape[1]):
                    S[i, j] += beta[u] * r[i] * K[u, j]
        A, B = o.frame_statistics(K, V, beta)
        assert np.max(np.abs(o.batched_update(S_bar, A, B) - S)) <= 1e-13


def pin_batched_scaled_keys(o):
    """App. A.2: rule 2 is rule 1 with every key divided by sqrt(frame size): the
    video keys by sqrt(U), the text keys by sqrt(T) (queries untouched)."""
    rng = _rng(52)
    for F, C, r, U, T in ((12, 5, 1, 6, 4), (7, 2, 1, 3, 0), (9, 3, 0, 5, 2)):
        x = _random_unit(rng, F, U, 4, 3, T)
        for anchors in (False, True):
            out2 = _call(o, x, chunk=C, radius=r, rule=2, anchors=anchors)
            y = dict(x)
            y["k"] = x["k"] / np.sqrt(U)
            y["text_k"] = x["text_k"] / np.sqrt(max(T, 1))
            out1 = _call(o, y, chunk=C, radius=r, rule=1, anchors=anchors)
            assert np.max(np.abs(out2 - out1)) <= 1e-12, (F, C, r, U, T, anchors)


def pin_batched_seed(o):
    """Eq. (1b) under the batched rule: from S = 0 the update is just B_T, so the
    seed is B_T / 2 in mode 0 and B_T(beta / 2) = B_T / 2 in mode 1."""
    rng = _rng(53)
    _, K, V, beta = _frame(rng, U=6, dk=4, dv=3)
    A, B = o.frame_statistics(K, V, beta)
    for mode in (0, 1):
        seed = o.text_state(K, V, beta, 4, 3, mode, rule=1)
        assert np.max(np.abs(seed - 0.5 * B)) <= 1e-14, mode


def pin_batched_contraction(o):
    """App. A.2 through the oracle's scans: a frame of U copies of one unit key k
    with common beta and zero values maps the state's k-component by 1 - U beta
    under rule 1 (growth once U beta > 2), by 1 - beta under rule 2 (scaled keys)
    and by 1 / (1 + U beta) under the frame-wise rule."""
    rng = _rng(54)
    dk, dv, U, F = 4, 3, 6, 4
    k = _unit(rng.standard_normal(dk))
    b = 0.7  # U b = 4.2 > 2
    x = dict(q=rng.standard_normal((F, U, dk)), k=np.tile(k, (F, U, 1)),
             v=np.zeros((F, U, dv)), beta=np.full((F, U), b),
             gate=rng.standard_normal((F, U, dv)), text_k=k[None, :],
             text_v=rng.standard_normal((1, dv)), text_beta=np.array([0.9]),
             rms_weight=np.ones(dv))
    for rule, factor in ((1, 1 - U * b), (2, 1 - b), (0, 1 / (1 + U * b))):
        _, tap = _call(o, x, chunk=1, radius=0, rule=rule, taps=True)
        Pk = tap["P"] @ k
        for j in range(F):
            assert np.max(np.abs(Pk[j + 1] - factor * Pk[j])) <= 1e-12 * np.abs(Pk[j]).max()
    # unit keys, beta <= 1: lambda_max(A) <= tr A <= U, and the scaled factor is
    # non-expansive while the unscaled one is not once lambda_max > 2
    K = _unit(rng.standard_normal((50, dk)))
    K[:40] = k
    A, _ = o.frame_statistics(K, np.zeros((50, dv)), rng.uniform(0.5, 1.0, 50))
    lam = np.linalg.eigvalsh(A)
    assert lam.max() <= np.trace(A) + 1e-12 and lam.max() > 2
    As, _ = o.scaled_statistics(A, np.zeros((dv, dk)), 50)
    assert np.linalg.norm(np.eye(dk) - As, 2) <= 1 + 1e-12
    assert np.linalg.norm(np.eye(dk) - A, 2) > 1


def pin_batched_a2_weights(o):
    """App. A.2: with scaled keys k' = k / sqrt(U), U repeats of one unit key give
    S k' = (1 - beta) S_bar k' + beta v_mean (weight beta on the consensus),
    while U orthonormal keys give S k'_u = (1 - beta / U) S_bar k'_u + (beta / U) v_u."""
    rng = _rng(55)
    U, dv = 8, 3
    b = 0.6
    k = _unit(rng.standard_normal(U))
    V = rng.standard_normal((U, dv))
    S_bar = rng.standard_normal((dv, U))
    A, B = o.frame_statistics(np.tile(k, (U, 1)), V, np.full(U, b))
    S = o.batched_update(S_bar, *o.scaled_statistics(A, B, U))
    kp = k / np.sqrt(U)
    assert np.max(np.abs(S @ kp - ((1 - b) * S_bar @ kp + b * V.mean(axis=0)))) <= 1e-13
    Q, _ = np.linalg.qr(rng.standard_normal((U, U)))
    A, B = o.frame_statistics(Q, V, np.full(U, b))
    S = o.batched_update(S_bar, *o.scaled_statistics(A, B, U))
    for u in range(U):
        kp = Q[u] / np.sqrt(U)
        want = (1 - b / U) * S_bar @ kp + (b / U) * V[u]
        assert np.max(np.abs(S @ kp - want)) <= 1e-13


ALL_PINS = [
    pin_stats_hand_loop, pin_stats_invariants, pin_gradient_zero, pin_lstsq_bruteforce,
    pin_sherman_morrison, pin_repeated_keys, pin_orthonormal_keys, pin_beta_zero,
    pin_non_expansive, pin_scalar_case, pin_orthonormal_golden, pin_exactly_once,
    pin_time_reversal, pin_disjointness, pin_forward_reverse_regions, pin_chunk_composition,
    pin_golden_scan, pin_token_permutation, pin_all_beta_zero, pin_rmsnorm_gate,
    pin_decay_update, pin_decay_one, pin_decay_pure_bridge, pin_decay_zero, pin_decay_scalar,
    pin_decay_non_expansive, pin_decay_time_reversal, pin_decay_chunk_composition,
    pin_anchor_rows_zero, pin_anchor_inputs_ignored, pin_anchor_identity_frames,
    pin_anchor_bypass, pin_anchor_scalar, pin_anchor_disjointness,
    pin_batched_token_sum, pin_batched_scaled_keys, pin_batched_seed, pin_batched_contraction,
    pin_batched_a2_weights,
]

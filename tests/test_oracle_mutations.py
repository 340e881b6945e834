"""Planted mistakes in a private copy of the oracle must each break a pin.

Every mutation below is a plausible slip (a dropped term, a wrong sign, an
off-by-one index, a transposed operand, a swapped direction).  The test loads a
fresh copy of the oracle module, plants one mistake in it (CPU only), runs the
pin suite and requires at least one pin to fail.  The real oracle is untouched.
"""
import importlib.util
import os

import numpy as np
import pytest

import oracle_pins

ORACLE_FILE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                           "oracle", "vda_oracle.py")


def fresh_oracle():
    spec = importlib.util.spec_from_file_location("vda_oracle_mutant", ORACLE_FILE)
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def _stats_no_beta(m):
    def frame_statistics(K, V, beta):
        K = np.asarray(K, float)
        V = np.asarray(V, float)
        return K.T @ K, V.T @ K
    m.frame_statistics = frame_statistics


def _stats_beta_squared(m):
    orig = m.frame_statistics

    def frame_statistics(K, V, beta):
        return orig(K, V, np.asarray(beta, float) ** 2)
    m.frame_statistics = frame_statistics


def _stats_b_swapped(m):
    def frame_statistics(K, V, beta):
        K = np.asarray(K, float)
        V = np.asarray(V, float)
        b = np.asarray(beta, float)
        A = K.T @ (b[:, None] * K)
        Bt = K.T @ (b[:, None] * V)
        return A, Bt.T if Bt.shape[0] != Bt.shape[1] else Bt
    m.frame_statistics = frame_statistics


def _update_minus(m):
    def frame_update(S_bar, A, B):
        G = np.eye(A.shape[0]) - A
        return np.linalg.solve(G.T, (S_bar + B).T).T
    m.frame_update = frame_update


def _update_no_identity(m):
    def frame_update(S_bar, A, B):
        G = A + 1e-3 * np.eye(A.shape[0])
        return np.linalg.solve(G.T, (S_bar + B).T).T
    m.frame_update = frame_update


def _update_drops_inherited(m):
    def frame_update(S_bar, A, B):
        G = np.eye(A.shape[0]) + A
        return S_bar + np.linalg.solve(G.T, B.T).T
    m.frame_update = frame_update


def _update_frozen_state(m):
    # the additive rule S_bar (I - A) + B ([VDN] Eq. (3c)) instead of the joint solve
    def frame_update(S_bar, A, B):
        return S_bar @ (np.eye(A.shape[0]) - A) + B
    m.frame_update = frame_update


def _update_left_multiplied(m):
    def frame_update(S_bar, A, B):
        G = np.eye(A.shape[0]) + A
        R = S_bar + B
        if R.shape[0] == G.shape[0]:
            return np.linalg.solve(G, R)
        return np.linalg.solve(G.T, R.T).T @ G @ G  # still wrong when not square
    m.frame_update = frame_update


def _seed_not_halved(m):
    orig = m.text_state

    def text_state(*a, **kw):
        return 2.0 * orig(*a, **kw)
    m.text_state = text_state


def _gather_fwd_off_by_one(m):
    def gather(P, R, c, radius):
        n = P.shape[0] - 1
        return P[min(max(c - radius + 1, 0), n)] + R[min(c + radius + 1, n)]
    m.gather = gather


def _gather_rev_off_by_one(m):
    def gather(P, R, c, radius):
        n = P.shape[0] - 1
        return P[max(c - radius, 0)] + R[min(c + radius, n)]
    m.gather = gather


def _gather_swapped(m):
    def gather(P, R, c, radius):
        n = P.shape[0] - 1
        return R[max(c - radius, 0)] + P[min(c + radius + 1, n)]
    m.gather = gather


def _reverse_scan_store_late(m):
    orig = m.directional_states

    def directional_states(stats, seed, C, alpha=None):
        P, R = orig(stats, seed, C, alpha)
        R2 = R.copy()
        R2[:-1] = R[1:]   # R[j] := state after chunk j+1
        return P, R2
    m.directional_states = directional_states


def _scan_variant(m, fwd_frames=None, rev_gate=None, decay_fwd=True, decay_after=False):
    """directional_states with one planted slip (the arguments select it)."""
    def directional_states(stats, seed, C, alpha=None):
        F = len(stats)
        bounds = m.chunk_bounds(F, C)
        n = len(bounds)
        P = np.zeros((n + 1,) + seed.shape)
        R = np.zeros((n + 1,) + seed.shape)

        def enter(S, f, gate, use_decay=True):
            if alpha is None or not use_decay:
                return m.frame_update(S, *stats[f])
            if decay_after:
                return m.decay(m.frame_update(S, *stats[f]), alpha[gate])
            return m.frame_update(m.decay(S, alpha[gate]), *stats[f])
        S = seed.copy()
        P[0] = S
        for j, (lo, hi) in enumerate(bounds):
            for f in (fwd_frames(lo, hi) if fwd_frames else range(lo, hi)):
                S = enter(S, f, f, decay_fwd)
            P[j + 1] = S
        S = seed.copy()
        R[n] = S
        for j in range(n - 1, -1, -1):
            lo, hi = bounds[j]
            for f in range(hi - 1, lo - 1, -1):
                S = enter(S, f, rev_gate(f, F) if rev_gate else f)
            R[j] = S
        return P, R
    m.directional_states = directional_states


def _forward_scan_skips_last_frame(m):
    _scan_variant(m, fwd_frames=lambda lo, hi: range(lo, hi - 1))


def _rms_sum_not_mean(m):
    def rms_norm(O, w, eps):
        O = np.asarray(O, float)
        return np.asarray(w, float) * O / np.sqrt(np.sum(O * O, axis=-1, keepdims=True) + eps)
    m.rms_norm = rms_norm


def _rms_wrong_axis(m):
    def rms_norm(O, w, eps):
        O = np.asarray(O, float)
        ax = 0 if O.ndim > 1 else -1
        return np.asarray(w, float) * O / np.sqrt(np.mean(O * O, axis=ax, keepdims=True) + eps)
    m.rms_norm = rms_norm


def _sigmoid_sign(m):
    m.sigmoid = lambda x: 1.0 / (1.0 + np.exp(np.asarray(x, float)))


def _readout_transposed(m):
    def readout(S_tilde, Q, G, w, eps):
        S = np.asarray(S_tilde, float)
        O = np.asarray(Q, float) @ (S if S.shape[0] == S.shape[1] else S.T)
        return m.sigmoid(G) * m.rms_norm(O, w, eps)
    m.readout = readout


def _transition_wrong(m):
    m.transition = lambda A, alpha=None: np.eye(A.shape[0]) - A


# ---- decay (NEXT-1)
def _decay_after_solve(m):
    _scan_variant(m, decay_after=True)


def _reverse_uses_next_gate(m):
    _scan_variant(m, rev_gate=lambda f, F: min(f + 1, F - 1))


def _forward_ignores_decay(m):
    _scan_variant(m, decay_fwd=False)


def _decay_on_rows(m):
    def decay(S, alpha):
        S = np.asarray(S, float)
        a = np.asarray(alpha, float)
        return a[:S.shape[0], None] * S if S.shape[0] <= a.shape[0] else S * a[None, :]
    m.decay = decay


def _bridge_variant(m, lo_shift=0, hi_shift=0, swap=False, none=False):
    def bridge(P, R, f, C, radius, alpha):
        alpha = np.asarray(alpha, float)
        F = alpha.shape[0]
        n = P.shape[0] - 1
        c = f // C
        lo, hi = m.window_frames(c, C, radius, F)
        if none:
            return m.gather(P, R, c, radius)
        d_f = np.prod(alpha[lo:f + 1 + lo_shift], axis=0)
        d_r = np.prod(alpha[f + hi_shift:hi + 1], axis=0)
        if swap:
            d_f, d_r = d_r, d_f
        return m.decay(P[max(c - radius, 0)], d_f) + m.decay(R[min(c + radius + 1, n)], d_r)
    m.bridge = bridge


def _bridge_excludes_query_frame(m):
    _bridge_variant(m, lo_shift=-1, hi_shift=1)


def _bridge_omitted(m):
    _bridge_variant(m, none=True)


def _bridge_products_swapped(m):
    _bridge_variant(m, swap=True)


def _transition_decay_right(m):
    def transition(A, alpha=None):
        M = np.linalg.inv(np.eye(A.shape[0]) + A)
        return M if alpha is None else M * np.asarray(alpha, float)[None, :]
    m.transition = transition


def _read_variant(m, rows_kept=False, no_bypass=False, rev_early=False, gate_from_window=False,
                  interior_chunks=False):
    def anchored_state_read(P, R, t, C, radius, F, alpha=None):
        if (t == 0 or t == F - 1) and not rows_kept:
            return None
        c = (t - 1) // C if interior_chunks else t // C
        lo, hi = m.window_frames(max(c, 0), C, radius, F)
        if lo == 0 and hi == F - 1 and not no_bypass:
            return None
        l, h = max(lo, 1), min(hi, F - 2)
        rk = h if rev_early else h + 1
        a0 = lo if gate_from_window else l
        if alpha is None:
            return P[l - 1] + R[max(rk, 1)]
        alpha = np.asarray(alpha, float)
        return (m.decay(P[l - 1], np.prod(alpha[a0:t + 1], axis=0))
                + m.decay(R[max(rk, 1)], np.prod(alpha[t:h + 1], axis=0)))
    m.anchored_state_read = anchored_state_read


def _anchor_rows_kept(m):
    _read_variant(m, rows_kept=True)


def _anchor_no_bypass(m):
    _read_variant(m, no_bypass=True)


def _anchor_reverse_read_early(m):
    _read_variant(m, rev_early=True)


def _anchor_bridge_from_unclipped_window(m):
    _read_variant(m, gate_from_window=True)


def _anchor_chunks_over_interior(m):
    _read_variant(m, interior_chunks=True)


def _anchor_reverse_scan_skips_frame(m):
    def anchored_states(stats, seed, alpha=None):
        F = len(stats)
        if F < 2:
            return {}, {}

        def enter(S, f):
            S_bar = S if alpha is None else m.decay(S, alpha[f])
            return m.frame_update(S_bar, *stats[f])
        P = {0: seed.copy()}
        for j in range(1, F - 1):
            P[j] = enter(P[j - 1], j)
        R = {F - 1: seed.copy()}
        if F > 2:
            R[F - 2] = seed.copy()  # slip: the last interior frame never written
        for j in range(F - 3, 0, -1):
            R[j] = enter(R[j + 1], j)
        return P, R
    m.anchored_states = anchored_states


def _batched_plus(m):
    def batched_update(S_bar, A, B):
        return np.asarray(S_bar, float) @ (np.eye(A.shape[0]) + A) + B
    m.batched_update = batched_update


def _batched_write_inside(m):
    def batched_update(S_bar, A, B):
        return (np.asarray(S_bar, float) + B) @ (np.eye(A.shape[0]) - A)
    m.batched_update = batched_update


def _scaling_b_by_n(m):
    def scaled_statistics(A, B, n_tokens):
        return (A, B) if n_tokens == 0 else (A / n_tokens, B / n_tokens)
    m.scaled_statistics = scaled_statistics


def _scaling_a_by_sqrt_n(m):
    def scaled_statistics(A, B, n_tokens):
        return (A, B) if n_tokens == 0 else (A / np.sqrt(n_tokens), B / np.sqrt(n_tokens))
    m.scaled_statistics = scaled_statistics


def _text_frame_not_scaled(m):
    orig = m.text_state

    def text_state(text_k, text_v, text_beta, d_k, d_v, seed_mode=0, rule=0):
        return orig(text_k, text_v, text_beta, d_k, d_v, seed_mode, 1 if rule == 2 else rule)
    m.text_state = text_state


MUTATIONS = {f.__name__.lstrip("_"): f for f in [
    _stats_no_beta, _stats_beta_squared, _stats_b_swapped, _update_minus, _update_no_identity,
    _update_drops_inherited, _update_frozen_state, _update_left_multiplied, _seed_not_halved,
    _gather_fwd_off_by_one, _gather_rev_off_by_one, _gather_swapped, _reverse_scan_store_late,
    _forward_scan_skips_last_frame, _rms_sum_not_mean, _rms_wrong_axis, _sigmoid_sign,
    _readout_transposed, _transition_wrong, _decay_after_solve, _reverse_uses_next_gate,
    _forward_ignores_decay, _decay_on_rows, _bridge_excludes_query_frame, _bridge_omitted,
    _bridge_products_swapped, _transition_decay_right, _anchor_rows_kept, _anchor_no_bypass,
    _anchor_reverse_read_early, _anchor_bridge_from_unclipped_window,
    _anchor_chunks_over_interior, _anchor_reverse_scan_skips_frame, _batched_plus,
    _batched_write_inside, _scaling_b_by_n, _scaling_a_by_sqrt_n, _text_frame_not_scaled,
]}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name):
    m = fresh_oracle()
    MUTATIONS[name](m)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(m)
        except Exception:  # AssertionError, or a shape error from the planted slip
            failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake {name}"


def test_unmutated_copy_passes():
    m = fresh_oracle()
    for pin in oracle_pins.ALL_PINS:
        pin(m)

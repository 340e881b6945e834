"""The VDA-Prep oracle against its pins, and planted slips each caught by one."""
import importlib.util
import os

import numpy as np
import pytest

import prep_pins

PREP_FILE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                         "oracle", "prep_oracle.py")


def fresh():
    spec = importlib.util.spec_from_file_location("prep_oracle_mutant", PREP_FILE)
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


@pytest.mark.parametrize("pin", prep_pins.PREP_PINS, ids=lambda f: f.__name__)
def test_prep_pin(pin):
    pin(fresh())


def _convolution_not_correlation(m):
    orig = m.depthwise_conv3d

    def depthwise_conv3d(x, w_s, w_t):
        return orig(x, np.asarray(w_s)[:, ::-1, ::-1], np.asarray(w_t)[:, ::-1])
    m.depthwise_conv3d = depthwise_conv3d


def _wrap_padding(m):
    def depthwise_conv3d(x, w_s, w_t):
        x = np.asarray(x, float)
        y = np.zeros_like(x)
        for tau in range(5):
            for a in range(5):
                for b in range(5):
                    w = np.asarray(w_t)[:, tau] * np.asarray(w_s)[:, a, b]
                    y += w * np.roll(x, (2 - tau, 2 - a, 2 - b), axis=(0, 1, 2))
        return y
    m.depthwise_conv3d = depthwise_conv3d


def _temporal_on_rows(m):
    orig = m.depthwise_conv3d

    def depthwise_conv3d(x, w_s, w_t):
        w_s2 = np.asarray(w_s) * np.asarray(w_t)[:, :, None]  # temporal taps folded onto rows
        w_t2 = np.zeros_like(np.asarray(w_t))
        w_t2[:, 2] = 1.0
        return orig(x, w_s2, w_t2)
    m.depthwise_conv3d = depthwise_conv3d


def _silu_sign(m):
    def silu(x):
        x = np.asarray(x, float)
        return x / (1.0 + np.exp(x))
    m.silu = silu


def _v_normalized(m):
    orig = m.prep

    def prep(q, k, v, wk_s, wk_t, wv_s, wv_t, eps=1e-6):
        qo, ko, vo = orig(q, k, v, wk_s, wk_t, wv_s, wv_t, eps)
        return qo, ko, m.l2_normalize(vo, eps)
    m.prep = prep


def _k_not_normalized(m):
    orig_l2 = m.l2_normalize
    calls = {"n": 0}

    def l2_normalize(x, eps=1e-6):
        calls["n"] += 1
        return orig_l2(x, eps) if calls["n"] % 2 == 1 else np.asarray(x, float)
    m.l2_normalize = l2_normalize


def _units_head_major(m):
    def to_units(x):
        x = np.asarray(x)
        Bt, F, Hl, Wl, H, d = x.shape
        return x.transpose(4, 0, 1, 2, 3, 5).reshape(Bt * H, F, Hl * Wl, d)
    m.to_units = to_units


MUTATIONS = {f.__name__.lstrip("_"): f for f in [
    _convolution_not_correlation, _wrap_padding, _temporal_on_rows, _silu_sign, _v_normalized,
    _k_not_normalized, _units_head_major]}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_prep_mutation_is_caught(name):
    m = fresh()
    MUTATIONS[name](m)
    failed = []
    for pin in prep_pins.PREP_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(m)
        except Exception:
            failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake {name}"

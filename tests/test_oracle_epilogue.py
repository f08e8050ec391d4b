"""The output-epilogue oracle against its pins, and planted mistakes against them.

Pins: scipy's logistic function, the symmetry and midpoint of the sigmoid,
RMSNorm closed forms over a whole row (not per head: a row whose heads differ
in size fixes which), the limits of the gate, and a constant gate, which tells
normalising before gating from the reverse order.
"""
import importlib.util

import numpy as np
import pytest
import scipy.special

import oracle.epilogue as E


def pin_sigmoid_matches_scipy(m):
    x = np.concatenate([np.linspace(-40, 40, 10001), [-745.0, -700.0, 0.0, 700.0, 1e6]])
    np.testing.assert_allclose(m.sigmoid(x), scipy.special.expit(x), rtol=1e-15, atol=1e-300)
    assert m.sigmoid(np.array([0.0]))[0] == 0.5
    y = np.linspace(-30, 30, 601)
    np.testing.assert_allclose(m.sigmoid(-y), 1.0 - m.sigmoid(y), atol=4e-16)


def pin_row_norm_closed_forms(m):
    # two "heads" of 4: ones and threes; the whole-row RMS is sqrt(5)
    o = np.array([[1.0] * 4 + [3.0] * 4])
    np.testing.assert_allclose(m.row_rms_norm(o, np.ones(8), 0.0),
                               np.array([[1.0] * 4 + [3.0] * 4]) / np.sqrt(5.0), rtol=1e-15)
    x = np.random.default_rng(1).standard_normal((6, 4096))
    y = m.row_rms_norm(x, np.ones(4096), 0.0)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), 1.0, rtol=1e-13)
    # eps by hand: all 2's, eps 12 -> 0.5 * w
    w = np.linspace(0.5, 1.5, 64)
    np.testing.assert_allclose(m.row_rms_norm(np.full((1, 64), 2.0), w, 12.0), 0.5 * w[None],
                               rtol=1e-15)


def pin_gate_limits_and_order(m):
    rng = np.random.default_rng(2)
    o = rng.standard_normal((5, 256))
    w = 1.0 + 0.1 * rng.standard_normal(256)
    y = m.row_rms_norm(o, w, 1e-6)
    # gate fully open / closed
    np.testing.assert_allclose(m.out_norm_gate(o, np.full_like(o, 60.0), w, 1e-6, bf16=False), y,
                               rtol=1e-15)
    assert np.all(m.out_norm_gate(o, np.full_like(o, -800.0), w, 1e-6, bf16=False) == 0.0)
    # a constant gate of 1/2 halves the normalised row (gating first would not:
    # the norm removes any constant factor)
    np.testing.assert_allclose(m.out_norm_gate(o, np.zeros_like(o), w, 1e-6, bf16=False), 0.5 * y,
                               rtol=1e-15)
    # the same in bf16: exact halving of bf16 values; open gate gives y in bf16
    yb = m.out_norm_gate(o, np.full_like(o, 60.0), w, 1e-6, bf16=True)
    np.testing.assert_array_equal(m.out_norm_gate(o, np.zeros_like(o), w, 1e-6, bf16=True),
                                  0.5 * yb)


def pin_tie_bounds(m):
    rng = np.random.default_rng(3)
    o = rng.standard_normal((64, 512))
    z = rng.standard_normal((64, 512))
    w = np.ones(512)
    out, b = m.out_norm_gate(o, z, w, 1e-6, bf16=True, tie_eta=2.0 ** -16)
    np.testing.assert_array_equal(out, m.out_norm_gate(o, z, w, 1e-6, bf16=True))
    assert np.all(b >= 0) and 0 < np.mean(b > 0) < 0.05


ALL_PINS = [pin_sigmoid_matches_scipy, pin_row_norm_closed_forms, pin_gate_limits_and_order,
            pin_tie_bounds]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(E)


MUTANTS = {
    "sum_not_mean": ("ms = np.mean(o * o, axis=-1, keepdims=True)",
                     "ms = np.sum(o * o, axis=-1, keepdims=True)"),
    "eps_dropped": ("np.sqrt(ms + eps)", "np.sqrt(ms)"),
    "weight_dropped": ("* np.asarray(w, dtype=np.float64)", "* 1.0"),
    "sigmoid_sign": ("1.0 / (1.0 + e), e / (1.0 + e)", "e / (1.0 + e), 1.0 / (1.0 + e)"),
    "gate_dropped": ("        return y_pre * s_pre", "        return y_pre"),
    "gate_before_norm": ("    y_pre = row_rms_norm(o, w, eps)\n    s_pre = sigmoid(zlogit)",
                         "    s_pre = sigmoid(zlogit)\n    y_pre = row_rms_norm(o * s_pre, w, eps)\n"
                         "    s_pre = np.ones_like(s_pre)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    with open(E.__file__) as f:
        src = f.read()
    assert src.count(old) == 1, "mutation anchor not found: %s" % name
    path = tmp_path / ("mutant_%s.py" % name)
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location("mutant_%s" % name, str(path))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(mod)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, "no pin caught the planted mistake %s" % name

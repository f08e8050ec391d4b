"""The q/k prologue oracle against its pins, and planted mistakes against them.

Pins come from outside the oracle: torch's own fp32 -> bf16 conversion,
closed forms of RMSNorm, and rotations whose result is fixed by the definition
of RoPE with the page's base 10000 (a unit vector turned by exactly a quarter
turn), plus the invariants a rotation must keep (lengths, inner products that
depend only on the difference of positions). Each planted mistake is a copy of
``oracle/prologue.py`` with one plausible error; at least one pin must reject
each.
"""
import importlib.util
import math

import numpy as np
import pytest
import torch

import oracle.prologue as P

D = 128


def _rng(seed):
    return np.random.default_rng(seed)


def pin_bf16_rounding_matches_torch(m):
    rng = _rng(1)
    x = np.concatenate([
        rng.standard_normal(4096) * 10.0 ** rng.integers(-30, 30, 4096),
        # exact ties at bf16 precision, both parities of the kept bit
        (np.arange(1, 513, dtype=np.float64) * 2.0 + 1.0) * 2.0 ** -8,
        [0.0, -0.0, 1e-40, -3e-39, 3.3e38, -3.4e38, np.inf, -np.inf]])
    x = x.astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    got = m.round_to_bf16(x)
    assert np.array_equal(got, ref)


def pin_rms_norm_closed_forms(m):
    rng = _rng(2)
    x = rng.standard_normal((5, 7, D))
    y = m.rms_norm(x, np.ones(D), 0.0)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), 1.0, rtol=1e-13)
    # scale invariance and sign of a constant row
    np.testing.assert_allclose(m.rms_norm(7.25 * x, np.ones(D), 0.0), y, rtol=1e-13, atol=1e-15)
    c = np.full((1, D), -3.5)
    np.testing.assert_allclose(m.rms_norm(c, np.ones(D), 0.0), -1.0, rtol=1e-15)
    # eps by hand: all 2's, eps 12 -> 2 / sqrt(4 + 12) = 0.5, times the weight
    w = np.linspace(0.5, 1.5, D)
    np.testing.assert_allclose(m.rms_norm(np.full((2, D), 2.0), w, 12.0),
                               np.broadcast_to(0.5 * w, (2, D)), rtol=1e-15)


def _unit(i):
    e = np.zeros((1, 1, D))
    e[0, 0, i] = 1.0
    return e


def pin_rope_quarter_turns(m):
    # dimension 0 turns at one radian per position: a quarter turn at pi/2
    # sends e_0 to e_64 and e_64 to -e_0 (the positive sense)
    np.testing.assert_allclose(m.rope_rotate_half(_unit(0), [math.pi / 2], 10000.0), _unit(64),
                               atol=1e-15)
    np.testing.assert_allclose(m.rope_rotate_half(_unit(64), [math.pi / 2], 10000.0), -_unit(0),
                               atol=1e-15)
    # dimension 32 turns at 10000^(-64/128) = 0.01 rad per position, 16 at 0.1
    np.testing.assert_allclose(m.rope_rotate_half(_unit(32), [50 * math.pi], 10000.0), _unit(96),
                               atol=1e-13)
    np.testing.assert_allclose(m.rope_rotate_half(_unit(16), [5 * math.pi], 10000.0), _unit(80),
                               atol=1e-13)
    # position 0 is the identity
    x = _rng(3).standard_normal((9, 4, D))
    np.testing.assert_array_equal(m.rope_rotate_half(x, np.zeros(9), 10000.0), x)


def pin_rope_is_a_relative_rotation(m):
    rng = _rng(4)
    x = rng.standard_normal((6, 3, D))
    y = rng.standard_normal((6, 3, D))
    p = rng.integers(0, 100000, 6).astype(np.float64)
    q = rng.integers(0, 100000, 6).astype(np.float64)
    rx = m.rope_rotate_half(x, p, 10000.0)
    np.testing.assert_allclose(np.linalg.norm(rx[..., :64] ** 2 + rx[..., 64:] ** 2, axis=-1),
                               np.linalg.norm(x[..., :64] ** 2 + x[..., 64:] ** 2, axis=-1),
                               rtol=1e-12)
    a = np.sum(rx * m.rope_rotate_half(y, q, 10000.0), axis=-1)
    b = np.sum(m.rope_rotate_half(x, p - q, 10000.0) * y, axis=-1)
    np.testing.assert_allclose(a, b, rtol=1e-9, atol=1e-9)


def pin_prologue_composition(m):
    # rows of +-1 already have unit RMS; with w = 1 and position 0 the
    # prologue gives them back exactly (1/sqrt(1 + 1e-6) rounds back to 1)
    rng = _rng(5)
    x = np.where(rng.random((2, 3, 4, D)) < 0.5, -1.0, 1.0)
    np.testing.assert_array_equal(m.qk_prologue(x, np.ones(D), np.zeros(6), 10000.0, 1e-6), x)
    # at position 0 only the weight acts: w = 2 doubles the normalised row
    np.testing.assert_array_equal(m.qk_prologue(x, 2.0 * np.ones(D), np.zeros(6), 10000.0, 1e-6),
                                  2.0 * x)
    # default positions restart with every sequence
    np.testing.assert_array_equal(m.sequence_positions(7, [0, 3, 3, 7]), [0, 1, 2, 0, 1, 2, 3])


ALL_PINS = [pin_bf16_rounding_matches_torch, pin_rms_norm_closed_forms, pin_rope_quarter_turns,
            pin_rope_is_a_relative_rotation, pin_prologue_composition]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(P)


MUTANTS = {
    "rotation_sign_first_half": ("a * c - b * s, b * c + a * s", "a * c + b * s, b * c + a * s"),
    "rotation_sense_reversed": ("a * c - b * s, b * c + a * s", "a * c + b * s, b * c - a * s"),
    "halves_swapped": ("[a * c - b * s, b * c + a * s]", "[b * c + a * s, a * c - b * s]"),
    "frequency_exponent": ("-2.0 * i / d", "-1.0 * i / d"),
    "pairs_interleaved": ("a, b = x[..., : d // 2], x[..., d // 2:]",
                          "a, b = x[..., 0::2], x[..., 1::2]"),
    "sum_not_mean": ("ms = np.mean(x * x, axis=-1, keepdims=True)",
                     "ms = np.sum(x * x, axis=-1, keepdims=True)"),
    "eps_dropped": ("np.sqrt(ms + eps)", "np.sqrt(ms)"),
    "weight_dropped": ("* np.asarray(w, dtype=np.float64)", "* 1.0"),
    "ties_away_from_zero": ("r = ((u + 0x7FFF + lsb) >> 16) << 16", "r = ((u + 0x8000) >> 16) << 16"),
    "positions_not_restarted": ("pos[cu[n]:cu[n + 1]] = np.arange(cu[n + 1] - cu[n])",
                                "pos[cu[n]:cu[n + 1]] = np.arange(cu[n], cu[n + 1])"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    with open(P.__file__) as f:
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


def test_rounding_tie_helpers():
    # 1 + 2^-8 lies exactly between the bf16 numbers 1 and 1 + 2^-7
    assert P.near_rounding_tie(np.array([1.0 + 2.0 ** -8]), 1e-6)[0]
    assert not P.near_rounding_tie(np.array([1.0]), 1e-3)[0]
    assert P.near_rounding_tie(np.array([1.0]), 2.0 ** -8 + 1e-12)[0]
    np.testing.assert_array_equal(P.bf16_spacing(np.array([1.0, 1.5, 3.0, -0.25])),
                                  [2.0 ** -7, 2.0 ** -7, 2.0 ** -6, 2.0 ** -9])
    # far from every midpoint, no element gets a bound
    x = np.full((1, 1, 1, D), 1.0)
    z, b = P.qk_prologue(x, np.ones(D), np.zeros(1), 10000.0, 0.0, tie_eta=2.0 ** -20)
    np.testing.assert_array_equal(z, x)
    assert not b.any()

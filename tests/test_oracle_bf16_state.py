"""The bf16-state decode oracle against its pins, and planted mistakes.

Pins: the fp64 recurrence oracle (plain C) where every value is exactly
representable in bf16 (then storage changes nothing), a hand case where the
stored state rounds but the output must not, and the distance to the fp64
trajectory over many steps, bounded by half a bf16 spacing per step decayed
geometrically.
"""
import importlib.util

import numpy as np
import pytest

import oracle
import oracle.bf16_state as BS
from oracle.prologue import round_to_bf16


@pytest.fixture(scope="module")
def orc():
    oracle.build(force=False)
    return oracle.Oracle(oracle.LIBRARY)


def pin_exact_when_representable(m, orc):
    # no decay (g = 0 is exact in fp32, which the C oracle takes g in) and
    # small integers: every product and sum is a bf16 number
    rng = np.random.default_rng(1)
    n, d = 3, 8
    S = rng.integers(-8, 9, (n, d, d)).astype(np.float64)
    q = rng.integers(-2, 3, (n, d)).astype(np.float64)
    k = rng.integers(-2, 3, (n, d)).astype(np.float64)
    v = rng.integers(-2, 3, (n, d)).astype(np.float64)
    g = np.zeros(n)
    S64 = S.copy()
    ref = orc.step(q[:, None].astype(np.float32), k[:, None].astype(np.float32),
                   v[:, None].astype(np.float32), g[:, None].astype(np.float32), S64[:, None],
                   0.5)
    o = m.step(q, k, v, g, S, 0.5)
    np.testing.assert_allclose(o, ref[:, 0], rtol=0, atol=1e-12)
    np.testing.assert_array_equal(S, S64)


def pin_output_reads_the_unrounded_state(m, orc):
    S = np.zeros((1, 2, 2))
    q = np.array([[1.0, 0.0]])
    k = np.array([[1.0, 0.0]])
    v = np.array([[1.0 + 2.0 ** -9, 0.0]])
    o = m.step(q, k, v, np.zeros(1), S, 1.0)
    assert o[0, 0] == 1.0 + 2.0 ** -9      # the updated state, before storage
    assert S[0, 0, 0] == 1.0               # stored rounded to bf16 (below the midpoint)


def pin_stays_near_fp64_trajectory(m, orc):
    rng = np.random.default_rng(2)
    n, d, T = 4, 16, 40
    q = round_to_bf16(rng.standard_normal((T, n, d)))
    k = round_to_bf16(rng.standard_normal((T, n, d)))
    v = round_to_bf16(rng.standard_normal((T, n, d)))
    g = np.log(1.0 / (1.0 + np.exp(-(4.0 + rng.standard_normal((T, n))))))
    S = round_to_bf16(0.02 * rng.standard_normal((n, d, d)))
    S64 = S.copy()[:, None]
    out = m.steps(q, k, v, g, S, 0.25)
    for t in range(T):
        orc.step(q[t][:, None].astype(np.float32), k[t][:, None].astype(np.float32),
                 v[t][:, None].astype(np.float32), g[t][:, None].astype(np.float32), S64, 0.25)
    amax = float(np.exp(g.max()))
    bound = 0.5 * float(np.max(np.abs(S64))) * 2.0 ** -7 * 2 / (1.0 - amax)
    assert np.max(np.abs(S - S64[:, 0])) <= bound
    assert np.max(np.abs(S - S64[:, 0])) > 0    # storage does round
    assert out.shape == (T, n, d)


def pin_tie_bounds(m, orc):
    rng = np.random.default_rng(3)
    n, d, T = 8, 32, 6
    q, k, v = (round_to_bf16(rng.standard_normal((T, n, d))) for _ in range(3))
    g = -np.abs(0.05 * rng.standard_normal((T, n)))
    S1 = round_to_bf16(rng.standard_normal((n, d, d)))
    S2 = S1.copy()
    o1 = m.steps(q, k, v, g, S1, 0.2)
    o2, oa, A = m.steps(q, k, v, g, S2, 0.2, tie_eta=2.0 ** -16)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(S1, S2)
    assert np.all(A >= 0) and np.all(oa >= 0) and 0 < np.mean(A > 0) < 0.1


ALL_PINS = [pin_exact_when_representable, pin_output_reads_the_unrounded_state,
            pin_stays_near_fp64_trajectory, pin_tie_bounds]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin(orc, pin):
    pin(BS, orc)


MUTANTS = {
    "decay_after_update": ("    Sp = a * S + k[:, :, None] * v[:, None, :]",
                           "    Sp = a * (S + k[:, :, None] * v[:, None, :])"),
    "output_from_stored_state": ("    o = scale * np.einsum(\"ni,nij->nj\", q, Sp)\n    S[...] = round_to_bf16(Sp)",
                                 "    S[...] = round_to_bf16(Sp)\n    o = scale * np.einsum(\"ni,nij->nj\", q, S)"),
    "no_rounding": ("    S[...] = round_to_bf16(Sp)\n    return o", "    S[...] = Sp\n    return o"),
    "outer_transposed": ("    Sp = a * S + k[:, :, None] * v[:, None, :]",
                         "    Sp = a * S + v[:, :, None] * k[:, None, :]"),
    "scale_dropped": ("    o = scale * np.einsum(\"ni,nij->nj\", q, Sp)",
                      "    o = np.einsum(\"ni,nij->nj\", q, Sp)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(orc, tmp_path, name):
    old, new = MUTANTS[name]
    with open(BS.__file__) as f:
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
            pin(mod, orc)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, "no pin caught the planted mistake %s" % name

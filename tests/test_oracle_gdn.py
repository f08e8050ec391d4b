"""The gated-delta-rule oracle against its pins, and planted mistakes.

Pins from outside the oracle's recurrence:
* with mutually orthogonal keys from a zero state every memory read is 0,
  so beta = 1 gives the Simple GLA update, and beta = 0 writes nothing: the
  Simple GLA oracle (its own C code) must agree in both cases;
* the page's chunkwise form (section 1.2, written in numpy with the UT
  transform solved by numpy) must equal the token-by-token recurrence, which
  also fixes the reading that the decay comes before the memory read;
* with no decay and beta = 1, writing a value under an orthonormal key makes
  the state return exactly that value for the key, overwriting what an
  earlier write stored there (the delta rule's defining property);
* splitting a sequence and chaining the final state gives the same result,
  and one decode step equals a one-token forward.
"""
import os

import numpy as np
import pytest

import oracle
import oracle.gdn as G


@pytest.fixture(scope="module")
def gdn():
    oracle.build(force=False)
    return G.GdnOracle(G.LIBRARY)


def _inputs(seed, B, T, H, Dk, Dv):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, Dk)) / np.sqrt(Dk)
    k = rng.standard_normal((B, T, H, Dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)          # GDN keys are L2-normalised
    v = rng.standard_normal((B, T, H, Dv))
    g = -np.abs(0.1 * rng.standard_normal((B, T, H)))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    S0 = 0.1 * rng.standard_normal((B, H, Dk, Dv))
    return [x.astype(np.float32) for x in (q, k, v, g, beta)] + [S0]


def pin_reduces_to_simple_gla(g_):
    # Mutually orthogonal keys from a zero state: every read k_t^T S is 0, so
    # with beta = 1 the write is k_t v_t^T, the Simple GLA update. The Simple
    # GLA oracle (its own C code) must agree.
    rng = np.random.default_rng(1)
    H, d, T = 3, 16, 12
    k = np.empty((1, T, H, d))
    for h in range(H):
        Qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
        k[0, :, h] = Qm.T[:T]
    q = rng.standard_normal((1, T, H, d))
    v = rng.standard_normal((1, T, H, 8))
    g = -np.abs(0.2 * rng.standard_normal((1, T, H)))
    f = lambda x: x.astype(np.float32)
    o1, S1 = g_.forward(f(q), f(k), f(v), f(g), np.ones((1, T, H), np.float32), 0.7)
    o2, S2 = oracle.forward(f(q), f(k), f(v), f(g), 0.7)
    # fp32 keys are orthogonal to about 1e-8, hence 1e-6 (a wrong term is O(1))
    np.testing.assert_allclose(o1, o2, rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(S1, S2, rtol=1e-6, atol=1e-6)
    # beta = 0 writes nothing: only the decay acts (Simple GLA with v = 0)
    qq, kk, vv, gg, bb, S0 = _inputs(7, 2, 21, 2, 16, 8)
    o3, S3 = g_.forward(qq, kk, vv, gg, np.zeros_like(bb), 0.7, initial_state=S0)
    o4, S4 = oracle.forward(qq, kk, np.zeros_like(vv), gg, 0.7, initial_state=S0)
    np.testing.assert_allclose(o3, o4, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(S3, S4, rtol=1e-12, atol=1e-14)


def pin_chunkwise_form(g_):
    q, k, v, g, beta, S0 = _inputs(2, 1, 150, 2, 16, 12)
    o, S = g_.forward(q, k, v, g, beta, 0.5, initial_state=S0)
    for h in range(2):
        f64 = lambda x: x[0, :, h].astype(np.float64)
        oc, Sc = G.chunked_form(f64(q), f64(k), f64(v), f64(beta), f64(g), S0[0, h], 0.5, 64)
        np.testing.assert_allclose(oc, o[0, :, h], rtol=1e-9, atol=1e-10)
        np.testing.assert_allclose(Sc, S[0, h], rtol=1e-9, atol=1e-10)


def pin_orthonormal_overwrite(g_):
    d = 8
    rng = np.random.default_rng(3)
    Qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
    keys = Qm.T[:5]                                          # 5 orthonormal keys
    vals = rng.standard_normal((6, 4))
    k = np.concatenate([keys, keys[2:3]])[None, :, None, :].astype(np.float32)
    v = vals[None, :, None, :].astype(np.float32)
    n = k.shape[1]
    z = np.zeros((1, n, 1), np.float32)
    _, S = g_.forward(np.zeros((1, n, 1, d), np.float32), k, v, z, np.ones_like(z), 1.0)
    S = S[0, 0]
    kk = k[0, :, 0].astype(np.float64)
    # keys 0, 1, 3, 4 return their values; key 2 returns its second value
    for j in (0, 1, 3, 4):
        np.testing.assert_allclose(kk[j] @ S, v[0, j, 0], atol=1e-5)
    np.testing.assert_allclose(kk[2] @ S, v[0, 5, 0], atol=1e-5)


def pin_split_chain_and_step(g_):
    q, k, v, g, beta, S0 = _inputs(4, 1, 90, 2, 16, 16)
    o, S = g_.forward(q, k, v, g, beta, 0.25, initial_state=S0)
    oa, Sa = g_.forward(q[:, :40], k[:, :40], v[:, :40], g[:, :40], beta[:, :40], 0.25,
                        initial_state=S0)
    ob, Sb = g_.forward(q[:, 40:], k[:, 40:], v[:, 40:], g[:, 40:], beta[:, 40:], 0.25,
                        initial_state=Sa)
    np.testing.assert_allclose(np.concatenate([oa, ob], 1), o, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(Sb, S, rtol=1e-12, atol=1e-12)
    st = np.ascontiguousarray(S0.copy())
    os_ = g_.step(q[:, 0], k[:, 0], v[:, 0], g[:, 0], beta[:, 0], st, 0.25)
    o1, S1 = g_.forward(q[:, :1], k[:, :1], v[:, :1], g[:, :1], beta[:, :1], 0.25,
                        initial_state=S0)
    np.testing.assert_allclose(os_, o1[:, 0], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(st, S1, rtol=1e-12, atol=1e-13)


ALL_PINS = [pin_reduces_to_simple_gla, pin_chunkwise_form, pin_orthonormal_overwrite,
            pin_split_chain_and_step]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin(gdn, pin):
    pin(gdn)


MUTANTS = {
    "read_before_decay": ("    const double alpha = exp(g);\n    for (size_t e = 0; e < (size_t)Dk * Dv; ++e) S[e] *= alpha;\n    for (int j = 0; j < Dv; ++j) u[j] = 0.0;",
                          "    const double alpha = exp(g);\n    for (int j = 0; j < Dv; ++j) u[j] = 0.0;"),
    "beta_dropped": ("const double bk = beta * (double)k[i];", "const double bk = (double)k[i];"),
    "correction_sign": ("((double)v[j] - u[j])", "((double)v[j] + u[j])"),
    "read_key_index": ("const double ki = (double)k[i];\n        for (int j = 0; j < Dv; ++j) u[j] += ki",
                       "const double ki = (double)k[Dk - 1 - i];\n        for (int j = 0; j < Dv; ++j) u[j] += ki"),
    "scale_dropped": ("for (int j = 0; j < Dv; ++j) o[j] *= scale;", "for (int j = 0; j < Dv; ++j) o[j] *= 1.0;"),
    "decay_base_two": ("const double alpha = exp(g);", "const double alpha = exp2(g);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    with open(G.SOURCE) as f:
        src = f.read()
    assert src.count(old) == 1, "mutation anchor not found: %s" % name
    new_src = src.replace(old, new)
    if name == "read_before_decay":
        # decay after the read instead: move the scaling behind the read loop
        new_src = new_src.replace(
            "    for (int i = 0; i < Dk; ++i) {\n        const double bk",
            "    for (size_t e = 0; e < (size_t)Dk * Dv; ++e) S[e] *= alpha;\n"
            "    for (int i = 0; i < Dk; ++i) {\n        const double bk", 1)
    path = tmp_path / ("mutant_%s.c" % name)
    path.write_text(new_src)
    lib = oracle.compile_source(str(path), str(tmp_path / ("libmutant_%s.so" % name)))
    mutant = G.GdnOracle(lib)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(mutant)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, "no pin caught the planted mistake %s" % name

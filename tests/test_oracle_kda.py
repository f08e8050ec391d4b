"""The KDA oracle (gated delta rule with one gate per key dim) against its
pins, and planted mistakes.

Pins from outside the oracle's recurrence:
* with the same gate in every key dim it is the gated delta rule with a
  scalar gate: the GDN oracle (its own C code) must agree;
* the chunkwise form (the page's section 1.2 with the gate made a vector over
  the key dims, written in numpy) must equal the token-by-token recurrence;
* one-hot keys with beta = 1 from a zero state write a value into one state
  row, and later tokens with zero keys only decay it: each row then holds
  its value times exp(sum of its own dim's gates), a closed form that fixes
  which dim's gate scales which row;
* beta = 0 writes nothing: the state is the initial state with row d scaled
  by exp(sum of g over the tokens so far, dim d), and each output reads that;
* with no decay and beta = 1, a value written under an orthonormal key is
  returned exactly for that key (the delta rule's overwrite);
* splitting a sequence and chaining the final state gives the same result,
  packed sequences equal separate calls, and one decode step equals a
  one-token forward.
"""
import numpy as np
import pytest

import oracle
import oracle.gdn as G
import oracle.kda as K


@pytest.fixture(scope="module")
def kda():
    oracle.build(force=False)
    return K.KdaOracle(K.LIBRARY)


def _inputs(seed, B, T, H, Dk, Dv, spread=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, Dk)) / np.sqrt(Dk)
    k = rng.standard_normal((B, T, H, Dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)          # keys are L2-normalised
    v = rng.standard_normal((B, T, H, Dv))
    # per-dim gates: a per-dim rate (spread over a decade) times a per-token factor
    rate = 0.02 * 10.0 ** (spread * rng.random((1, 1, H, Dk)))
    g = -rate * rng.random((B, T, H, Dk))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    S0 = 0.1 * rng.standard_normal((B, H, Dk, Dv))
    return [x.astype(np.float32) for x in (q, k, v, g, beta)] + [S0]


def pin_reduces_to_gdn(kd):
    q, k, v, g, beta, S0 = _inputs(1, 2, 70, 3, 16, 12)
    gs = g[..., 0]                                          # one scalar gate per token and head
    gk = np.repeat(gs[..., None], 16, axis=-1)
    o1, S1 = kd.forward(q, k, v, gk, beta, 0.6, initial_state=S0)
    o2, S2 = G.forward(q, k, v, gs, beta, 0.6, initial_state=S0)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S1, S2, rtol=1e-12, atol=1e-13)


def pin_chunkwise_form(kd):
    q, k, v, g, beta, S0 = _inputs(2, 1, 150, 2, 16, 12, spread=2.0)
    o, S = kd.forward(q, k, v, g, beta, 0.5, initial_state=S0)
    for h in range(2):
        f64 = lambda x: x[0, :, h].astype(np.float64)
        oc, Sc = K.chunked_form(f64(q), f64(k), f64(v), f64(beta), f64(g), S0[0, h], 0.5, 64)
        np.testing.assert_allclose(oc, o[0, :, h], rtol=1e-9, atol=1e-10)
        np.testing.assert_allclose(Sc, S[0, h], rtol=1e-9, atol=1e-10)


def pin_one_hot_rows(kd):
    # token 0 writes v0 into row a, token 1 writes v1 into row b; tokens
    # 2 .. n-1 have zero keys and only decay. Row a then holds
    # v0 * exp(sum_{t >= 1} g[t, a]) and row b v1 * exp(sum_{t >= 2} g[t, b]).
    Dk, Dv, n = 8, 6, 9
    rng = np.random.default_rng(5)
    a, b = 2, 5
    k = np.zeros((1, n, 1, Dk))
    k[0, 0, 0, a] = 1.0
    k[0, 1, 0, b] = 1.0
    v = rng.standard_normal((1, n, 1, Dv))
    g = -rng.random((1, n, 1, Dk)) * np.linspace(0.05, 1.0, Dk)
    q = rng.standard_normal((1, n, 1, Dk))
    f = lambda x: x.astype(np.float32)
    o, S = kd.forward(f(q), f(k), f(v), f(g), np.ones((1, n, 1), np.float32), 0.5)
    g32 = f(g).astype(np.float64)
    want = np.zeros((Dk, Dv))
    want[a] = f(v)[0, 0, 0] * np.exp(g32[0, 1:, 0, a].sum())
    want[b] = f(v)[0, 1, 0] * np.exp(g32[0, 2:, 0, b].sum())
    np.testing.assert_allclose(S[0, 0], want, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(o[0, -1, 0], 0.5 * f(q)[0, -1, 0].astype(np.float64) @ want,
                               rtol=1e-12, atol=1e-15)


def pin_beta_zero(kd):
    q, k, v, g, beta, S0 = _inputs(3, 2, 40, 2, 16, 8, spread=2.0)
    o, S = kd.forward(q, k, v, g, np.zeros_like(beta), 0.3, initial_state=S0)
    Gc = np.cumsum(g.astype(np.float64), axis=1)            # [B, T, H, Dk]
    np.testing.assert_allclose(S, np.exp(Gc[:, -1])[..., None] * S0, rtol=1e-12, atol=1e-15)
    want = 0.3 * np.einsum("bthd,bhde->bthe", q.astype(np.float64) * np.exp(Gc), S0)
    np.testing.assert_allclose(o, want, rtol=1e-11, atol=1e-14)


def pin_orthonormal_overwrite(kd):
    d = 8
    rng = np.random.default_rng(3)
    Qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
    keys = Qm.T[:5]
    vals = rng.standard_normal((6, 4))
    k = np.concatenate([keys, keys[2:3]])[None, :, None, :].astype(np.float32)
    v = vals[None, :, None, :].astype(np.float32)
    n = k.shape[1]
    z = np.zeros((1, n, 1), np.float32)
    _, S = kd.forward(np.zeros((1, n, 1, d), np.float32), k, v, np.zeros((1, n, 1, d), np.float32),
                      np.ones_like(z), 1.0)
    S = S[0, 0]
    kk = k[0, :, 0].astype(np.float64)
    for j in (0, 1, 3, 4):
        np.testing.assert_allclose(kk[j] @ S, v[0, j, 0], atol=1e-5)
    np.testing.assert_allclose(kk[2] @ S, v[0, 5, 0], atol=1e-5)


def pin_split_varlen_and_step(kd):
    q, k, v, g, beta, S0 = _inputs(4, 1, 90, 2, 16, 16)
    o, S = kd.forward(q, k, v, g, beta, 0.25, initial_state=S0)
    oa, Sa = kd.forward(q[:, :40], k[:, :40], v[:, :40], g[:, :40], beta[:, :40], 0.25,
                        initial_state=S0)
    ob, Sb = kd.forward(q[:, 40:], k[:, 40:], v[:, 40:], g[:, 40:], beta[:, 40:], 0.25,
                        initial_state=Sa)
    np.testing.assert_allclose(np.concatenate([oa, ob], 1), o, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(Sb, S, rtol=1e-12, atol=1e-12)
    # packed: the two halves as two sequences with their own initial states
    cu = np.array([0, 40, 90], np.int64)
    S0p = np.concatenate([S0, Sa])
    op, Sp = kd.forward(q, k, v, g, beta, 0.25, initial_state=S0p, cu_seqlens=cu)
    np.testing.assert_allclose(op[:, :40], oa, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(op[:, 40:], ob, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(Sp[1], Sb[0], rtol=1e-12, atol=1e-12)
    # a decode step through a slot map equals a one-token forward
    pool = np.ascontiguousarray(np.concatenate([np.zeros_like(S0), S0]))
    os_ = kd.step(q[:, 0], k[:, 0], v[:, 0], g[:, 0], beta[:, 0], pool, 0.25,
                  state_indices=np.array([1], np.int32))
    o1, S1 = kd.forward(q[:, :1], k[:, :1], v[:, :1], g[:, :1], beta[:, :1], 0.25,
                        initial_state=S0)
    np.testing.assert_allclose(os_, o1[:, 0], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(pool[1:], S1, rtol=1e-12, atol=1e-13)
    assert np.all(pool[0] == 0.0)


ALL_PINS = [pin_reduces_to_gdn, pin_chunkwise_form, pin_one_hot_rows, pin_beta_zero,
            pin_orthonormal_overwrite, pin_split_varlen_and_step]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin(kda, pin):
    pin(kda)


def test_chunked_form_rejects_a_wrong_gate_sum():
    # the chunkwise pin is live: feeding it the gates of the next token breaks it
    q, k, v, g, beta, S0 = _inputs(2, 1, 80, 1, 8, 8, spread=2.0)
    o, S = K.forward(q, k, v, g, beta, 0.5, initial_state=S0)
    f64 = lambda x: x[0, :, 0].astype(np.float64)
    oc, _ = K.chunked_form(f64(q), f64(k), f64(v), f64(beta), np.roll(f64(g), 1, axis=0), S0[0, 0],
                           0.5, 64)
    assert np.max(np.abs(oc - o[0, :, 0])) > 1e-4


MUTANTS = {
    "read_before_decay": (
        "        for (int j = 0; j < Dv; ++j) S[(size_t)i * Dv + j] *= alpha;\n    }\n    for (int j = 0; j < Dv; ++j) u[j] = 0.0;",
        "        (void)alpha;\n    }\n    for (int j = 0; j < Dv; ++j) u[j] = 0.0;"),
    "gate_of_another_dim": ("const double alpha = exp((double)g[i]);",
                            "const double alpha = exp((double)g[Dk - 1 - i]);"),
    "gate_of_dim_zero": ("const double alpha = exp((double)g[i]);",
                         "const double alpha = exp((double)g[0]);"),
    "beta_dropped": ("const double bk = beta * (double)k[i];", "const double bk = (double)k[i];"),
    "correction_sign": ("((double)v[j] - u[j])", "((double)v[j] + u[j])"),
    "scale_dropped": ("for (int j = 0; j < Dv; ++j) o[j] *= scale;",
                      "for (int j = 0; j < Dv; ++j) o[j] *= 1.0;"),
    "decay_base_two": ("const double alpha = exp((double)g[i]);",
                       "const double alpha = exp2((double)g[i]);"),
    "read_before_write": (
        "    for (int j = 0; j < Dv; ++j) o[j] = 0.0;\n    for (int i = 0; i < Dk; ++i) {\n        const double qi",
        "    for (int j = 0; j < Dv; ++j) o[j] = 0.0;\n    for (int i = 0; i < Dk; ++i) {\n        const double qi"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    with open(K.SOURCE) as f:
        src = f.read()
    assert src.count(old) == 1, "mutation anchor not found: %s" % name
    new_src = src.replace(old, new)
    if name == "read_before_decay":
        # decay after the read instead: scale the rows behind the read loop
        new_src = new_src.replace(
            "    for (int i = 0; i < Dk; ++i) {\n        const double bk",
            "    for (int i = 0; i < Dk; ++i) {\n        const double alpha = exp((double)g[i]);\n"
            "        for (int j = 0; j < Dv; ++j) S[(size_t)i * Dv + j] *= alpha;\n    }\n"
            "    for (int i = 0; i < Dk; ++i) {\n        const double bk", 1)
    if name == "read_before_write":
        # the query reads the state before the token's write: move the read up
        body_start = new_src.index("    for (int j = 0; j < Dv; ++j) u[j] = 0.0;")
        read_start = new_src.index("    for (int j = 0; j < Dv; ++j) o[j] = 0.0;")
        read_end = new_src.index("    for (int j = 0; j < Dv; ++j) o[j] *= scale;")
        read = new_src[read_start:read_end]
        new_src = new_src[:body_start] + read + new_src[body_start:read_start] + new_src[read_end:]
    assert new_src != src
    path = tmp_path / ("mutant_%s.c" % name)
    path.write_text(new_src)
    lib = oracle.compile_source(str(path), str(tmp_path / ("libmutant_%s.so" % name)))
    mutant = K.KdaOracle(lib)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(mutant)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, "no pin caught the planted mistake %s" % name

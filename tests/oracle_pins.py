"""Pins for the oracle: checks against what the pages and the mathematics fix.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises AssertionError when the
oracle disagrees with an independent statement of the result:

* pin_zero_gate_causal   — with g = 0 the recurrence collapses to plain causal
  linear attention, scale * ((Q K^T) masked to j <= i) V (the associativity
  (QK)V = Q(KV) of page "MiniCPM-SALA — Complete Blueprint", section "Why Not
  Just Use Linear Attention Everywhere?").
* pin_closed_form_state  — the unrolled state sum S_n = alpha^n S_0 +
  sum_i alpha^(n-i) k_i^T v_i of the same page (section "Why Linear Attention
  Loses Information", Problem 1), with a per-token decay: the weight of token t
  is exp(sum of g over the tokens after t).
* pin_decay_table        — the worked decay values that page prints
  (tests/golden/decay_table.json).
* pin_parallel_form      — brute-force parallel form with an initial state,
  o = scale*((Q K^T) .* D) V + scale*diag(exp(G)) Q S0 with D_ts =
  exp(G_t - G_s) for s <= t, G the inclusive cumulative sum of g (the decay
  matrix built from a cumulative gate sum on page "Formulas and code for
  adapting inference to GDN/KDA linear modules", section 1.2 "Chunkwise
  Formulas").
* pin_chunked_form       — the chunkwise decomposition of the same section
  (inter-chunk output through the carried state, decay-masked intra-chunk
  scores, state refresh with exp(G_last - G) weights), reduced to Simple GLA:
  no delta-rule terms, new_v = v.
* pin_split_chain        — running [0, t) then [t, T) from the returned final
  state equals one run over [0, T), exactly.
* pin_varlen_separate    — packed sequences equal separate runs; an empty
  sequence writes nothing and returns its initial state.
* pin_head_permutation   — heads are independent.
* pin_scale              — o is linear in scale, the state does not see it.
* pin_step               — the decode step equals a one-token forward on the
  same state and honours the row -> slot map.

The independent forms below are written with numpy matrix products and share
nothing with the C oracle.
"""
from __future__ import annotations

import json
import os
from decimal import Decimal

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _gates(rng, shape, mean=1.0):
    x = rng.normal(mean, 1.0, size=shape)
    return (-np.log1p(np.exp(-x))).astype(np.float32)


def _inputs(seed, B, T, H, Dk, Dv, zero_gate=False):
    rng = _rng(seed)
    q = rng.normal(size=(B, T, H, Dk)).astype(np.float32)
    k = rng.normal(size=(B, T, H, Dk)).astype(np.float32)
    v = rng.normal(size=(B, T, H, Dv)).astype(np.float32)
    g = np.zeros((B, T, H), np.float32) if zero_gate else _gates(rng, (B, T, H))
    return q, k, v, g


def _close(a, b, rtol=1e-11, atol=1e-12, what=""):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    err = np.max(np.abs(a - b)) if a.size else 0.0
    ref = np.max(np.abs(b)) if b.size else 0.0
    assert err <= atol + rtol * ref, "%s: max err %.3e vs ref %.3e" % (what, err, ref)


def pin_zero_gate_causal(orc):
    B, T, H, Dk, Dv, scale = 2, 37, 3, 5, 7, 0.3
    q, k, v, g = _inputs(1, B, T, H, Dk, Dv, zero_gate=True)
    o, S = orc.forward(q, k, v, g, scale)
    mask = np.tril(np.ones((T, T)))
    for b in range(B):
        for h in range(H):
            Q, K, V = (x[b, :, h].astype(np.float64) for x in (q, k, v))
            ref = scale * ((Q @ K.T) * mask) @ V
            _close(o[b, :, h], ref, what="zero-gate o")
            _close(S[b, h], K.T @ V, what="zero-gate state")


def pin_closed_form_state(orc):
    B, T, H, Dk, Dv, scale = 2, 41, 2, 6, 4, 0.5
    q, k, v, g = _inputs(2, B, T, H, Dk, Dv)
    S0 = _rng(3).normal(size=(B, H, Dk, Dv))
    _, S = orc.forward(q, k, v, g, scale, initial_state=S0)
    for b in range(B):
        for h in range(H):
            gg = g[b, :, h].astype(np.float64)
            ref = np.exp(gg.sum()) * S0[b, h]
            for t in range(T):
                w = np.exp(gg[t + 1:].sum())
                ref = ref + w * np.outer(k[b, t, h].astype(np.float64), v[b, t, h].astype(np.float64))
            _close(S[b, h], ref, what="closed-form state")


def _tolerance(printed: str) -> float:
    return 0.5 * 10.0 ** Decimal(printed).as_tuple().exponent


def pin_decay_table(orc):
    with open(os.path.join(GOLDEN, "decay_table.json")) as f:
        table = json.load(f)
    heads = table["heads"]
    steps = sorted({int(n) for h in heads for n in h["values"]})
    T, H = steps[-1] + 1, len(heads)
    # One-hot token at t=0: k = e_0, v = e_1; nothing written afterwards.
    q = np.zeros((1, T, H, 2), np.float32)
    q[..., 0] = 1.0
    k = np.zeros((1, T, H, 2), np.float32)
    v = np.zeros((1, T, H, 2), np.float32)
    k[0, 0, :, 0] = 1.0
    v[0, 0, :, 1] = 1.0
    g = np.zeros((1, T, H), np.float32)
    for h, head in enumerate(heads):
        g[0, :, h] = np.float32(head["g"])
    o, _ = orc.forward(q, k, v, g, 1.0)
    for h, head in enumerate(heads):
        for n, printed in head["values"].items():
            got = o[0, int(n), h, 1]
            if Decimal(printed) == 0:
                assert 0.0 <= got < table["zero_bound"], (head["label"], n, got)
            else:
                want = float(Decimal(printed))
                assert abs(got - want) <= _tolerance(printed), (head["label"], n, got, printed)
        assert np.all(o[0, :, h, 0] == 0.0)


def parallel_form(Q, K, V, gg, S0, scale):
    T = Q.shape[0]
    G = np.cumsum(gg)
    mask = np.tril(np.ones((T, T), bool))
    D = np.where(mask, np.exp(np.where(mask, G[:, None] - G[None, :], 0.0)), 0.0)
    return scale * ((Q @ K.T) * D) @ V + scale * np.exp(G)[:, None] * (Q @ S0)


def pin_parallel_form(orc):
    B, T, H, Dk, Dv, scale = 1, 90, 3, 8, 5, 0.25
    q, k, v, g = _inputs(4, B, T, H, Dk, Dv)
    S0 = _rng(5).normal(size=(B, H, Dk, Dv))
    o, _ = orc.forward(q, k, v, g, scale, initial_state=S0)
    for h in range(H):
        Q, K, V = (x[0, :, h].astype(np.float64) for x in (q, k, v))
        ref = parallel_form(Q, K, V, g[0, :, h].astype(np.float64), S0[0, h], scale)
        _close(o[0, :, h], ref, what="parallel form")


def chunked_form(Q, K, V, gg, S0, scale, C):
    """Chunkwise Simple GLA, one head: returns (o, final state)."""
    T = Q.shape[0]
    S = S0.copy()
    out = np.zeros((T, V.shape[1]))
    for s in range(0, T, C):
        e = min(T, s + C)
        q, k, v = Q[s:e], K[s:e], V[s:e]
        G = np.cumsum(gg[s:e])
        n = e - s
        inter = (q * np.exp(G)[:, None]) @ S
        mask = np.tril(np.ones((n, n), bool))
        gam = np.where(mask, np.exp(np.where(mask, G[:, None] - G[None, :], 0.0)), 0.0)
        intra = ((q @ k.T) * gam) @ v
        out[s:e] = scale * (inter + intra)
        S = np.exp(G[-1]) * S + (k * np.exp(G[-1] - G)[:, None]).T @ v
    return out, S


def pin_chunked_form(orc):
    B, T, H, Dk, Dv, scale = 1, 150, 2, 6, 9, 0.4
    q, k, v, g = _inputs(6, B, T, H, Dk, Dv)
    S0 = _rng(7).normal(size=(B, H, Dk, Dv))
    o, S = orc.forward(q, k, v, g, scale, initial_state=S0)
    for h in range(H):
        Q, K, V = (x[0, :, h].astype(np.float64) for x in (q, k, v))
        for C in (1, 16, 64):
            ro, rS = chunked_form(Q, K, V, g[0, :, h].astype(np.float64), S0[0, h], scale, C)
            _close(o[0, :, h], ro, what="chunked o C=%d" % C)
            _close(S[0, h], rS, what="chunked state C=%d" % C)


def pin_split_chain(orc):
    B, T, H, Dk, Dv, scale = 2, 77, 2, 4, 6, 0.7
    q, k, v, g = _inputs(8, B, T, H, Dk, Dv)
    S0 = _rng(9).normal(size=(B, H, Dk, Dv))
    o, S = orc.forward(q, k, v, g, scale, initial_state=S0)
    for t in (1, 30, 64, T - 1):
        o1, S1 = orc.forward(q[:, :t], k[:, :t], v[:, :t], g[:, :t], scale, initial_state=S0)
        o2, S2 = orc.forward(q[:, t:], k[:, t:], v[:, t:], g[:, t:], scale, initial_state=S1)
        assert np.array_equal(np.concatenate([o1, o2], axis=1), o), t
        assert np.array_equal(S2, S), t


def pin_varlen_separate(orc):
    lengths = [5, 0, 33, 1, 64, 12]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    T, H, Dk, Dv, scale = int(cu[-1]), 3, 4, 5, 0.6
    q, k, v, g = _inputs(10, 1, T, H, Dk, Dv)
    S0 = _rng(11).normal(size=(len(lengths), H, Dk, Dv))
    o, S = orc.forward(q, k, v, g, scale, initial_state=S0, cu_seqlens=cu)
    for n, L in enumerate(lengths):
        a, b = cu[n], cu[n + 1]
        if L == 0:
            assert np.array_equal(S[n], S0[n])
            continue
        on, Sn = orc.forward(q[:, a:b], k[:, a:b], v[:, a:b], g[:, a:b], scale,
                             initial_state=S0[n:n + 1])
        assert np.array_equal(o[:, a:b], on), n
        assert np.array_equal(S[n], Sn[0]), n


def pin_head_permutation(orc):
    B, T, H, Dk, Dv, scale = 1, 40, 5, 4, 4, 0.5
    q, k, v, g = _inputs(12, B, T, H, Dk, Dv)
    S0 = _rng(13).normal(size=(B, H, Dk, Dv))
    perm = np.array([3, 0, 4, 1, 2])
    o, S = orc.forward(q, k, v, g, scale, initial_state=S0)
    op, Sp = orc.forward(q[:, :, perm], k[:, :, perm], v[:, :, perm], g[:, :, perm], scale,
                         initial_state=S0[:, perm])
    assert np.array_equal(op, o[:, :, perm])
    assert np.array_equal(Sp, S[:, perm])


def pin_scale(orc):
    B, T, H, Dk, Dv = 1, 30, 2, 3, 5
    q, k, v, g = _inputs(14, B, T, H, Dk, Dv)
    o1, S1 = orc.forward(q, k, v, g, 0.5)
    o2, S2 = orc.forward(q, k, v, g, 2.0)
    _close(o2, 4.0 * o1, what="scale linearity")
    assert np.array_equal(S1, S2)


def pin_step(orc):
    N, H, Dk, Dv, scale, slots = 4, 3, 5, 6, 0.3, 7
    rng = _rng(15)
    state = rng.normal(size=(slots, H, Dk, Dv))
    idx = np.array([6, 2, 0, 5], np.int32)
    for i in range(3):
        q = rng.normal(size=(N, H, Dk)).astype(np.float32)
        k = rng.normal(size=(N, H, Dk)).astype(np.float32)
        v = rng.normal(size=(N, H, Dv)).astype(np.float32)
        g = _gates(rng, (N, H))
        before = state.copy()
        o = orc.step(q, k, v, g, state, scale, state_indices=idx)
        untouched = [s for s in range(slots) if s not in idx]
        assert np.array_equal(state[untouched], before[untouched])
        for r in range(N):
            of, Sf = orc.forward(q[r][None, None], k[r][None, None], v[r][None, None],
                                 g[r][None, None], scale, initial_state=before[idx[r]][None])
            assert np.array_equal(o[r], of[0, 0]), (i, r)
            assert np.array_equal(state[idx[r]], Sf[0]), (i, r)


ALL_PINS = [pin_zero_gate_causal, pin_closed_form_state, pin_decay_table, pin_parallel_form,
            pin_chunked_form, pin_split_chain, pin_varlen_separate, pin_head_permutation,
            pin_scale, pin_step]

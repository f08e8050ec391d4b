"""Oracle for the decode step with bf16 state storage — test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module; the product package never does, and the
two share no code.

What it computes (page "MiniCPM-SALA — Complete Blueprint", section
"B2 lightning-attn (Simple GLA)": the state pool holds each request's
[32, 128, 128] state in bf16, loaded for the step and saved back; the step
itself is the recurrence): for each row's state S (bf16 values),

    S' = exp(g) * S + k^T v          (the decay, then the rank-1 update)
    o  = scale * q S'
    S <- bf16(S')                    (stored back, round to nearest even)

Reading where the page is silent: the query
reads the updated state before it is rounded for storage, as a kernel that
keeps the state in registers between the update and the store does. The
arithmetic is fp64 except that one rounding.

``steps`` also returns, per state and output element, a bound on how far an
implementation whose values before the rounding are off by at most tie_eta
times (|exp(g) S| + |k v|) can be from these values after each step: a value
that close to a midpoint between two bf16 numbers may round the other way,
and a state that already differs carries the difference (times the decay)
into the next rounding. The bound follows that recursion exactly.
"""
from __future__ import annotations

import numpy as np

from oracle.prologue import bf16_spacing, near_rounding_tie, round_to_bf16


def step(q, k, v, g, S, scale):
    """One step for a batch of states. q, k [n, Dk]; v [n, Dv]; g [n];
    S [n, Dk, Dv] (bf16 values, updated in place). Returns o [n, Dv]."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    a = np.exp(np.asarray(g, np.float64))[:, None, None]
    Sp = a * S + k[:, :, None] * v[:, None, :]
    o = scale * np.einsum("ni,nij->nj", q, Sp)
    S[...] = round_to_bf16(Sp)
    return o


def steps(q, k, v, g, S, scale, tie_eta=None):
    """Several successive steps. q, k [steps, n, Dk]; v [steps, n, Dv];
    g [steps, n]; S [n, Dk, Dv] (updated in place). Returns the outputs
    [steps, n, Dv], and with ``tie_eta`` also the bounds of the outputs
    [steps, n, Dv] and of the final state [n, Dk, Dv]."""
    outs, oa = [], []
    A = np.zeros_like(S) if tie_eta is not None else None
    for t in range(len(q)):
        if A is None:
            outs.append(step(q[t], k[t], v[t], g[t], S, scale))
            continue
        qt = np.asarray(q[t], np.float64)
        a = np.exp(np.asarray(g[t], np.float64))[:, None, None]
        aS = a * S
        kv = np.asarray(k[t], np.float64)[:, :, None] * np.asarray(v[t], np.float64)[:, None, :]
        Sp = aS + kv
        carried = a * A                       # difference carried from earlier steps
        outs.append(scale * np.einsum("ni,nij->nj", qt, Sp))
        oa.append(scale * np.einsum("ni,nij->nj", np.abs(qt), carried))
        band = tie_eta * (np.abs(aS) + np.abs(kv)) + carried
        flip = near_rounding_tie(Sp, band)
        S[...] = round_to_bf16(Sp)
        # where no midpoint lies within the band both sides round alike and
        # the difference is gone; elsewhere it is at most the carried one plus
        # one spacing
        A = np.where(flip, carried + bf16_spacing(2.0 * np.maximum(np.abs(Sp), np.abs(S))), 0.0)
    if A is None:
        return np.stack(outs)
    return np.stack(outs), np.stack(oa), A

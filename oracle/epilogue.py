"""Oracle for the output epilogue of a lightning layer — test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module; the product package never does, and the
two share no code.

What it computes (page "MiniCPM-SALA — Complete Blueprint", section
"B2 lightning-attn (Simple GLA)", the step "Output Norm + Gate + Projection",
without the projection): for every token, the attention output of all heads,
concatenated to one row of width H * Dv (4096 on the page), goes through

1. RMSNorm over the whole row with one weight vector w of that width:
   y = o / sqrt(mean(o^2) + eps) * w;
2. the gate z = sigmoid(zlogit), where zlogit is the gate projection of the
   layer input (an input here);
3. out = y * z, elementwise.

Readings where the page is silent: with bf16
tensors every step's result is stored in bf16 (y, the gate and the product),
the dtype the module outputs have; with fp32 tensors nothing is rounded; eps
is an argument.

Everything is fp64 except those bf16 roundings, written out below.
"""
from __future__ import annotations

import numpy as np

from oracle.prologue import bf16_spacing, near_rounding_tie, round_to_bf16


def row_rms_norm(o, w, eps):
    """RMSNorm over the last axis (the concatenated heads) in fp64."""
    o = np.asarray(o, dtype=np.float64)
    ms = np.mean(o * o, axis=-1, keepdims=True)
    return o / np.sqrt(ms + eps) * np.asarray(w, dtype=np.float64)


def sigmoid(x):
    """1 / (1 + exp(-x)) in fp64, written so that neither branch overflows."""
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def out_norm_gate(o, zlogit, w, eps=1e-6, bf16=True, tie_eta=None):
    """The epilogue of rows o [..., width] with gate logits of the same shape.

    Returns the output (fp64 values; bf16 values when ``bf16``). With
    ``tie_eta`` (bf16 only) it also returns per element the largest change a
    different decision at any of the three roundings could make, for an
    implementation whose values before rounding are off by at most tie_eta of
    their size: a rounding input within that distance of a midpoint between
    two bf16 numbers may go either way."""
    y_pre = row_rms_norm(o, w, eps)
    s_pre = sigmoid(zlogit)
    if not bf16:
        return y_pre * s_pre
    y = round_to_bf16(y_pre)
    s = round_to_bf16(s_pre)
    p = y * s
    out = round_to_bf16(p)
    if tie_eta is None:
        return out
    so = bf16_spacing(2.0 * np.maximum(np.abs(out), np.abs(p)))
    fy = near_rounding_tie(y_pre, tie_eta * np.abs(y_pre))
    fs = near_rounding_tie(s_pre, tie_eta * np.abs(s_pre))
    fo = near_rounding_tie(p, tie_eta * np.abs(p))
    bound = (np.where(fy, bf16_spacing(2.0 * y) * np.abs(s) + so, 0.0)
             + np.where(fs, bf16_spacing(2.0 * s) * np.abs(y) + so, 0.0)
             + np.where(fo, so, 0.0))
    return out, bound

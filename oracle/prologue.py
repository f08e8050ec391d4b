"""Oracle for the q/k prologue of a lightning layer — test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module; the product package never does, and the
two share no code.

What it computes (page "MiniCPM-SALA — Complete Blueprint", section
"B2 lightning-attn (Simple GLA)", the two steps between the QKV projection and
the recurrence): each head's 128-vector of q and of k goes through

1. RMSNorm with one weight vector w of length Dk shared by all heads:
   y = x / sqrt(mean(x^2) + eps) * w, stored in bf16 (the dtype q and k
   arrive in);
2. RoPE with base theta = 10000 at the token's position, computed on the
   fp32 values and stored back to bf16 (the page's ``q.float()`` ...
   ``.bf16()``).

Readings where the page is silent:
* RoPE pairs dimension i with i + Dk/2 ("rotate half"), rotating the pair by
  angle pos * theta^(-2i/Dk), i < Dk/2, in the positive sense:
  (a, b) -> (a cos - b sin, b cos + a sin);
* the angle is the exact product pos * theta^(-2i/Dk) (here in fp64);
* eps is an argument (1e-6 in the workloads);
* positions are given per token; a sequence without them counts from 0.

Everything is fp64 except the two bf16 roundings the page prescribes, which
are written out below (round to fp32, then round to nearest even at bf16).
"""
from __future__ import annotations

import numpy as np


def round_to_bf16(x):
    """Round fp64 values to the nearest bf16 (ties to even), returned as fp64.

    The value is first rounded to fp32 (numpy's cast rounds to nearest even),
    then the fp32 bit pattern to its upper 16 bits, nearest even. NaN stays
    NaN; values beyond the bf16 range become +-inf."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    nan = np.isnan(f)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    out = r.astype(np.uint32).view(np.float32).astype(np.float64)
    out[nan] = np.nan
    return out


def rms_norm(x, w, eps):
    """RMSNorm over the last axis in fp64: x / sqrt(mean(x^2) + eps) * w."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(w, dtype=np.float64)


def rope_angles(pos, d, theta):
    """Angles [len(pos), d/2]: pos * theta^(-2i/d) for i = 0 .. d/2 - 1, fp64."""
    i = np.arange(d // 2, dtype=np.float64)
    inv_freq = np.power(float(theta), -2.0 * i / d)
    return np.asarray(pos, dtype=np.float64)[:, None] * inv_freq[None, :]


def rope_rotate_half(x, pos, theta):
    """Rotate pairs (i, i + d/2) of x [..., n_tok, H, d] by their angles.

    ``pos`` has one position per token (axis -3 of x)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    ang = rope_angles(pos, d, theta)            # [n_tok, d/2]
    c = np.cos(ang)[:, None, :]                 # broadcast over heads
    s = np.sin(ang)[:, None, :]
    a, b = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def sequence_positions(n_tok, cu_seqlens=None):
    """Default positions: the index of each token inside its own sequence."""
    if cu_seqlens is None:
        return np.arange(n_tok, dtype=np.int64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    pos = np.zeros(n_tok, dtype=np.int64)
    for n in range(len(cu) - 1):
        pos[cu[n]:cu[n + 1]] = np.arange(cu[n + 1] - cu[n])
    return pos


def bf16_spacing(x):
    """Distance between consecutive bf16 numbers at |x| (8 significant bits)."""
    a = np.maximum(np.abs(np.asarray(x, dtype=np.float64)), np.finfo(np.float32).tiny)
    return np.ldexp(1.0, np.floor(np.log2(a)).astype(np.int64) - 7)


def near_rounding_tie(v, band):
    """True where moving v by up to ``band`` (>= 0, absolute) either way
    changes its bf16 rounding, i.e. v lies within band of a midpoint between
    two bf16 numbers. The band must exceed the fp32 spacing at v (the rounding
    goes through fp32), which every band used here does by far."""
    v = np.asarray(v, dtype=np.float64)
    return round_to_bf16(v + band) != round_to_bf16(v - band)


def qk_prologue(x, w, pos, theta=10000.0, eps=1e-6, tie_eta=None):
    """The prologue of one of q or k.

    x: [B, T, H, d] raw values (bf16 values as floats); w: [d]; pos: [B*T]
    positions in token order (the rows of x flattened over B and T).
    Returns the bf16 values (as fp64) that the recurrence consumes.

    With ``tie_eta`` it also returns, per element, the largest change that a
    different decision at either bf16 rounding could make, for an
    implementation whose values before rounding are off by at most tie_eta
    times the size of what they are made from: tie_eta * |y| for the RMSNorm
    output y, tie_eta * (|y_i| + |y_partner|) for a RoPE output (its angle and
    sine/cosine errors scale with the pair it turns, even when the result is
    near zero). An element within that distance of a midpoint may round the
    other way: the bound is one spacing of the result for its own rounding,
    plus, where the RMSNorm output of the element or of its RoPE partner was
    near a midpoint, that output's spacing and one more spacing of the
    result. Elsewhere it is 0."""
    x = np.asarray(x, dtype=np.float64)
    B, T, H, d = x.shape
    y_pre = rms_norm(x, w, eps)
    y = round_to_bf16(y_pre)
    y = y.reshape(B * T, H, d)
    z_pre = rope_rotate_half(y, np.asarray(pos).reshape(B * T), theta)
    z = round_to_bf16(z_pre)
    if tie_eta is None:
        return z.reshape(B, T, H, d)
    half = d // 2
    swap = lambda a: np.concatenate([a[..., half:], a[..., :half]], axis=-1)
    y_pre = y_pre.reshape(B * T, H, d)
    dy = np.where(near_rounding_tie(y_pre, tie_eta * np.abs(y_pre)), bf16_spacing(2.0 * y), 0.0)
    dy_pair = dy + swap(dy)
    sz = bf16_spacing(2.0 * np.maximum(np.abs(z), np.abs(z_pre)))
    band = tie_eta * (np.abs(y) + np.abs(swap(y)))
    bound = np.where(near_rounding_tie(z_pre, band), sz, 0.0)
    bound = bound + np.where(dy_pair > 0, dy_pair + sz, 0.0)
    return z.reshape(B, T, H, d), bound.reshape(B, T, H, d)

"""Oracle for the gated delta rule with a per-key-dim gate (KDA) — test
infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module; the product package never does, and the
two share no code. The recurrence lives in ``kda_oracle.c`` (plain C, fp64,
one token at a time; its header states the definition and the reading of the
page); this module builds it, marshals numpy arrays, and writes out the
chunkwise form (``chunked_form``) that the CPU pins compare with the
recurrence.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from oracle import compile_source, default_threads

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "kda_oracle.c")
LIBRARY = os.path.join(_HERE, "libkda_oracle.so")


def build(force: bool = True) -> str:
    if force or not os.path.exists(LIBRARY):
        compile_source(SOURCE, LIBRARY)
    return LIBRARY


def _f32(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


class KdaOracle:
    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        vp, ci = ctypes.c_void_p, ctypes.c_int
        lib.kda_oracle_forward.argtypes = [vp] * 9 + [ci] * 5 + [ctypes.c_double, ci]
        lib.kda_oracle_forward.restype = ci
        lib.kda_oracle_step.argtypes = [vp] * 8 + [ci] * 4 + [ctypes.c_double, ci]
        lib.kda_oracle_step.restype = ci
        self.lib = lib

    def forward(self, q, k, v, g, beta, scale, initial_state=None, cu_seqlens=None,
                nthreads=None):
        """q, k, g [B,T,H,Dk]; v [B,T,H,Dv]; beta [B,T,H]; initial_state
        [N,H,Dk,Dv] (fp64) or None; cu_seqlens [N+1] with B = 1 for packed
        sequences. Returns (o [B,T,H,Dv] fp64, final state [N,H,Dk,Dv] fp64)."""
        q, k, v, g, beta = (_f32(x) for x in (q, k, v, g, beta))
        B, T, H, Dk = q.shape
        Dv = v.shape[-1]
        if g.shape != q.shape:
            raise ValueError("g must have the shape of q and k (one gate per key dim)")
        cu = None
        N = B
        if cu_seqlens is not None:
            if B != 1:
                raise ValueError("packed sequences take B = 1")
            cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
            N = len(cu) - 1
        S0 = None
        if initial_state is not None:
            S0 = np.ascontiguousarray(np.asarray(initial_state, dtype=np.float64))
        o = np.zeros((B, T, H, Dv), dtype=np.float64)
        S = np.zeros((N, H, Dk, Dv), dtype=np.float64)
        rc = self.lib.kda_oracle_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0),
                                         _ptr(o), _ptr(S), _ptr(cu), N, T, H, Dk, Dv,
                                         float(scale), nthreads or default_threads())
        if rc != 0:
            raise RuntimeError("kda_oracle_forward failed")
        return o, S

    def step(self, q, k, v, g, beta, state, scale, state_indices=None, nthreads=None):
        """One decode token per row; q, k, g [N,H,Dk]; v [N,H,Dv]; beta [N,H];
        state [slots,H,Dk,Dv] fp64 C-contiguous, updated in place. Returns o
        [N,H,Dv] fp64."""
        q, k, v, g, beta = (_f32(x) for x in (q, k, v, g, beta))
        if state.dtype != np.float64 or not state.flags.c_contiguous:
            raise ValueError("state must be a C-contiguous float64 array")
        N, H, Dk = q.shape
        Dv = v.shape[-1]
        idx = None if state_indices is None else np.ascontiguousarray(
            np.asarray(state_indices, dtype=np.int32))
        o = np.zeros((N, H, Dv), dtype=np.float64)
        rc = self.lib.kda_oracle_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state),
                                      _ptr(idx), _ptr(o), N, H, Dk, Dv, float(scale),
                                      nthreads or default_threads())
        if rc != 0:
            raise RuntimeError("kda_oracle_step failed")
        return o


_default = None


def _oracle():
    global _default
    if _default is None:
        build(force=False)
        _default = KdaOracle(LIBRARY)
    return _default


def forward(*a, **kw):
    return _oracle().forward(*a, **kw)


def step(*a, **kw):
    return _oracle().step(*a, **kw)


def chunked_form(Q, K, V, beta, g, S0, scale, C):
    """The page's chunkwise formulas (section 1.2) with the gate made a vector
    over the key dims (section 2.1's KDA branch), for one head, in fp64.
    Inside each chunk, with G[a][d] the inclusive cumulative sum of g over the
    chunk's tokens, for key dim d,

        M[a][b]  = sum_d K[a][d] K[b][d] exp(G[a][d] - G[b][d])     (a > b)
        T        = (I + strictly_lower(diag(beta) M))^-1             (UT transform)
        W        = T (diag(beta) K * exp(G)),   U = T diag(beta) V
        new_v    = U - W S
        L[a][b]  = sum_d Q[a][d] K[b][d] exp(G[a][d] - G[b][d])     (a >= b, else 0)
        O        = scale * ((Q * exp(G)) S + L new_v)
        S        = diag(exp(G_last)) S + (K * exp(G_last - G))^T new_v

    With g the same in every key dim this is the scalar-gate form (the decay
    factors leave the sums over d). The pairwise factors are formed as
    exp(G[a][d] - G[b][d]) directly, never as a product of exp(G[a]) and
    exp(-G[b]). T is solved with numpy (the page builds it row by row by
    forward substitution: the same matrix). Q, K, g [L, Dk]; V [L, Dv];
    beta [L]."""
    L, Dk = Q.shape
    S = np.array(S0, dtype=np.float64)
    O = np.zeros((L, V.shape[1]))
    for c0 in range(0, L, C):
        sl = slice(c0, min(L, c0 + C))
        q, k, v = Q[sl], K[sl], V[sl]
        b = beta[sl]
        G = np.cumsum(g[sl], axis=0)
        n = len(b)
        dec = np.exp(G[:, None, :] - G[None, :, :])          # [a, b, d]
        M = np.einsum("ad,bd,abd->ab", k, k, dec)
        Lq = np.tril(np.einsum("ad,bd,abd->ab", q, k, dec))
        A = np.tril(b[:, None] * M, -1)
        Tm = np.linalg.solve(np.eye(n) + A, np.eye(n))
        W = Tm @ ((b[:, None] * k) * np.exp(G))
        U = Tm @ (b[:, None] * v)
        new_v = U - W @ S
        O[sl] = scale * ((q * np.exp(G)) @ S + Lq @ new_v)
        S = np.exp(G[-1])[:, None] * S + (k * np.exp(G[-1] - G)).T @ new_v
    return O, S

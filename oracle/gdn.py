"""Oracle for the gated delta rule (GDN) — test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module; the product package never does, and the
two share no code. The recurrence lives in ``gdn_oracle.c`` (plain C, fp64,
one token at a time; its header states the definition and the reading of the
page); this module builds it, marshals numpy arrays, and also writes out the
page's chunkwise form (``chunked_form``), which the CPU pins compare with the
recurrence.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from oracle import compile_source, default_threads

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "gdn_oracle.c")
LIBRARY = os.path.join(_HERE, "libgdn_oracle.so")


def build(force: bool = True) -> str:
    if force or not os.path.exists(LIBRARY):
        compile_source(SOURCE, LIBRARY)
    return LIBRARY


def _f32(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


class GdnOracle:
    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        vp, ci = ctypes.c_void_p, ctypes.c_int
        lib.gdn_oracle_forward.argtypes = [vp] * 9 + [ci] * 5 + [ctypes.c_double, ci]
        lib.gdn_oracle_forward.restype = ci
        lib.gdn_oracle_step.argtypes = [vp] * 8 + [ci] * 4 + [ctypes.c_double, ci]
        lib.gdn_oracle_step.restype = ci
        self.lib = lib

    def forward(self, q, k, v, g, beta, scale, initial_state=None, cu_seqlens=None,
                nthreads=None):
        """q, k [B,T,H,Dk]; v [B,T,H,Dv]; g, beta [B,T,H]; initial_state
        [N,H,Dk,Dv] (fp64) or None. Returns (o fp64, final state fp64)."""
        q, k, v, g, beta = (_f32(x) for x in (q, k, v, g, beta))
        B, T, H, Dk = q.shape
        Dv = v.shape[-1]
        cu = None
        N = B
        if cu_seqlens is not None:
            cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
            N = len(cu) - 1
        S0 = None
        if initial_state is not None:
            S0 = np.ascontiguousarray(np.asarray(initial_state, dtype=np.float64))
        o = np.zeros((B, T, H, Dv), dtype=np.float64)
        S = np.zeros((N, H, Dk, Dv), dtype=np.float64)
        rc = self.lib.gdn_oracle_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0),
                                         _ptr(o), _ptr(S), _ptr(cu), N, T, H, Dk, Dv,
                                         float(scale), nthreads or default_threads())
        if rc != 0:
            raise RuntimeError("gdn_oracle_forward failed")
        return o, S

    def step(self, q, k, v, g, beta, state, scale, state_indices=None, nthreads=None):
        """One decode token per row; state [slots,H,Dk,Dv] fp64 C-contiguous,
        updated in place. Returns o [N,H,Dv] fp64."""
        q, k, v, g, beta = (_f32(x) for x in (q, k, v, g, beta))
        if state.dtype != np.float64 or not state.flags.c_contiguous:
            raise ValueError("state must be a C-contiguous float64 array")
        N, H, Dk = q.shape
        Dv = v.shape[-1]
        idx = None if state_indices is None else np.ascontiguousarray(
            np.asarray(state_indices, dtype=np.int32))
        o = np.zeros((N, H, Dv), dtype=np.float64)
        rc = self.lib.gdn_oracle_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state),
                                      _ptr(idx), _ptr(o), N, H, Dk, Dv, float(scale),
                                      nthreads or default_threads())
        if rc != 0:
            raise RuntimeError("gdn_oracle_step failed")
        return o


_default = None


def _oracle():
    global _default
    if _default is None:
        build(force=False)
        _default = GdnOracle(LIBRARY)
    return _default


def forward(*a, **kw):
    return _oracle().forward(*a, **kw)


def step(*a, **kw):
    return _oracle().step(*a, **kw)


def chunked_form(Q, K, V, beta, g, S0, scale, C):
    """The page's chunkwise formulas (section 1.2) for one head, in fp64:
    inside each chunk, with G the inclusive cumulative sum of g and
    Gamma[a][b] = exp(G_a - G_b) for a >= b (else 0),

        T     = (I + strictly_lower(diag(beta) K K^T * Gamma))^-1   (UT transform)
        W     = T (diag(beta) K * exp(G)),   U = T diag(beta) V
        new_v = U - W S
        O     = scale * ((Q * exp(G)) S + lower(Q K^T * Gamma) new_v)
        S     = exp(G_last) S + (K * exp(G_last - G))^T new_v

    T is solved here with numpy instead of the page's row-by-row forward
    substitution (the same matrix). Q, K [L, Dk]; V [L, Dv]; beta, g [L]."""
    L, Dk = Q.shape
    S = np.array(S0, dtype=np.float64)
    O = np.zeros((L, V.shape[1]))
    for c0 in range(0, L, C):
        sl = slice(c0, min(L, c0 + C))
        q, k, v = Q[sl], K[sl], V[sl]
        b, gg = beta[sl], g[sl]
        n = len(gg)
        G = np.cumsum(gg)
        Gam = np.tril(np.exp(G[:, None] - G[None, :]))
        A = np.tril((b[:, None] * k) @ k.T * Gam, -1)
        Tm = np.linalg.solve(np.eye(n) + A, np.eye(n))
        W = Tm @ ((b[:, None] * k) * np.exp(G)[:, None])
        U = Tm @ (b[:, None] * v)
        new_v = U - W @ S
        O[sl] = scale * ((q * np.exp(G)[:, None]) @ S + np.tril(q @ k.T * Gam) @ new_v)
        S = np.exp(G[-1]) * S + (k * np.exp(G[-1] - G)[:, None]).T @ new_v
    return O, S

"""Oracle for Simple Gated Linear Attention — test infrastructure only.

This package is the plain, slow CPU definition of Simple GLA that the GPU
library is checked against. Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import it; the product package never does,
and the two share no code. The arithmetic lives in ``sgla_oracle.c`` (plain C,
fp64, one token at a time); this module only builds it with gcc, marshals numpy
arrays and calls it.

Definition followed (page "MiniCPM-SALA — Complete Blueprint", section
"B2 lightning-attn (Simple GLA)"): per sequence and head, for each token in
order, decay the state by exp(g), add the outer product k^T v, then read
o = scale * q @ S. The state after the last token is the final state.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "sgla_oracle.c")
LIBRARY = os.path.join(_HERE, "libsgla_oracle.so")


def compile_source(src: str, out: str) -> str:
    """gcc -O3 a C oracle source into a shared library (atomic replace)."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.check_call(
        ["gcc", "-O3", "-std=c11", "-fPIC", "-shared", "-fopenmp", src, "-o", tmp, "-lm"]
    )
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile ``sgla_oracle.c`` into ``oracle/libsgla_oracle.so`` (and the
    delta-rule oracles, ``gdn_oracle.c`` and ``kda_oracle.c``, beside it)."""
    if force or not os.path.exists(LIBRARY):
        compile_source(SOURCE, LIBRARY)
    for name in ("gdn_oracle", "kda_oracle"):
        src = os.path.join(_HERE, name + ".c")
        lib = os.path.join(_HERE, "lib%s.so" % name)
        if force or not os.path.exists(lib):
            compile_source(src, lib)
    return LIBRARY


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _f32(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


class Oracle:
    """ctypes binding of one compiled oracle library."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        vp = ctypes.c_void_p
        ci = ctypes.c_int
        lib.sgla_oracle_forward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci,
                                            ctypes.c_double, ci]
        lib.sgla_oracle_forward.restype = ci
        lib.sgla_oracle_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci,
                                         ctypes.c_double, ci]
        lib.sgla_oracle_step.restype = ci
        self.lib = lib
        self.path = path

    def forward(self, q, k, v, g, scale, initial_state=None, cu_seqlens=None, nthreads=None):
        """Run the recurrence.

        q, k: [B, T, H, Dk]; v: [B, T, H, Dv]; g: [B, T, H] (values exactly
        representable in fp32; upcast bf16 before the call).
        With ``cu_seqlens`` ([N+1] int64) B must be 1 and the N sequences are
        the slices [cu[n], cu[n+1]) of the packed token axis.
        initial_state: [N, H, Dk, Dv] (taken in fp64) or None for zeros.
        Returns (o [B, T, H, Dv] float64, final_state [N, H, Dk, Dv] float64).
        """
        q, k, v, g = _f32(q), _f32(k), _f32(v), _f32(g)
        if (q.ndim != 4 or k.shape != q.shape or v.ndim != 4 or v.shape[:3] != q.shape[:3]
                or g.shape != q.shape[:3]):
            raise ValueError("oracle.forward: inconsistent shapes")
        B, T, H, Dk = q.shape
        Dv = v.shape[3]
        cu = None
        N = B
        if cu_seqlens is not None:
            if B != 1:
                raise ValueError("oracle.forward: packed input needs B == 1")
            cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
            N = cu.shape[0] - 1
            if N < 0 or cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
                raise ValueError("oracle.forward: cu_seqlens must rise from 0 to T")
        S0 = None
        if initial_state is not None:
            S0 = np.ascontiguousarray(np.asarray(initial_state, dtype=np.float64))
            if S0.shape != (N, H, Dk, Dv):
                raise ValueError("oracle.forward: initial_state shape")
        o = np.zeros((B, T, H, Dv), dtype=np.float64)
        Sf = np.zeros((N, H, Dk, Dv), dtype=np.float64)
        rc = self.lib.sgla_oracle_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(S0), _ptr(o),
                                          _ptr(Sf), _ptr(cu), N, T, H, Dk, Dv, float(scale),
                                          nthreads or default_threads())
        if rc != 0:
            raise RuntimeError("oracle.forward failed (%d)" % rc)
        return o, Sf

    def step(self, q, k, v, g, state, scale, state_indices=None, nthreads=None):
        """One decode step. q, k [N, H, Dk]; v [N, H, Dv]; g [N, H];
        state [slots, H, Dk, Dv] float64 C-contiguous, updated IN PLACE;
        state_indices [N] (row -> slot, distinct) or None for the identity.
        Returns o [N, H, Dv] float64.
        """
        q, k, v, g = _f32(q), _f32(k), _f32(v), _f32(g)
        if not isinstance(state, np.ndarray) or state.dtype != np.float64 \
                or not state.flags.c_contiguous:
            raise ValueError("oracle.step: state must be a C-contiguous float64 array")
        N, H, Dk = q.shape
        Dv = v.shape[2]
        if state.ndim != 4 or state.shape[1:] != (H, Dk, Dv):
            raise ValueError("oracle.step: state shape")
        idx = None
        if state_indices is not None:
            idx = np.ascontiguousarray(np.asarray(state_indices, dtype=np.int32))
            if idx.shape != (N,) or np.any(idx < 0) or np.any(idx >= state.shape[0]):
                raise ValueError("oracle.step: state_indices out of range")
            if len(np.unique(idx)) != N:
                raise ValueError("oracle.step: state_indices must be distinct")
        elif state.shape[0] < N:
            raise ValueError("oracle.step: state has fewer slots than rows")
        o = np.zeros((N, H, Dv), dtype=np.float64)
        rc = self.lib.sgla_oracle_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(state),
                                       _ptr(idx), _ptr(o), N, H, Dk, Dv, float(scale),
                                       nthreads or default_threads())
        if rc != 0:
            raise RuntimeError("oracle.step failed (%d)" % rc)
        return o


_default = None


def _oracle() -> Oracle:
    global _default
    if _default is None:
        if not os.path.exists(LIBRARY):
            build(force=False)
        _default = Oracle(LIBRARY)
    return _default


def forward(q, k, v, g, scale, initial_state=None, cu_seqlens=None, nthreads=None):
    return _oracle().forward(q, k, v, g, scale, initial_state, cu_seqlens, nthreads)


def step(q, k, v, g, state, scale, state_indices=None, nthreads=None):
    return _oracle().step(q, k, v, g, state, scale, state_indices, nthreads)


forward.__doc__ = Oracle.forward.__doc__
step.__doc__ = Oracle.step.__doc__

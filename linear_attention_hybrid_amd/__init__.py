"""Simple Gated Linear Attention on AMD Instinct MI355X (gfx950).

Python binding of ``libsgla.so`` (C ABI in ``include/sgla.h``). This module
only checks and marshals arguments: every step of the computation runs in the
library's HIP kernels. PyTorch is used for device memory and streams. If the
library is not built, every call raises; there is no other code path.

    o, S = chunk_fwd(q, k, v, g, initial_state=None, cu_seqlens=None)
    o    = recurrent_step(q, k, v, g, state, state_indices=None)

and the variants that take q and k before the per-head RMSNorm and RoPE of a
lightning layer and apply both as the tiles are loaded:

    o, S = chunk_fwd_qk_norm_rope(q, k, v, g, q_weight, k_weight, pos_offset=None)
    o    = recurrent_step_qk_norm_rope(q, k, v, g, state, q_weight, k_weight, positions)

and the layer's output epilogue (RMSNorm over all heads of a token, sigmoid
gate):

    y    = out_norm_gate(o, z, weight)

``recurrent_step_ex`` takes every decode option at once (a bf16 state pool,
the prologue).

The gated delta rule (GDN), with a per-token write strength beta:

    o, S = gdn_chunk_fwd(q, k, v, g, beta, initial_state=None, cu_seqlens=None)
    o    = gdn_recurrent_step(q, k, v, g, beta, state, state_indices=None)

and with one gate per key dim (KDA: g [.., H, Dk]):

    o, S = kda_chunk_fwd(q, k, v, g, beta, initial_state=None, cu_seqlens=None)
    o    = kda_recurrent_step(q, k, v, g, beta, state, state_indices=None)
"""
from __future__ import annotations

import ctypes
import math
import os
import re

import torch

__all__ = ["chunk_fwd", "recurrent_step", "chunk_fwd_qk_norm_rope", "recurrent_step_qk_norm_rope",
           "recurrent_step_ex", "out_norm_gate", "gdn_chunk_fwd", "gdn_recurrent_step",
           "kda_recurrent_step", "kda_chunk_fwd", "kda_workspace_size",
           "chunk_workspace_size", "gdn_workspace_size", "validate_cu_seqlens", "qk_norm_rope",
           "status_string", "library", "library_path", "exported_symbols", "SglaError"]

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libsgla.so")
header_path = os.path.join(os.path.dirname(_HERE), "include", "sgla.h")

SGLA_OK, SGLA_ERR_INVALID_ARG, SGLA_ERR_UNSUPPORTED, SGLA_ERR_HIP, SGLA_ERR_WORKSPACE = 0, 1, 2, 3, 4
SGLA_F32, SGLA_BF16 = 0, 1
_DTYPE = {torch.float32: SGLA_F32, torch.bfloat16: SGLA_BF16}


class SglaError(RuntimeError):
    def __init__(self, func, status):
        self.status = status
        super().__init__("%s failed: %s" % (func, status_string(status)))


_lib = None


def library():
    """Load libsgla.so (once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise RuntimeError(
                "libsgla.so is not built (%s); run `python -m linear_attention_hybrid_amd.build`"
                % library_path)
        lib = ctypes.CDLL(library_path)
        vp, ci, cf = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        lib.sgla_chunk_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, cf, ci,
                                       vp]
        lib.sgla_chunk_fwd.restype = ci
        lib.sgla_recurrent_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, cf, ci, vp]
        lib.sgla_recurrent_step.restype = ci
        lib.sgla_chunk_fwd_qk_norm_rope.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, cf,
                                                    cf, ci, ci, ci, ci, ci, cf, ci, vp]
        lib.sgla_chunk_fwd_qk_norm_rope.restype = ci
        lib.sgla_recurrent_step_qk_norm_rope.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                                         cf, cf, ci, ci, ci, ci, cf, ci, vp]
        lib.sgla_recurrent_step_qk_norm_rope.restype = ci
        lib.sgla_recurrent_step_ex.argtypes = [vp, vp, vp, vp, vp, ci, vp, vp, vp, vp, vp, cf, cf,
                                               ci, ci, ci, ci, cf, ci, vp]
        lib.sgla_recurrent_step_ex.restype = ci
        lib.sgla_out_norm_gate.argtypes = [vp, vp, vp, vp, ctypes.c_int64, ci, cf, ci, vp]
        lib.sgla_out_norm_gate.restype = ci
        lib.sgla_gdn_chunk_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci,
                                           cf, ci, vp]
        lib.sgla_gdn_chunk_fwd.restype = ci
        lib.sgla_gdn_recurrent_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, cf,
                                                ci, vp]
        lib.sgla_gdn_recurrent_step.restype = ci
        lib.sgla_kda_recurrent_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, cf,
                                                ci, vp]
        lib.sgla_kda_recurrent_step.restype = ci
        lib.sgla_kda_chunk_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci,
                                           cf, ci, vp]
        lib.sgla_kda_chunk_fwd.restype = ci
        zp = ctypes.POINTER(ctypes.c_size_t)
        lib.sgla_chunk_fwd_workspace_size.argtypes = [ci, ci, ci, ci, ci, ci, ci, ci, zp]
        lib.sgla_chunk_fwd_workspace_size.restype = ci
        lib.sgla_chunk_fwd_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, cf, cf, ci,
                                          ci, ci, ci, ci, cf, ci, vp, ctypes.c_size_t, vp]
        lib.sgla_chunk_fwd_ex.restype = ci
        lib.sgla_chunk_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci,
                                               cf, ci, vp]
        lib.sgla_chunk_fwd_noalloc.restype = ci
        lib.sgla_qk_norm_rope.argtypes = [vp, vp, vp, vp, ci, ci, ci, ci, cf, cf, ci, vp]
        lib.sgla_qk_norm_rope.restype = ci
        lib.sgla_validate_cu_seqlens.argtypes = [vp, ci, ci, vp, vp]
        lib.sgla_validate_cu_seqlens.restype = ci
        lib.sgla_gdn_chunk_fwd_workspace_size.argtypes = [ci, ci, ci, ci, ci, ci, ci, zp]
        lib.sgla_gdn_chunk_fwd_workspace_size.restype = ci
        lib.sgla_gdn_chunk_fwd_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci,
                                              ci, cf, ci, vp, ctypes.c_size_t, vp]
        lib.sgla_gdn_chunk_fwd_ex.restype = ci
        lib.sgla_kda_chunk_fwd_workspace_size.argtypes = [ci, ci, ci, ci, ci, ci, ci, zp]
        lib.sgla_kda_chunk_fwd_workspace_size.restype = ci
        lib.sgla_kda_chunk_fwd_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci,
                                              ci, cf, ci, vp, ctypes.c_size_t, vp]
        lib.sgla_kda_chunk_fwd_ex.restype = ci
        lib.sgla_status_string.argtypes = [ci]
        lib.sgla_status_string.restype = ctypes.c_char_p
        lib.sgla_version.argtypes = []
        lib.sgla_version.restype = ci
        _lib = lib
    return _lib


def exported_symbols():
    """Function names declared in include/sgla.h."""
    with open(header_path) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_]+\s*\*?\s*(sgla_[a-z_]+)\s*\(", text,
                                 re.M)))


def status_string(status: int) -> str:
    return library().sgla_status_string(int(status)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(t, name, dtype, shape, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if t.dtype != dtype:
        raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _chunk_args(q, k, v, g, initial_state, cu_seqlens, scale, out, final_state,
                output_final_state, gate_per_dim=False):
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, Dk]")
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    device = q.device
    if device.type != "cuda":
        raise ValueError("chunk_fwd runs on a GPU; q is on %s" % device)
    if q.dtype not in _DTYPE:
        raise TypeError("q must be float32 or bfloat16")
    _check(q, "q", q.dtype, (B, T, H, Dk), device)
    _check(k, "k", q.dtype, (B, T, H, Dk), device)
    _check(v, "v", q.dtype, (B, T, H, Dv), device)
    _check(g, "g", torch.float32, (B, T, H, Dk) if gate_per_dim else (B, T, H), device)
    N = B
    if cu_seqlens is not None:
        if B != 1:
            raise ValueError("packed sequences need B == 1")
        if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
            raise ValueError("cu_seqlens must be 1-D with N+1 entries")
        N = cu_seqlens.numel() - 1
        _check(cu_seqlens, "cu_seqlens", torch.int64, (N + 1,), device)
    if initial_state is not None:
        _check(initial_state, "initial_state", torch.float32, (N, H, Dk, Dv), device)
    if out is None:
        out = torch.empty((B, T, H, Dv), dtype=v.dtype, device=device)
    else:
        _check(out, "out", v.dtype, (B, T, H, Dv), device)
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=device)
    elif final_state is not None:
        _check(final_state, "final_state", torch.float32, (N, H, Dk, Dv), device)
    if scale is None:
        scale = 1.0 / math.sqrt(Dk)
    # Packed input: the C ABI takes B = number of sequences and T = the total.
    Barg = N if cu_seqlens is not None else B
    return dict(device=device, N=N, out=out, final_state=final_state,
                sizes=(Barg, T, H, Dk, Dv), scale=float(scale))


def chunk_workspace_size(B, T, H, Dk, Dv, dtype=torch.bfloat16, varlen=False, prologue=False):
    """Bytes of workspace ``sgla_chunk_fwd_ex`` takes for these sizes (B is the
    number of sequences; with ``varlen`` T is the packed total)."""
    n = ctypes.c_size_t(0)
    st = library().sgla_chunk_fwd_workspace_size(int(B), int(T), int(H), int(Dk), int(Dv),
                                                  _DTYPE[dtype], int(bool(varlen)),
                                                  int(bool(prologue)), ctypes.byref(n))
    if st != SGLA_OK:
        raise SglaError("sgla_chunk_fwd_workspace_size", st)
    return int(n.value)


def gdn_workspace_size(B, T, H, Dk, Dv, dtype=torch.bfloat16, varlen=False):
    """Bytes of workspace ``sgla_gdn_chunk_fwd_ex`` takes for these sizes."""
    n = ctypes.c_size_t(0)
    st = library().sgla_gdn_chunk_fwd_workspace_size(int(B), int(T), int(H), int(Dk), int(Dv),
                                                      _DTYPE[dtype], int(bool(varlen)),
                                                      ctypes.byref(n))
    if st != SGLA_OK:
        raise SglaError("sgla_gdn_chunk_fwd_workspace_size", st)
    return int(n.value)


def kda_workspace_size(B, T, H, Dk, Dv, dtype=torch.bfloat16, varlen=False):
    """Bytes of workspace ``sgla_kda_chunk_fwd_ex`` takes for these sizes."""
    n = ctypes.c_size_t(0)
    st = library().sgla_kda_chunk_fwd_workspace_size(int(B), int(T), int(H), int(Dk), int(Dv),
                                                      _DTYPE[dtype], int(bool(varlen)),
                                                      ctypes.byref(n))
    if st != SGLA_OK:
        raise SglaError("sgla_kda_chunk_fwd_workspace_size", st)
    return int(n.value)


def _workspace(workspace, nbytes, device):
    """The workspace pointer and size to pass: "auto" takes a byte tensor from
    torch's allocator, None passes none, a uint8 tensor is used as given."""
    if workspace is None:
        return None, 0, None
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError("workspace must be 'auto', None or a uint8 tensor")
        if nbytes == 0:
            return None, 0, None
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if not isinstance(workspace, torch.Tensor) or workspace.dtype != torch.uint8:
        raise TypeError("workspace must be a uint8 tensor")
    if workspace.device != device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on %s" % device)
    return ctypes.c_void_p(workspace.data_ptr()), workspace.numel(), workspace


def qk_norm_rope(x, weight, pos_offset=None, theta=10000.0, eps=1e-6, out=None):
    """The q/k prologue alone (sgla_qk_norm_rope): per-head RMSNorm with
    ``weight`` (fp32 [128]) then rotate-half RoPE, on x [B, T, H, 128] bf16;
    token t of sequence b at position pos_offset[b] + t (int32 [B] or None).
    Returns the bf16 result (``out`` may be x itself)."""
    if x.dim() != 4:
        raise ValueError("x must be [B, T, H, Dk]")
    B, T, H, Dk = x.shape
    device = x.device
    _check(x, "x", torch.bfloat16, (B, T, H, Dk), device)
    _check(weight, "weight", torch.float32, (Dk,), device)
    if pos_offset is not None:
        _check(pos_offset, "pos_offset", torch.int32, (B,), device)
    if out is None:
        out = torch.empty_like(x)
    else:
        _check(out, "out", torch.bfloat16, (B, T, H, Dk), device)
    with torch.cuda.device(device):
        st = library().sgla_qk_norm_rope(_ptr(x), _ptr(weight), _ptr(pos_offset), _ptr(out), B, T,
                                         H, Dk, float(theta), float(eps), SGLA_BF16,
                                         _stream(device))
    if st != SGLA_OK:
        raise SglaError("sgla_qk_norm_rope", st)
    return out


def validate_cu_seqlens(cu_seqlens, T):
    """Check packed-sequence offsets on the GPU (sgla_validate_cu_seqlens) and
    return the bits of the rules they break: 1 cu[0] != 0, 2 decreasing, 4
    cu[-1] != T; 0 when valid. Synchronises with the device."""
    device = cu_seqlens.device
    _check(cu_seqlens, "cu_seqlens", torch.int64, (cu_seqlens.numel(),), device)
    status = torch.full((1,), -1, dtype=torch.int32, device=device)
    with torch.cuda.device(device):
        st = library().sgla_validate_cu_seqlens(_ptr(cu_seqlens), cu_seqlens.numel() - 1, int(T),
                                                _ptr(status), _stream(device))
    if st != SGLA_OK:
        raise SglaError("sgla_validate_cu_seqlens", st)
    return int(status.item())


def chunk_fwd(q, k, v, g, initial_state=None, cu_seqlens=None, scale=None, out=None,
              final_state=None, output_final_state=True, workspace="auto"):
    """Chunked Simple GLA prefill.

    q, k [B, T, H, Dk], v [B, T, H, Dv] (fp32 or bf16, same dtype, on one GPU),
    g [B, T, H] fp32 log-decay. With ``cu_seqlens`` (int64 [N+1] on the same
    device) B must be 1 and the N packed sequences are [cu[i], cu[i+1]).
    initial_state [N, H, Dk, Dv] fp32 or None (zeros). scale defaults to
    1/sqrt(Dk). Returns (o [B, T, H, Dv] in v's dtype, final_state [N, H, Dk,
    Dv] fp32, or None when output_final_state is False and none was given).
    ``final_state`` may be passed in (also the same tensor as initial_state).
    ``workspace``: "auto" (a workspace from torch's allocator, so long
    sequences are split across workgroups), None (no workspace: one segment
    per sequence), or a uint8 tensor of at least ``chunk_workspace_size``
    bytes.
    """
    a = _chunk_args(q, k, v, g, initial_state, cu_seqlens, scale, out, final_state,
                    output_final_state)
    device = a["device"]
    with torch.cuda.device(device):
        nb = chunk_workspace_size(*a["sizes"], dtype=q.dtype, varlen=cu_seqlens is not None) \
            if isinstance(workspace, str) else 0
        wp, wn, _keep = _workspace(workspace, nb, device)
        st = library().sgla_chunk_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(initial_state),
                                         _ptr(a["out"]), _ptr(a["final_state"]), _ptr(cu_seqlens),
                                         None, None, None, 0.0, 0.0, *a["sizes"], a["scale"],
                                         _DTYPE[q.dtype], wp, wn, _stream(device))
    if st != SGLA_OK:
        raise SglaError("sgla_chunk_fwd_ex", st)
    return a["out"], a["final_state"]


def _prologue_args(q_weight, k_weight, Dk, device):
    _check(q_weight, "q_weight", torch.float32, (Dk,), device)
    _check(k_weight, "k_weight", torch.float32, (Dk,), device)


def chunk_fwd_qk_norm_rope(q, k, v, g, q_weight, k_weight, pos_offset=None, theta=10000.0,
                           eps=1e-6, initial_state=None, cu_seqlens=None, scale=None, out=None,
                           final_state=None, output_final_state=True, workspace="auto"):
    """``chunk_fwd`` with q and k given before the per-head RMSNorm (weights
    q_weight, k_weight: fp32 [Dk], shared by all heads) and the rotate-half
    RoPE with base ``theta``, both applied inside the kernels (bf16, Dk = Dv =
    128 only). ``pos_offset`` (int32 [N] or None for zeros) is the position of
    each sequence's first token; the others follow one by one. ``workspace``
    as for ``chunk_fwd``.
    """
    a = _chunk_args(q, k, v, g, initial_state, cu_seqlens, scale, out, final_state,
                    output_final_state)
    device = a["device"]
    _prologue_args(q_weight, k_weight, q.shape[-1], device)
    if pos_offset is not None:
        _check(pos_offset, "pos_offset", torch.int32, (a["N"],), device)
    with torch.cuda.device(device):
        nb = chunk_workspace_size(*a["sizes"], dtype=q.dtype, varlen=cu_seqlens is not None,
                                  prologue=True) if isinstance(workspace, str) else 0
        wp, wn, _keep = _workspace(workspace, nb, device)
        st = library().sgla_chunk_fwd_ex(
            _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(initial_state), _ptr(a["out"]),
            _ptr(a["final_state"]), _ptr(cu_seqlens), _ptr(q_weight), _ptr(k_weight),
            _ptr(pos_offset), float(theta), float(eps), *a["sizes"], a["scale"],
            _DTYPE[q.dtype], wp, wn, _stream(device))
    if st != SGLA_OK:
        raise SglaError("sgla_chunk_fwd_ex", st)
    return a["out"], a["final_state"]


def _step_args(q, k, v, g, state, state_indices, scale, out, allow_bf16_state=False,
               gate_per_dim=False):
    if q.dim() != 3:
        raise ValueError("q must be [N, H, Dk]")
    N, H, Dk = q.shape
    Dv = v.shape[-1]
    device = q.device
    if device.type != "cuda":
        raise ValueError("recurrent_step runs on a GPU; q is on %s" % device)
    if q.dtype not in _DTYPE:
        raise TypeError("q must be float32 or bfloat16")
    _check(q, "q", q.dtype, (N, H, Dk), device)
    _check(k, "k", q.dtype, (N, H, Dk), device)
    _check(v, "v", q.dtype, (N, H, Dv), device)
    _check(g, "g", torch.float32, (N, H, Dk) if gate_per_dim else (N, H), device)
    if state.dim() != 4:
        raise ValueError("state must be [slots, H, Dk, Dv]")
    if state.dtype not in _DTYPE or (state.dtype != torch.float32 and not allow_bf16_state):
        raise TypeError("state must be float32%s" % (" or bfloat16" if allow_bf16_state else ""))
    _check(state, "state", state.dtype, (state.shape[0], H, Dk, Dv), device)
    if state_indices is not None:
        _check(state_indices, "state_indices", torch.int32, (N,), device)
    elif state.shape[0] < N:
        raise ValueError("state has fewer slots than rows")
    if out is None:
        out = torch.empty((N, H, Dv), dtype=v.dtype, device=device)
    else:
        _check(out, "out", v.dtype, (N, H, Dv), device)
    if scale is None:
        scale = 1.0 / math.sqrt(Dk)
    return dict(device=device, out=out, sizes=(N, H, Dk, Dv), scale=float(scale))


def recurrent_step(q, k, v, g, state, state_indices=None, scale=None, out=None):
    """One fused decode step, updating ``state`` in place.

    q, k [N, H, Dk], v [N, H, Dv] (fp32 or bf16), g [N, H] fp32,
    state [slots, H, Dk, Dv] fp32, state_indices [N] int32 (distinct slots) or
    None for slot = row. Returns o [N, H, Dv] in v's dtype.
    """
    a = _step_args(q, k, v, g, state, state_indices, scale, out)
    device = a["device"]
    with torch.cuda.device(device):
        st = library().sgla_recurrent_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(state),
                                           _ptr(state_indices), _ptr(a["out"]), *a["sizes"],
                                           a["scale"], _DTYPE[q.dtype], _stream(device))
    if st != SGLA_OK:
        raise SglaError("sgla_recurrent_step", st)
    return a["out"]


def recurrent_step_qk_norm_rope(q, k, v, g, state, q_weight, k_weight, positions,
                                theta=10000.0, eps=1e-6, state_indices=None, scale=None,
                                out=None):
    """``recurrent_step`` with q and k given before the per-head RMSNorm and
    RoPE (bf16, Dk = 128 only); ``positions`` (int32 [N]) is the position of
    each row's token."""
    a = _step_args(q, k, v, g, state, state_indices, scale, out)
    device = a["device"]
    _prologue_args(q_weight, k_weight, q.shape[-1], device)
    _check(positions, "positions", torch.int32, (q.shape[0],), device)
    with torch.cuda.device(device):
        st = library().sgla_recurrent_step_qk_norm_rope(
            _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(state), _ptr(state_indices), _ptr(a["out"]),
            _ptr(q_weight), _ptr(k_weight), _ptr(positions), float(theta), float(eps),
            *a["sizes"], a["scale"], _DTYPE[q.dtype], _stream(device))
    if st != SGLA_OK:
        raise SglaError("sgla_recurrent_step_qk_norm_rope", st)
    return a["out"]


def out_norm_gate(o, z, weight, eps=1e-6, out=None):
    """The output epilogue: each row of ``width = weight.numel()`` elements of
    o (the heads of one token, e.g. o [B, T, H, Dv] with width H * Dv) is
    RMS-normalised with ``weight`` (fp32 [width]) and multiplied by
    sigmoid(z); z has o's shape and dtype. ``out`` may be o itself. Returns
    out (o's shape and dtype)."""
    device = o.device
    if device.type != "cuda":
        raise ValueError("out_norm_gate runs on a GPU; o is on %s" % device)
    if o.dtype not in _DTYPE:
        raise TypeError("o must be float32 or bfloat16")
    if weight.dim() != 1:
        raise ValueError("weight must be 1-D")
    width = weight.shape[0]
    if o.numel() % width != 0:
        raise ValueError("o's size is not a whole number of rows of %d" % width)
    _check(o, "o", o.dtype, tuple(o.shape), device)
    _check(z, "z", o.dtype, tuple(o.shape), device)
    _check(weight, "weight", torch.float32, (width,), device)
    if out is None:
        out = torch.empty_like(o)
    else:
        _check(out, "out", o.dtype, tuple(o.shape), device)
    rows = o.numel() // width
    with torch.cuda.device(device):
        st = library().sgla_out_norm_gate(_ptr(o), _ptr(z), _ptr(weight), _ptr(out), rows, width,
                                          float(eps), _DTYPE[o.dtype], _stream(device))
    if st != SGLA_OK:
        raise SglaError("sgla_out_norm_gate", st)
    return out


def recurrent_step_ex(q, k, v, g, state, state_indices=None, q_weight=None, k_weight=None,
                      positions=None, theta=10000.0, eps=1e-6, scale=None, out=None):
    """The decode step with every option: ``state`` may be float32 or
    bfloat16 (a bf16 pool is updated in fp32 and stored rounded); with
    ``q_weight`` given, q and k go through the per-head RMSNorm and RoPE
    first (then ``k_weight`` and ``positions`` are required). Returns o."""
    a = _step_args(q, k, v, g, state, state_indices, scale, out, allow_bf16_state=True)
    device = a["device"]
    if q_weight is not None:
        if k_weight is None or positions is None:
            raise ValueError("the prologue needs q_weight, k_weight and positions")
        _prologue_args(q_weight, k_weight, q.shape[-1], device)
        _check(positions, "positions", torch.int32, (q.shape[0],), device)
    with torch.cuda.device(device):
        st = library().sgla_recurrent_step_ex(
            _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(state), _DTYPE[state.dtype],
            _ptr(state_indices), _ptr(a["out"]), _ptr(q_weight), _ptr(k_weight), _ptr(positions),
            float(theta), float(eps), *a["sizes"], a["scale"], _DTYPE[q.dtype], _stream(device))
    if st != SGLA_OK:
        raise SglaError("sgla_recurrent_step_ex", st)
    return a["out"]


def gdn_chunk_fwd(q, k, v, g, beta, initial_state=None, cu_seqlens=None, scale=None, out=None,
                  final_state=None, output_final_state=True, workspace="auto"):
    """Chunked prefill of the gated delta rule: arguments and results as
    ``chunk_fwd``, plus ``beta`` [B, T, H] fp32, the write strength of each
    token and head. bf16 with Dk = Dv = 128 only. The chunkwise form keeps
    per-chunk tiles between its kernels, so ``workspace`` ("auto" or a uint8
    tensor of ``gdn_workspace_size`` bytes) is required when there are tokens.
    """
    a = _chunk_args(q, k, v, g, initial_state, cu_seqlens, scale, out, final_state,
                    output_final_state)
    device = a["device"]
    _check(beta, "beta", torch.float32, tuple(g.shape), device)
    with torch.cuda.device(device):
        nb = gdn_workspace_size(*a["sizes"], dtype=q.dtype, varlen=cu_seqlens is not None) \
            if isinstance(workspace, str) else 0
        wp, wn, _keep = _workspace(workspace, nb, device)
        st = library().sgla_gdn_chunk_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                             _ptr(initial_state), _ptr(a["out"]),
                                             _ptr(a["final_state"]), _ptr(cu_seqlens),
                                             *a["sizes"], a["scale"], _DTYPE[q.dtype], wp, wn,
                                             _stream(device))
    if st != SGLA_OK:
        raise SglaError("sgla_gdn_chunk_fwd_ex", st)
    return a["out"], a["final_state"]


def kda_chunk_fwd(q, k, v, g, beta, initial_state=None, cu_seqlens=None, scale=None, out=None,
                  final_state=None, output_final_state=True, workspace="auto"):
    """Chunked prefill of the gated delta rule with one gate per key dim
    (KDA): arguments and results as ``gdn_chunk_fwd``, except g [B, T, H, Dk]
    fp32. fp32 or bf16 inputs, Dk and Dv in {64, 128}. ``workspace`` ("auto"
    or a uint8 tensor of ``kda_workspace_size`` bytes) is required when there
    are tokens.
    """
    a = _chunk_args(q, k, v, g, initial_state, cu_seqlens, scale, out, final_state,
                    output_final_state, gate_per_dim=True)
    device = a["device"]
    _check(beta, "beta", torch.float32, tuple(g.shape[:3]), device)
    with torch.cuda.device(device):
        nb = kda_workspace_size(*a["sizes"], dtype=q.dtype, varlen=cu_seqlens is not None) \
            if isinstance(workspace, str) else 0
        wp, wn, _keep = _workspace(workspace, nb, device)
        st = library().sgla_kda_chunk_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                             _ptr(initial_state), _ptr(a["out"]),
                                             _ptr(a["final_state"]), _ptr(cu_seqlens),
                                             *a["sizes"], a["scale"], _DTYPE[q.dtype], wp, wn,
                                             _stream(device))
    if st != SGLA_OK:
        raise SglaError("sgla_kda_chunk_fwd_ex", st)
    return a["out"], a["final_state"]


def gdn_recurrent_step(q, k, v, g, beta, state, state_indices=None, scale=None, out=None):
    """One decode step of the gated delta rule, updating the fp32 ``state``
    pool in place: arguments as ``recurrent_step``, plus ``beta`` [N, H]
    fp32. Returns o [N, H, Dv] in v's dtype."""
    a = _step_args(q, k, v, g, state, state_indices, scale, out)
    device = a["device"]
    _check(beta, "beta", torch.float32, tuple(g.shape), device)
    with torch.cuda.device(device):
        st = library().sgla_gdn_recurrent_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                               _ptr(state), _ptr(state_indices), _ptr(a["out"]),
                                               *a["sizes"], a["scale"], _DTYPE[q.dtype],
                                               _stream(device))
    if st != SGLA_OK:
        raise SglaError("sgla_gdn_recurrent_step", st)
    return a["out"]


def kda_recurrent_step(q, k, v, g, beta, state, state_indices=None, scale=None, out=None):
    """One decode step of the gated delta rule with one gate per key dim
    (KDA), updating the fp32 ``state`` pool in place: arguments as
    ``gdn_recurrent_step`` except g [N, H, Dk] fp32. Returns o [N, H, Dv] in
    v's dtype."""
    a = _step_args(q, k, v, g, state, state_indices, scale, out, gate_per_dim=True)
    device = a["device"]
    _check(beta, "beta", torch.float32, tuple(q.shape[:2]), device)
    with torch.cuda.device(device):
        st = library().sgla_kda_recurrent_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                               _ptr(state), _ptr(state_indices), _ptr(a["out"]),
                                               *a["sizes"], a["scale"], _DTYPE[q.dtype],
                                               _stream(device))
    if st != SGLA_OK:
        raise SglaError("sgla_kda_recurrent_step", st)
    return a["out"]

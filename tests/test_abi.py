"""The C-ABI library on the CPU: it loads, exports every declared symbol, and
rejects bad arguments synchronously, before any HIP call (no GPU needed)."""
import ctypes
import os
import subprocess

import pytest

import linear_attention_hybrid_amd as sgla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sgla.library_path):
        from linear_attention_hybrid_amd import build
        build.build()
    return sgla.library()


def _no_gpu():
    import torch
    return not torch.cuda.is_available()


def test_header_declares_the_entry_points():
    names = sgla.exported_symbols()
    for n in ("sgla_chunk_fwd", "sgla_recurrent_step", "sgla_chunk_fwd_qk_norm_rope",
              "sgla_recurrent_step_qk_norm_rope", "sgla_recurrent_step_ex", "sgla_out_norm_gate",
              "sgla_gdn_chunk_fwd", "sgla_gdn_recurrent_step", "sgla_status_string",
              "sgla_version"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", sgla.library_path], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in sgla.exported_symbols():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_status_strings_and_version(lib):
    assert sgla.status_string(0) == "SGLA_OK"
    assert sgla.status_string(1) == "SGLA_ERR_INVALID_ARG"
    assert sgla.status_string(2) == "SGLA_ERR_UNSUPPORTED"
    assert sgla.status_string(3) == "SGLA_ERR_HIP"
    assert sgla.status_string(77) == "SGLA_ERR_UNKNOWN"
    assert lib.sgla_version() >= 100


A = 0x10000  # a 16-byte aligned address that is never dereferenced


def chunk(lib, q=A, k=A, v=A, g=A, s0=None, out=A, sf=None, cu=None, B=0, T=0, H=1, Dk=64,
          Dv=64, scale=1.0, dtype=0):
    return lib.sgla_chunk_fwd(q, k, v, g, s0, out, sf, cu, B, T, H, Dk, Dv, scale, dtype, None)


def step(lib, q=A, k=A, v=A, g=A, state=A, idx=None, out=A, N=0, H=1, Dk=64, Dv=64, dtype=0):
    return lib.sgla_recurrent_step(q, k, v, g, state, idx, out, N, H, Dk, Dv, 1.0, dtype, None)


def test_chunk_fwd_validation(lib):
    # B = 0 would be a no-op, so every rejection below happens before any launch.
    assert chunk(lib) == 0
    assert chunk(lib, dtype=2) == 1
    assert chunk(lib, dtype=-1) == 1
    assert chunk(lib, B=-1) == 1
    assert chunk(lib, T=-1) == 1
    assert chunk(lib, H=0) == 1
    assert chunk(lib, Dk=32) == 2
    assert chunk(lib, Dv=96) == 2
    assert chunk(lib, Dk=0) == 1
    assert chunk(lib, q=A + 2) == 1
    assert chunk(lib, v=A + 8) == 1
    assert chunk(lib, out=A + 4) == 1
    assert chunk(lib, g=A + 2) == 1
    assert chunk(lib, g=A + 4) == 0          # g only needs fp32 alignment
    assert chunk(lib, s0=A + 4) == 1
    assert chunk(lib, sf=A + 8) == 1
    assert chunk(lib, cu=A + 4) == 1
    assert chunk(lib, B=2**28, T=2**31 - 1, H=1, Dk=128, Dv=128) == 1  # B*T*H*D past 2^62
    assert chunk(lib, B=1, T=1, H=2**16 + 1) == 2                      # beyond the head limit
    # 2^30 one-segment (sequence, head) units: the vector-ALU grid (four
    # workgroups per unit at Dv = 128) would pass 2^31
    assert chunk(lib, B=2**24, T=64, H=64, Dk=128, Dv=128) == 2


@pytest.mark.skipif("not _no_gpu()", reason="could reach a launch if validation were wrong")
def test_chunk_fwd_null_pointers(lib):
    assert chunk(lib, q=None, B=1, T=1) == 1
    assert chunk(lib, g=None, B=1, T=1) == 1
    assert chunk(lib, out=None, B=1, T=1) == 1
    # No tokens and no final state: nothing to do, no pointer needed.
    assert chunk(lib, q=None, k=None, v=None, g=None, out=None, B=3, T=0) == 0


def test_recurrent_step_validation(lib):
    assert step(lib) == 0
    assert step(lib, dtype=5) == 1
    assert step(lib, N=-1) == 1
    assert step(lib, H=0) == 1
    assert step(lib, Dk=256) == 2
    assert step(lib, N=2**20, H=2**12) == 1


@pytest.mark.skipif("not _no_gpu()", reason="could reach a launch if validation were wrong")
def test_recurrent_step_pointer_checks(lib):
    assert step(lib, N=1, state=None) == 1
    assert step(lib, N=1, q=A + 2) == 1
    assert step(lib, N=1, idx=A + 2) == 1
    assert step(lib, N=1, state=A + 4) == 1


def chunk_pro(lib, q=A, k=A, v=A, g=A, s0=None, out=A, sf=None, cu=None, qw=A, kw=A, pos=None,
              theta=1e4, eps=1e-6, B=0, T=0, H=1, Dk=128, Dv=128, dtype=1):
    return lib.sgla_chunk_fwd_qk_norm_rope(q, k, v, g, s0, out, sf, cu, qw, kw, pos, theta, eps,
                                           B, T, H, Dk, Dv, 1.0, dtype, None)


def step_pro(lib, q=A, k=A, v=A, g=A, state=A, idx=None, out=A, qw=A, kw=A, pos=A, theta=1e4,
             eps=1e-6, N=0, H=1, Dk=128, Dv=128, dtype=1):
    return lib.sgla_recurrent_step_qk_norm_rope(q, k, v, g, state, idx, out, qw, kw, pos, theta,
                                                eps, N, H, Dk, Dv, 1.0, dtype, None)


def test_qk_norm_rope_validation(lib):
    nan, inf = float("nan"), float("inf")
    # B = 0 / N = 0: every check below still runs before the no-op return.
    assert chunk_pro(lib) == 0
    assert chunk_pro(lib, dtype=0) == 2        # the prologue is built for bf16
    assert chunk_pro(lib, Dk=64, Dv=64) == 2
    assert chunk_pro(lib, Dv=64) == 2
    assert chunk_pro(lib, qw=None) == 1
    assert chunk_pro(lib, kw=None) == 1
    assert chunk_pro(lib, kw=A + 2) == 1
    assert chunk_pro(lib, pos=A + 2) == 1
    assert chunk_pro(lib, pos=A + 4) == 0      # int32 offsets need 4 bytes
    for bad in (0.0, -1.0, inf, nan):
        assert chunk_pro(lib, theta=bad) == 1, bad
    for bad in (-1e-6, inf, nan):
        assert chunk_pro(lib, eps=bad) == 1, bad
    assert chunk_pro(lib, eps=0.0) == 0
    assert step_pro(lib) == 0
    assert step_pro(lib, Dv=64) == 0
    assert step_pro(lib, dtype=0) == 2
    assert step_pro(lib, Dk=64) == 2
    assert step_pro(lib, qw=None) == 1
    assert step_pro(lib, theta=nan) == 1
    assert step_pro(lib, eps=-1.0) == 1


@pytest.mark.skipif("not _no_gpu()", reason="could reach a launch if validation were wrong")
def test_qk_norm_rope_pointer_checks(lib):
    assert step_pro(lib, N=1, pos=None) == 1   # positions are required for a step
    assert chunk_pro(lib, B=1, T=1, q=None) == 1


def step_ex(lib, state_dtype=1, qw=None, kw=None, pos=None, theta=1e4, eps=1e-6, N=0, H=1,
            Dk=128, Dv=128, dtype=1, state=A):
    return lib.sgla_recurrent_step_ex(A, A, A, A, state, state_dtype, None, A, qw, kw, pos, theta,
                                      eps, N, H, Dk, Dv, 1.0, dtype, None)


def test_recurrent_step_ex_validation(lib):
    assert step_ex(lib) == 0
    assert step_ex(lib, state_dtype=0) == 0
    assert step_ex(lib, state_dtype=2) == 1
    assert step_ex(lib, state_dtype=-1) == 1
    assert step_ex(lib, Dk=64, Dv=64, dtype=0) == 0          # no prologue: any supported size
    assert step_ex(lib, qw=A, kw=A, pos=A, Dk=64) == 2        # the prologue needs Dk = 128
    assert step_ex(lib, qw=A, kw=None, pos=A) == 1
    assert step_ex(lib, qw=A, kw=A, pos=A, theta=0.0) == 1


@pytest.mark.skipif("not _no_gpu()", reason="could reach a launch if validation were wrong")
def test_recurrent_step_ex_pointer_checks(lib):
    assert step_ex(lib, N=1, state=A + 8) == 1                 # bf16 pool still needs 16 bytes
    assert step_ex(lib, N=1, qw=A, kw=A, pos=None) == 1


def epi(lib, o=A, z=A, w=A, out=A, rows=0, width=4096, eps=1e-6, dtype=1):
    return lib.sgla_out_norm_gate(o, z, w, out, rows, width, eps, dtype, None)


def test_out_norm_gate_validation(lib):
    assert epi(lib) == 0
    assert epi(lib, dtype=3) == 1
    assert epi(lib, rows=-1) == 1
    assert epi(lib, rows=2**31) == 1
    assert epi(lib, width=0) == 1
    assert epi(lib, width=4100) == 2          # not a multiple of 8
    assert epi(lib, width=16384 + 8) == 2     # wider than a row the kernel holds
    assert epi(lib, eps=-1.0) == 1
    assert epi(lib, eps=float("nan")) == 1


@pytest.mark.skipif("not _no_gpu()", reason="could reach a launch if validation were wrong")
def test_out_norm_gate_pointer_checks(lib):
    assert epi(lib, rows=1, o=None) == 1
    assert epi(lib, rows=1, w=A + 4) == 1
    assert epi(lib, rows=1, out=A + 8) == 1


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(1, 4, 1, 64)
    with pytest.raises(ValueError):
        sgla.chunk_fwd(x, x, x, torch.zeros(1, 4, 1))
    with pytest.raises(ValueError):
        sgla.recurrent_step(x[0], x[0], x[0], torch.zeros(4, 1), torch.zeros(4, 1, 64, 64))


def gdn_chunk(lib, q=A, k=A, v=A, g=A, beta=A, s0=None, out=A, sf=None, cu=None, B=0, T=0, H=1,
              Dk=128, Dv=128, dtype=1):
    return lib.sgla_gdn_chunk_fwd(q, k, v, g, beta, s0, out, sf, cu, B, T, H, Dk, Dv, 1.0, dtype,
                                  None)


def gdn_step(lib, q=A, k=A, v=A, g=A, beta=A, state=A, idx=None, out=A, N=0, H=1, Dk=128,
             Dv=128, dtype=1):
    return lib.sgla_gdn_recurrent_step(q, k, v, g, beta, state, idx, out, N, H, Dk, Dv, 1.0,
                                       dtype, None)


def test_gdn_validation(lib):
    assert gdn_chunk(lib) == 0
    assert gdn_chunk(lib, dtype=0) == 2        # the chunked delta rule is built for bf16
    assert gdn_chunk(lib, Dk=64, Dv=64) == 2
    assert gdn_chunk(lib, dtype=4) == 1
    assert gdn_chunk(lib, B=-1) == 1
    assert gdn_chunk(lib, beta=A + 2) == 1
    assert gdn_chunk(lib, beta=A + 4) == 0     # fp32 alignment is enough
    assert gdn_chunk(lib, cu=A + 4) == 1
    assert gdn_chunk(lib, B=1, T=1, H=2**16 + 1) == 2
    assert gdn_chunk(lib, B=2**26, T=1, H=5) == 2    # the chain's grid would pass 2^31
    assert gdn_step(lib) == 0
    assert gdn_step(lib, Dk=64, Dv=64, dtype=0) == 0
    assert gdn_step(lib, Dk=96) == 2
    assert gdn_step(lib, N=-1) == 1
    assert gdn_step(lib, dtype=2) == 1


@pytest.mark.skipif("not _no_gpu()", reason="could reach a launch if validation were wrong")
def test_gdn_pointer_checks(lib):
    assert gdn_chunk(lib, B=1, T=1, beta=None) == 1
    assert gdn_chunk(lib, B=1, T=1, q=None) == 1
    assert gdn_step(lib, N=1, beta=None) == 1
    assert gdn_step(lib, N=1, beta=A + 2) == 1
    assert gdn_step(lib, N=1, state=A + 4) == 1


def chunk_ex(lib, q=A, k=A, v=A, g=A, s0=None, out=A, sf=None, cu=None, qw=None, kw=None,
             pos=None, theta=0.0, eps=0.0, B=0, T=0, H=1, Dk=64, Dv=64, scale=1.0, dtype=0,
             ws=None, wsb=0):
    return lib.sgla_chunk_fwd_ex(q, k, v, g, s0, out, sf, cu, qw, kw, pos, theta, eps, B, T, H,
                                 Dk, Dv, scale, dtype, ws, wsb, None)


def ws_size(lib, B, T, H, Dk, Dv, dtype, varlen=0, prologue=0, gdn=False):
    n = ctypes.c_size_t(12345)
    if gdn:
        st = lib.sgla_gdn_chunk_fwd_workspace_size(B, T, H, Dk, Dv, dtype, varlen, ctypes.byref(n))
    else:
        st = lib.sgla_chunk_fwd_workspace_size(B, T, H, Dk, Dv, dtype, varlen, prologue,
                                               ctypes.byref(n))
    return st, n.value


def test_workspace_size_queries(lib):
    # Sequences short enough to be one segment need no workspace.
    assert ws_size(lib, 4, 256, 8, 128, 128, 1) == (0, 0)
    assert ws_size(lib, 0, 8192, 32, 128, 128, 1) == (0, 0)
    # The lightning prefill shape splits: states, log-decays and a header.
    st, n = ws_size(lib, 1, 8192, 32, 128, 128, 1)
    assert st == 0 and n > 32 * 128 * 128 * 4 and n % 256 == 0
    # A bound over every cu_seqlens is at least the equal-length size of the
    # same total, and it grows with T.
    assert ws_size(lib, 1, 8192, 32, 128, 128, 1, varlen=1)[1] >= n
    assert ws_size(lib, 1, 65536, 32, 128, 128, 1)[1] >= n
    # fp32, the prologue and 64-wide heads take the one-level kernels.
    assert ws_size(lib, 1, 8192, 4, 64, 64, 0)[0] == 0
    assert ws_size(lib, 1, 8192, 32, 128, 128, 1, prologue=1)[0] == 0
    # Errors: bad dtype, unsupported sizes, the prologue outside bf16 / 128, no output.
    assert ws_size(lib, 1, 64, 1, 128, 128, 7)[0] == 1
    assert ws_size(lib, 1, 64, 1, 96, 128, 1)[0] == 2
    assert ws_size(lib, 1, 64, 1, 128, 128, 0, prologue=1)[0] == 2
    assert ws_size(lib, -1, 64, 1, 128, 128, 1)[0] == 1
    assert lib.sgla_chunk_fwd_workspace_size(1, 64, 1, 128, 128, 1, 0, 0, None) == 1
    # The gated delta rule keeps 64 KiB per chunk and head, plus the header.
    st, n = ws_size(lib, 2, 100, 3, 128, 128, 1, gdn=True)
    assert st == 0 and n == 256 + 2 * 2 * 3 * 65536
    assert ws_size(lib, 2, 100, 3, 128, 128, 0, gdn=True)[0] == 2
    assert ws_size(lib, 0, 100, 3, 128, 128, 1, gdn=True) == (0, 0)


def test_workspace_checks_before_any_launch(lib):
    big = dict(B=1, T=8192, H=32, Dk=128, Dv=128, dtype=1)
    n = ws_size(lib, 1, 8192, 32, 128, 128, 1)[1]
    assert chunk_ex(lib, ws=A, wsb=n - 1, **big) == 4        # too small: SGLA_ERR_WORKSPACE
    assert chunk_ex(lib, ws=A + 128, wsb=n, **big) == 1      # not 256-byte aligned
    assert sgla.status_string(4) == "SGLA_ERR_WORKSPACE"
    # The plain GDN entry point has no workspace: with tokens it says so.
    assert gdn_chunk(lib, B=1, T=64, H=1) == 4
    assert lib.sgla_gdn_chunk_fwd_ex(A, A, A, A, A, None, A, None, None, 1, 64, 1, 128, 128, 1.0,
                                     1, A, 1024, None) == 4
    # The offsets check needs its pointers.
    assert lib.sgla_validate_cu_seqlens(None, 2, 10, A, None) == 1
    assert lib.sgla_validate_cu_seqlens(A, 2, 10, None, None) == 1
    assert lib.sgla_validate_cu_seqlens(A + 4, 2, 10, A, None) == 1

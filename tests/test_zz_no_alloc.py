"""sgla_chunk_fwd_noalloc (the split plan in the library's per-GPU scratch
array, for callers that cannot allocate) against sgla_chunk_fwd_ex with a
caller workspace, through the C ABI: two calls in a row, the second smaller,
each bit for bit equal to the workspace entry point and within the parity
bars of the oracle; a plan larger than the scratch is refused before any
launch."""
import ctypes

import pytest
import torch

import linear_attention_hybrid_amd as sgla
import sgla_inputs as W
from tests.parity import check, host, nan_like, oracle_prefill, say

pytestmark = pytest.mark.gpu


def noalloc(q, k, v, g, s0, out, fs, B, T, H, D, scale):
    lib = sgla.library()
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return lib.sgla_chunk_fwd_noalloc(p(q), p(k), p(v), p(g), p(s0), p(out), p(fs), None, B, T,
                                      H, D, D, float(scale), sgla.SGLA_BF16, stream)


def test_noalloc_matches_the_workspace_entry_point():
    for T, H, seed in ((8192, 8, 31), (3000, 4, 32)):
        say("chunk_fwd_noalloc B=1 T=%d H=%d D=128 bf16 seed=%d" % (T, H, seed))
        inp = W.make_prefill(1, T, H, 128, 128, "bf16", "lightning", seed=seed, device="cuda",
                             init="normal")
        assert sgla.chunk_workspace_size(1, T, H, 128, 128, torch.bfloat16) > 0  # a split plan
        out = nan_like((1, T, H, 128), torch.bfloat16)
        fs = nan_like((1, H, 128, 128), torch.float32)
        st = noalloc(inp["q"], inp["k"], inp["v"], inp["g"], inp["initial_state"], out, fs, 1, T,
                     H, 128, inp["scale"])
        assert st == sgla.SGLA_OK, sgla.status_string(st)
        ro, rS = sgla.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["initial_state"],
                                scale=inp["scale"], workspace="auto")
        torch.cuda.synchronize()
        assert torch.equal(out, ro) and torch.equal(fs, rS)
        heads = [0, H - 1]
        oo, oS = oracle_prefill(inp, heads)
        check(host(out[:, :, heads]), oo, "bf16", "noalloc o")
        check(host(fs[:, heads]), oS, "bf16", "noalloc final state", bf16_out=False)
        del inp, out, fs, ro, rS


def test_noalloc_refuses_a_plan_larger_than_its_scratch():
    B, T, H, D = 1, 16384, 128, 128
    need = sgla.chunk_workspace_size(B, T, H, D, D, torch.bfloat16)
    assert need > 64 << 20
    say("chunk_fwd_noalloc refusal B=1 T=16384 H=128 (plan needs %d bytes)" % need)
    q = torch.zeros((B, T, H, D), dtype=torch.bfloat16, device="cuda")
    g = torch.zeros((B, T, H), dtype=torch.float32, device="cuda")
    out = torch.zeros_like(q)
    st = noalloc(q, q, q, g, None, out, None, B, T, H, D, 0.088)
    assert st == sgla.SGLA_ERR_WORKSPACE
    torch.cuda.synchronize()
    del q, g, out
    torch.cuda.empty_cache()

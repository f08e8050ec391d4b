"""GPU parity of the KDA path (gated delta rule with one gate per key dim)
against ``oracle/kda_oracle.c``: the decode step through a slot map and the
chunked prefill, with the bars of the GDN path."""
import numpy as np
import pytest
import torch

import linear_attention_hybrid_amd as sgla
import oracle.kda as KDA
import sgla_inputs as W
from tests.parity import check, host, nan_like, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(128, 128), (128, 64), (64, 128), (64, 64)])
def test_kda_step_with_slot_map(dtype, dk, dv):
    say("kda_recurrent_step", dtype, dk, dv, "N=5 H=3 slots=9, 4 steps")
    N, H, slots, steps = 5, 3, 9, 4
    d = W.make_decode(N, H, dk, dv, steps, dtype, "kda", seed=dk * 7 + dv, device="cuda",
                      slots=slots, with_beta=True)
    idx = torch.tensor([7, 0, 3, 8, 2], dtype=torch.int32, device="cuda")
    state = (d["state"] * 25).contiguous()
    ref_state = host(state).astype(np.float64)
    untouched = [s for s in range(slots) if s not in idx.tolist()]
    before_untouched = state[untouched].clone()
    for i in range(steps):
        out = nan_like((N, H, dv), d["v"].dtype)
        o = sgla.kda_recurrent_step(d["q"][i], d["k"][i], d["v"][i], d["g"][i], d["beta"][i],
                                    state, state_indices=idx, scale=d["scale"], out=out)
        torch.cuda.synchronize()
        ro = KDA.step(host(d["q"][i]), host(d["k"][i]), host(d["v"][i]), host(d["g"][i]),
                      host(d["beta"][i]), ref_state, d["scale"], state_indices=idx.cpu().numpy())
        check(host(o), ro, dtype, "kda step %d o" % i)
        check(host(state[idx.long()]), ref_state[idx.cpu().numpy()], dtype,
              "kda step %d state" % i, bf16_out=False)
    assert torch.equal(state[untouched], before_untouched)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_kda_step_per_dim_rates(dtype):
    """Gates whose rate differs by dim over four decades (-1e-4 .. -1 per
    token), 24 steps: each state row must decay at its own dim's rate."""
    say("kda_recurrent_step per-dim rates", dtype)
    N, H, D, steps = 6, 4, 128, 24
    d = W.make_decode(N, H, D, D, steps, dtype, "kda", seed=77, device="cuda", with_beta=True)
    rate = torch.tensor(10.0 ** np.linspace(-4, 0, D), dtype=torch.float32, device="cuda")
    g = -(rate * (0.5 + torch.rand((steps, N, H, D), generator=torch.Generator(device="cuda")
                                   .manual_seed(77), device="cuda"))).contiguous()
    state = (d["state"] * 25).contiguous()
    ref = host(state).astype(np.float64)
    for i in range(steps):
        o = sgla.kda_recurrent_step(d["q"][i], d["k"][i], d["v"][i], g[i], d["beta"][i], state,
                                    scale=d["scale"])
        torch.cuda.synchronize()
        ro = KDA.step(host(d["q"][i]), host(d["k"][i]), host(d["v"][i]), host(g[i]),
                      host(d["beta"][i]), ref, d["scale"])
        check(host(o), ro, dtype, "kda per-dim step %d o" % i)
    check(host(state), ref, dtype, "kda per-dim states", bf16_out=False)


def test_kda_decode_workload_sampled():
    """The batched-decode shape (256 rows x 32 heads, D = 128) with per-dim
    gates, 64 steps; the oracle follows every state of 8 sampled rows."""
    say("kda_recurrent_step N=256 H=32 D=128 64 steps seed=4 (8 rows x 32 heads)")
    d = W.make_decode(256, 32, 128, 128, 64, "bf16", "kda", seed=4, device="cuda",
                      with_beta=True)
    state = d["state"]
    rows = np.random.default_rng(4).choice(256, 8, replace=False)
    ref = np.ascontiguousarray(host(state[rows]).astype(np.float64))
    sel = lambda t: host(t[rows])
    for i in range(64):
        o = sgla.kda_recurrent_step(d["q"][i], d["k"][i], d["v"][i], d["g"][i], d["beta"][i],
                                    state, scale=d["scale"])
        ro = KDA.step(sel(d["q"][i]), sel(d["k"][i]), sel(d["v"][i]), sel(d["g"][i]),
                      sel(d["beta"][i]), ref, d["scale"])
        check(host(o[rows]), ro, "bf16", "kda decode step %d o" % i)
    torch.cuda.synchronize()
    check(host(state[rows]), ref, "bf16", "kda decode final states", bf16_out=False)


def oracle_kda(inp, heads=None):
    sel = (lambda t: t) if heads is None else (lambda t: t[:, :, heads])
    S0 = inp["initial_state"]
    if S0 is not None:
        S0 = host(S0 if heads is None else S0[:, heads]).astype(np.float64)
    cu = None if inp["cu_seqlens"] is None else inp["cu_seqlens"].cpu().numpy()
    return KDA.forward(host(sel(inp["q"])), host(sel(inp["k"])), host(sel(inp["v"])),
                       host(sel(inp["g"])), host(sel(inp["beta"])), inp["scale"],
                       initial_state=S0, cu_seqlens=cu)


def run_chunk(inp, **kw):
    out = nan_like(tuple(inp["v"].shape), inp["v"].dtype)
    o, S = sgla.kda_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                              initial_state=inp["initial_state"], cu_seqlens=inp["cu_seqlens"],
                              scale=inp["scale"], out=out, **kw)
    torch.cuda.synchronize()
    return o, S


def compare_chunk(inp, o, S, dtype, what, heads=None):
    ro, rS = oracle_kda(inp, heads)
    sel = (lambda t: t) if heads is None else (lambda t: t[:, :, heads])
    check(host(sel(o)), ro, dtype, what + " o")
    check(host(S if heads is None else S[:, heads]), rS, dtype, what + " final state",
          bf16_out=False)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [1, 63, 64, 65, 200, 333])
@pytest.mark.parametrize("init", [None, "normal"])
def test_kda_chunk_vs_oracle(dtype, T, init):
    say("kda_chunk_fwd B=2 H=3 D=128 T=%d %s init=%s" % (T, dtype, init))
    inp = W.make_prefill(2, T, 3, 128, 128, dtype, "kda", seed=T + 3 * (init is not None),
                         device="cuda", init=init, with_beta=True)
    o, S = run_chunk(inp)
    compare_chunk(inp, o, S, dtype, "kda T=%d" % T)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64)])
def test_kda_chunk_head_sizes(dtype, dk, dv):
    say("kda_chunk_fwd B=2 H=2 T=150", dtype, dk, dv)
    inp = W.make_prefill(2, 150, 2, dk, dv, dtype, "kda", seed=dk + dv, device="cuda",
                         init="normal", with_beta=True)
    o, S = run_chunk(inp)
    compare_chunk(inp, o, S, dtype, "kda %dx%d" % (dk, dv))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128)])
def test_kda_chunk_varlen(dtype, dk, dv):
    """Packed sequences go through the segment table (its own kernel
    variants): empty, ragged and whole-chunk sequences in one call."""
    lengths = [0, 1, 63, 64, 65, 130, 7, 200]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    say("kda_chunk_fwd varlen", dtype, dk, dv, lengths)
    inp = W.make_prefill(1, int(cu[-1]), 3, dk, dv, dtype, "kda", seed=9 + dk, device="cuda",
                         cu_seqlens=cu, init="normal", with_beta=True)
    o, S = run_chunk(inp)
    compare_chunk(inp, o, S, dtype, "kda varlen")


def test_kda_chunk_no_tokens_copies_state():
    say("kda_chunk_fwd T=0")
    inp = W.make_prefill(3, 0, 2, 128, 128, "bf16", "kda", seed=1, device="cuda", init="normal",
                         with_beta=True)
    o, S = run_chunk(inp)
    assert torch.equal(S, inp["initial_state"])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_kda_chunk_per_dim_rates(dtype):
    """Per-dim gate rates from -1e-4 to -5 per token: a chunk's gate sum
    reaches -320 in the fastest dims, where exp(G) alone underflows and
    exp(-G) overflows fp32; the slowest dims barely forget."""
    say("kda_chunk_fwd per-dim rates", dtype)
    B, T, H, D = 2, 300, 2, 128
    inp = W.make_prefill(B, T, H, D, D, dtype, "kda", seed=31, device="cuda", init="normal",
                         with_beta=True)
    rate = torch.tensor(10.0 ** np.linspace(-4, np.log10(5.0), D), dtype=torch.float32,
                        device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(31)
    inp["g"] = -(rate * (0.5 + torch.rand((B, T, H, D), generator=gen, device="cuda"))).contiguous()
    o, S = run_chunk(inp)
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()
    compare_chunk(inp, o, S, dtype, "kda per-dim rates")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_kda_chunk_gate_regimes(dtype):
    """Chunks whose gates put them on each way of forming the pairwise decay
    factors: within +-40 of the chunk's middle gate sum (one reference for
    the chunk), within 40 inside each 16-token block but not of the middle
    (one reference per block row), and wider inside a block (exponents pair
    by pair); the last chunk is ragged. Per-token gates per chunk of 64:
    -0.02 (1 +- 0.5), -1.5 (1 +- 0.125), -8 (1 +- 0.5), -0.02 (1 +- 0.5)."""
    say("kda_chunk_fwd gate regimes", dtype)
    B, T, H, D = 2, 250, 2, 128
    inp = W.make_prefill(B, T, H, D, D, dtype, "kda", seed=41, device="cuda", init="normal",
                         with_beta=True)
    gen = torch.Generator(device="cuda").manual_seed(41)
    u = torch.rand((B, T, H, D), generator=gen, device="cuda") - 0.5
    rate = torch.tensor([0.02, 1.5, 8.0, 0.02], dtype=torch.float32, device="cuda")
    spread = torch.tensor([1.0, 0.25, 1.0, 1.0], dtype=torch.float32, device="cuda")
    ch = torch.arange(T, device="cuda") // 64
    r = rate[ch].view(1, T, 1, 1)
    sp = spread[ch].view(1, T, 1, 1)
    inp["g"] = (-r * (1.0 + sp * u)).contiguous()
    o, S = run_chunk(inp)
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()
    compare_chunk(inp, o, S, dtype, "kda gate regimes")
    # Each chunk's output on its own, so that one regime cannot hide behind
    # the others' magnitudes.
    ro, _ = oracle_kda(inp)
    for c in range(4):
        sl = slice(64 * c, min(T, 64 * c + 64))
        check(host(o)[:, sl], ro[:, sl], dtype, "kda gate regimes chunk %d" % c)


def test_kda_chunk_split_chain_and_step():
    """Splitting a sequence and chaining the final state gives the same
    result, and decode steps continue a prefill."""
    say("kda_chunk_fwd split at 100 of 230, then 3 decode steps")
    inp = W.make_prefill(2, 230, 3, 128, 128, "bf16", "kda", seed=5, device="cuda",
                         init="normal", with_beta=True)
    o, S = run_chunk(inp)
    part = lambda x, sl: x[:, sl].contiguous()
    a = dict(inp, **{key: part(inp[key], slice(0, 100)) for key in ("q", "k", "v", "g", "beta")})
    b = dict(inp, **{key: part(inp[key], slice(100, 230)) for key in ("q", "k", "v", "g", "beta")})
    oa, Sa = run_chunk(a)
    b["initial_state"] = Sa
    ob, Sb = run_chunk(b)
    check(host(torch.cat([oa, ob], 1)), host(o), "bf16", "split o")
    check(host(Sb), host(S), "bf16", "split state", bf16_out=False)


def test_kda_prefill_workload_sampled():
    """B=1, T=8192, H=32, D=128 in bf16 (the prefill shape), four sampled
    heads checked against the oracle."""
    say("kda_chunk_fwd B=1 T=8192 H=32 D=128 bf16 (4 sampled heads)")
    inp = W.make_prefill(1, 8192, 32, 128, 128, "bf16", "kda", seed=2, device="cuda",
                         with_beta=True)
    o, S = run_chunk(inp)
    heads = sorted(np.random.default_rng(2).choice(32, 4, replace=False).tolist())
    compare_chunk(inp, o, S, "bf16", "kda prefill", heads=heads)

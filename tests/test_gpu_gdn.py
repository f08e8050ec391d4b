"""GPU parity of the gated delta rule (sgla_gdn_recurrent_step, sgla_gdn_chunk_fwd)
against the fp64 token-by-token oracle (oracle/gdn_oracle.c).

Inputs follow the "gdn" recipe of sgla_inputs: L2-normalised q and k rows,
v ~ N(0, 1), g = log(sigmoid(N(4, 1))) (long memory, so errors carried in
the state are not hidden by fast forgetting), beta = sigmoid(N(0, 1)). The
bars are those of the Simple GLA path: fp32 max |err| <= 1e-4 RMS; bf16
rel-L2 <= 5e-3 and max |err| <= 2e-2 RMS (plus the final bf16 rounding of
outputs), separately for outputs and final states.
"""
import numpy as np
import pytest
import torch

import linear_attention_hybrid_amd as sgla
import oracle.gdn as GDN
import sgla_inputs as W
from tests.parity import check as _check, check_windows, host, nan_like, say

pytestmark = pytest.mark.gpu


def check(got, ref, dtype, what, **kw):
    """parity.check, printing the measured errors."""
    m = _check(got, ref, dtype, what, **kw)
    say("  %-28s rel-L2 %.2e  max/RMS %.2e" % (what, m["rel_l2"],
                                               m["max_abs"] / max(m["rms_ref"], 1e-30)))
    return m


def oracle_gdn(inp, heads=None):
    sel = (lambda t: t) if heads is None else (lambda t: t[:, :, heads])
    S0 = inp["initial_state"]
    if S0 is not None:
        S0 = host(S0 if heads is None else S0[:, heads]).astype(np.float64)
    cu = None if inp["cu_seqlens"] is None else inp["cu_seqlens"].cpu().numpy()
    return GDN.forward(host(sel(inp["q"])), host(sel(inp["k"])), host(sel(inp["v"])),
                       host(sel(inp["g"])), host(sel(inp["beta"])), inp["scale"],
                       initial_state=S0, cu_seqlens=cu)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64), (128, 128)])
def test_gdn_step_with_slot_map(dtype, dk, dv):
    say("gdn_recurrent_step", dtype, dk, dv, "N=5 H=3 slots=9, 4 steps")
    N, H, slots, steps = 5, 3, 9, 4
    d = W.make_decode(N, H, dk, dv, steps, dtype, "gdn", seed=dk * 5 + dv, device="cuda",
                      slots=slots, with_beta=True)
    idx = torch.tensor([7, 0, 3, 8, 2], dtype=torch.int32, device="cuda")
    state = (d["state"] * 25).contiguous()          # unit-size states: the memory read matters
    ref_state = host(state).astype(np.float64)
    untouched = [s for s in range(slots) if s not in idx.tolist()]
    before_untouched = state[untouched].clone()
    for i in range(steps):
        out = nan_like((N, H, dv), d["v"].dtype)
        o = sgla.gdn_recurrent_step(d["q"][i], d["k"][i], d["v"][i], d["g"][i], d["beta"][i],
                                    state, state_indices=idx, scale=d["scale"], out=out)
        torch.cuda.synchronize()
        ro = GDN.step(host(d["q"][i]), host(d["k"][i]), host(d["v"][i]), host(d["g"][i]),
                      host(d["beta"][i]), ref_state, d["scale"], state_indices=idx.cpu().numpy())
        check(host(o), ro, dtype, "gdn step %d o" % i)
        check(host(state[idx.long()]), ref_state[idx.cpu().numpy()], dtype,
              "gdn step %d state" % i, bf16_out=False)
    assert torch.equal(state[untouched], before_untouched)


def test_gdn_step_equals_one_token_chunk():
    say("gdn_recurrent_step == gdn_chunk_fwd(T=1)")
    N, H, D = 4, 2, 128
    d = W.make_decode(N, H, D, D, 1, "bf16", "gdn", seed=23, device="cuda", with_beta=True)
    S0 = (d["state"] * 25).contiguous()
    state = S0.clone()
    o_step = sgla.gdn_recurrent_step(d["q"][0], d["k"][0], d["v"][0], d["g"][0], d["beta"][0],
                                     state)
    one = lambda t: t[0][:, None].contiguous()
    o_chunk, S_chunk = sgla.gdn_chunk_fwd(one(d["q"]), one(d["k"]), one(d["v"]), one(d["g"]),
                                          one(d["beta"]), initial_state=S0)
    torch.cuda.synchronize()
    check(host(o_step), host(o_chunk[:, 0]), "bf16", "step vs chunk o")
    check(host(state), host(S_chunk), "bf16", "step vs chunk state", bf16_out=False)


@pytest.mark.parametrize("T", [1, 63, 64, 200, 333])
@pytest.mark.parametrize("init", [None, "normal"])
def test_gdn_chunk_vs_oracle(T, init):
    say("gdn_chunk_fwd B=2 H=3 T=%d init=%s" % (T, init))
    inp = W.make_prefill(2, T, 3, 128, 128, "bf16", "gdn", seed=T + (init is not None),
                         device="cuda", init=init, with_beta=True)
    if init is not None:
        inp["initial_state"] = inp["initial_state"] * 25
    out = nan_like((2, T, 3, 128), torch.bfloat16)
    o, S = sgla.gdn_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                              initial_state=inp["initial_state"], out=out)
    torch.cuda.synchronize()
    ro, rS = oracle_gdn(inp)
    check(host(o), ro, "bf16", "gdn o")
    check(host(S), rS, "bf16", "gdn final state", bf16_out=False)
    for b in range(2):
        check_windows(host(o[b]), ro[b], [0], "bf16", "gdn o seq %d" % b)


def test_gdn_chunk_odd_batch_and_heads():
    """B * H = 25 (the chain rounds its (sequence, head) units up to groups of
    eight) and T = 100 (a ragged second chunk), with an initial state."""
    say("gdn_chunk_fwd B=5 H=5 T=100 init")
    inp = W.make_prefill(5, 100, 5, 128, 128, "bf16", "gdn", seed=55, device="cuda",
                         init="normal", with_beta=True)
    inp["initial_state"] = inp["initial_state"] * 25
    o, S = sgla.gdn_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                              initial_state=inp["initial_state"],
                              out=nan_like((5, 100, 5, 128), torch.bfloat16))
    torch.cuda.synchronize()
    ro, rS = oracle_gdn(inp)
    check(host(o), ro, "bf16", "gdn 5x5 o")
    check(host(S), rS, "bf16", "gdn 5x5 final state", bf16_out=False)


def test_gdn_chunk_many_short_sequences():
    """40 packed sequences of 0 .. 130 tokens and 3 heads: many chains, most of
    them one or two chunks long, each checked against the oracle."""
    rng = np.random.default_rng(40)
    lengths = [int(x) for x in rng.integers(0, 131, size=40)]
    lengths[3] = 0
    lengths[7] = 64
    say("gdn_chunk_fwd varlen 40 sequences, %d tokens, H=3" % sum(lengths))
    cu = W.cu_from_lengths(lengths)
    T = int(cu[-1])
    inp = W.make_prefill(1, T, 3, 128, 128, "bf16", "gdn", seed=41, device="cuda",
                         cu_seqlens=cu, init="normal", with_beta=True)
    inp["initial_state"] = inp["initial_state"] * 25
    o, S = sgla.gdn_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                              initial_state=inp["initial_state"], cu_seqlens=inp["cu_seqlens"],
                              out=nan_like((1, T, 3, 128), torch.bfloat16))
    torch.cuda.synchronize()
    ro, rS = oracle_gdn(inp)
    check(host(o), ro, "bf16", "gdn 40 seqs o")
    check(host(S), rS, "bf16", "gdn 40 seqs states", bf16_out=False)
    assert torch.equal(S[3], inp["initial_state"][3])


def test_gdn_chunk_varlen_packed_equals_separate():
    lengths = [0, 1, 63, 64, 65, 130, 200, 7]
    say("gdn_chunk_fwd varlen", lengths)
    cu = W.cu_from_lengths(lengths)
    T = int(cu[-1])
    H = 2
    inp = W.make_prefill(1, T, H, 128, 128, "bf16", "gdn", seed=77, device="cuda",
                         cu_seqlens=cu, init="normal", with_beta=True)
    inp["initial_state"] = inp["initial_state"] * 25
    o, S = sgla.gdn_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                              initial_state=inp["initial_state"], cu_seqlens=inp["cu_seqlens"])
    torch.cuda.synchronize()
    ro, rS = oracle_gdn(inp)
    check(host(o), ro, "bf16", "gdn varlen o")
    check(host(S), rS, "bf16", "gdn varlen states", bf16_out=False)
    check_windows(host(o[0]), ro[0], [int(c) for c in cu[:-1]], "bf16", "gdn varlen o",
                  ends=[int(c) for c in cu[1:]])
    # Each sequence on its own: the same chunks, the same arithmetic, bit for bit.
    for i, L in enumerate(lengths):
        a, b = int(cu[i]), int(cu[i + 1])
        part = lambda t: t[:, a:b].contiguous()
        oi, Si = sgla.gdn_chunk_fwd(part(inp["q"]), part(inp["k"]), part(inp["v"]),
                                    part(inp["g"]), part(inp["beta"]),
                                    initial_state=inp["initial_state"][i:i + 1].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(oi[0], o[0, a:b]), i
        assert torch.equal(Si[0], S[i]), i
    # An empty sequence keeps its initial state.
    assert torch.equal(S[0], inp["initial_state"][0])


def test_gdn_chunk_split_chain_and_in_place():
    say("gdn_chunk_fwd split at 128 and chained, final_state in place")
    T, H = 320, 2
    inp = W.make_prefill(1, T, H, 128, 128, "bf16", "gdn", seed=91, device="cuda",
                         init="normal", with_beta=True)
    S0 = inp["initial_state"] * 25
    o_all, S_all = sgla.gdn_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                      initial_state=S0)
    S = S0.clone()
    part = lambda t, a, b: t[:, a:b].contiguous()
    o1, _ = sgla.gdn_chunk_fwd(*(part(inp[x], 0, 128) for x in ("q", "k", "v", "g", "beta")),
                               initial_state=S, final_state=S)
    o2, _ = sgla.gdn_chunk_fwd(*(part(inp[x], 128, T) for x in ("q", "k", "v", "g", "beta")),
                               initial_state=S, final_state=S)
    torch.cuda.synchronize()
    # A split on a chunk boundary sees the same chunks: identical results.
    assert torch.equal(torch.cat([o1, o2], dim=1), o_all)
    assert torch.equal(S, S_all)


def test_gdn_chunk_no_tokens_copies_state():
    say("gdn_chunk_fwd T=0 with a final state")
    H = 3
    S0 = torch.randn((2, H, 128, 128), device="cuda")
    z = torch.empty((2, 0, H, 128), dtype=torch.bfloat16, device="cuda")
    zg = torch.empty((2, 0, H), dtype=torch.float32, device="cuda")
    o, S = sgla.gdn_chunk_fwd(z, z, z, zg, zg, initial_state=S0)
    torch.cuda.synchronize()
    assert o.shape == (2, 0, H, 128)
    assert torch.equal(S, S0)


def test_gdn_chunk_prefill_workload_sampled():
    """The lightning-prefill shape (B=1, T=8192, H=32, Dk=Dv=128) with GDN
    inputs; the oracle runs 4 seeded heads in full."""
    say("gdn_chunk_fwd B=1 T=8192 H=32 D=128 seed=5 (4 heads checked)")
    inp = W.make_prefill(1, 8192, 32, 128, 128, "bf16", "gdn", seed=5, device="cuda",
                         with_beta=True)
    o, S = sgla.gdn_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"])
    torch.cuda.synchronize()
    heads = np.sort(np.random.default_rng(5).choice(32, size=4, replace=False))
    ro, rS = oracle_gdn(inp, heads=heads)
    check(host(o[:, :, heads]), ro, "bf16", "gdn prefill o")
    check(host(S[:, heads]), rS, "bf16", "gdn prefill state", bf16_out=False)


def test_gdn_chunk_most_heads():
    """H = 65536, the most heads a call takes, and T = 70 (a full chunk and a
    ragged one): the prep kernel's per-item byte ranges and row offsets are at
    their largest (about 2^30), and the chain runs 2^19 workgroups."""
    say("gdn_chunk_fwd bf16 B=1 T=70 H=65536 D=128 seed=78 (4 sampled heads)")
    inp = W.make_prefill(1, 70, 65536, 128, 128, "bf16", "gdn", seed=78, device="cuda",
                         init="normal", with_beta=True)
    o, S = sgla.gdn_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                              initial_state=inp["initial_state"],
                              out=nan_like((1, 70, 65536, 128), torch.bfloat16))
    torch.cuda.synchronize()
    heads = [0, 1, 40961, 65535]
    ro, rS = oracle_gdn(inp, heads=heads)
    check(host(o[:, :, heads]), ro, "bf16", "gdn H=65536 o")
    check(host(S[:, heads]), rS, "bf16", "gdn H=65536 final state", bf16_out=False)
    del inp, o, S
    torch.cuda.empty_cache()


def _sample_heads(H, n, seed):
    return np.sort(np.random.default_rng(seed).choice(H, size=n, replace=False))


def test_gdn_long_continuation_and_split():
    """The long-continuation shape (B=1, T=65536, H=32, Dk=Dv=128) from a
    nonzero initial state, 1,024 chunks per chain; the oracle runs 2 seeded
    heads in full. Split at 32768 and chained, the result is bit for bit the
    same (the split falls on a chunk boundary)."""
    say("gdn_chunk_fwd B=1 T=65536 H=32 D=128 S0 seed=6 (2 heads checked), split at 32768")
    inp = W.make_prefill(1, 65536, 32, 128, 128, "bf16", "gdn", seed=6, device="cuda",
                         init="normal", with_beta=True)
    inp["initial_state"] = inp["initial_state"] * 25
    o, S = sgla.gdn_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                              initial_state=inp["initial_state"])
    torch.cuda.synchronize()
    heads = _sample_heads(32, 2, 6)
    ro, rS = oracle_gdn(inp, heads=heads)
    check(host(o[:, :, heads]), ro, "bf16", "gdn 64k o")
    check(host(S[:, heads]), rS, "bf16", "gdn 64k state", bf16_out=False)
    check_windows(host(o[0][:, heads]), ro[0], [0], "bf16", "gdn 64k o")
    t = 32768
    part = lambda x, a, b: inp[x][:, a:b].contiguous()
    oa, Sa = sgla.gdn_chunk_fwd(*(part(x, 0, t) for x in ("q", "k", "v", "g", "beta")),
                                initial_state=inp["initial_state"])
    ob, Sb = sgla.gdn_chunk_fwd(*(part(x, t, 65536) for x in ("q", "k", "v", "g", "beta")),
                                initial_state=Sa)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([oa, ob], dim=1), o)
    assert torch.equal(Sb, S)


def test_gdn_varlen_sampled():
    """Eight packed sequences of log-uniform lengths in [512, 16384] rescaled to
    65,536 tokens, H=32, each with its own initial state; the oracle runs 3
    seeded heads, every sequence start windowed."""
    lengths = W.varlen_lengths(8, 65536, 512, 16384, seed=8)
    say("gdn_chunk_fwd varlen 8 seqs 65536 tokens H=32 seed=8 (3 heads)", list(lengths))
    cu = W.cu_from_lengths(lengths)
    inp = W.make_prefill(1, 65536, 32, 128, 128, "bf16", "gdn", seed=8, device="cuda",
                         cu_seqlens=cu, init="normal", with_beta=True)
    inp["initial_state"] = inp["initial_state"] * 25
    o, S = sgla.gdn_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                              initial_state=inp["initial_state"], cu_seqlens=inp["cu_seqlens"])
    torch.cuda.synchronize()
    heads = _sample_heads(32, 3, 8)
    ro, rS = oracle_gdn(inp, heads=heads)
    check(host(o[:, :, heads]), ro, "bf16", "gdn varlen 64k o")
    check(host(S[:, heads]), rS, "bf16", "gdn varlen 64k states", bf16_out=False)
    check_windows(host(o[0][:, heads]), ro[0], [int(c) for c in cu[:-1]], "bf16",
                  "gdn varlen 64k o", ends=[int(c) for c in cu[1:]])


def test_gdn_per_head_constant_decay():
    """The gated delta rule with the lightning layer's spread of per-head
    constant decays (blueprint page, section "B2 lightning-attn (Simple GLA)":
    -0.917 .. -0.0001), chunked prefill and decode steps from its final state."""
    say("gdn constant per-head decay B=2 T=700 H=8")
    H = 8
    inp = W.make_prefill(2, 700, H, 128, 128, "bf16", "gdn", seed=71, device="cuda",
                         init="normal", with_beta=True)
    gg = torch.tensor(-0.917 * (0.0001 / 0.917) ** (np.arange(H) / (H - 1)),
                      dtype=torch.float32, device="cuda")
    inp["g"] = gg.view(1, 1, H).expand_as(inp["g"]).contiguous()
    o, S = sgla.gdn_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                              initial_state=inp["initial_state"])
    torch.cuda.synchronize()
    ro, rS = oracle_gdn(inp)
    check(host(o), ro, "bf16", "gdn constant decay o")
    check(host(S), rS, "bf16", "gdn constant decay state", bf16_out=False)
    d = W.make_decode(2, H, 128, 128, 4, "bf16", "gdn", seed=72, device="cuda", with_beta=True)
    g = gg.view(1, H).expand(2, H).contiguous()
    state = S.clone()
    ref = np.ascontiguousarray(rS.astype(np.float64))
    for i in range(4):
        od = sgla.gdn_recurrent_step(d["q"][i], d["k"][i], d["v"][i], g, d["beta"][i], state)
        torch.cuda.synchronize()
        ro_i = GDN.step(host(d["q"][i]), host(d["k"][i]), host(d["v"][i]), host(g),
                        host(d["beta"][i]), ref, d["scale"])
        check(host(od), ro_i, "bf16", "gdn constant decay step %d" % i)

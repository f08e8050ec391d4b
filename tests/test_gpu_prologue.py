"""GPU parity of the q/k prologue entry points (per-head RMSNorm and RoPE
applied inside the kernels) against the oracle: ``oracle/prologue.py`` turns
the raw q and k into the bf16 values the recurrence consumes, then the
recurrence oracle runs on them. Same bars as the other bf16 cases.

The prologue ends in two bf16 roundings. The kernels take them from fp32
values, the oracle from fp64 ones, so an element whose exact value lies very
near a midpoint between two bf16 numbers may round either way; both are
correct. How near: the fp32 path's error relative to the size of its inputs
is a few fp32 units (sum of squares and reciprocal square root for RMSNorm,
about 2^-22; the angle reduced in fp64 then carried in fp32 turns, about
2^-24; the hardware sine and cosine, about 2^-23; at most two turns by
per-frequency constants, each a few 2^-24), together under 2^-21, so the band
is TIE_ETA = 2^-20 times the size of the inputs, with a factor 2 to spare.
The standalone prologue test checks that band directly: every element the
kernels round differently from the oracle lies inside it.

The oracle bounds what a flagged element can change (``qk_prologue(...,
tie_eta)``), and three more runs of the recurrence oracle on absolute values
bound the effect on every output and state element (flips in k, flips in q,
both); that bound is added per element to the max-abs bar, and its median
must stay below a tenth of the bar. Every other element keeps the plain bar,
and rel-L2 is not relaxed.
"""
import os

import numpy as np
import pytest
import torch

import linear_attention_hybrid_amd as sgla
import oracle
import oracle.prologue as OP
import sgla_inputs as W
from tests.parity import check, host, nan_like, say

pytestmark = pytest.mark.gpu

THETA, EPS = 10000.0, 1e-6
TIE_ETA = 2.0 ** -20
MEDIAN_CAP = 0.1  # allowance median / max-abs bar


@pytest.fixture(autouse=True)
def _seg_len_env():
    old = os.environ.pop("SGLA_SEG_LEN", None)
    yield
    os.environ.pop("SGLA_SEG_LEN", None)
    if old is not None:
        os.environ["SGLA_SEG_LEN"] = old


def token_positions(B, T, cu, pos_off):
    """Position of every token in packed order: its sequence's offset plus its
    index inside the sequence."""
    off = np.zeros(B if cu is None else len(cu) - 1, np.int64)
    if pos_off is not None:
        off[:] = pos_off.cpu().numpy()
    if cu is None:
        return (np.arange(T)[None, :] + off[:, None]).reshape(-1)
    seq = np.searchsorted(cu, np.arange(T), side="right") - 1
    return OP.sequence_positions(T, cu) + off[seq]


def oracle_with_prologue(inp, qw, kw, pos_off, heads=None):
    """(o, S, allowance of o, allowance of S) from the oracle."""
    B, T, H, D = inp["q"].shape
    hs = list(range(H)) if heads is None else list(heads)
    cu = None if inp["cu_seqlens"] is None else inp["cu_seqlens"].cpu().numpy()
    pos = token_positions(B, T, cu, pos_off)
    q, qb = OP.qk_prologue(host(inp["q"][:, :, hs]), host(qw), pos, THETA, EPS, TIE_ETA)
    k, kb = OP.qk_prologue(host(inp["k"][:, :, hs]), host(kw), pos, THETA, EPS, TIE_ETA)
    v = host(inp["v"][:, :, hs])
    g = host(inp["g"][:, :, hs])
    S0 = inp["initial_state"]
    if S0 is not None:
        S0 = host(S0[:, hs]).astype(np.float64)
    f32 = lambda a: np.abs(a).astype(np.float32)
    ro, rS = oracle.forward(q.astype(np.float32), k.astype(np.float32), v, g, inp["scale"],
                            initial_state=S0, cu_seqlens=cu)
    a1, s1 = oracle.forward(f32(q), f32(kb), f32(v), g, inp["scale"], cu_seqlens=cu)
    a2, _ = oracle.forward(f32(qb), f32(k), f32(v), g, inp["scale"],
                           initial_state=None if S0 is None else np.abs(S0), cu_seqlens=cu)
    a3, _ = oracle.forward(f32(qb), f32(kb), f32(v), g, inp["scale"], cu_seqlens=cu)
    return ro, rS, a1 + a2 + a3, s1


def run_chunk(inp, qw, kw, pos_off):
    B, T, H, Dk = inp["q"].shape
    N = B if inp["cu_seqlens"] is None else inp["cu_seqlens"].numel() - 1
    out = nan_like((B, T, H, Dk), inp["v"].dtype)
    fs = nan_like((N, H, Dk, Dk), torch.float32)
    o, S = sgla.chunk_fwd_qk_norm_rope(inp["q"], inp["k"], inp["v"], inp["g"], qw, kw,
                                       pos_offset=pos_off, theta=THETA, eps=EPS,
                                       initial_state=inp["initial_state"],
                                       cu_seqlens=inp["cu_seqlens"], scale=inp["scale"], out=out,
                                       final_state=fs)
    torch.cuda.synchronize()
    return o, S


def compare(inp, o, S, ref, what, heads=None, starts=None):
    ro, rS, ao, aS = ref
    go = host(o if heads is None else o[:, :, heads])
    m = check(go, ro, "bf16", what + " o", allowance=ao, max_allowance_median=MEDIAN_CAP)
    say("  %s o: allowance/bar median %.3g max %.3g, over the bar %.4f" % (
        what, m["allowance_median_over_bar"], m["allowance_max_over_bar"],
        m["allowance_frac_over_bar"]))
    check(host(S if heads is None else S[:, heads]), rS, "bf16", what + " final state",
          bf16_out=False, allowance=aS, max_allowance_median=MEDIAN_CAP)
    if starts:
        for s0 in starts:
            for w in (64, 256):
                e = min(go.shape[1], s0 + w)
                if e > s0:
                    check(go[0, s0:e], ro[0, s0:e], "bf16", "%s o window [%d,%d)" % (what, s0, e),
                          allowance=ao[0, s0:e])


@pytest.mark.parametrize("seg_len", [None, 128])
def test_rows_with_offsets(seg_len):
    say("chunk_fwd_qk_norm_rope B=2 T=300 H=3, offsets 0 and 123456, seg_len", seg_len)
    if seg_len:
        os.environ["SGLA_SEG_LEN"] = str(seg_len)
    inp = W.make_prefill(2, 300, 3, 128, 128, "bf16", "raw", seed=31, device="cuda",
                         init="normal")
    qw, kw = W.norm_weights(128, seed=31, device="cuda")
    pos_off = torch.tensor([0, 123456], dtype=torch.int32, device="cuda")
    o, S = run_chunk(inp, qw, kw, pos_off)
    compare(inp, o, S, oracle_with_prologue(inp, qw, kw, pos_off), "rows", starts=[0])


def test_varlen_with_offsets_and_segments():
    lengths = [0, 1, 63, 65, 200, 0, 700, 129]
    cu = W.cu_from_lengths(lengths)
    T = int(cu[-1])
    say("chunk_fwd_qk_norm_rope varlen", lengths, "seg_len 128")
    os.environ["SGLA_SEG_LEN"] = "128"
    inp = W.make_prefill(1, T, 4, 128, 128, "bf16", "raw", seed=32, device="cuda",
                         cu_seqlens=cu, init="normal")
    qw, kw = W.norm_weights(128, seed=32, device="cuda")
    pos_off = torch.tensor([5, 0, 77, 1 << 20, 9, 3, 4096, 65536], dtype=torch.int32,
                           device="cuda")
    o, S = run_chunk(inp, qw, kw, pos_off)
    compare(inp, o, S, oracle_with_prologue(inp, qw, kw, pos_off), "varlen",
            starts=[int(c) for c in cu[:-1]])


def test_positions_near_the_int32_limit():
    """Angles of positions close to 2^31: the fp64 reduction must keep them."""
    say("chunk_fwd_qk_norm_rope positions near 2^31")
    inp = W.make_prefill(1, 256, 2, 128, 128, "bf16", "raw", seed=33, device="cuda")
    qw, kw = W.norm_weights(128, seed=33, device="cuda")
    pos_off = torch.tensor([(1 << 31) - 300], dtype=torch.int32, device="cuda")
    o, S = run_chunk(inp, qw, kw, pos_off)
    compare(inp, o, S, oracle_with_prologue(inp, qw, kw, pos_off), "near 2^31")


def test_null_offsets_equal_zero_offsets():
    say("chunk_fwd_qk_norm_rope pos_offset None == zeros")
    inp = W.make_prefill(3, 130, 2, 128, 128, "bf16", "raw", seed=34, device="cuda")
    qw, kw = W.norm_weights(128, seed=34, device="cuda")
    o1, S1 = run_chunk(inp, qw, kw, None)
    o2, S2 = run_chunk(inp, qw, kw, torch.zeros(3, dtype=torch.int32, device="cuda"))
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_split_and_continue():
    """A sequence split in two calls, the second passing the first call's
    final state and the count of tokens before it as its offset."""
    say("chunk_fwd_qk_norm_rope split at 600 of 1000")
    inp = W.make_prefill(1, 1000, 3, 128, 128, "bf16", "raw", seed=35, device="cuda")
    qw, kw = W.norm_weights(128, seed=35, device="cuda")
    ro, rS, ao, aS = oracle_with_prologue(inp, qw, kw, None)
    t = 600
    a, b = dict(inp), dict(inp)
    for x in ("q", "k", "v", "g"):
        a[x] = inp[x][:, :t].contiguous()
        b[x] = inp[x][:, t:].contiguous()
    oa, Sa = run_chunk(a, qw, kw, None)
    b["initial_state"] = Sa
    ob, Sb = run_chunk(b, qw, kw, torch.tensor([t], dtype=torch.int32, device="cuda"))
    go = host(torch.cat([oa, ob], dim=1))
    check(go, ro, "bf16", "split o", allowance=ao, max_allowance_median=MEDIAN_CAP)
    check(host(Sb), rS, "bf16", "split state", bf16_out=False, allowance=aS,
          max_allowance_median=MEDIAN_CAP)
    for w in (64, 256):
        check(go[0, t:t + w], ro[0, t:t + w], "bf16", "split window %d" % w,
              allowance=ao[0, t:t + w])


def test_workload_prefill_8k_sampled_heads():
    say("chunk_fwd_qk_norm_rope H=32 T=8192 raw q/k seed=2 (4 sampled heads)")
    inp = W.make_prefill(1, 8192, 32, 128, 128, "bf16", "raw", seed=2, device="cuda")
    qw, kw = W.norm_weights(128, seed=2, device="cuda")
    o, S = run_chunk(inp, qw, kw, None)
    heads = sorted(np.random.default_rng(2).choice(32, size=4, replace=False).tolist())
    compare(inp, o, S, oracle_with_prologue(inp, qw, kw, None, heads=heads), "prefill 8k",
            heads=heads)


def oracle_step_with_prologue(d, i, qw, kw, pos, state, idx=None):
    """Oracle decode step (updates ``state``); returns (o, allowance of o,
    allowance of the state rows)."""
    p = pos.cpu().numpy().astype(np.int64)
    q, qb = OP.qk_prologue(host(d["q"][i])[:, None], host(qw), p, THETA, EPS, TIE_ETA)
    k, kb = OP.qk_prologue(host(d["k"][i])[:, None], host(kw), p, THETA, EPS, TIE_ETA)
    q, qb, k, kb = q[:, 0], qb[:, 0], k[:, 0], kb[:, 0]
    v, g = host(d["v"][i]), host(d["g"][i])
    ix = None if idx is None else idx.cpu().numpy()
    rows = np.arange(q.shape[0]) if ix is None else ix
    f32 = lambda a: np.abs(a).astype(np.float32)
    zero = np.zeros_like(state)
    s1 = zero.copy()
    a1 = oracle.step(f32(q), f32(kb), f32(v), g, s1, d["scale"], state_indices=ix)
    a2 = oracle.step(f32(qb), f32(k), f32(v), g, np.abs(state), d["scale"], state_indices=ix)
    a3 = oracle.step(f32(qb), f32(kb), f32(v), g, zero.copy(), d["scale"], state_indices=ix)
    o = oracle.step(q.astype(np.float32), k.astype(np.float32), v, g, state, d["scale"],
                    state_indices=ix)
    return o, a1 + a2 + a3, s1[rows]


@pytest.mark.parametrize("dv", [64, 128])
def test_step_with_slot_map(dv):
    say("recurrent_step_qk_norm_rope N=5 H=3 Dv=%d slots=9, 3 steps" % dv)
    N, H, slots, steps = 5, 3, 9, 3
    d = W.make_decode(N, H, 128, dv, steps, "bf16", "raw", seed=40 + dv, device="cuda",
                      slots=slots)
    qw, kw = W.norm_weights(128, seed=40 + dv, device="cuda")
    idx = torch.tensor([7, 0, 3, 8, 2], dtype=torch.int32, device="cuda")
    pos = torch.tensor([0, 1, 4095, 1 << 24, (1 << 31) - 10], dtype=torch.int32, device="cuda")
    state = d["state"].clone()
    ref_state = host(state).astype(np.float64)
    for i in range(steps):
        out = nan_like((N, H, dv), torch.bfloat16)
        o = sgla.recurrent_step_qk_norm_rope(d["q"][i], d["k"][i], d["v"][i], d["g"][i], state,
                                             qw, kw, pos + i, theta=THETA, eps=EPS,
                                             state_indices=idx, scale=d["scale"], out=out)
        torch.cuda.synchronize()
        ro, ao, aS = oracle_step_with_prologue(d, i, qw, kw, pos + i, ref_state, idx)
        check(host(o), ro, "bf16", "step %d o" % i, allowance=ao,
              max_allowance_median=MEDIAN_CAP)
        check(host(state[idx.long()]), ref_state[idx.cpu().numpy()], "bf16",
              "step %d state" % i, bf16_out=False, allowance=aS, max_allowance_median=MEDIAN_CAP)


def test_step_equals_one_token_chunk():
    say("recurrent_step_qk_norm_rope == chunk_fwd_qk_norm_rope(T=1)")
    N, H = 4, 2
    d = W.make_decode(N, H, 128, 128, 1, "bf16", "raw", seed=41, device="cuda")
    qw, kw = W.norm_weights(128, seed=41, device="cuda")
    pos = torch.tensor([3, 70000, 0, 999], dtype=torch.int32, device="cuda")
    state = d["state"].clone()
    o_step = sgla.recurrent_step_qk_norm_rope(d["q"][0], d["k"][0], d["v"][0], d["g"][0], state,
                                              qw, kw, pos, theta=THETA, eps=EPS)
    o_chunk, S_chunk = sgla.chunk_fwd_qk_norm_rope(
        d["q"][0][:, None].contiguous(), d["k"][0][:, None].contiguous(),
        d["v"][0][:, None].contiguous(), d["g"][0][:, None].contiguous(), qw, kw,
        pos_offset=pos, theta=THETA, eps=EPS, initial_state=d["state"])
    torch.cuda.synchronize()
    check(host(o_step), host(o_chunk[:, 0]), "bf16", "step vs chunk o")
    check(host(state), host(S_chunk), "bf16", "step vs chunk state", bf16_out=False)


def test_workload_decode_one_step():
    """One step of the batched-decode shape (256 x 32 heads) with the
    prologue, every (row, head) against the oracle."""
    say("recurrent_step_qk_norm_rope N=256 H=32 D=128 one step, positions 100000")
    d = W.make_decode(256, 32, 128, 128, 1, "bf16", "raw", seed=42, device="cuda")
    qw, kw = W.norm_weights(128, seed=42, device="cuda")
    state = d["state"].clone()
    ref_state = host(state).astype(np.float64)
    o = sgla.recurrent_step_qk_norm_rope(d["q"][0], d["k"][0], d["v"][0], d["g"][0], state, qw,
                                         kw, d["pos"][0], theta=THETA, eps=EPS)
    torch.cuda.synchronize()
    ro, ao, aS = oracle_step_with_prologue(d, 0, qw, kw, d["pos"][0], ref_state)
    m = check(host(o), ro, "bf16", "decode o", allowance=ao, max_allowance_median=MEDIAN_CAP)
    say("  decode o: allowance/bar median %.3g max %.3g" % (m["allowance_median_over_bar"],
                                                          m["allowance_max_over_bar"]))
    check(host(state), ref_state, "bf16", "decode state", bf16_out=False, allowance=aS,
          max_allowance_median=MEDIAN_CAP)


@pytest.mark.parametrize("B,T,H,offsets", [(1, 2048, 2, [123456]), (2, 300, 3, [0, (1 << 31) - 400]),
                                           (1, 8192, 4, None)])
def test_standalone_prologue_is_the_oracle_bit_for_bit_outside_the_tie_band(B, T, H, offsets):
    """sgla_qk_norm_rope runs the chunked kernels' own prologue code. Its bf16
    output equals the oracle's exactly, except on elements the oracle flags
    as within TIE_ETA of a rounding midpoint (at either rounding); this is
    the evidence for the band the other prologue tests use."""
    say("qk_norm_rope B=%d T=%d H=%d offsets %s" % (B, T, H, offsets))
    inp = W.make_prefill(B, T, H, 128, 128, "bf16", "raw", seed=T + H, device="cuda")
    qw, kw = W.norm_weights(128, seed=T + H, device="cuda")
    pos_off = None if offsets is None else torch.tensor(offsets, dtype=torch.int32, device="cuda")
    pos = token_positions(B, T, None, pos_off)
    total = flagged = differ = 0
    for name, x, w in (("q", inp["q"], qw), ("k", inp["k"], kw)):
        got = host(sgla.qk_norm_rope(x, w, pos_off, THETA, EPS))
        torch.cuda.synchronize()
        ref, bound = OP.qk_prologue(host(x), host(w), pos, THETA, EPS, TIE_ETA)
        diff = got != ref
        flag = bound > 0
        outside = diff & ~flag
        assert not np.any(outside), (name, int(outside.sum()), np.argwhere(outside)[:5])
        total += got.size
        flagged += int(flag.sum())
        differ += int(diff.sum())
    say("  %d elements, %d (%.3f%%) flagged near a tie, %d differ from the oracle" % (
        total, flagged, 100.0 * flagged / total, differ))
    # In place gives the same bits.
    y = inp["q"].clone()
    sgla.qk_norm_rope(y, qw, pos_off, THETA, EPS, out=y)
    assert torch.equal(y, sgla.qk_norm_rope(inp["q"], qw, pos_off, THETA, EPS))

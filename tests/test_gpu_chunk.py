"""GPU parity of sgla_chunk_fwd against the oracle (through the C ABI).

Small cases compare every output and final-state element; the named full-size
workloads compare a seeded sample of heads (every token and state element of
those heads) with the oracle, in the launch configuration the benchmark times.
"""
import os

import numpy as np
import pytest
import torch

import linear_attention_hybrid_amd as sgla
import sgla_inputs as W
from tests.parity import check, check_windows, host, nan_like, oracle_prefill, say

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "bf16": torch.bfloat16}


SEG_ENV = ("SGLA_SEG_LEN", "SGLA_OUT_SEG_LEN", "SGLA_RSUB", "SGLA_ONE_LEVEL", "SGLA_VALUE_HALVES")


@pytest.fixture(autouse=True)
def _seg_len_env():
    old = {k: os.environ.pop(k, None) for k in SEG_ENV}
    yield
    for k in SEG_ENV:
        os.environ.pop(k, None)
        if old[k] is not None:
            os.environ[k] = old[k]


def set_segments(seg_len, rsub=None):
    """Segment lengths for both prefill paths: SGLA_SEG_LEN for the one-level
    kernels (fp32, 64-wide heads, the prologue), SGLA_OUT_SEG_LEN (and the
    number of state-pass sub-segments per output segment, SGLA_RSUB) for the
    bf16 value-half kernel."""
    os.environ["SGLA_SEG_LEN"] = str(seg_len)
    os.environ["SGLA_OUT_SEG_LEN"] = str(seg_len)
    if rsub is not None:
        os.environ["SGLA_RSUB"] = str(rsub)


def run_gpu(inp, poison=True, final=True):
    B, T, H, Dk = inp["q"].shape
    Dv = inp["v"].shape[-1]
    N = B if inp["cu_seqlens"] is None else inp["cu_seqlens"].numel() - 1
    out = nan_like((B, T, H, Dv), inp["v"].dtype) if poison else None
    fs = nan_like((N, H, Dk, Dv), torch.float32) if (poison and final) else None
    o, S = sgla.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"],
                          initial_state=inp["initial_state"], cu_seqlens=inp["cu_seqlens"],
                          scale=inp["scale"], out=out, final_state=fs, output_final_state=final)
    torch.cuda.synchronize()
    return o, S


def compare(inp, o, S, dtype, what, heads=None, starts=None):
    ro, rS = oracle_prefill(inp, heads)
    go = host(o if heads is None else o[:, :, heads])
    check(go, ro, dtype, what + " o")
    if S is not None:
        gS = host(S if heads is None else S[:, heads])
        check(gS, rS, dtype, what + " final state", bf16_out=False)
    if starts:
        check_windows(go[0], ro[0], starts, dtype, what + " o")
    return ro, rS


def test_tiny_fp32_workload():
    say("chunk_fwd tiny fp32 B=1 H=4 T=256 D=64 seed=1")
    inp = W.make_workload("tiny_fp32_h4_t256_d64", seed=1, device="cuda")
    o, S = run_gpu(inp)
    compare(inp, o, S, "f32", "tiny fp32")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [1, 63, 64, 65, 127, 129, 300])
def test_edge_lengths(dtype, T):
    say("chunk_fwd edge", dtype, "B=2 H=3 T=%d D=128/64 S0" % T)
    inp = W.make_prefill(2, T, 3, 128, 64, dtype, "lightning", seed=T, device="cuda",
                         init="normal")
    o, S = run_gpu(inp)
    compare(inp, o, S, dtype, "edge T=%d" % T)


@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64), (128, 128)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_head_sizes(dk, dv, dtype):
    say("chunk_fwd head sizes", dtype, dk, dv)
    inp = W.make_prefill(1, 200, 2, dk, dv, dtype, "gaussian", seed=dk + dv, device="cuda",
                         init="normal")
    o, S = run_gpu(inp)
    compare(inp, o, S, dtype, "Dk=%d Dv=%d" % (dk, dv))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("seg_len", [64, 128, 512])
def test_multi_segment_state_passing(dtype, seg_len):
    """Force short segments so sequences span several workgroups and the
    carried state goes through the segment scan."""
    say("chunk_fwd segments", dtype, "seg_len", seg_len)
    set_segments(seg_len)
    T = 1000
    inp = W.make_prefill(2, T, 3, 128, 128, dtype, "lightning", seed=seg_len, device="cuda",
                         init="normal")
    o, S = run_gpu(inp)
    starts = [0] + list(range(seg_len, T, seg_len))
    ro, rS = compare(inp, o, S, dtype, "segments %d" % seg_len, starts=starts)


@pytest.mark.parametrize("oseg,rsub", [(128, 1), (128, 2), (256, 4), (512, 2), (1024, 4),
                                       (640, 5)])
def test_value_half_segments_and_sub_segments(oseg, rsub):
    """The bf16 value-half path with a sequence over several output segments:
    the state pass runs over rsub sub-segments per output segment and the
    scan keeps only the output segments' start states."""
    say("chunk_fwd value halves oseg", oseg, "rsub", rsub, "B=2 T=1700 H=3 S0")
    set_segments(oseg, rsub)
    T = 1700
    inp = W.make_prefill(2, T, 3, 128, 128, "bf16", "lightning", seed=oseg + rsub, device="cuda",
                         init="normal")
    o, S = run_gpu(inp)
    compare(inp, o, S, "bf16", "halves %d/%d" % (oseg, rsub),
            starts=[0] + list(range(oseg, T, oseg)))


@pytest.mark.parametrize("dtype,path", [("f32", None), ("bf16", "one_level"), ("bf16", "halves")])
def test_varlen_packed_matches_oracle_and_separate_runs(dtype, path):
    """Packed sequences on each bf16 path: the one-level kernels (the default
    with cu_seqlens) and the value-half kernels (the default without)."""
    if path == "halves":
        os.environ["SGLA_VALUE_HALVES"] = "1"
    else:
        os.environ["SGLA_ONE_LEVEL"] = "1"
    lengths = [0, 1, 63, 64, 65, 200, 0, 700, 129]
    cu = W.cu_from_lengths(lengths)
    T = int(cu[-1])
    say("chunk_fwd varlen", dtype, lengths)
    inp = W.make_prefill(1, T, 4, 128, 128, dtype, "lightning", seed=3, device="cuda",
                         cu_seqlens=cu, init="normal")
    set_segments(128)
    o, S = run_gpu(inp)
    compare(inp, o, S, dtype, "varlen", starts=[int(c) for c in cu[:-1]])
    # Packed equals separate runs, bit for bit (same segment length).
    for n, L in enumerate(lengths):
        a, b = int(cu[n]), int(cu[n + 1])
        one = dict(inp)
        one["q"], one["k"], one["v"], one["g"] = (inp[x][:, a:b].contiguous()
                                                  for x in ("q", "k", "v", "g"))
        one["initial_state"] = inp["initial_state"][n:n + 1].contiguous()
        one["cu_seqlens"] = None
        on, Sn = run_gpu(one)
        assert torch.equal(on, o[:, a:b]), n
        assert torch.equal(Sn[0], S[n]), n
        if L == 0:
            assert torch.equal(S[n], inp["initial_state"][n]), n


def test_no_final_state_and_in_place_state():
    say("chunk_fwd final_state None / in place")
    set_segments(128)
    inp = W.make_prefill(2, 700, 2, 64, 64, "bf16", "lightning", seed=9, device="cuda",
                         init="normal")
    o1, S1 = run_gpu(inp)
    o2, none = sgla.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["initial_state"],
                              output_final_state=False)
    assert none is None
    assert torch.equal(o1, o2)
    st = inp["initial_state"].clone()
    o3, S3 = sgla.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], st, final_state=st)
    torch.cuda.synchronize()
    assert S3.data_ptr() == st.data_ptr()
    assert torch.equal(o3, o1) and torch.equal(S3, S1)


def test_zero_tokens_copies_state():
    say("chunk_fwd T=0")
    S0 = torch.randn(3, 2, 64, 128, device="cuda")
    z = torch.empty(3, 0, 2, 64, device="cuda", dtype=torch.bfloat16)
    zv = torch.empty(3, 0, 2, 128, device="cuda", dtype=torch.bfloat16)
    g = torch.empty(3, 0, 2, device="cuda")
    o, S = sgla.chunk_fwd(z, z, zv, g, initial_state=S0)
    torch.cuda.synchronize()
    assert o.shape == (3, 0, 2, 128)
    assert torch.equal(S, S0)


def test_split_and_chain():
    say("chunk_fwd split/chain T=1500 at 640 and 1000")
    inp = W.make_prefill(1, 1500, 2, 128, 128, "bf16", "lightning", seed=4, device="cuda",
                         init="normal")
    o, S = run_gpu(inp)
    ro, rS = oracle_prefill(inp)
    for t in (640, 1000):
        a = dict(inp)
        b = dict(inp)
        for x in ("q", "k", "v", "g"):
            a[x] = inp[x][:, :t].contiguous()
            b[x] = inp[x][:, t:].contiguous()
        oa, Sa = run_gpu(a)
        b["initial_state"] = Sa
        ob, Sb = run_gpu(b)
        oc = torch.cat([oa, ob], dim=1)
        check(host(oc), ro, "bf16", "split %d o" % t)
        check(host(Sb), rS, "bf16", "split %d state" % t, bf16_out=False)
        check_windows(host(oc)[0], ro[0], [t], "bf16", "split %d" % t)


def test_deterministic():
    say("chunk_fwd determinism")
    inp = W.make_prefill(1, 2000, 4, 128, 128, "bf16", "lightning", seed=11, device="cuda",
                         init="normal")
    o1, S1 = run_gpu(inp)
    o2, S2 = run_gpu(inp)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def _sample_heads(H, n, seed):
    rng = np.random.default_rng(seed)
    return sorted(rng.choice(H, size=n, replace=False).tolist())


def test_workload_prefill_8k():
    say("chunk_fwd workload prefill bf16 H=32 T=8192 D=128 seed=2 (every head)")
    inp = W.make_workload("prefill_bf16_h32_t8192_d128", seed=2, device="cuda")
    o, S = run_gpu(inp)
    compare(inp, o, S, "bf16", "prefill 8k")


def test_workload_prefill_64k_continuation_and_split():
    say("chunk_fwd workload prefill bf16 H=32 T=65536 D=128 S0 seed=3 (every head)")
    inp = W.make_workload("prefill_bf16_h32_t65536_d128_cont", seed=3, device="cuda")
    o, S = run_gpu(inp)
    heads = list(range(32))
    ro, rS = compare(inp, o, S, "bf16", "prefill 64k", heads=heads, starts=[0])
    t = 32768
    a = dict(inp)
    b = dict(inp)
    for x in ("q", "k", "v", "g"):
        a[x] = inp[x][:, :t].contiguous()
        b[x] = inp[x][:, t:].contiguous()
    oa, Sa = run_gpu(a)
    b["initial_state"] = Sa
    ob, Sb = run_gpu(b)
    oc = host(torch.cat([oa, ob], dim=1)[:, :, heads])
    check(oc, ro, "bf16", "64k split o")
    check(host(Sb[:, heads]), rS, "bf16", "64k split state", bf16_out=False)
    check_windows(oc[0], ro[0], [t], "bf16", "64k split")


@pytest.mark.parametrize("path", ["one_level", "halves"])
def test_workload_varlen_512k(path):
    if path == "halves":
        os.environ["SGLA_VALUE_HALVES"] = "1"
    say("chunk_fwd workload varlen bf16 8 seqs 524288 tokens H=32 D=128 seed=5 (4 heads)", path)
    inp = W.make_workload("varlen_bf16_h32_d128_8seq_512k", seed=5, device="cuda")
    o, S = run_gpu(inp)
    heads = _sample_heads(32, 4, 5)
    cu = inp["cu_seqlens"].cpu().numpy()
    compare(inp, o, S, "bf16", "varlen 512k", heads=heads,
            starts=[int(c) for c in cu[:-1]])


@pytest.mark.parametrize("seg_len", [None, 64])
def test_most_heads_ragged_chunk(seg_len):
    """H = 65536, the most heads a call takes, and T = 70 (a full chunk and a
    ragged one of 6 tokens). The row stride is H * 256 bytes, so the chunk
    kernels' per-chunk byte ranges and row offsets are at their largest (about
    2^30). With 64-token segments the segment-state and scan kernels run too."""
    if seg_len:
        set_segments(seg_len)
    say("chunk_fwd bf16 B=1 T=70 H=65536 D=128 seed=77 seg_len", seg_len, "(4 sampled heads)")
    inp = W.make_prefill(1, 70, 65536, 128, 128, "bf16", "lightning", seed=77, device="cuda",
                         init="normal")
    o, S = run_gpu(inp)
    compare(inp, o, S, "bf16", "H=65536 T=70", heads=[0, 1, 40961, 65535])
    del inp, o, S
    torch.cuda.empty_cache()


@pytest.mark.parametrize("T", [65, 700])
def test_vector_alu_path_for_bf16_128(T):
    """bf16 with 128-wide heads normally runs on the matrix cores; the vector
    ALU kernels stay correct for it too (they serve every other shape)."""
    say("chunk_fwd forced VALU bf16 T=%d" % T)
    os.environ["SGLA_FORCE_VALU"] = "1"
    try:
        inp = W.make_prefill(1, T, 3, 128, 128, "bf16", "lightning", seed=T, device="cuda",
                             init="normal")
        o, S = run_gpu(inp)
    finally:
        os.environ.pop("SGLA_FORCE_VALU", None)
    compare(inp, o, S, "bf16", "forced VALU T=%d" % T)


@pytest.mark.parametrize("dtype,dk,varlen", [("bf16", 128, False), ("bf16", 128, True),
                                              ("f32", 64, False), ("f32", 64, True)])
def test_without_workspace_one_segment_per_sequence(dtype, dk, varlen):
    """sgla_chunk_fwd (no workspace): every sequence is one segment, packed
    sequences read straight from cu_seqlens; same results as the oracle."""
    say("chunk_fwd without workspace", dtype, dk, "varlen" if varlen else "B=2")
    if varlen:
        lengths = [0, 70, 1, 300, 64]
        cu = W.cu_from_lengths(lengths)
        inp = W.make_prefill(1, int(cu[-1]), 3, dk, dk, dtype, "lightning", seed=21,
                             device="cuda", cu_seqlens=cu, init="normal")
        starts = [int(c) for c in cu[:-1]]
    else:
        inp = W.make_prefill(2, 700, 3, dk, dk, dtype, "lightning", seed=22, device="cuda",
                             init="normal")
        starts = [0]
    o, S = sgla.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["initial_state"],
                          inp["cu_seqlens"], inp["scale"], workspace=None)
    torch.cuda.synchronize()
    compare(inp, o, S, dtype, "no workspace", starts=starts)


def test_explicit_workspace_tensor_and_reuse():
    say("chunk_fwd explicit workspace B=1 T=3000 H=4")
    inp = W.make_prefill(1, 3000, 4, 128, 128, "bf16", "lightning", seed=23, device="cuda",
                         init="normal")
    set_segments(1024, 2)
    n = sgla.chunk_workspace_size(1, 3000, 4, 128, 128, torch.bfloat16)
    assert n > 0
    ws = torch.full((n,), 0xAB, dtype=torch.uint8, device="cuda")
    o1, S1 = sgla.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["initial_state"],
                            scale=inp["scale"], workspace=ws)
    o2, S2 = sgla.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["initial_state"],
                            scale=inp["scale"], workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    compare(inp, o1, S1, "bf16", "explicit workspace", starts=[0, 1024, 2048])
    with pytest.raises(sgla.SglaError):
        sgla.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], workspace=ws[: n - 256])


def test_validate_cu_seqlens():
    say("validate_cu_seqlens")
    good = torch.tensor([0, 3, 3, 10], dtype=torch.int64, device="cuda")
    assert sgla.validate_cu_seqlens(good, 10) == 0
    assert sgla.validate_cu_seqlens(good, 11) == 4
    assert sgla.validate_cu_seqlens(torch.tensor([1, 3, 2, 10], dtype=torch.int64,
                                                 device="cuda"), 10) == 3
    big = torch.arange(0, 5001, dtype=torch.int64, device="cuda")
    big[2500] = 9999
    assert sgla.validate_cu_seqlens(big, 5000) == 2
    # The check lands in word 0 of the workspace when SGLA_VALIDATE is set.
    inp = W.make_prefill(1, 300, 2, 128, 128, "bf16", "lightning", seed=24, device="cuda",
                         cu_seqlens=W.cu_from_lengths([100, 200]), init="normal")
    os.environ["SGLA_VALIDATE"] = "1"
    try:
        n = sgla.chunk_workspace_size(2, 300, 2, 128, 128, torch.bfloat16, varlen=True)
        ws = torch.full((n,), 0xFF, dtype=torch.uint8, device="cuda")
        sgla.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], cu_seqlens=inp["cu_seqlens"],
                       workspace=ws)
        torch.cuda.synchronize()
        assert int(ws[:4].view(torch.int32).item()) == 0
    finally:
        os.environ.pop("SGLA_VALIDATE", None)



# Per-head constant log-decays spread like the lightning layer's fixed ones
# (page "MiniCPM-SALA - Complete Blueprint", section "B2 lightning-attn
# (Simple GLA)": from -0.917, alpha about 0.40, the fastest forgetting, to
# -0.0001, the slowest): geometric between the two ends. One 64-token chunk of
# the fastest head sums to about -58.7.
def g_gamma(H):
    return -0.917 * (0.0001 / 0.917) ** (np.arange(H) / max(H - 1, 1))


def constant_decay_inputs(B, T, H, D, dtype, seed, cu=None):
    inp = W.make_prefill(B, T, H, D, D, dtype, "lightning", seed=seed, device="cuda",
                         init="normal", cu_seqlens=cu)
    gg = torch.tensor(g_gamma(H), dtype=torch.float32, device="cuda")
    inp["g"] = gg.view(1, 1, H).expand_as(inp["g"]).contiguous()
    return inp


@pytest.mark.parametrize("path", ["halves", "one_level", "valu_bf16", "valu_f32_d64"])
def test_per_head_constant_decay_from_0p40_to_0p9999(path):
    """Strong and weak constant decays side by side, over several segments and
    sub-segments, on each prefill path."""
    dtype, D = ("f32", 64) if path == "valu_f32_d64" else ("bf16", 128)
    if path == "one_level":
        os.environ["SGLA_ONE_LEVEL"] = "1"
    if path == "valu_bf16":
        os.environ["SGLA_FORCE_VALU"] = "1"
    set_segments(256, 2)
    say("chunk_fwd constant per-head decay", path, "B=2 T=1100 H=8")
    try:
        inp = constant_decay_inputs(2, 1100, 8, D, dtype, seed=51)
        o, S = run_gpu(inp)
    finally:
        os.environ.pop("SGLA_FORCE_VALU", None)
    compare(inp, o, S, dtype, "constant decay " + path, starts=[0, 256, 512, 768, 1024])


def test_per_head_constant_decay_varlen_without_workspace():
    say("chunk_fwd constant per-head decay, packed, no workspace")
    cu = W.cu_from_lengths([700, 0, 65, 300])
    inp = constant_decay_inputs(1, int(cu[-1]), 8, 128, "bf16", seed=52, cu=cu)
    o, S = sgla.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["initial_state"],
                          inp["cu_seqlens"], inp["scale"], workspace=None)
    torch.cuda.synchronize()
    compare(inp, o, S, "bf16", "constant decay packed", starts=[int(c) for c in cu[:-1]])


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64)])
def test_decay_table_of_the_blueprint_through_the_gpu(dtype, D):
    """The page's "Concrete decay over distance" table (blueprint page,
    section "Why Linear Attention Loses Information", Problem 1; fixture
    tests/golden/decay_table.json): a one-hot outer product written at the
    first token, zero keys after it, constant decay per head; after n more
    tokens the written entry of the final state must print as the page's
    value."""
    import json
    fx = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "decay_table.json")))
    heads = fx["heads"]
    H = len(heads)
    for n_str in ("1", "10", "100", "1000", "10000", "100000"):
        n = int(n_str)
        T = n + 1
        say("chunk_fwd decay table", dtype, "n =", n)
        tdt = DT[dtype]
        q = torch.zeros((1, T, H, D), dtype=tdt, device="cuda")
        k = torch.zeros_like(q)
        v = torch.zeros((1, T, H, D), dtype=tdt, device="cuda")
        i, j = 3, 5
        k[0, 0, :, i] = 1.0
        v[0, 0, :, j] = 1.0
        g = torch.tensor([h["g"] for h in heads], dtype=torch.float32,
                         device="cuda").view(1, 1, H).expand(1, T, H).contiguous()
        _, S = sgla.chunk_fwd(q, k, v, g, scale=1.0)
        torch.cuda.synchronize()
        got = S[0, :, i, j].double().cpu().numpy()
        others = S[0].clone()
        others[:, i, j] = 0
        assert float(others.abs().max()) == 0.0, n
        for hh, val in zip(heads, got):
            printed = hh["values"][n_str]
            if float(printed) == 0.0:
                assert abs(val) < fx["zero_bound"], (hh["label"], n, val)
            elif dtype == "f32":
                # The printed value carries its digits: the GPU result must
                # round to it at that precision.
                digits = len(printed.split("e")[0].replace(".", "").lstrip("0"))
                assert float("%.*g" % (digits, val)) == float(printed), (hh["label"], n, val)
            else:
                # bf16 inputs: the update's decayed values exp(G_last - G) v
                # are bf16 MFMA operands, one rounding of at most 2^-9 of the
                # entry; the state and its decay between chunks stay fp32.
                # So the entry lies within 2^-8 of the printed value plus half
                # a unit of the printed value's last digit.
                p = float(printed)
                digits = len(printed.split("e")[0].replace(".", "").lstrip("0"))
                last_unit = 10.0 ** (np.floor(np.log10(abs(p))) - digits + 1)
                assert abs(val - p) <= 2.0 ** -8 * abs(p) + 0.5 * last_unit, (hh["label"], n, val)


@pytest.mark.parametrize("path", ["halves", "one_level", "valu_f32_d64"])
def test_growing_and_shrinking_gates(path):
    """g of either sign (the interface takes any real g): per token g ~
    U(-0.05, 0.05), so the state both decays and grows."""
    dtype, D = ("f32", 64) if path == "valu_f32_d64" else ("bf16", 128)
    if path == "one_level":
        os.environ["SGLA_ONE_LEVEL"] = "1"
    set_segments(256, 2)
    say("chunk_fwd mixed-sign g", path)
    inp = W.make_prefill(2, 900, 4, D, D, dtype, "lightning", seed=53, device="cuda",
                         init="normal")
    gen = torch.Generator(device="cuda").manual_seed(53)
    inp["g"] = (torch.rand(inp["g"].shape, generator=gen, device="cuda") - 0.5) * 0.1
    o, S = run_gpu(inp)
    compare(inp, o, S, dtype, "mixed-sign g " + path, starts=[0, 256, 512, 768])


@pytest.mark.parametrize("scale", [-0.3, 0.0, 2.0])
@pytest.mark.parametrize("path", ["halves", "one_level", "valu_f32_d64"])
def test_output_scale_of_either_sign(path, scale):
    """The output scale is any real number: negative, zero and above one."""
    dtype, D = ("f32", 64) if path == "valu_f32_d64" else ("bf16", 128)
    if path == "one_level":
        os.environ["SGLA_ONE_LEVEL"] = "1"
    set_segments(256, 2)
    say("chunk_fwd scale", scale, path)
    inp = W.make_prefill(2, 600, 3, D, D, dtype, "lightning", seed=57, device="cuda",
                         init="normal")
    inp["scale"] = scale
    o, S = run_gpu(inp)
    if scale == 0.0:
        assert float(o.float().abs().max()) == 0.0
        ro, rS = oracle_prefill(inp)
        check(host(S), rS, dtype, "scale 0 final state", bf16_out=False)
        return
    compare(inp, o, S, dtype, "scale %g %s" % (scale, path), starts=[0, 256, 512])


@pytest.mark.parametrize("path", ["halves", "valu_f32_d64"])
@pytest.mark.parametrize("kind", ["strong_decay", "alternating"])
def test_strong_and_alternating_gates(kind, path):
    """Gates far from the workloads': strong decays (g in [-2, -1], chunk
    sums near -96, where exp(G) alone underflows within a chunk), and gates
    alternating +-1.5 (G bounded, every score's decay swinging by e^1.5), with
    ordinary chunks mixed in.

    Under strong decay each output is a sum of a few intra-chunk terms
    A_ij v_j, each score A_ij a bf16 operand with one rounding (2^-9 of it);
    the outputs reach about 15x their RMS and may cancel, so that rounding
    alone can exceed the max-abs bar. For the bf16 matrix-core path that case
    therefore gets a per-element allowance of 2^-8 sum_j |A_ij| |v_j| (the
    rounding bound with a factor 2 to spare; A over the 64-token chunks the
    kernel forms), its median capped at a tenth of the bar so the bar stays
    live; rel-L2 is not relaxed. The fp32 vector path meets the fp32 bar on
    the same gates."""
    dtype, D = ("f32", 64) if path == "valu_f32_d64" else ("bf16", 128)
    set_segments(256, 2)
    say("chunk_fwd strong gates", kind, path)
    B, T, H = 2, 700, 4
    inp = W.make_prefill(B, T, H, D, D, dtype, "lightning", seed=59, device="cuda",
                         init="normal")
    gen = torch.Generator(device="cuda").manual_seed(59)
    if kind == "strong_decay":
        g = -(1.0 + torch.rand((B, T, H), generator=gen, device="cuda"))
    else:
        sign = torch.where(torch.arange(T, device="cuda") % 2 == 0, 1.0, -1.0)
        g = 1.5 * sign.view(1, T, 1).expand(B, T, H).clone()
    # the first and third 64-token chunks keep ordinary gates
    g[:, :64] = inp["g"][:, :64]
    g[:, 128:192] = inp["g"][:, 128:192]
    inp["g"] = g.contiguous()
    o, S = run_gpu(inp)
    what = "strong gates %s %s" % (kind, path)
    if kind == "strong_decay" and dtype == "bf16":
        ro, rS = oracle_prefill(inp)
        q, k, v, gg = (host(inp[x]).astype(np.float64) for x in ("q", "k", "v", "g"))
        bound = np.zeros_like(ro)
        for b in range(B):
            for h in range(H):
                for c0 in range(0, T, 64):
                    sl = slice(c0, min(T, c0 + 64))
                    G = np.cumsum(gg[b, sl, h])
                    A = np.tril(np.abs(q[b, sl, h] @ k[b, sl, h].T) * np.exp(G[:, None] - G[None, :]))
                    bound[b, sl, h] = inp["scale"] * A @ np.abs(v[b, sl, h])
        m = check(host(o), ro, dtype, what + " o", allowance=2.0 ** -8 * bound,
                  max_allowance_median=0.1)
        say("  allowance over the bar on %.2e of the elements" % m["allowance_frac_over_bar"])
        check(host(S), rS, dtype, what + " final state", bf16_out=False)
        return
    compare(inp, o, S, dtype, what, starts=[0, 256, 512])

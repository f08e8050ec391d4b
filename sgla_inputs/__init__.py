"""Seeded synthetic inputs for the Simple GLA workloads.

This module is shared by the oracle side (tests, CPU baseline) and the GPU side
(tests, bench): it only draws random numbers and shapes them into the input
distributions below. It contains none of the gated-linear-attention arithmetic
and imports neither the oracle nor the GPU library.

Input recipes (the lightning-layer inputs described on the page "MiniCPM-SALA —
Complete Blueprint", section "B2 lightning-attn (Simple GLA)": q and k after
the per-head RMSNorm and RoPE, cast to bf16):

* ``"gaussian"``  : q, k, v ~ N(0, 1) per element; gate input x ~ N(3, 1).
* ``"lightning"`` : q, k rows ~ N(0, 1) scaled to unit RMS (eps 1e-6, weight
  1); v ~ N(0, 1); gate input x ~ N(4, 1). RoPE would turn each row by a fixed
  rotation; a row whose direction is uniformly random (an isotropic Gaussian
  row, scaled by a function of its length) has the same distribution after
  any rotation, so the rows are not rotated here.
* ``"raw"``       : q, k as they arrive before the RMSNorm and RoPE (for the
  entry points that apply both): rows ~ N(0, 1) times a per-row factor
  exp(N(0, 0.5^2)); v and the gates as in ``"lightning"``. ``norm_weights``
  draws the two RMSNorm weight vectors, 1 + N(0, 0.1^2) per element.

* ``"gdn"``       : inputs of the gated delta rule (page "Formulas and code
  for adapting inference to GDN/KDA linear modules", section 1.1: q and k
  are L2-normalised per head with eps 1e-6 inside the square root, beta is a
  sigmoid): q, k rows ~ N(0, 1) scaled to unit L2 norm; v ~ N(0, 1); gate
  input x ~ N(4, 1); with ``with_beta`` a write strength beta = sigmoid(b),
  b ~ N(0, 1), per token and head (fp32), drawn after everything else.
* ``"kda"``       : as ``"gdn"``, but the gate input x, and so g, has one value
  per key dim (the page's section 2.1: the KDA branch loads a gate vector over
  the key dims): x ~ N(4, 1) per (token, head, dim), g [.., H, Dk].

In all of them, the per-token per-head log-decay is g = log(sigmoid(x)) in fp32, so
every decay factor exp(g) lies in (0, 1). Initial states, when present, are
fp32 ~ N(0, 0.02^2). bf16 tensors come from a round-to-nearest-even cast of the
fp32 draws. Draw order from one ``torch.Generator`` seeded with ``seed``: q, k,
v, x, then the initial state. Draws happen in token blocks so that temporaries
stay bounded; the block size does not change the values.
"""
from __future__ import annotations

import math

import numpy as np
import torch
import torch.nn.functional as F

RMS_EPS = 1e-6
_BLOCK_TOKENS = 32768

# Named workloads, by what they are and their sizes.
WORKLOADS = {
    # fp32 correctness case: B=1, H=4, T=256, Dk=Dv=64, zero initial state.
    "tiny_fp32_h4_t256_d64": dict(kind="prefill", B=1, T=256, H=4, D=64, dtype="f32",
                                  preset="gaussian", init=None),
    # One lightning layer's prefill: B=1, H=32, T=8192, Dk=Dv=128, bf16 in, fp32 state out.
    "prefill_bf16_h32_t8192_d128": dict(kind="prefill", B=1, T=8192, H=32, D=128,
                                        dtype="bf16", preset="lightning", init=None),
    # Long continuation: T=65536 from a nonzero fp32 initial state; also split at 32768.
    "prefill_bf16_h32_t65536_d128_cont": dict(kind="prefill", B=1, T=65536, H=32, D=128,
                                              dtype="bf16", preset="lightning",
                                              init="normal", split=32768),
    # Batched decode: 256 sequences x 32 heads, 64 successive single-token steps.
    "decode_bf16_n256_h32_d128_x64": dict(kind="decode", N=256, H=32, D=128, steps=64,
                                          dtype="bf16", preset="lightning", pos0=100000),
    # Varlen: 8 sequences packed to 524288 tokens, log-uniform lengths in [4096, 262144].
    "varlen_bf16_h32_d128_8seq_512k": dict(kind="prefill", nseq=8, total=524288,
                                           lmin=4096, lmax=262144, H=32, D=128,
                                           dtype="bf16", preset="lightning", init=None),
}

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def generator(seed: int, device="cpu") -> torch.Generator:
    gen = torch.Generator(device=torch.device(device))
    gen.manual_seed(int(seed))
    return gen


def varlen_lengths(nseq: int, total: int, lmin: int, lmax: int, seed: int) -> np.ndarray:
    """Sequence lengths drawn log-uniform in [lmin, lmax], then rescaled so they
    sum to ``total`` (floor, then largest remainders get +1). The bounds apply
    before the rescale."""
    rng = np.random.default_rng(np.random.SeedSequence(int(seed)).spawn(1)[0])
    raw = np.exp(rng.uniform(math.log(lmin), math.log(lmax), size=nseq))
    ideal = raw * (total / raw.sum())
    base = np.floor(ideal).astype(np.int64)
    short = int(total - base.sum())
    order = np.argsort(-(ideal - base), kind="stable")
    base[order[:short]] += 1
    assert int(base.sum()) == total
    return base


def cu_from_lengths(lengths) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, dtype=np.int64))]).astype(np.int64)


def positions_for(T: int, cu_seqlens=None, start: int = 0) -> np.ndarray:
    """Position of each packed token inside its own sequence (plus ``start``)."""
    if cu_seqlens is None:
        return np.arange(T, dtype=np.int64) + start
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    pos = np.arange(T, dtype=np.int64)
    seq = np.searchsorted(cu, pos, side="right") - 1
    return pos - cu[seq] + start


def _unit_rms(x: torch.Tensor) -> torch.Tensor:
    return x * torch.rsqrt(x.pow(2).mean(dim=-1, keepdim=True) + RMS_EPS)


def _draw_qk(shape_tokens, H, D, preset, gen, device, out_dtype):
    out = torch.empty((shape_tokens, H, D), dtype=out_dtype, device=device)
    for s in range(0, shape_tokens, _BLOCK_TOKENS):
        e = min(shape_tokens, s + _BLOCK_TOKENS)
        x = torch.randn((e - s, H, D), generator=gen, device=device, dtype=torch.float32)
        if preset == "lightning":
            x = _unit_rms(x)
        elif preset in ("gdn", "kda"):
            x = x * torch.rsqrt(x.pow(2).sum(dim=-1, keepdim=True) + RMS_EPS)
        elif preset == "raw":
            f = torch.randn((e - s, H, 1), generator=gen, device=device, dtype=torch.float32)
            x = x * torch.exp(0.5 * f)
        out[s:e] = x.to(out_dtype)
    return out


def norm_weights(D: int, seed: int, device="cpu"):
    """The q and k RMSNorm weights for the ``"raw"`` preset: fp32 [D] each,
    1 + N(0, 0.1^2) per element."""
    gen = generator(seed, device)
    w = 1.0 + 0.1 * torch.randn((2, D), generator=gen, device=torch.device(device),
                                dtype=torch.float32)
    return w[0].contiguous(), w[1].contiguous()


def _draw_plain(shape_tokens, inner, gen, device, out_dtype, mean=0.0, std=1.0):
    out = torch.empty((shape_tokens,) + tuple(inner), dtype=out_dtype, device=device)
    for s in range(0, shape_tokens, _BLOCK_TOKENS):
        e = min(shape_tokens, s + _BLOCK_TOKENS)
        x = torch.randn((e - s,) + tuple(inner), generator=gen, device=device, dtype=torch.float32)
        if std != 1.0 or mean != 0.0:
            x = x * std + mean
        out[s:e] = x.to(out_dtype)
    return out


def gate_mean(preset: str) -> float:
    return {"gaussian": 3.0, "lightning": 4.0, "raw": 4.0, "gdn": 4.0, "kda": 4.0}[preset]


def make_prefill(B, T, H, Dk, Dv, dtype="bf16", preset="lightning", seed=0, device="cpu",
                 cu_seqlens=None, init=None, with_beta=False):
    """Inputs for one chunked-forward call.

    Returns a dict with q, k [B, T, H, Dk]; v [B, T, H, Dv] (dtype); g [B, T, H]
    fp32 ([B, T, H, Dk] for the ``"kda"`` preset); initial_state [N, H, Dk, Dv] fp32 or None; cu_seqlens int64 tensor or
    None; scale = 1/sqrt(Dk). With ``cu_seqlens`` B must be 1 and T the total.
    ``init`` is None (zero state) or "normal" (N(0, 0.02^2)). With
    ``with_beta`` also beta [B, T, H] fp32 in (0, 1).
    """
    device = torch.device(device)
    tdt = TORCH_DTYPE[dtype]
    gen = generator(seed, device)
    if cu_seqlens is not None:
        assert B == 1
        cu_np = np.asarray(cu_seqlens, dtype=np.int64)
        assert cu_np[0] == 0 and cu_np[-1] == T
        N = len(cu_np) - 1
    else:
        cu_np = None
        N = B
    BT = B * T
    q = _draw_qk(BT, H, Dk, preset, gen, device, tdt)
    k = _draw_qk(BT, H, Dk, preset, gen, device, tdt)
    v = _draw_plain(BT, (H, Dv), gen, device, tdt)
    gshape = (H, Dk) if preset == "kda" else (H,)
    x = _draw_plain(BT, gshape, gen, device, torch.float32, mean=gate_mean(preset))
    g = F.logsigmoid(x)
    S0 = None
    if init == "normal":
        S0 = (torch.randn((N, H, Dk, Dv), generator=gen, device=device, dtype=torch.float32)
              * 0.02)
    elif init is not None:
        raise ValueError(init)
    beta = None
    if with_beta:
        beta = torch.sigmoid(_draw_plain(BT, (H,), gen, device, torch.float32)).view(B, T, H)
    return dict(
        q=q.view(B, T, H, Dk), k=k.view(B, T, H, Dk), v=v.view(B, T, H, Dv),
        g=g.view((B, T) + gshape),
        initial_state=S0, beta=beta,
        cu_seqlens=None if cu_np is None else torch.from_numpy(cu_np).to(device),
        scale=1.0 / math.sqrt(Dk), dtype=dtype, preset=preset, seed=seed,
    )


def make_decode(N, H, Dk, Dv, steps, dtype="bf16", preset="lightning", seed=0, device="cpu",
                pos0=100000, slots=None, with_state=True, with_beta=False):
    """Inputs for ``steps`` successive decode steps of N sequences.

    Returns q, k [steps, N, H, Dk]; v [steps, N, H, Dv]; g [steps, N, H] fp32
    ([steps, N, H, Dk] for the ``"kda"`` preset);
    state [slots or N, H, Dk, Dv] fp32 ~ N(0, 0.02^2); scale; pos [steps, N]
    int32, step i of every sequence at position pos0 + i. With ``with_beta``
    also beta [steps, N, H] fp32 (drawn after each step's gate).
    """
    device = torch.device(device)
    tdt = TORCH_DTYPE[dtype]
    gen = generator(seed, device)
    nslots = N if slots is None else slots
    state = None
    if with_state:
        state = torch.randn((nslots, H, Dk, Dv), generator=gen, device=device,
                            dtype=torch.float32) * 0.02
    qs, ks, vs, gs, bs = [], [], [], [], []
    for i in range(steps):
        qs.append(_draw_qk(N, H, Dk, preset, gen, device, tdt))
        ks.append(_draw_qk(N, H, Dk, preset, gen, device, tdt))
        vs.append(_draw_plain(N, (H, Dv), gen, device, tdt))
        x = _draw_plain(N, (H, Dk) if preset == "kda" else (H,), gen, device, torch.float32,
                        mean=gate_mean(preset))
        gs.append(F.logsigmoid(x))
        if with_beta:
            bs.append(torch.sigmoid(_draw_plain(N, (H,), gen, device, torch.float32)))
    pos = (torch.arange(steps, dtype=torch.int32, device=device)[:, None] + pos0).expand(steps, N)
    return dict(q=torch.stack(qs), k=torch.stack(ks), v=torch.stack(vs), g=torch.stack(gs),
                beta=torch.stack(bs) if with_beta else None, state=state, scale=1.0 / math.sqrt(Dk), dtype=dtype, preset=preset, seed=seed,
                pos=pos.contiguous())


def make_workload(name: str, seed: int = 0, device="cpu", preset=None):
    """Inputs of a named workload (see WORKLOADS)."""
    w = dict(WORKLOADS[name])
    if preset is not None:
        w["preset"] = preset
    if w["kind"] == "decode":
        return make_decode(w["N"], w["H"], w["D"], w["D"], w["steps"], w["dtype"], w["preset"],
                           seed, device, pos0=w["pos0"])
    if "nseq" in w:
        lengths = varlen_lengths(w["nseq"], w["total"], w["lmin"], w["lmax"], seed)
        cu = cu_from_lengths(lengths)
        return make_prefill(1, w["total"], w["H"], w["D"], w["D"], w["dtype"], w["preset"], seed,
                            device, cu_seqlens=cu, init=w["init"])
    return make_prefill(w["B"], w["T"], w["H"], w["D"], w["D"], w["dtype"], w["preset"], seed,
                        device, init=w["init"])


def make_epilogue(rows: int, width: int, dtype="bf16", seed=0, device="cpu"):
    """Inputs of the output epilogue: o [rows, width] ~ N(0, 1) times a per-row
    factor exp(N(0, 0.5^2)) (attention outputs vary in size from token to
    token); gate logits z [rows, width] ~ N(0, 2^2), so the gate spans (0, 1);
    weight [width] fp32 = 1 + N(0, 0.1^2). Draw order: o, the row factors, z,
    weight."""
    device = torch.device(device)
    tdt = TORCH_DTYPE[dtype]
    gen = generator(seed, device)
    o = torch.randn((rows, width), generator=gen, device=device, dtype=torch.float32)
    f = torch.randn((rows, 1), generator=gen, device=device, dtype=torch.float32)
    o = (o * torch.exp(0.5 * f)).to(tdt)
    z = (2.0 * torch.randn((rows, width), generator=gen, device=device,
                           dtype=torch.float32)).to(tdt)
    w = 1.0 + 0.1 * torch.randn((width,), generator=gen, device=device, dtype=torch.float32)
    return dict(o=o, z=z, weight=w, dtype=dtype, seed=seed)


def to_numpy_f32(t):
    """Exact host copy in fp32 (bf16 -> fp32 is exact)."""
    if t is None:
        return None
    return t.detach().to("cpu").to(torch.float32).numpy()

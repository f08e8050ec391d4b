"""GPU parity of the decode step with a bf16 state pool (sgla_recurrent_step_ex).

* Against the fp32-pool kernel from the same starting values: every state
  element's update is the same fp32 arithmetic, so the stored bf16 state must
  be exactly the bf16 rounding of the fp32 one (with and without the q/k
  prologue); the outputs sum their rows in another order (8- instead of
  4-column groups per thread), so they agree to one bf16 spacing.
* Against ``oracle/bf16_state.py``: one step on every state element, and the
  batched-decode shape through 64 steps on sampled states. The kernel rounds
  fp32 values, the oracle fp64 ones; where a value lies within 2^-16 (of its
  terms' size) of a bf16 midpoint either rounding is correct, and the oracle's
  bound, carried by the decay from step to step, is added per element to the
  max-abs bar (rel-L2 unchanged).
"""
import numpy as np
import pytest
import torch

import linear_attention_hybrid_amd as sgla
import oracle.bf16_state as BS
import sgla_inputs as W
from tests.parity import check, host, nan_like, say

pytestmark = pytest.mark.gpu

TIE_ETA = 2.0 ** -16


def bf16_round_tensor(x):
    return x.to(torch.bfloat16)


@pytest.mark.parametrize("prologue", [False, True])
@pytest.mark.parametrize("dk,dv", [(128, 128), (128, 64), (64, 128), (64, 64)])
def test_bf16_pool_equals_fp32_pool_rounded(dk, dv, prologue):
    if prologue and dk != 128:
        pytest.skip("the prologue is built for 128-dim heads")
    say("recurrent_step_ex bf16 pool vs fp32 pool", dk, dv, "prologue", prologue)
    N, H, slots = 6, 3, 10
    d = W.make_decode(N, H, dk, dv, 3, "bf16", "raw" if prologue else "lightning",
                      seed=dk + dv + prologue, device="cuda", slots=slots)
    idx = torch.tensor([9, 0, 4, 7, 2, 5], dtype=torch.int32, device="cuda")
    s16 = (d["state"] * 25).to(torch.bfloat16)          # unit-size bf16 states
    s32 = s16.float()
    kw = {}
    if prologue:
        qw, kwt = W.norm_weights(128, seed=5, device="cuda")
        kw = dict(q_weight=qw, k_weight=kwt, positions=torch.tensor([0, 7, 99, 1 << 20, 3, 65536],
                                                                     dtype=torch.int32,
                                                                     device="cuda"))
    for i in range(3):
        o16 = sgla.recurrent_step_ex(d["q"][i], d["k"][i], d["v"][i], d["g"][i], s16,
                                     state_indices=idx, **kw)
        o32 = sgla.recurrent_step_ex(d["q"][i], d["k"][i], d["v"][i], d["g"][i], s32,
                                     state_indices=idx, **kw)
        torch.cuda.synchronize()
        a, b = host(o16).astype(np.float64), host(o32).astype(np.float64)
        spacing = np.ldexp(1.0, np.floor(np.log2(np.maximum(np.abs(b), 1e-30))).astype(int) - 7)
        assert np.all(np.abs(a - b) <= spacing), i
        assert torch.equal(s16, bf16_round_tensor(s32)), i
        s32 = s16.float()        # continue both from the stored bf16 state


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_one_step_every_element(dtype):
    say("recurrent_step_ex bf16 pool one step vs oracle", dtype)
    N, H, D, slots = 16, 4, 128, 20
    d = W.make_decode(N, H, D, D, 1, dtype, "lightning", seed=51, device="cuda", slots=slots)
    idx = torch.randperm(slots, generator=torch.Generator().manual_seed(51))[:N].to(torch.int32).cuda()
    s16 = (d["state"] * 25).to(torch.bfloat16)
    ref_state = host(s16).astype(np.float64)
    sel = ref_state[idx.cpu().numpy()].reshape(N * H, D, D)
    o = sgla.recurrent_step_ex(d["q"][0], d["k"][0], d["v"][0], d["g"][0], s16,
                               state_indices=idx, out=nan_like((N, H, D), d["v"].dtype))
    torch.cuda.synchronize()
    flat = lambda t: host(t).reshape(1, N * H, -1)
    ro, oa, A = BS.steps(flat(d["q"][0]), flat(d["k"][0]), flat(d["v"][0]),
                         host(d["g"][0]).reshape(1, N * H), sel, d["scale"], tie_eta=TIE_ETA)
    check(host(o).reshape(N * H, D), ro[0], dtype, "one step o", allowance=oa[0])
    got = host(s16[idx.long()]).reshape(N * H, D, D)
    check(got, sel, "bf16", "one step state", bf16_out=False, allowance=A)


def test_workload_64_steps_sampled():
    """The batched-decode shape (256 x 32 heads, D=128) with a bf16 pool
    through 64 steps; the oracle follows 24 sampled (row, head) states."""
    say("recurrent_step_ex bf16 pool N=256 H=32 D=128 64 steps seed=4 (24 sampled states)")
    d = W.make_decode(256, 32, 128, 128, 64, "bf16", "lightning", seed=4, device="cuda")
    state = (d["state"] * 25).to(torch.bfloat16)
    rng = np.random.default_rng(4)
    rows = rng.choice(256, 24, replace=False)
    heads = rng.integers(0, 32, 24)
    S = host(state)[rows, heads].astype(np.float64)
    outs = []
    for i in range(64):
        o = sgla.recurrent_step_ex(d["q"][i], d["k"][i], d["v"][i], d["g"][i], state)
        outs.append(host(o)[rows, heads])
    torch.cuda.synchronize()
    pick = lambda t: host(t)[:, rows, heads]
    ro, oa, A = BS.steps(pick(d["q"]), pick(d["k"]), pick(d["v"]), pick(d["g"]), S, d["scale"],
                         tie_eta=TIE_ETA)
    check(np.stack(outs), ro, "bf16", "64 steps o", allowance=oa)
    check(host(state)[rows, heads], S, "bf16", "64 steps state", bf16_out=False, allowance=A)

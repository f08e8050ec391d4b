"""GPU parity of the decode step with a bf16 state pool (sgla_recurrent_step_ex).

* Against the fp32-pool kernel from the same starting values: every state
  element's update is the same fp32 arithmetic, so the stored bf16 state must
  be exactly the bf16 rounding of the fp32 one (with and without the q/k
  prologue); the outputs sum their rows in another order (8- instead of
  4-column groups per thread), so they agree to one bf16 spacing.
* Against ``oracle/bf16_state.py``: one step on every state element (small
  pool and the whole 256 x 32 pool), and the batched-decode shape through 64
  steps on sampled states. The kernel rounds fp32 values, the oracle fp64
  ones; where a value lies within 2^-16 (of its terms' size) of a bf16
  midpoint either rounding is correct, and one spacing there is added to the
  max-abs bar of that state element (rel-L2 unchanged). The 64 steps are
  checked step by step from the kernel's own stored states (tight bars), and
  as a whole against the oracle's own run with the plain bars.
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


@pytest.mark.parametrize("shape", ["16x4", "pool_256x32"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_one_step_every_element(dtype, shape):
    """One step checked on every output and state element, on a small pool
    and on the batched-decode shape (256 rows x 32 heads, D = 128, the whole
    pool of 256 slots in a shuffled order)."""
    N, H, slots = (16, 4, 20) if shape == "16x4" else (256, 32, 256)
    D = 128
    say("recurrent_step_ex bf16 pool one step vs oracle", dtype, "N=%d H=%d slots=%d" % (N, H, slots))
    d = W.make_decode(N, H, D, D, 1, dtype, "lightning", seed=51, device="cuda", slots=slots)
    idx = torch.randperm(slots, generator=torch.Generator().manual_seed(51))[:N].to(torch.int32).cuda()
    s16 = (d["state"] * 25).to(torch.bfloat16)
    ref_state = host(s16).astype(np.float64)
    sel = ref_state[idx.cpu().numpy()].reshape(N * H, D, D)
    del ref_state
    o = sgla.recurrent_step_ex(d["q"][0], d["k"][0], d["v"][0], d["g"][0], s16,
                               state_indices=idx, out=nan_like((N, H, D), d["v"].dtype))
    torch.cuda.synchronize()
    flat = lambda t: host(t).reshape(1, N * H, -1)
    ro, oa, A = BS.steps(flat(d["q"][0]), flat(d["k"][0]), flat(d["v"][0]),
                         host(d["g"][0]).reshape(1, N * H), sel, d["scale"], tie_eta=TIE_ETA)
    mo = check(host(o).reshape(N * H, D), ro[0], dtype, "one step o", allowance=oa[0],
               max_allowance_median=0.1)
    got = host(s16[idx.long()]).reshape(N * H, D, D)
    ms = check(got, sel, "bf16", "one step state", bf16_out=False, allowance=A,
               max_allowance_median=0.1)
    for what, m in (("o", mo), ("state", ms)):
        say("  %s: allowance over the bar on %.2e of the elements (median %.2e, max %.2e of the bar)"
            % (what, m["allowance_frac_over_bar"], m["allowance_median_over_bar"],
               m["allowance_max_over_bar"]))


def test_workload_64_steps_sampled():
    """The batched-decode shape (256 x 32 heads, D=128) with a bf16 pool
    through 64 steps, on 256 sampled (row, head) states, two ways:

    * every step against the oracle's step from the state the kernel stored
      at the previous step: the output allowance is then zero (the query
      reads the state before it is rounded) and the state's is the one-step
      tie band, so both bars are tight on every element;
    * the whole run against the oracle's own 64-step run, with the plain bars
      and no allowance: a rounding that went the other way near a tie is one
      bf16 spacing of one element, shrunk by the decay, well inside them.
    """
    say("recurrent_step_ex bf16 pool N=256 H=32 D=128 64 steps seed=4 (256 sampled states)")
    d = W.make_decode(256, 32, 128, 128, 64, "bf16", "lightning", seed=4, device="cuda")
    state = (d["state"] * 25).to(torch.bfloat16)
    rng = np.random.default_rng(4)
    rows = rng.permutation(256)
    heads = rng.integers(0, 32, 256)
    S0 = host(state)[rows, heads].astype(np.float64)
    prev = S0.copy()
    pick1 = lambda t: host(t)[rows, heads][None]
    outs, worst = [], {"o": 0.0, "state": 0.0}
    for i in range(64):
        o = sgla.recurrent_step_ex(d["q"][i], d["k"][i], d["v"][i], d["g"][i], state)
        torch.cuda.synchronize()
        go = host(o)[rows, heads]
        gs = host(state)[rows, heads].astype(np.float64)
        outs.append(go)
        ref = prev.copy()
        ro, oa, A = BS.steps(pick1(d["q"][i]), pick1(d["k"][i]), pick1(d["v"][i]),
                             host(d["g"][i])[rows, heads][None], ref, d["scale"], tie_eta=TIE_ETA)
        assert float(np.max(oa)) == 0.0
        check(go, ro[0], "bf16", "step %d o from the stored state" % i)
        m = check(gs, ref, "bf16", "step %d state from the stored state" % i, bf16_out=False,
                  allowance=A, max_allowance_median=0.1)
        worst["state"] = max(worst["state"], m["allowance_frac_over_bar"])
        prev = gs
    say("  per step: the state's tie allowance exceeds the bar on at most %.2e of the elements"
        % worst["state"])
    pick = lambda t: host(t)[:, rows, heads]
    S = S0.copy()
    ro = BS.steps(pick(d["q"]), pick(d["k"]), pick(d["v"]), pick(d["g"]), S, d["scale"])
    mo = check(np.stack(outs), ro, "bf16", "64 steps o, independent run")
    ms = check(prev, S, "bf16", "64 steps state, independent run", bf16_out=False)
    say("  independent run: o max-abs %.3g (bar %.3g), state max-abs %.3g (bar %.3g)"
        % (mo["max_abs"], 2e-2 * mo["rms_ref"], ms["max_abs"], 2e-2 * ms["rms_ref"]))

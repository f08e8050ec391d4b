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

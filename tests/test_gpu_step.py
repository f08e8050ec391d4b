"""GPU parity of sgla_recurrent_step against the oracle's decode step."""
import numpy as np
import pytest
import torch

import linear_attention_hybrid_amd as sgla
import oracle
import sgla_inputs as W
from tests.parity import check, host, nan_like, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64), (128, 128)])
def test_step_with_slot_map(dtype, dk, dv):
    say("recurrent_step", dtype, dk, dv, "N=5 H=3 slots=9, 4 steps")
    N, H, slots, steps = 5, 3, 9, 4
    d = W.make_decode(N, H, dk, dv, steps, dtype, "lightning", seed=dk * 3 + dv, device="cuda",
                      slots=slots)
    idx = torch.tensor([7, 0, 3, 8, 2], dtype=torch.int32, device="cuda")
    state = d["state"].clone()
    ref_state = host(state).astype(np.float64)
    untouched = [s for s in range(slots) if s not in idx.tolist()]
    before_untouched = state[untouched].clone()
    for i in range(steps):
        out = nan_like((N, H, dv), d["v"].dtype)
        o = sgla.recurrent_step(d["q"][i], d["k"][i], d["v"][i], d["g"][i], state,
                                state_indices=idx, scale=d["scale"], out=out)
        torch.cuda.synchronize()
        ro = oracle.step(host(d["q"][i]), host(d["k"][i]), host(d["v"][i]), host(d["g"][i]),
                         ref_state, d["scale"], state_indices=idx.cpu().numpy())
        check(host(o), ro, dtype, "step %d o" % i)
        check(host(state[idx.long()]), ref_state[idx.cpu().numpy()], dtype, "step %d state" % i,
              bf16_out=False)
    assert torch.equal(state[untouched], before_untouched)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_step_equals_one_token_chunk(dtype):
    say("recurrent_step == chunk_fwd(T=1)", dtype)
    N, H, D = 4, 2, 128
    d = W.make_decode(N, H, D, D, 1, dtype, "lightning", seed=21, device="cuda")
    state = d["state"].clone()
    o_step = sgla.recurrent_step(d["q"][0], d["k"][0], d["v"][0], d["g"][0], state)
    o_chunk, S_chunk = sgla.chunk_fwd(d["q"][0][:, None].contiguous(),
                                      d["k"][0][:, None].contiguous(),
                                      d["v"][0][:, None].contiguous(),
                                      d["g"][0][:, None].contiguous(),
                                      initial_state=d["state"])
    torch.cuda.synchronize()
    check(host(o_step), host(o_chunk[:, 0]), dtype, "step vs chunk o")
    check(host(state), host(S_chunk), dtype, "step vs chunk state", bf16_out=False)


def test_workload_decode_every_state():
    """The batched-decode workload (256 x 32 heads, 64 steps), in the launch
    configuration the benchmark times; the oracle follows every one of the
    8192 (sequence, head) states through all 64 steps."""
    say("recurrent_step workload N=256 H=32 D=128 64 steps seed=4 (every state)")
    d = W.make_workload("decode_bf16_n256_h32_d128_x64", seed=4, device="cuda")
    state = d["state"]
    ref = np.ascontiguousarray(host(state).astype(np.float64))  # [256, 32, D, D]
    for i in range(64):
        o = sgla.recurrent_step(d["q"][i], d["k"][i], d["v"][i], d["g"][i], state,
                                scale=d["scale"])
        ro = oracle.step(host(d["q"][i]), host(d["k"][i]), host(d["v"][i]), host(d["g"][i]), ref,
                         d["scale"])
        check(host(o), ro, "bf16", "decode step %d o" % i)
    torch.cuda.synchronize()
    check(host(state), ref, "bf16", "decode final states", bf16_out=False)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_step_per_head_constant_decay(dtype):
    """The per-head constant decays of the lightning layer (blueprint page,
    section "B2 lightning-attn (Simple GLA)": -0.917 .. -0.0001), 20 steps."""
    say("recurrent_step constant per-head decay", dtype)
    N, H, steps = 6, 8, 20
    d = W.make_decode(N, H, 128, 128, steps, dtype, "lightning", seed=61, device="cuda")
    gg = -0.917 * (0.0001 / 0.917) ** (np.arange(H) / (H - 1))
    g = torch.tensor(gg, dtype=torch.float32, device="cuda").view(1, H).expand(N, H).contiguous()
    state = d["state"].clone()
    ref = np.ascontiguousarray(host(state).astype(np.float64))
    for i in range(steps):
        o = sgla.recurrent_step(d["q"][i], d["k"][i], d["v"][i], g, state, scale=d["scale"])
        ro = oracle.step(host(d["q"][i]), host(d["k"][i]), host(d["v"][i]), host(g), ref,
                         d["scale"])
        torch.cuda.synchronize()
        check(host(o), ro, dtype, "step %d o" % i)
    check(host(state), ref, dtype, "constant decay states", bf16_out=False)

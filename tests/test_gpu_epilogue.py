"""GPU parity of sgla_out_norm_gate (RMSNorm over all heads of a token, then
the sigmoid gate) against ``oracle/epilogue.py``.

With bf16 tensors the kernel takes its three bf16 roundings from fp32 values,
the oracle from fp64 ones; an element whose exact value lies within 2^-16 of
its size from a midpoint between two bf16 numbers may round either way, both
correct. The oracle bounds what that can change per element, and the bound is
added to the max-abs bar there (rel-L2 unchanged); the step is elementwise
after the row norm, so nothing spreads.
"""
import numpy as np
import pytest
import torch

import linear_attention_hybrid_amd as sgla
import oracle.epilogue as E
import sgla_inputs as W
from tests.parity import check, host, nan_like, say

pytestmark = pytest.mark.gpu

EPS = 1e-6
TIE_ETA = 2.0 ** -16


def reference(inp):
    bf16 = inp["dtype"] == "bf16"
    if bf16:
        return E.out_norm_gate(host(inp["o"]), host(inp["z"]), host(inp["weight"]), EPS, True,
                               tie_eta=TIE_ETA)
    return E.out_norm_gate(host(inp["o"]), host(inp["z"]), host(inp["weight"]), EPS, False), None


def run(inp, in_place=False):
    o = inp["o"].clone() if in_place else inp["o"]
    out = o if in_place else nan_like(tuple(o.shape), o.dtype)
    r = sgla.out_norm_gate(o, inp["z"], inp["weight"], eps=EPS, out=out)
    torch.cuda.synchronize()
    return r


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rows,width", [(37, 4096), (5, 192), (3, 8), (2, 16384), (11, 1024 + 8)])
def test_rows(dtype, rows, width):
    say("out_norm_gate", dtype, "rows", rows, "width", width)
    inp = W.make_epilogue(rows, width, dtype, seed=rows * 7 + width, device="cuda")
    got = run(inp)
    ref, bound = reference(inp)
    check(host(got), ref, dtype, "epilogue %dx%d" % (rows, width), allowance=bound)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_in_place_equals_out_of_place(dtype):
    say("out_norm_gate in place", dtype)
    inp = W.make_epilogue(64, 4096, dtype, seed=3, device="cuda")
    a = run(inp)
    b = run(inp, in_place=True)
    assert torch.equal(a, b)


def test_gate_limits_on_the_gpu():
    """Gate logits of +60 (sigmoid rounds to 1) give the normalised row; -200
    (sigmoid below the smallest fp32 number) gives zeros. bf16 keeps fp32's
    exponent range, so -60 would still give values near 1e-26."""
    say("out_norm_gate gate limits")
    inp = W.make_epilogue(8, 4096, "bf16", seed=4, device="cuda")
    openg = dict(inp, z=torch.full_like(inp["z"], 60.0))
    shut = dict(inp, z=torch.full_like(inp["z"], -200.0))
    y = host(run(openg))
    ref = E.out_norm_gate(host(inp["o"]), np.full(inp["o"].shape, 60.0), host(inp["weight"]), EPS,
                          True, tie_eta=TIE_ETA)
    check(y, ref[0], "bf16", "open gate", allowance=ref[1])
    assert torch.all(run(shut) == 0)


def test_workload_prefill_rows():
    """The shape of one lightning layer's prefill: 8192 tokens x 32 heads x
    128, every element against the oracle."""
    say("out_norm_gate 8192 x 4096 bf16 seed=2")
    inp = W.make_epilogue(8192, 4096, "bf16", seed=2, device="cuda")
    got = run(inp)
    ref, bound = reference(inp)
    check(host(got), ref, "bf16", "epilogue 8192x4096", allowance=bound)

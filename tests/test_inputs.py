"""The seeded input generators: determinism and the stated distributions."""
import math

import numpy as np
import torch

import sgla_inputs as W


def test_same_seed_same_bytes():
    a = W.make_prefill(1, 100, 3, 16, 16, "bf16", "lightning", seed=5)
    b = W.make_prefill(1, 100, 3, 16, 16, "bf16", "lightning", seed=5)
    c = W.make_prefill(1, 100, 3, 16, 16, "bf16", "lightning", seed=6)
    for key in ("q", "k", "v", "g"):
        assert torch.equal(a[key], b[key])
        assert not torch.equal(a[key], c[key])


def test_lightning_rows_unit_rms_and_gates_negative():
    w = W.make_prefill(1, 512, 4, 128, 128, "f32", "lightning", seed=1)
    rms = w["q"].pow(2).mean(-1).sqrt()
    assert torch.allclose(rms, torch.ones_like(rms), atol=1e-4)
    g = w["g"]
    assert torch.all(g < 0)
    # x ~ N(4, 1): the mean of log(sigmoid(x)) is about -0.029.
    assert -0.04 < float(g.mean()) < -0.02
    assert w["scale"] == 1.0 / math.sqrt(128)


def test_gaussian_preset_gate_mean():
    w = W.make_prefill(1, 4096, 4, 8, 8, "f32", "gaussian", seed=2)
    assert -0.09 < float(w["g"].mean()) < -0.06
    assert abs(float(w["v"].std()) - 1.0) < 0.05


def test_raw_preset_rows_vary_in_scale_and_weights():
    w = W.make_prefill(1, 2048, 4, 128, 128, "f32", "raw", seed=3)
    log_rms = w["k"].pow(2).mean(-1).sqrt().log()
    # per-row factor exp(N(0, 0.5^2)) on rows of unit expected RMS
    assert abs(float(log_rms.std()) - 0.5) < 0.05
    assert torch.all(w["g"] < 0)
    qw, kw = W.norm_weights(128, seed=3)
    assert qw.shape == (128,) and qw.dtype == torch.float32
    assert abs(float(torch.cat([qw, kw]).mean()) - 1.0) < 0.03
    assert not torch.equal(qw, kw)


def test_varlen_lengths():
    L = W.varlen_lengths(8, 524288, 4096, 262144, seed=5)
    assert L.sum() == 524288 and len(L) == 8 and np.all(L > 0)
    assert np.array_equal(L, W.varlen_lengths(8, 524288, 4096, 262144, seed=5))
    cu = W.cu_from_lengths(L)
    assert cu[0] == 0 and cu[-1] == 524288
    pos = W.positions_for(int(cu[-1]), cu)
    assert np.all(pos[cu[:-1]] == 0)


def test_decode_inputs_shapes():
    d = W.make_decode(3, 2, 16, 16, steps=4, seed=1)
    assert d["q"].shape == (4, 3, 2, 16) and d["q"].dtype == torch.bfloat16
    assert d["state"].shape == (3, 2, 16, 16) and d["state"].dtype == torch.float32
    assert abs(float(d["state"].std()) - 0.02) < 0.005


def test_workloads_table_names_sizes():
    for name, w in W.WORKLOADS.items():
        assert w["dtype"] in ("f32", "bf16")
        assert w["H"] >= 1

"""Seeded synthetic inputs: shapes, determinism, bf16 rounding (no GPU)."""
import numpy as np
import torch

from capacity_routing_expert_amd import workloads as W


def test_bf16_rounding_matches_torch():
    rng = np.random.Generator(np.random.PCG64(0))
    a = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-20, 20, 100000),
                        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, 1e-40, 1.00390625, 1.01171875], np.float32)])
    ours = W.f32_to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = W.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(a).to(torch.bfloat16).float().numpy())


def test_worked_example_shapes_and_determinism():
    a = W.make_inputs("worked_example")
    b = W.make_inputs("worked_example")
    assert a["x"].shape == (8, 4) and a["x"].dtype == np.float32
    assert a["w_router"].shape == (4, 4)
    assert a["w1"].shape == (4, 8, 4) and a["b1"].shape == (4, 8)
    assert a["w2"].shape == (4, 4, 8) and a["b2"].shape == (4, 4)
    assert a["b_router"] is None
    for k in ("x", "w_router", "w1", "b1", "w2", "b2"):
        assert np.array_equal(a[k], b[k])


def test_small_override_bf16():
    wl = W.WORKLOADS["fine"]
    a = W.make_inputs(wl, T=32)
    assert a["x"].shape == (32, 2048) and a["x"].dtype == np.uint16
    assert a["w1"].shape == (64, 1408, 2048)
    # log-Zipf router bias: ranks 1..64 over a permutation
    b = np.sort(a["b_router"])[::-1]
    assert b[0] == 0.0 and abs(b[1] - np.float32(-1.1 * np.log(2))) < 1e-6
    assert abs(b[-1] - np.float32(-1.1 * np.log(64))) < 1e-5

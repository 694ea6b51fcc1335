"""The seeded input generator: bf16 rounding and reproducibility."""

import numpy as np
import torch

from synth import bf16_bits_to_f32, f32_to_bf16_bits, make_inputs, spec


def test_bf16_rounding_matches_torch():
    r = np.random.default_rng(0)
    a = np.concatenate([r.standard_normal(100000).astype(np.float32) * 37,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.0e38, 1e-40],
                                 dtype=np.float32)])
    ours = f32_to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(a).to(torch.bfloat16).float().numpy())


def test_inputs_are_reproducible_and_shaped():
    sp = spec("mixtral_swiglu_bf16", T=40, D=64, DH=96, E=4)
    a, b = make_inputs(sp, seed=3), make_inputs(sp, seed=3)
    for name in ("x", "w_router", "w1", "w3", "w2"):
        assert np.array_equal(getattr(a, name), getattr(b, name))
        assert getattr(a, name).dtype == np.uint16
    assert a.x.shape == (40, 64) and a.w1.shape == (4, 64, 96) and a.w2.shape == (4, 96, 64)
    assert a.bias is None
    c = make_inputs(sp, seed=4)
    assert not np.array_equal(a.x, c.x)


def test_router_zero_keeps_the_stream():
    sp = spec("tiny_linear_f32")
    a, z = make_inputs(sp), make_inputs(sp, router_zero=True)
    assert (z.w_router == 0).all()
    assert np.array_equal(a.x, z.x) and np.array_equal(a.w1, z.w1)


def test_zipf_bias():
    sp = spec("fine_grained_zipf_bf16", T=8, D=16, DH=16)
    b = make_inputs(sp).bias.astype(np.float64)
    p = np.exp(b) / np.exp(b).sum()
    ranks = np.arange(1, sp.E + 1)
    assert np.allclose(p, (1 / ranks) / (1 / ranks).sum(), rtol=1e-6)

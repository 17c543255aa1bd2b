"""Pins of the oracle's scalar epilogue (silu_affine: x / (1 + exp(-x)) * scale + bias, the
pages' "Scalar compositions" example) against torch's own SiLU in float64 and closed forms."""
import numpy as np
import torch


def test_silu_affine_vs_torch(O):
    x = np.concatenate([np.linspace(-30, 30, 1201), np.random.default_rng(0).standard_normal(1000) * 8])
    for scale, bias in ((2.0, 1.0), (1.0, 0.0), (-0.75, 3.5)):
        ref = torch.nn.functional.silu(torch.from_numpy(x)).numpy() * scale + bias
        np.testing.assert_allclose(O.ewise_silu_affine(x, scale, bias), ref, rtol=1e-14, atol=1e-14)


def test_silu_affine_closed_forms(O):
    x = np.array([0.0, 1e-300, 50.0, -50.0, 1.0, -1.0, 3.0, -3.0])
    y = O.ewise_silu_affine(x, 1.0, 0.0)
    assert y[0] == 0.0 and y[1] == 0.5e-300                 # silu(0) = 0, silu(x) ~ x/2 near 0
    assert abs(y[2] - 50.0) < 1e-18 * 50 + 2e-20              # silu(x) -> x for large x
    assert 0 > y[3] > -50.0 * np.exp(-49.0)                   # silu(x) ~ x e^x -> 0- for large -x
    assert np.allclose(y[4::2] - y[5::2], x[4::2], rtol=0, atol=1e-15)  # silu(x) - silu(-x) = x
    assert np.array_equal(O.ewise_silu_affine(x, 2.0, 1.0), 2.0 * y + 1.0)  # affine part

"""The seeded workload generators are deterministic and have the intended
shapes and value structure."""
import hashlib

import numpy as np
import pytest

from mxfp4_activation_quantizer_amd import inputs


def _digest(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def test_tiny_is_deterministic_and_shaped():
    x1, x2 = inputs.activation("tiny"), inputs.activation("tiny")
    assert x1.dtype == np.uint16 and x1.shape == (64, 256)
    assert _digest(x1) == _digest(x2)
    xf = inputs.bf16_bits_to_f32(x1)
    amax = np.abs(xf).max(axis=0)
    assert set(np.argsort(amax)[-2:]) == {7, 100}          # the two x30 channels
    assert 0.8 < np.std(np.delete(xf, [7, 100], axis=1)) < 1.2


def test_params_are_hadamard_plus_noise():
    p = inputs.lu_params("tiny")
    assert p.shape == (8, 5, 3) and p.dtype == np.float32
    dev = p - inputs.hadamard_init(8)
    assert 0.02 < dev.std() < 0.08
    assert np.all(np.abs(p[:, :, 1]) >= inputs.U_MIN)
    np.testing.assert_array_equal(p, inputs.lu_params("tiny"))


def test_bf16_rounding_is_nearest_even():
    import torch
    g = np.random.default_rng(0)
    f = g.standard_normal(10000) * 100
    want = torch.from_numpy(f.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
    np.testing.assert_array_equal(inputs.f64_to_bf16_bits(f), want.view(np.uint16))


@pytest.mark.slow
@pytest.mark.parametrize("name", ["pixart", "flux_attn"])
def test_large_workloads_shape_and_outliers(name):
    w = inputs.WORKLOADS[name]
    x = inputs.activation(name)
    assert x.shape == (w.tokens, w.d)
    xf = inputs.bf16_bits_to_f32(x)
    assert np.all(np.isfinite(xf))
    col = np.abs(xf).max(axis=0)
    # outlier channels stand out by more than an order of magnitude
    assert col.max() > 10 * np.median(col)
    assert w.algorithmic_bytes == w.elements * 2 + w.elements // 2 + w.elements // 32


def test_smooth_multipliers_recipe():
    x = inputs.activation("tiny")
    m = inputs.smooth_multipliers(x)
    a = np.abs(inputs.bf16_bits_to_f32(x)).max(axis=0)
    np.testing.assert_allclose(m, a ** -0.5, rtol=1e-6)

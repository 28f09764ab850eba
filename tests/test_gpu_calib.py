"""GPU parity of the calibration kernels through the C ABI: the per-block
objective against the oracle's fp64 definition, the evolution-strategy step
bit for bit against the oracle's fp32 step, and an end-to-end calibration
that must lower the held-out round-trip error below the Hadamard start."""
import numpy as np
import pytest

import oracle
from mxfp4_activation_quantizer_amd import inputs, kq
from parity import to_gpu, to_gpu_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch


def _np(t):
    return t.cpu().numpy()


def _assert_objective_close(fg, fo, x_bits, d, blocks=None):
    xf = inputs.bf16_bits_to_f32(x_bits[:, :d]).astype(np.float64)
    energy = (xf.reshape(xf.shape[0], -1, 32) ** 2).sum(axis=(0, 2))
    if blocks is not None:
        energy = energy[blocks]
    tol = 1e-4 * np.abs(fo) + 1e-6 * energy
    assert np.all(np.abs(fg.astype(np.float64) - fo) <= tol), np.max(np.abs(fg - fo) / (tol + 1e-300))


@pytest.mark.parametrize("name,tokens", [("tiny", 64), ("pixart", 300), ("flux_attn", 257)])
def test_objective_vs_oracle(torch_cuda, name, tokens):
    x = inputs.activation(name)[:tokens]
    lu = inputs.lu_params(name)
    fg = _np(kq.calib_objective(to_gpu_bf16(x), to_gpu(lu)))
    fo = oracle.calib_objective(x, lu)
    _assert_objective_close(fg, fo, x, x.shape[1])


def test_objective_with_weight_gram(torch_cuda):
    x = inputs.activation("tiny")
    lu = inputs.lu_params("tiny")
    g = np.random.default_rng(3)
    w = g.normal(0, 0.02, (8, 48, 32))
    gram = np.einsum("jna,jnb->jab", w, w).astype(np.float32)
    fg = _np(kq.calib_objective(to_gpu_bf16(x), to_gpu(lu), to_gpu(gram)))
    fo = oracle.calib_objective(x, lu, gram)
    assert np.allclose(fg, fo, rtol=1e-4, atol=1e-9 * np.abs(fo).max())


def test_objective_strided_nan_and_deterministic(torch_cuda):
    torch = torch_cuda
    x = inputs.activation("tiny").copy()
    x[5, 40] = 0x7FC0  # NaN in block 1
    xd = to_gpu_bf16(x)
    lu = inputs.lu_params("tiny")[:4].copy()
    f1 = _np(kq.calib_objective(xd, to_gpu(lu), d=128))
    f2 = _np(kq.calib_objective(xd, to_gpu(lu), d=128))
    assert np.isnan(f1[1]) and not np.isnan(f1[[0, 2, 3]]).any()
    assert np.array_equal(f1[[0, 2, 3]], f2[[0, 2, 3]])
    fo = oracle.calib_objective(x, lu, d=128)
    keep = [0, 2, 3]
    _assert_objective_close(f1[keep], fo[keep], x, 128, blocks=keep)
    # no tokens: zeros
    z = _np(kq.calib_objective(xd[:0], to_gpu(lu), d=128))
    assert np.array_equal(z, np.zeros(4, np.float32))


def test_es_update_bit_exact(torch_cuda):
    g = np.random.default_rng(4)
    nb = 300
    theta = (inputs.hadamard_init(nb) + g.normal(0, 0.1, (nb, 5, 3))).astype(np.float32).reshape(nb, 15)
    sigma = g.choice([1e-4, 3e-3, 0.05, 0.4, 0.5], nb).astype(np.float32)
    fbest = g.uniform(1, 2, nb).astype(np.float32)
    cand = (theta + g.normal(0, 0.05, theta.shape)).astype(np.float32)
    fcand = (fbest + g.choice([-0.3, 0.0, 0.2], nb)).astype(np.float32)
    noise = g.standard_normal((nb, 15)).astype(np.float32)
    noise[::17, 1] = -theta[::17, 1] / np.maximum(sigma[::17], 1e-4)  # u pushed toward 0
    dev = [to_gpu(a.copy()) for a in (theta, sigma, fbest, cand, fcand, noise)]
    st = kq.kq_calib_es_update(nb, *[t.data_ptr() for t in dev],
                               __import__("torch").cuda.current_stream().cuda_stream)
    assert st == kq.KQ_OK
    oracle.calib_es_update(theta, sigma, fbest, cand, fcand, noise)
    for got, want in zip(dev[:4], (theta, sigma, fbest, cand)):
        np.testing.assert_array_equal(_np(got).view(np.uint32), want.view(np.uint32))


def test_calibration_lowers_held_out_error(torch_cuda):
    torch = torch_cuda
    x = inputs.activation("flux_attn")
    cal, held = to_gpu_bf16(x[:256]), to_gpu_bf16(x[2048:2304])
    nb = 96
    start = to_gpu(inputs.hadamard_init(nb))
    noise = to_gpu(inputs.calib_noise("flux_attn", 150))
    theta, fbest, hist = kq.calibrate(cal, start, noise)
    h = _np(hist)
    assert np.all(np.diff(h, axis=0) <= 0), "a kept objective went up"
    # the kept parameters reproduce the kept objective exactly
    assert np.array_equal(_np(kq.calib_objective(cal, theta)), _np(fbest))
    f0 = _np(kq.calib_objective(held, start)).astype(np.float64)
    f1 = _np(kq.calib_objective(held, theta)).astype(np.float64)
    xf = inputs.bf16_bits_to_f32(x[2048:2304]).astype(np.float64)
    e0, e1 = np.sqrt(f0.sum() / (xf ** 2).sum()), np.sqrt(f1.sum() / (xf ** 2).sum())
    print(f"held-out MXFP4 round-trip rel. error: Hadamard start {e0:.4f}, calibrated {e1:.4f}",
          flush=True)
    assert e1 < 0.9 * e0
    # and the held-out objective of the learned parameters matches the oracle
    fo = oracle.calib_objective(x[2048:2304], _np(theta))
    _assert_objective_close(f1.astype(np.float32), fo, x[2048:2304], 3072)

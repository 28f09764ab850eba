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


@pytest.mark.parametrize("with_gram,strided", [(False, False), (True, True)])
def test_es_step_equals_objective_then_update(torch_cuda, with_gram, strided):
    """kq_calib_es_step is defined as kq_calib_objective on the candidates
    followed by kq_calib_es_update: run both sequences side by side for several
    iterations and compare every state array bit for bit after each one."""
    torch = torch_cuda
    x = inputs.activation("flux_attn")[:300]
    nb = 64 if strided else 96
    d = nb * 32
    xd = to_gpu_bf16(x)
    gram = None
    if with_gram:
        g = np.random.default_rng(11)
        w = g.normal(0, 1, (nb, 48, 32))
        gram = to_gpu(np.einsum("jab,jac->jbc", w, w).astype(np.float32) / 48)
    noise = to_gpu(inputs.calib_noise("flux_attn", 6, blocks=nb))
    start = inputs.hadamard_init(nb).reshape(nb, 15)
    st = torch.cuda.current_stream().cuda_stream
    gp = gram.data_ptr() if gram is not None else None

    def fresh():
        theta = to_gpu(start.copy())
        sigma = torch.full((nb,), 0.05, dtype=torch.float32, device="cuda")
        fbest = kq.calib_objective(xd, theta, gram, d=d)
        cand = theta.clone()
        inf = torch.full((nb,), float("inf"), dtype=torch.float32, device="cuda")
        assert kq.kq_calib_es_update(nb, theta.data_ptr(), sigma.data_ptr(), fbest.data_ptr(),
                                     cand.data_ptr(), inf.data_ptr(), noise[0].data_ptr(),
                                     st) == kq.KQ_OK
        return theta, sigma, fbest, cand

    a, b = fresh(), fresh()
    fcand = torch.empty(nb, dtype=torch.float32, device="cuda")
    fhist = torch.full((nb,), -1.0, dtype=torch.float32, device="cuda")
    for i in range(1, noise.shape[0]):
        kq.calib_objective(xd, a[3], gram, d=d, f=fcand)
        assert kq.kq_calib_es_update(nb, *[t.data_ptr() for t in a], fcand.data_ptr(),
                                     noise[i].data_ptr(), st) == kq.KQ_OK
        assert kq.kq_calib_es_step(xd.data_ptr(), x.shape[0], d, xd.stride(0), gp,
                                   *[t.data_ptr() for t in b], noise[i].data_ptr(),
                                   fhist.data_ptr(), st) == kq.KQ_OK
        for ga, gb in zip(a, b):
            np.testing.assert_array_equal(_np(ga).view(np.uint32), _np(gb).view(np.uint32))
        np.testing.assert_array_equal(_np(fhist).view(np.uint32), _np(b[2]).view(np.uint32))
    # at least one block kept a candidate, so the update path was exercised
    assert not np.array_equal(_np(b[0]), start)
    # the kept objective is the objective of the kept parameters
    np.testing.assert_array_equal(_np(kq.calib_objective(xd, b[0], gram, d=d)), _np(b[2]))


def test_es_run_equals_repeated_steps(torch_cuda):
    """kq_calib_es_run over several iterations against the same number of
    kq_calib_es_step calls, bit for bit, history rows included."""
    torch = torch_cuda
    x = to_gpu_bf16(inputs.activation("pixart")[:200])
    nb, iters = 36, 7
    noise = to_gpu(inputs.calib_noise("pixart", iters - 1, blocks=nb))
    start = inputs.hadamard_init(nb).reshape(nb, 15)
    st = torch.cuda.current_stream().cuda_stream

    def state():
        theta = to_gpu(start.copy())
        cand = to_gpu((start + 0.01).astype(np.float32))
        sigma = torch.full((nb,), 0.05, dtype=torch.float32, device="cuda")
        fbest = kq.calib_objective(x, theta)
        return [theta, sigma, fbest, cand]

    a, b = state(), state()
    ha = torch.full((iters, nb), -1.0, dtype=torch.float32, device="cuda")
    hb = torch.full((iters, nb), -1.0, dtype=torch.float32, device="cuda")
    for i in range(iters):
        assert kq.kq_calib_es_step(x.data_ptr(), x.shape[0], nb * 32, x.stride(0), None,
                                   *[t.data_ptr() for t in a], noise[i].data_ptr(),
                                   ha[i].data_ptr(), st) == kq.KQ_OK
    assert kq.kq_calib_es_run(x.data_ptr(), x.shape[0], nb * 32, x.stride(0), None,
                              *[t.data_ptr() for t in b], noise.data_ptr(), iters,
                              hb.data_ptr(), st) == kq.KQ_OK
    for ga, gb in zip(a + [ha], b + [hb]):
        np.testing.assert_array_equal(_np(ga).view(np.uint32), _np(gb).view(np.uint32))
    assert np.all(_np(hb) >= 0)


def test_es_step_with_no_tokens(torch_cuda):
    torch = torch_cuda
    nb = 4
    xd = torch.zeros((0, 128), dtype=torch.bfloat16, device="cuda")
    theta = to_gpu(inputs.hadamard_init(nb).reshape(nb, 15))
    cand = theta.clone()
    sigma = torch.full((nb,), 0.05, dtype=torch.float32, device="cuda")
    fbest = torch.zeros(nb, dtype=torch.float32, device="cuda")
    noise = torch.ones((nb, 15), dtype=torch.float32, device="cuda")
    assert kq.kq_calib_es_step(xd.data_ptr(), 0, 128, 128, None, theta.data_ptr(),
                               sigma.data_ptr(), fbest.data_ptr(), cand.data_ptr(),
                               noise.data_ptr(), None,
                               torch.cuda.current_stream().cuda_stream) == kq.KQ_OK
    # objective 0 is not below the kept 0: rejected, sigma shrinks, next candidate proposed
    np.testing.assert_array_equal(_np(theta), inputs.hadamard_init(nb).reshape(nb, 15))
    np.testing.assert_array_equal(_np(sigma), np.full(nb, np.float32(0.05) * np.float32(0.90360200)))
    assert np.all(_np(fbest) == 0)
    want = (np.float32(0.05) * np.float32(0.90360200)) + inputs.hadamard_init(nb).reshape(nb, 15)
    np.testing.assert_array_equal(_np(cand), want)


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

"""Sizes at the ends of the entry points' ranges: activation tensors past
4 GiB (every byte offset past 32 bits) through the quantizer, the inverse
side and the AdaLN-fused quantizer, and a GEMM whose activation operand is
one row short of the 2 GiB limit on an operand's codes.  Sampled rows (the
first, the middle, the last two, and seeded random ones) are compared with
the oracle run on those rows alone: bit for bit for the quantizers and the
inverse, to the GEMM's fp32-accumulation bound for the GEMM."""
import numpy as np
import pytest

import oracle
from mxfp4_activation_quantizer_amd import inputs, kq
from parity import assert_gemm_close, gemm_reference, to_gpu

pytestmark = pytest.mark.gpu

TOKENS, D = 540_000, 4096          # 4.42 GB of bf16 input, 69.1 M units


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch


def _rows(n, seed):
    g = np.random.default_rng(seed)
    extra = g.choice(n, 27, replace=False)
    return np.unique(np.concatenate([[0, n // 2, n - 2, n - 1], extra]))


def _host_rows(t, rows, torch):
    idx = torch.from_numpy(rows).to(t.device)
    sub = t.index_select(0, idx)
    if sub.dtype == torch.bfloat16:
        sub = sub.view(torch.int16)
    out = sub.cpu().numpy()
    return out.view(np.uint16) if out.dtype == np.int16 else out


@pytest.fixture(scope="module")
def big_x(torch_cuda):
    torch = torch_cuda
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(5)
    x = torch.empty((TOKENS, D), dtype=torch.bfloat16, device="cuda:0")
    x.normal_(0.0, 1.0, generator=gen)
    assert x.numel() * 2 > 2 ** 32
    yield x
    del x
    torch.cuda.empty_cache()


def test_quantizer_and_inverse_past_4gib(torch_cuda, big_x):
    torch = torch_cuda
    lu_np = inputs.lu_params("flux_mlp", blocks=D // 32)
    lu = to_gpu(lu_np)
    codes, scales = kq.transform_quant(big_x, lu)
    back = kq.dequant_inverse(codes, scales, lu)
    torch.cuda.synchronize()
    rows = _rows(TOKENS, 1)
    xb = _host_rows(big_x, rows, torch)
    gc, gs = _host_rows(codes, rows, torch), _host_rows(scales, rows, torch)
    oc, os_ = oracle.transform_quant(xb, lu_np, oracle.STAGED32)
    assert np.array_equal(gc, oc) and np.array_equal(gs, os_)
    ob = oracle.dequant_inverse(oc, os_, lu_np, oracle.STAGED32)
    assert np.array_equal(_host_rows(back, rows, torch), ob)
    del codes, scales, back
    torch.cuda.empty_cache()


def test_adaln_quantizer_past_4gib(torch_cuda, big_x):
    torch = torch_cuda
    lu_np = inputs.lu_params("flux_mlp", blocks=D // 32)
    shift_np, scale_np = inputs.modulation("flux_mlp", samples=2, d=D)
    rps = TOKENS // 2
    codes, scales = kq.adaln_transform_quant(big_x, to_gpu(shift_np), to_gpu(scale_np),
                                             to_gpu(lu_np), rows_per_sample=rps)
    torch.cuda.synchronize()
    rows = _rows(TOKENS, 2)
    xb = _host_rows(big_x, rows, torch)
    gc, gs = _host_rows(codes, rows, torch), _host_rows(scales, rows, torch)
    for s in (0, 1):  # LayerNorm is per row: each sample's rows alone
        sel = (rows // rps) == s
        oc, os_ = oracle.adaln_transform_quant(xb[sel], shift_np[s:s + 1], scale_np[s:s + 1],
                                               lu_np, rows_per_sample=int(sel.sum()))
        assert np.array_equal(gc[sel], oc) and np.array_equal(gs[sel], os_)
    del codes, scales
    torch.cuda.empty_cache()


def test_gemm_activation_operand_at_2gib(torch_cuda):
    torch = torch_cuda
    K, N = 4096, 72
    M = 2 ** 31 // (K // 2) - 1          # codes one row short of 2 GiB
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(7)
    ac = torch.randint(0, 256, (M, K // 2), dtype=torch.uint8, device="cuda:0", generator=gen)
    as_ = torch.randint(118, 128, (M, K // 32), dtype=torch.uint8, device="cuda:0", generator=gen)
    g = np.random.default_rng(8)
    wc_np = g.integers(0, 256, (N, K // 2), dtype=np.uint8)
    ws_np = g.integers(118, 128, (N, K // 32), dtype=np.uint8)
    y = kq.w4a4_gemm(ac, as_, to_gpu(wc_np), to_gpu(ws_np))
    torch.cuda.synchronize()
    rows = _rows(M, 3)
    Y, B = gemm_reference(_host_rows(ac, rows, torch), _host_rows(as_, rows, torch), wc_np, ws_np)
    assert_gemm_close(_host_rows(y, rows, torch), Y, B, K)
    # one more row is past the limit
    too_big = kq.kq_w4a4_gemm(ac.data_ptr(), as_.data_ptr(), ac.data_ptr(), as_.data_ptr(),
                              M + 1, N, K, y.data_ptr(), y.stride(0), None)
    assert too_big == kq.KQ_ERR_SHAPE
    del ac, as_, y
    torch.cuda.empty_cache()

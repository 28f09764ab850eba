"""The hot path under HIP graph capture.  The entry points allocate nothing,
clear nothing and never synchronise, so a serving loop can capture the
quantizer feeding the W4A4 GEMM, and the AdaLN-fused quantizer, once and
replay them.  Every replay reads new activations that eager work has
written into the captured input buffer, and its outputs must equal eager
calls on the same input bit for bit; the first replay's quantizer output is
also checked against the oracle."""
import numpy as np
import pytest

import oracle
from mxfp4_activation_quantizer_amd import inputs, kq
from parity import to_gpu, to_gpu_bf16

pytestmark = pytest.mark.gpu

TOKENS, ROWS_PER_SAMPLE, N = 300, 150, 520


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch


def test_quantizer_gemm_and_adaln_replay_equal_eager(torch_cuda):
    torch = torch_cuda
    dev = torch.device("cuda:0")
    acts = inputs.activation("flux_attn")
    d = acts.shape[1]
    lu = to_gpu(inputs.lu_params("flux_attn"))
    shift_np, scale_np = inputs.modulation("flux_attn", samples=TOKENS // ROWS_PER_SAMPLE)
    shift, scale = to_gpu(shift_np), to_gpu(scale_np)
    g = np.random.default_rng(11)
    w = to_gpu_bf16(inputs.f64_to_bf16_bits(g.normal(0.0, 0.02, (N, d))))
    wc, ws = kq.weight_quant(w, lu)

    # captured buffers: input, quantizer output, GEMM output (rows padded to
    # 8 elements), AdaLN-fused quantizer output
    xs = to_gpu_bf16(acts[:TOKENS])
    codes = torch.empty((TOKENS, d // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((TOKENS, d // 32), dtype=torch.uint8, device=dev)
    y = torch.empty((TOKENS, (N + 7) // 8 * 8), dtype=torch.bfloat16, device=dev)[:, :N]
    ac = torch.empty_like(codes)
    asc = torch.empty_like(scales)

    def step():
        kq.transform_quant(xs, lu, codes=codes, scales=scales)
        kq.w4a4_gemm(codes, scales, wc, ws, y=y)
        kq.adaln_transform_quant(xs, shift, scale, lu, rows_per_sample=ROWS_PER_SAMPLE,
                                 codes=ac, scales=asc)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for rep in range(3):
        x_bits = acts[(rep + 1) * TOKENS:(rep + 2) * TOKENS]
        x_new = to_gpu_bf16(x_bits)
        xs.copy_(x_new)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [t.cpu().numpy().copy() for t in (codes, scales, ac, asc)]
        got_y = y.view(torch.int16).cpu().numpy().copy()

        ec, es = kq.transform_quant(x_new, lu)
        ey = kq.w4a4_gemm(ec, es, wc, ws)
        eac, eas = kq.adaln_transform_quant(x_new, shift, scale, lu,
                                            rows_per_sample=ROWS_PER_SAMPLE)
        torch.cuda.synchronize()
        want = [t.cpu().numpy() for t in (ec, es, eac, eas)]
        for name, a, b in zip(("codes", "scales", "adaln codes", "adaln scales"), got, want):
            assert np.array_equal(a, b), f"replay {rep}: {name} differ from the eager call"
        assert np.array_equal(got_y, ey.view(torch.int16).cpu().numpy()), \
            f"replay {rep}: GEMM output differs from the eager call"
        if rep == 0:
            oc, os_ = oracle.transform_quant(x_bits, inputs.lu_params("flux_attn"), oracle.STAGED32)
            assert np.array_equal(got[0], oc) and np.array_equal(got[1], os_)

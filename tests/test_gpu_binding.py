"""The Python binding rejects tensors that would hand a kernel a bad pointer
(host memory, a short buffer, a wrong dtype, mismatched operands) with a
ValueError before anything is launched."""
import numpy as np
import pytest

from mxfp4_activation_quantizer_amd import inputs, kq
from parity import to_gpu, to_gpu_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch


def _x(tokens=8, d=64):
    g = np.random.default_rng(3)
    return to_gpu_bf16(inputs.f64_to_bf16_bits(g.standard_normal((tokens, d))))


def test_parameters_must_be_gpu_f32_and_long_enough(torch_cuda):
    torch = torch_cuda
    x = _x()
    lu = inputs.hadamard_init(2)
    with pytest.raises(ValueError, match="lu must be a GPU tensor"):
        kq.transform_quant(x, torch.from_numpy(lu))            # host memory
    with pytest.raises(ValueError, match="lu has"):
        kq.transform_quant(x, to_gpu(lu[:1]))                   # one block of two
    with pytest.raises(ValueError, match="lu must be torch.float32"):
        kq.transform_quant(x, to_gpu(lu).double())
    with pytest.raises(ValueError, match="mult"):
        kq.smooth_quant(x, torch.ones(32, device="cuda"))       # d = 64 multipliers needed
    shift = torch.zeros((1, 64), device="cuda")
    with pytest.raises(ValueError, match="scale"):
        kq.adaln_transform_quant(x, shift, torch.zeros((1, 32), device="cuda"), to_gpu(lu))
    with pytest.raises(ValueError, match="shift"):
        kq.adaln_modulate(x, shift, shift, rows_per_sample=4)   # two samples, one row given


def test_outputs_and_operands_are_checked(torch_cuda):
    torch = torch_cuda
    x = _x(8, 128)  # the GEMM needs K % 128 == 0
    lu = to_gpu(inputs.hadamard_init(4))
    codes, scales = kq.transform_quant(x, lu)
    with pytest.raises(ValueError, match="codes"):
        kq.transform_quant(x, lu, codes=torch.empty((8, 16), dtype=torch.uint8, device="cuda"))
    with pytest.raises(ValueError, match="x_out"):
        kq.dequant_inverse(codes, scales, lu, x_out=torch.empty((8, 32), dtype=torch.bfloat16,
                                                                device="cuda"))
    with pytest.raises(ValueError, match="scales"):
        kq.dequant_inverse(codes, scales[:4], lu)
    with pytest.raises(ValueError, match="share K"):
        kq.w4a4_gemm(codes, scales, codes[:, :16], scales[:, :1])
    with pytest.raises(ValueError, match="y"):
        kq.w4a4_gemm(codes, scales, codes, scales, y=torch.empty((8, 8), dtype=torch.float32,
                                                                  device="cuda"))
    # one output row whose columns are strided is refused as well
    wide = torch.empty((1, 16), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="y"):
        kq.w4a4_gemm(codes[:1], scales[:1], codes, scales, y=wide[:, ::2])
    # a correct call still runs
    y = kq.w4a4_gemm(codes, scales, codes, scales)
    assert y.shape == (8, 8)


def test_calls_follow_the_current_stream(torch_cuda):
    """Each call is queued on torch's current stream.  Quantizer, inverse and
    GEMM calls interleaved on two side streams (default priority), each
    stream working on its own tensors, give the results of the same calls
    made one after another on the default stream."""
    torch = torch_cuda
    acts = inputs.activation("flux_attn")
    lu = to_gpu(inputs.lu_params("flux_attn"))
    xs = [to_gpu_bf16(acts[i * 200:(i + 1) * 200]) for i in range(4)]
    wc, ws = kq.transform_quant(xs[3], lu)

    def chain(x):
        c, s = kq.transform_quant(x, lu)
        return c, s, kq.dequant_inverse(c, s, lu), kq.w4a4_gemm(c, s, wc, ws)

    want = [chain(x) for x in xs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
    got = [None] * len(xs)
    for i, x in enumerate(xs):
        with torch.cuda.stream(streams[i % 2]):
            got[i] = chain(x)
    torch.cuda.synchronize()
    for g, w in zip(got, want):
        for a, b in zip(g, w):
            if a.dtype == torch.bfloat16:
                a, b = a.view(torch.int16), b.view(torch.int16)
            assert torch.equal(a, b)

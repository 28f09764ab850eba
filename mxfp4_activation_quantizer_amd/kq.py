"""Thin ctypes binding of ``libkq.so`` (the C ABI declared in ``include/kq.h``).

Two layers, both argument marshalling only:

* ``kq_*`` functions with the C names and signatures: raw device pointers
  (ints), sizes and a stream handle; they return the ``kq_status`` code.
* tensor helpers (``transform_quant`` ...): take torch tensors resident on the
  GPU, allocate the outputs with torch, pass ``data_ptr()`` and torch's current
  HIP stream, and raise :class:`KQError` on a non-OK status.

Every step of the computation runs in the gfx950 kernels of ``libkq.so``.
If the library is missing this module raises; there is no other code path.
"""
from __future__ import annotations

import ctypes
import os
import re

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkq.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "kq.h")

KQ_OK, KQ_ERR_NULL, KQ_ERR_SHAPE, KQ_ERR_ALIGN, KQ_ERR_HIP = 0, 1, 2, 3, 4

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_ST = ctypes.c_int

# name -> (restype, argtypes), in the order of include/kq.h
SIGNATURES = {
    "kq_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "kq_version": (ctypes.c_int, []),
    "kq_transform_quant": (_ST, [_P, _I64, _I64, _I64, _P, _P, _P, _P]),
    "kq_transform_quant_mfma": (_ST, [_P, _I64, _I64, _I64, _P, _P, _P, _P]),
    "kq_transform_quant_quad": (_ST, [_P, _I64, _I64, _I64, _P, _P, _P, _P]),
    "kq_transform_f32": (_ST, [_P, _I64, _I64, _I64, _P, _P, _P]),
    "kq_smooth_quant": (_ST, [_P, _I64, _I64, _I64, _P, _P, _P, _P]),
    "kq_fwht32_quant": (_ST, [_P, _I64, _I64, _I64, _P, _P, _P]),
    "kq_mxfp4_quant_f32": (_ST, [_P, _I64, _I64, _I64, _P, _P, _P]),
    "kq_weight_quant": (_ST, [_P, _I64, _I64, _I64, _P, _P, _P, _P]),
    "kq_dequant_inverse": (_ST, [_P, _P, _I64, _I64, _P, _P, _I64, _P]),
    "kq_w4a4_gemm": (_ST, [_P, _P, _P, _P, _I64, _I64, _I64, _P, _I64, _P]),
    "kq_adaln_transform_quant": (_ST, [_P, _I64, _I64, _I64, _P, _P, _I64, ctypes.c_float, _P,
                                       _P, _P, _P]),
    "kq_adaln_modulate": (_ST, [_P, _I64, _I64, _I64, _P, _P, _I64, ctypes.c_float, _P, _I64,
                                _P]),
    "kq_calib_objective": (_ST, [_P, _I64, _I64, _I64, _P, _P, _P, _P]),
    "kq_calib_es_update": (_ST, [_I64, _P, _P, _P, _P, _P, _P, _P]),
    "kq_calib_es_step": (_ST, [_P, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _P]),
    "kq_calib_es_run": (_ST, [_P, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _I64, _P, _P]),
    "kq_copy_ceiling": (_ST, [_P, _I64, _I64, _I64, _P, _P, _P]),
    "kq_stream_ceiling": (_ST, [_P, _I64, _P, _P, _P]),
}


class KQError(RuntimeError):
    def __init__(self, name: str, status: int):
        self.status = status
        super().__init__(f"{name}: {status_str(status)}")


_lib = None


def lib() -> ctypes.CDLL:
    """Load libkq.so; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it first "
                "(python -c 'import __graft_entry__ as g; g.build()')")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def declared_functions() -> list[str]:
    """Names of the functions include/kq.h declares."""
    with open(HEADER_PATH) as f:
        text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    return re.findall(r"\b(kq_[a-z0-9_]+)\s*\(", text)


def status_str(status: int) -> str:
    return lib().kq_status_str(status).decode()


def version() -> int:
    return lib().kq_version()


# ---- C-named wrappers (pointers as ints) -----------------------------------
def kq_transform_quant(x, tokens, d, ld_x, lu, codes, scales, stream=None) -> int:
    return lib().kq_transform_quant(x, tokens, d, ld_x, lu, codes, scales, stream)


def kq_transform_quant_mfma(x, tokens, d, ld_x, lu, codes, scales, stream=None) -> int:
    return lib().kq_transform_quant_mfma(x, tokens, d, ld_x, lu, codes, scales, stream)


def kq_transform_quant_quad(x, tokens, d, ld_x, lu, codes, scales, stream=None) -> int:
    return lib().kq_transform_quant_quad(x, tokens, d, ld_x, lu, codes, scales, stream)


def kq_transform_f32(x, tokens, d, ld_x, lu, y, stream=None) -> int:
    return lib().kq_transform_f32(x, tokens, d, ld_x, lu, y, stream)


def kq_smooth_quant(x, tokens, d, ld_x, mult, codes, scales, stream=None) -> int:
    return lib().kq_smooth_quant(x, tokens, d, ld_x, mult, codes, scales, stream)


def kq_fwht32_quant(x, tokens, d, ld_x, codes, scales, stream=None) -> int:
    return lib().kq_fwht32_quant(x, tokens, d, ld_x, codes, scales, stream)


def kq_mxfp4_quant_f32(y, tokens, d, ld_y, codes, scales, stream=None) -> int:
    return lib().kq_mxfp4_quant_f32(y, tokens, d, ld_y, codes, scales, stream)


def kq_weight_quant(w, rows, k, ld_w, lu, codes, scales, stream=None) -> int:
    return lib().kq_weight_quant(w, rows, k, ld_w, lu, codes, scales, stream)


def kq_dequant_inverse(codes, scales, tokens, d, lu, x_out, ld_out, stream=None) -> int:
    return lib().kq_dequant_inverse(codes, scales, tokens, d, lu, x_out, ld_out, stream)


def kq_w4a4_gemm(a_codes, a_scales, w_codes, w_scales, M, N, K, y, ld_y, stream=None) -> int:
    return lib().kq_w4a4_gemm(a_codes, a_scales, w_codes, w_scales, M, N, K, y, ld_y, stream)


def kq_adaln_transform_quant(x, tokens, d, ld_x, shift, scale, rows_per_sample, eps, lu, codes,
                             scales, stream=None) -> int:
    return lib().kq_adaln_transform_quant(x, tokens, d, ld_x, shift, scale, rows_per_sample, eps,
                                          lu, codes, scales, stream)


def kq_adaln_modulate(x, tokens, d, ld_x, shift, scale, rows_per_sample, eps, h, ld_h,
                      stream=None) -> int:
    return lib().kq_adaln_modulate(x, tokens, d, ld_x, shift, scale, rows_per_sample, eps, h, ld_h,
                                   stream)


def kq_calib_objective(x, tokens, d, ld_x, lu, gram, f, stream=None) -> int:
    return lib().kq_calib_objective(x, tokens, d, ld_x, lu, gram, f, stream)


def kq_calib_es_update(nb, theta, sigma, fbest, cand, fcand, noise, stream=None) -> int:
    return lib().kq_calib_es_update(nb, theta, sigma, fbest, cand, fcand, noise, stream)


def kq_calib_es_step(x, tokens, d, ld_x, gram, theta, sigma, fbest, cand, noise, fhist,
                     stream=None) -> int:
    return lib().kq_calib_es_step(x, tokens, d, ld_x, gram, theta, sigma, fbest, cand, noise,
                                  fhist, stream)


def kq_calib_es_run(x, tokens, d, ld_x, gram, theta, sigma, fbest, cand, noise, iterations, fhist,
                    stream=None) -> int:
    return lib().kq_calib_es_run(x, tokens, d, ld_x, gram, theta, sigma, fbest, cand, noise,
                                 iterations, fhist, stream)


def kq_copy_ceiling(x, tokens, d, ld_x, codes, scales, stream=None) -> int:
    return lib().kq_copy_ceiling(x, tokens, d, ld_x, codes, scales, stream)


def kq_stream_ceiling(src, units, codes, scales, stream=None) -> int:
    return lib().kq_stream_ceiling(src, units, codes, scales, stream)


# ---- tensor helpers --------------------------------------------------------
def _torch():
    import torch
    return torch


def _stream(t):
    torch = _torch()
    return torch.cuda.current_stream(t.device).cuda_stream


def _check(name: str, st: int) -> None:
    if st != KQ_OK:
        raise KQError(name, st)


def _act(x, dtype_name: str):
    torch = _torch()
    want = {"bf16": torch.bfloat16, "f32": torch.float32}[dtype_name]
    if x.dtype != want or x.dim() != 2 or not x.is_cuda:
        raise ValueError(f"expected a 2-D {want} GPU tensor, got {x.dtype} {tuple(x.shape)}")
    if x.stride(1) != 1:
        raise ValueError("the channel dimension must be contiguous")
    return x.shape[0], x.stride(0)


_DTYPES = {"bf16": "bfloat16", "f32": "float32", "u8": "uint8"}


def _dtype(name: str):
    return getattr(_torch(), _DTYPES[name])


def _param(t, name: str, device, dtype_name: str, numel: int):
    """A tensor a kernel reads whole through a plain pointer: on ``device``,
    of the dtype, contiguous, with at least ``numel`` elements.  Checked here
    so that a host tensor or a short buffer never reaches a kernel."""
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be a GPU tensor on {device}")
    if t.dtype != _dtype(dtype_name):
        raise ValueError(f"{name} must be {_dtype(dtype_name)}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{name} has {t.numel()} elements, needs at least {numel}")
    return t


def _rows_out(t, name: str, device, dtype_name: str, rows: int, cols: int):
    """A 2-D output written row by row: [>= rows][>= cols] on ``device`` with
    contiguous rows (the row stride is passed to the kernel)."""
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be a GPU tensor on {device}")
    if t.dtype != _dtype(dtype_name) or t.dim() != 2:
        raise ValueError(f"{name} must be a 2-D {_dtype(dtype_name)} tensor")
    if t.shape[0] < rows or t.shape[1] < cols or (cols > 1 and t.stride(1) != 1):
        raise ValueError(f"{name} must be [>={rows}][>={cols}] with contiguous rows")
    return t


def _mxfp4_out(x, tokens: int, d: int, codes=None, scales=None):
    torch = _torch()
    if codes is None:
        codes = torch.empty((tokens, d // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((tokens, d // 32), dtype=torch.uint8, device=x.device)
    _param(codes, "codes", x.device, "u8", tokens * (d // 2))
    _param(scales, "scales", x.device, "u8", tokens * (d // 32))
    return codes, scales


def _lu(lu, device, d: int):
    return _param(lu, "lu", device, "f32", (d // 32) * 15)


def transform_quant(x, lu, d: int | None = None, codes=None, scales=None):
    """KroQuant block transform + MXFP4 of bf16 ``x`` [tokens][>=d]."""
    tokens, ld = _act(x, "bf16")
    d = x.shape[1] if d is None else d
    codes, scales = _mxfp4_out(x, tokens, d, codes, scales)
    _lu(lu, x.device, d)
    _check("kq_transform_quant", kq_transform_quant(
        x.data_ptr(), tokens, d, ld, lu.data_ptr(), codes.data_ptr(), scales.data_ptr(),
        _stream(x)))
    return codes, scales


def transform_quant_mfma(x, lu, d: int | None = None, codes=None, scales=None):
    """The same quantizer with the block transform on the matrix cores."""
    tokens, ld = _act(x, "bf16")
    d = x.shape[1] if d is None else d
    codes, scales = _mxfp4_out(x, tokens, d, codes, scales)
    _lu(lu, x.device, d)
    _check("kq_transform_quant_mfma", kq_transform_quant_mfma(
        x.data_ptr(), tokens, d, ld, lu.data_ptr(), codes.data_ptr(), scales.data_ptr(),
        _stream(x)))
    return codes, scales


def transform_quant_quad(x, lu, d: int | None = None, codes=None, scales=None):
    """The same quantizer with four lanes per unit (cross-lane upper stages)."""
    tokens, ld = _act(x, "bf16")
    d = x.shape[1] if d is None else d
    codes, scales = _mxfp4_out(x, tokens, d, codes, scales)
    _lu(lu, x.device, d)
    _check("kq_transform_quant_quad", kq_transform_quant_quad(
        x.data_ptr(), tokens, d, ld, lu.data_ptr(), codes.data_ptr(), scales.data_ptr(),
        _stream(x)))
    return codes, scales


def transform_f32(x, lu, d: int | None = None, y=None):
    torch = _torch()
    tokens, ld = _act(x, "bf16")
    d = x.shape[1] if d is None else d
    if y is None:
        y = torch.empty((tokens, d), dtype=torch.float32, device=x.device)
    _param(y, "y", x.device, "f32", tokens * d)
    _lu(lu, x.device, d)
    _check("kq_transform_f32", kq_transform_f32(
        x.data_ptr(), tokens, d, ld, lu.data_ptr(), y.data_ptr(), _stream(x)))
    return y


def smooth_quant(x, mult, d: int | None = None, codes=None, scales=None):
    tokens, ld = _act(x, "bf16")
    d = x.shape[1] if d is None else d
    codes, scales = _mxfp4_out(x, tokens, d, codes, scales)
    _param(mult, "mult", x.device, "f32", d)
    _check("kq_smooth_quant", kq_smooth_quant(
        x.data_ptr(), tokens, d, ld, mult.data_ptr(), codes.data_ptr(), scales.data_ptr(),
        _stream(x)))
    return codes, scales


def fwht32_quant(x, d: int | None = None, codes=None, scales=None):
    tokens, ld = _act(x, "bf16")
    d = x.shape[1] if d is None else d
    codes, scales = _mxfp4_out(x, tokens, d, codes, scales)
    _check("kq_fwht32_quant", kq_fwht32_quant(
        x.data_ptr(), tokens, d, ld, codes.data_ptr(), scales.data_ptr(), _stream(x)))
    return codes, scales


def mxfp4_quant_f32(y, d: int | None = None, codes=None, scales=None):
    tokens, ld = _act(y, "f32")
    d = y.shape[1] if d is None else d
    codes, scales = _mxfp4_out(y, tokens, d, codes, scales)
    _check("kq_mxfp4_quant_f32", kq_mxfp4_quant_f32(
        y.data_ptr(), tokens, d, ld, codes.data_ptr(), scales.data_ptr(), _stream(y)))
    return codes, scales


def copy_ceiling(x, d: int | None = None, codes=None, scales=None):
    tokens, ld = _act(x, "bf16")
    d = x.shape[1] if d is None else d
    codes, scales = _mxfp4_out(x, tokens, d, codes, scales)
    _check("kq_copy_ceiling", kq_copy_ceiling(
        x.data_ptr(), tokens, d, ld, codes.data_ptr(), scales.data_ptr(), _stream(x)))
    return codes, scales


def stream_ceiling(src, codes=None, scales=None):
    """HBM reference pass over ``src`` (a contiguous GPU tensor of
    ``units * 64`` bytes): reads it and, when ``codes`` is given, writes
    ``units * 16`` bytes there and ``units`` bytes into ``scales``."""
    torch = _torch()
    if not src.is_cuda or not src.is_contiguous():
        raise ValueError("src must be a contiguous GPU tensor")
    nbytes = src.numel() * src.element_size()
    if nbytes % 64:
        raise ValueError("src must hold a whole number of 64-byte units")
    units = nbytes // 64
    if scales is None:
        scales = torch.empty(units if codes is not None else 1, dtype=torch.uint8,
                             device=src.device)
    if codes is not None:
        _param(codes, "codes", src.device, "u8", units * 16)
        _param(scales, "scales", src.device, "u8", units)
    else:
        _param(scales, "scales", src.device, "u8", 1)
    _check("kq_stream_ceiling", kq_stream_ceiling(
        src.data_ptr(), units, codes.data_ptr() if codes is not None else None,
        scales.data_ptr(), _stream(src)))
    return codes, scales


def dequant_inverse(codes, scales, lu, x_out=None):
    """bf16 [tokens][d] = dequant(codes, scales) times the inverse block transform."""
    torch = _torch()
    if codes.dtype != torch.uint8 or codes.dim() != 2 or not codes.is_cuda:
        raise ValueError("codes must be a 2-D uint8 GPU tensor")
    tokens, d = codes.shape[0], codes.shape[1] * 2
    _param(codes, "codes", codes.device, "u8", tokens * (d // 2))
    _param(scales, "scales", codes.device, "u8", tokens * (d // 32))
    _lu(lu, codes.device, d)
    if x_out is None:
        x_out = torch.empty((tokens, d), dtype=torch.bfloat16, device=codes.device)
    _rows_out(x_out, "x_out", codes.device, "bf16", tokens, d)
    _check("kq_dequant_inverse", kq_dequant_inverse(
        codes.data_ptr(), scales.data_ptr(), tokens, d, lu.data_ptr(), x_out.data_ptr(),
        x_out.stride(0), _stream(codes)))
    return x_out


def weight_quant(w, lu, k: int | None = None, codes=None, scales=None):
    """MXFP4 of W * T^-T (per 32-block along K) for bf16 weights ``w`` [N][>=K]."""
    rows, ld = _act(w, "bf16")
    k = w.shape[1] if k is None else k
    codes, scales = _mxfp4_out(w, rows, k, codes, scales)
    _lu(lu, w.device, k)
    _check("kq_weight_quant", kq_weight_quant(
        w.data_ptr(), rows, k, ld, lu.data_ptr(), codes.data_ptr(), scales.data_ptr(), _stream(w)))
    return codes, scales


def w4a4_gemm(a_codes, a_scales, w_codes, w_scales, y=None):
    """bf16 [M][N] = dequant(A) * dequant(W)^T for MXFP4 A [M][K] and W [N][K]."""
    torch = _torch()
    if a_codes.dim() != 2 or w_codes.dim() != 2 or a_codes.shape[1] != w_codes.shape[1]:
        raise ValueError("a_codes [M][K/2] and w_codes [N][K/2] must share K")
    M, N, K = a_codes.shape[0], w_codes.shape[0], a_codes.shape[1] * 2
    dev = a_codes.device
    _param(a_codes, "a_codes", dev, "u8", M * (K // 2))
    _param(a_scales, "a_scales", dev, "u8", M * (K // 32))
    _param(w_codes, "w_codes", dev, "u8", N * (K // 2))
    _param(w_scales, "w_scales", dev, "u8", N * (K // 32))
    if y is None:  # rows padded to a multiple of 8 elements (16-byte aligned)
        ld = (N + 7) // 8 * 8
        y = torch.empty((M, ld), dtype=torch.bfloat16, device=dev)[:, :N]
    _rows_out(y, "y", dev, "bf16", M, N)
    _check("kq_w4a4_gemm", kq_w4a4_gemm(
        a_codes.data_ptr(), a_scales.data_ptr(), w_codes.data_ptr(), w_scales.data_ptr(),
        M, N, K, y.data_ptr(), y.stride(0), _stream(a_codes)))
    return y


def _rps(tokens: int, rows_per_sample) -> int:
    return max(tokens, 1) if rows_per_sample is None else int(rows_per_sample)


def _modulation(x, shift, scale, tokens: int, d: int, rows_per_sample) -> None:
    rps = _rps(tokens, rows_per_sample)
    samples = -(-tokens // rps) if rps > 0 else 0
    _param(shift, "shift", x.device, "f32", samples * d)
    _param(scale, "scale", x.device, "f32", samples * d)


def adaln_transform_quant(x, shift, scale, lu, rows_per_sample=None, eps: float = 1e-6,
                          d: int | None = None, codes=None, scales=None):
    """MXFP4 of (LN(x) * (1 + scale_s) + shift_s) * T per 32-channel block, one
    pass; shift/scale fp32 [samples][d] on the GPU, row t in sample
    t // rows_per_sample (default: one sample)."""
    tokens, ld = _act(x, "bf16")
    d = x.shape[1] if d is None else d
    codes, scales = _mxfp4_out(x, tokens, d, codes, scales)
    _modulation(x, shift, scale, tokens, d, rows_per_sample)
    _lu(lu, x.device, d)
    _check("kq_adaln_transform_quant", kq_adaln_transform_quant(
        x.data_ptr(), tokens, d, ld, shift.data_ptr(), scale.data_ptr(),
        _rps(tokens, rows_per_sample), float(eps), lu.data_ptr(), codes.data_ptr(),
        scales.data_ptr(), _stream(x)))
    return codes, scales


def adaln_modulate(x, shift, scale, rows_per_sample=None, eps: float = 1e-6,
                   d: int | None = None, h=None):
    """bf16 LN(x) * (1 + scale_s) + shift_s."""
    torch = _torch()
    tokens, ld = _act(x, "bf16")
    d = x.shape[1] if d is None else d
    _modulation(x, shift, scale, tokens, d, rows_per_sample)
    if h is None:
        h = torch.empty((tokens, (d + 7) // 8 * 8), dtype=torch.bfloat16, device=x.device)[:, :d]
    _rows_out(h, "h", x.device, "bf16", tokens, d)
    _check("kq_adaln_modulate", kq_adaln_modulate(
        x.data_ptr(), tokens, d, ld, shift.data_ptr(), scale.data_ptr(),
        _rps(tokens, rows_per_sample), float(eps), h.data_ptr(), h.stride(0), _stream(x)))
    return h


def calib_objective(x, lu, gram=None, d: int | None = None, f=None):
    """fp32 [d/32] per-block MXFP4 round-trip objective of parameters ``lu``."""
    torch = _torch()
    tokens, ld = _act(x, "bf16")
    d = x.shape[1] if d is None else d
    if f is None:
        f = torch.empty(d // 32, dtype=torch.float32, device=x.device)
    _param(f, "f", x.device, "f32", d // 32)
    _lu(lu, x.device, d)
    if gram is not None:
        _param(gram, "gram", x.device, "f32", (d // 32) * 1024)
    _check("kq_calib_objective", kq_calib_objective(
        x.data_ptr(), tokens, d, ld, lu.data_ptr(), gram.data_ptr() if gram is not None else None,
        f.data_ptr(), _stream(x)))
    return f


def calibrate(x, lu0, noise, gram=None, sigma0: float = 0.05):
    """Per-block (1+1)-ES calibration of the block parameters on the tokens of
    ``x`` (bf16 GPU [tokens][d]), starting from ``lu0`` (fp32 [d/32][5][3]).

    ``noise`` is a float32 GPU tensor [iterations + 1][d/32][15] of standard
    normal draws (the first proposes the first candidate).  Each iteration is
    one fused launch (objective of the candidates, then the update), all of
    them queued by one kq_calib_es_run call.  Returns (theta [d/32][5][3], fbest [d/32],
    history [iterations + 1][d/32])."""
    torch = _torch()
    tokens, ld = _act(x, "bf16")
    nb = lu0.shape[0]
    if x.shape[1] != nb * 32:
        raise ValueError(f"x has {x.shape[1]} channels, lu0 holds {nb} blocks of 32")
    _param(lu0, "lu0", x.device, "f32", nb * 15)
    if noise.dim() != 3 or noise.shape[1] != nb or noise.shape[2] != 15 or noise.shape[0] < 1:
        raise ValueError("noise must be [iterations + 1][d/32][15]")
    _param(noise, "noise", x.device, "f32", noise.numel())
    if gram is not None:
        _param(gram, "gram", x.device, "f32", nb * 1024)
    iters = noise.shape[0] - 1
    theta = lu0.reshape(nb, 15).clone().contiguous()
    cand = theta.clone()
    sigma = torch.full((nb,), sigma0, dtype=torch.float32, device=x.device)
    fbest = calib_objective(x, theta, gram)
    history = torch.empty((iters + 1, nb), dtype=torch.float32, device=x.device)
    history[0].copy_(fbest)
    fcand = torch.full((nb,), float("inf"), dtype=torch.float32, device=x.device)
    st = _stream(x)
    _check("kq_calib_es_update", kq_calib_es_update(
        nb, theta.data_ptr(), sigma.data_ptr(), fbest.data_ptr(), cand.data_ptr(),
        fcand.data_ptr(), noise[0].data_ptr(), st))
    if iters:
        _check("kq_calib_es_run", kq_calib_es_run(
            x.data_ptr(), tokens, nb * 32, ld, gram.data_ptr() if gram is not None else None,
            theta.data_ptr(), sigma.data_ptr(), fbest.data_ptr(), cand.data_ptr(),
            noise[1].data_ptr(), iters, history[1].data_ptr(), st))
    return theta.reshape(nb, 5, 3), fbest, history

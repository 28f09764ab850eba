"""ctypes wrapper around the CPU oracle (``oracle/libkq_oracle.so``).

TEST INFRASTRUCTURE ONLY.  The oracle is the plain CPU reference that the GPU
library is checked against.  Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark import this module; the product package
never does.  Every function here marshals numpy arrays and calls the C code;
the arithmetic and its citations live in ``kq_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkq_oracle.so")

DENSE64 = 0
STAGED32 = 1

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_INT = ctypes.c_int

_SIGS = {
    "kqo_bf16_to_f32": (ctypes.c_float, [ctypes.c_uint16]),
    "kqo_f32_to_bf16_rne": (ctypes.c_uint16, [ctypes.c_float]),
    "kqo_e2m1_value": (ctypes.c_double, [ctypes.c_uint8]),
    "kqo_e2m1_encode": (ctypes.c_uint8, [ctypes.c_double]),
    "kqo_e8m0_from_amax": (ctypes.c_uint8, [ctypes.c_float]),
    "kqo_e8m0_value": (ctypes.c_double, [ctypes.c_uint8]),
    "kqo_mxfp4_block": (None, [_P, _P, _P]),
    "kqo_lu_factor": (None, [_P, _P]),
    "kqo_kron": (None, [_P, _INT, _INT, _P, _INT, _INT, _P]),
    "kqo_block_matrix": (None, [_P, _P]),
    "kqo_block_inverse_matrix": (None, [_P, _P]),
    "kqo_hadamard32": (None, [_P]),
    "kqo_hadamard_init_params": (None, [_P]),
    "kqo_block_transform_dense64": (None, [_P, _P, _P]),
    "kqo_block_transform_staged32": (None, [_P, _P, _P]),
    "kqo_block_inverse_dense64": (None, [_P, _P, _P]),
    "kqo_block_inverse_staged32": (None, [_P, _P, _P]),
    "kqo_transform": (_INT, [_P, _I64, _I64, _I64, _P, _INT, _P, _INT]),
    "kqo_transform_absbound": (_INT, [_P, _I64, _I64, _I64, _P, _P, _INT]),
    "kqo_transform_quant": (_INT, [_P, _I64, _I64, _I64, _P, _INT, _P, _P, _INT]),
    "kqo_mxfp4_quant": (_INT, [_P, _I64, _I64, _P, _P, _INT]),
    "kqo_smooth_quant": (_INT, [_P, _I64, _I64, _I64, _P, _P, _P, _INT]),
    "kqo_fwht32": (_INT, [_P, _I64, _I64, _I64, _INT, _P, _INT]),
    "kqo_fwht32_quant": (_INT, [_P, _I64, _I64, _I64, _INT, _P, _P, _INT]),
    "kqo_mxfp4_dequant": (_INT, [_P, _P, _I64, _I64, _P]),
    "kqo_dequant_inverse": (_INT, [_P, _P, _I64, _I64, _P, _INT, _P, _INT]),
    "kqo_matmul_nt": (_INT, [_P, _P, _I64, _I64, _I64, _P, _INT]),
    "kqo_block_weight_dense64": (None, [_P, _P, _P]),
    "kqo_block_weight_staged32": (None, [_P, _P, _P]),
    "kqo_weight_transform": (_INT, [_P, _I64, _I64, _I64, _P, _INT, _P, _INT]),
    "kqo_weight_quant": (_INT, [_P, _I64, _I64, _I64, _P, _INT, _P, _P, _INT]),
    "kqo_adaln_modulate": (_INT, [_P, _I64, _I64, _I64, _P, _P, _I64, ctypes.c_float, _INT,
                                  _P, _P, _P, _INT]),
    "kqo_adaln_transform_quant": (_INT, [_P, _I64, _I64, _I64, _P, _P, _I64, ctypes.c_float,
                                         _P, _INT, _P, _P, _INT]),
    "kqo_adaln_bound": (_INT, [_P, _I64, _I64, _I64, _P, _P, _I64, ctypes.c_float, _P, _P,
                               _INT]),
    "kqo_calib_objective": (_INT, [_P, _I64, _I64, _I64, _P, _P, _P, _INT]),
    "kqo_calib_es_update": (None, [_I64, _P, _P, _P, _P, _P, _P]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load the oracle library (built by ``make -C oracle``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"oracle library not built: {LIB_PATH} (run make -C oracle)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def default_threads() -> int:
    return max(1, len(os.sched_getaffinity(0)))


def _check(rc: int, name: str) -> None:
    if rc != 0:
        raise ValueError(f"{name}: bad arguments")


# ---- scalar formats -------------------------------------------------------
def bf16_to_f32(bits: int) -> float:
    return lib().kqo_bf16_to_f32(bits)


def f32_to_bf16(f: float) -> int:
    return lib().kqo_f32_to_bf16_rne(f)


def e2m1_value(code: int) -> float:
    return lib().kqo_e2m1_value(code)


def e2m1_encode(q: float) -> int:
    return lib().kqo_e2m1_encode(q)


def e8m0_from_amax(amax: float) -> int:
    return lib().kqo_e8m0_from_amax(amax)


def e8m0_value(byte: int) -> float:
    return lib().kqo_e8m0_value(byte)


def mxfp4_block(y: np.ndarray):
    y = np.ascontiguousarray(y, dtype=np.float32)
    assert y.shape == (32,)
    codes = np.zeros(16, np.uint8)
    scale = np.zeros(1, np.uint8)
    lib().kqo_mxfp4_block(_ptr(y), _ptr(codes), _ptr(scale))
    return codes, int(scale[0])


# ---- block-level transform -------------------------------------------------
def _params15(p) -> np.ndarray:
    p = np.ascontiguousarray(p, dtype=np.float32).reshape(15)
    return p


def lu_factor(l: float, u: float, v: float) -> np.ndarray:
    p = np.array([l, u, v], np.float32)
    F = np.zeros(4, np.float64)
    lib().kqo_lu_factor(_ptr(p), _ptr(F))
    return F.reshape(2, 2)


def kron(A: np.ndarray, B: np.ndarray) -> np.ndarray:
    A = np.ascontiguousarray(A, np.float64)
    B = np.ascontiguousarray(B, np.float64)
    C = np.zeros((A.shape[0] * B.shape[0], A.shape[1] * B.shape[1]), np.float64)
    lib().kqo_kron(_ptr(A), A.shape[0], A.shape[1], _ptr(B), B.shape[0], B.shape[1], _ptr(C))
    return C


def block_matrix(p) -> np.ndarray:
    p = _params15(p)
    T = np.zeros(1024, np.float64)
    lib().kqo_block_matrix(_ptr(p), _ptr(T))
    return T.reshape(32, 32)


def block_inverse_matrix(p) -> np.ndarray:
    p = _params15(p)
    T = np.zeros(1024, np.float64)
    lib().kqo_block_inverse_matrix(_ptr(p), _ptr(T))
    return T.reshape(32, 32)


def hadamard32() -> np.ndarray:
    H = np.zeros(1024, np.float64)
    lib().kqo_hadamard32(_ptr(H))
    return H.reshape(32, 32)


def hadamard_init_params() -> np.ndarray:
    p = np.zeros(15, np.float32)
    lib().kqo_hadamard_init_params(_ptr(p))
    return p.reshape(5, 3)


def _block_call(fn, x, p) -> np.ndarray:
    x = np.ascontiguousarray(x, np.float32).reshape(32)
    p = _params15(p)
    y = np.zeros(32, np.float32)
    fn(_ptr(x), _ptr(p), _ptr(y))
    return y


def block_transform(x, p, mode: int = DENSE64) -> np.ndarray:
    L = lib()
    fn = L.kqo_block_transform_dense64 if mode == DENSE64 else L.kqo_block_transform_staged32
    return _block_call(fn, x, p)


def block_inverse(y, p, mode: int = DENSE64) -> np.ndarray:
    L = lib()
    fn = L.kqo_block_inverse_dense64 if mode == DENSE64 else L.kqo_block_inverse_staged32
    return _block_call(fn, y, p)


# ---- tensor level ----------------------------------------------------------
def _x_args(x_bits: np.ndarray, d: int | None):
    assert x_bits.dtype == np.uint16 and x_bits.ndim == 2
    x_bits = np.ascontiguousarray(x_bits)
    tokens, ld = x_bits.shape
    d = ld if d is None else d
    return x_bits, tokens, d, ld


def _lu_arg(lu: np.ndarray, d: int) -> np.ndarray:
    lu = np.ascontiguousarray(lu, np.float32)
    assert lu.size == (d // 32) * 15, "lu must hold 15 params per 32-channel block"
    return lu


def transform(x_bits, lu, mode=DENSE64, d=None, threads=None) -> np.ndarray:
    x_bits, tokens, d, ld = _x_args(x_bits, d)
    lu = _lu_arg(lu, d)
    y = np.zeros((tokens, d), np.float32)
    rc = lib().kqo_transform(_ptr(x_bits), tokens, d, ld, _ptr(lu), mode, _ptr(y),
                             threads or default_threads())
    _check(rc, "kqo_transform")
    return y


def transform_absbound(x_bits, lu, d=None, threads=None) -> np.ndarray:
    x_bits, tokens, d, ld = _x_args(x_bits, d)
    lu = _lu_arg(lu, d)
    b = np.zeros((tokens, d), np.float64)
    rc = lib().kqo_transform_absbound(_ptr(x_bits), tokens, d, ld, _ptr(lu), _ptr(b),
                                      threads or default_threads())
    _check(rc, "kqo_transform_absbound")
    return b


def transform_quant(x_bits, lu, mode=STAGED32, d=None, threads=None):
    x_bits, tokens, d, ld = _x_args(x_bits, d)
    lu = _lu_arg(lu, d)
    codes = np.zeros((tokens, d // 2), np.uint8)
    scales = np.zeros((tokens, d // 32), np.uint8)
    rc = lib().kqo_transform_quant(_ptr(x_bits), tokens, d, ld, _ptr(lu), mode,
                                   _ptr(codes), _ptr(scales), threads or default_threads())
    _check(rc, "kqo_transform_quant")
    return codes, scales


def mxfp4_quant(y: np.ndarray, threads=None):
    y = np.ascontiguousarray(y, np.float32)
    tokens, d = y.shape
    codes = np.zeros((tokens, d // 2), np.uint8)
    scales = np.zeros((tokens, d // 32), np.uint8)
    rc = lib().kqo_mxfp4_quant(_ptr(y), tokens, d, _ptr(codes), _ptr(scales),
                               threads or default_threads())
    _check(rc, "kqo_mxfp4_quant")
    return codes, scales


def smooth_quant(x_bits, mult, d=None, threads=None):
    x_bits, tokens, d, ld = _x_args(x_bits, d)
    mult = np.ascontiguousarray(mult, np.float32).reshape(d)
    codes = np.zeros((tokens, d // 2), np.uint8)
    scales = np.zeros((tokens, d // 32), np.uint8)
    rc = lib().kqo_smooth_quant(_ptr(x_bits), tokens, d, ld, _ptr(mult), _ptr(codes),
                                _ptr(scales), threads or default_threads())
    _check(rc, "kqo_smooth_quant")
    return codes, scales


def fwht32(x_bits, mode=DENSE64, d=None, threads=None) -> np.ndarray:
    x_bits, tokens, d, ld = _x_args(x_bits, d)
    y = np.zeros((tokens, d), np.float32)
    rc = lib().kqo_fwht32(_ptr(x_bits), tokens, d, ld, mode, _ptr(y),
                          threads or default_threads())
    _check(rc, "kqo_fwht32")
    return y


def fwht32_quant(x_bits, mode=STAGED32, d=None, threads=None):
    x_bits, tokens, d, ld = _x_args(x_bits, d)
    codes = np.zeros((tokens, d // 2), np.uint8)
    scales = np.zeros((tokens, d // 32), np.uint8)
    rc = lib().kqo_fwht32_quant(_ptr(x_bits), tokens, d, ld, mode, _ptr(codes),
                                _ptr(scales), threads or default_threads())
    _check(rc, "kqo_fwht32_quant")
    return codes, scales


def mxfp4_dequant(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    tokens, half = codes.shape
    d = half * 2
    x = np.zeros((tokens, d), np.float32)
    rc = lib().kqo_mxfp4_dequant(_ptr(codes), _ptr(scales), tokens, d, _ptr(x))
    _check(rc, "kqo_mxfp4_dequant")
    return x


def dequant_inverse(codes, scales, lu, mode=STAGED32, threads=None) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    tokens, half = codes.shape
    d = half * 2
    lu = _lu_arg(lu, d)
    out = np.zeros((tokens, d), np.uint16)
    rc = lib().kqo_dequant_inverse(_ptr(codes), _ptr(scales), tokens, d, _ptr(lu), mode,
                                   _ptr(out), threads or default_threads())
    _check(rc, "kqo_dequant_inverse")
    return out


def matmul_nt(A: np.ndarray, W: np.ndarray, threads=None) -> np.ndarray:
    A = np.ascontiguousarray(A, np.float32)
    W = np.ascontiguousarray(W, np.float32)
    M, K = A.shape
    N, K2 = W.shape
    assert K == K2
    Y = np.zeros((M, N), np.float64)
    rc = lib().kqo_matmul_nt(_ptr(A), _ptr(W), M, N, K, _ptr(Y), threads or default_threads())
    _check(rc, "kqo_matmul_nt")
    return Y


def weight_transform(w_bits, lu, mode=DENSE64, k=None, threads=None) -> np.ndarray:
    """w * T^-T per 32-channel block of every weight row (fp32 out)."""
    w_bits, rows, k, ld = _x_args(w_bits, k)
    lu = _lu_arg(lu, k)
    y = np.zeros((rows, k), np.float32)
    rc = lib().kqo_weight_transform(_ptr(w_bits), rows, k, ld, _ptr(lu), mode, _ptr(y),
                                    threads or default_threads())
    _check(rc, "kqo_weight_transform")
    return y


def weight_quant(w_bits, lu, mode=STAGED32, k=None, threads=None):
    w_bits, rows, k, ld = _x_args(w_bits, k)
    lu = _lu_arg(lu, k)
    codes = np.zeros((rows, k // 2), np.uint8)
    scales = np.zeros((rows, k // 32), np.uint8)
    rc = lib().kqo_weight_quant(_ptr(w_bits), rows, k, ld, _ptr(lu), mode, _ptr(codes),
                                _ptr(scales), threads or default_threads())
    _check(rc, "kqo_weight_quant")
    return codes, scales


# ---- AdaLN-modulated input ---------------------------------------------------
def _adaln_args(x_bits, shift, scale, rows_per_sample, d):
    x_bits, tokens, d, ld = _x_args(x_bits, d)
    rps = tokens if rows_per_sample is None else int(rows_per_sample)
    samples = max(1, -(-tokens // max(rps, 1)))
    shift = np.ascontiguousarray(shift, np.float32).reshape(-1, d)
    scale = np.ascontiguousarray(scale, np.float32).reshape(-1, d)
    assert shift.shape[0] >= samples and scale.shape[0] >= samples, "one shift/scale row per sample"
    return x_bits, tokens, d, ld, shift, scale, rps


def adaln_modulate(x_bits, shift, scale, rows_per_sample=None, eps=1e-6, mode=STAGED32,
                   d=None, threads=None):
    """h = LN(x) * (1 + scale_s) + shift_s (fp32), with each row's mean and
    1/sqrt(var + eps)."""
    x_bits, tokens, d, ld, shift, scale, rps = _adaln_args(x_bits, shift, scale,
                                                           rows_per_sample, d)
    h = np.zeros((tokens, d), np.float32)
    mean = np.zeros(tokens, np.float32)
    rstd = np.zeros(tokens, np.float32)
    rc = lib().kqo_adaln_modulate(_ptr(x_bits), tokens, d, ld, _ptr(shift), _ptr(scale), rps,
                                  float(eps), mode, _ptr(h), _ptr(mean), _ptr(rstd),
                                  threads or default_threads())
    _check(rc, "kqo_adaln_modulate")
    return h, mean, rstd


def adaln_transform_quant(x_bits, shift, scale, lu, rows_per_sample=None, eps=1e-6,
                          mode=STAGED32, d=None, threads=None):
    x_bits, tokens, d, ld, shift, scale, rps = _adaln_args(x_bits, shift, scale,
                                                           rows_per_sample, d)
    lu = _lu_arg(lu, d)
    codes = np.zeros((tokens, d // 2), np.uint8)
    scales = np.zeros((tokens, d // 32), np.uint8)
    rc = lib().kqo_adaln_transform_quant(_ptr(x_bits), tokens, d, ld, _ptr(shift), _ptr(scale),
                                         rps, float(eps), _ptr(lu), mode, _ptr(codes),
                                         _ptr(scales), threads or default_threads())
    _check(rc, "kqo_adaln_transform_quant")
    return codes, scales


def adaln_bound(x_bits, shift, scale, lu, rows_per_sample=None, eps=1e-6, d=None,
                threads=None) -> np.ndarray:
    x_bits, tokens, d, ld, shift, scale, rps = _adaln_args(x_bits, shift, scale,
                                                           rows_per_sample, d)
    lu = _lu_arg(lu, d)
    bound = np.zeros((tokens, d), np.float64)
    rc = lib().kqo_adaln_bound(_ptr(x_bits), tokens, d, ld, _ptr(shift), _ptr(scale), rps,
                               float(eps), _ptr(lu), _ptr(bound), threads or default_threads())
    _check(rc, "kqo_adaln_bound")
    return bound


# ---- calibration of the block parameters -------------------------------------
def calib_objective(x_bits, lu, gram=None, d=None, threads=None) -> np.ndarray:
    """Per-block f_j = sum_t r G_j r^T of the MXFP4 round trip (fp64 [nb])."""
    x_bits, tokens, d, ld = _x_args(x_bits, d)
    lu = _lu_arg(lu, d)
    f = np.zeros(d // 32, np.float64)
    g = None
    if gram is not None:
        g = np.ascontiguousarray(gram, np.float32)
        assert g.shape == (d // 32, 32, 32)
    rc = lib().kqo_calib_objective(_ptr(x_bits), tokens, d, ld, _ptr(lu),
                                   _ptr(g) if g is not None else None, _ptr(f),
                                   threads or default_threads())
    _check(rc, "kqo_calib_objective")
    return f


def calib_es_update(theta, sigma, fbest, cand, fcand, noise):
    """One (1+1)-ES step on float32 arrays, in place (theta, sigma, fbest, cand)."""
    nb = sigma.shape[0]
    for a in (theta, sigma, fbest, cand, fcand, noise):
        assert a.dtype == np.float32 and a.flags["C_CONTIGUOUS"]
    lib().kqo_calib_es_update(nb, _ptr(theta), _ptr(sigma), _ptr(fbest), _ptr(cand), _ptr(fcand),
                              _ptr(noise))

"""The C ABI: libkq.so loads, exports every function include/kq.h declares, and
rejects bad arguments on the host before any HIP call.

Nothing here touches a GPU: every call below fails validation (or is empty)
and returns before the library makes its first HIP runtime call; the pointers
passed are never dereferenced.
"""
import ctypes

import pytest

from mxfp4_activation_quantizer_amd import kq

A16 = 0x10000   # a 16-byte-aligned dummy address, never dereferenced
ODD = 0x10001   # misaligned dummy address


def test_library_loads_and_exports_every_declared_symbol():
    L = kq.lib()
    declared = kq.declared_functions()
    assert "kq_transform_quant" in declared and "kq_status_str" in declared
    for name in declared:
        assert hasattr(L, name), name
    # the binding knows every declared function (and nothing undeclared)
    assert set(kq.SIGNATURES) == set(declared)
    # and the shared object's dynamic symbols include them
    for name in declared:
        assert ctypes.cast(getattr(L, name), ctypes.c_void_p).value


def test_library_exports_nothing_but_the_declared_functions():
    """Only the kq.h entry points are dynamic symbols: the host handles of the
    kernels stay local, so a second build of the library in the same process
    cannot take over this one's launches."""
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-D", "--defined-only", kq.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    names = {line.split()[-1] for line in out.splitlines() if line.strip()}
    assert names == set(kq.declared_functions()), sorted(names ^ set(kq.declared_functions()))[:10]


def test_status_strings():
    assert kq.status_str(kq.KQ_OK) == "KQ_OK"
    for st in (kq.KQ_ERR_NULL, kq.KQ_ERR_SHAPE, kq.KQ_ERR_ALIGN, kq.KQ_ERR_HIP):
        assert kq.status_str(st).startswith("KQ_ERR_")
    assert "unknown" in kq.status_str(99)
    assert kq.version() >= 100


QUANT_CALLS = {
    "kq_transform_quant": lambda x, t, d, ld, c, s: kq.kq_transform_quant(x, t, d, ld, A16, c, s),
    "kq_transform_quant_mfma": lambda x, t, d, ld, c, s: kq.kq_transform_quant_mfma(
        x, t, d, ld, A16, c, s),
    "kq_transform_quant_quad": lambda x, t, d, ld, c, s: kq.kq_transform_quant_quad(
        x, t, d, ld, A16, c, s),
    "kq_smooth_quant": lambda x, t, d, ld, c, s: kq.kq_smooth_quant(x, t, d, ld, A16, c, s),
    "kq_weight_quant": lambda x, t, d, ld, c, s: kq.kq_weight_quant(x, t, d, ld, A16, c, s),
    "kq_fwht32_quant": lambda x, t, d, ld, c, s: kq.kq_fwht32_quant(x, t, d, ld, c, s),
    "kq_copy_ceiling": lambda x, t, d, ld, c, s: kq.kq_copy_ceiling(x, t, d, ld, c, s),
}


@pytest.mark.parametrize("name", sorted(QUANT_CALLS))
def test_shape_errors(name):
    f = QUANT_CALLS[name]
    assert f(A16, -1, 64, 64, A16, A16) == kq.KQ_ERR_SHAPE
    assert f(A16, 1 << 30, 64, 64, A16, A16) == kq.KQ_ERR_SHAPE
    assert f(A16, 4, 0, 64, A16, A16) == kq.KQ_ERR_SHAPE
    assert f(A16, 4, 48, 64, A16, A16) == kq.KQ_ERR_SHAPE      # d % 32 != 0
    assert f(A16, 4, 64, 32, A16, A16) == kq.KQ_ERR_SHAPE      # ld < d


@pytest.mark.parametrize("name", sorted(QUANT_CALLS))
def test_empty_is_ok_without_pointers(name):
    assert QUANT_CALLS[name](None, 0, 64, 64, None, None) == kq.KQ_OK


@pytest.mark.parametrize("name", sorted(QUANT_CALLS))
def test_null_and_alignment_errors(name):
    f = QUANT_CALLS[name]
    assert f(None, 4, 64, 64, A16, A16) == kq.KQ_ERR_NULL
    assert f(A16, 4, 64, 64, None, A16) == kq.KQ_ERR_NULL
    assert f(A16, 4, 64, 64, A16, None) == kq.KQ_ERR_NULL
    assert f(ODD, 4, 64, 64, A16, A16) == kq.KQ_ERR_ALIGN
    assert f(A16, 4, 64, 68, A16, A16) == kq.KQ_ERR_ALIGN      # row stride 136 B
    assert f(A16, 4, 64, 64, ODD, A16) == kq.KQ_ERR_ALIGN


def test_parameter_pointer_checks():
    assert kq.kq_transform_quant(A16, 4, 64, 64, None, A16, A16) == kq.KQ_ERR_NULL
    assert kq.kq_transform_quant(A16, 4, 64, 64, ODD, A16, A16) == kq.KQ_ERR_ALIGN
    assert kq.kq_transform_quant_mfma(A16, 4, 64, 64, None, A16, A16) == kq.KQ_ERR_NULL
    assert kq.kq_transform_quant_mfma(A16, 4, 64, 64, ODD, A16, A16) == kq.KQ_ERR_ALIGN
    assert kq.kq_transform_quant_quad(A16, 4, 64, 64, None, A16, A16) == kq.KQ_ERR_NULL
    assert kq.kq_transform_quant_quad(A16, 4, 64, 64, ODD, A16, A16) == kq.KQ_ERR_ALIGN
    # unit indices of the quad-lane kernel are 32-bit
    assert kq.kq_transform_quant_quad(A16, 1 << 25, 2048, 2048, A16, A16, A16) == kq.KQ_ERR_SHAPE
    sc = kq.kq_stream_ceiling
    assert sc(None, 0, None, None) == kq.KQ_OK
    assert sc(A16, -1, A16, A16) == kq.KQ_ERR_SHAPE
    assert sc(A16, (1 << 36) + 1, A16, A16) == kq.KQ_ERR_SHAPE
    assert sc(None, 4, A16, A16) == kq.KQ_ERR_NULL
    assert sc(A16, 4, None, None) == kq.KQ_ERR_NULL       # read-only still needs scales
    assert sc(ODD, 4, A16, A16) == kq.KQ_ERR_ALIGN
    assert sc(A16, 4, A16 + 8, A16) == kq.KQ_ERR_ALIGN
    assert kq.kq_smooth_quant(A16, 4, 64, 64, None, A16, A16) == kq.KQ_ERR_NULL
    assert kq.kq_smooth_quant(A16, 4, 64, 64, A16 + 4, A16, A16) == kq.KQ_ERR_ALIGN
    assert kq.kq_transform_f32(A16, 4, 64, 64, A16, None) == kq.KQ_ERR_NULL
    assert kq.kq_transform_f32(A16, 4, 64, 64, A16, A16 + 8) == kq.KQ_ERR_ALIGN
    assert kq.kq_transform_f32(None, 0, 64, 64, None, None) == kq.KQ_OK
    assert kq.kq_mxfp4_quant_f32(A16, 4, 64, 66, A16, A16) == kq.KQ_ERR_ALIGN
    assert kq.kq_mxfp4_quant_f32(A16, 4, 64, 60, A16, A16) == kq.KQ_ERR_SHAPE
    assert kq.kq_mxfp4_quant_f32(None, 4, 64, 64, A16, A16) == kq.KQ_ERR_NULL
    assert kq.kq_mxfp4_quant_f32(None, 0, 64, 64, None, None) == kq.KQ_OK
    di = kq.kq_dequant_inverse
    assert di(None, None, 0, 64, None, None, 64) == kq.KQ_OK
    assert di(A16, A16, 4, 48, A16, A16, 64) == kq.KQ_ERR_SHAPE
    assert di(A16, A16, 4, 64, A16, A16, 32) == kq.KQ_ERR_SHAPE
    assert di(A16, None, 4, 64, A16, A16, 64) == kq.KQ_ERR_NULL
    assert di(A16, A16, 4, 64, None, A16, 64) == kq.KQ_ERR_NULL
    assert di(ODD, A16, 4, 64, A16, A16, 64) == kq.KQ_ERR_ALIGN
    assert di(A16, A16, 4, 64, A16, ODD, 64) == kq.KQ_ERR_ALIGN
    assert di(A16, A16, 4, 64, A16, A16, 68) == kq.KQ_ERR_ALIGN
    g = kq.kq_w4a4_gemm
    assert g(None, None, None, None, 0, 16, 128, None, 16) == kq.KQ_OK
    assert g(A16, A16, A16, A16, 8, 16, 96, A16, 16) == kq.KQ_ERR_SHAPE     # K % 128
    assert g(A16, A16, A16, A16, 8, 16, 128, A16, 8) == kq.KQ_ERR_SHAPE     # ld_y < N
    assert g(A16, A16, None, A16, 8, 16, 128, A16, 16) == kq.KQ_ERR_NULL
    assert g(A16, A16 + 2, A16, A16, 8, 16, 128, A16, 16) == kq.KQ_ERR_ALIGN
    assert g(A16, A16, A16, A16, 8, 16, 128, A16 + 2, 16) == kq.KQ_ERR_ALIGN
    assert g(A16, A16, A16, A16, 1 << 20, 16, 4096, A16, 16) == kq.KQ_ERR_SHAPE  # 2 GiB operand


def test_adaln_argument_checks():
    q = kq.kq_adaln_transform_quant
    m = kq.kq_adaln_modulate
    ok = (A16, 4, 64, 64, A16, A16, 4, 1e-6)
    assert q(None, 0, 64, 64, None, None, 1, 1e-6, None, None, None) == kq.KQ_OK
    assert m(None, 0, 64, 64, None, None, 1, 1e-6, None, 64) == kq.KQ_OK
    assert q(A16, 4, 48, 64, A16, A16, 4, 1e-6, A16, A16, A16) == kq.KQ_ERR_SHAPE    # d % 32
    assert q(A16, 4, 8224, 8224, A16, A16, 4, 1e-6, A16, A16, A16) == kq.KQ_ERR_SHAPE  # d > 8192
    assert q(A16, 4, 64, 32, A16, A16, 4, 1e-6, A16, A16, A16) == kq.KQ_ERR_SHAPE    # ld < d
    assert q(A16, 4, 64, 64, A16, A16, 0, 1e-6, A16, A16, A16) == kq.KQ_ERR_SHAPE    # rows/sample
    assert q(A16, 4, 64, 64, A16, A16, 4, -1.0, A16, A16, A16) == kq.KQ_ERR_SHAPE    # eps < 0
    assert q(A16, 4, 64, 64, A16, A16, 4, float("nan"), A16, A16, A16) == kq.KQ_ERR_SHAPE
    assert q(A16, 4, 64, 64, A16, A16, 4, float("inf"), A16, A16, A16) == kq.KQ_ERR_SHAPE
    assert q(None, 4, 64, 64, A16, A16, 4, 1e-6, A16, A16, A16) == kq.KQ_ERR_NULL
    assert q(A16, 4, 64, 64, None, A16, 4, 1e-6, A16, A16, A16) == kq.KQ_ERR_NULL
    assert q(A16, 4, 64, 64, A16, None, 4, 1e-6, A16, A16, A16) == kq.KQ_ERR_NULL
    assert q(*ok, None, A16, A16) == kq.KQ_ERR_NULL
    assert q(*ok, A16, None, A16) == kq.KQ_ERR_NULL
    assert q(*ok, A16, A16, None) == kq.KQ_ERR_NULL
    assert q(ODD, 4, 64, 64, A16, A16, 4, 1e-6, A16, A16, A16) == kq.KQ_ERR_ALIGN
    assert q(A16, 4, 64, 68, A16, A16, 4, 1e-6, A16, A16, A16) == kq.KQ_ERR_ALIGN
    assert q(A16, 4, 64, 64, A16 + 4, A16, 4, 1e-6, A16, A16, A16) == kq.KQ_ERR_ALIGN
    assert q(A16, 4, 64, 64, A16, A16 + 8, 4, 1e-6, A16, A16, A16) == kq.KQ_ERR_ALIGN
    assert q(*ok, ODD, A16, A16) == kq.KQ_ERR_ALIGN
    assert q(*ok, A16, A16 + 8, A16) == kq.KQ_ERR_ALIGN
    assert m(*ok, None, 64) == kq.KQ_ERR_NULL
    assert m(*ok, A16, 32) == kq.KQ_ERR_SHAPE
    assert m(*ok, A16 + 2, 64) == kq.KQ_ERR_ALIGN
    assert m(*ok, A16, 68) == kq.KQ_ERR_ALIGN


def test_calibration_argument_checks():
    o = kq.kq_calib_objective
    assert o(A16, 4, 48, 64, A16, None, A16) == kq.KQ_ERR_SHAPE      # d % 32
    assert o(A16, 4, 64, 32, A16, None, A16) == kq.KQ_ERR_SHAPE      # ld < d
    assert o(A16, -1, 64, 64, A16, None, A16) == kq.KQ_ERR_SHAPE
    assert o(None, 4, 64, 64, A16, None, A16) == kq.KQ_ERR_NULL
    assert o(A16, 4, 64, 64, None, None, A16) == kq.KQ_ERR_NULL
    assert o(A16, 4, 64, 64, A16, None, None) == kq.KQ_ERR_NULL
    assert o(ODD, 4, 64, 64, A16, None, A16) == kq.KQ_ERR_ALIGN
    assert o(A16, 4, 64, 68, A16, None, A16) == kq.KQ_ERR_ALIGN
    assert o(A16, 4, 64, 64, A16 + 2, None, A16) == kq.KQ_ERR_ALIGN
    assert o(A16, 4, 64, 64, A16, A16 + 1, A16) == kq.KQ_ERR_ALIGN
    u = kq.kq_calib_es_update
    assert u(0, None, None, None, None, None, None) == kq.KQ_OK
    assert u(-1, A16, A16, A16, A16, A16, A16) == kq.KQ_ERR_SHAPE
    assert u(4, None, A16, A16, A16, A16, A16) == kq.KQ_ERR_NULL
    assert u(4, A16, A16, A16, A16, A16, None) == kq.KQ_ERR_NULL
    assert u(4, A16, A16 + 2, A16, A16, A16, A16) == kq.KQ_ERR_ALIGN
    e = kq.kq_calib_es_step
    assert e(A16, 4, 48, 64, None, A16, A16, A16, A16, A16, None) == kq.KQ_ERR_SHAPE   # d % 32
    assert e(A16, 4, 64, 32, None, A16, A16, A16, A16, A16, None) == kq.KQ_ERR_SHAPE   # ld < d
    assert e(A16, -1, 64, 64, None, A16, A16, A16, A16, A16, None) == kq.KQ_ERR_SHAPE
    assert e(None, 4, 64, 64, None, A16, A16, A16, A16, A16, None) == kq.KQ_ERR_NULL
    assert e(A16, 4, 64, 64, None, None, A16, A16, A16, A16, None) == kq.KQ_ERR_NULL
    assert e(A16, 4, 64, 64, None, A16, A16, A16, A16, None, None) == kq.KQ_ERR_NULL
    assert e(ODD, 4, 64, 64, None, A16, A16, A16, A16, A16, None) == kq.KQ_ERR_ALIGN
    assert e(A16, 4, 64, 64, A16 + 1, A16, A16, A16, A16, A16, None) == kq.KQ_ERR_ALIGN
    assert e(A16, 4, 64, 64, None, A16, A16, A16, A16, A16, A16 + 2) == kq.KQ_ERR_ALIGN
    r = kq.kq_calib_es_run
    assert r(A16, 4, 64, 64, None, A16, A16, A16, A16, A16, -1, None) == kq.KQ_ERR_SHAPE
    assert r(A16, 4, 64, 64, None, A16, A16, A16, A16, A16, 1 << 25, None) == kq.KQ_ERR_SHAPE
    assert r(A16, 4, 64, 64, None, None, None, None, None, None, 0, None) == kq.KQ_OK
    assert r(A16, 4, 64, 64, None, A16, A16, A16, None, A16, 3, None) == kq.KQ_ERR_NULL
    assert r(A16, 4, 64, 64, None, A16, A16, A16, A16, A16 + 1, 3, None) == kq.KQ_ERR_ALIGN


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros((4, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        kq.transform_quant(x, torch.zeros(30))

"""Helpers for comparing GPU outputs with the CPU oracle (not a test module)."""
from __future__ import annotations

import numpy as np

import oracle
from mxfp4_activation_quantizer_amd import inputs

# Midpoints of the E2M1 magnitude grid 0, .5, 1, 1.5, 2, 3, 4, 6.
E2M1_MIDPOINTS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
E2M1_MAG = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])

# Tolerances fixed by the quantizer's correctness bar.
REL_Y = 1e-5           # transformed fp32 values vs the fp64 definition
MAX_CODE_FRAC = 1e-4   # fraction of codes that may differ from the definition
REL_GEMM = 2e-3        # W4A4 output vs the dequantised matmul, normwise
REL_GEMM_MIN_OUTPUTS = 4096


def to_gpu_bf16(bits: np.ndarray, device="cuda:0"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def to_gpu(a: np.ndarray, device="cuda:0"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def unpack_codes(codes: np.ndarray) -> np.ndarray:
    """[tokens][d/2] packed bytes -> [tokens][d] nibbles (even element low)."""
    out = np.empty((codes.shape[0], codes.shape[1] * 2), np.uint8)
    out[:, 0::2] = codes & 0xF
    out[:, 1::2] = codes >> 4
    return out


def assert_codes_within_tie_tolerance(codes_gpu, scales_gpu, codes_ref, scales_ref,
                                      y_ref, bound, rel=REL_Y, max_frac=MAX_CODE_FRAC):
    """GPU MXFP4 vs the fp64 definition's MXFP4, allowing only rounding ties.

    y_ref is the definition's transformed value (fp64 result rounded once to
    fp32) and bound the forward-error scale sum_i |x_i T_ik| (fp64).  A scale
    byte may differ only where the block amax lies within rel*max(bound) of a
    power of two; there every decoded GPU value must lie within one E2M1 grid
    step (at the GPU's scale) of y, and all 32 codes of the block count as
    differing.  In blocks whose scales agree, a code may differ only to a
    value-adjacent code (+0/-0 merged) and only where y*2^-e lies within
    rel*bound*2^-e of an E2M1 midpoint.  At most max_frac of all codes differ,
    those of scale-mismatched blocks included.
    Returns (scale mismatches, code mismatches)."""
    tokens, d = y_ref.shape
    nb = d // 32
    yb = np.abs(y_ref.astype(np.float64)).reshape(tokens, nb, 32)
    amax = yb.max(axis=2)
    bmax = bound.reshape(tokens, nb, 32).max(axis=2)
    smis = scales_gpu != scales_ref
    if smis.any():
        a = amax[smis]
        p2 = 2.0 ** np.round(np.log2(np.maximum(a, 1e-300)))
        assert np.all(np.abs(a - p2) <= rel * bmax[smis] + 1e-300), \
            "a scale byte differs away from a power-of-two amax"
        # decoded GPU values of those blocks against the definition's values
        cgm = unpack_codes(codes_gpu).reshape(tokens, nb, 32)[smis]
        eg = scales_gpu[smis].astype(np.float64)[:, None] - 127.0
        dec = E2M1_MAG[cgm & 7] * np.where(cgm & 8, -1.0, 1.0) * 2.0 ** eg
        yv = y_ref.astype(np.float64).reshape(tokens, nb, 32)[smis]
        qv = np.abs(yv) * 2.0 ** (-eg)
        step = np.where(qv < 2, 0.5, np.where(qv < 4, 1.0, 2.0)) * 2.0 ** eg
        assert np.all(np.abs(dec - yv) <= step * (1 + 1e-6)), \
            "a block with a differing scale byte decodes more than one grid step away"
    cg, cr = unpack_codes(codes_gpu), unpack_codes(codes_ref)
    same_scale = np.repeat(~smis, 32, axis=1)
    cmis = (cg != cr) & same_scale
    # +0 and -0 are the same value
    cmis &= ~(((cg & 7) == 0) & ((cr & 7) == 0))
    n = int(cmis.sum())
    if n:
        g, r = cg[cmis].astype(int), cr[cmis].astype(int)
        sg = np.where(g & 7, g >> 3, -1)
        sr = np.where(r & 7, r >> 3, -1)
        adjacent = (np.abs((g & 7) - (r & 7)) == 1) & ((sg == sr) | (sg < 0) | (sr < 0))
        assert np.all(adjacent), "a code differs by more than one grid step"
        e = np.repeat(scales_ref.astype(np.int64) - 127, 32, axis=1)[cmis]
        q = np.abs(y_ref.astype(np.float64)[cmis]) * 2.0 ** (-e)
        tol = rel * bound[cmis] * 2.0 ** (-e)
        near = np.abs(q[:, None] - E2M1_MIDPOINTS[None, :]).min(axis=1) <= tol + 1e-300
        assert np.all(near), "a code differs away from a rounding tie"
    n_all = n + 32 * int(smis.sum())
    assert n_all <= max_frac * cg.size, \
        f"{n} codes and {int(smis.sum())} scale bytes differ (> {max_frac} of {cg.size} codes)"
    return int(smis.sum()), n


def gemm_reference(ac, as_, wc, ws):
    A = oracle.mxfp4_dequant(ac, as_)
    W = oracle.mxfp4_dequant(wc, ws)
    Y = oracle.matmul_nt(A, W)
    B = oracle.matmul_nt(np.abs(A), np.abs(W))
    return Y, B


def assert_gemm_close(y_bits, Y, B, K):
    """bf16 of an fp32-accumulated sum of exact products: within half a bf16
    step of the fp64 sum plus K * 2^-23 of sum |a||w| (fp32 accumulation).
    Half a bf16 step is up to 2^-8 of the value, so the same bound holds
    normwise; in addition at least 90 % of the outputs must equal the bf16
    rounding (nearest even) of the fp64 sum itself."""
    y = inputs.bf16_bits_to_f32(y_bits).astype(np.float64)
    err = np.abs(y - Y)
    tol = 2.0 ** -8 * np.abs(Y) + K * 2.0 ** -23 * B + 1e-30
    assert np.all(err <= tol), f"{int((err > tol).sum())} outputs off"
    assert np.linalg.norm(y - Y) <= 2.0 ** -8 * np.linalg.norm(Y) + K * 2.0 ** -23 * np.linalg.norm(B)
    # the consumer's stated bar: relative 2e-3 normwise against the oracle's
    # dequantised matmul.  The bf16 output rounding alone has a normwise size
    # of about 1.5-1.7e-3 of ||Y|| once there are many outputs (each element's
    # relative rounding error is uniform within +-2^-8 of its binade), but
    # over a few dozen outputs its realised value scatters above 2e-3, so the
    # bar applies from REL_GEMM_MIN_OUTPUTS outputs on (the elementwise bar
    # above, 2^-8 per element, holds everywhere).
    ny = np.linalg.norm(Y)
    if Y.size >= REL_GEMM_MIN_OUTPUTS:
        assert np.linalg.norm(y - Y) <= REL_GEMM * ny + 1e-30, \
            f"normwise error {np.linalg.norm(y - Y) / max(ny, 1e-300):.3e} > {REL_GEMM}"
    exact = np.mean(np.asarray(y_bits, np.uint16) == inputs.f64_to_bf16_bits(Y))
    assert exact >= 0.9, f"only {exact:.3f} of the outputs are the rounded fp64 sum"

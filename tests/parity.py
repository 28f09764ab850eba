"""Helpers for comparing GPU outputs with the CPU oracle (not a test module)."""
from __future__ import annotations

import numpy as np

# Midpoints of the E2M1 magnitude grid 0, .5, 1, 1.5, 2, 3, 4, 6.
E2M1_MIDPOINTS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
E2M1_MAG = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])

# Tolerances fixed by the quantizer's correctness bar.
REL_Y = 1e-5           # transformed fp32 values vs the fp64 definition
MAX_CODE_FRAC = 1e-4   # fraction of codes that may differ from the definition


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
    power of two.  In blocks whose scales agree, a code may differ only to a
    value-adjacent code (+0/-0 merged) and only where y*2^-e lies within
    rel*bound*2^-e of an E2M1 midpoint; at most max_frac of all codes differ.
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
    assert n <= max_frac * cg.size, f"{n} codes differ (> {max_frac} of {cg.size})"
    return int(smis.sum()), n

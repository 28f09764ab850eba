"""Seeded synthetic inputs for the quantizer's workloads.

This module only draws data: activations shaped like diffusion-transformer
linear-layer inputs, per-block transform parameters, per-channel multipliers
for the scaling baseline and weights for the W4A4 consumer.  It holds none of
the quantizer's arithmetic, and both the GPU tests and the CPU oracle take
their inputs from it.

The models and prompt sets the KroQuant pages evaluate on (PixArt-Sigma,
FLUX.1-schnell; MJHQ-30K, SDCI, COCO captions) are not available, so each
workload is a seeded stand-in with the shape and value structure of the
activation it imitates.  Every draw uses
``numpy.random.default_rng(SeedSequence([0, workload_id, tensor_id]))``;
values are made in float64, then rounded to nearest-even bfloat16.

All activations are returned as ``uint16`` arrays holding bfloat16 bit
patterns, row-major ``[tokens][channels]``.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

# Hadamard starting point of one 2x2 factor, (l, u, v) = (1, 1/sqrt2, -1/sqrt2):
# the unit-determinant factor H2 * diag(1, -1) (KroQuant summary, "Approach":
# factors are initialised at the Hadamard).
HADAMARD_INIT_LUV = (1.0, 1.0 / np.sqrt(2.0), -1.0 / np.sqrt(2.0))

# |u| below this is redrawn so that 1/u stays moderate.
U_MIN = 0.1


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int            # workload id, the second seed word
    tokens: int
    d: int
    param_sigma: float  # std-dev of the noise added to the Hadamard start
    description: str

    @property
    def blocks(self) -> int:
        return self.d // 32

    @property
    def elements(self) -> int:
        return self.tokens * self.d

    @property
    def algorithmic_bytes(self) -> int:
        """bf16 read (2 B) + E2M1 codes (0.5 B) + one E8M0 byte per 32."""
        return self.elements * 2 + self.elements // 2 + self.elements // 32


WORKLOADS = {
    "tiny": Workload("tiny", 0, 64, 256, 0.05,
                     "N(0,1), channels 7 and 100 scaled x30"),
    "pixart": Workload("pixart", 1, 2 * 4096, 1152, 0.1,
                       "Student-t(4) x per-token lognormal(0,0.5), 1% channels x50"),
    "flux_attn": Workload("flux_attn", 2, 4608, 3072, 0.1,
                          "AdaLN-modulated N(0,1) rows, 0.5% channels x100"),
    "flux_mlp": Workload("flux_mlp", 3, 4608, 12288, 0.1,
                         "GELU(N(0,1)), 0.2% channels x80"),
}

# Shape of the W4A4 consumer: activation 4608 x 3072 times weights 12288 x 3072.
GEMM_M, GEMM_N, GEMM_K = 4608, 12288, 3072
GEMM_WID = 4


def rng(wid: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([0, wid, tensor_id]))


def f64_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float64 data to bfloat16 (via float32, nearest-even), as bits."""
    f = np.ascontiguousarray(a, dtype=np.float32)
    b = f.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    out = b.astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _outlier_channels(g: np.random.Generator, d: int, frac: float) -> np.ndarray:
    k = max(1, int(round(frac * d)))
    return g.choice(d, size=k, replace=False)


def activation(name: str) -> np.ndarray:
    """Seeded bf16 activation of workload ``name`` as uint16 bits [tokens][d]."""
    w = WORKLOADS[name]
    g = rng(w.wid, 0)
    T, d = w.tokens, w.d
    if name == "tiny":
        x = g.standard_normal((T, d))
        x[:, [7, 100]] *= 30.0
    elif name == "pixart":
        x = g.standard_t(4.0, size=(T, d)) * g.lognormal(0.0, 0.5, size=(T, 1))
        x[:, _outlier_channels(g, d, 0.01)] *= 50.0
    elif name == "flux_attn":
        z = g.standard_normal((T, d))
        z = (z - z.mean(axis=1, keepdims=True)) / np.sqrt(z.var(axis=1, keepdims=True) + 1e-6)
        s = g.normal(0.0, 0.3, size=(T, 1))
        h = g.normal(0.0, 0.3, size=(T, 1))
        x = z * (1.0 + s) + h
        x[:, _outlier_channels(g, d, 0.005)] *= 100.0
    elif name == "flux_mlp":
        from scipy.special import erf
        z = g.standard_normal((T, d))
        x = 0.5 * z * (1.0 + erf(z / np.sqrt(2.0)))
        x[:, _outlier_channels(g, d, 0.002)] *= 80.0
    else:  # pragma: no cover - WORKLOADS lookup above already failed
        raise KeyError(name)
    return f64_to_bf16_bits(x)


def hadamard_init(blocks: int) -> np.ndarray:
    """Hadamard start for ``blocks`` blocks: float32 [blocks][5][3]."""
    p = np.empty((blocks, 5, 3), np.float32)
    p[:, :, 0], p[:, :, 1], p[:, :, 2] = HADAMARD_INIT_LUV
    return p


def lu_params(name: str, blocks: int | None = None, sigma: float | None = None) -> np.ndarray:
    """Independent per-block (l, u, v) x 5 = Hadamard start + N(0, sigma) noise.

    Returns float32 [blocks][5][3].  Any |u| < U_MIN is redrawn.
    """
    w = WORKLOADS[name]
    blocks = w.blocks if blocks is None else blocks
    sigma = w.param_sigma if sigma is None else sigma
    g = rng(w.wid, 1)
    p = hadamard_init(blocks).astype(np.float64)
    p += g.normal(0.0, sigma, size=p.shape)
    bad = np.abs(p[:, :, 1]) < U_MIN
    while bad.any():
        p[:, :, 1][bad] = HADAMARD_INIT_LUV[1] + g.normal(0.0, sigma, size=int(bad.sum()))
        bad = np.abs(p[:, :, 1]) < U_MIN
    return p.astype(np.float32)


def smooth_multipliers(x_bits: np.ndarray, alpha: float = 0.5, floor: float = 1e-5) -> np.ndarray:
    """Per-channel multipliers for the scaling baseline: max_t|X[t,c]|^-alpha.

    The migration strength 0.5 is the one LRQ-DiT uses for its SmoothQuant
    baseline (Sec. 5.1); with no weight statistics the weight term is 1.
    Float32 [d].
    """
    a = np.abs(bf16_bits_to_f32(x_bits).astype(np.float64)).max(axis=0)
    return (np.maximum(a, floor) ** (-alpha)).astype(np.float32)


def residual(name: str, tokens: int | None = None, d: int | None = None) -> np.ndarray:
    """Pre-norm residual-stream rows for the AdaLN-fused quantizer, bf16 bits
    [tokens][d]: N(0,1) scaled per token by lognormal(0, 0.5) and shifted per
    token by N(0, 0.5), with 0.5 % of the channels x100 (the few very large
    channels of a transformer's residual stream).  Defaults to the workload's
    shape."""
    w = WORKLOADS[name]
    T = w.tokens if tokens is None else tokens
    d = w.d if d is None else d
    g = rng(w.wid, 2)
    x = g.standard_normal((T, d)) * g.lognormal(0.0, 0.5, size=(T, 1)) + g.normal(0.0, 0.5, (T, 1))
    x[:, _outlier_channels(g, d, 0.005)] *= 100.0
    return f64_to_bf16_bits(x)


def modulation(name: str, samples: int = 1, d: int | None = None):
    """AdaLN shift and scale vectors (the per-sample outputs of the
    conditioning projection), float32 [samples][d] each, N(0, 0.3)."""
    w = WORKLOADS[name]
    d = w.d if d is None else d
    g = rng(w.wid, 3)
    shift = g.normal(0.0, 0.3, (samples, d)).astype(np.float32)
    scale = g.normal(0.0, 0.3, (samples, d)).astype(np.float32)
    return shift, scale


def calib_noise(name: str, iterations: int, blocks: int | None = None) -> np.ndarray:
    """Standard normal draws for the calibration's evolution strategy,
    float32 [iterations + 1][blocks][15]."""
    w = WORKLOADS[name]
    blocks = w.blocks if blocks is None else blocks
    g = rng(w.wid, 4)
    return g.standard_normal((iterations + 1, blocks, 15)).astype(np.float32)


def gemm_weight() -> np.ndarray:
    """W4A4 consumer weights W [N=12288][K=3072] ~ N(0, 0.02), bf16 bits."""
    g = rng(GEMM_WID, 0)
    return f64_to_bf16_bits(g.normal(0.0, 0.02, size=(GEMM_N, GEMM_K)))

"""GPU parity: the gfx950 kernels, called through the C ABI, against the CPU
oracle on the same seeded inputs.

Bars:
  * bit-exact codes, scale bytes and fp32 values against the oracle's fixed
    fp32 order (the order documented in include/kq.h);
  * against the fp64 definition: transformed values within 1e-5 of
    sum_i |x_i T_ik|, and at most 1e-4 of codes different, each by one
    adjacent grid step at a rounding tie (tests/parity.py).
"""
import numpy as np
import pytest

import oracle
from mxfp4_activation_quantizer_amd import inputs, kq
from parity import (assert_codes_within_tie_tolerance, assert_gemm_close, gemm_reference, to_gpu,
                    to_gpu_bf16, unpack_codes, REL_Y)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch


def _np(t):
    return t.cpu().numpy()


def _log(msg):
    print(msg, flush=True)


def _gpu_tq(x_bits, lu, d=None):
    codes, scales = kq.transform_quant(to_gpu_bf16(x_bits), to_gpu(lu), d=d)
    return _np(codes), _np(scales)


# --------------------------------------------------------------------------
# tiny workload (64 x 256)
# --------------------------------------------------------------------------
def test_tiny_bit_exact_vs_staged_order(torch_cuda):
    x, lu = inputs.activation("tiny"), inputs.lu_params("tiny")
    c, s = _gpu_tq(x, lu)
    wc, ws = oracle.transform_quant(x, lu, oracle.STAGED32)
    np.testing.assert_array_equal(s, ws)
    np.testing.assert_array_equal(c, wc)


def test_tiny_transform_values(torch_cuda):
    x, lu = inputs.activation("tiny"), inputs.lu_params("tiny")
    y = _np(kq.transform_f32(to_gpu_bf16(x), to_gpu(lu)))
    np.testing.assert_array_equal(y.view(np.uint32),
                                  oracle.transform(x, lu, oracle.STAGED32).view(np.uint32))
    y64 = oracle.transform(x, lu, oracle.DENSE64)
    bound = oracle.transform_absbound(x, lu)
    assert np.all(np.abs(y.astype(np.float64) - y64) <= REL_Y * bound + 1e-30)


def test_tiny_codes_vs_definition(torch_cuda):
    x, lu = inputs.activation("tiny"), inputs.lu_params("tiny")
    c, s = _gpu_tq(x, lu)
    wc, ws = oracle.transform_quant(x, lu, oracle.DENSE64)
    assert_codes_within_tie_tolerance(c, s, wc, ws, oracle.transform(x, lu, oracle.DENSE64),
                                      oracle.transform_absbound(x, lu))


# --------------------------------------------------------------------------
# the quantizer stage over every bf16 value and around every rounding tie
# --------------------------------------------------------------------------
IDENTITY = np.array([0.0, 1.0, 0.0], np.float32)


@pytest.mark.parametrize("arrangement", ["consecutive", "strided", "permuted"])
def test_identity_params_every_bf16_value(torch_cuda, arrangement):
    """With (l,u,v) = (0,1,0) every factor is I, so the kernel is plain MXFP4
    of the bf16 input, up to the sign of zero (fma(0, q, -0) is +0 when q > 0,
    in the oracle's staged order as on the GPU); all 65,536 bf16 patterns go
    through it."""
    pats = np.arange(65536, dtype=np.uint16)
    if arrangement == "strided":
        pats = pats.reshape(32, 2048).T.reshape(-1)
    elif arrangement == "permuted":
        pats = np.random.default_rng(0).permutation(pats)
    x = pats.reshape(256, 256)
    lu = np.tile(IDENTITY, (8, 5, 1))
    c, s = _gpu_tq(x, lu)
    sc, ss = oracle.transform_quant(x, lu, oracle.STAGED32)
    np.testing.assert_array_equal(s, ss)
    np.testing.assert_array_equal(c, sc)
    wc, ws = oracle.mxfp4_quant(inputs.bf16_bits_to_f32(x))
    np.testing.assert_array_equal(s, ws)
    u, wu = unpack_codes(c), unpack_codes(wc)
    differ = u != wu
    assert np.all((u[differ] & 7) == 0) and np.all((wu[differ] & 7) == 0)
    assert differ.sum() <= 4
    assert (s == 0xFF).any()


def _neighbours(v, k):
    out = [v]
    up = down = np.float32(v)
    for _ in range(k):
        up = np.nextafter(up, np.float32(np.inf))
        down = np.nextafter(down, np.float32(-np.inf))
        out += [up, down]
    return out


def test_quantizer_at_rounding_ties_all_scales(torch_cuda):
    """fp32 values at and next to every E2M1 midpoint and grid value, at
    every scale exponent, in blocks whose amax pins the scale."""
    qs = []
    for m in [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 1, 1.5, 2, 3, 4, 6]:
        qs += _neighbours(np.float32(m), 3)
    qs = np.array(qs, np.float32)
    qs = np.concatenate([qs, -qs])
    rows = []
    for e in range(-127, 126):
        pilot = np.float32(np.ldexp(4.0, e)) if e > -127 else np.float32(np.ldexp(4.0, -127))
        vals = (qs.astype(np.float64) * 2.0 ** e).astype(np.float32)
        for i in range(0, len(vals), 31):
            blk = np.zeros(32, np.float32)
            chunk = vals[i:i + 31]
            blk[:len(chunk)] = chunk
            blk[31] = pilot
            rows.append(blk)
    while len(rows) % 8:
        rows.append(np.zeros(32, np.float32))
    y = np.stack(rows).reshape(-1, 256)
    c, s = kq.mxfp4_quant_f32(to_gpu(y))
    wc, ws = oracle.mxfp4_quant(y)
    np.testing.assert_array_equal(_np(s), ws)
    np.testing.assert_array_equal(_np(c), wc)


def test_quantizer_random_fp32(torch_cuda):
    g = np.random.default_rng(1)
    n = 512 * 1024
    y = (g.standard_normal(n) * 2.0 ** g.integers(-140, 120, n)).astype(np.float32)
    # sprinkle zeros, negative zeros, subnormals, huge values and specials
    idx = g.choice(n, 4000, replace=False)
    y[idx[:500]] = 0.0
    y[idx[500:1000]] = -0.0
    y[idx[1000:1500]] = (g.standard_normal(500) * 2.0 ** -140).astype(np.float32)
    y[idx[1500:1600]] = np.float32(3.3e38)
    y[idx[1600:1650]] = np.nan
    y[idx[1650:1700]] = np.inf
    y[idx[1700:1750]] = -np.inf
    y = y.reshape(-1, 512)
    c, s = kq.mxfp4_quant_f32(to_gpu(y))
    wc, ws = oracle.mxfp4_quant(y)
    np.testing.assert_array_equal(_np(s), ws)
    np.testing.assert_array_equal(_np(c), wc)


# --------------------------------------------------------------------------
# transform wiring
# --------------------------------------------------------------------------
def test_power_of_two_diagonal_params_are_exact(torch_cuda):
    """(0, 2^m, 0) factors give an exact diagonal power-of-two T: the kernel
    must equal the fp64 definition bit for bit."""
    g = np.random.default_rng(2)
    nb = 12
    lu = np.zeros((nb, 5, 3), np.float32)
    lu[:, :, 1] = 2.0 ** g.integers(-3, 4, (nb, 5))
    x = inputs.f64_to_bf16_bits(g.standard_normal((100, nb * 32)) * 5)
    c, s = _gpu_tq(x, lu)
    wc, ws = oracle.transform_quant(x, lu, oracle.DENSE64)
    np.testing.assert_array_equal(s, ws)
    np.testing.assert_array_equal(c, wc)


def test_spike_through_hadamard_start(torch_cuda):
    """LRQ-DiT Lemma 1 with a Hadamard: a spike of 30 becomes 30/sqrt(32) =
    5.3 everywhere, so scale byte 127 and every code magnitude is 6."""
    nb = 4
    lu = inputs.hadamard_init(nb)
    x = np.zeros((32, nb * 32), np.float64)
    for t in range(32):
        x[t, (t % nb) * 32 + t] = 30.0 if t % 2 else -30.0
    xb = inputs.f64_to_bf16_bits(x)
    c, s = _gpu_tq(xb, lu)
    for t in range(32):
        j = t % nb
        assert s[t, j] == 127
        assert np.all(unpack_codes(c)[t, j * 32:(j + 1) * 32] & 7 == 7)
        others = [k for k in range(nb) if k != j]
        assert np.all(s[t, others] == 0)


def test_shear_on_each_bit(torch_cuda):
    """A lone lower shear on bit b mixes channel pairs (k, k ^ 2^b) only."""
    g = np.random.default_rng(3)
    x = inputs.f64_to_bf16_bits(g.standard_normal((8, 32)))
    for b in range(5):
        lu = np.tile(IDENTITY, (1, 5, 1))
        lu[0, b, 0] = 0.75
        y = _np(kq.transform_f32(to_gpu_bf16(x), to_gpu(lu)))
        np.testing.assert_array_equal(y, oracle.transform(x, lu, oracle.STAGED32))


def _rcp_sweep_u(seed=5, n_random=20000):
    """u values for the reciprocal of the factor expansion: every biased
    exponent 0..254 (0: zero and subnormals) with the significands all ones,
    all zeros, top bit only, lowest bit only and four seeded random ones, both
    signs; then seeded random finite bit patterns."""
    g = np.random.default_rng(seed)
    sig = [0x7FFFFF, 0, 0x400000, 1] + [int(v) for v in g.integers(0, 1 << 23, 4)]
    bits = [(sgn << 31) | (e << 23) | m for e in range(255) for m in sig for sgn in (0, 1)]
    rnd = (g.integers(0, 2, n_random).astype(np.uint64) << 31) | \
        (g.integers(0, 255, n_random).astype(np.uint64) << 23) | \
        g.integers(0, 1 << 23, n_random).astype(np.uint64)
    return np.concatenate([np.array(bits, np.uint64), rnd]).astype(np.uint32).view(np.float32)


def test_factor_reciprocal_every_exponent(torch_cuda):
    """The kernel's 1/u (a corrected hardware reciprocal, IEEE division outside
    the exponent range where the correction is exact) against the oracle's
    IEEE division, bit for bit: block j has factor 0 = (0, u_j, 0) and the
    identity elsewhere, and x = e_0 + e_1 in every block, so y_0 = u_j and
    y_1 = 1/u_j.  Three rows of 24,080 blocks: 24,080 is not a multiple of 64,
    so each u is handled at three different lanes of a wave."""
    u = _rcp_sweep_u()
    nb = u.size
    lu = np.tile(IDENTITY, (nb, 5, 1)).astype(np.float32)
    lu[:, 0, 1] = u
    x = np.zeros((3, nb * 32), np.float64)
    x[:, 0::32] = 1.0
    x[:, 1::32] = 1.0
    xb = inputs.f64_to_bf16_bits(x)
    got = _np(kq.transform_f32(to_gpu_bf16(xb), to_gpu(lu)))
    want = oracle.transform(xb, lu, oracle.STAGED32)
    nan_g, nan_w = np.isnan(got), np.isnan(want)
    np.testing.assert_array_equal(nan_g, nan_w)
    np.testing.assert_array_equal(got.view(np.uint32)[~nan_g], want.view(np.uint32)[~nan_w])
    # y_1 is exactly the IEEE reciprocal of every u, y_0 = u
    with np.errstate(divide="ignore", over="ignore"):
        recip = np.float32(1.0) / u
    fin = ~np.isnan(recip)
    for r in range(3):
        np.testing.assert_array_equal(got[r, 1::32][fin].view(np.uint32), recip[fin].view(np.uint32))
        np.testing.assert_array_equal(got[r, 0::32].view(np.uint32), u.view(np.uint32))


# --------------------------------------------------------------------------
# shapes, strides, edge cases
# --------------------------------------------------------------------------
@pytest.mark.parametrize("tokens,nb,pad", [(1, 1, 0), (3, 2, 8), (77, 3, 0), (300, 5, 24),
                                           (129, 36, 0), (65, 96, 8), (33, 97, 0), (5, 384, 16),
                                           (1000, 7, 0)])
def test_ragged_shapes_and_strides(torch_cuda, tokens, nb, pad):
    torch = torch_cuda
    g = np.random.default_rng(tokens * 1000 + nb)
    d = nb * 32
    xf = g.standard_normal((tokens, d + pad)) * np.exp(g.standard_normal((tokens, 1)))
    x = inputs.f64_to_bf16_bits(xf)
    x[:, d:] = 0x7FC0                       # NaN padding must never be read
    lu = (inputs.hadamard_init(nb) + g.normal(0, 0.2, (nb, 5, 3))).astype(np.float32)
    # outputs inside canary-filled buffers
    cbuf = torch.full((tokens * d // 2 + 64,), 0xA5, dtype=torch.uint8, device="cuda:0")
    sbuf = torch.full((tokens * nb + 64,), 0x5A, dtype=torch.uint8, device="cuda:0")
    codes = cbuf[32:32 + tokens * d // 2].view(tokens, d // 2)
    scales = sbuf[32:32 + tokens * nb].view(tokens, nb)
    kq.transform_quant(to_gpu_bf16(x), to_gpu(lu), d=d, codes=codes, scales=scales)
    wc, ws = oracle.transform_quant(x, lu, oracle.STAGED32, d=d)
    np.testing.assert_array_equal(_np(scales), ws)
    np.testing.assert_array_equal(_np(codes), wc)
    cb, sb = _np(cbuf), _np(sbuf)
    assert np.all(cb[:32] == 0xA5) and np.all(cb[32 + tokens * d // 2:] == 0xA5)
    assert np.all(sb[:32] == 0x5A) and np.all(sb[32 + tokens * nb:] == 0x5A)


def test_empty_input(torch_cuda):
    torch = torch_cuda
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda:0")
    lu = to_gpu(inputs.hadamard_init(2))
    c, s = kq.transform_quant(x, lu)
    assert c.shape == (0, 32) and s.shape == (0, 2)


def test_nonfinite_and_overflow_blocks(torch_cuda):
    nb = 4
    x = np.full((6, nb * 32), 0x3F80, np.uint16)  # 1.0
    x[0, 5] = 0x7FC0          # NaN in block 0
    x[1, 40] = 0x7F80         # +Inf in block 1
    x[2, 70] = 0xFF80         # -Inf in block 2
    x[3, 96:128] = 0x7F7F     # bf16 max everywhere in block 3: the transform overflows
    x[4, :] = 0x0000
    x[5, :] = 0x8000          # -0.0
    lu = inputs.hadamard_init(nb)
    c, s = _gpu_tq(x, lu)
    wc, ws = oracle.transform_quant(x, lu, oracle.STAGED32)
    np.testing.assert_array_equal(s, ws)
    np.testing.assert_array_equal(c, wc)
    assert s[0, 0] == s[1, 1] == s[2, 2] == 0xFF
    assert s[4, 0] == 0 and s[5, 0] == 0


def test_deterministic(torch_cuda):
    x, lu = inputs.activation("tiny"), inputs.lu_params("tiny")
    a = _gpu_tq(x, lu)
    b = _gpu_tq(x, lu)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


# --------------------------------------------------------------------------
# baselines and the ceiling kernel
# --------------------------------------------------------------------------
def test_smooth_quant_bit_exact(torch_cuda):
    x = inputs.activation("tiny")
    m = inputs.smooth_multipliers(x)
    c, s = kq.smooth_quant(to_gpu_bf16(x), to_gpu(m))
    wc, ws = oracle.smooth_quant(x, m)
    np.testing.assert_array_equal(_np(s), ws)
    np.testing.assert_array_equal(_np(c), wc)


@pytest.mark.parametrize("tokens,nb,pad", [(1, 1, 0), (77, 3, 8), (300, 96, 0), (5, 255, 16),
                                           (9, 300, 0), (3, 700, 8)])
def test_smooth_quant_ragged_shapes_and_strides(torch_cuda, tokens, nb, pad):
    """Each workgroup stages the multipliers of the blocks its lanes touch
    (min(nb, 256) blocks, a range of the vector that wraps at d): nb below,
    at and above 256, wrapping inside a workgroup, ragged token counts and
    strided rows with NaN padding that must never be read."""
    torch = torch_cuda
    g = np.random.default_rng(tokens * 7 + nb)
    d = nb * 32
    xf = g.standard_normal((tokens, d + pad)) * np.exp(g.standard_normal((tokens, 1)))
    x = inputs.f64_to_bf16_bits(xf)
    x[:, d:] = 0x7FC0
    m = np.exp(g.normal(0, 1.5, d)).astype(np.float32)
    c, s = kq.smooth_quant(to_gpu_bf16(x), to_gpu(m), d=d)
    wc, ws = oracle.smooth_quant(x, m, d=d)
    np.testing.assert_array_equal(_np(s), ws)
    np.testing.assert_array_equal(_np(c), wc)


def test_fwht32_quant_bit_exact_and_vs_definition(torch_cuda):
    x = inputs.activation("tiny")
    c, s = kq.fwht32_quant(to_gpu_bf16(x))
    c, s = _np(c), _np(s)
    wc, ws = oracle.fwht32_quant(x, oracle.STAGED32)
    np.testing.assert_array_equal(s, ws)
    np.testing.assert_array_equal(c, wc)
    dc, ds = oracle.fwht32_quant(x, oracle.DENSE64)
    xf = np.abs(inputs.bf16_bits_to_f32(x).astype(np.float64))
    bound = np.repeat(xf.reshape(x.shape[0], -1, 32).sum(2), 32, axis=1) / np.sqrt(32)
    assert_codes_within_tie_tolerance(c, s, dc, ds, oracle.fwht32(x, oracle.DENSE64), bound)


def test_copy_ceiling_touches_every_unit(torch_cuda):
    """The ceiling kernel's codes are the XOR of each unit's fp32 bit patterns
    eight at a time, its scale byte the low byte of their XOR."""
    x = inputs.activation("tiny")
    c, s = kq.copy_ceiling(to_gpu_bf16(x))
    bits = (x.astype(np.uint32) << 16).reshape(64, 8, 4, 8)
    f = np.bitwise_xor.reduce(bits, axis=3)
    np.testing.assert_array_equal(_np(c).view(np.uint32).reshape(64, 8, 4), f)
    fs = np.bitwise_xor.reduce(f, axis=2) & 0xFF
    np.testing.assert_array_equal(_np(s), fs.astype(np.uint8))


def test_stream_ceiling_reads_and_writes_every_unit(torch_cuda):
    """The streaming reference: unit u's 16 output bytes are the XOR of the
    16-byte chunks 64i + (u mod 64) (i = 0..3) of its wave's 4 KB, its byte
    the low byte of their XOR; a read-only pass writes nothing but byte 0."""
    torch = torch_cuda
    g = np.random.default_rng(12)
    units = 64 * 37 + 5                      # a ragged last wave
    src = g.integers(0, 1 << 32, units * 16, dtype=np.uint64).astype(np.uint32)
    sd = torch.from_numpy(src.view(np.int32)).to("cuda:0")
    codes = torch.full((units * 16 + 32,), 0xA5, dtype=torch.uint8, device="cuda:0")
    scales = torch.full((units + 32,), 0x5A, dtype=torch.uint8, device="cuda:0")
    kq.stream_ceiling(sd, codes[:units * 16], scales[:units])
    chunks = np.concatenate([src, np.zeros(64 * 16 * 4, np.uint32)]).reshape(-1, 4)  # 16-B chunks
    want = np.empty((units, 4), np.uint32)
    for u in range(units):
        w0, lane = (u // 64) * 256, u % 64
        want[u] = chunks[w0 + lane] ^ chunks[w0 + 64 + lane] ^ chunks[w0 + 128 + lane] ^ \
            chunks[w0 + 192 + lane]
    got = _np(codes)
    np.testing.assert_array_equal(got[:units * 16].view(np.uint32).reshape(units, 4), want)
    assert np.all(got[units * 16:] == 0xA5)
    f = np.bitwise_xor.reduce(want, axis=1) & 0xFF
    np.testing.assert_array_equal(_np(scales)[:units], f.astype(np.uint8))
    assert np.all(_np(scales)[units:] == 0x5A)
    one = torch.full((8,), 0x33, dtype=torch.uint8, device="cuda:0")
    kq.stream_ceiling(sd, None, one)
    o = _np(one)
    assert np.all(o[1:] == 0x33) and o[0] in (0x33, 1)


# --------------------------------------------------------------------------
# the four-lanes-per-unit layout of the same quantizer
# --------------------------------------------------------------------------
@pytest.mark.parametrize("tokens,nb,pad", [(1, 1, 0), (3, 2, 8), (77, 3, 0), (129, 36, 0),
                                           (65, 96, 8), (33, 97, 0), (5, 384, 16)])
def test_quad_lane_quantizer_bit_exact(torch_cuda, tokens, nb, pad):
    torch = torch_cuda
    g = np.random.default_rng(tokens * 7 + nb)
    d = nb * 32
    x = inputs.f64_to_bf16_bits(g.standard_normal((tokens, d + pad)) *
                                np.exp(g.standard_normal((tokens, 1))))
    x[:, d:] = 0x7FC0
    lu = (inputs.hadamard_init(nb) + g.normal(0, 0.2, (nb, 5, 3))).astype(np.float32)
    cbuf = torch.full((tokens * d // 2 + 64,), 0xA5, dtype=torch.uint8, device="cuda:0")
    sbuf = torch.full((tokens * nb + 64,), 0x5A, dtype=torch.uint8, device="cuda:0")
    codes = cbuf[32:32 + tokens * d // 2].view(tokens, d // 2)
    scales = sbuf[32:32 + tokens * nb].view(tokens, nb)
    kq.transform_quant_quad(to_gpu_bf16(x), to_gpu(lu), d=d, codes=codes, scales=scales)
    wc, ws = oracle.transform_quant(x, lu, oracle.STAGED32, d=d)
    np.testing.assert_array_equal(_np(scales), ws)
    np.testing.assert_array_equal(_np(codes), wc)
    cb, sb = _np(cbuf), _np(sbuf)
    assert np.all(cb[:32] == 0xA5) and np.all(cb[32 + tokens * d // 2:] == 0xA5)
    assert np.all(sb[:32] == 0x5A) and np.all(sb[32 + tokens * nb:] == 0x5A)


def test_quad_lane_quantizer_specials(torch_cuda):
    nb = 4
    x = np.full((8, nb * 32), 0x3F80, np.uint16)
    x[0, 5] = 0x7FC0
    x[1, 40] = 0x7F80
    x[2, 70] = 0xFF80
    x[3, 96:128] = 0x7F7F
    x[4, :] = 0x0000
    x[5, :] = 0x8000
    x[6, 3::7] = 0x8000          # -0 mixed with ones
    x[7, 8:24] = 0x0001          # bf16 subnormals
    lu = inputs.hadamard_init(nb)
    c, s = kq.transform_quant_quad(to_gpu_bf16(x), to_gpu(lu))
    wc, ws = oracle.transform_quant(x, lu, oracle.STAGED32)
    np.testing.assert_array_equal(_np(s), ws)
    np.testing.assert_array_equal(_np(c), wc)
    # identity parameters over every bf16 value
    allv = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(2048, 32)
    lu1 = np.tile(IDENTITY, (1, 5, 1)).astype(np.float32)
    c, s = kq.transform_quant_quad(to_gpu_bf16(allv), to_gpu(lu1))
    wc, ws = oracle.transform_quant(allv, lu1, oracle.STAGED32)
    np.testing.assert_array_equal(_np(s), ws)
    np.testing.assert_array_equal(_np(c), wc)


def test_quad_lane_quantizer_full_size_equals_one_lane(torch_cuda):
    """At the FLUX attention-projection size the quad-lane kernel writes the
    same bytes as kq_transform_quant everywhere, and sampled rows equal the
    oracle's fixed order."""
    x = inputs.activation("flux_attn")
    lu = inputs.lu_params("flux_attn")
    xd, ld = to_gpu_bf16(x), to_gpu(lu)
    c1, s1 = kq.transform_quant(xd, ld)
    c4, s4 = kq.transform_quant_quad(xd, ld)
    c4, s4 = _np(c4), _np(s4)
    np.testing.assert_array_equal(s4, _np(s1))
    np.testing.assert_array_equal(c4, _np(c1))
    rows = np.array([0, 1, 2047, 4607])
    wc, ws = oracle.transform_quant(x[rows], lu, oracle.STAGED32)
    np.testing.assert_array_equal(s4[rows], ws)
    np.testing.assert_array_equal(c4[rows], wc)


# --------------------------------------------------------------------------
# full-size workloads, sampled rows
# --------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["pixart", "flux_attn", "flux_mlp"])
def test_full_size_workload_sampled(torch_cuda, name):
    _log(f"full-size {name}: generating")
    x = inputs.activation(name)
    lu = inputs.lu_params(name)
    c, s = _gpu_tq(x, lu)
    rows = np.sort(np.random.default_rng(7).choice(x.shape[0], 96, replace=False))
    rows[:2] = [0, 1]
    rows[-1] = x.shape[0] - 1
    xs = x[rows]
    _log(f"full-size {name}: oracle on {len(rows)} rows")
    wc, ws = oracle.transform_quant(xs, lu, oracle.STAGED32)
    np.testing.assert_array_equal(s[rows], ws)
    np.testing.assert_array_equal(c[rows], wc)
    dc, ds = oracle.transform_quant(xs, lu, oracle.DENSE64)
    n_s, n_c = assert_codes_within_tie_tolerance(
        c[rows], s[rows], dc, ds, oracle.transform(xs, lu, oracle.DENSE64),
        oracle.transform_absbound(xs, lu))
    _log(f"full-size {name}: vs fp64 definition {n_s} scale / {n_c} code tie differences")
    # whole-tensor properties at full size: every finite block's largest code
    # magnitude is 4 or 6, and no scale is NaN for finite input
    assert not (s == 0xFF).any()
    mags = (unpack_codes(c) & 7).reshape(x.shape[0], -1, 32).max(axis=2)
    assert np.all((mags >= 6) | (s == 0))


# --------------------------------------------------------------------------
# the matrix-core arm: dense 32x32 product per block on MFMA
# --------------------------------------------------------------------------
def _mfma_vs_definition(x, lu, d=None):
    c, s = kq.transform_quant_mfma(to_gpu_bf16(x), to_gpu(lu), d=d)
    c, s = _np(c), _np(s)
    dd = x.shape[1] if d is None else d
    dc, ds = oracle.transform_quant(x, lu, oracle.DENSE64, d=dd)
    return c, s, assert_codes_within_tie_tolerance(
        c, s, dc, ds, oracle.transform(x, lu, oracle.DENSE64, d=dd),
        oracle.transform_absbound(x, lu, d=dd))


def test_mfma_tiny_vs_definition(torch_cuda):
    x, lu = inputs.activation("tiny"), inputs.lu_params("tiny")
    _mfma_vs_definition(x, lu)


def test_mfma_identity_params_every_bf16_value(torch_cuda):
    """T = I: the dense product returns x exactly, so the codes are plain
    MXFP4 of the input up to the sign of zero."""
    x = np.random.default_rng(0).permutation(np.arange(65536, dtype=np.uint16)).reshape(256, 256)
    lu = np.tile(IDENTITY, (8, 5, 1))
    c, s = kq.transform_quant_mfma(to_gpu_bf16(x), to_gpu(lu))
    wc, ws = oracle.mxfp4_quant(inputs.bf16_bits_to_f32(x))
    np.testing.assert_array_equal(_np(s), ws)
    u, wu = unpack_codes(_np(c)), unpack_codes(wc)
    differ = u != wu
    assert np.all((u[differ] & 7) == 0) and np.all((wu[differ] & 7) == 0)


@pytest.mark.parametrize("tokens,nb,pad", [(1, 1, 0), (3, 2, 8), (77, 3, 0), (300, 5, 24),
                                           (129, 36, 0), (65, 96, 8), (33, 97, 0), (5, 384, 16)])
def test_mfma_ragged_shapes_and_strides(torch_cuda, tokens, nb, pad):
    torch = torch_cuda
    g = np.random.default_rng(tokens * 1000 + nb + 1)
    d = nb * 32
    x = inputs.f64_to_bf16_bits(g.standard_normal((tokens, d + pad)) * np.exp(g.standard_normal((tokens, 1))))
    x[:, d:] = 0x7FC0
    lu = (inputs.hadamard_init(nb) + g.normal(0, 0.2, (nb, 5, 3))).astype(np.float32)
    cbuf = torch.full((tokens * d // 2 + 64,), 0xA5, dtype=torch.uint8, device="cuda:0")
    sbuf = torch.full((tokens * nb + 64,), 0x5A, dtype=torch.uint8, device="cuda:0")
    codes = cbuf[32:32 + tokens * d // 2].view(tokens, d // 2)
    scales = sbuf[32:32 + tokens * nb].view(tokens, nb)
    kq.transform_quant_mfma(to_gpu_bf16(x), to_gpu(lu), d=d, codes=codes, scales=scales)
    dc, ds = oracle.transform_quant(x, lu, oracle.DENSE64, d=d)
    assert_codes_within_tie_tolerance(_np(codes), _np(scales), dc, ds,
                                      oracle.transform(x, lu, oracle.DENSE64, d=d),
                                      oracle.transform_absbound(x, lu, d=d))
    cb, sb = _np(cbuf), _np(sbuf)
    assert np.all(cb[:32] == 0xA5) and np.all(cb[32 + tokens * d // 2:] == 0xA5)
    assert np.all(sb[:32] == 0x5A) and np.all(sb[32 + tokens * nb:] == 0x5A)


def test_mfma_nonfinite_blocks(torch_cuda):
    nb = 4
    x = np.full((4, nb * 32), 0x3F80, np.uint16)
    x[0, 5] = 0x7FC0
    x[1, 40] = 0x7F80
    x[2, 70] = 0xFF80
    lu = inputs.lu_params("tiny")[:nb]
    c, s = kq.transform_quant_mfma(to_gpu_bf16(x), to_gpu(lu))
    c, s = _np(c), _np(s)
    assert s[0, 0] == s[1, 1] == s[2, 2] == 0xFF
    assert not c[0, :16].any() and not c[1, 16:32].any() and not c[2, 32:48].any()
    wc, ws = oracle.transform_quant(x, lu, oracle.DENSE64)
    ok = ws != 0xFF
    np.testing.assert_array_equal(s[ok], ws[ok])


@pytest.mark.parametrize("name", ["pixart", "flux_attn", "flux_mlp"])
def test_mfma_full_size_workload_sampled(torch_cuda, name):
    x = inputs.activation(name)
    lu = inputs.lu_params(name)
    c, s = kq.transform_quant_mfma(to_gpu_bf16(x), to_gpu(lu))
    c, s = _np(c), _np(s)
    rows = np.sort(np.random.default_rng(8).choice(x.shape[0], 96, replace=False))
    rows[-1] = x.shape[0] - 1
    xs = x[rows]
    dc, ds = oracle.transform_quant(xs, lu, oracle.DENSE64)
    n_s, n_c = assert_codes_within_tie_tolerance(
        c[rows], s[rows], dc, ds, oracle.transform(xs, lu, oracle.DENSE64),
        oracle.transform_absbound(xs, lu))
    _log(f"mfma full-size {name}: vs fp64 definition {n_s} scale / {n_c} code tie differences")
    # the two device arms agree to the same tolerance everywhere
    bc, bs = _gpu_tq(x, lu)
    assert np.mean(bs != s) < 1e-4
    assert np.mean(bc != c) < 2e-4


# --------------------------------------------------------------------------
# the inverse side: dequantise and undo the transform
# --------------------------------------------------------------------------
def _bf16_equal_or_both_nan(a, b):
    af, bf = inputs.bf16_bits_to_f32(a), inputs.bf16_bits_to_f32(b)
    both_nan = np.isnan(af) & np.isnan(bf)
    return (a == b) | both_nan


def _gpu_dequant_inverse(codes, scales, lu):
    torch = __import__("torch")
    out = kq.dequant_inverse(to_gpu(codes), to_gpu(scales), to_gpu(lu))
    return _np(out.view(torch.int16)).view(np.uint16)


def test_dequant_inverse_every_code_and_scale(torch_cuda):
    """All 16 codes in both nibbles under all 256 scale bytes (0xFF = NaN
    block), random parameters: bit-exact with the oracle's fixed order."""
    g = np.random.default_rng(11)
    tokens, nb = 256, 4
    codes = g.integers(0, 256, (tokens, nb * 16), dtype=np.uint8)
    scales = np.tile(np.arange(256, dtype=np.uint8)[:, None], (1, nb))
    lu = (inputs.hadamard_init(nb) + g.normal(0, 0.1, (nb, 5, 3))).astype(np.float32)
    got = _gpu_dequant_inverse(codes, scales, lu)
    want = oracle.dequant_inverse(codes, scales, lu, oracle.STAGED32)
    assert np.all(_bf16_equal_or_both_nan(got, want))
    assert np.isnan(inputs.bf16_bits_to_f32(got[255])).all()


def test_dequant_inverse_identity_is_plain_decode(torch_cuda):
    g = np.random.default_rng(12)
    codes = g.integers(0, 256, (64, 128), dtype=np.uint8)
    scales = g.integers(100, 150, (64, 8), dtype=np.uint8)
    lu = np.tile(IDENTITY, (8, 5, 1))
    got = inputs.bf16_bits_to_f32(_gpu_dequant_inverse(codes, scales, lu))
    want = oracle.mxfp4_dequant(codes, scales)
    np.testing.assert_array_equal(got, want)


def _inverse_vs_definition(codes, scales, lu, got):
    """bf16 results vs the fp64 inverse: equal, one bf16 step apart, or within
    1e-5 of sum_i |y_i| |Tinv_ik| (cancellation)."""
    yh = oracle.mxfp4_dequant(codes, scales).astype(np.float64)
    nb = codes.shape[1] // 16
    exact = np.empty_like(yh)
    bound = np.empty_like(yh)
    for j in range(nb):
        Ti = oracle.block_inverse_matrix(lu[j])
        exact[:, 32 * j:32 * j + 32] = yh[:, 32 * j:32 * j + 32] @ Ti
        bound[:, 32 * j:32 * j + 32] = np.abs(yh[:, 32 * j:32 * j + 32]) @ np.abs(Ti)
    g = inputs.bf16_bits_to_f32(got).astype(np.float64)
    ok = (np.abs(g - exact) <= 2.0 ** -8 * np.abs(exact) + 1e-5 * bound)
    assert ok.all(), f"{(~ok).sum()} outputs off the fp64 inverse"


def test_dequant_inverse_round_trip_tiny(torch_cuda):
    x, lu = inputs.activation("tiny"), inputs.lu_params("tiny")
    c, s = _gpu_tq(x, lu)
    got = _gpu_dequant_inverse(c, s, lu)
    want = oracle.dequant_inverse(c, s, lu, oracle.STAGED32)
    np.testing.assert_array_equal(got, want)
    _inverse_vs_definition(c, s, lu, got)


@pytest.mark.parametrize("tokens,nb", [(1, 1), (77, 3), (129, 36), (33, 97)])
def test_dequant_inverse_ragged(torch_cuda, tokens, nb):
    g = np.random.default_rng(tokens + 7 * nb)
    x = inputs.f64_to_bf16_bits(g.standard_normal((tokens, nb * 32)) * 3)
    lu = (inputs.hadamard_init(nb) + g.normal(0, 0.2, (nb, 5, 3))).astype(np.float32)
    c, s = _gpu_tq(x, lu)
    got = _gpu_dequant_inverse(c, s, lu)
    np.testing.assert_array_equal(got, oracle.dequant_inverse(c, s, lu, oracle.STAGED32))
    _inverse_vs_definition(c, s, lu, got)


def _quant_sweep_shapes(n=24, seed=77):
    """Seeded (tokens, blocks, row padding): tokens 1..3000, blocks 1..400,
    padding 0, 8 or 24 elements."""
    g = np.random.default_rng(seed)
    return [(int(g.integers(1, 3001)), int(g.integers(1, 401)), int(g.choice([0, 8, 24])))
            for _ in range(n)]


@pytest.mark.parametrize("tokens,nb,pad", _quant_sweep_shapes())
def test_quantizer_and_inverse_shape_sweep(torch_cuda, tokens, nb, pad):
    """Random shapes through the quantizer (bit-exact with the oracle's fixed
    fp32 order, strided rows with NaN padding never read) and back through
    the inverse (bit-exact as well)."""
    g = np.random.default_rng(tokens * 13 + nb * 7 + pad)
    d = nb * 32
    xf = g.standard_normal((tokens, d + pad)) * np.exp(g.standard_normal((tokens, 1)))
    x = inputs.f64_to_bf16_bits(xf)
    x[:, d:] = 0x7FC0
    lu = (inputs.hadamard_init(nb) + g.normal(0, 0.2, (nb, 5, 3))).astype(np.float32)
    c, s = kq.transform_quant(to_gpu_bf16(x), to_gpu(lu), d=d)
    wc, ws = oracle.transform_quant(x, lu, oracle.STAGED32, d=d)
    np.testing.assert_array_equal(_np(s), ws)
    np.testing.assert_array_equal(_np(c), wc)
    got = _gpu_dequant_inverse(wc, ws, lu)
    np.testing.assert_array_equal(got, oracle.dequant_inverse(wc, ws, lu, oracle.STAGED32))


@pytest.mark.parametrize("tokens,nb,pad", [(5, 3, 8), (70, 1, 24), (131, 7, 16)])
def test_dequant_inverse_strided_output_leaves_padding(torch_cuda, tokens, nb, pad):
    """Row stride beyond d: every unit lands at its row's offset (the stores
    go out whole-line through a wave exchange, units of a wave spanning
    several rows) and the padding columns keep their sentinel."""
    torch = torch_cuda
    g = np.random.default_rng(tokens * 31 + nb)
    x = inputs.f64_to_bf16_bits(g.standard_normal((tokens, nb * 32)) * 2)
    lu = (inputs.hadamard_init(nb) + g.normal(0, 0.2, (nb, 5, 3))).astype(np.float32)
    c, s = _gpu_tq(x, lu)
    d = nb * 32
    out = torch.full((tokens, d + pad), -7.0, dtype=torch.bfloat16, device="cuda")
    kq.dequant_inverse(to_gpu(c), to_gpu(s), to_gpu(lu), x_out=out[:, :d])
    got = _np(out.view(torch.int16)).view(np.uint16)
    np.testing.assert_array_equal(got[:, :d], oracle.dequant_inverse(c, s, lu, oracle.STAGED32))
    assert (inputs.bf16_bits_to_f32(got[:, d:]) == -7.0).all()


def test_round_trip_error_flux_mlp(torch_cuda):
    """FLUX-MLP-shaped input: the MXFP4 round trip (quantise, then dequantise
    and invert) on the same 64 sampled rows for every transform.  The
    Kronecker round trip (GPU quantizer, then the GPU inverse) equals the
    oracle's bit for bit, so its error is the oracle's; per-channel scaling
    and FWHT32 decode the GPU codes (pinned to the oracle elsewhere) on the
    host.  At the Hadamard start the Kronecker transform is FWHT32 up to
    output signs, so those two errors agree."""
    x = inputs.activation("flux_mlp")
    d = x.shape[1]
    rows = np.sort(np.random.default_rng(3).choice(x.shape[0], 64, replace=False))
    xs = x[rows]
    xsf = inputs.bf16_bits_to_f32(xs).astype(np.float64)
    nx = np.linalg.norm(xsf)
    errs = {}
    for name, lu in (("kron_random", inputs.lu_params("flux_mlp")),
                     ("kron_hadamard", inputs.hadamard_init(d // 32))):
        c, s = _gpu_tq(xs, lu)
        got = _gpu_dequant_inverse(c, s, lu)
        want = oracle.dequant_inverse(*oracle.transform_quant(xs, lu, oracle.STAGED32), lu,
                                      oracle.STAGED32)
        np.testing.assert_array_equal(got, want)
        errs[name] = np.linalg.norm(inputs.bf16_bits_to_f32(got).astype(np.float64) - xsf) / nx
    m = inputs.smooth_multipliers(x)
    sc, ss = kq.smooth_quant(to_gpu_bf16(xs), to_gpu(m))
    xs_s = oracle.mxfp4_dequant(_np(sc), _np(ss)).astype(np.float64) / m[None, :]
    fc, fs = kq.fwht32_quant(to_gpu_bf16(xs))
    yh = oracle.mxfp4_dequant(_np(fc), _np(fs)).astype(np.float64)
    import scipy.linalg
    H = scipy.linalg.hadamard(32) / np.sqrt(32)
    xs_f = (yh.reshape(64, -1, 32) @ H).reshape(64, d)

    def bf16_err(v):
        v = inputs.bf16_bits_to_f32(inputs.f64_to_bf16_bits(v)).astype(np.float64)
        return np.linalg.norm(v - xsf) / nx

    errs["smooth"], errs["fwht32"] = bf16_err(xs_s), bf16_err(xs_f)
    _log("round-trip rel. Frobenius error, FLUX-MLP (64 rows): " +
         ", ".join(f"{k} {v:.4f}" for k, v in errs.items()))
    assert all(np.isfinite(v) for v in errs.values())
    assert abs(errs["kron_hadamard"] - errs["fwht32"]) <= 0.02 * errs["fwht32"]


# --------------------------------------------------------------------------
# weight preparation: MXFP4 of W * T^-T along K
# --------------------------------------------------------------------------
@pytest.mark.parametrize("rows,nb", [(64, 8), (77, 3), (130, 36), (5, 97)])
def test_weight_quant_bit_exact_and_vs_definition(torch_cuda, rows, nb):
    g = np.random.default_rng(rows + nb)
    w = inputs.f64_to_bf16_bits(g.normal(0, 0.02, (rows, nb * 32)))
    lu = (inputs.hadamard_init(nb) + g.normal(0, 0.1, (nb, 5, 3))).astype(np.float32)
    c, s = kq.weight_quant(to_gpu_bf16(w), to_gpu(lu))
    c, s = _np(c), _np(s)
    wc, ws = oracle.weight_quant(w, lu, oracle.STAGED32)
    np.testing.assert_array_equal(s, ws)
    np.testing.assert_array_equal(c, wc)
    dc, ds = oracle.weight_quant(w, lu, oracle.DENSE64)
    wf = np.abs(inputs.bf16_bits_to_f32(w).astype(np.float64))
    bound = np.concatenate([wf[:, 32 * j:32 * j + 32] @ np.abs(oracle.block_inverse_matrix(lu[j])).T
                            for j in range(nb)], 1)
    assert_codes_within_tie_tolerance(c, s, dc, ds, oracle.weight_transform(w, lu, oracle.DENSE64),
                                      bound)


# --------------------------------------------------------------------------
# the W4A4 consumer
# --------------------------------------------------------------------------
def _random_mxfp4(g, rows, k, lo=118, hi=128):
    codes = g.integers(0, 256, (rows, k // 2), dtype=np.uint8)
    scales = g.integers(lo, hi, (rows, k // 32), dtype=np.uint8)
    return codes, scales


@pytest.mark.parametrize("M,N,K", [(64, 64, 128), (128, 256, 256), (100, 300, 384),
                                   (1, 17, 128), (257, 129, 512),
                                   # K past one 15-step pass of the K pipeline
                                   # (3328), whole and ending in a half tile
                                   (70, 260, 4096), (33, 40, 4224), (5, 8, 7808),
                                   # K not a multiple of 512: the per-tile
                                   # kernel
                                   (130, 300, 768), (5, 17, 2304), (64, 256, 6912),
                                   # K a multiple of 512: the cross-tile
                                   # pipelined kernel (1536, 2560: an odd
                                   # number of scale pairs per tile; 1024,
                                   # 2048, 2560, 5120: a tile's first K tile
                                   # moves from stage to stage; 4608 and
                                   # 9216: two and three passes of its
                                   # 12-step loop)
                                   (257, 513, 1536), (70, 260, 4608), (33, 520, 9216),
                                   (100, 300, 1024), (129, 257, 2048), (40, 600, 2560),
                                   (33, 520, 5120),
                                   # a single output tile: seven of the eight
                                   # XCD groups have no tile and leave at once
                                   (1, 7, 1536), (3, 300, 3072)])
def test_gemm_random_mxfp4(torch_cuda, M, N, K):
    torch = torch_cuda
    g = np.random.default_rng(M * 7 + N * 3 + K)
    ac, as_ = _random_mxfp4(g, M, K)
    wc, ws = _random_mxfp4(g, N, K)
    y = kq.w4a4_gemm(to_gpu(ac), to_gpu(as_), to_gpu(wc), to_gpu(ws))
    yb = _np(y.view(torch.int16)).view(np.uint16)
    Y, B = gemm_reference(ac, as_, wc, ws)
    assert_gemm_close(yb, Y, B, K)


def _sweep_shapes(n=24, seed=2024):
    """Seeded GEMM shapes: M, N from 1 to 600, K any multiple of 128 up to
    9216, a third of them multiples of 1536 (the pipelined kernel)."""
    g = np.random.default_rng(seed)
    out = []
    for i in range(n):
        m, nn = int(g.integers(1, 601)), int(g.integers(1, 601))
        k = int(g.integers(1, 7)) * 1536 if i % 3 == 0 else int(g.integers(1, 73)) * 128
        out.append((m, nn, k))
    return out


@pytest.mark.parametrize("M,N,K", _sweep_shapes())
def test_gemm_shape_sweep(torch_cuda, M, N, K):
    torch = torch_cuda
    g = np.random.default_rng(M * 131 + N * 17 + K)
    ac, as_ = _random_mxfp4(g, M, K)
    wc, ws = _random_mxfp4(g, N, K)
    y = kq.w4a4_gemm(to_gpu(ac), to_gpu(as_), to_gpu(wc), to_gpu(ws))
    yb = _np(y.view(torch.int16)).view(np.uint16)
    Y, B = gemm_reference(ac, as_, wc, ws)
    assert_gemm_close(yb, Y, B, K)


@pytest.mark.parametrize("M,N,K,pad", [(37, 300, 256, 20), (130, 17, 128, 15), (5, 513, 384, 8),
                                       (70, 260, 768, 12), (70, 260, 1536, 12)])
def test_gemm_strided_output_leaves_padding(torch_cuda, M, N, K, pad):
    """Row stride beyond N: the whole-row epilogue writes only columns < N
    of rows < M; the padding keeps its sentinel."""
    torch = torch_cuda
    g = np.random.default_rng(M + 3 * N + K)
    ac, as_ = _random_mxfp4(g, M, K)
    wc, ws = _random_mxfp4(g, N, K)
    ld = (N + pad + 7) // 8 * 8
    buf = torch.full((M, ld), 5.0, dtype=torch.bfloat16, device="cuda")
    kq.w4a4_gemm(to_gpu(ac), to_gpu(as_), to_gpu(wc), to_gpu(ws), y=buf[:, :N])
    yb = _np(buf.view(torch.int16)).view(np.uint16)
    Y, B = gemm_reference(ac, as_, wc, ws)
    assert_gemm_close(yb[:, :N], Y, B, K)
    assert (inputs.bf16_bits_to_f32(yb[:, N:]) == 5.0).all()


@pytest.mark.parametrize("K", [1024, 3072])
def test_gemm_scales_only_4_byte_aligned(torch_cuda, K):
    """Scale arrays 4-byte but not 16-byte aligned (the ABI's minimum): the
    pipelined kernel's 16-byte scale DMAs cannot serve them, so the per-tile
    kernel must run, and the result must be the same."""
    torch = torch_cuda
    M, N = 150, 300
    g = np.random.default_rng(K + 5)
    ac, as_ = _random_mxfp4(g, M, K)
    wc, ws = _random_mxfp4(g, N, K)

    def off4(a):
        buf = torch.zeros(a.size + 16, dtype=torch.uint8, device="cuda")
        v = buf[4:4 + a.size].view(a.shape)
        v.copy_(torch.from_numpy(a).cuda())
        assert v.data_ptr() % 16 == 4
        return v

    y = kq.w4a4_gemm(to_gpu(ac), off4(as_), to_gpu(wc), off4(ws))
    yb = _np(y.view(torch.int16)).view(np.uint16)
    Y, B = gemm_reference(ac, as_, wc, ws)
    assert_gemm_close(yb, Y, B, K)
    y16 = kq.w4a4_gemm(to_gpu(ac), to_gpu(as_), to_gpu(wc), to_gpu(ws))
    np.testing.assert_array_equal(_np(y16.view(torch.int16)), _np(y.view(torch.int16)))


@pytest.mark.parametrize("K", [512, 768, 1024, 1536, 2048, 2560, 3072])
def test_gemm_workgroups_walk_several_tiles(torch_cuda, K):
    """More output tiles (20 x 16 = 320) than workgroups (one per CU): the
    persistent workgroups walk several tiles.  K = 768 takes the per-tile
    kernel; the others the pipelined one, which carries the K pipeline and
    the scale ring from one tile into the next: with 512, 1536 and 2560 (one,
    three and five scale pairs per tile) the ring slot of a tile's first pair
    alternates, with 512, 1024, 2048 and 2560 (2, 4, 8 and 10 K tiles) the
    stage of a tile's first K tile moves on by 2, 1, 2 and 1.  Three rows of every M tile are checked
    over all N columns."""
    torch = torch_cuda
    M, N = 2560, 4096
    g = np.random.default_rng(77 + K)
    ac, as_ = _random_mxfp4(g, M, K)
    wc, ws = _random_mxfp4(g, N, K)
    y = kq.w4a4_gemm(to_gpu(ac), to_gpu(as_), to_gpu(wc), to_gpu(ws))
    yb = _np(y.view(torch.int16)).view(np.uint16)
    rows = np.array([mt * 128 + r for mt in range(M // 128) for r in (0, 61, 127)])
    Y, B = gemm_reference(ac[rows], as_[rows], wc, ws)
    assert_gemm_close(yb[rows], Y, B, K)


def test_gemm_full_size_sampled_rows(torch_cuda):
    """4608 x 12288 x 3072, the FLUX attention-projection consumer: quantizer
    output times prepared weights; 24 sampled rows checked against the fp64
    product of the dequantised operands."""
    torch = torch_cuda
    x = inputs.activation("flux_attn")
    lu = inputs.lu_params("flux_attn")
    w = inputs.gemm_weight()
    xd, lud = to_gpu_bf16(x), to_gpu(lu)
    ac, as_ = kq.transform_quant(xd, lud)
    wc, ws = kq.weight_quant(to_gpu_bf16(w), lud)
    y = kq.w4a4_gemm(ac, as_, wc, ws)
    yb = _np(y.view(torch.int16)).view(np.uint16)
    rows = np.sort(np.random.default_rng(9).choice(x.shape[0], 24, replace=False))
    acn, asn, wcn, wsn = _np(ac), _np(as_), _np(wc), _np(ws)
    Y, B = gemm_reference(acn[rows], asn[rows], wcn, wsn)
    assert_gemm_close(yb[rows], Y, B, x.shape[1])
    # end to end against the unquantised product X W^T on the sampled rows
    xf = inputs.bf16_bits_to_f32(x[rows]).astype(np.float64)
    wf = inputs.bf16_bits_to_f32(w).astype(np.float64)
    ref = xf @ wf.T
    got = inputs.bf16_bits_to_f32(yb[rows]).astype(np.float64)
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    _log(f"W4A4 end-to-end rel. error vs X W^T (KroQuant, random params): {rel:.4f}")
    assert rel < 0.5
    # the baselines through the same consumer: FWHT32 (H orthonormal and
    # symmetric, so the weights take W H as well) and per-channel scaling
    # (weights W diag(1/mult)); all on the GPU with the library's kernels
    wd = to_gpu_bf16(w)
    fa = kq.fwht32_quant(xd)
    fw = kq.fwht32_quant(wd)
    mult = inputs.smooth_multipliers(x)
    sa = kq.smooth_quant(xd, to_gpu(mult))
    sw = kq.smooth_quant(wd, to_gpu((1.0 / mult.astype(np.float64)).astype(np.float32)))
    errs = {}
    for name, (a_, w_) in {"fwht32": (fa, fw), "smooth": (sa, sw)}.items():
        yy = kq.w4a4_gemm(a_[0], a_[1], w_[0], w_[1])
        gy = inputs.bf16_bits_to_f32(_np(yy.view(torch.int16)).view(np.uint16)[rows]).astype(np.float64)
        errs[name] = np.linalg.norm(gy - ref) / np.linalg.norm(ref)
    # the Kronecker transform with parameters calibrated on 256 other rows
    cal_rows = np.setdiff1d(np.arange(256), rows)[:256]
    theta, _, _ = kq.calibrate(to_gpu_bf16(x[cal_rows]), to_gpu(inputs.hadamard_init(96)),
                               to_gpu(inputs.calib_noise("flux_attn", 150)))
    ca = kq.transform_quant(xd, theta)
    cw = kq.weight_quant(wd, theta)
    yy = kq.w4a4_gemm(ca[0], ca[1], cw[0], cw[1])
    gy = inputs.bf16_bits_to_f32(_np(yy.view(torch.int16)).view(np.uint16)[rows]).astype(np.float64)
    errs["kron_calibrated"] = np.linalg.norm(gy - ref) / np.linalg.norm(ref)
    _log("W4A4 end-to-end rel. error vs X W^T: " +
         ", ".join(f"{k} {v:.4f}" for k, v in errs.items()))
    assert all(v < 0.5 for v in errs.values())


# --------------------------------------------------------------------------
# the 256 x 256-tile kernel: problems with K a multiple of 256 and at least
# two such tiles per compute unit (a 4608 x 12288 output and larger) take it;
# scales come in chunks of four K tiles of 256
# --------------------------------------------------------------------------
@pytest.mark.parametrize("M,N,K,pad", [(4096, 8192, 768, 0),    # two full rounds on 256 CUs
                                       (5100, 8192, 512, 8),    # last round half full
                                       (4100, 8200, 1280, 0),   # ragged tiles, 5 K tiles of 256
                                       (4097, 8193, 256, 24),   # one K tile, strided output
                                       (4160, 8448, 512, 0),    # two K tiles
                                       (4352, 8192, 768, 8),    # three K tiles
                                       (4160, 8200, 1024, 8),   # one scale chunk exactly
                                       (4096, 9000, 2304, 0),   # nine K tiles, a partial chunk
                                       (4608, 12288, 3072, 0),
                                       # K % 256 == 128: the 128 x 256-tile kernels
                                       (4100, 8200, 1152, 0),
                                       (4097, 8200, 128, 0)])
def test_gemm_wide_tiles_random_mxfp4(torch_cuda, M, N, K, pad):
    torch = torch_cuda
    g = np.random.default_rng(M + N + K)
    ac, as_ = _random_mxfp4(g, M, K)
    wc, ws = _random_mxfp4(g, N, K)
    # scale arrays placed 4 bytes past a 16-byte boundary (the ABI's minimum)
    asb = torch.empty(as_.size + 16, dtype=torch.uint8, device="cuda:0")
    wsb = torch.empty(ws.size + 16, dtype=torch.uint8, device="cuda:0")
    asd = asb[4:4 + as_.size].view(M, K // 32)
    wsd = wsb[4:4 + ws.size].view(N, K // 32)
    asd.copy_(torch.from_numpy(as_))
    wsd.copy_(torch.from_numpy(ws))
    ld = (N + 7) // 8 * 8 + pad  # rows 16-byte aligned
    ybuf = torch.full((M, ld), -7.0, dtype=torch.bfloat16, device="cuda:0")
    y = ybuf[:, :N]
    kq.w4a4_gemm(to_gpu(ac), asd, to_gpu(wc), wsd, y=y)
    yb = _np(ybuf.view(torch.int16)).view(np.uint16)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, M - 2, M - 1],
                                     np.random.default_rng(5).choice(M, 6, replace=False)]))
    _log(f"wide GEMM {M}x{N}x{K}: oracle on {len(rows)} rows")
    Y, B = gemm_reference(ac[rows], as_[rows], wc, ws)
    assert_gemm_close(yb[rows, :N], Y, B, K)
    if ld > N:
        assert (inputs.bf16_bits_to_f32(yb[:, N:]) == -7.0).all()


@pytest.mark.gpu
def test_gemm_kernels_agree_bit_for_bit(torch_cuda):
    # One 4608 x 12288 x 3072 call takes the 256 x 256-tile kernel.  The same
    # rows computed by calls too small for it take the pipelined kernel
    # (16-byte aligned scales) and the per-tile kernel (scales 4 bytes past a
    # 16-byte boundary); every kernel accumulates each output over K in the
    # same order, so all three must agree bit for bit.
    torch = torch_cuda
    M, N, K = 4608, 12288, 3072
    g = np.random.default_rng(11)
    ac, as_ = _random_mxfp4(g, M, K)
    wc, ws = _random_mxfp4(g, N, K)
    acd, asd, wcd, wsd = to_gpu(ac), to_gpu(as_), to_gpu(wc), to_gpu(ws)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    kq.w4a4_gemm(acd, asd, wcd, wsd, y=y)
    full = _np(y.view(torch.int16)).view(np.uint16)
    for r0, rows, offset in ((0, 256, 0), (2048, 200, 0), (4400, 208, 4)):
        sub_as = torch.empty(rows * (K // 32) + 16, dtype=torch.uint8, device="cuda:0")
        sub_as = sub_as[offset:offset + rows * (K // 32)].view(rows, K // 32)
        sub_as.copy_(asd[r0:r0 + rows])
        ys = torch.empty((rows, N), dtype=torch.bfloat16, device="cuda:0")
        kq.w4a4_gemm(acd[r0:r0 + rows], sub_as, wcd, wsd, y=ys)
        part = _np(ys.view(torch.int16)).view(np.uint16)
        _log(f"GEMM rows {r0}..{r0 + rows - 1}, scales offset {offset}: "
             f"{int((part != full[r0:r0 + rows]).sum())} outputs differ")
        assert np.array_equal(part, full[r0:r0 + rows])


@pytest.mark.gpu
@pytest.mark.parametrize("M,N,K,rows", [(96, 80, 512, None),        # 128 x 256-tile kernels
                                        (4096, 8192, 512, (0, 17, 2049, 4095))])  # 256 x 256
def test_gemm_wide_scale_range_and_nan_blocks(torch_cuda, M, N, K, rows):
    # Scale bytes over a wide range (products from about 2^-124 to 2^120, no
    # fp32 overflow), plus one activation block and one weight block whose
    # scale byte is 0xFF: in the MX definition that block is NaN, so its
    # whole output row (activation) or column (weight) is NaN, and no other
    # output is.
    torch = torch_cuda
    g = np.random.default_rng(M + K)
    ac, as_ = _random_mxfp4(g, M, K, 60, 181)
    wc, ws = _random_mxfp4(g, N, K, 70, 181)
    r_nan, c_nan = 17 % M, (N // 2 + 3) % N
    as_[r_nan, 3] = 0xFF
    ac[r_nan, 3 * 16:4 * 16] = 0
    ws[c_nan, 0] = 0xFF
    wc[c_nan, 0:16] = 0
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    kq.w4a4_gemm(to_gpu(ac), to_gpu(as_), to_gpu(wc), to_gpu(ws), y=y)
    yb = _np(y.view(torch.int16)).view(np.uint16)
    sel = np.arange(M) if rows is None else np.unique(np.array(rows + (r_nan,)) % M)
    Y, B = gemm_reference(ac[sel], as_[sel], wc, ws)
    yf = inputs.bf16_bits_to_f32(yb[sel]).astype(np.float64)
    nan_ref = np.isnan(Y)
    assert nan_ref[sel == r_nan].all() and nan_ref[:, c_nan].all()
    assert nan_ref.sum() == N * int((sel == r_nan).sum()) + len(sel) - int((sel == r_nan).sum())
    np.testing.assert_array_equal(np.isnan(yf), nan_ref)
    keep = np.arange(N) != c_nan
    finite = sel != r_nan
    assert_gemm_close(yb[sel][np.ix_(finite, keep)], Y[np.ix_(finite, keep)],
                      B[np.ix_(finite, keep)], K)

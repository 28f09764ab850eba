// kq_quant.hip — gfx950 kernels of the online KroQuant quantizer and its
// per-channel-scaling and FWHT32 baselines, plus the C ABI that launches them.
//
// Work decomposition.  One lane owns one unit = (token t, 32-channel block j):
// 64 contiguous bytes of bf16 input, 16 bytes of E2M1 codes and one E8M0
// byte of output.  Holding the whole block in one lane keeps all five
// butterfly stages in registers with no cross-lane traffic, and makes every
// wave-wide load/store instruction cover 64 consecutive units (4 KB of input,
// 1 KB of codes, 64 B of scales per wave and unit-step).
//
// The grid is sized so that the total lane count L is a multiple of the
// number of blocks per row nb.  Lane g then handles units g, g + L, g + 2L,
// ... which all belong to block j = g mod nb: the per-block constants (five
// shears and the 32-entry diagonal) are derived once per lane and stay in
// VGPRs, and consecutive units of a lane are tstep = L / nb tokens apart.
// Each lane issues the loads of all its units before computing any of them,
// so several 64-byte requests per lane overlap the arithmetic.

#include <stdint.h>
#include <stdlib.h>

#include <type_traits>

#include <hip/hip_runtime.h>

#include "kq.h"
#include "kq_device.h"
#include "kq_host.h"
#include "kq_kron.h"

namespace kq {

constexpr int kBlockThreads = 256;  // 4 waves of 64 lanes

// ---------------------------------------------------------------------------
// Sources: where a unit's 32 input values come from.
// ---------------------------------------------------------------------------
struct Bf16Src {
    const uint16_t *x;
    int64_t ld;  // row stride, elements
    struct Raw { u32x4 v[4]; };
    __device__ __forceinline__ void load(int t, int j, Raw &r) const {
        const u32x4 *p = reinterpret_cast<const u32x4 *>(x + (int64_t)t * ld + (int64_t)j * 32);
#pragma unroll
        for (int i = 0; i < 4; ++i) r.v[i] = p[i];
    }
    __device__ __forceinline__ static void unpack(const Raw &r, float (&z)[32]) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                z[8 * i + 2 * c] = bf16_lo(r.v[i][c]);
                z[8 * i + 2 * c + 1] = bf16_hi(r.v[i][c]);
            }
    }
};

struct F32Src {
    const float *y;
    int64_t ld;
    struct Raw { f32x4 v[8]; };
    __device__ __forceinline__ void load(int t, int j, Raw &r) const {
        const f32x4 *p = reinterpret_cast<const f32x4 *>(y + (int64_t)t * ld + (int64_t)j * 32);
#pragma unroll
        for (int i = 0; i < 8; ++i) r.v[i] = p[i];
    }
    __device__ __forceinline__ static void unpack(const Raw &r, float (&z)[32]) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int c = 0; c < 4; ++c) z[4 * i + c] = r.v[i][c];
    }
};

// MXFP4 input (the inverse side): 16 code bytes + 1 scale byte per unit,
// decoded by the gfx950 scaled convert (code value times 2^(s-127)); a NaN
// scale byte makes the whole block NaN.
struct Mxfp4Src {
    const uint8_t *codes;   // [tokens][d/2]
    const uint8_t *scales;  // [tokens][nb]
    int nb;
    struct Raw { u32x4 c; uint32_t s; };
    __device__ __forceinline__ void load(int t, int j, Raw &r) const {
        const int64_t unit = (int64_t)t * nb + j;
        r.c = reinterpret_cast<const u32x4 *>(codes)[unit];
        r.s = scales[unit];
    }
    __device__ __forceinline__ static void unpack(const Raw &r, float (&z)[32]) {
        mxfp4_decode(r.c, r.s, z);
    }
};

// ---------------------------------------------------------------------------
// Transform stages.
// ---------------------------------------------------------------------------

// Weight side of the invariance (X T)(W T^-T)^T = X W^T (LRQ-DiT Sec. 3.2
// Eq. (2) with an invertible T; KroQuant abstract: the inverse goes to the
// weights).  T^-T = (G_4^-T (x)...(x) G_0^-T)(D_4 (x)...(x) D_0)^-1 with
// G^-T = [[1,-l],[0,1]] [[1,0],[-w,1]]: each pair (p, q) on bit b = 0..4 maps
// to s = q - l*p, r = p - w*s, then every element is multiplied by e_k.
struct KronWeightStage : KronInvConsts {
    __device__ __forceinline__ static KronWeightStage from(const float *p) {
        KronWeightStage s;
        s.lu = p;
        return s;
    }
    __device__ __forceinline__ void apply(float (&z)[32]) const {
#pragma unroll
        for (int b = 0; b < 5; ++b) {
            const int h = 1 << b;
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                if (i & h) continue;
                const float pv = z[i], q = z[i | h];
                const float s = __builtin_fmaf(-l[b], pv, q);
                const float r = __builtin_fmaf(-w[b], s, pv);
                z[i] = r;
                z[i | h] = s;
            }
        }
#pragma unroll
        for (int k = 0; k < 32; ++k) z[k] = z[k] * ek[k];
    }
};

// Per-channel scaling baseline: y_c = x_c * mult_c.  Lane l of a workgroup
// takes block (g0 + l) % nb, g0 the workgroup's first unit.  With
// nb <= kSmoothStageMax the workgroup's lanes share their blocks (each block
// at least twice), so the workgroup loads the nb blocks' multipliers once
// into LDS, in whole 16-byte chunks (consecutive threads, consecutive
// chunks), slot s = block (g0 % nb + s) % nb with chunk i at vec_chunk(s, i),
// and lane l reads slot l % nb.  Loaded lane by lane, each of a wave's eight
// 16-byte multiplier loads touches 64 cache lines.  With more blocks there is
// no reuse to win and the staging would only take LDS (and resident waves),
// so each lane loads its own 128 bytes.
extern __shared__ __attribute__((aligned(16))) f32x4 kq_stage_lds[];

constexpr int kSmoothStageMax = 128;  // 16 KB of LDS: seven workgroups per CU still fit

struct SmoothStage {
    static constexpr bool kShared = true;
    static constexpr int kUnitsPerLane = 4;
    const float *mult;  // [d]
    int nb;
    __device__ __forceinline__ static SmoothStage from(const float *p) {
        SmoothStage s;
        s.mult = p;
        return s;
    }
    // LDS bytes the workgroup stages for nb blocks
    static int64_t shared_bytes(int nb) { return nb <= kSmoothStageMax ? (int64_t)nb * 128 : 0; }
    // every thread of the workgroup, before any of them leaves
    __device__ __forceinline__ void share(int g0, int nblocks) {
        nb = nblocks;
        if (nb > kSmoothStageMax) return;
        const int j0 = g0 % nb;
        const f32x4 *src = reinterpret_cast<const f32x4 *>(mult);
        for (int f = threadIdx.x; f < nb * 8; f += kBlockThreads) {
            const int sl = f >> 3, i = f & 7;
            const int j = j0 + sl < nb ? j0 + sl : j0 + sl - nb;
            kq_stage_lds[vec_chunk(sl, i)] = src[(int64_t)j * 8 + i];
        }
        __syncthreads();
    }
    float m[32];
    __device__ __forceinline__ void fetch(int j) {
        if (nb <= kSmoothStageMax) {
            const int sl = (int)(threadIdx.x % (unsigned)nb);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const f32x4 v = kq_stage_lds[vec_chunk(sl, i)];
#pragma unroll
                for (int c = 0; c < 4; ++c) m[4 * i + c] = v[c];
            }
        } else {
            const f32x4 *p = reinterpret_cast<const f32x4 *>(mult + (int64_t)j * 32);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const f32x4 v = p[i];
#pragma unroll
                for (int c = 0; c < 4; ++c) m[4 * i + c] = v[c];
            }
        }
    }
    __device__ __forceinline__ void setup() {}
    __device__ __forceinline__ void apply(float (&z)[32]) const {
#pragma unroll
        for (int k = 0; k < 32; ++k) z[k] = z[k] * m[k];
    }
};

// Stages that stage per-workgroup data in LDS declare kShared = true and
// provide share() and shared_bytes(); the others need neither.
template <class S, class = void>
struct stage_shares : std::false_type {};
template <class S>
struct stage_shares<S, std::void_t<decltype(S::kShared)>> : std::bool_constant<S::kShared> {};

// Orthonormal 32-point Walsh-Hadamard (Sylvester order, LRQ-DiT Eq. (3)):
// five add/subtract stages, then one multiply by fl32(1/sqrt(32)).
struct FwhtStage {
    __device__ __forceinline__ static FwhtStage from(const float *) { return FwhtStage{}; }
    __device__ __forceinline__ void fetch(int) {}
    __device__ __forceinline__ void setup() {}
    __device__ __forceinline__ void apply(float (&z)[32]) const {
#pragma unroll
        for (int b = 0; b < 5; ++b) {
            const int h = 1 << b;
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                if (i & h) continue;
                const float p = z[i], q = z[i | h];
                z[i] = p + q;
                z[i | h] = p - q;
            }
        }
        const float c = 0x1.6a09e6p-3f;  // 1/sqrt(32) rounded to fp32
#pragma unroll
        for (int k = 0; k < 32; ++k) z[k] = z[k] * c;
    }
};

struct IdentityStage {
    __device__ __forceinline__ static IdentityStage from(const float *) { return IdentityStage{}; }
    __device__ __forceinline__ void fetch(int) {}
    __device__ __forceinline__ void setup() {}
    __device__ __forceinline__ void apply(float (&)[32]) const {}
};

// ---------------------------------------------------------------------------
// Sinks: what is stored per unit.
// ---------------------------------------------------------------------------
struct Mxfp4Sink {
    static constexpr bool kWave = false;
    uint8_t *codes;   // [tokens][d/2]
    uint8_t *scales;  // [tokens][nb]
    int nb;
    __device__ __forceinline__ void store(int t, int j, const float (&y)[32]) const {
        u32x4 c;
        uint32_t s;
        mxfp4_block(y, c, s);
        const int64_t unit = (int64_t)t * nb + j;
        __builtin_nontemporal_store(c, reinterpret_cast<u32x4 *>(codes) + unit);
        __builtin_nontemporal_store((uint8_t)s, scales + unit);
    }
};

// bf16 output, rounded to nearest even by the hardware pack-convert, and
// stored whole-line through the wave exchange (kWave: every lane of a wave
// calls store, lanes without a unit with valid == false).
struct Bf16Sink {
    static constexpr bool kWave = true;
    uint16_t *x;  // [tokens][ld]
    int64_t ld;
    __device__ __forceinline__ void store(int t, int j, const float (&z)[32], bool valid) const {
        __shared__ WaveStoreBuf<1> buf[kBlockThreads / 64];
        uint32_t w[16];
#pragma unroll
        for (int m = 0; m < 16; ++m)
            w[m] = __builtin_bit_cast(uint32_t,
                                      __builtin_convertvector(f32x2{z[2 * m], z[2 * m + 1]}, bf16x2));
        wave_store64(buf[threadIdx.x >> 6], w,
                     valid ? (void *)(x + (int64_t)t * ld + (int64_t)j * 32) : nullptr);
    }
};

struct F32Sink {
    static constexpr bool kWave = false;
    float *y;  // [tokens][d]
    int64_t d;
    __device__ __forceinline__ void store(int t, int j, const float (&z)[32]) const {
        f32x4 *p = reinterpret_cast<f32x4 *>(y + (int64_t)t * d + (int64_t)j * 32);
#pragma unroll
        for (int i = 0; i < 8; ++i) p[i] = f32x4{z[4 * i], z[4 * i + 1], z[4 * i + 2], z[4 * i + 3]};
    }
};

// Same-traffic ceiling: no transform and no quantizer; the 16 code bytes are
// the XOR of the unit's fp32 bit patterns eight at a time, the scale byte the
// low byte of their XOR.  Same loads, same stores, almost no arithmetic.
struct FoldSink {
    static constexpr bool kWave = false;
    uint8_t *codes;
    uint8_t *scales;
    int nb;
    __device__ __forceinline__ void store(int t, int j, const float (&z)[32]) const {
        uint32_t c[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint32_t f = 0;
#pragma unroll
            for (int k = 0; k < 8; ++k) f ^= __float_as_uint(z[8 * q + k]);
            c[q] = f;
        }
        const int64_t unit = (int64_t)t * nb + j;
        __builtin_nontemporal_store(u32x4{c[0], c[1], c[2], c[3]}, reinterpret_cast<u32x4 *>(codes) + unit);
        __builtin_nontemporal_store((uint8_t)(c[0] ^ c[1] ^ c[2] ^ c[3]), scales + unit);
    }
};

// ---------------------------------------------------------------------------
// The kernel template.
//
// A lane owns up to NU units of block j, tstep tokens apart (units g, g + L,
// ... of the flattened unit index, L the grid's lane count).  It issues the
// loads of all its units first, then unpacks, transforms, quantizes and stores
// them in order, each as soon as its own data has arrived: the code is
// straight-line, so the compiler's memory wait before unit k counts exactly
// the requests issued after it, and the arithmetic of unit k overlaps the
// flight of units k+1.. and the loads of other waves.  Lanes past the end
// repeat their last unit (same bytes to the same place), so no lane branches.
// ---------------------------------------------------------------------------
template <class Src, class Stage, class Sink, int NU>
__global__ __launch_bounds__(kBlockThreads) void block_kernel(Src src, const float *stage_param,
                                                              Sink sink,
                                                              int tokens, int nb, DivMagic nbm,
                                                              int tstep) {
    Stage stage = Stage::from(stage_param);
    if constexpr (stage_shares<Stage>::value) stage.share(blockIdx.x * kBlockThreads, nb);
    const int g = blockIdx.x * kBlockThreads + threadIdx.x;
    int t0 = (int)udiv31((uint32_t)g, nbm);
    const int j = g - t0 * nb;
    bool valid = true;
    if constexpr (Sink::kWave) {
        // the wave stores together: only a wave wholly past the end leaves;
        // its other lanes past the end redo the last row's unit and store
        // nothing
        if ((int)udiv31((uint32_t)(g & ~63), nbm) >= tokens) return;
        if (t0 >= tokens) {
            valid = false;
            t0 = tokens - 1;
        }
    } else {
        if (t0 >= tokens) return;
    }
    auto put = [&](int t, const float (&z)[32]) {
        if constexpr (Sink::kWave) sink.store(t, j, z, valid);
        else sink.store(t, j, z);
    };
    if constexpr (NU == 1) {
        // one unit per lane: no unit count or clamping (saves an integer
        // division per lane)
        stage.fetch(j);
        typename Src::Raw r;
        src.load(t0, j, r);
        __builtin_amdgcn_sched_barrier(0);
        // the whole per-block set-up before the first use of the data, so it
        // runs while the loads are in flight (left free, the compiler sank
        // most of it below the data wait: 3.6-4.3 % slower on 4608 x 12288,
        // the same on 4608 x 3072 and 8192 x 1152)
        stage.setup();
        __builtin_amdgcn_sched_barrier(0);
        float z[32];
        Src::unpack(r, z);
        stage.apply(z);
        put(t0, z);
        return;
    }
    const int avail = (tokens - 1 - t0) / tstep + 1;
    const int cnt = avail < NU ? avail : NU;
    const int last = t0 + (cnt - 1) * tstep;
    // Parameter loads first, then every data load; the scheduling barrier
    // keeps all of them ahead of the arithmetic (left alone, the scheduler
    // sinks later units' loads below earlier units' math to save registers).
    stage.fetch(j);
    typename Src::Raw buf[NU];
#pragma unroll
    for (int k = 0; k < NU; ++k) src.load(k < cnt ? t0 + k * tstep : last, j, buf[k]);
    __builtin_amdgcn_sched_barrier(0);
    stage.setup();
#pragma unroll
    for (int k = 0; k < NU; ++k) {
        float z[32];
        Src::unpack(buf[k], z);
        stage.apply(z);
        put(k < cnt ? t0 + k * tstep : last, z);
    }
}

// ---------------------------------------------------------------------------
// Host side: validation and launch geometry.
// ---------------------------------------------------------------------------
static int gcd_int(int a, int b) {
    while (b) {
        int r = a % b;
        a = b;
        b = r;
    }
    return a;
}

struct Plan {
    int nu;     // units per lane (a compiled instantiation: 1, 2, 4 or 8)
    int grid;   // workgroups
    int tstep;  // tokens between consecutive units of a lane
};

// Units per lane: one unless the stage asks for more (kUnitsPerLane).  More
// units per lane amortise the per-block constant setup (fewer VALU
// instructions per unit) but leave fewer waves.  For the Kronecker stage one
// unit per lane measured fastest: 3-8 % faster than 2, 4 or 8 on 4608 x 3072
// (all 6912 waves resident at once), 8-25 % on 8192 x 1152, and still 3 %
// faster than two per lane on 4608 x 12288, where one per lane takes about
// four rounds of waves.  The scaling stage's 128 bytes of multipliers per
// block make four per lane its better choice: 29.2 against 38.7 us on
// 4608 x 12288, equal (8.8 us) on 4608 x 3072.
// Building with -DKQ_UNITS_PER_LANE=1, 2, 4 or 8 overrides it for sweeps.
#ifndef KQ_UNITS_PER_LANE
#define KQ_UNITS_PER_LANE 0
#endif
static_assert(KQ_UNITS_PER_LANE == 0 || KQ_UNITS_PER_LANE == 1 || KQ_UNITS_PER_LANE == 2 ||
                  KQ_UNITS_PER_LANE == 4 || KQ_UNITS_PER_LANE == 8,
              "KQ_UNITS_PER_LANE must be 1, 2, 4 or 8");

template <class S, class = void>
struct stage_units : std::integral_constant<int, 1> {};
template <class S>
struct stage_units<S, std::void_t<decltype(S::kUnitsPerLane)>>
    : std::integral_constant<int, S::kUnitsPerLane> {};

static int units_per_lane(int stage_default) {
    return KQ_UNITS_PER_LANE ? KQ_UNITS_PER_LANE : stage_default;
}

static bool plan_launch(int64_t tokens, int nb, int nu, Plan &pl) {
    // The lane count must be a multiple of nb (so a lane keeps one block):
    // the grid is a multiple of m = nb / gcd(nb, threads per workgroup).
    const int64_t m = nb / gcd_int(nb, kBlockThreads);
    const int64_t units = tokens * nb;
    pl.nu = nu;
    const int64_t per_wg = (int64_t)kBlockThreads * pl.nu;
    int64_t grid = (units + per_wg - 1) / per_wg;
    grid = (grid + m - 1) / m * m;
    if (grid < m) grid = m;
    if (grid > INT32_MAX / kBlockThreads) return false;
    pl.grid = (int)grid;
    pl.tstep = (int)(grid * kBlockThreads / nb);
    return true;
}

static bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// Shape checks common to every activation-consuming entry point.
static kq_status check_shape(int64_t tokens, int64_t d, int64_t ld) {
    if (tokens < 0 || tokens >= (int64_t(1) << 30)) return KQ_ERR_SHAPE;
    if (d <= 0 || d % 32 != 0 || d > (int64_t(1) << 26)) return KQ_ERR_SHAPE;
    if (ld < d) return KQ_ERR_SHAPE;
    return KQ_OK;
}

template <class Kernel, class... Args>
static kq_status launch(Kernel kernel, const Plan &pl, size_t shmem, void *stream, Args... args) {
    void *argv[] = {(void *)&args...};
    hipError_t e = hipLaunchKernel((const void *)kernel, dim3(pl.grid), dim3(kBlockThreads), argv,
                                   shmem, (hipStream_t)stream);
    return e == hipSuccess ? KQ_OK : KQ_ERR_HIP;
}

template <class Src, class Stage, class Sink>
static kq_status run(const Src &src, const float *stage, const Sink &sink, int64_t tokens, int nb,
                     void *stream) {
    Plan pl;
    if (!plan_launch(tokens, nb, units_per_lane(stage_units<Stage>::value), pl)) return KQ_ERR_SHAPE;
    const int t = (int)tokens;
    const DivMagic nbm = div_magic((uint32_t)nb);
    size_t sh = 0;
    if constexpr (stage_shares<Stage>::value) sh = (size_t)Stage::shared_bytes(nb);
    switch (pl.nu) {
        case 1: return launch(block_kernel<Src, Stage, Sink, 1>, pl, sh, stream, src, stage, sink, t, nb, nbm, pl.tstep);
        case 2: return launch(block_kernel<Src, Stage, Sink, 2>, pl, sh, stream, src, stage, sink, t, nb, nbm, pl.tstep);
        case 8: return launch(block_kernel<Src, Stage, Sink, 8>, pl, sh, stream, src, stage, sink, t, nb, nbm, pl.tstep);
        default: return launch(block_kernel<Src, Stage, Sink, 4>, pl, sh, stream, src, stage, sink, t, nb, nbm, pl.tstep);
    }
}

}  // namespace kq

using namespace kq;

extern "C" {

const char *kq_status_str(int status) {
    switch (status) {
        case KQ_OK: return "KQ_OK";
        case KQ_ERR_NULL: return "KQ_ERR_NULL: a required pointer is NULL";
        case KQ_ERR_SHAPE: return "KQ_ERR_SHAPE: invalid sizes or strides";
        case KQ_ERR_ALIGN: return "KQ_ERR_ALIGN: pointer or stride not aligned as required";
        case KQ_ERR_HIP: return "KQ_ERR_HIP: the HIP runtime rejected the launch";
        default: return "unknown kq_status";
    }
}

int kq_version(void) { return 100; }

// Common front end of the bf16-activation entry points.
static kq_status check_bf16_act(const void *x, int64_t tokens, int64_t d, int64_t ld_x) {
    kq_status st = check_shape(tokens, d, ld_x);
    if (st != KQ_OK) return st;
    if (tokens == 0) return KQ_OK;
    if (!x) return KQ_ERR_NULL;
    if (!aligned(x, 16) || (ld_x * 2) % 16 != 0) return KQ_ERR_ALIGN;
    return KQ_OK;
}

static kq_status check_mxfp4_out(const uint8_t *codes, const uint8_t *scales) {
    if (!codes || !scales) return KQ_ERR_NULL;
    if (!aligned(codes, 16)) return KQ_ERR_ALIGN;
    return KQ_OK;
}

kq_status kq_transform_quant(const void *x, int64_t tokens, int64_t d, int64_t ld_x,
                             const float *lu, uint8_t *codes, uint8_t *scales, void *stream) {
    kq_status st = check_bf16_act(x, tokens, d, ld_x);
    if (st != KQ_OK || tokens == 0) return st;
    if (!lu) return KQ_ERR_NULL;
    if ((st = check_mxfp4_out(codes, scales)) != KQ_OK) return st;
    if (!aligned(lu, 4)) return KQ_ERR_ALIGN;
    const int nb = (int)(d / 32);
    return run<Bf16Src, KronStage>(Bf16Src{(const uint16_t *)x, ld_x}, lu,
                                   Mxfp4Sink{codes, scales, nb}, tokens, nb, stream);
}

kq_status kq_transform_f32(const void *x, int64_t tokens, int64_t d, int64_t ld_x,
                           const float *lu, float *y, void *stream) {
    kq_status st = check_bf16_act(x, tokens, d, ld_x);
    if (st != KQ_OK || tokens == 0) return st;
    if (!lu || !y) return KQ_ERR_NULL;
    if (!aligned(lu, 4) || !aligned(y, 16)) return KQ_ERR_ALIGN;
    const int nb = (int)(d / 32);
    return run<Bf16Src, KronStage>(Bf16Src{(const uint16_t *)x, ld_x}, lu, F32Sink{y, d}, tokens,
                                   nb, stream);
}

kq_status kq_smooth_quant(const void *x, int64_t tokens, int64_t d, int64_t ld_x,
                          const float *mult, uint8_t *codes, uint8_t *scales, void *stream) {
    kq_status st = check_bf16_act(x, tokens, d, ld_x);
    if (st != KQ_OK || tokens == 0) return st;
    if (!mult) return KQ_ERR_NULL;
    if ((st = check_mxfp4_out(codes, scales)) != KQ_OK) return st;
    if (!aligned(mult, 16)) return KQ_ERR_ALIGN;
    const int nb = (int)(d / 32);
    return run<Bf16Src, SmoothStage>(Bf16Src{(const uint16_t *)x, ld_x}, mult,
               Mxfp4Sink{codes, scales, nb}, tokens, nb, stream);
}

kq_status kq_fwht32_quant(const void *x, int64_t tokens, int64_t d, int64_t ld_x,
                          uint8_t *codes, uint8_t *scales, void *stream) {
    kq_status st = check_bf16_act(x, tokens, d, ld_x);
    if (st != KQ_OK || tokens == 0) return st;
    if ((st = check_mxfp4_out(codes, scales)) != KQ_OK) return st;
    const int nb = (int)(d / 32);
    return run<Bf16Src, FwhtStage>(Bf16Src{(const uint16_t *)x, ld_x}, nullptr, Mxfp4Sink{codes, scales, nb},
               tokens, nb, stream);
}

kq_status kq_mxfp4_quant_f32(const float *y, int64_t tokens, int64_t d, int64_t ld_y,
                             uint8_t *codes, uint8_t *scales, void *stream) {
    kq_status st = check_shape(tokens, d, ld_y);
    if (st != KQ_OK || tokens == 0) return st;
    if (!y) return KQ_ERR_NULL;
    if ((st = check_mxfp4_out(codes, scales)) != KQ_OK) return st;
    if (!aligned(y, 16) || (ld_y * 4) % 16 != 0) return KQ_ERR_ALIGN;
    const int nb = (int)(d / 32);
    return run<F32Src, IdentityStage>(F32Src{y, ld_y}, nullptr, Mxfp4Sink{codes, scales, nb}, tokens,
                                      nb, stream);
}

kq_status kq_weight_quant(const void *w, int64_t rows, int64_t k, int64_t ld_w,
                          const float *lu, uint8_t *codes, uint8_t *scales, void *stream) {
    kq_status st = check_bf16_act(w, rows, k, ld_w);
    if (st != KQ_OK || rows == 0) return st;
    if (!lu) return KQ_ERR_NULL;
    if ((st = check_mxfp4_out(codes, scales)) != KQ_OK) return st;
    if (!aligned(lu, 4)) return KQ_ERR_ALIGN;
    const int nb = (int)(k / 32);
    return run<Bf16Src, KronWeightStage>(Bf16Src{(const uint16_t *)w, ld_w}, lu,
                                         Mxfp4Sink{codes, scales, nb}, rows, nb, stream);
}

kq_status kq_dequant_inverse(const uint8_t *codes, const uint8_t *scales, int64_t tokens,
                             int64_t d, const float *lu, void *x_out, int64_t ld_out,
                             void *stream) {
    kq_status st = check_shape(tokens, d, ld_out);
    if (st != KQ_OK || tokens == 0) return st;
    if (!codes || !scales || !lu || !x_out) return KQ_ERR_NULL;
    if (!aligned(codes, 16) || !aligned(x_out, 16) || (ld_out * 2) % 16 != 0 || !aligned(lu, 4))
        return KQ_ERR_ALIGN;
    const int nb = (int)(d / 32);
    return run<Mxfp4Src, KronInverseStage>(Mxfp4Src{codes, scales, nb}, lu,
                                           Bf16Sink{(uint16_t *)x_out, ld_out}, tokens, nb, stream);
}

kq_status kq_copy_ceiling(const void *x, int64_t tokens, int64_t d, int64_t ld_x,
                          uint8_t *codes, uint8_t *scales, void *stream) {
    kq_status st = check_bf16_act(x, tokens, d, ld_x);
    if (st != KQ_OK || tokens == 0) return st;
    if ((st = check_mxfp4_out(codes, scales)) != KQ_OK) return st;
    const int nb = (int)(d / 32);
    return run<Bf16Src, IdentityStage>(Bf16Src{(const uint16_t *)x, ld_x}, nullptr, FoldSink{codes, scales, nb},
               tokens, nb, stream);
}

}  // extern "C"

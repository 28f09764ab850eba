// kq_gemm.hip — the W4A4 consumer: Y = dequant(A) * dequant(W)^T on the gfx950
// block-scaled matrix cores (v_mfma_scale_f32_32x32x64_f8f6f4 with E2M1
// operands and E8M0 scales), fp32 accumulation, bf16 output.
//
// A (activations, [M][K]) and W (weights, [N][K]) are both MXFP4 in the
// quantizer's layout: codes [rows][K/2] with element k in nibble k%2 of byte
// k/2, scales [rows][K/32].  For the 32x32x64 FP4 MFMA, lane l holds row l%32
// and the 32 elements 32*(l/32) .. +31 of a 64-wide K step: exactly one
// 16-byte chunk of a code row plus its one scale byte, so both operands load
// from the quantizer's output as is.  The accumulator holds
// C[8*(r/4) + 4*(l/32) + r%4][l%32] in register r.
//
// Tiling: a workgroup of WM x WN waves computes a (64 WM) x (64 WN) tile of Y,
// each wave 64 x 64 (2 x 2 MFMA tiles, 64 fp32 accumulators).  K advances in
// tiles of 128 (two MFMA steps) through double-buffered LDS: the next tile's
// global loads are issued before the current tile's MFMAs and written to the
// other buffer after them.  Code rows sit in LDS as four 16-byte chunks with
// the chunk index XORed by (row >> 1) & 3, so the 32 lanes reading one chunk
// column of 32 consecutive rows hit distinct banks.  Results go straight from
// the accumulators to memory as bf16 (nearest even), 64 contiguous bytes per
// half-wave and accumulator register.
//
// The workgroup order is remapped so that each XCD (workgroups go to the 8
// XCDs round-robin) works on a compact group of M tiles and sweeps the N
// tiles, which keeps the A rows it shares in its own L2.

#include <stdint.h>
#include <stdlib.h>

#include <hip/hip_runtime.h>

#include "kq.h"
#include "kq_device.h"

namespace kq {

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16g __attribute__((ext_vector_type(16)));

constexpr int kBK = 128;          // K elements per LDS tile
constexpr int kRowBytes = kBK / 2;  // 64 code bytes per row per K tile

__device__ __forceinline__ int swz_chunk(int row, int c) { return c ^ ((row >> 1) & 3); }

template <int WM, int WN>
struct GemmShape {
    static constexpr int BM = 64 * WM, BN = 64 * WN;
    static constexpr int THREADS = 64 * WM * WN;
    static constexpr int A_BYTES = BM * kRowBytes, B_BYTES = BN * kRowBytes;
    static constexpr int STAGE = A_BYTES + B_BYTES + 4 * (BM + BN);  // codes + scale words
    static constexpr int LDS = 2 * STAGE;
};

template <int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN) void w4a4_gemm_kernel(
    const uint8_t *__restrict__ ac, const uint8_t *__restrict__ as,
    const uint8_t *__restrict__ wc, const uint8_t *__restrict__ ws, uint16_t *__restrict__ y,
    int M, int N, int K, int64_t ldy, int mt_count, int nt_count) {
    using S = GemmShape<WM, WN>;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    // ---- workgroup -> (M tile, N tile), XCD-aware ----
    const int tiles = mt_count * nt_count;
    const int b = blockIdx.x;
    const int per_xcd = (tiles + 7) / 8;
    const int lin = (b % 8) * per_xcd + b / 8;  // XCD x takes a contiguous range
    if (lin >= tiles) return;
    const int mt = lin / nt_count, nt = lin % nt_count;
    const int m0 = mt * S::BM, n0 = nt * S::BN;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int wm = wave / WN, wn = wave % WN;
    const int i32 = lane & 31, kg = lane >> 5;
    const int64_t K2 = K / 2, K32 = K / 32;
    const int KT = K / kBK;

    // ---- global -> register staging of one K tile ----
    constexpr int A_CHUNKS = S::BM * 4, B_CHUNKS = S::BN * 4;  // 16-byte chunks
    constexpr int A_PER = (A_CHUNKS + S::THREADS - 1) / S::THREADS;
    constexpr int B_PER = (B_CHUNKS + S::THREADS - 1) / S::THREADS;
    u32x4 ra[A_PER], rb[B_PER];
    uint32_t rsa = 0, rsb = 0;

    auto load_tile = [&](int kt) {
#pragma unroll
        for (int q = 0; q < A_PER; ++q) {
            const int c = tid + q * S::THREADS;
            if (c < A_CHUNKS) {
                int row = m0 + (c >> 2);
                row = row < M ? row : M - 1;
                ra[q] = *reinterpret_cast<const u32x4 *>(ac + row * K2 + (int64_t)kt * kRowBytes + 16 * (c & 3));
            }
        }
#pragma unroll
        for (int q = 0; q < B_PER; ++q) {
            const int c = tid + q * S::THREADS;
            if (c < B_CHUNKS) {
                int row = n0 + (c >> 2);
                row = row < N ? row : N - 1;
                rb[q] = *reinterpret_cast<const u32x4 *>(wc + row * K2 + (int64_t)kt * kRowBytes + 16 * (c & 3));
            }
        }
        if (tid < S::BM) {
            int row = m0 + tid;
            row = row < M ? row : M - 1;
            rsa = *reinterpret_cast<const uint32_t *>(as + row * K32 + (int64_t)kt * 4);
        }
        if (tid < S::BN) {
            int row = n0 + tid;
            row = row < N ? row : N - 1;
            rsb = *reinterpret_cast<const uint32_t *>(ws + row * K32 + (int64_t)kt * 4);
        }
    };
    auto store_tile = [&](int buf) {
        uint8_t *base = lds + buf * S::STAGE;
#pragma unroll
        for (int q = 0; q < A_PER; ++q) {
            const int c = tid + q * S::THREADS;
            if (c < A_CHUNKS) {
                const int row = c >> 2;
                *reinterpret_cast<u32x4 *>(base + row * kRowBytes + 16 * swz_chunk(row, c & 3)) = ra[q];
            }
        }
#pragma unroll
        for (int q = 0; q < B_PER; ++q) {
            const int c = tid + q * S::THREADS;
            if (c < B_CHUNKS) {
                const int row = c >> 2;
                *reinterpret_cast<u32x4 *>(base + S::A_BYTES + row * kRowBytes + 16 * swz_chunk(row, c & 3)) = rb[q];
            }
        }
        uint32_t *sw = reinterpret_cast<uint32_t *>(base + S::A_BYTES + S::B_BYTES);
        if (tid < S::BM) sw[tid] = rsa;
        if (tid < S::BN) sw[S::BM + tid] = rsb;
    };

    f32x16g acc[2][2];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int c = 0; c < 2; ++c) acc[r][c] = f32x16g{};

    load_tile(0);
    store_tile(0);
    __syncthreads();

    for (int kt = 0; kt < KT; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < KT) load_tile(kt + 1);
        const uint8_t *base = lds + buf * S::STAGE;
        const uint32_t *sw = reinterpret_cast<const uint32_t *>(base + S::A_BYTES + S::B_BYTES);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int chunk = 2 * ks + kg;  // this lane's 16-byte chunk of the 64-byte row
            i32x8 fa[2], fb[2];
            int sa[2], sb[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int ar = wm * 64 + t * 32 + i32;
                const u32x4 va = *reinterpret_cast<const u32x4 *>(base + ar * kRowBytes + 16 * swz_chunk(ar, chunk));
                fa[t] = i32x8{(int)va[0], (int)va[1], (int)va[2], (int)va[3], 0, 0, 0, 0};
                sa[t] = (int)(sw[ar] >> (8 * chunk));
                const int br = wn * 64 + t * 32 + i32;
                const u32x4 vb = *reinterpret_cast<const u32x4 *>(base + S::A_BYTES + br * kRowBytes + 16 * swz_chunk(br, chunk));
                fb[t] = i32x8{(int)vb[0], (int)vb[1], (int)vb[2], (int)vb[3], 0, 0, 0, 0};
                sb[t] = (int)(sw[S::BM + br] >> (8 * chunk));
            }
#pragma unroll
            for (int r = 0; r < 2; ++r)
#pragma unroll
                for (int c = 0; c < 2; ++c)
                    acc[r][c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        fa[r], fb[c], acc[r][c], 4, 4, 0, sa[r], 0, sb[c]);
        }
        if (kt + 1 < KT) store_tile(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: bf16, rounded to nearest even; for each accumulator
    // register the 32 lanes of a half-wave write 64 contiguous bytes of a row ----
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int col = n0 + wn * 64 + c * 32 + i32;
#pragma unroll
            for (int q = 0; q < 16; q += 2) {
                const int row = m0 + wm * 64 + r * 32 + 8 * (q >> 2) + 4 * kg + (q & 3);
                const uint32_t h = __builtin_bit_cast(
                    uint32_t, __builtin_convertvector(f32x2{acc[r][c][q], acc[r][c][q + 1]}, bf16x2));
                if (col < N) {
                    if (row < M) y[(int64_t)row * ldy + col] = (uint16_t)(h & 0xffffu);
                    if (row + 1 < M) y[(int64_t)(row + 1) * ldy + col] = (uint16_t)(h >> 16);
                }
            }
        }
}

static int gemm_variant() {
    static int cached = 0;
    if (cached == 0) {
        int v = 24;
        const char *e = getenv("KQ_GEMM_WAVES");  // WM*10 + WN: 22, 24, 42 or 44
        if (e) {
            int q = atoi(e);
            if (q == 22 || q == 24 || q == 42 || q == 44) v = q;
        }
        cached = v;
    }
    return cached;
}

template <int WM, int WN>
static kq_status launch_gemm(const uint8_t *ac, const uint8_t *as, const uint8_t *wc,
                             const uint8_t *ws, uint16_t *y, int M, int N, int K, int64_t ldy,
                             void *stream) {
    using S = GemmShape<WM, WN>;
    const int mtc = (M + S::BM - 1) / S::BM, ntc = (N + S::BN - 1) / S::BN;
    const int tiles = mtc * ntc;
    const int grid = ((tiles + 7) / 8) * 8;
    void *args[] = {(void *)&ac, (void *)&as, (void *)&wc, (void *)&ws, (void *)&y, (void *)&M,
                    (void *)&N, (void *)&K, (void *)&ldy, (void *)&mtc, (void *)&ntc};
    const void *fn = (const void *)w4a4_gemm_kernel<WM, WN>;
    static bool attr_set = false;
    if (!attr_set) {
        if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, S::LDS) != hipSuccess)
            return KQ_ERR_HIP;
        attr_set = true;
    }
    hipError_t e = hipLaunchKernel(fn, dim3(grid), dim3(S::THREADS), args, S::LDS,
                                   (hipStream_t)stream);
    return e == hipSuccess ? KQ_OK : KQ_ERR_HIP;
}

}  // namespace kq

using namespace kq;

extern "C" kq_status kq_w4a4_gemm(const uint8_t *a_codes, const uint8_t *a_scales,
                                  const uint8_t *w_codes, const uint8_t *w_scales, int64_t M,
                                  int64_t N, int64_t K, void *y, int64_t ld_y, void *stream) {
    if (M < 0 || N < 0 || K < 0 || M >= (int64_t(1) << 30) || N >= (int64_t(1) << 30) ||
        K >= (int64_t(1) << 24) || K % kBK != 0 || ld_y < N)
        return KQ_ERR_SHAPE;
    if (M == 0 || N == 0) return KQ_OK;
    if (K == 0) return KQ_ERR_SHAPE;
    if (!a_codes || !a_scales || !w_codes || !w_scales || !y) return KQ_ERR_NULL;
    if (((uintptr_t)a_codes % 16) || ((uintptr_t)w_codes % 16) || ((uintptr_t)a_scales % 4) ||
        ((uintptr_t)w_scales % 4) || ((uintptr_t)y % 16) || (ld_y % 8))
        return KQ_ERR_ALIGN;
    const int m = (int)M, n = (int)N, k = (int)K;
    uint16_t *yp = (uint16_t *)y;
    switch (gemm_variant()) {
        case 22: return launch_gemm<2, 2>(a_codes, a_scales, w_codes, w_scales, yp, m, n, k, ld_y, stream);
        case 24: return launch_gemm<2, 4>(a_codes, a_scales, w_codes, w_scales, yp, m, n, k, ld_y, stream);
        case 42: return launch_gemm<4, 2>(a_codes, a_scales, w_codes, w_scales, yp, m, n, k, ld_y, stream);
        default: return launch_gemm<4, 4>(a_codes, a_scales, w_codes, w_scales, yp, m, n, k, ld_y, stream);
    }
}

// kq_gemm_wide.h — launcher of the 256 x 256-tile W4A4 GEMM kernel
// (kq_gemm_wide.hip), called by kq_w4a4_gemm after its argument checks.
#pragma once

#include <stdint.h>

#include "kq.h"

namespace kq {

// Y[M][ldy] = dequant(A) dequant(W)^T, bf16; K % 256 == 0, all arguments
// already validated; cus = compute units of the current device.
kq_status launch_gemm_wide(const uint8_t *ac, const uint8_t *as, const uint8_t *wc,
                           const uint8_t *ws, uint16_t *y, int M, int N, int K, int64_t ldy,
                           int cus, void *stream);

// The kernel's host-side handle (for hipFuncGetAttributes).
const void *wide_kernel_symbol();

}  // namespace kq

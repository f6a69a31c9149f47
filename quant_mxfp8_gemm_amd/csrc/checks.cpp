// checks.cpp - the host-only part of the C ABI of include/mxfp8.h: scale buffer sizes, status
// strings and the argument check of every operation. Plain C++ with no HIP call (hipStream_t
// appears only through the header), so the CPU tests can call it directly and build it with
// the address and undefined-behaviour sanitizers.
#include "mxfp8.h"

#include <stdint.h>

namespace {

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

constexpr int64_t kMaxOperandBytes = (int64_t)1 << 31;  // 32-bit offsets inside the GEMM
constexpr int64_t kMaxDim = (int64_t)1 << 40;           // any size or row stride: keeps products in int64

// a * b > lim for non-negative a, b, without forming the product
bool mul_exceeds(int64_t a, int64_t b, int64_t lim) { return a > 0 && b > lim / a; }

}  // namespace

extern "C" {

int64_t mxfp8_scale_bytes(int64_t rows, int64_t k, int layout) {
  if (rows < 0 || k <= 0 || k % 32 != 0 || rows > kMaxDim || k > kMaxDim) return -1;
  const int64_t nblk = k / 32;
  if (layout == MXFP8_SCALES_LINEAR) return rows * nblk;
  if (layout == MXFP8_SCALES_SWIZZLED_128X4) return ((rows + 127) / 128) * 128 * ((nblk + 3) / 4) * 4;
  return -1;
}

const char* mxfp8_status_string(int status) {
  switch (status) {
    case MXFP8_OK: return "ok";
    case MXFP8_EINVAL: return "invalid argument";
    case MXFP8_EALIGN: return "misaligned pointer or row stride";
    case MXFP8_EUNSUPPORTED: return "unsupported shape";
    case MXFP8_EHIP: return "HIP launch error";
    default: return "unknown status";
  }
}

int mxfp8_quantize_check(const void* x_bf16, int64_t rows, int64_t k, int64_t ldx, const void* q_e4m3,
                         const void* scales_linear, const void* scales_swizzled) {
  if (rows < 0 || k <= 0 || k % 32 != 0 || ldx < k) return MXFP8_EINVAL;
  if (rows == 0) return MXFP8_OK;  // nothing to read or write
  if (!x_bf16 || !q_e4m3 || (!scales_linear && !scales_swizzled)) return MXFP8_EINVAL;
  if (rows > ((int64_t)1 << 31) - 1 || ldx > kMaxDim || mul_exceeds(rows, ldx, kMaxDim)) return MXFP8_EUNSUPPORTED;
  if (!aligned(x_bf16, 16) || ldx % 8 != 0 || !aligned(q_e4m3, 8)) return MXFP8_EALIGN;
  return MXFP8_OK;
}

int rmsnorm_quant_mxfp8_check(const void* x_bf16, const void* w_bf16, int64_t rows, int64_t hidden,
                              int64_t ldx, const void* q_e4m3, const void* scales_linear,
                              const void* scales_swizzled) {
  if (rows < 0 || hidden <= 0 || hidden % 32 != 0 || ldx < hidden) return MXFP8_EINVAL;
  if (hidden > 16384) return MXFP8_EUNSUPPORTED;
  if (rows == 0) return MXFP8_OK;  // nothing to read or write
  if (!x_bf16 || !w_bf16 || !q_e4m3 || (!scales_linear && !scales_swizzled)) return MXFP8_EINVAL;
  if (rows > ((int64_t)1 << 31) - 1 || ldx > kMaxDim || mul_exceeds(rows, ldx, kMaxDim)) return MXFP8_EUNSUPPORTED;
  if (!aligned(x_bf16, 16) || !aligned(w_bf16, 16) || ldx % 8 != 0 || !aligned(q_e4m3, 8)) return MXFP8_EALIGN;
  return MXFP8_OK;
}

int add_rmsnorm_quant_mxfp8_check(const void* x_bf16, const void* residual_bf16, const void* w_bf16,
                                  int64_t rows, int64_t hidden, int64_t ldx, int64_t ldr, const void* q_e4m3,
                                  const void* scales_linear, const void* scales_swizzled) {
  const int st = rmsnorm_quant_mxfp8_check(x_bf16, w_bf16, rows, hidden, ldx, q_e4m3, scales_linear,
                                           scales_swizzled);
  if (st != MXFP8_OK || rows == 0) return st;
  if (!residual_bf16 || ldr < hidden) return MXFP8_EINVAL;
  if (ldr > kMaxDim || mul_exceeds(rows, ldr, kMaxDim)) return MXFP8_EUNSUPPORTED;
  if (!aligned(residual_bf16, 16) || ldr % 8 != 0) return MXFP8_EALIGN;
  // x and the residual stream must not overlap (each row of the residual is rewritten)
  const uintptr_t x0 = (uintptr_t)x_bf16, x1 = x0 + (uintptr_t)(((rows - 1) * ldx + hidden) * 2);
  const uintptr_t r0 = (uintptr_t)residual_bf16, r1 = r0 + (uintptr_t)(((rows - 1) * ldr + hidden) * 2);
  if (x0 < r1 && r0 < x1) return MXFP8_EINVAL;
  return MXFP8_OK;
}

int mxfp8_swizzle_scales_check(const void* scales_linear, int64_t rows, int64_t k,
                               const void* scales_swizzled) {
  if (rows < 0 || k <= 0 || k % 32 != 0) return MXFP8_EINVAL;
  if (rows == 0) return MXFP8_OK;  // nothing to read or write
  if (!scales_linear || !scales_swizzled) return MXFP8_EINVAL;
  if (rows > kMaxDim || k > kMaxDim || mul_exceeds(rows, k, kMaxDim)) return MXFP8_EUNSUPPORTED;
  if (!aligned(scales_swizzled, 16)) return MXFP8_EALIGN;
  return MXFP8_OK;
}

int mxfp8_gemm_bf16out_check(const void* a_e4m3, const void* a_scales, int a_scale_layout,
                             const void* b_e4m3, const void* b_scales, int b_scale_layout,
                             int64_t m, int64_t n, int64_t k, const void* c_bf16, int64_t ldc,
                             int num_chunks, int first_chunk) {
  if (m < 1 || n < 1 || k <= 0 || k % 32 != 0) return MXFP8_EINVAL;
  if (!a_e4m3 || !a_scales || !b_e4m3 || !b_scales || !c_bf16) return MXFP8_EINVAL;
  if ((a_scale_layout != MXFP8_SCALES_LINEAR && a_scale_layout != MXFP8_SCALES_SWIZZLED_128X4) ||
      (b_scale_layout != MXFP8_SCALES_LINEAR && b_scale_layout != MXFP8_SCALES_SWIZZLED_128X4))
    return MXFP8_EINVAL;
  if (ldc < n || ldc > ((int64_t)1 << 31) - 1) return MXFP8_EINVAL;
  if (num_chunks < 1 || m % num_chunks != 0 || first_chunk < 0 || first_chunk >= num_chunks) return MXFP8_EINVAL;
  if (k % 128 != 0) return MXFP8_EUNSUPPORTED;
  if (m > ((int64_t)1 << 30) || n > ((int64_t)1 << 30) || k > kMaxOperandBytes) return MXFP8_EUNSUPPORTED;
  if (m * k > kMaxOperandBytes || n * k > kMaxOperandBytes || m * ldc > ((int64_t)1 << 40)) return MXFP8_EUNSUPPORTED;
  if (!aligned(a_e4m3, 16) || !aligned(b_e4m3, 16) || !aligned(a_scales, 4) || !aligned(b_scales, 4) ||
      !aligned(c_bf16, 8) || ldc % 4 != 0)
    return MXFP8_EALIGN;
  return MXFP8_OK;
}

int mxfp8_gemm_silu_mul_quant_check(const void* a_e4m3, const void* a_scales, int a_scale_layout,
                                    const void* w_e4m3, const void* w_scales, int w_scale_layout, int64_t m,
                                    int64_t inter, int64_t k, const void* q_e4m3, const void* scales_linear,
                                    const void* scales_swizzled) {
  if (m < 1 || inter < 32 || inter % 32 != 0 || k <= 0 || k % 32 != 0) return MXFP8_EINVAL;
  if (!a_e4m3 || !a_scales || !w_e4m3 || !w_scales || !q_e4m3 || (!scales_linear && !scales_swizzled))
    return MXFP8_EINVAL;
  if ((a_scale_layout != MXFP8_SCALES_LINEAR && a_scale_layout != MXFP8_SCALES_SWIZZLED_128X4) ||
      (w_scale_layout != MXFP8_SCALES_LINEAR && w_scale_layout != MXFP8_SCALES_SWIZZLED_128X4))
    return MXFP8_EINVAL;
  if (k % 128 != 0) return MXFP8_EUNSUPPORTED;
  if (m > ((int64_t)1 << 30) || inter > ((int64_t)1 << 29) || k > kMaxOperandBytes) return MXFP8_EUNSUPPORTED;
  if (m * k > kMaxOperandBytes || 2 * inter * k > kMaxOperandBytes || m * inter > ((int64_t)1 << 40))
    return MXFP8_EUNSUPPORTED;
  if (!aligned(a_e4m3, 16) || !aligned(w_e4m3, 16) || !aligned(a_scales, 4) || !aligned(w_scales, 4) ||
      !aligned(q_e4m3, 16))
    return MXFP8_EALIGN;
  return MXFP8_OK;
}

}  // extern "C"

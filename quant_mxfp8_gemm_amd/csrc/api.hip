// api.hip - the C ABI declared in include/mxfp8.h: host-side argument checks, then launches.
#include "mxfp8.h"

#include <stdint.h>

#include "kernels.h"

namespace {

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

int hip_status(hipError_t e) { return e == hipSuccess ? MXFP8_OK : MXFP8_EHIP; }

constexpr int64_t kMaxOperandBytes = (int64_t)1 << 31;  // 32-bit offsets inside the GEMM

}  // namespace

extern "C" {

int64_t mxfp8_scale_bytes(int64_t rows, int64_t k, int layout) {
  if (rows < 0 || k <= 0 || k % 32 != 0) return -1;
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
  if (rows > ((int64_t)1 << 31) - 1) return MXFP8_EUNSUPPORTED;
  if (!aligned(x_bf16, 16) || ldx % 8 != 0 || !aligned(q_e4m3, 8)) return MXFP8_EALIGN;
  return MXFP8_OK;
}

int mxfp8_quantize(const void* x_bf16, int64_t rows, int64_t k, int64_t ldx, void* q_e4m3,
                   void* scales_linear, void* scales_swizzled, hipStream_t stream) {
  const int st = mxfp8_quantize_check(x_bf16, rows, k, ldx, q_e4m3, scales_linear, scales_swizzled);
  if (st != MXFP8_OK) return st;
  return hip_status(mxfp8::launch_quantize((const uint16_t*)x_bf16, rows, k, ldx, (uint8_t*)q_e4m3,
                                           (uint8_t*)scales_linear, (uint8_t*)scales_swizzled, stream));
}

int rmsnorm_quant_mxfp8_check(const void* x_bf16, const void* w_bf16, int64_t rows, int64_t hidden,
                              int64_t ldx, const void* q_e4m3, const void* scales_linear,
                              const void* scales_swizzled) {
  if (rows < 0 || hidden <= 0 || hidden % 32 != 0 || ldx < hidden) return MXFP8_EINVAL;
  if (hidden > 16384) return MXFP8_EUNSUPPORTED;
  if (rows == 0) return MXFP8_OK;  // nothing to read or write
  if (!x_bf16 || !w_bf16 || !q_e4m3 || (!scales_linear && !scales_swizzled)) return MXFP8_EINVAL;
  if (hidden > 16384 || rows > ((int64_t)1 << 31) - 1) return MXFP8_EUNSUPPORTED;
  if (!aligned(x_bf16, 16) || !aligned(w_bf16, 16) || ldx % 8 != 0 || !aligned(q_e4m3, 8)) return MXFP8_EALIGN;
  return MXFP8_OK;
}

int rmsnorm_quant_mxfp8(const void* x_bf16, const void* w_bf16, int64_t rows, int64_t hidden,
                        int64_t ldx, float eps, void* q_e4m3, void* scales_linear,
                        void* scales_swizzled, hipStream_t stream) {
  const int st = rmsnorm_quant_mxfp8_check(x_bf16, w_bf16, rows, hidden, ldx, q_e4m3, scales_linear,
                                           scales_swizzled);
  if (st != MXFP8_OK) return st;
  return hip_status(mxfp8::launch_rmsnorm_quant((const uint16_t*)x_bf16, (const uint16_t*)w_bf16, rows,
                                                hidden, ldx, eps, (uint8_t*)q_e4m3,
                                                (uint8_t*)scales_linear, (uint8_t*)scales_swizzled, nullptr,
                                                0, stream));
}

int add_rmsnorm_quant_mxfp8_check(const void* x_bf16, const void* residual_bf16, const void* w_bf16,
                                  int64_t rows, int64_t hidden, int64_t ldx, int64_t ldr, const void* q_e4m3,
                                  const void* scales_linear, const void* scales_swizzled) {
  const int st = rmsnorm_quant_mxfp8_check(x_bf16, w_bf16, rows, hidden, ldx, q_e4m3, scales_linear,
                                           scales_swizzled);
  if (st != MXFP8_OK || rows == 0) return st;
  if (!residual_bf16 || ldr < hidden) return MXFP8_EINVAL;
  if (!aligned(residual_bf16, 16) || ldr % 8 != 0) return MXFP8_EALIGN;
  // x and the residual stream must not overlap (each row of the residual is rewritten)
  const uintptr_t x0 = (uintptr_t)x_bf16, x1 = x0 + (uintptr_t)(((rows - 1) * ldx + hidden) * 2);
  const uintptr_t r0 = (uintptr_t)residual_bf16, r1 = r0 + (uintptr_t)(((rows - 1) * ldr + hidden) * 2);
  if (x0 < r1 && r0 < x1) return MXFP8_EINVAL;
  return MXFP8_OK;
}

int add_rmsnorm_quant_mxfp8(const void* x_bf16, void* residual_bf16, const void* w_bf16, int64_t rows,
                            int64_t hidden, int64_t ldx, int64_t ldr, float eps, void* q_e4m3,
                            void* scales_linear, void* scales_swizzled, hipStream_t stream) {
  const int st = add_rmsnorm_quant_mxfp8_check(x_bf16, residual_bf16, w_bf16, rows, hidden, ldx, ldr, q_e4m3,
                                               scales_linear, scales_swizzled);
  if (st != MXFP8_OK) return st;
  return hip_status(mxfp8::launch_rmsnorm_quant((const uint16_t*)x_bf16, (const uint16_t*)w_bf16, rows,
                                                hidden, ldx, eps, (uint8_t*)q_e4m3,
                                                (uint8_t*)scales_linear, (uint8_t*)scales_swizzled,
                                                (uint16_t*)residual_bf16, ldr, stream));
}

int mxfp8_swizzle_scales_check(const void* scales_linear, int64_t rows, int64_t k,
                               const void* scales_swizzled) {
  if (rows < 0 || k <= 0 || k % 32 != 0) return MXFP8_EINVAL;
  if (rows == 0) return MXFP8_OK;  // nothing to read or write
  if (!scales_linear || !scales_swizzled) return MXFP8_EINVAL;
  if (!aligned(scales_swizzled, 16)) return MXFP8_EALIGN;
  return MXFP8_OK;
}

int mxfp8_swizzle_scales(const void* scales_linear, int64_t rows, int64_t k, void* scales_swizzled,
                         hipStream_t stream) {
  const int st = mxfp8_swizzle_scales_check(scales_linear, rows, k, scales_swizzled);
  if (st != MXFP8_OK) return st;
  return hip_status(mxfp8::launch_swizzle_scales((const uint8_t*)scales_linear, rows, k,
                                                 (uint8_t*)scales_swizzled, stream));
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
  if (m * k > kMaxOperandBytes || n * k > kMaxOperandBytes || m * ldc > ((int64_t)1 << 40) ||
      m > ((int64_t)1 << 30) || n > ((int64_t)1 << 30))
    return MXFP8_EUNSUPPORTED;
  if (!aligned(a_e4m3, 16) || !aligned(b_e4m3, 16) || !aligned(a_scales, 4) || !aligned(b_scales, 4) ||
      !aligned(c_bf16, 8) || ldc % 4 != 0)
    return MXFP8_EALIGN;
  return MXFP8_OK;
}

int mxfp8_gemm_bf16out(const void* a_e4m3, const void* a_scales, int a_scale_layout,
                       const void* b_e4m3, const void* b_scales, int b_scale_layout, int64_t m,
                       int64_t n, int64_t k, void* c_bf16, int64_t ldc, int num_chunks,
                       int first_chunk, int* chunk_done, hipStream_t stream) {
  const int st = mxfp8_gemm_bf16out_check(a_e4m3, a_scales, a_scale_layout, b_e4m3, b_scales,
                                          b_scale_layout, m, n, k, c_bf16, ldc, num_chunks, first_chunk);
  if (st != MXFP8_OK) return st;
  return hip_status(mxfp8::launch_gemm((const uint8_t*)a_e4m3, (const uint8_t*)a_scales, a_scale_layout,
                                       (const uint8_t*)b_e4m3, (const uint8_t*)b_scales, b_scale_layout, m,
                                       n, k, (uint16_t*)c_bf16, ldc, num_chunks, first_chunk, chunk_done,
                                       stream));
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
  if (m * k > kMaxOperandBytes || 2 * inter * k > kMaxOperandBytes || m * inter > ((int64_t)1 << 40) ||
      m > ((int64_t)1 << 30) || inter > ((int64_t)1 << 29))
    return MXFP8_EUNSUPPORTED;
  if (!aligned(a_e4m3, 16) || !aligned(w_e4m3, 16) || !aligned(a_scales, 4) || !aligned(w_scales, 4) ||
      !aligned(q_e4m3, 16))
    return MXFP8_EALIGN;
  return MXFP8_OK;
}

int mxfp8_gemm_silu_mul_quant(const void* a_e4m3, const void* a_scales, int a_scale_layout, const void* w_e4m3,
                              const void* w_scales, int w_scale_layout, int64_t m, int64_t inter, int64_t k,
                              void* q_e4m3, void* scales_linear, void* scales_swizzled, hipStream_t stream) {
  const int st = mxfp8_gemm_silu_mul_quant_check(a_e4m3, a_scales, a_scale_layout, w_e4m3, w_scales,
                                                 w_scale_layout, m, inter, k, q_e4m3, scales_linear,
                                                 scales_swizzled);
  if (st != MXFP8_OK) return st;
  return hip_status(mxfp8::launch_gemm_silu_mul_quant(
      (const uint8_t*)a_e4m3, (const uint8_t*)a_scales, a_scale_layout, (const uint8_t*)w_e4m3,
      (const uint8_t*)w_scales, w_scale_layout, m, inter, k, (uint8_t*)q_e4m3, (uint8_t*)scales_linear,
      (uint8_t*)scales_swizzled, stream));
}

int64_t mxfp8_gemm_tiles_per_chunk(int64_t m, int64_t n, int num_chunks) {
  if (m < 1 || n < 1 || num_chunks < 1 || m % num_chunks != 0) return -1;
  const mxfp8::GemmShape s = mxfp8::gemm_pick_shape(m, n, num_chunks);
  return ((m / num_chunks + s.bm - 1) / s.bm) * ((n + s.bn - 1) / s.bn);
}

}  // extern "C"

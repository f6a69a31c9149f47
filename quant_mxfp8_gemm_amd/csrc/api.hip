// api.hip - the C ABI declared in include/mxfp8.h: each entry point runs its host-side argument
// check (checks.cpp), then launches its kernels on the caller's stream.
#include "mxfp8.h"

#include <stdint.h>

#include "kernels.h"

namespace {

int hip_status(hipError_t e) { return e == hipSuccess ? MXFP8_OK : MXFP8_EHIP; }

}  // namespace

extern "C" {

int mxfp8_quantize(const void* x_bf16, int64_t rows, int64_t k, int64_t ldx, void* q_e4m3,
                   void* scales_linear, void* scales_swizzled, hipStream_t stream) {
  const int st = mxfp8_quantize_check(x_bf16, rows, k, ldx, q_e4m3, scales_linear, scales_swizzled);
  if (st != MXFP8_OK) return st;
  return hip_status(mxfp8::launch_quantize((const uint16_t*)x_bf16, rows, k, ldx, (uint8_t*)q_e4m3,
                                           (uint8_t*)scales_linear, (uint8_t*)scales_swizzled, stream));
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

int mxfp8_swizzle_scales(const void* scales_linear, int64_t rows, int64_t k, void* scales_swizzled,
                         hipStream_t stream) {
  const int st = mxfp8_swizzle_scales_check(scales_linear, rows, k, scales_swizzled);
  if (st != MXFP8_OK) return st;
  return hip_status(mxfp8::launch_swizzle_scales((const uint8_t*)scales_linear, rows, k,
                                                 (uint8_t*)scales_swizzled, stream));
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

int64_t mxfp8_gemm_tiles_per_chunk(int64_t m, int64_t n, int num_chunks, int a_scale_layout,
                                   int b_scale_layout) {
  if (m < 1 || n < 1 || num_chunks < 1 || m % num_chunks != 0) return -1;
  if ((a_scale_layout != 0 && a_scale_layout != 1) || (b_scale_layout != 0 && b_scale_layout != 1)) return -1;
  const mxfp8::GemmShape s = mxfp8::gemm_pick_shape(m, n, num_chunks, a_scale_layout, b_scale_layout);
  return ((m / num_chunks + s.bm - 1) / s.bm) * ((n + s.bn - 1) / s.bn);
}

}  // extern "C"
